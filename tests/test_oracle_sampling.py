"""Pins of the oracle's sampling side against what the pages and mathematics fix.

Page tags: [ZSM] "Accelerating Large Language Model Decoding with Speculative Sampling"
(zeroshotmind); [CANON] "57 Speculative Decoding" (ml-canon); [LENS] "Speculative
Decoding from Scratch" (ta-paperlens); [NOTE] "NOTE-159" (anthology-of-the-sota).
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

from oracle import philox, sampling, theory


# ---------------------------------------------------------------- knob transform ---

def test_transform_plain_softmax():
    rng = np.random.default_rng(0)
    l = rng.normal(0, 2, 1000).astype(np.float32)
    np.testing.assert_allclose(sampling.transform(l, 1.0), softmax(l.astype(np.float64)),
                               rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("T", [0.8, 0.25, 1.7])
def test_transform_temperature(T):
    rng = np.random.default_rng(1)
    l = rng.normal(0, 2, 500).astype(np.float32)
    Tf = float(np.float32(T))
    np.testing.assert_allclose(sampling.transform(l, T), softmax(l.astype(np.float64) / Tf),
                               rtol=1e-12)


@pytest.mark.parametrize("knobs", [dict(), dict(top_k=5), dict(top_p=0.9), dict(top_k=3, top_p=0.5)])
def test_greedy_is_the_zero_temperature_limit(knobs):
    """T = 0 (argmax decoding) is the T -> 0 limit of the softmax path: once T is small
    against the gap between the two largest logits, exp((l - max) / T) underflows to
    exactly 0 for every other token, so the ordinary T > 0 path already returns the
    one-hot row -- with or without top-k / top-p."""
    rng = np.random.default_rng(2)
    for _ in range(6):
        l = rng.normal(0, 2, 300).astype(np.float32)
        top2 = np.sort(l.astype(np.float64))[-2:]
        T = (top2[1] - top2[0]) / 1000.0   # exp(-1000) is 0 in float64
        lim = sampling.transform(l, T, **knobs)
        assert np.count_nonzero(lim) == 1
        assert np.array_equal(lim, sampling.transform(l, 0.0, **knobs))


def test_greedy_ties_take_the_lowest_id():
    """Equal largest logits: the lowest token id (the reading for argmax decoding)."""
    l = np.array([0.5, 3.0, -1.0, 3.0, 3.0], np.float32)
    assert np.array_equal(sampling.transform(l, 0.0), [0, 1, 0, 0, 0])
    assert np.array_equal(sampling.transform(l[::-1].copy(), 0.0), [1, 0, 0, 0, 0])


def test_greedy_rule_keeps_the_target_argmax_prefix():
    """With one-hot rows the unchanged rule keeps the drafts up to the first one that is
    not argmax p, then emits argmax p there (or the bonus argmax p_K): checked against a
    direct comparison walk on random logits, with drafts that agree and disagree."""
    rng = np.random.default_rng(3)
    V, K = 50, 6
    for trial in range(200):
        pl = rng.normal(0, 1, (K + 1, V)).astype(np.float32)
        ql = rng.normal(0, 1, (K, V)).astype(np.float32)
        amax_p = pl.argmax(axis=1)
        n_agree = rng.integers(0, K + 1)
        xt = np.where(np.arange(K) < n_agree, amax_p[:K], rng.integers(0, V, K))
        u_acc, u_res = rng.random(K), rng.random(K + 1)
        toks, n, a, st = sampling.accept_resample_logits(pl, ql, xt, u_acc, u_res, 0.0)
        walk = []
        for j in range(K):
            if xt[j] != amax_p[j]:
                walk.append(int(amax_p[j]))
                break
            walk.append(int(xt[j]))
        else:
            walk.append(int(amax_p[K]))
        assert toks == walk and n == len(walk)


def _brute_top_k(l, k):
    # kept iff fewer than k tokens are strictly larger
    keep = np.array([np.sum(l > v) < k for v in l])
    return keep


def _brute_top_p(s, top_p):
    # kept iff the mass of tokens strictly more likely than it is below top_p
    return np.array([s[s > v].sum() < top_p for v in s])


@pytest.mark.parametrize("seed", range(6))
def test_top_k_brute_force(seed):
    rng = np.random.default_rng(seed)
    V = 40
    l = np.round(rng.normal(0, 1, V), 1).astype(np.float32)   # rounding creates ties
    for k in [1, 3, 7, 39]:
        s = sampling.transform(l, 1.0, top_k=k)
        keep = _brute_top_k(l.astype(np.float64), k)
        assert np.array_equal(s > 0, keep)
        np.testing.assert_allclose(s[keep], softmax(l[keep].astype(np.float64)), rtol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_top_p_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    V = 50
    l = rng.normal(0, 1.5, V).astype(np.float32)
    base = softmax(l.astype(np.float64))
    for tp in [0.3, 0.8, 0.95, 0.999]:
        if sampling.top_p_threshold_margin(base, tp) < 1e-9:
            continue
        s = sampling.transform(l, 1.0, top_p=tp)
        keep = _brute_top_p(base, float(np.float32(tp)))
        assert np.array_equal(s > 0, keep)
        np.testing.assert_allclose(s.sum(), 1.0, rtol=1e-12)
        np.testing.assert_allclose(s[keep], base[keep] / base[keep].sum(), rtol=1e-12)
        # the kept set is the smallest top set reaching the mass
        assert base[keep].sum() >= float(np.float32(tp))


def test_top_p_ties_are_kept():
    l = np.array([3.0, 1.0, 1.0, 1.0, -2.0], dtype=np.float32)
    s0 = softmax(l.astype(np.float64))
    tp = s0[0] + s0[1] * 0.5       # the cut falls inside the tied group
    s = sampling.transform(l, 1.0, top_p=tp)
    assert np.array_equal(s > 0, [True, True, True, True, False])


def _kept_set(l, T, top_p):
    return sampling.transform(l, T, top_p=top_p) > 0


@pytest.mark.parametrize("seed", range(8))
def test_top_p_threshold_margin_is_the_distance_to_the_next_membership_change(seed):
    """top_p_threshold_margin(s, tp) is the distance from tp to the nearest top-p mass at
    which the kept set changes, found here by bisection on the transform itself (which
    the brute-force tests pin): the kept set is the same for every threshold within the
    margin and differs just beyond it on one side.  Rows with tied probabilities are
    included (ties move in and out of the kept set together)."""
    rng = np.random.default_rng(40 + seed)
    V = 24
    l = rng.normal(0, 1.5, V).astype(np.float32)
    if seed % 2:
        l[rng.choice(V, 6, replace=False)] = l[0]   # a tied group
    T = 1.0
    base = sampling.transform(l, T)
    for tp in [0.35, 0.6, 0.9]:
        tp32 = float(np.float32(tp))
        m = sampling.top_p_threshold_margin(base, tp32)
        assert m > 1e-5, "the margins below are resolved to ~1e-7 only"
        ref = _kept_set(l, T, tp32)
        for f in (-0.98, -0.5, 0.5, 0.98):
            t = tp32 + f * m
            if 0.0 < t <= 1.0:
                assert np.array_equal(_kept_set(l, T, t), ref), (tp, f, m)
        # brute force: the nearest threshold (within [0, 1]) where the set changes
        def changes(t):
            return not np.array_equal(_kept_set(l, T, t), ref)

        best = np.inf
        for direction in (-1.0, 1.0):
            lo, hi = 0.0, None
            step = 1e-4
            while hi is None and step < 2.0:
                t = tp32 + direction * step
                if not 0.0 < t <= 1.0:
                    break
                if changes(t):
                    hi = step
                else:
                    lo, step = step, step * 1.5
            if hi is None:
                continue
            for _ in range(60):
                mid = 0.5 * (lo + hi)
                if changes(tp32 + direction * mid):
                    hi = mid
                else:
                    lo = mid
            best = min(best, hi)
        assert abs(best - m) <= 1e-6 * max(1.0, m) + 1e-9, (tp, best, m)


def test_knob_order_temperature_then_top_k_then_top_p():
    rng = np.random.default_rng(5)
    l = rng.normal(0, 2, 64).astype(np.float32)
    T, k, tp = 0.7, 10, 0.9
    z = l.astype(np.float64) / float(np.float32(T))
    keep_k = _brute_top_k(z, k)
    s = np.where(keep_k, np.exp(z - z.max()), 0.0)
    s /= s.sum()
    keep_p = _brute_top_p(s, float(np.float32(tp)))
    out = sampling.transform(l, T, top_k=k, top_p=tp)
    assert np.array_equal(out > 0, keep_p & keep_k)


# ------------------------------------------------------------- inverse-CDF sampling -

GRID = np.arange(2**24, dtype=np.float64) * 2.0 ** -24


def test_sample_full_grid_law():
    w = np.array([0.1, 0.0, 0.35, 0.05, 0.0, 0.5])
    idx = sampling.sample(w, GRID)
    counts = np.bincount(idx, minlength=w.size)
    assert counts[1] == 0 and counts[4] == 0            # zero mass is never drawn
    np.testing.assert_allclose(counts / 2**24, w / w.sum(), atol=2.0 ** -24)


def test_sample_smallest_index_rule():
    w = np.array([0.25, 0.25, 0.5])
    # C = [0.25, 0.5, 1.0]; u*S exactly on a boundary goes right (C_i > u*S strictly)
    assert sampling.sample(w, 0.25) == 1
    assert sampling.sample(w, 0.0) == 0
    assert sampling.sample(w, 0.5) == 2
    assert sampling.sample(np.zeros(3), 0.5) == -1


# ------------------------------------------- the rule: exact law by enumeration ------

def _dyadic_cases(n_cases, seed):
    """(p, q) with q a dyadic partition (powers of two >= 2**-6), p on a 1/16 grid, and
    the residual mass 1 - sum min(p, q) a power of two, so a 64-point uniform grid
    realises every probability of the rule exactly."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n_cases:
        V = int(rng.integers(4, 9))
        q = [Fraction(1)]
        while len(q) < V:
            i = int(rng.integers(len(q)))
            if q[i] <= Fraction(1, 64):
                continue
            h = q.pop(i) / 2
            q += [h, h]
        rng.shuffle(q)
        cuts = np.sort(rng.integers(0, 17, V - 1))
        parts = np.diff(np.concatenate([[0], cuts, [16]]))
        p = [Fraction(int(a), 16) for a in parts]
        S = sum(max(Fraction(0), pi - qi) for pi, qi in zip(p, q))
        if S == 0 or (S.numerator != 1) or (S.denominator & (S.denominator - 1)):
            continue
        out.append((p, q))
    return out


@pytest.mark.parametrize("p,q", _dyadic_cases(5, seed=2))
def test_rule_exact_identity_by_enumeration(p, q):
    """Pr[return x] = p(x) exactly ([ZSM] "Why the output distribution is exactly the
    target's"; [CANON] eq. for Pr[return x]; [LENS] §A.1), with the draft token weighted
    by q and both uniforms enumerated over a grid on which every decision is exact."""
    V = len(p)
    P = np.array([[float(v) for v in p], np.full(V, 1.0 / V)])     # row 1: bonus row
    Q = np.array([[float(v) for v in q]])
    G = 64
    law = [Fraction(0)] * V
    for xt in range(V):
        counts = np.zeros(V, dtype=np.int64)
        for i in range(G):
            for i2 in range(G):
                toks, n_out, a, st = sampling.accept_resample(
                    P, Q, [xt], [i / G], [i2 / G, 0.5])
                assert st == 0 and 1 <= n_out <= 2
                counts[toks[0]] += 1
        for x in range(V):
            law[x] += q[xt] * Fraction(int(counts[x]), G * G)
    assert law == p


def test_rule_identity_random_within_grid_bound():
    """Same identity for random (non-dyadic) p, q over the full 2**24 grid of each
    uniform, using the two decisions the rule is built from."""
    rng = np.random.default_rng(7)
    V = 6
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    r = np.maximum(0.0, p - q)
    res_law = np.bincount(sampling.sample(r, GRID), minlength=V) / 2**24
    law = np.zeros(V)
    for xt in range(V):
        acc = np.mean(sampling.accept_test(p[xt], q[xt], GRID))
        law[xt] += q[xt] * acc
        law += q[xt] * (1 - acc) * res_law
    np.testing.assert_allclose(law, p, atol=V * 2.0 ** -24)


# -------------------------------------------------------------------- special cases --

def test_q_le_p_always_accepts():
    """[LENS] §2.3: if q(x) <= p(x), accept unconditionally (also at u = 1 - 2**-24)."""
    P = np.array([[0.5, 0.3, 0.2], [1 / 3, 1 / 3, 1 / 3]])
    Q = np.array([[0.4, 0.3, 0.3]])
    for xt in (0, 1):
        for u in (0.0, 0.5, 1 - 2.0 ** -24):
            toks, n, a, st = sampling.accept_resample(P, Q, [xt], [u], [0.3, 0.3])
            assert a == 1 and toks[0] == xt and n == 2


def test_q_equals_p_emits_k_plus_1():
    rng = np.random.default_rng(3)
    K, V = 5, 30
    P = rng.dirichlet(np.ones(V), size=K + 1)
    Q = P[:K].copy()
    for t in range(200):
        xt = [int(rng.integers(V)) for _ in range(K)]
        toks, n, a, st = sampling.accept_resample(P, Q, xt, rng.random(K), rng.random(K + 1))
        assert n == K + 1 and toks[:K] == xt


def test_disjoint_supports_emit_one_token_from_p0():
    K, V = 3, 8
    P = np.zeros((K + 1, V)); P[:, :4] = 0.25
    Q = np.zeros((K, V)); Q[:, 4:] = 0.25
    rng = np.random.default_rng(4)
    seen = np.zeros(V)
    for t in range(4000):
        xt = [int(rng.integers(4, 8)) for _ in range(K)]
        toks, n, a, st = sampling.accept_resample(P, Q, xt, rng.random(K), rng.random(K + 1))
        assert n == 1 and a == 0
        seen[toks[0]] += 1
    assert seen[4:].sum() == 0
    assert stats.chisquare(seen[:4]).pvalue > 1e-4


def test_empty_residual_falls_back_to_p():
    # p == q but the draft is rejected (p(x~) = q(x~) = 0 -> reject under u*q < p)
    P = np.array([[0.5, 0.5, 0.0], [0.5, 0.5, 0.0]])
    Q = np.array([[0.5, 0.5, 0.0]])
    toks, n, a, st = sampling.accept_resample(P, Q, [2], [0.1], [0.75, 0.2])
    assert a == 0 and n == 1 and toks == [1]
    assert st & sampling.ST_RESIDUAL_EMPTY and st & sampling.ST_Q_ZERO


def test_non_finite_and_bad_token_rows_emit_nothing():
    p = np.zeros((3, 4), np.float32); q = np.zeros((2, 4), np.float32)
    p[1, 2] = np.nan
    assert sampling.accept_resample_logits(p, q, [0, 1], [0.1, 0.1], [0.1] * 3)[1:] == \
        (0, 0, sampling.ST_NONFINITE)
    p[1, 2] = 0.0
    assert sampling.accept_resample_logits(p, q, [0, 4], [0.1, 0.1], [0.1] * 3)[1:] == \
        (0, 0, sampling.ST_BAD_TOKEN)


# ------------------------------------------------ Monte Carlo over Philox uniforms ---

def _rounds(P, Q, n_rounds, seed):
    """Run the rule n_rounds times with draft tokens drawn from Q (purpose 0)."""
    K, V = Q.shape
    r = np.arange(n_rounds)
    xt = np.stack([sampling.sample(Q[j], philox.uniform(seed, r, j, 0, 0))
                   for j in range(K)], axis=1)
    ua = np.stack([philox.uniform(seed, r, j, 0, 1) for j in range(K)], axis=1)
    ur = np.stack([philox.uniform(seed, r, j, 0, 2) for j in range(K + 1)], axis=1)
    first = np.zeros(n_rounds, dtype=np.int64)
    n_out = np.zeros(n_rounds, dtype=np.int64)
    acc = np.zeros((n_rounds, K), dtype=bool)
    for i in range(n_rounds):
        toks, n, a, st = sampling.accept_resample(P, Q, xt[i], ua[i], ur[i])
        first[i], n_out[i] = toks[0], n
        acc[i, :a] = True
        if a < K:
            acc[i, a] = False
    return first, n_out, xt, ua


@pytest.fixture(scope="module")
def mc_million():
    rng = np.random.default_rng(11)
    K, V = 3, 8
    P = rng.dirichlet(np.ones(V) * 0.8, size=K + 1)
    Q = np.clip(P[:K] + rng.normal(0, 0.05, (K, V)), 0.005, None)
    Q /= Q.sum(axis=1, keepdims=True)
    first, n_out, xt, ua = _rounds(P, Q, 10**6, seed=123)
    return P, Q, first, n_out, xt, ua


def test_chi_square_first_token_is_p0(mc_million):
    """10**6 rounds: the first emitted token follows P_0 (the lossless property)."""
    P, Q, first, n_out, _, _ = mc_million
    counts = np.bincount(first, minlength=P.shape[1])
    res = stats.chisquare(counts, P[0] * first.size)
    assert res.pvalue > 1e-4, res


def test_tokens_per_call_bounds_and_expectation(mc_million):
    """1 <= n_out <= K+1 ([LENS] §2.1; [NOTE] "At least one token per loop"), and the
    mean equals sum_j prod_{i<j} beta_i with beta_i = sum min(P_i, Q_i) ([LENS] §3.1-3.2)."""
    P, Q, first, n_out, _, _ = mc_million
    K = Q.shape[0]
    assert n_out.min() >= 1 and n_out.max() <= K + 1
    betas = [theory.acceptance_rate(P[j], Q[j]) for j in range(K)]
    expect = theory.expected_tokens_rows(betas)
    sem = n_out.std() / np.sqrt(n_out.size)
    assert abs(n_out.mean() - expect) < 4 * sem


def test_acceptance_frequency_is_alpha(mc_million):
    """Per position, P(accept x~_0) = sum_x min(p(x), q(x)) (Theorem 3.5 / Cor. 3.6)."""
    P, Q, first, n_out, xt, ua = mc_million
    acc0 = ua[:, 0] * Q[0][xt[:, 0]] < P[0][xt[:, 0]]
    # the oracle accepted x~_0 exactly when at least 2 tokens came out
    assert np.array_equal(acc0, n_out >= 2)
    beta = theory.acceptance_rate(P[0], Q[0])
    sem = np.sqrt(beta * (1 - beta) / acc0.size)
    assert abs(acc0.mean() - beta) < 4 * sem


def test_multi_round_law_on_bigram_tables():
    """Across rounds, the first 3 tokens of the generated sequence follow the target's
    own chain law prod p(y_i | y_{i-1}) ([ZSM] "Why the output distribution is exactly
    the target's"), for prefix-dependent (bigram) target and draft tables."""
    rng = np.random.default_rng(21)
    V, K = 4, 2
    Pt = rng.dirichlet(np.ones(V), size=V)       # p(next | last)
    Qt = rng.dirichlet(np.ones(V), size=V)
    start = 1
    n_seq = 40000
    s_all = np.arange(n_seq)
    # each round emits >= 1 token, so 3 rounds always suffice for 3 tokens
    U0 = [[philox.uniform(9, rnd, j, s_all, 0) for j in range(K)] for rnd in range(3)]
    UA = [[philox.uniform(9, rnd, j, s_all, 1) for j in range(K)] for rnd in range(3)]
    UR = [[philox.uniform(9, rnd, j, s_all, 2) for j in range(K + 1)] for rnd in range(3)]
    seqs = np.zeros((n_seq, 3), dtype=np.int64)
    for s in range(n_seq):
        out, last, rnd = [], start, 0
        while len(out) < 3:
            xt, ctx = [], last
            for j in range(K):
                x = sampling.sample(Qt[ctx], float(U0[rnd][j][s]))
                xt.append(x)
                ctx = x
            chain = [last] + xt
            P = np.stack([Pt[c] for c in chain])          # rows 0..K
            Q = np.stack([Qt[c] for c in chain[:K]])
            ua = [UA[rnd][j][s] for j in range(K)]
            ur = [UR[rnd][j][s] for j in range(K + 1)]
            toks, n, a, st = sampling.accept_resample(P, Q, xt, ua, ur)
            out += toks
            last = toks[-1]
            rnd += 1
        seqs[s] = out[:3]
    idx = seqs[:, 0] * V * V + seqs[:, 1] * V + seqs[:, 2]
    counts = np.bincount(idx, minlength=V**3)
    law = np.einsum("a,ab,bc->abc", Pt[start], Pt, Pt).reshape(-1)
    res = stats.chisquare(counts, law * n_seq)
    assert res.pvalue > 1e-4, res
