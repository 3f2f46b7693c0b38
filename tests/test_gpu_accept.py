"""GPU parity of spec_accept_resample (the fused vocab kernel) against the oracle.

Inputs follow the accept/resample-only workload: target logits ~ N(0, 2^2) [B, K+1, V],
draft logits = target + N(0, 0.5^2), draft tokens drawn from the oracle's processed q
with Philox purpose-0 uniforms.
"""
import numpy as np
import pytest
import torch
from scipy import stats

from oracle import philox, sampling, theory
from speculative_decoding_forward_amd import binding, synth

from helpers import DEV, Tally, check_accept_against_oracle, gpu_accept, to_dev

pytestmark = pytest.mark.gpu


def draft_tokens(q, knobs, seed, rnd):
    T, k, tp = knobs
    B, K, V = q.shape
    xt = np.zeros((B, K), dtype=np.int64)
    for b in range(B):
        for j in range(K):
            u = float(philox.uniform(seed, rnd, j, b, 0))
            xt[b, j] = sampling.draft_sample(q[b, j], u, T, k, tp)
    return xt


def case(B, K, V, knobs, seed=0, rnd=0, p_sigma=2.0, noise=0.5):
    p, q = synth.vocab_logits(seed, B, K, V, p_sigma, noise)
    xt = draft_tokens(q, knobs, seed, rnd)
    return p, q, xt


@pytest.mark.parametrize("B,K,V,knobs", [
    (32, 8, 32000, (0.8, 0, 1.0)),          # the accept/resample-only workload
    (8, 5, 32000, (0.8, 0, 0.95)),          # 7B-shape knobs: T=0.8, top-p 0.95
    (4, 3, 1000, (1.0, 40, 0.9)),           # top-k then top-p, one partial slab
    (2, 2, 32768, (1.3, 0, 1.0)),           # largest vocabulary
    (3, 16, 17, (1.0, 0, 1.0)),             # tiny vocabulary, largest K
    (5, 1, 1029, (0.5, 7, 1.0)),            # ragged tail, K = 1, top-k
])
def test_accept_parity(B, K, V, knobs):
    p, q, xt = case(B, K, V, knobs, seed=B * 1000 + V)
    g = gpu_accept(p, q, xt, knobs, seed=11, rnd=3)
    tally = Tally()
    check_accept_against_oracle(p, q, xt, knobs, 11, 3, g, tally)
    print(f"B={B} K={K} V={V} knobs={knobs}: {tally.report()}")
    assert np.all(g["status"] == 0)
    near = sum(tally.near.values())
    assert near <= max(2, 0.01 * tally.exact), tally.report()


def test_deterministic_repeat():
    p, q, xt = case(32, 8, 32000, (0.8, 0, 1.0))
    a = gpu_accept(p, q, xt, (0.8, 0, 1.0), 5, 9)
    b = gpu_accept(p, q, xt, (0.8, 0, 1.0), 5, 9)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_q_equal_p_accepts_everything():
    B, K, V = 6, 5, 4096
    p, _ = synth.vocab_logits(1, B, K, V)
    q = p[:, :K].copy()
    xt = draft_tokens(q, (0.9, 0, 0.95), 1, 0)
    g = gpu_accept(p, q, xt, (0.9, 0, 0.95), 2, 0)
    assert np.all(g["n_out"] == K + 1) and np.all(g["status"] == 0)
    assert np.array_equal(g["out"][:, :K], xt)


def test_status_rows():
    B, K, V = 4, 3, 2048
    p, q, xt = case(B, K, V, (1.0, 0, 1.0), seed=4)
    p[1, 2, 77] = np.nan                    # non-finite target logit in row 1
    xt[2, 1] = V + 5                        # draft token out of range in row 2
    q[3, 0, :] = -1000.0                    # row 3: q(x~_0) underflows to exactly 0
    q[3, 0, 5] = 10.0
    xt[3, 0] = 6
    g = gpu_accept(p, q, xt, (1.0, 0, 1.0), 7, 1)
    assert g["n_out"][1] == 0 and g["status"][1] & binding.ROW_NONFINITE
    assert np.all(g["out"][1] == -1)
    assert g["n_out"][2] == 0 and g["status"][2] & binding.ROW_BAD_TOKEN
    assert g["status"][3] & binding.ROW_Q_ZERO
    # q = 0, p > 0 at the draft: accepted under u*q < p
    assert g["acc"][3, 0] == 1
    assert g["status"][0] == 0 and 1 <= g["n_out"][0] <= K + 1


@pytest.mark.parametrize("B,K,V,knobs", [
    (8, 5, 32000, (0.0, 0, 0.95)),          # 7B-shape knobs at T = 0 (top-p inert)
    (6, 4, 1029, (0.0, 7, 1.0)),            # ragged tail, top-k inert
    (4, 16, 17, (0.0, 0, 1.0)),             # tiny vocabulary, largest K
    (2, 2, 32768, (0.0, 0, 1.0)),           # largest vocabulary
])
def test_greedy_bit_exact(B, K, V, knobs):
    """T = 0 (argmax decoding): every decision is an exact comparison of the same fp32
    logits on both sides, so the processed rows (one-hot), accept flags, candidates,
    outputs and status equal the oracle's bit for bit.  Row b agrees with the target
    for its first b % (K + 1) positions (q = p there, so argmax q = argmax p), and every
    row carries a planted tie at its maximum, placed before or after the first maximum."""
    rng = np.random.default_rng(V + K)
    p, q = synth.vocab_logits(B * 7 + V, B, K, V)
    for b in range(B):
        for j in range(K + 1):
            i = int(rng.integers(0, V))
            p[b, j, i] = p[b, j].max()
            if j < K:
                i = int(rng.integers(0, V))
                q[b, j, i] = q[b, j].max()
        n_agree = b % (K + 1)
        q[b, :n_agree] = p[b, :n_agree]
    xt = q.argmax(axis=2)                    # the greedy draft: argmax q, lowest id
    g = gpu_accept(p, q, xt, knobs, seed=3, rnd=1)
    T, k, tp = knobs
    for b in range(B):
        P = np.stack([sampling.transform(r, T, k, tp) for r in p[b]])
        Q = np.stack([sampling.transform(r, T, k, tp) for r in q[b]])
        assert np.array_equal(g["pp"][b], P) and np.array_equal(g["qp"][b], Q)
        ua = philox.uniform(3, 1, np.arange(K), b, 1)
        ur = philox.uniform(3, 1, np.arange(K + 1), b, 2)
        toks, n, a, st = sampling.accept_resample_logits(p[b], q[b], xt[b], ua, ur, T, k, tp)
        assert a >= b % (K + 1)
        assert g["n_out"][b] == n and list(g["out"][b, :n]) == toks, (b, g["out"][b], toks)
        assert np.all(g["out"][b, n:] == -1) and g["status"][b] == st == 0
        amax = p[b].argmax(axis=1)
        assert np.array_equal(g["acc"][b], (xt[b] == amax[:K]).astype(g["acc"].dtype))
        for j in range(K + 1):
            want = -1 if (j < K and xt[b, j] == amax[j]) else amax[j]
            assert g["cand"][b, j] == want, (b, j)


def test_argument_errors():
    B, K, V = 2, 2, 64
    p, q, xt = case(B, K, V, (1.0, 0, 1.0))
    with pytest.raises(binding.SpecError) as e:
        gpu_accept(p, q, xt, (-0.5, 0, 1.0), 0, 0)
    assert e.value.status == binding.SPEC_E_INVALID
    with pytest.raises(binding.SpecError) as e:
        gpu_accept(p, q, xt, (1.0, 0, 1.5), 0, 0)
    assert e.value.status == binding.SPEC_E_INVALID
    big = np.zeros((1, 2, 40000), np.float32)
    with pytest.raises(binding.SpecError) as e:
        gpu_accept(big, big[:, :1], np.zeros((1, 1), np.int64), (1.0, 0, 1.0), 0, 0)
    assert e.value.status == binding.SPEC_E_UNSUPPORTED


def test_chi_square_million_rounds_on_gpu():
    """10^6 GPU rounds of the rule on one fixed (p, q) pair: the first emitted token
    follows P_0 (lossless), n_out stays in [1, K+1] and its mean matches
    sum_j prod_{i<j} beta_i."""
    V, K, B = 16, 3, 8192
    rng = np.random.default_rng(5)
    pl = rng.normal(0, 1.0, (K + 1, V)).astype(np.float32)
    ql = (pl[:K] + rng.normal(0, 0.7, (K, V))).astype(np.float32)
    P = np.stack([sampling.transform(r, 1.0) for r in pl])
    Q = np.stack([sampling.transform(r, 1.0) for r in ql])
    p = np.broadcast_to(pl, (B, K + 1, V)).copy()
    q = np.broadcast_to(ql, (B, K, V)).copy()
    Pd, Qd = to_dev(p), to_dev(q)
    rounds = 123
    counts = np.zeros(V, dtype=np.int64)
    nsum, n = 0, 0
    ws = binding.accept_workspace(B, K)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=DEV)
    n_out = torch.empty(B, dtype=torch.int32, device=DEV)
    st = torch.empty(B, dtype=torch.int32, device=DEV)
    for r in range(rounds):
        # draft tokens ~ Q with purpose-0 uniforms of this round (drawn by the oracle)
        u0 = np.stack([philox.uniform(1, r, j, np.arange(B), 0) for j in range(K)], axis=1)
        xt = np.stack([sampling.sample(Q[j], u0[:, j]) for j in range(K)], axis=1)
        binding.accept_resample(Pd, Qd, to_dev(xt.astype(np.int32)), (1.0, 0, 1.0), 1, r, out,
                                n_out, st, ws)
        o = out.cpu().numpy()
        nn = n_out.cpu().numpy()
        assert nn.min() >= 1 and nn.max() <= K + 1
        counts += np.bincount(o[:, 0], minlength=V)
        nsum += int(nn.sum())
        n += B
    assert n >= 10**6
    res = stats.chisquare(counts, P[0] * n)
    assert res.pvalue > 1e-4, res
    betas = [theory.acceptance_rate(P[j], Q[j]) for j in range(K)]
    expect = theory.expected_tokens_rows(betas)
    print(f"mean n_out {nsum / n:.4f} expected {expect:.4f}")
    assert abs(nsum / n - expect) < 0.01


def test_empty_residual_falls_back_to_p():
    """A rejection whose residual max(0, p - q) is empty ([LENS] §2.3; the reading that
    such a row samples P_a): q = p row for row, and each row's first draft token lies
    outside the top-k set, so p(x~) = q(x~) = 0 on both sides and the token is rejected
    with nothing left in the residual.  The GPU must set SPEC_ROW_RESIDUAL_EMPTY (and
    Q_ZERO) and emit the oracle's draw from P_0 with the resample uniform."""
    B, K, V = 6, 3, 4096
    knobs = (0.9, 16, 1.0)
    p, _ = synth.vocab_logits(21, B, K, V)
    q = p[:, :K].copy()
    xt = np.zeros((B, K), dtype=np.int64)
    for b in range(B):
        P0 = sampling.transform(p[b, 0], *knobs)
        xt[b, 0] = int(np.nonzero(P0 == 0)[0][b])       # outside the kept set
        xt[b, 1:] = np.argmax(p[b, 1:K], axis=-1)
    g = gpu_accept(p, q, xt, knobs, seed=13, rnd=2)
    for b in range(B):
        P = np.stack([sampling.transform(r, *knobs) for r in p[b]])
        Q = np.stack([sampling.transform(r, *knobs) for r in q[b]])
        ua = philox.uniform(13, 2, np.arange(K), b, 1)
        ur = philox.uniform(13, 2, np.arange(K + 1), b, 2)
        toks, n, a, st = sampling.accept_resample(P, Q, xt[b], ua, ur)
        assert a == 0 and st & sampling.ST_RESIDUAL_EMPTY
        assert g["n_out"][b] == 1 and g["out"][b, 0] == toks[0], (b, g["out"][b], toks)
        assert g["status"][b] & binding.ROW_RESIDUAL_EMPTY
        assert g["status"][b] & binding.ROW_Q_ZERO
        assert g["cand"][b, 0] == toks[0]


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_top_k_ties_are_kept(T):
    """Ties at the k-th largest logit are all kept on both p and q ([NOTE] Recommendation
    R3: knobs before the rule; the tie reading): rows with a tie planted across the
    top-k threshold keep every tied token, exactly as the oracle's transform does."""
    B, K, V, k = 4, 2, 2048, 10
    p, q = synth.vocab_logits(31, B, K, V)
    rng = np.random.default_rng(5)
    for arr in (p, q):
        for b in range(arr.shape[0]):
            for j in range(arr.shape[1]):
                row = arr[b, j]
                order = np.argsort(-row)
                tied = rng.choice(np.arange(8, 40), 6, replace=False)  # straddle rank k
                row[order[tied]] = row[order[k - 1]]
    knobs = (T, k, 1.0)
    xt = draft_tokens(q, knobs, 31, 0)
    g = gpu_accept(p, q, xt, knobs, seed=17, rnd=1)
    for b in range(B):
        for j in range(K + 1):
            P = sampling.transform(p[b, j], *knobs)
            assert np.array_equal(g["pp"][b, j] > 0, P > 0), (b, j)
            assert (P > 0).sum() > k                       # the ties were kept
            assert np.abs(g["pp"][b, j] - P).max() <= 1e-6
        for j in range(K):
            Q = sampling.transform(q[b, j], *knobs)
            assert np.array_equal(g["qp"][b, j] > 0, Q > 0), (b, j)
    tally = Tally()
    check_accept_against_oracle(p, q, xt, knobs, 17, 1, g, tally)
    assert sum(tally.near.values()) <= 1, tally.report()
