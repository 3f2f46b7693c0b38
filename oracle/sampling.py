"""The sampling side of speculative sampling, written out plainly in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).  Page tags ([ZSM], [CANON],
[LENS], [GC], [NOTE]) are defined in ``oracle/__init__``.

Notation: p is the target distribution, q the draft distribution ([CANON] "The idea
and the mechanism"; [LENS] §2.3).  [NOTE] "Method" swaps the letters; we do not.
Indices are 0-based: drafts x~_0..x~_{K-1}; target rows P_0..P_K, row j scores draft
j and row K is the bonus row; draft rows Q_0..Q_{K-1}.

Functions and what pins them (tests/test_oracle_sampling.py):
  transform      -- temperature, then top-k, then top-p, applied to a logit row before
                    the rule ([NOTE] "Key results", robust-to-knobs item, and
                    Recommendation R3).  Pinned: T=1 with knobs off equals
                    scipy.special.softmax; top-k / top-p against brute-force sorted
                    enumeration on small V.
  sample         -- inverse-CDF draw in token-id order.  Pinned by brute force over the
                    full 2**24 uniform grid (law equals w/sum(w) within 2**-24 per token).
  accept_resample-- accept x~_j iff u*q(x~_j) < p(x~_j) ([ZSM] "The algorithm",
                    acceptance eq.; [CANON] eq. for alpha(x); [LENS] §2.3 rule), resample
                    the first rejection from norm(max(0, p - q)) ([CANON] residual eq.;
                    [LENS] §2.3 eq. for p'), bonus token from P_K when all K are accepted
                    ([LENS] §2.1 step 3; [GC] "How It Works" step 4).  Pinned: exact
                    identity Pr[return x] = p(x) ([ZSM] "Why the output distribution is
                    exactly the target's"; [CANON] eq. for Pr[return x]; [LENS] §A.1) by
                    brute force over the uniform grid on dyadic distributions (exact
                    equality in rationals) and on random ones (within V * 2**-24);
                    chi-square of the first emitted token over 10**6 rounds; the
                    1 <= n_out <= K+1 bound ([LENS] §2.1; [NOTE] "At least one token per
                    loop"); q <= p => accept ([LENS] §2.3); acceptance frequency equals
                    alpha = sum min(p, q) ([LENS] §3.1-3.2, Theorem 3.5 / Cor. 3.6).

Readings of points the pages leave open (each is listed in the design notes):
  * accept test without division: u*q < p equals u < min(1, p/q) whenever q > 0; with
    q = 0 and p > 0 it accepts, with p = q = 0 it rejects (and the row is flagged).
  * strict '<' with u in [0, 1) on a 2**-24 grid ([CANON] listing and [LENS] numpy
    snippet both use random() < min(1, ...)).
  * knob order temperature -> top-k -> top-p -> renormalise; ties at the top-k or top-p
    threshold are all kept; top_k = 0 and top_p = 1 mean "off".
  * inverse CDF: smallest i with C_i > u*S, C the running sum in token-id order,
    S = C_{V-1}.  An empty residual (S = 0 after a rejection) falls back to sampling P_a.
  * temperature and top_p are float32 parameters: their float32 values are used.
  * T = 0 is argmax decoding ([LENS] "How much faster in practice?", the argmax column of
    Table 2, and the practice notes contrasting temperature 0 with 1; [NOTE]
    Recommendation R3 names greedy decoding as the other mode): every processed row is
    one-hot at the largest logit, the lowest token id among equal largest logits.  The
    largest logit survives every top-k and top-p cut, so those knobs change nothing at
    T = 0.  With one-hot rows the rule itself is unchanged: the draft proposes argmax q,
    a draft is accepted iff it is argmax p, and the resample and bonus are argmax p.
"""
import numpy as np

# row_status bits, shared meaning with the library's documented status bits
ST_NONFINITE = 1          # a logit row of this sequence holds NaN or +-Inf: nothing emitted
ST_Q_ZERO = 2             # q(x~_j) == 0 at an evaluated position (total rule still applies)
ST_RESIDUAL_EMPTY = 4     # max(0, p - q) summed to 0 at the first rejection: sampled P_a
ST_KV_OVERFLOW = 8        # the cache could not hold the appended tokens
ST_BAD_TOKEN = 16         # a draft token id outside [0, V): nothing emitted


def f32(x):
    """The float32 value of a scalar parameter, as a Python float."""
    return float(np.float32(x))


def transform(logits, temperature, top_k=0, top_p=1.0):
    """Processed probability row (float64) from one logit row.

    0. T = 0: one-hot at the first index holding the largest logit (argmax decoding).
    1. z = logits / T                          (T > 0, float32 value)
    2. top-k (0 < k < V): z_i -> -inf where z_i < (k-th largest z); ties kept.
    3. s = exp(z - max z) / sum(exp(z - max z)).
    4. top-p (top_p < 1): sort s descending; tau = the value at the first sorted index
       whose running sum reaches top_p; keep s_i >= tau (ties kept); renormalise.
    """
    T = f32(temperature)
    tp = f32(top_p)
    if T == 0.0:
        l = np.asarray(logits, dtype=np.float64)
        s = np.zeros(l.size)
        s[int(np.argmax(l))] = 1.0  # numpy's argmax returns the first maximal index
        return s
    z = np.asarray(logits, dtype=np.float64) / T
    V = z.size
    if 0 < top_k < V:
        kth = np.sort(z)[::-1][top_k - 1]
        z = np.where(z >= kth, z, -np.inf)
    e = np.exp(z - z.max())
    s = e / e.sum()
    if tp < 1.0:
        order = np.argsort(-s, kind="stable")
        run = np.cumsum(s[order])
        reached = np.nonzero(run >= tp)[0]
        if reached.size:
            tau = s[order][reached[0]]
            s = np.where(s >= tau, s, 0.0)
            s = s / s.sum()
    return s


def top_p_threshold_margin(probs_before_top_p, top_p):
    """Distance of top_p from the running sums next to the top-p cut (near-boundary test).

    Returns min over sorted positions i of |exclusive running sum at i - top_p| for the
    tokens on either side of the cut: a membership decision whose margin is below the
    numeric error of the two sides is "near-boundary" and counted, not failed.
    """
    s = np.asarray(probs_before_top_p, dtype=np.float64)
    tp = f32(top_p)
    order = np.argsort(-s, kind="stable")
    run = np.cumsum(s[order])
    excl = run - s[order]
    return float(np.min(np.abs(excl - tp)))


def sample(w, u):
    """Inverse-CDF draw from weights w (need not be normalised) with uniform(s) u.

    C = running sum of w in token-id order, S = C[-1]; returns the smallest i with
    C_i > u*S (vectorised over u).  Returns -1 where S == 0 (the caller decides).
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    S = C[-1]
    u = np.asarray(u, dtype=np.float64)
    if not S > 0.0:
        return np.full(u.shape, -1, dtype=np.int64) if u.ndim else -1
    idx = np.searchsorted(C, u * S, side="right")
    # u*S < S always holds for u <= 1 - 2**-24, so idx < V; keep the documented fallback
    last_pos = int(np.nonzero(w > 0)[0][-1])
    idx = np.where(idx >= w.size, last_pos, idx)
    return idx if u.ndim else int(idx)


def accept_test(p_x, q_x, u):
    """accept <=> u * q(x~) < p(x~)  (vectorised)."""
    return np.asarray(u, np.float64) * np.asarray(q_x, np.float64) < np.asarray(p_x, np.float64)


def accept_resample(P, Q, xt, u_acc, u_res):
    """One sequence row of the rule, walked left to right as the pages state it.

    P: (K+1, V) processed target rows; Q: (K, V) processed draft rows; xt: (K,) draft
    tokens; u_acc: (K,) accept uniforms (purpose 1); u_res: (K+1,) resample / bonus
    uniforms (purpose 2).  Returns (tokens list, n_out, a, status) with a = number of
    accepted drafts.
    """
    P = np.asarray(P, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    K = len(xt)
    V = P.shape[1]
    status = 0
    if any(int(x) < 0 or int(x) >= V for x in xt):
        return [], 0, 0, ST_BAD_TOKEN
    a = K
    for j in range(K):
        x = int(xt[j])
        if Q[j, x] == 0.0:
            status |= ST_Q_ZERO
        if not accept_test(P[j, x], Q[j, x], u_acc[j]):
            a = j
            break
    if a < K:
        r = np.maximum(0.0, P[a] - Q[a])
        y = sample(r, u_res[a])
        if y < 0:
            status |= ST_RESIDUAL_EMPTY
            y = sample(P[a], u_res[a])
    else:
        y = sample(P[K], u_res[K])
    toks = [int(x) for x in xt[:a]] + [int(y)]
    return toks, a + 1, a, status


def accept_resample_logits(p_logits, q_logits, xt, u_acc, u_res, temperature=1.0,
                           top_k=0, top_p=1.0):
    """accept_resample on raw logit rows, applying the knobs to both p and q first.

    A row holding a non-finite logit emits nothing (status ST_NONFINITE).
    """
    p_logits = np.asarray(p_logits)
    q_logits = np.asarray(q_logits)
    if not (np.all(np.isfinite(p_logits)) and np.all(np.isfinite(q_logits))):
        return [], 0, 0, ST_NONFINITE
    P = np.stack([transform(r, temperature, top_k, top_p) for r in p_logits])
    Q = np.stack([transform(r, temperature, top_k, top_p) for r in q_logits])
    return accept_resample(P, Q, xt, u_acc, u_res)


def draft_sample(q_logits_row, u, temperature=1.0, top_k=0, top_p=1.0):
    """x~_j = sample(transform(draft logits at step j), U(purpose 0, j))."""
    return sample(transform(q_logits_row, temperature, top_k, top_p), u)
