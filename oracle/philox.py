"""Philox4x64-10 counter-based generator and the uniforms the sampling rule draws.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Definition followed: Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3" (SC'11), the Philox-4x64 bijection with 10 rounds.  One round maps
the counter (X0, X1, X2, X3) and key (k0, k1) to

    (hi(M0*X0), lo(M0*X0)) , (hi(M1*X2), lo(M1*X2))
    X' = (hi(M1*X2) ^ X1 ^ k0,  lo(M1*X2),  hi(M0*X0) ^ X3 ^ k1,  lo(M0*X0))

and between rounds the key is bumped by the Weyl constants (W0, W1).  The
multipliers and Weyl constants are the ones the paper publishes for 4x64.

Uniform mapping (our reading; the pages only say "Philox uniforms keyed on (seed,
round, position)"): key = (seed, 0), counter = (round, j, b, purpose), and
u = (word0 >> 40) * 2**-24, i.e. the top 24 bits of the first output word, so u
lies on the grid {0, 2**-24, ..., 1 - 2**-24}.  Purposes: 0 = draft sample,
1 = accept test, 2 = resample / bonus sample.

Pinned by tests/test_oracle_philox.py against ``numpy.random.Philox`` (an
independent implementation of the same published generator).
"""
import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
ROUNDS = 10

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_RESAMPLE = 2

_MASK64 = (1 << 64) - 1


def philox4x64_scalar(counter, key, rounds=ROUNDS):
    """Philox4x64 on Python ints (used on small cases and to check the vector form)."""
    x0, x1, x2, x3 = (int(c) & _MASK64 for c in counter)
    k0, k1 = (int(k) & _MASK64 for k in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + W0) & _MASK64
            k1 = (k1 + W1) & _MASK64
        p0 = M0 * x0
        p1 = M1 * x2
        hi0, lo0 = p0 >> 64, p0 & _MASK64
        hi1, lo1 = p1 >> 64, p1 & _MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return (x0, x1, x2, x3)


def _mulhilo64(a, b):
    """Full 64x64 -> 128 product of uint64 arrays, via 32-bit limbs (numpy wraps mod 2**64)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a_lo, a_hi = a & m32, a >> s32
    b_lo, b_hi = b & m32, b >> s32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> s32) + (lh & m32) + (hl & m32)
    lo = (ll & m32) | ((mid & m32) << s32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, lo


def philox4x64(c0, c1, c2, c3, k0, k1, rounds=ROUNDS):
    """Vectorised Philox4x64 over broadcastable uint64 arrays; returns four uint64 arrays."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    kk0 = np.asarray(k0, dtype=np.uint64)
    kk1 = np.asarray(k1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for r in range(rounds):
            if r > 0:
                kk0 = kk0 + np.uint64(W0)
                kk1 = kk1 + np.uint64(W1)
            hi0, lo0 = _mulhilo64(np.uint64(M0), x0)
            hi1, lo1 = _mulhilo64(np.uint64(M1), x2)
            x0, x1, x2, x3 = hi1 ^ x1 ^ kk0, lo1, hi0 ^ x3 ^ kk1, lo0
    return x0, x1, x2, x3


def uniform(seed, rnd, j, b, purpose):
    """u in [0, 1 - 2**-24] on a 2**-24 grid, for counter (rnd, j, b, purpose), key (seed, 0).

    Arguments broadcast (numpy arrays of non-negative ints).  Returns float64.
    """
    w0, _, _, _ = philox4x64(rnd, j, b, purpose, seed, 0)
    return (w0 >> np.uint64(40)).astype(np.float64) * 2.0 ** -24
