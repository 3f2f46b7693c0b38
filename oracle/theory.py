"""Closed forms the pages state for speculative sampling.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

  acceptance_rate      alpha = sum_x min(p(x), q(x))      [LENS] §3.1-3.2 (Theorem 3.5, Cor. 3.6)
  expected_tokens_iid  (1 - alpha**(K+1)) / (1 - alpha)    [ZSM] "How much faster"; [LENS] §3.1
  expected_tokens_rows sum_{j=0..K} prod_{i<j} beta_i      (the same count without the i.i.d.
                                                            assumption [LENS] "Limitations" names)
  walltime_improvement (1 - alpha**(g+1)) / ((1 - alpha)(g c + 1))   [LENS] §3.3

Pinned by tests/test_oracle_theory.py: the value [LENS] §3.1 quotes from Table 1
(alpha = 0.8, gamma = 5 -> 3.69x), the K -> limits, and Monte Carlo over the oracle's
own rule.  [ZSM] "How much faster" quotes ~2.8 tokens at alpha = 0.8, K = 4; the formula
printed next to it gives 3.3616, so that number is not used as a pin.
"""
import numpy as np


def acceptance_rate(p, q):
    """beta for one position: sum_x min(p(x), q(x))."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def expected_tokens_iid(alpha, K):
    """Expected tokens emitted per target call when every beta equals alpha."""
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def expected_tokens_rows(betas):
    """Expected tokens emitted per target call given per-position acceptance probabilities.

    P(a >= j) = prod_{i<j} beta_i (drafts of different positions drawn independently),
    E[n_out] = E[a + 1] = sum_{j=0..K} P(a >= j).
    """
    total, run = 1.0, 1.0
    for b in betas:
        run *= float(b)
        total += run
    return total


def walltime_improvement(alpha, gamma, c):
    """Expected wall-time improvement factor with draft/target cost ratio c."""
    return expected_tokens_iid(alpha, gamma) / (gamma * c + 1.0)
