"""Pins of the oracle's closed forms: printed page values, limits and Monte Carlo."""
import json
import os

import numpy as np

from oracle import theory

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "theory_values.json")


def test_table1_value_from_the_pages():
    g = json.load(open(GOLDEN))["table1_speed_factor"]
    v = theory.walltime_improvement(g["alpha"], g["gamma"], g["c"])
    assert round(v, g["decimals"]) == g["value"]
    assert abs(v - 3.68928) < 1e-9


def test_formula_limits():
    # alpha -> 1: every draft accepted, K+1 tokens; alpha = 0: one token per call
    for K in range(1, 9):
        assert theory.expected_tokens_iid(0.0, K) == 1.0
        assert theory.expected_tokens_iid(1.0, K) == K + 1
        assert abs(theory.expected_tokens_iid(1 - 1e-9, K) - (K + 1)) < 1e-6
    # K -> infinity: geometric mean run 1 / (1 - alpha)
    assert abs(theory.expected_tokens_iid(0.8, 400) - 5.0) < 1e-9
    # the printed formula at alpha = 0.8, K = 4 (the page's "about 2.8" disagrees with it)
    assert abs(theory.expected_tokens_iid(0.8, 4) - 3.3616) < 1e-12


def test_rows_form_reduces_to_iid_form():
    for a in (0.1, 0.5, 0.8, 0.95):
        for K in (1, 3, 5, 7):
            assert abs(theory.expected_tokens_rows([a] * K) -
                       theory.expected_tokens_iid(a, K)) < 1e-12


def test_bounds_of_tokens_per_call():
    g = json.load(open(GOLDEN))["tokens_per_call_bounds"]
    rng = np.random.default_rng(0)
    for _ in range(100):
        K = int(rng.integers(1, 9))
        b = rng.random(K)
        e = theory.expected_tokens_rows(b)
        assert g["min"] <= e <= K + g["max_minus_gamma"]


def test_speedup_exists_iff_alpha_above_c():
    # Cor. 3.9 (ta-paperlens §3.3): some gamma gives improvement > 1 iff alpha > c
    for alpha in (0.2, 0.5, 0.8):
        for c in (0.05, 0.3, 0.6, 0.9):
            best = max(theory.walltime_improvement(alpha, g, c) for g in range(1, 60))
            assert (best > 1.0) == (alpha > c)


def test_acceptance_rate_overlap():
    p = np.array([0.5, 0.25, 0.25, 0.0])
    q = np.array([0.25, 0.25, 0.25, 0.25])
    assert theory.acceptance_rate(p, q) == 0.75
    assert theory.acceptance_rate(p, p) == 1.0
    assert theory.acceptance_rate([1, 0], [0, 1]) == 0.0
