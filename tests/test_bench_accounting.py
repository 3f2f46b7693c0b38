"""The bench's byte accounting (every roofline fraction it reports rests on it) against an
independent layer-by-layer count from the model shapes, and its wall-time formula against
the oracle's pinned one.

Algorithmic bytes of one verify call: every weight matrix once (the embedding table is not
streamed: only the rows of the call's tokens), the norm gains (fp32), the gathered
embedding rows, the KV cache read over the context plus the new positions and written for
the new positions, and the fp32 logits.
"""
import numpy as np
import pytest

import bench
from oracle import theory
from speculative_decoding_forward_amd import synth


def layer_by_layer_verify_bytes(shape, B, K, ctx):
    d, F, V, L, e = shape.d_model, shape.d_ffn, shape.vocab, shape.n_layers, shape.elt_bytes()
    M = B * (K + 1)
    ffn_mats = 3 if shape.ffn_kind == "swiglu" else 2
    per_layer = (3 * d * d + d * d + ffn_mats * d * F) * e + 2 * d * 4   # matrices + 2 gains
    weights = L * per_layer + V * d * e + d * 4                        # + LM head + final gain
    kv_read = B * L * 2 * (ctx + K + 1) * d * e
    kv_write = B * L * 2 * (K + 1) * d * e
    return weights + M * d * e + kv_read + kv_write + M * V * 4


@pytest.mark.parametrize("wl_name,B,K,lo,hi", [
    ("7b", 1, 5, 14.29e9, 14.31e9),     # the headline configuration's stated 14.29-14.30 GB
    ("7b", 8, 5, 21.84e9, 21.88e9),     # its B = 8 figure, 21.84-21.88 GB
    ("70b", 1, 4, 132.0e9, 132.2e9),    # the 70B shape's 132.09 GB
    ("small", 1, 4, 2.64e9, 2.66e9),    # the small model's 2.65 GB
    ("tiny", 1, 4, 2.1e6, 2.3e6),       # the tiny model's 2.2 MB (fp32)
])
def test_verify_bytes(wl_name, B, K, lo, hi):
    wl = synth.WORKLOADS[wl_name]
    got = bench.verify_bytes(wl.target, B, K, [wl.ctx] * B)
    ref = layer_by_layer_verify_bytes(wl.target, B, K, wl.ctx)
    assert got == ref
    assert lo <= got <= hi, got


@pytest.mark.parametrize("wl_name,R", [("7b", 6), ("7b", 48), ("70b", 5), ("small", 5)])
def test_gemm_bytes_cover_every_streamed_weight_once(wl_name, R):
    """The GEMM launches' algorithmic bytes: the weight part equals every matrix of the
    layers plus the LM head once, and the rest is activation traffic that grows with R."""
    shape = synth.WORKLOADS[wl_name].target
    d, F, V, L, e = shape.d_model, shape.d_ffn, shape.vocab, shape.n_layers, shape.elt_bytes()
    ffn_mats = 3 if shape.ffn_kind == "swiglu" else 2
    weights = L * (4 * d * d + ffn_mats * d * F) * e + V * d * e
    total, n = bench.gemm_bytes_per_verify(shape, R)
    assert n == 4 * L + 1
    total0, _ = bench.gemm_bytes_per_verify(shape, 0)
    assert total0 == weights
    assert total > total0 and total - total0 < 0.05 * weights


@pytest.mark.parametrize("alpha,K,c", [(0.8, 5, 0.0), (0.26, 5, 0.27), (0.6, 3, 0.05),
                                       (0.29, 4, 0.035)])
def test_speedup_formula_matches_oracle(alpha, K, c):
    assert bench.speedup_formula(alpha, K, c) == pytest.approx(
        theory.walltime_improvement(alpha, K, c), rel=1e-12)



def test_recorded_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    """The line's `traffic` comes from the committed counter summary only while the GEMM
    sources hash to the value recorded with it; otherwise (other sources, no summary) it
    is None, never a stale figure."""
    summary = tmp_path / "traffic.md"
    current = bench.gemm_source_hash()
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.recorded_traffic() is None                       # no summary
    summary.write_text(f"traffic_bytes_per_launch: 123456\nkernel_sources_sha256: {current}\n")
    assert bench.recorded_traffic() == 123456.0
    other = "0" * 16 if current != "0" * 16 else "1" * 16
    summary.write_text(f"traffic_bytes_per_launch: 123456\nkernel_sources_sha256: {other}\n")
    assert bench.recorded_traffic() is None                       # taken on other sources
    summary.write_text(f"kernel_sources_sha256: {current}\n")
    assert bench.recorded_traffic() is None                       # no figure
