"""Pins of the oracle's transformer forward.

The pages fix only that one target call scores K+1 positions with the weights and the
KV cache read once ([ZSM] "One pass can score many tokens"; [LENS] §2.1 step 2 and
§3.4).  The layer definition is our own spec (parity unpinned with respect to the
pages); these tests pin it by structure and by independent library routines.
"""
import math

import numpy as np
import pytest
import torch

from oracle import model
from speculative_decoding_forward_amd import synth


def micro(dtype="f32", kind="gelu"):
    return synth.ModelShape(n_layers=2, d_model=32, n_heads=2, head_dim=16, d_ffn=64,
                            vocab=50, ffn_kind=kind, dtype=dtype)


def weights(shape, seed=0):
    W = synth.weights_to_numpy(synth.make_weights(shape, seed=seed))
    # non-unit norm gains so a dropped gain would show
    rng = np.random.default_rng(seed + 100)
    for n in W:
        if n.split(".")[-1].startswith("norm"):
            W[n] = (1.0 + 0.1 * rng.standard_normal(W[n].shape)).astype(np.float32)
    return W


CASES = [("f32", "gelu"), ("f32", "swiglu"), ("bf16", "gelu"), ("bf16", "swiglu")]


@pytest.mark.parametrize("dtype,kind", CASES)
def test_verify_equals_sequential_single_token_calls(dtype, kind):
    """K+1 positions in one call give the same logits as K+1 one-token calls."""
    s = micro(dtype, kind)
    W = weights(s)
    rng = np.random.default_rng(1)
    ctx = rng.integers(0, s.vocab, (2, 7))
    new = rng.integers(0, s.vocab, (2, 6))
    c1 = model.KVCache(s, 2, 32)
    model.forward(s, W, c1, ctx)
    c2 = c1.copy()
    big = model.forward(s, W, c1, new)
    seq = np.concatenate([model.forward(s, W, c2, new[:, j:j + 1]) for j in range(6)], axis=1)
    np.testing.assert_allclose(big, seq, rtol=0, atol=1e-12)
    assert np.array_equal(c1.len, c2.len) and np.array_equal(c1.len, [13, 13])


@pytest.mark.parametrize("dtype,kind", CASES)
def test_cached_equals_full_recompute(dtype, kind):
    s = micro(dtype, kind)
    W = weights(s, seed=2)
    rng = np.random.default_rng(2)
    toks = rng.integers(0, s.vocab, (1, 12))
    c1 = model.KVCache(s, 1, 16)
    model.forward(s, W, c1, toks[:, :8])
    inc = model.forward(s, W, c1, toks[:, 8:])
    c2 = model.KVCache(s, 1, 16)
    full = model.forward(s, W, c2, toks)
    np.testing.assert_allclose(inc, full[:, 8:], rtol=0, atol=1e-12)


def test_causality():
    s = micro("bf16", "swiglu")
    W = weights(s, seed=3)
    rng = np.random.default_rng(3)
    toks = rng.integers(0, s.vocab, (1, 10))
    alt = toks.copy()
    alt[0, 6:] = (alt[0, 6:] + 7) % s.vocab
    a = model.forward(s, W, model.KVCache(s, 1, 16), toks)
    b = model.forward(s, W, model.KVCache(s, 1, 16), alt)
    np.testing.assert_array_equal(a[:, :6], b[:, :6])
    assert np.abs(a[:, 6:] - b[:, 6:]).max() > 1e-3


def test_rollback_then_reappend_equals_fresh():
    s = micro("bf16", "gelu")
    W = weights(s, seed=4)
    rng = np.random.default_rng(4)
    ctx = rng.integers(0, s.vocab, (2, 5))
    drafts = rng.integers(0, s.vocab, (2, 4))
    c = model.KVCache(s, 2, 20)
    model.forward(s, W, c, ctx)
    model.forward(s, W, c, drafts)            # row 0 keeps 1 draft, row 1 keeps none
    c.rollback([6, 5])
    nxt = rng.integers(0, s.vocab, (2, 3))
    got = model.forward(s, W, c, nxt, n_tok=[3, 2])
    assert np.array_equal(c.len, [9, 7])
    fresh = model.KVCache(s, 2, 20)
    seq0 = np.concatenate([ctx[0], drafts[0, :1], nxt[0]])[None]
    seq1 = np.concatenate([ctx[1], nxt[1, :2]])[None]
    f0 = model.forward(s, W, model.KVCache(s, 1, 20), seq0)
    f1 = model.forward(s, W, model.KVCache(s, 1, 20), seq1)
    np.testing.assert_allclose(got[0], f0[0, 6:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1, :2], f1[0, 5:], rtol=0, atol=1e-12)


def test_ragged_rows_and_padding_rows_untouched():
    s = micro("f32", "gelu")
    W = weights(s, seed=5)
    rng = np.random.default_rng(5)
    toks = rng.integers(0, s.vocab, (3, 4))
    c = model.KVCache(s, 3, 6)
    out = model.forward(s, W, c, toks, n_tok=[4, 1, 0])
    assert np.array_equal(c.len, [4, 1, 0])
    assert np.all(out[1, 1:] == 0) and np.all(out[2] == 0)
    single = model.forward(s, W, model.KVCache(s, 1, 8), toks[1:2, :1])
    np.testing.assert_allclose(out[1, :1], single[0], rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        model.forward(s, W, c, toks, n_tok=[4, 1, 0])


# ------------------------------------------------------------------ layer pieces ----

def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(6)
    n, H, hd, P = 5, 3, 16, 20
    pos = np.arange(P - n, P)
    q = rng.standard_normal((n, H, hd))
    Kc = rng.standard_normal((H, P, hd))
    Vc = rng.standard_normal((H, P, hd))
    got = model.attend(q, Kc, Vc, pos)
    mask = torch.tensor(np.arange(P)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q).permute(1, 0, 2), torch.tensor(Kc), torch.tensor(Vc), attn_mask=mask)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_rmsnorm_closed_form():
    x = np.array([[3.0, -4.0, 0.0, 0.0]])
    g = np.array([1.0, 2.0, 1.0, 1.0])
    y = model.rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(y, [[3 / 2.5, -8 / 2.5, 0, 0]], rtol=1e-15)
    rng = np.random.default_rng(7)
    z = rng.standard_normal((4, 64)) * 5
    y = model.rmsnorm(z, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)


def test_normed_input_closed_form():
    """The input of a normalised product is bf16(RMSNorm(x) * g): RMSNorm of [3, -4, 0, 0]
    (rms 2.5) with gains [1, 2, 1, 1] is [1.2, -3.2, 0, 0], which rounds to the bf16
    values 1.203125 and -3.203125 (8 significant bits; 1.2 = 1.0011001...b)."""
    x = np.array([[3.0, -4.0, 0.0, 0.0]])
    g = np.array([1.0, 2.0, 1.0, 1.0])
    h = model.normed_input(x, g, 0.0, model.round_bf16)
    np.testing.assert_array_equal(h, [[1.203125, -3.203125, 0.0, 0.0]])
    # the row factor scales before the one rounding: a row and the same row times 2^k
    # (any k) normalise to the same bf16 input
    rng = np.random.default_rng(10)
    z = rng.standard_normal((3, 64))
    np.testing.assert_array_equal(model.normed_input(z, np.ones(64), 0.0, model.round_bf16),
                                  model.normed_input(z * 2.0 ** 37, np.ones(64), 0.0,
                                                     model.round_bf16))


def test_forward_is_the_composition_of_its_halves():
    """forward() = embedding -> (attention half, FFN half) per layer -> LM head, row by
    row; the halves fed the same rows reproduce its logits and its cache entries."""
    s = micro("bf16", "swiglu")
    W = weights(s, seed=11)
    rng = np.random.default_rng(11)
    ctx = rng.integers(0, s.vocab, (1, 5))
    new = rng.integers(0, s.vocab, (1, 3))
    c1 = model.KVCache(s, 1, 16)
    model.forward(s, W, c1, ctx)
    c2 = c1.copy()
    got = model.forward(s, W, c1, new)
    x = W["embed"][new[0]].astype(np.float64)
    pos = 5 + np.arange(3)
    for l in range(s.n_layers):
        x = model.ffn_half(s, W, l, model.attention_half(s, W, c2, l, 0, x, pos))
    np.testing.assert_array_equal(model.lm_head(s, W, x), got[0])
    for l in range(s.n_layers):
        np.testing.assert_array_equal(c1.k[l][0, :, :8], c2.k[l][0, :, :8])
        np.testing.assert_array_equal(c1.v[l][0, :, :8], c2.v[l][0, :, :8])


def test_rope_properties():
    rng = np.random.default_rng(8)
    hd = 32
    t = rng.standard_normal((6, 2, hd))
    pos = np.array([0, 1, 5, 17, 300, 2047])
    r = model.rope(t, pos, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(t, axis=-1),
                               rtol=1e-13)
    np.testing.assert_allclose(r[0], t[0], rtol=0, atol=0)        # position 0: identity
    # q_m . k_n depends only on m - n
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    d1 = np.sum(model.rope(q, [10], 1e4) * model.rope(k, [3], 1e4))
    d2 = np.sum(model.rope(q, [107], 1e4) * model.rope(k, [100], 1e4))
    assert abs(d1 - d2) < 1e-12
    # pair (i, i + hd/2) rotates by pos * theta^(-2i/hd)
    e = np.zeros((1, 1, hd)); e[0, 0, 3] = 1.0
    ang = 7 * 10000.0 ** (-6 / hd)
    rr = model.rope(e, [7], 10000.0)
    assert abs(rr[0, 0, 3] - math.cos(ang)) < 1e-15 and abs(rr[0, 0, 3 + hd // 2] - math.sin(ang)) < 1e-15


def test_activations_match_torch():
    x = np.linspace(-6, 6, 1001)
    np.testing.assert_allclose(model.gelu(x), torch.nn.functional.gelu(
        torch.tensor(x), approximate="none").numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(model.silu(x), torch.nn.functional.silu(
        torch.tensor(x)).numpy(), rtol=1e-12, atol=1e-15)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, 1.0, -1.0, 1 + 2**-8, 1 + 3 * 2**-8, 2.0**-130, 3.0e38]])
    x32 = x.astype(np.float32)
    ref = torch.tensor(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(model.round_bf16(x32.astype(np.float64)), ref)
