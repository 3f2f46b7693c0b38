"""GPU parity of spec_verify_forward (the verify pass) against the oracle forward.

Tolerances: logits within 1e-4 abs for fp32 models and 1e-2 abs (mean 1e-3) for bf16
models (fp32 accumulation).  Cache contents of the appended positions are compared too.
Full-depth parity, half-layer by half-layer, is in tests/test_gpu_layers.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import model as omodel
from speculative_decoding_forward_amd import binding, synth

from helpers import DEV, to_dev
from helpers_trace import check_head, check_layers, end_to_end, traced_verify

pytestmark = pytest.mark.gpu


def bf16_micro(kind, hd=128, L=2, d=256, F=512, V=1024):
    return synth.ModelShape(n_layers=L, d_model=d, n_heads=d // hd, head_dim=hd, d_ffn=F,
                            vocab=V, ffn_kind=kind, dtype="bf16")


def setup(shape, seed=0, model_id=synth.TARGET):
    Wd = synth.make_weights(shape, seed=seed, model_id=model_id, device=DEV)
    Wn = synth.weights_to_numpy(Wd)
    return binding.Model(shape, Wd), Wn


def gpu_forward(m, kv, tokens, n_tok=None, max_len=None):
    B, M = tokens.shape
    ws = m.workspace(B, M, kv.max_len)
    logits = torch.full((B, M, m.shape.vocab), 7.0, dtype=torch.float32, device=DEV)
    st = torch.zeros(B, dtype=torch.int32, device=DEV)
    nt = None if n_tok is None else to_dev(np.asarray(n_tok, np.int32))
    binding.verify_forward(m, kv, to_dev(tokens.astype(np.int32)), logits, ws, n_tok=nt,
                           row_status=st)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), st.cpu().numpy()


def prefill_both(m, kv, Wn, shape, ctx, chunk, oc):
    """Feed ctx[:, :n] through the GPU in chunks and through the oracle."""
    B, n = ctx.shape
    for s in range(0, n, chunk):
        gpu_forward(m, kv, ctx[:, s:s + chunk])
    omodel.forward(shape, Wn, oc, ctx)


@pytest.mark.parametrize("name", ["tiny_target", "tiny_draft"])
def test_fp32_tiny_prefill_then_verify(name):
    wl = synth.WORKLOADS["tiny"]
    shape = wl.target if name == "tiny_target" else wl.draft
    m, Wn = setup(shape, model_id=synth.TARGET if name == "tiny_target" else synth.DRAFT)
    B, max_len = 2, 96
    kv = binding.KVCache(shape, B, max_len)
    oc = omodel.KVCache(shape, B, max_len)
    ctx = synth.context_ids(0, B, wl.ctx - 1, shape.vocab)
    prefill_both(m, kv, Wn, shape, ctx, 7, oc)
    assert np.array_equal(kv.len.cpu().numpy(), oc.len)
    new = synth.context_ids(1, B, wl.K + 1, shape.vocab)
    g, st = gpu_forward(m, kv, new)
    o = omodel.forward(shape, Wn, oc, new)
    err = np.abs(g - o).max()
    print(f"{name}: max |logit diff| = {err:.3e}")
    assert err <= 1e-4
    assert np.all(st == 0)
    assert np.array_equal(kv.len.cpu().numpy(), oc.len)
    # cache contents of every written position
    data = kv.export(max_len).cpu().numpy()
    for l in range(shape.n_layers):
        for b in range(B):
            n = oc.len[b]
            np.testing.assert_allclose(data[l, b, 0, :, :n], oc.k[l][b, :, :n], atol=1e-5)
            np.testing.assert_allclose(data[l, b, 1, :, :n], oc.v[l][b, :, :n], atol=1e-5)


@pytest.mark.parametrize("kind,hd", [("swiglu", 128), ("gelu", 128), ("swiglu", 64)])
def test_bf16_micro_ragged(kind, hd):
    """bf16 with cache lengths crossing several 64-position attention chunks, ragged
    rows (n_tok 6, 3, 0) and a prefill chunk of 64 tokens."""
    shape = bf16_micro(kind, hd=hd)
    m, Wn = setup(shape, seed=3)
    B, max_len = 3, 256
    kv = binding.KVCache(shape, B, max_len)
    oc = omodel.KVCache(shape, B, max_len)
    ctx = synth.context_ids(2, B, 150, shape.vocab)
    prefill_both(m, kv, Wn, shape, ctx, 64, oc)
    new = synth.context_ids(3, B, 6, shape.vocab)
    n_tok = [6, 3, 0]
    g, st = gpu_forward(m, kv, new, n_tok=n_tok)
    o = omodel.forward(shape, Wn, oc, new, n_tok=n_tok)
    for b in range(B):
        n = n_tok[b]
        if n:
            err = np.abs(g[b, :n] - o[b, :n]).max()
            print(f"{kind} hd={hd} row {b}: max |logit diff| = {err:.3e}")
            assert err <= 1e-2      # two narrow layers: within 1e-2 outright
        assert np.all(g[b, n:] == 0)
    assert np.array_equal(kv.len.cpu().numpy(), oc.len)
    data = kv.export(max_len).float().cpu().numpy()
    for b in range(B):
        s0, n = 150, n_tok[b]
        if n == 0:
            continue
        for l in range(shape.n_layers):
            kd = data[l, b, 0, :, s0:s0 + n]
            ko = oc.k[l][b, :, s0:s0 + n]
            assert np.abs(kd - ko).max() <= 2 ** -7 * max(1.0, np.abs(ko).max())


@pytest.mark.parametrize("M", [1, 6])
def test_unwritten_cache_positions_are_ignored(M):
    """Positions at or past a row's length hold whatever the caller's arena held: with
    the arena first filled with NaN bytes, a verify pass (one token, and K+1 = 6) gives
    bitwise the logits and appended entries of the same pass over a zero-filled arena.
    The context ends inside a 32-key block, so the last block read straddles the end."""
    shape = bf16_micro("gelu", hd=128, d=512)
    m, _ = setup(shape, seed=7)
    B, max_len, n = 2, 160, 77
    fill = synth.kv_fill(shape, B, max_len, n, seed=7, device=DEV)
    new = synth.context_ids(8, B, M, shape.vocab)
    res = []
    for word in (0, -1):  # 0xFFFF is a NaN in bf16
        kv = binding.KVCache(shape, B, max_len)
        kv.data().view(torch.int16).fill_(word)  # the K/V elements only
        kv.import_(fill[:, :, :, :, :n].contiguous())
        kv.len.fill_(n)
        g, st = gpu_forward(m, kv, new)
        assert np.all(st == 0) and np.all(np.isfinite(g))
        res.append((g, kv.export(n + M).float().cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])


def test_overflow_and_bad_tokens_flagged():
    shape = bf16_micro("swiglu")
    m, Wn = setup(shape, seed=4)
    B, max_len = 3, 40
    kv = binding.KVCache(shape, B, max_len)
    ctx = synth.context_ids(4, B, 36, shape.vocab)
    gpu_forward(m, kv, ctx)
    new = synth.context_ids(5, B, 4, shape.vocab)
    new[2, 1] = shape.vocab + 3
    g, st = gpu_forward(m, kv, new, n_tok=[4, 5 - 1, 4])
    assert np.all(st[:2] == 0) and st[2] & binding.ROW_BAD_TOKEN
    # now every row is full: a further token overflows and is skipped
    g, st = gpu_forward(m, kv, new[:, :1])
    assert np.all(st & binding.ROW_KV_OVERFLOW)
    assert np.all(g == 0)
    assert np.array_equal(kv.len.cpu().numpy(), [40, 40, 40])


def test_rollback():
    shape = bf16_micro("gelu")
    m, _ = setup(shape, seed=5)
    kv = binding.KVCache(shape, 2, 64)
    gpu_forward(m, kv, synth.context_ids(6, 2, 10, shape.vocab))
    kv.rollback(to_dev(np.array([4, 20], np.int32)))
    torch.cuda.synchronize()
    assert np.array_equal(kv.len.cpu().numpy(), [4, 10])


@pytest.mark.parametrize("wl_name,B,K", [("small", 1, 4), ("7b", 1, 5), ("7b", 8, 5),
                                         ("small", 8, 7), ("7b", 8, 7), ("7b", 8, 3),
                                         ("7b", 5, 6), ("70b", 1, 4), ("7b", 16, 4),
                                         ("small", 12, 7), ("7b", 16, 7), ("70b", 16, 4)])
def test_full_width_two_layers(wl_name, B, K):
    """Full-width layers (d, F, H, V and context of the workload) on the first two
    layers of the target, teacher-forced half by half (tests/helpers_trace.py), with the
    rows' cache lengths staggered by 7 positions.  Rows 6 and 5 take the one-row-tile GEMM
    that forms its normalised input itself; 32, 35 (a ragged last row tile), 48 and 64
    rows the normalise pass and the K-outer GEMM with two to four row tiles where a
    workgroup owns several column tiles, else the tile-at-a-time one; 80, 96 and 128 rows
    split the normalised products into row blocks of at most 64 (64 + 16, 64 + 32, 64 + 64)
    that read the weights with ordinary loads, side by side on one XCD (the 70B shape's 80
    rows at d = 8192 among them), and run the residual products split by wave slot over
    all 5, 6 or 8 row tiles at once."""
    wl = synth.WORKLOADS[wl_name]
    shape = dataclasses.replace(wl.target, n_layers=2)
    t = traced_verify(shape, B, K + 1, [wl.ctx - 7 * b for b in range(B)], seed=0)
    check_layers(t, [0, 1])
    check_head(t)
    end_to_end(t)


@pytest.mark.parametrize("B,n_in", [(1, 2), (1, 1), (2, 1)])
def test_draft_steps_match_oracle(B, n_in):
    """Draft steps through the C ABI at the 7B draft's full width (2 layers, context
    2048): step 0 (n_in pending tokens at two rows; one pending token leaves a padding
    row) and step 1.  Their logits are bitwise those of the traced verify entry point over
    the same tokens and cache, whose every half-layer and LM head are checked against the
    oracle teacher-forced."""
    wl = synth.WORKLOADS["7b"]
    shape = dataclasses.replace(wl.draft, n_layers=2)
    m, _ = setup(shape, seed=3, model_id=synth.DRAFT)
    K, V = 2, shape.vocab
    max_len = wl.ctx + 4
    kv = binding.KVCache(shape, B, max_len)
    fill = synth.kv_fill(shape, B, max_len, wl.ctx, seed=3, model_id=synth.DRAFT, device=DEV)
    kv.import_(fill)
    kv.len.fill_(wl.ctx)
    toks = synth.context_ids(11, B, 2, V)
    in_np = np.full((B, 2), -1, np.int32)
    in_np[:, :n_in] = toks[:, :n_in]
    in_tok, n_in_t = to_dev(in_np), to_dev(np.full(B, n_in, np.int32))
    x_tilde = torch.zeros((B, K), dtype=torch.int32, device=DEV)
    q_logits = torch.zeros((B, K, V), dtype=torch.float32, device=DEV)
    ws = m.workspace(B, 2, max_len)
    for step in range(K):
        binding.draft_step(m, kv, in_tok, n_in_t, step, (0.8, 0, 0.95), 7, 0, x_tilde,
                           q_logits, ws)
    torch.cuda.synchronize()
    assert np.array_equal(kv.len.cpu().numpy(), [wl.ctx + n_in + 1] * B)
    seq = np.concatenate([toks[:, :n_in], x_tilde.cpu().numpy()[:, :1]], axis=1)
    g = q_logits.cpu().numpy()
    # the same tokens through the traced verify entry point
    t = traced_verify(shape, B, n_in + 1, [wl.ctx] * B, seed=3, model_id=synth.DRAFT,
                      tokens=seq)
    assert np.array_equal(g[:, 0], t.logits[:, n_in - 1])
    assert np.array_equal(g[:, 1], t.logits[:, n_in])
    check_layers(t, [0, 1])
    check_head(t)


@pytest.mark.parametrize("wl_name,B,K", [("small", 1, None), ("7b", 1, None), ("7b", 8, None),
                                         ("7b", 8, 3), ("7b", 8, 7), ("small", 8, 5),
                                         ("7b", 16, 4), ("7b", 16, 7)])
def test_verify_equals_single_token_calls_bitwise(wl_name, B, K):
    """At full size: one call over K+1 positions gives bitwise the logits of K+1
    one-token calls (the premise of the verify pass), and the appended cache entries
    are bitwise equal; repeating the call is bitwise deterministic.  At B = 8 the verify
    rows span 2, 3 and 4 row tiles (32, 48 and 64 rows), where the residual products run
    split by wave slot over four-tile workgroups (8 rows of one-token calls: one row tile,
    tile at a time); the small model's residual products have 128 tiles (32 groups).  At
    B = 16 (80 and 128 rows) the residual products take all 5 or 8 row tiles in one pass
    and the other products two row blocks (16 rows of one-token calls: one row tile)."""
    wl = synth.WORKLOADS[wl_name]
    K = K or wl.K
    shape = wl.target
    m, _ = (binding.Model(shape, synth.make_weights(shape, seed=0, device=DEV)), None)
    max_len = wl.ctx + K + 1
    fill = synth.kv_fill(shape, B, max_len, wl.ctx, seed=0, device=DEV)
    new = synth.context_ids(9, B, K + 1, shape.vocab)
    kv1 = binding.KVCache(shape, B, max_len)
    kv1.import_(fill)
    kv1.len.fill_(wl.ctx)
    g1, st1 = gpu_forward(m, kv1, new)
    kv2 = binding.KVCache(shape, B, max_len)
    kv2.import_(fill)
    kv2.len.fill_(wl.ctx)
    g2 = np.concatenate([gpu_forward(m, kv2, new[:, j:j + 1])[0] for j in range(K + 1)], axis=1)
    assert np.array_equal(g1, g2)
    assert torch.equal(kv1.export(max_len), kv2.export(max_len))
    kv3 = binding.KVCache(shape, B, max_len)
    kv3.import_(fill)
    kv3.len.fill_(wl.ctx)
    g3, _ = gpu_forward(m, kv3, new)
    assert np.array_equal(g1, g3)
    # causality: changing the last token leaves earlier rows bitwise unchanged
    alt = new.copy()
    alt[:, -1] = (alt[:, -1] + 1) % shape.vocab
    kv3.len.fill_(wl.ctx)
    g4, _ = gpu_forward(m, kv3, alt)
    assert np.array_equal(g1[:, :K], g4[:, :K])
    assert not np.array_equal(g1[:, K], g4[:, K])


@pytest.mark.parametrize("dtype,hd,max_len", [("bf16", 128, 100), ("bf16", 64, 64), ("f32", 32, 40)])
def test_kv_import_export_roundtrip(dtype, hd, max_len):
    """Natural-order positions written with spec_kv_import read back unchanged with
    spec_kv_export (bf16 caches store them in the attention's packed order), and
    positions past the imported range are left alone."""
    shape = synth.ModelShape(n_layers=2, d_model=2 * hd, n_heads=2, head_dim=hd, d_ffn=256,
                             vocab=64, ffn_kind="gelu", dtype=dtype)
    B = 3
    kv = binding.KVCache(shape, B, max_len)
    full = synth.kv_fill(shape, B, max_len, max_len, seed=5, device=DEV)
    kv.import_(full)
    assert torch.equal(kv.export(max_len), full)
    part = synth.kv_fill(shape, B, max_len, max_len, seed=6, device=DEV)
    n = max_len // 2 + 1
    kv.import_(part[:, :, :, :, :n].contiguous())
    got = kv.export(max_len)
    assert torch.equal(got[:, :, :, :, :n], part[:, :, :, :, :n])
    assert torch.equal(got[:, :, :, :, n:], full[:, :, :, :, n:])


def test_draft_step_flags_non_finite_rows():
    """A draft step whose logits are not all finite (a NaN planted in row 1's cache at a
    valid position) sets SPEC_ROW_NONFINITE for that row only and emits the placeholder
    token 0 for it; the other row samples as usual."""
    shape = bf16_micro("swiglu")
    m, _ = setup(shape, seed=8, model_id=synth.DRAFT)
    B, max_len, n = 2, 64, 40
    fill = synth.kv_fill(shape, B, max_len, n, seed=8, device=DEV)
    fill[0, 1, 1, 0, 5, :] = float("nan")          # layer 0, row 1, V, head 0, position 5
    kv = binding.KVCache(shape, B, max_len)
    kv.import_(fill)
    kv.len.fill_(n)
    K, V = 2, shape.vocab
    in_tok = to_dev(np.array([[3, -1], [4, -1]], np.int32))
    n_in = to_dev(np.array([1, 1], np.int32))
    x_tilde = torch.full((B, K), -7, dtype=torch.int32, device=DEV)
    q_logits = torch.zeros((B, K, V), dtype=torch.float32, device=DEV)
    st = torch.zeros(B, dtype=torch.int32, device=DEV)
    binding.draft_step(m, kv, in_tok, n_in, 0, (1.0, 0, 1.0), 3, 0, x_tilde, q_logits,
                       m.workspace(B, 2, max_len), row_status=st)
    torch.cuda.synchronize()
    s = st.cpu().numpy()
    assert s[0] == 0 and s[1] & binding.ROW_NONFINITE
    xt = x_tilde.cpu().numpy()
    assert xt[1, 0] == 0 and 0 <= xt[0, 0] < V
    assert np.all(np.isfinite(q_logits[0, 0].cpu().numpy()))
