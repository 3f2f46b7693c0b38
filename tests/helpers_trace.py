"""Teacher-forced parity helpers for the verify pass (shared by the GPU tests).

spec_verify_forward_trace exports the residual stream after the embedding and after each
half of every layer, and each layer's rotated queries q, rounded attention output o and
FFN activation a.  Each half is checked on the GPU's own input rows, in three parts:

  1. the products' rounded outputs (q and the K/V entries the layer appends; the FFN
     activation a) against the oracle's, computed in float64 from the same input rows;
  2. attention recomputed in float64 from the GPU's own q, K and V against the GPU's o:
     only the attention arithmetic differs there;
  3. the residual update given the GPU's own rounded activation: x + o W_o^T and
     x + a W_down^T in float64 against the GPU's rows.
The LM head is checked on the GPU's final rows.

Why split there: both sides evaluate the same definition, fp32 against float64, and round
the same activations to bf16.  Where the two values of an activation fall on different
sides of a bf16 rounding boundary (a crossing) they differ by one bf16 step, and the next
product spreads that step over a whole row; from layer to layer such moves compound.
Checked this way, every comparison is of one smooth computation on identical inputs.

The normalised products inside the layers round their input at a different point than
the oracle: the kernel multiplies bf16(x * g) and scales the product row by the RMS
factor s afterwards, the oracle multiplies bf16(s * x * g).  Part 1 therefore allows, on
top of two bf16 steps, the exact effect of that move on each output, computed in float64
from the same rows: s (bf16(x g) W^T) - bf16(s x g) W^T, carried through RoPE (a rotation)
or through the activation (first order, with a 25% margin).  The LM head's input is
rounded after the row factor on both sides.

Bounds (u = 2^-24):
  * residual updates: |GPU - oracle| <= 2u (K + 2) (|act| |W|^T + |x| + |y|) per element,
    the forward error bound of an fp32 dot product of K terms with exact products and one
    fp32 addition (Higham, Accuracy and Stability of Numerical Algorithms, §3.1), doubled
    so it holds for any rounding mode of the accumulator;
  * attention on the GPU's q, K, V: within one bf16 step, in at most 2% of the elements;
  * product outputs: within 2 bf16 steps + the rounding-point effect + ROW_SHIFT per
    element, where ROW_SHIFT covers a crossing in the product's own bf16 input (a whole
    row moves by step(h) * |w| <= 2^-6 * 0.12 for |h| < 4 and weights within six standard
    deviations of N(0, 0.02^2));
  * logits of the LM head on the GPU's final rows: <= 1e-2 per element, <= 1e-3 mean.
"""
import dataclasses

import numpy as np
import torch

from oracle import model as omodel
from speculative_decoding_forward_amd import binding, synth

from helpers import DEV

TOL_MAX, TOL_MEAN = 1e-2, 1e-3   # logits
U = 2.0 ** -24
ROW_SHIFT = 2.0 ** -6 * 0.12     # one crossing in a product's bf16 input, per output


def fold_shift(x, g, w, eps):
    """The exact effect, per output, of the kernel's rounding point on x's normalised
    product with w [N, K]: s (bf16(x g) w^T) - bf16(s x g) w^T (float64), s the RMS
    factor of each row."""
    x = np.asarray(x, np.float64)
    xg = x * np.asarray(g, np.float64)
    s = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return s * omodel.matmul(omodel.round_bf16(xg), w) - omodel.matmul(omodel.round_bf16(s * xg), w)


class _LayerCache:
    """The oracle's cache for one layer of a verify pass: K/V [B, H, max_len, hd] of
    layer l from the seeded fill, and the rows' lengths."""

    def __init__(self, n_layers, l, fill_l, lens):
        self.k = [None] * n_layers
        self.v = [None] * n_layers
        self.k[l] = np.ascontiguousarray(fill_l[:, 0])
        self.v[l] = np.ascontiguousarray(fill_l[:, 1])
        self.len = np.asarray(lens, np.int64)


def _numpy_layer(W, shape, l):
    pre = f"l{l}."
    return {n: W[n].float().cpu().numpy() for n in shape.weight_names() if n.startswith(pre)}


@dataclasses.dataclass
class Traced:
    shape: object
    W: dict           # device weights
    lens: np.ndarray  # cache length of each row before the pass
    new: np.ndarray   # [B, M] token ids
    trace: np.ndarray  # [2L+1, B*M, d]
    logits: np.ndarray
    kv_new: torch.Tensor  # [L, B, 2, H, M, hd] the appended entries (device)
    fill: torch.Tensor    # [L, B, 2, H, max_len, hd] (device)
    n_tok: np.ndarray     # [B] real tokens per row
    q: torch.Tensor       # [L, B*M, d] each layer's rotated queries (device)
    attn: torch.Tensor    # [L, B*M, d] each layer's rounded attention output (device)
    ffn: torch.Tensor     # [L, B*M, F] each layer's rounded FFN activation (device)


def traced_verify(shape, B, M, lens, seed, model_id=synth.TARGET, keep=None, n_tok=None,
                  tokens=None):
    """Build the model tensor by tensor (keeping on the device only the tensors `keep`
    accepts, for the oracle), fill the cache (rows at their own lengths) and run one
    traced verify pass over M new tokens per row (n_tok[b] of them real; `tokens` [B, M],
    else seeded ids)."""
    print(f"building L{shape.n_layers} d{shape.d_model} model, B={B} M={M}", flush=True)
    m = binding.Model(shape, None)
    W = {}
    for i, nm in enumerate(shape.weight_names()):
        if i % 64 == 63:
            print(f"  {i + 1} tensors loaded", flush=True)
        w = synth.make_weight(shape, nm, seed=seed, model_id=model_id, device=DEV)
        m.load_weight(nm, w)
        if keep is None or keep(nm):
            W[nm] = w
        del w
    lens = np.asarray(lens, np.int64)
    max_len = int(lens.max()) + M + 1
    kv = binding.KVCache(shape, B, max_len)
    fill = synth.kv_fill(shape, B, max_len, int(lens.max()), seed=seed, model_id=model_id,
                         device=DEV)
    kv.import_(fill)
    kv.len.copy_(torch.from_numpy(lens.astype(np.int32)))
    new = synth.context_ids(seed + 9, B, M, shape.vocab) if tokens is None else \
        np.asarray(tokens, np.int64)
    R, L, d = B * M, shape.n_layers, shape.d_model
    trace = torch.full((2 * L + 1, R, d), float("nan"), device=DEV)
    adt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    attn = torch.zeros((L, R, d), dtype=adt, device=DEV)
    qt = torch.zeros((L, R, d), dtype=adt, device=DEV)
    ffn = torch.zeros((L, R, shape.d_ffn), dtype=adt, device=DEV)
    logits = torch.zeros((B, M, shape.vocab), device=DEV)
    st = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = m.workspace(B, M, max_len)
    nt = None if n_tok is None else torch.from_numpy(np.asarray(n_tok, np.int32)).to(DEV)
    binding.verify_forward_trace(m, kv, torch.from_numpy(new.astype(np.int32)).to(DEV), logits,
                                 trace, ws, q=qt, attn_out=attn, ffn_act=ffn, n_tok=nt,
                                 row_status=st)
    torch.cuda.synchronize()
    print("traced verify pass done", flush=True)
    assert np.all(st.cpu().numpy() == 0)
    n_tok = np.full(B, M, np.int64) if n_tok is None else np.asarray(n_tok, np.int64)
    assert np.array_equal(kv.len.cpu().numpy(), lens + n_tok)
    exp = kv.export(max_len)
    kv_new = torch.stack([exp[:, b, :, :, int(lens[b]):int(lens[b]) + M] for b in range(B)],
                         dim=1).contiguous()
    del exp, kv, m, ws
    return Traced(shape, W, lens, new, trace.cpu().numpy(), logits.cpu().numpy(), kv_new,
                  fill, n_tok, qt, attn, ffn)


def _keep_layers(layers):
    names = {f"l{l}." for l in layers}
    return lambda nm: "." not in nm or nm[:nm.index(".") + 1] in names


def _report(what, err):
    print(f"{what}: max {err.max():.3e} mean {err.mean():.3e}", flush=True)


def _bf16_step(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    mag = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(mag)) - 7)


def check_rounded(got, ref, shift, what, steps=2, max_differing=1.0):
    """A rounded activation: within `steps` bf16 steps (at the larger magnitude) plus
    `shift` of the reference, and equal in all but max_differing of the elements."""
    got = np.asarray(got, np.float64)
    diff = np.abs(got - ref)
    allowed = steps * _bf16_step(np.maximum(np.abs(got), np.abs(ref))) + shift
    frac = np.count_nonzero(diff) / diff.size
    worst = float((diff / allowed).max())
    assert worst <= 1.0, (what, "largest difference", float(diff.max()), worst)
    assert frac <= max_differing, (what, "fraction differing", frac)
    return frac, worst


def check_update(x_in, act, w, got, what):
    """x_in + act W^T in float64 against the GPU's rows, within the fp32 dot-product
    bound 2u (K + 2) (|act| |W|^T + |x_in| + |y|)."""
    y = omodel.matmul(act, w)
    ref = x_in + y
    K = act.shape[-1]
    bound = 2 * U * (K + 2) * (np.abs(act) @ np.abs(w).T + np.abs(x_in) + np.abs(y))
    err = np.abs(got - ref)
    worst = float((err / bound).max())
    assert worst <= 1.0, (what, float(err.max()), worst)
    return err, worst


def check_layers(t: Traced, layers):
    """Every half of the given layers, rows of every sequence, on the GPU's own inputs
    (module docstring)."""
    shape = t.shape
    c = omodel.OracleConfig(shape)
    B, M = t.new.shape
    H, hd, d = shape.n_heads, shape.head_dim, shape.d_model
    out = []
    for l in layers:
        Wl = {k: v.astype(np.float64) for k, v in _numpy_layer(t.W, shape, l).items()}
        w_o = Wl[f"l{l}.wo"]
        swiglu = shape.ffn_kind == "swiglu"
        w_down = Wl[f"l{l}.wdown"] if swiglu else Wl[f"l{l}.w2"]
        fill_l = t.fill[l].float().cpu().numpy()
        cache = _LayerCache(shape.n_layers, l, fill_l, t.lens)
        kv_l = t.kv_new[l].float().cpu().numpy()   # [B, 2, H, M, hd]
        o_l = t.attn[l].float().cpu().numpy().astype(np.float64)
        q_l = t.q[l].float().cpu().numpy().astype(np.float64)
        a_l = t.ffn[l].float().cpu().numpy().astype(np.float64)
        st = {"ea": [], "ef": [], "wa": 0.0, "wf": 0.0, "fq": 0.0, "fkv": 0.0, "fa": 0.0,
              "fog": 0.0, "halves": []}
        for b in range(B):
            n = int(t.n_tok[b])
            if n == 0:
                continue
            rows = slice(b * M, b * M + n)
            pos = int(t.lens[b]) + np.arange(n)
            x0, x1, x2 = t.trace[2 * l][rows], t.trace[2 * l + 1][rows], t.trace[2 * l + 2][rows]
            rec = {}
            xa = omodel.attention_half(shape, Wl, cache, l, b, x0, pos, record=rec)
            st["halves"].append(np.abs(xa - x1).max())
            # 1. q, K, V against the oracle's, allowing the rounding-point effect
            sh = fold_shift(x0, Wl[f"l{l}.norm1"], Wl[f"l{l}.wqkv"], c.norm_eps)
            sq = np.abs(omodel.rope(sh[:, :d].reshape(n, H, hd), pos, c.rope_theta))
            sk = np.abs(omodel.rope(sh[:, d:2 * d].reshape(n, H, hd), pos, c.rope_theta))
            sv = np.abs(sh[:, 2 * d:].reshape(n, H, hd))
            f, _ = check_rounded(q_l[rows], rec["q"], sq.reshape(n, d) + ROW_SHIFT,
                                 f"layer {l} row {b} q")
            st["fq"] = max(st["fq"], f)
            for kvi, arr, shv in ((0, cache.k[l], sk), (1, cache.v[l], sv)):
                f, _ = check_rounded(kv_l[b, kvi][:, :n], arr[b, :, pos[0]:pos[0] + n],
                                     shv.transpose(1, 0, 2) + ROW_SHIFT,
                                     f"layer {l} row {b} {'KV'[kvi]}")
                st["fkv"] = max(st["fkv"], f)
            # 2. attention on the GPU's own q and K/V: only the attention arithmetic differs
            kc = cache.k[l][b, :, :pos[-1] + 1].copy()
            vc = cache.v[l][b, :, :pos[-1] + 1].copy()
            kc[:, pos[0]:] = kv_l[b, 0][:, :n]
            vc[:, pos[0]:] = kv_l[b, 1][:, :n]
            o_given = omodel.round_bf16(
                omodel.attend(q_l[rows].reshape(n, H, hd), kc, vc, pos).reshape(n, -1))
            f, _ = check_rounded(o_l[rows], o_given, 1e-6, f"layer {l} row {b} o (GPU q, K, V)",
                                 steps=1, max_differing=0.02)
            st["fog"] = max(st["fog"], f)
            # 3. the residual update given the GPU's o
            e, wr = check_update(x0, o_l[rows], w_o, x1, f"layer {l} row {b} x + o Wo")
            st["ea"].append(e)
            st["wa"] = max(st["wa"], wr)
            # FFN half: 1. a against the oracle's, allowing the rounding-point effect
            rec = {}
            xf = omodel.ffn_half(shape, Wl, l, x1, record=rec)
            st["halves"].append(np.abs(xf - x2).max())
            g2 = Wl[f"l{l}.norm2"]
            hp = omodel.normed_input(x1, g2, c.norm_eps, omodel.round_bf16)
            if swiglu:
                wg, wu = Wl[f"l{l}.wgate"], Wl[f"l{l}.wup"]
                gt, up = omodel.matmul(hp, wg), omodel.matmul(hp, wu)
                dg = np.abs(fold_shift(x1, g2, wg, c.norm_eps))
                du = np.abs(fold_shift(x1, g2, wu, c.norm_eps))
                sig = 1.0 / (1.0 + np.exp(-gt))
                d_act = (np.abs(sig * (1.0 + gt * (1.0 - sig)) * up) * dg +
                         np.abs(gt * sig) * du + dg * du)
            else:
                w1 = Wl[f"l{l}.w1"]
                y = omodel.matmul(hp, w1)
                dy = np.abs(fold_shift(x1, g2, w1, c.norm_eps))
                phi = np.exp(-0.5 * y * y) / np.sqrt(2 * np.pi)
                d_act = np.abs(0.5 * (1 + omodel.erf(y / np.sqrt(2.0))) + y * phi) * dy + dy * dy
            f, _ = check_rounded(a_l[rows], rec["a"], 1.25 * d_act + 8.0 * ROW_SHIFT,
                                 f"layer {l} row {b} a")
            st["fa"] = max(st["fa"], f)
            # 3. the residual update given the GPU's a
            e, wr = check_update(x1, a_l[rows], w_down, x2, f"layer {l} row {b} x + a Wd")
            st["ef"].append(e)
            st["wf"] = max(st["wf"], wr)
        ea, ef = np.concatenate(st["ea"]), np.concatenate(st["ef"])
        print(f"layer {l}: x+oWo err max {ea.max():.2e} ({st['wa']:.2f} of bound), "
              f"x+aWd err max {ef.max():.2e} ({st['wf']:.2f} of bound); rounded values "
              f"differing from the oracle's: q {st['fq']:.1%}, K/V {st['fkv']:.1%}, "
              f"a {st['fa']:.1%}; o on the GPU's q/K/V {st['fog']:.2%}; whole half vs the "
              f"oracle's own half: max {max(st['halves']):.2e}", flush=True)
        out.append(max(st["halves"]))
    return out


def check_head(t: Traced):
    shape = t.shape
    B, M = t.new.shape
    Wh = {"norm_f": t.W["norm_f"].float().cpu().numpy().astype(np.float64),
          "head": t.W["head"].float().cpu().numpy().astype(np.float64)}
    ref = omodel.lm_head(shape, Wh, t.trace[2 * shape.n_layers]).reshape(B, M, -1)
    real = np.arange(M)[None, :] < t.n_tok[:, None]
    err = np.abs(ref - t.logits)[real]
    assert np.all(t.logits[~real] == 0)
    _report("LM head on the GPU's final rows", err)
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN
    return err.max()


def end_to_end(t: Traced):
    """The oracle's own forward from the tokens (not teacher-forced): reported."""
    shape = t.shape
    B, M = t.new.shape
    Wn = synth.weights_to_numpy(t.W)
    oc = omodel.KVCache(shape, B, int(t.lens.max()) + M + 1)
    oc.fill(t.fill.float().cpu().numpy(), t.lens)
    o = omodel.forward(shape, Wn, oc, t.new, n_tok=t.n_tok)
    err = np.abs(o - t.logits)
    _report(f"end to end over {shape.n_layers} layers (not teacher-forced)", err)
    return err


