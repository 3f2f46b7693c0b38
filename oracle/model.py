"""Decoder-only transformer forward with a KV cache: the verify pass, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the pages fix: one target call scores the context plus the K drafted tokens and
yields the target's distribution at every one of those K+1 positions at once ([ZSM]
"The algorithm" and "One pass can score many tokens"; [LENS] §2.1 step 2, the gamma+1
prefixes; [GC] "How It Works" step 2, "like a mini-prefill"); weights and the KV cache
are read once per call ([LENS] §3.4).  The pages only say "transformer", so the layer
definition below is OUR spec, shared by the oracle and the GPU path: parity unpinned
with respect to the pages.  It is pinned by structural properties (K+1 positions in one
call equal K+1 single-token calls; cached equals uncached; causality; rollback then
re-append equals a fresh run) and by library cross-checks (attention against
torch.nn.functional.scaled_dot_product_attention on CPU, RMSNorm and RoPE closed forms)
in tests/test_oracle_model.py.

Layer spec (pre-norm decoder, no biases, untied embedding and LM head):
  x = E[tok]                                     residual stream (float64 here)
  per layer:
    h = bf16(RMSNorm(x) * g1)
    q, k, v = h W_qkv^T                          W_qkv rows: [q heads | k heads | v heads]
    RoPE on q, k at absolute position (half-split pairs (i, i + hd/2),
       angle = pos * theta^(-2i/hd))
    q, k, v = bf16(.); k, v appended to the cache
    o = bf16(softmax(q K^T / sqrt(hd), causal) V)
    x += o W_o^T                                 (the "attention half" of the layer)
    h = bf16(RMSNorm(x) * g2)
    GELU:   a = bf16(gelu(h W1^T)),              x += a W2^T
    SwiGLU: a = bf16(silu(h Wg^T) * (h Wu^T)),   x += a Wd^T   (the "FFN half")
  logits = bf16(RMSNorm(x) * g_f) W_head^T
with RMSNorm(x) = x / sqrt(mean(x^2) + eps) per row, gelu(t) = t * Phi(t),
silu(t) = t / (1 + e^-t).  For float32 models every bf16() is the identity.  Arithmetic
is float64 throughout; bf16() rounds the float64 value to nearest-even bf16 directly.

The halves are exposed on their own (attention_half, ffn_half, lm_head) so a test can
feed one of them the residual rows another implementation produced and compare that
half alone.

Weights are given as float32 numpy arrays (bf16-representable values for bf16 models)
in a dict with keys: embed [V,d], head [V,d], norm_f [d], and per layer l:
  l{l}.norm1 [d], l{l}.wqkv [3d,d], l{l}.wo [d,d], l{l}.norm2 [d],
  SwiGLU: l{l}.wgate [F,d], l{l}.wup [F,d], l{l}.wdown [d,F]
  GELU:   l{l}.w1 [F,d],    l{l}.w2 [d,F]
"""
import math

import numpy as np
from scipy.special import erf


def round_bf16(x):
    """Round float64 values to the nearest bf16 (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)            # below 2**-126 the bf16 spacing stays 2**-133
    quantum = np.ldexp(1.0, e - 8)     # 8 significant bits in [2**(e-1), 2**e)
    return np.rint(x / quantum) * quantum


def _cfg(cfg, key):
    return cfg[key] if isinstance(cfg, dict) else getattr(cfg, key)


class OracleConfig:
    """The few numbers the forward needs, read from a dict or an object with attributes."""

    def __init__(self, cfg):
        self.n_layers = int(_cfg(cfg, "n_layers"))
        self.d_model = int(_cfg(cfg, "d_model"))
        self.n_heads = int(_cfg(cfg, "n_heads"))
        self.head_dim = int(_cfg(cfg, "head_dim"))
        self.d_ffn = int(_cfg(cfg, "d_ffn"))
        self.vocab = int(_cfg(cfg, "vocab"))
        self.ffn_kind = str(_cfg(cfg, "ffn_kind"))
        self.dtype = str(_cfg(cfg, "dtype"))
        self.norm_eps = float(np.float32(_cfg(cfg, "norm_eps")))
        self.rope_theta = float(np.float32(_cfg(cfg, "rope_theta")))
        assert self.n_heads * self.head_dim == self.d_model
        assert self.ffn_kind in ("gelu", "swiglu")
        assert self.dtype in ("f32", "bf16")


def rmsnorm(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope(t, pos, theta):
    """Rotate t [n, H, hd] at absolute positions pos [n] (half-split pairing)."""
    hd = t.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]   # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = t[..., :half], t[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def gelu(t):
    return 0.5 * t * (1.0 + erf(t / math.sqrt(2.0)))


def silu(t):
    return t / (1.0 + np.exp(-t))


def attend(q, Kc, Vc, pos):
    """Causal attention of queries q [n, H, hd] at positions pos [n] over cache rows
    Kc, Vc [H, P, hd] (cache position t is visible to a query at position s iff t <= s).
    Returns [n, H, hd] float64."""
    q = np.asarray(q, dtype=np.float64)
    Kc = np.asarray(Kc, dtype=np.float64)
    Vc = np.asarray(Vc, dtype=np.float64)
    hd = q.shape[-1]
    P = Kc.shape[1]
    scores = np.einsum("ihd,hpd->hip", q, Kc) / math.sqrt(hd)        # [H, n, P]
    visible = np.arange(P)[None, :] <= np.asarray(pos)[:, None]      # [n, P]
    scores = np.where(visible[None], scores, -np.inf)
    scores = scores - scores.max(axis=-1, keepdims=True)
    pr = np.exp(scores)
    pr = pr / pr.sum(axis=-1, keepdims=True)
    return np.einsum("hip,hpd->ihd", pr, Vc)


class KVCache:
    """Per-layer K and V arrays [B, H, max_len, hd] (float64) plus lengths [B]."""

    def __init__(self, cfg, batch, max_len):
        c = OracleConfig(cfg)
        self.max_len = int(max_len)
        shape = (batch, c.n_heads, max_len, c.head_dim)
        # bf16 models store bf16 values, which float32 holds exactly; float32 models
        # keep the float64 values
        dt = np.float32 if c.dtype == "bf16" else np.float64
        self.k = [np.zeros(shape, dtype=dt) for _ in range(c.n_layers)]
        self.v = [np.zeros(shape, dtype=dt) for _ in range(c.n_layers)]
        self.len = np.zeros(batch, dtype=np.int64)

    def copy(self):
        other = object.__new__(KVCache)
        other.max_len = self.max_len
        other.k = [a.copy() for a in self.k]
        other.v = [a.copy() for a in self.v]
        other.len = self.len.copy()
        return other

    def fill(self, kv, lens):
        """Set contents from an array laid out [L, B, 2, H, max_len, hd] and lengths [B]."""
        kv = np.asarray(kv)
        for l in range(len(self.k)):
            self.k[l][...] = kv[l, :, 0]
            self.v[l][...] = kv[l, :, 1]
        self.len = np.asarray(lens, dtype=np.int64).copy()

    def rollback(self, new_len):
        """Shorten rows to new_len (entries past it become stale; nothing is erased)."""
        new_len = np.asarray(new_len, dtype=np.int64)
        assert np.all(new_len <= self.len) and np.all(new_len >= 0)
        self.len = new_len.copy()


def matmul(a, w):
    """a [n, in] times a weight stored [out, in]: the forward's only contraction (a
    library product in float64; a test may swap in a lower-precision accumulation to
    measure how far a correct fp32-accumulating evaluation can drift)."""
    return a @ w.T


def _rb(c):
    return round_bf16 if c.dtype == "bf16" else (lambda t: np.asarray(t, dtype=np.float64))


def _w(W, name):
    return np.asarray(W[name], dtype=np.float64)


def layer_weights(W, l):
    """The float64 tensors of layer l (a dict with the same keys as W)."""
    pre = f"l{l}."
    return {k: _w(W, k) for k in W if k.startswith(pre)}


def normed_input(x, g, eps, rb):
    """h = bf16(RMSNorm(x) * g): the input of a normalised product."""
    return rb(rmsnorm(x, g, eps))


def attention_half(cfg, W, cache, l, b, x, pos, record=None):
    """First half of layer l for sequence row b: n new rows x [n, d] at absolute
    positions pos [n] (pos[0] = the row's cache length before them).  Appends their
    K/V to cache layer l at pos and returns x + o W_o^T (float64).  record (a dict, or
    None) receives q [n, d], the rounded rotated queries, and o [n, d], the rounded
    attention output the product takes."""
    c = OracleConfig(cfg)
    rb = _rb(c)
    H, hd, d = c.n_heads, c.head_dim, c.d_model
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    s0 = int(pos[0])
    h = normed_input(x, _w(W, f"l{l}.norm1"), c.norm_eps, rb)
    qkv = matmul(h, _w(W, f"l{l}.wqkv"))
    q = qkv[:, :d].reshape(n, H, hd)
    k = qkv[:, d:2 * d].reshape(n, H, hd)
    v = qkv[:, 2 * d:].reshape(n, H, hd)
    q = rb(rope(q, pos, c.rope_theta))
    k = rb(rope(k, pos, c.rope_theta))
    v = rb(v)
    cache.k[l][b, :, s0:s0 + n] = k.transpose(1, 0, 2)
    cache.v[l][b, :, s0:s0 + n] = v.transpose(1, 0, 2)
    o = rb(attend(q, cache.k[l][b, :, :s0 + n], cache.v[l][b, :, :s0 + n], pos).reshape(n, d))
    if record is not None:
        record["q"] = q.reshape(n, d)
        record["o"] = o
    return x + matmul(o, _w(W, f"l{l}.wo"))


def ffn_half(cfg, W, l, x, record=None):
    """Second half of layer l: x + FFN(bf16(RMSNorm(x) * g2)) for rows x [n, d].  record
    (a dict, or None) receives a, the rounded activation the down product takes."""
    c = OracleConfig(cfg)
    rb = _rb(c)
    x = np.asarray(x, dtype=np.float64)
    h = normed_input(x, _w(W, f"l{l}.norm2"), c.norm_eps, rb)
    if c.ffn_kind == "swiglu":
        a = rb(silu(matmul(h, _w(W, f"l{l}.wgate"))) * matmul(h, _w(W, f"l{l}.wup")))
        w_out = _w(W, f"l{l}.wdown")
    else:
        a = rb(gelu(matmul(h, _w(W, f"l{l}.w1"))))
        w_out = _w(W, f"l{l}.w2")
    if record is not None:
        record["a"] = a
    return x + matmul(a, w_out)


def lm_head(cfg, W, x):
    """logits = bf16(RMSNorm(x) * g_f) W_head^T for rows x [n, d]."""
    c = OracleConfig(cfg)
    rb = _rb(c)
    return matmul(normed_input(x, _w(W, "norm_f"), c.norm_eps, rb), _w(W, "head"))


def forward(cfg, W, cache, tokens, n_tok=None, layers=None):
    """Score new tokens on top of the cache and append their K/V.

    tokens [B, M] int; n_tok [B] (row b uses its first n_tok[b] tokens, default M).
    Returns logits [B, M, V] float64 (rows j >= n_tok[b] are left at 0) and advances
    cache.len by n_tok.  ``layers`` limits the pass to the first n layers (the LM head
    still runs), which the timing of very large models uses.
    """
    c = OracleConfig(cfg)
    tokens = np.asarray(tokens, dtype=np.int64)
    B, M = tokens.shape
    n_tok = np.full(B, M, dtype=np.int64) if n_tok is None else np.asarray(n_tok, np.int64)
    n_layers = c.n_layers if layers is None else int(layers)
    if np.any(cache.len + n_tok > cache.max_len):
        raise ValueError("KV cache overflow")
    rows = [b for b in range(B) if n_tok[b] > 0]
    pos = {b: int(cache.len[b]) + np.arange(int(n_tok[b])) for b in rows}
    E = np.asarray(W["embed"])
    x = {b: E[tokens[b, :n_tok[b]]].astype(np.float64) for b in rows}
    for l in range(n_layers):
        Wl = layer_weights(W, l)   # float64 once per layer, shared by the rows
        for b in rows:
            x[b] = ffn_half(c, Wl, l, attention_half(c, Wl, cache, l, b, x[b], pos[b]))
    logits = np.zeros((B, M, c.vocab))
    Wh = {"norm_f": _w(W, "norm_f"), "head": _w(W, "head")}
    for b in rows:
        logits[b, :n_tok[b]] = lm_head(c, Wh, x[b])
    cache.len = cache.len + n_tok
    return logits
