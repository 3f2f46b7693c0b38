"""Seeded synthetic inputs: model shapes, random-init weights, logits, token ids, KV fills.

This module draws inputs only; it holds none of the method's arithmetic (no softmax,
no sampling rule, no layer math).  Tests and the benchmark take inputs from here and
hand the same arrays to the HIP library and, in tests, to the CPU oracle.

Recipes (stand-ins, by shape and distribution only, for the trained models and data
sets the pages measure on, none of which exist here):
  * weights: every matrix and embedding ~ N(0, 0.02^2) drawn in float32, rounded to
    nearest-even bf16 for bf16 models; RMSNorm gains = 1.  One generator per tensor,
    seeded from (seed, model_id, layer, tensor_id).
  * context ids: uniform over [0, V).
  * accept/resample-only workload: target logits ~ N(0, 2^2), draft logits = target
    rows + N(0, 0.5^2) noise ("N(0,s)" read as a standard deviation s).
  * KV-cache fills (to stand in for a long prefilled context without running the
    prefill): K and V entries ~ N(0, 1), rounded to the cache's element type.
"""
from dataclasses import dataclass, field, asdict

import numpy as np
import torch

TARGET, DRAFT = 0, 1


@dataclass
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    ffn_kind: str          # "gelu" | "swiglu"
    dtype: str             # "f32" | "bf16"
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0

    def as_dict(self):
        return asdict(self)

    def weight_names(self):
        """Canonical weight order (the order the library's model-create call takes)."""
        names = ["embed", "head", "norm_f"]
        for l in range(self.n_layers):
            names += [f"l{l}.norm1", f"l{l}.wqkv", f"l{l}.wo", f"l{l}.norm2"]
            if self.ffn_kind == "swiglu":
                names += [f"l{l}.wgate", f"l{l}.wup", f"l{l}.wdown"]
            else:
                names += [f"l{l}.w1", f"l{l}.w2"]
        return names

    def weight_shape(self, name):
        d, F, V = self.d_model, self.d_ffn, self.vocab
        base = name.split(".")[-1]
        return {
            "embed": (V, d), "head": (V, d), "norm_f": (d,), "norm1": (d,), "norm2": (d,),
            "wqkv": (3 * d, d), "wo": (d, d), "wgate": (F, d), "wup": (F, d),
            "wdown": (d, F), "w1": (F, d), "w2": (d, F),
        }[base]

    def n_params(self):
        return sum(int(np.prod(self.weight_shape(n))) for n in self.weight_names())

    def elt_bytes(self):
        return 2 if self.dtype == "bf16" else 4


@dataclass
class Workload:
    name: str
    target: ModelShape
    draft: ModelShape
    ctx: int
    K: int
    batch: int
    temperature: float
    top_k: int = 0
    top_p: float = 1.0
    rounds: int = 32
    seed: int = 0


def _shape(L, d, H, F, V, kind, dtype):
    return ModelShape(L, d, H, d // H, F, V, kind, dtype)


WORKLOADS = {
    # tiny end-to-end: fp32 2-layer target, 1-layer draft, vocab 1000
    "tiny": Workload("tiny", _shape(2, 128, 4, 512, 1000, "gelu", "f32"),
                     _shape(1, 64, 2, 256, 1000, "gelu", "f32"),
                     ctx=16, K=4, batch=1, temperature=1.0, rounds=32),
    # small: 24-layer bf16 target d=2048, 4-layer draft d=512
    "small": Workload("small", _shape(24, 2048, 16, 8192, 32000, "gelu", "bf16"),
                      _shape(4, 512, 4, 2048, 32000, "gelu", "bf16"),
                      ctx=512, K=4, batch=1, temperature=1.0),
    # 7B shape: 32 layers, d=4096, SwiGLU 11008; draft 16 layers d=2048 SwiGLU 5504
    "7b": Workload("7b", _shape(32, 4096, 32, 11008, 32000, "swiglu", "bf16"),
                   _shape(16, 2048, 16, 5504, 32000, "swiglu", "bf16"),
                   ctx=2048, K=5, batch=1, temperature=0.8, top_p=0.95),
    # 70B shape: 80 layers, d=8192, FFN 32768 (2-matrix GELU); draft 8 layers d=4096
    "70b": Workload("70b", _shape(80, 8192, 64, 32768, 32000, "gelu", "bf16"),
                    _shape(8, 4096, 32, 16384, 32000, "gelu", "bf16"),
                    ctx=1024, K=4, batch=1, temperature=1.0),
}

# the accept/resample-only workload: B=32 rows, K=8, V=32000, T=0.8, knobs off
VOCAB_WORKLOAD = dict(B=32, K=8, V=32000, temperature=0.8, top_k=0, top_p=1.0, seed=0,
                      p_sigma=2.0, noise_sigma=0.5)

_TENSOR_ID = {"embed": 1, "head": 2, "norm_f": 3, "norm1": 4, "wqkv": 5, "wo": 6,
              "norm2": 7, "wgate": 8, "wup": 9, "wdown": 10, "w1": 11, "w2": 12}


def _tensor_seed(seed, model_id, name):
    parts = name.split(".")
    layer = int(parts[0][1:]) + 1 if len(parts) == 2 else 0
    ss = np.random.SeedSequence([int(seed), int(model_id), layer, _TENSOR_ID[parts[-1]]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def make_weight(shape: ModelShape, name, seed=0, model_id=TARGET, device="cpu"):
    """One weight tensor (torch) on ``device``: float32 for f32 models, bfloat16 else.

    RMSNorm gains are float32 ones for every model.
    """
    dims = shape.weight_shape(name)
    if name.split(".")[-1].startswith("norm"):
        return torch.ones(dims, dtype=torch.float32, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(_tensor_seed(seed, model_id, name))
    w = torch.randn(dims, generator=g, dtype=torch.float32, device=device) * 0.02
    if shape.dtype == "bf16":
        w = w.to(torch.bfloat16)   # round to nearest even
    return w


def make_weights(shape: ModelShape, seed=0, model_id=TARGET, device="cpu"):
    """All weights of a model as {name: tensor}, in the canonical order."""
    return {n: make_weight(shape, n, seed, model_id, device) for n in shape.weight_names()}


def weights_to_numpy(W):
    """float32 numpy copies (bf16 values are exact in float32), for the CPU oracle."""
    return {n: t.detach().float().cpu().numpy() for n, t in W.items()}


def context_ids(seed, batch, n, vocab):
    rng = np.random.default_rng([int(seed), 0xC0])
    return rng.integers(0, vocab, size=(batch, n), dtype=np.int64)


def vocab_logits(seed=0, B=32, K=8, V=32000, p_sigma=2.0, noise_sigma=0.5):
    """Target logits [B, K+1, V] and draft logits [B, K, V] (float32 numpy)."""
    rng = np.random.default_rng([int(seed), 0x10])
    p = (rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(p_sigma))
    noise = rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(noise_sigma)
    q = (p[:, :K] + noise).astype(np.float32)
    return p.astype(np.float32), q


def kv_fill(shape: ModelShape, batch, max_len, fill_len, seed=0, model_id=TARGET,
            device="cpu"):
    """Random cache contents for the first ``fill_len`` positions of every row.

    Returns a tensor laid out [L, B, 2, H, max_len, hd] (positions >= fill_len zero),
    float32 for f32 models, bfloat16 else.
    """
    L, H, hd = shape.n_layers, shape.n_heads, shape.head_dim
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    out = torch.zeros((L, batch, 2, H, max_len, hd), dtype=dt, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(_tensor_seed(seed, 100 + model_id, "embed"))
    for l in range(L):
        blk = torch.randn((batch, 2, H, fill_len, hd), generator=g, dtype=torch.float32,
                          device=device)
        out[l, :, :, :, :fill_len] = blk.to(dt)
    return out
