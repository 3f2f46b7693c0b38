"""ctypes binding of libspecdec.so: argument marshalling only.

Every computation runs in the HIP library; this module converts torch tensors to device
pointers, torch streams to hipStream_t handles, and status codes to exceptions.  There
is no CPU fallback: if the library is missing, ``load()`` raises.
"""
import ctypes
import os

import torch

from . import synth

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecdec.so")

SPEC_OK, SPEC_E_INVALID, SPEC_E_UNSUPPORTED, SPEC_E_CAPACITY, SPEC_E_HIP = 0, -1, -2, -3, -4
ROW_NONFINITE, ROW_Q_ZERO, ROW_RESIDUAL_EMPTY, ROW_KV_OVERFLOW, ROW_BAD_TOKEN = 1, 2, 4, 8, 16
FFN = {"gelu": 0, "swiglu": 1}
DT = {"f32": 0, "bf16": 1}

SYMBOLS = [
    "spec_model_n_weights", "spec_model_bytes", "spec_model_create", "spec_model_load_weight",
    "spec_model_destroy", "spec_kv_bytes",
    "spec_kv_create", "spec_kv_destroy", "spec_kv_data", "spec_kv_import", "spec_kv_export",
    "spec_kv_rollback",
    "spec_workspace_bytes", "spec_verify_forward", "spec_verify_forward_trace", "spec_draft_step",
    "spec_accept_workspace_bytes", "spec_accept_resample", "spec_accept_resample_static",
    "spec_verify_tokens",
    "spec_status_str", "spec_last_hip_error", "spec_abi_version", "spec_timing_enable",
    "spec_timing_read",
]


class ModelCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("d_model", ctypes.c_int),
                ("n_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("d_ffn", ctypes.c_int), ("vocab", ctypes.c_int),
                ("ffn_kind", ctypes.c_int), ("dtype", ctypes.c_int),
                ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]

    @classmethod
    def from_shape(cls, s: "synth.ModelShape"):
        return cls(s.n_layers, s.d_model, s.n_heads, s.head_dim, s.d_ffn, s.vocab,
                   FFN[s.ffn_kind], DT[s.dtype], s.norm_eps, s.rope_theta)


class Sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int),
                ("top_p", ctypes.c_float)]


class SpecError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_LIB.spec_status_str(status).decode()} ({status})"
                         + (f", hip error {_LIB.spec_last_hip_error()}"
                            if status == SPEC_E_HIP else ""))


_LIB = None
P = ctypes.c_void_p
I32 = ctypes.c_int
U64 = ctypes.c_uint64
SZ = ctypes.c_size_t


def load(path=None):
    """Load the library (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m speculative_decoding_forward_amd.build_lib`")
    lib = ctypes.CDLL(path)
    cfgp = ctypes.POINTER(ModelCfg)
    smp = ctypes.POINTER(Sampling)
    sig = {
        "spec_model_n_weights": (I32, [cfgp]),
        "spec_model_bytes": (SZ, [cfgp]),
        "spec_model_create": (I32, [cfgp, P, SZ, ctypes.POINTER(P)]),
        "spec_model_load_weight": (I32, [P, I32, P, P]),
        "spec_model_destroy": (I32, [P]),
        "spec_kv_bytes": (SZ, [cfgp, I32, I32]),
        "spec_kv_create": (I32, [cfgp, I32, I32, P, SZ, P, P, ctypes.POINTER(P)]),
        "spec_kv_destroy": (I32, [P]),
        "spec_kv_data": (P, [P]),
        "spec_kv_import": (I32, [P, P, I32, P]),
        "spec_kv_export": (I32, [P, P, I32, P]),
        "spec_kv_rollback": (I32, [P, P, P]),
        "spec_workspace_bytes": (SZ, [cfgp, I32, I32, I32]),
        "spec_verify_forward": (I32, [P, P, P, P, I32, I32, P, P, P, SZ, P]),
        "spec_verify_forward_trace": (I32, [P, P, P, P, I32, I32, P, P, P, P, P, P, P, SZ, P]),
        "spec_draft_step": (I32, [P, P, P, P, I32, I32, I32, smp, U64, U64, P, P, P, P, P, SZ,
                                  P]),
        "spec_accept_workspace_bytes": (SZ, [I32, I32]),
        "spec_verify_tokens": (I32, [P, P, P, I32, I32, P, P]),
        "spec_accept_resample": (I32, [P, P, P, I32, I32, I32, smp, U64, U64, P, P, P, P, P, P,
                                       P, P, ctypes.POINTER(P), P, SZ, P]),
        "spec_accept_resample_static": (I32, [P, P, P, I32, I32, I32, smp, U64, U64, P, P, P, P,
                                              P, P, P, P, P]),
        "spec_status_str": (ctypes.c_char_p, [I32]),
        "spec_last_hip_error": (I32, []),
        "spec_abi_version": (I32, []),
        "spec_timing_enable": (I32, [I32]),
        "spec_timing_read": (I32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32),
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status, where):
    if status != SPEC_OK:
        raise SpecError(status, where)


def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous"
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _alloc(nbytes, device):
    """256-byte aligned device buffer (torch's allocator aligns to at least 512)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


class Model:
    """A model over a device store this object allocates (torch) and owns.

    weights: dict name -> device tensor (canonical names and shapes of the shape), copied
    into the store (bf16 matrices rearranged into GEMM tiles) on `stream`, in stream order:
    the caller may drop them afterwards (torch reuses freed memory in stream order).
    weights=None leaves the store unset: fill it tensor by tensor with ``load_weight`` (a
    loader's peak memory is then the store plus one tensor)."""

    def __init__(self, shape: "synth.ModelShape", weights=None, device="cuda", stream=None):
        lib = load()
        self.shape = shape
        self.cfg = ModelCfg.from_shape(shape)
        self.names = shape.weight_names()
        n = lib.spec_model_bytes(ctypes.byref(self.cfg))
        if n == 0:
            raise SpecError(SPEC_E_INVALID, "spec_model_bytes")
        self.store = _alloc(n, device)
        h = P()
        _check(lib.spec_model_create(ctypes.byref(self.cfg), _ptr(self.store), n,
                                     ctypes.byref(h)), "spec_model_create")
        self.handle = h
        if weights is not None:
            for nm in self.names:
                self.load_weight(nm, weights[nm], stream)

    def load_weight(self, name, tensor, stream=None):
        """Copy one tensor (canonical name) into the model on `stream`; the tensor must
        stay alive until the stream has passed the copy."""
        t = tensor.contiguous()
        _check(load().spec_model_load_weight(self.handle, self.names.index(name), _ptr(t),
                                             _stream(stream)), "spec_model_load_weight")

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.spec_model_destroy(self.handle)
            self.handle = None

    def workspace(self, batch, max_rows, max_len, device="cuda"):
        n = load().spec_workspace_bytes(ctypes.byref(self.cfg), batch, max_rows, max_len)
        if n == 0:
            raise SpecError(SPEC_E_INVALID, "spec_workspace_bytes")
        return _alloc(n, device)


class KVCache:
    """A KV arena + lengths for `batch` rows of up to `max_len` positions."""

    def __init__(self, shape: "synth.ModelShape", batch, max_len, device="cuda", stream=None):
        lib = load()
        self.shape = shape
        self.cfg = ModelCfg.from_shape(shape)
        self.batch, self.max_len = batch, max_len
        n = lib.spec_kv_bytes(ctypes.byref(self.cfg), batch, max_len)
        if n == 0:
            raise SpecError(SPEC_E_INVALID, "spec_kv_bytes")
        self.arena = _alloc(n, device)
        self.len = torch.zeros(batch, dtype=torch.int32, device=device)
        h = P()
        _check(lib.spec_kv_create(ctypes.byref(self.cfg), batch, max_len, _ptr(self.arena), n,
                                  _ptr(self.len), _stream(stream), ctypes.byref(h)),
               "spec_kv_create")
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.spec_kv_destroy(self.handle)
            self.handle = None

    def data(self):
        """The raw K/V element block (bf16 caches hold it in the attention's packed
        order; use import_/export for natural order)."""
        s = self.shape
        dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
        cap = (self.max_len + 31) // 32 * 32 if s.dtype == "bf16" else self.max_len
        n = s.n_layers * self.batch * 2 * s.n_heads * cap * s.head_dim
        return self.arena[: n * (2 if s.dtype == "bf16" else 4)].view(dt)

    def import_(self, src, stream=None):
        """Write positions [0, n) of every row from src [L, B, 2, H, n, hd] (device)."""
        t = src.contiguous()
        _check(load().spec_kv_import(self.handle, _ptr(t), t.shape[4], _stream(stream)),
               "spec_kv_import")

    def export(self, n, stream=None):
        """Positions [0, n) of every row as [L, B, 2, H, n, hd] (natural order)."""
        s = self.shape
        dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
        out = torch.empty((s.n_layers, self.batch, 2, s.n_heads, n, s.head_dim), dtype=dt,
                          device=self.arena.device)
        _check(load().spec_kv_export(self.handle, _ptr(out), n, _stream(stream)),
               "spec_kv_export")
        return out

    def rollback(self, new_len, stream=None):
        _check(load().spec_kv_rollback(self.handle, _ptr(new_len), _stream(stream)),
               "spec_kv_rollback")


def verify_forward(model: Model, kv: KVCache, tokens, logits, ws, n_tok=None, row_status=None,
                   stream=None):
    """tokens [B, M] int32, logits [B, M, V] fp32 (out)."""
    B, M = tokens.shape
    _check(load().spec_verify_forward(model.handle, kv.handle, _ptr(tokens), _ptr(n_tok), B, M,
                                      _ptr(logits), _ptr(row_status), _ptr(ws), ws.numel(),
                                      _stream(stream)), "spec_verify_forward")


def verify_forward_trace(model: Model, kv: KVCache, tokens, logits, resid, ws, q=None,
                         attn_out=None, ffn_act=None, n_tok=None, row_status=None, stream=None):
    """verify_forward that also fills resid [2L+1, B*M, d] fp32 with the residual stream
    after the embedding and after each half of every layer, and optionally q and attn_out
    [L, B*M, d] and ffn_act [L, B*M, F] (the model's activation type) with each layer's
    rotated queries, rounded attention output and FFN activation."""
    B, M = tokens.shape
    _check(load().spec_verify_forward_trace(model.handle, kv.handle, _ptr(tokens), _ptr(n_tok),
                                            B, M, _ptr(logits), _ptr(row_status), _ptr(resid),
                                            _ptr(q), _ptr(attn_out), _ptr(ffn_act), _ptr(ws),
                                            ws.numel(), _stream(stream)),
           "spec_verify_forward_trace")


def draft_step(model: Model, kv: KVCache, in_tok, n_in, step, knobs, seed, rnd, x_tilde,
               q_logits, ws, row_status=None, stream=None, round_dev=None):
    """round_dev: optional int64 device scalar holding the round number (graph replay)."""
    B, K = x_tilde.shape
    smp = Sampling(*knobs)
    _check(load().spec_draft_step(model.handle, kv.handle, _ptr(in_tok), _ptr(n_in), B, K, step,
                                  ctypes.byref(smp), seed, rnd, _ptr(round_dev), _ptr(x_tilde),
                                  _ptr(q_logits), _ptr(row_status), _ptr(ws), ws.numel(),
                                  _stream(stream)), "spec_draft_step")


def verify_tokens(pending, n_pending, x_tilde, tokens, stream=None):
    B, K = x_tilde.shape
    _check(load().spec_verify_tokens(_ptr(pending), _ptr(n_pending), _ptr(x_tilde), B, K,
                                     _ptr(tokens), _stream(stream)), "spec_verify_tokens")


def accept_workspace(B, K, device="cuda"):
    return _alloc(load().spec_accept_workspace_bytes(B, K), device)


def accept_resample(p_logits, q_logits, x_tilde, knobs, seed, rnd, out_tok, n_out, row_status,
                    ws, tkv=None, dkv=None, pending=None, n_pending=None, debug=None,
                    stream=None, round_dev=None):
    """p_logits [B, K+1, V], q_logits [B, K, V] fp32; x_tilde [B, K] int32.

    debug: optional (p_probs, q_probs, accept, cand) tensors or None entries.
    """
    B, K1, V = p_logits.shape
    K = K1 - 1
    smp = Sampling(*knobs)
    dbg = None
    if debug is not None:
        dbg = (P * 4)(*[(t.data_ptr() if t is not None else None) for t in debug])
    _check(load().spec_accept_resample(
        _ptr(p_logits), _ptr(q_logits), _ptr(x_tilde), B, K, V, ctypes.byref(smp), seed, rnd,
        _ptr(round_dev), _ptr(out_tok), _ptr(n_out), _ptr(row_status),
        tkv.handle if tkv else None,
        dkv.handle if dkv else None, _ptr(pending), _ptr(n_pending), dbg, _ptr(ws), ws.numel(),
        _stream(stream)), "spec_accept_resample")


def timing_enable(on=True):
    _check(load().spec_timing_enable(1 if on else 0), "spec_timing_enable")


def timing_read():
    """(gemm_ms, gemm_launches, attn_ms, attn_launches) since the last read."""
    gm, am = ctypes.c_double(), ctypes.c_double()
    gn, an = I32(), I32()
    _check(load().spec_timing_read(ctypes.byref(gm), ctypes.byref(gn), ctypes.byref(am),
                                   ctypes.byref(an)), "spec_timing_read")
    return gm.value, gn.value, am.value, an.value
