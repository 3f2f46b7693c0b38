"""spec_accept_resample_static, the accept/resample entry point that allocates nothing
(its scratch is a device array inside the library): through the C ABI, its outputs equal
spec_accept_resample's bit for bit on the same inputs, on two calls in a row (the second
smaller), it rejects a batch beyond its scratch with SPEC_E_CAPACITY before launching
anything, and the device's free memory does not change across a call."""
import ctypes

import numpy as np
import pytest
import torch

from speculative_decoding_forward_amd import binding, synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _inputs(seed, B, K, V):
    p, q = synth.vocab_logits(seed, B, K, V, 2.0, 0.5)
    P = torch.from_numpy(p).to(DEV)
    Q = torch.from_numpy(q).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    probs = torch.softmax(Q.double() / 0.8, dim=-1).reshape(B * K, V)
    X = torch.multinomial(probs, 1, generator=g).reshape(B, K).to(torch.int32).contiguous()
    return P, Q, X


def _outs(B, K):
    i32 = dict(dtype=torch.int32, device=DEV)
    return (torch.full((B, K + 1), -7, **i32), torch.full((B,), -7, **i32),
            torch.full((B,), -7, **i32))


def _run_both(lib, seed, B, K, V, knobs, rnd):
    P, Q, X = _inputs(seed, B, K, V)
    smp = binding.Sampling(*knobs)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = _outs(B, K)
    ws = binding.accept_workspace(B, K)
    st = lib.spec_accept_resample(_p(P), _p(Q), _p(X), B, K, V, ctypes.byref(smp), 11, rnd, None,
                                  _p(ref[0]), _p(ref[1]), _p(ref[2]), None, None, None, None,
                                  None, _p(ws), ws.numel(), stream)
    assert st == binding.SPEC_OK
    got = _outs(B, K)
    st = lib.spec_accept_resample_static(_p(P), _p(Q), _p(X), B, K, V, ctypes.byref(smp), 11,
                                         rnd, None, _p(got[0]), _p(got[1]), _p(got[2]), None,
                                         None, None, None, stream)
    assert st == binding.SPEC_OK
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    n = got[1].cpu().numpy()
    assert np.all((n >= 1) & (n <= K + 1))
    return got


def test_static_equals_workspace_entry_point_on_two_calls():
    lib = binding.load()
    _run_both(lib, 1, 32, 8, 32000, (0.8, 0, 1.0), 3)
    # second call, smaller: the shared scratch keeps the first call's contents
    _run_both(lib, 2, 3, 2, 1000, (1.0, 20, 0.9), 4)


def test_static_rejects_a_batch_beyond_its_scratch():
    lib = binding.load()
    smp = binding.Sampling(1.0, 0, 1.0)
    dummy = torch.zeros(16, dtype=torch.float32, device=DEV)
    st = lib.spec_accept_resample_static(_p(dummy), _p(dummy), _p(dummy), 1024, 16, 8,
                                         ctypes.byref(smp), 0, 0, None, _p(dummy), _p(dummy),
                                         _p(dummy), None, None, None, None, None)
    assert st == binding.SPEC_E_CAPACITY


def test_static_call_allocates_nothing():
    lib = binding.load()
    B, K, V = 8, 4, 4096
    P, Q, X = _inputs(5, B, K, V)
    out, n_out, rs = _outs(B, K)
    smp = binding.Sampling(0.8, 0, 0.95)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(rnd):
        return lib.spec_accept_resample_static(_p(P), _p(Q), _p(X), B, K, V, ctypes.byref(smp),
                                               1, rnd, None, _p(out), _p(n_out), _p(rs), None,
                                               None, None, None, stream)

    assert call(0) == binding.SPEC_OK
    torch.cuda.synchronize()
    before = torch.cuda.mem_get_info()[0]
    for r in range(1, 9):
        assert call(r) == binding.SPEC_OK
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == before
