"""The C-ABI library loads and exports every entry point include/specdec.h declares;
host-side size queries and argument checks (no kernel launches, no GPU needed)."""
import ctypes
import os
import re

import pytest

from speculative_decoding_forward_amd import binding, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "specdec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(binding.SYMBOLS)


def test_abi_version_and_status_strings():
    lib = binding.load()
    assert lib.spec_abi_version() == 2
    assert lib.spec_status_str(0) == b"ok"
    assert lib.spec_status_str(-3) == b"buffer too small"


def test_size_queries():
    lib = binding.load()
    s = synth.WORKLOADS["7b"].target
    cfg = binding.ModelCfg.from_shape(s)
    assert lib.spec_model_n_weights(ctypes.byref(cfg)) == 3 + 7 * 32
    g = synth.WORKLOADS["small"].target
    cg = binding.ModelCfg.from_shape(g)
    assert lib.spec_model_n_weights(ctypes.byref(cg)) == 3 + 6 * 24
    kvb = lib.spec_kv_bytes(ctypes.byref(cfg), 8, 2112)
    assert kvb >= 32 * 8 * 2 * 32 * 2112 * 128 * 2
    assert kvb % 256 == 0
    ws = lib.spec_workspace_bytes(ctypes.byref(cfg), 8, 6, 2112)
    assert 48 * 32000 * 4 < ws < 512 * 2**20
    assert lib.spec_accept_workspace_bytes(32, 8) >= 32 * 8 * 4 + 2 * 32 * 9 * 4
    bad = binding.ModelCfg.from_shape(s)
    bad.n_heads = 31
    assert lib.spec_model_n_weights(ctypes.byref(bad)) == -1
    assert lib.spec_kv_bytes(ctypes.byref(bad), 1, 16) == 0


def test_argument_checks_launch_nothing():
    lib = binding.load()
    smp = binding.Sampling(1.0, 0, 1.0)
    # null pointers -> invalid, before any launch
    st = lib.spec_accept_resample(None, None, None, 1, 1, 10, ctypes.byref(smp), 0, 0, None,
                                  None, None, None, None, None, None, None, None, None, 0, None)
    assert st == binding.SPEC_E_INVALID
    assert lib.spec_verify_forward(None, None, None, None, 1, 1, None, None, None, 0,
                                   None) == binding.SPEC_E_INVALID
    assert lib.spec_kv_rollback(None, None, None) == binding.SPEC_E_INVALID
    assert lib.spec_model_destroy(None) == binding.SPEC_E_INVALID
    assert lib.spec_verify_forward_trace(None, None, None, None, 1, 1, None, None, None, None,
                                         None, None, None, 0, None) == binding.SPEC_E_INVALID
    # model and cache binding: caller-owned buffers are checked on the host (these
    # addresses are never dereferenced: every check fails before anything is touched)
    cfg = binding.ModelCfg.from_shape(synth.WORKLOADS["small"].target)
    h = ctypes.c_void_p()
    need = lib.spec_model_bytes(ctypes.byref(cfg))
    assert need > 0 and need % 256 == 0
    assert lib.spec_model_create(ctypes.byref(cfg), None, need, ctypes.byref(h)) == \
        binding.SPEC_E_INVALID
    assert lib.spec_model_create(ctypes.byref(cfg), ctypes.c_void_p(4096 + 16), need,
                                 ctypes.byref(h)) == binding.SPEC_E_INVALID
    assert lib.spec_model_create(ctypes.byref(cfg), ctypes.c_void_p(4096), need - 256,
                                 ctypes.byref(h)) == binding.SPEC_E_CAPACITY
    kvb = lib.spec_kv_bytes(ctypes.byref(cfg), 2, 64)
    assert lib.spec_kv_create(ctypes.byref(cfg), 2, 64, ctypes.c_void_p(4096 + 8), kvb,
                              ctypes.c_void_p(4096), None, ctypes.byref(h)) == \
        binding.SPEC_E_INVALID
    assert lib.spec_kv_create(ctypes.byref(cfg), 2, 64, ctypes.c_void_p(4096), kvb - 256,
                              ctypes.c_void_p(4096), None, ctypes.byref(h)) == \
        binding.SPEC_E_CAPACITY


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        binding.load.__wrapped__(str(tmp_path / "missing.so")) if hasattr(
            binding.load, "__wrapped__") else _load_missing(tmp_path)


def _load_missing(tmp_path):
    saved = binding._LIB
    binding._LIB = None
    try:
        binding.load(str(tmp_path / "missing.so"))
    finally:
        binding._LIB = saved


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "specdec.h"
int main(void) {
  spec_model_cfg cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.n_layers = 2; cfg.d_model = 256; cfg.n_heads = 2; cfg.head_dim = 128;
  cfg.d_ffn = 512; cfg.vocab = 1024; cfg.ffn_kind = SPEC_FFN_SWIGLU; cfg.dtype = SPEC_DT_BF16;
  cfg.norm_eps = 1e-5f; cfg.rope_theta = 10000.0f;
  size_t m = spec_model_bytes(&cfg), w = spec_workspace_bytes(&cfg, 2, 6, 128);
  spec_model* h = 0;
  int bad = spec_model_create(&cfg, 0, m, &h);  /* null store: rejected, nothing launched */
  printf("%d %zu %zu %d %s\n", spec_abi_version(), m, w, bad, spec_status_str(bad));
  return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """include/specdec.h compiles as C11 with warnings as errors, and a C program links
    against the library and calls its host-side queries (no GPU needed)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(C_PROGRAM)
    lib_dir = os.path.dirname(binding.LIB_PATH)
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.dirname(HEADER), str(src), "-o", str(exe),
                        "-L", lib_dir, "-lspecdec", f"-Wl,-rpath,{lib_dir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr[-2000:]
    ver, m, w, bad, msg = out.stdout.split(maxsplit=4)
    assert int(ver) == 2 and int(m) > 0 and int(w) > 0
    assert int(bad) == binding.SPEC_E_INVALID
