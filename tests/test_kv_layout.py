"""The packed bf16 KV-cache order (csrc/kv_layout.h), written by the QKV GEMM's epilogue
and read by the attention kernel: compiled from the header (host code, hipcc) and checked
against the operand orders of v_mfma_f32_16x16x32_bf16 that the attention kernel assumes
(lane l of a wave: row / column l % 16, group l / 16).

  * K, blocks of 16 positions: block k, 32-wide slice s, lane l hold the 8 elements
    K[16k + l % 16][32s + 8(l / 16) .. +8] as 16 contiguous bytes at 16 l of a 1 KB block
    -- the A operand of S^T = K Q^T;
  * V, blocks of 32 positions: block k, 16-wide dim tile u, lane l hold
    V[32k + key(l / 16, e)][16u + l % 16] for e = 0..7, key(g, e) = 4g + e (e < 4) or
    16 + 4g + e - 4 -- the B operand of O = P V in the key order in which the rows of
    S^T leave the first product (two 16-key tiles: lane l holds keys 4(l/16)..+3 of each);
  * both are bijections onto a head region of capacity x hd elements.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "speculative_decoding_forward_amd", "csrc")

PROG = r"""
#include <cstdio>
#include <cstdlib>
#include "kv_layout.h"
using namespace specdec;
int main(int argc, char** argv) {
  const int n = atoi(argv[1]), hd = atoi(argv[2]);
  printf("%d\n", kv_capacity(n));
  for (int p = 0; p < kv_capacity(n); ++p)
    for (int i = 0; i < hd; ++i) printf("%zu %zu\n", kv_k_offset(p, i, hd), kv_v_offset(p, i, hd));
  return 0;
}
"""


@pytest.fixture(scope="module")
def kv_prog(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("kv")
    src, exe = d / "kv.cpp", d / "kv"
    src.write_text(PROG)
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", CSRC,
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("compiling the layout header failed:\n" + r.stderr[-2000:])
    return str(exe)


def key(g, e):
    return 4 * g + e if e < 4 else 16 + 4 * g + e - 4


@pytest.mark.parametrize("n,hd", [(40, 128), (64, 64), (33, 128)])
def test_kv_layout_matches_mfma_operand_orders(kv_prog, n, hd):
    out = subprocess.run([kv_prog, str(n), str(hd)], capture_output=True, text=True,
                         check=True).stdout.split()
    cap = int(out[0])
    assert cap == -(-n // 32) * 32
    kv = np.array(out[1:], dtype=np.int64).reshape(cap, hd, 2)
    koff, voff = kv[:, :, 0], kv[:, :, 1]
    for off in (koff, voff):
        assert np.array_equal(np.sort(off.ravel()), np.arange(cap * hd))
    lane = np.arange(64)
    for k in range(cap // 16):
        for s in range(hd // 32):
            base = (k * (hd // 32) + s) * 512
            for t in range(8):
                got = koff[16 * k + lane % 16, 32 * s + 8 * (lane // 16) + t]
                assert np.array_equal(got, base + 8 * lane + t)
    for k in range(cap // 32):
        for u in range(hd // 16):
            base = (k * (hd // 16) + u) * 512
            for e in range(8):
                pos = 32 * k + np.array([key(g, e) for g in lane // 16])
                got = voff[pos, 16 * u + lane % 16]
                assert np.array_equal(got, base + 8 * lane + e)
