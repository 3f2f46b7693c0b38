"""The packed activation order (csrc/act_layout.h) that every bf16 producer writes and every
GEMM's A operand reads: compiled from the header itself (host code, hipcc) and checked for
the properties the kernels rely on.

  * it is a bijection from the rows padded to whole 16-row tiles onto [0, act_rows(R) * K);
  * each aligned group of 8 columns is contiguous (one 16-byte store or load);
  * the 16 rows x 32 columns of one (row tile, 128-wide step, 32-wide slice) form one
    contiguous kilobyte, row n's group g at position 4n + g -- so a wave's A fragment
    for v_mfma_f32_16x16x32_bf16 (lane l: row l % 16, group l / 16) is a single 1 KB
    block, and row n's 32 columns of the slice are 64 contiguous bytes.

The fp32 order (act32_index) of a normalised product's x * g rows is checked the same
way: a bijection onto the padded buffer, aligned groups of 4 columns contiguous (one
16-byte load), and each (row tile, step, slice, half) one contiguous kilobyte in which
row n's four columns 8 g + 4 h .. + 4 sit at position 4n + g -- so lane l's two loads of
a slice (halves 0 and 1) are each one 1 KB wave load.
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
#include "act_layout.h"
using namespace specdec;
int main(int argc, char** argv) {
  const int R = atoi(argv[1]), K = atoi(argv[2]), f32 = argc > 3;
  printf("%d\n", act_rows(R));
  for (int r = 0; r < act_rows(R); ++r)
    for (int k = 0; k < K; ++k) printf("%zu\n", f32 ? act32_index(r, k, K) : act_index(r, k, K));
  return 0;
}
"""


@pytest.fixture(scope="module")
def act_prog(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("act")
    src, exe = d / "act.cpp", d / "act"
    src.write_text(PROG)
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", CSRC,
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("compiling the layout header failed:\n" + r.stderr[-2000:])
    return str(exe)


def layout(exe, R, K, f32=False):
    out = subprocess.run([exe, str(R), str(K)] + (["f32"] if f32 else []), capture_output=True,
                         text=True, check=True).stdout.split()
    rows = int(out[0])
    return rows, np.array(out[1:], dtype=np.int64).reshape(rows, K)


@pytest.mark.parametrize("R,K", [(1, 128), (6, 256), (17, 384), (48, 512)])
def test_act_layout_properties(act_prog, R, K):
    rows, idx = layout(act_prog, R, K)
    assert rows == -(-R // 16) * 16
    # bijection onto the padded buffer
    assert np.array_equal(np.sort(idx.ravel()), np.arange(rows * K))
    # aligned 8-column groups are contiguous
    g = idx.reshape(rows, K // 8, 8)
    assert np.all(g - g[:, :, :1] == np.arange(8))
    # one (row tile, step, slice) block: 1 KB contiguous, row n group g at 4n + g
    for mt in range(rows // 16):
        for js in range(K // 128):
            for s in range(4):
                blk = idx[16 * mt:16 * mt + 16, 128 * js + 32 * s:128 * js + 32 * s + 32]
                base = blk.min()
                assert base % 512 == 0 and blk.max() == base + 511
                pos = (blk[:, ::8] - base) // 8  # [row n, group g] -> 8-element slot
                assert np.array_equal(pos, 4 * np.arange(16)[:, None] + np.arange(4)[None, :])


@pytest.mark.parametrize("R,K", [(1, 128), (6, 256), (17, 384)])
def test_act32_layout_properties(act_prog, R, K):
    rows, idx = layout(act_prog, R, K, f32=True)
    assert rows == -(-R // 16) * 16
    assert np.array_equal(np.sort(idx.ravel()), np.arange(rows * K))
    g = idx.reshape(rows, K // 4, 4)
    assert np.all(g - g[:, :, :1] == np.arange(4))
    for mt in range(rows // 16):
        for js in range(K // 128):
            for s in range(4):
                for h in range(2):
                    cols = 128 * js + 32 * s + 8 * np.arange(4)[:, None] + 4 * h + np.arange(4)
                    blk = idx[16 * mt:16 * mt + 16][:, cols.ravel()]  # [16, 16]
                    base = blk.min()
                    assert base % 256 == 0 and blk.max() == base + 255
                    pos = (blk[:, ::4] - base) // 4   # [row n, group g] -> 16-byte slot
                    assert np.array_equal(pos, 4 * np.arange(16)[:, None] + np.arange(4)[None, :])
