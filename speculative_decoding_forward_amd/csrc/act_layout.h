// Element order of the bf16 activations the weight GEMMs read as their A operand (the
// normalised inputs, the attention output and the FFN activation).  Rows come in tiles
// of 16 and columns in 128-wide steps of four 32-wide slices: tile mt, step js and slice
// s form one 1 KB block, in which row 16 mt + n, columns 128 js + 32 s + 8 g .. + 8 (the
// 16 bytes that lane 16 g + n of v_mfma_f32_16x16x32_bf16's A operand holds) sit at
// position 4 n + g.  Every A fragment load of a wave is one contiguous 1 KB block, and a
// row's 64 bytes of a slice stay together (one cache line when a launch has one row).
// A tensor of R rows and K columns (K a multiple of 128) spans ceil(R / 16) * 16 * K
// elements.
#pragma once

#include <stddef.h>

#include <hip/hip_runtime.h>

namespace specdec {

__host__ __device__ inline size_t act_index(int r, int k, int K) {
  return ((((size_t)(r >> 4) * (size_t)(K >> 7) + (size_t)(k >> 7)) * 4 + ((k >> 5) & 3)) * 64 +
          (((r & 15) << 2) | ((k >> 3) & 3))) * 8 +
         (k & 7);
}

// fp32 rows of a normalised product's input (x * g, before the row factor) in the same
// tiling: tile mt, step js, slice s and half h (columns 8 g + 4 h .. + 4 of each 8-column
// group) form one 1 KB block, in which row 16 mt + n's four floats of group g sit at
// position 4 n + g.  A lane's 32 bytes of a slice are then two 16-byte loads, each wave
// load one contiguous kilobyte.  A tensor of R rows and K columns spans
// ceil(R / 16) * 16 * K floats.
__host__ __device__ inline size_t act32_index(int r, int k, int K) {
  return (((((size_t)(r >> 4) * (size_t)(K >> 7) + (size_t)(k >> 7)) * 4 + ((k >> 5) & 3)) * 2 +
           ((k >> 2) & 1)) * 64 +
          (((r & 15) << 2) | ((k >> 3) & 3))) * 4 +
         (k & 3);
}

// rows of an activation buffer: R rounded up to whole 16-row tiles
__host__ __device__ inline int act_rows(int R) { return (R + 15) / 16 * 16; }

}  // namespace specdec
