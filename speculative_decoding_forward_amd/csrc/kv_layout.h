// Element order of the packed bf16 KV cache (written by the QKV GEMM's epilogue, read
// by the attention kernel).
#pragma once

#include <stddef.h>

#include <hip/hip_runtime.h>

namespace specdec {

// Packed bf16 cache: element offsets inside one head region (see attention.hip).
__host__ __device__ inline size_t kv_k_offset(int p, int i, int hd) {
  return ((size_t)(p >> 4) * (hd >> 5) + (i >> 5)) * 512 + (((i & 31) >> 3) * 16 + (p & 15)) * 8 +
         (i & 7);
}
__host__ __device__ inline size_t kv_v_offset(int p, int i, int hd) {
  const int pk = p & 31;
  const int g = (pk & 15) >> 2, e = (pk & 3) + ((pk >> 4) << 2);
  return ((size_t)(p >> 5) * (hd >> 4) + (i >> 4)) * 512 + (g * 16 + (i & 15)) * 8 + e;
}
// positions a bf16 head region holds (max_len rounded up to whole 32-key blocks)
inline int kv_capacity(int max_len) { return (max_len + 31) / 32 * 32; }

}  // namespace specdec
