// Shared device helpers for the gfx950 kernels: bf16 <-> fp32, wave64 / block
// reductions, Philox4x64-10.  Wave size is 64 on CDNA4; all reductions use a fixed
// order (no float atomics), so repeated runs are bitwise identical.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPEC_WAVE 64

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

// ------------------------------------------------------------------ bf16 -----------

__device__ __forceinline__ float bf16_to_f32(u16 h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// round-to-nearest-even fp32 -> bf16 with the gfx950 conversion instruction (NaN stays
// NaN); straight-line code, so it never splits a wave's control flow
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  return __builtin_bit_cast(u16, (__bf16)f);
}

// Activation element type of a model: bf16 (stored as u16) or fp32.
template <typename T> struct Act;
template <> struct Act<u16> {
  static __device__ __forceinline__ float load(const u16* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ u16 cvt(float f) { return f32_to_bf16(f); }
};
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float cvt(float f) { return f; }
};

// ------------------------------------------------------------------ reductions -----

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, SPEC_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, SPEC_WAVE));
  return v;
}

// Block-wide sum; `red` is LDS scratch of >= blockDim/64 elements.  Every thread
// gets the result.  Fixed order: waves in index order.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  T t = 0;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

__device__ __forceinline__ int block_or(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, SPEC_WAVE);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < nw; ++i) t |= red[i];
  return t;
}

__device__ __forceinline__ int block_min_int(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, SPEC_WAVE));
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int t = 0x7fffffff;
  for (int i = 0; i < nw; ++i) t = min(t, red[i]);
  return t;
}

__device__ __forceinline__ int block_max_int(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, SPEC_WAVE));
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int t = -0x7fffffff - 1;
  for (int i = 0; i < nw; ++i) t = max(t, red[i]);
  return t;
}

// ------------------------------------------------------------------ Philox ---------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3", SC'11): per round (X0..X3) -> (hi(M1*X2)^X1^k0, lo(M1*X2),
// hi(M0*X0)^X3^k1, lo(M0*X0)); key bumped by the Weyl constants between rounds.

__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                 uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}

// u in [0, 1 - 2^-24]: top 24 bits of word 0 for counter (round, j, b, purpose),
// key (seed, 0).
__device__ __forceinline__ double philox_uniform(uint64_t seed, uint64_t round, uint64_t j,
                                                 uint64_t b, uint64_t purpose) {
  return (double)(philox_word0(round, j, b, purpose, seed, 0) >> 40) * (1.0 / 16777216.0);
}

// LDS exchange among the lanes of ONE wave (no workgroup barrier: other waves of
// the block may have left the kernel).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Device-coherent (agent-scope) relaxed store / load: they bypass the per-XCD L2 for
// data that one workgroup writes and another (possibly on another XCD) reads in the
// same kernel, so no L2 write-back fence is needed.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store_f64(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double coherent_load_f64(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-coherent 8/16-byte accesses through a buffer resource: cache policy sc1
// (device scope), so data written by one workgroup is seen by a workgroup on another
// XCD within the same kernel without an L2 write-back fence.
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
constexpr int kCoherentSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                           0x00020000);
}

// ------------------------------------------------------------------ misc -----------

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }
