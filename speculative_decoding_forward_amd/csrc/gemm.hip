// Weight-streaming skinny GEMM for the verify pass: C[R, N] (+)= A[R, K] . W[N, K]^T
// with R = (K+1) * batch <= 64 rows per launch tile, W row-major [out, in].
//
// Why this shape: one target call scores K+1 positions while reading every weight
// from HBM once ([ZSM] "The cost of one token is the cost of reading the weights" and
// "One pass can score many tokens"; [GC] "Why Standard Decoding Is Slow").  The
// arithmetic intensity is ~R FLOP/byte, far below the MFMA ridge, so the kernel is
// built to keep HBM busy: every weight byte is loaded once, 64 contiguous bytes per
// lane per row, with many loads in flight; the matrix cores are used only because
// the work is a dense contraction (R rows padded to 16-row MFMA tiles).
//
// bf16 path: v_mfma_f32_16x16x32_bf16.  A workgroup of 8 waves owns 16 output
// columns (16 rows of W) and all R rows; the 8 waves split K in 128-wide
// super-steps round-robin and their fp32 partials are summed in LDS in a fixed order.
// Within a super-step lane l (row n = l % 16, group g = l / 16) loads W[n][k0 + 32g ..
// k0 + 32g + 32) and the matching 32 elements of each A row; MFMA s (s = 0..3) takes
// elements 8s..8s+7 of every lane's chunk.  This permutes k identically for A and W,
// so each MFMA still sums over k, and each W row segment is read as 64 contiguous
// bytes per lane (256 contiguous bytes per row per super-step).
//
// fp32 path (small fp32 models): one wave per output column, lanes across K.
#include "common.h"
#include "internal.h"

namespace specdec {

constexpr int GW = 8;        // waves per workgroup
constexpr int GT = GW * 64;  // threads per workgroup

// Epilogue of one output element.  mode 0: C = v; mode 1: C += v.
// rows_per_seq / ntok_eff (optional): rows r with (r % rows_per_seq) >= ntok_eff[r /
// rows_per_seq] are written as 0 (padding rows of a ragged batch).
struct Epi {
  float* C;
  int ldc;
  int mode;
  const int32_t* ntok_eff;
  int rows_per_seq;
};

__device__ __forceinline__ void epi_store(const Epi& e, int r, int n, float v) {
  float* p = e.C + (size_t)r * e.ldc + n;
  if (e.ntok_eff && (r % e.rows_per_seq) >= e.ntok_eff[r / e.rows_per_seq]) v = 0.f;
  if (e.mode == 1) *p += v;
  else *p = v;
}

// 16 bytes of bf16 at p (8 elements) or zeros if the range is out of bounds.
__device__ __forceinline__ bf16x8 ld8(const u16* p, bool ok) {
  if (!ok) return bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 ld8_nt(const u16* p, bool ok) {
  if (!ok) return bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return __builtin_bit_cast(bf16x8, u);
}

// MT = number of 16-row M tiles (R <= 16 * MT within this launch's row block).
template <int MT>
__global__ __launch_bounds__(GT) void k_gemm_bf16(const u16* __restrict__ A, int lda,
                                                  const u16* __restrict__ W,
                                                  const u16* __restrict__ W2, int N1, int R,
                                                  int K, Epi epi) {
  __shared__ float red[GW][MT * 16][17];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int r0 = blockIdx.y * (MT * 16);
  const int nl = lane & 15, g = lane >> 4;
  // W row owned by this lane (two-matrix case: rows >= N1 come from W2)
  const u16* wrow = n0 < N1 ? W + (size_t)(n0 + nl) * K : W2 + (size_t)(n0 - N1 + nl) * K;
  const u16* arow[MT];
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = r0 + mt * 16 + nl;
    aok[mt] = r < R;
    arow[mt] = A + (size_t)(aok[mt] ? r : 0) * lda;
  }
  floatx4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nsuper = (K + 127) / 128;
  for (int ss = wv; ss < nsuper; ss += GW) {
    const int kb = ss * 128 + g * 32;
    bf16x8 wf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) wf[s] = ld8_nt(wrow + kb + 8 * s, kb + 8 * s + 8 <= K);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      bf16x8 af[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) af[s] = ld8(arow[mt] + kb + 8 * s, aok[mt] && kb + 8 * s + 8 <= K);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], wf[s], acc[mt], 0, 0, 0);
    }
  }
  // D layout: lane holds rows 4g..4g+3 of the tile, column nl
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wv][mt * 16 + 4 * g + e][nl] = acc[mt][e];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * 16 * 16; idx += GT) {
    const int rr = idx >> 4, c = idx & 15;
    const int r = r0 + rr;
    if (r >= R) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < GW; ++w) v += red[w][rr][c];
    epi_store(epi, r, n0 + c, v);
  }
}

// fp32: one wave per output column n, lanes stride K; rows looped.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, int lda,
                                                  const float* __restrict__ W,
                                                  const float* __restrict__ W2, int N1, int N,
                                                  int R, int K, Epi epi) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* wrow = n < N1 ? W + (size_t)n * K : W2 + (size_t)(n - N1) * K;
  for (int r = 0; r < R; ++r) {
    const float* arow = A + (size_t)r * lda;
    float s = 0.f;
    for (int k = lane; k < K; k += 64) s = fmaf(arow[k], wrow[k], s);
    s = wave_sum(s);
    if (lane == 0) epi_store(epi, r, n, s);
  }
}

// dtype: SPEC_DT_BF16 or SPEC_DT_F32.  W2/N1: rows n >= N1 of the logical [N, K]
// matrix come from W2 (row n - N1); pass W2 = W, N1 = N for a single matrix.
hipError_t launch_gemm_ex(int dtype, const void* A, const void* W, const void* W2, int R,
                          int N, int N1, int K, float* C, int accumulate,
                          const int32_t* ntok_eff, int rows_per_seq, hipStream_t s) {
  Epi epi{C, N, accumulate ? 1 : 0, ntok_eff, rows_per_seq > 0 ? rows_per_seq : 1};
  if (!W2) { W2 = W; N1 = N; }
  if (dtype == SPEC_DT_F32) {
    k_gemm_f32<<<cdiv(N, 4), 256, 0, s>>>((const float*)A, K, (const float*)W,
                                          (const float*)W2, N1, N, R, K, epi);
    return hipGetLastError();
  }
  const int tiles = cdiv(R, 16);
  const dim3 grid(N / 16, 1);
  if (tiles <= 1) {
    k_gemm_bf16<1><<<grid, GT, 0, s>>>((const u16*)A, K, (const u16*)W, (const u16*)W2, N1, R, K, epi);
  } else if (tiles <= 2) {
    k_gemm_bf16<2><<<grid, GT, 0, s>>>((const u16*)A, K, (const u16*)W, (const u16*)W2, N1, R, K, epi);
  } else if (tiles <= 3) {
    k_gemm_bf16<3><<<grid, GT, 0, s>>>((const u16*)A, K, (const u16*)W, (const u16*)W2, N1, R, K, epi);
  } else {
    const dim3 g4(N / 16, cdiv(R, 64));
    k_gemm_bf16<4><<<g4, GT, 0, s>>>((const u16*)A, K, (const u16*)W, (const u16*)W2, N1, R, K, epi);
  }
  return hipGetLastError();
}

}  // namespace specdec
