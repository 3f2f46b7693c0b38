// Weight-streaming skinny GEMM for the verify pass: Y[R, N] = A[R, K] . W[N, K]^T with
// R = rows of the call (K+1 per sequence, times the batch) and W row-major [out, in],
// plus the fused epilogues of each matrix of a layer.
//
// Why this shape: one target call scores K+1 positions while reading every weight
// from HBM once ([ZSM] "The cost of one token is the cost of reading the weights" and
// "One pass can score many tokens"; [GC] "Why Standard Decoding Is Slow").  With R <= 64
// the arithmetic intensity is ~R FLOP/byte, far below the matrix-core ridge, so the
// kernel is built to keep HBM busy: each weight byte is loaded once with many loads in
// flight; the matrix cores are used because the work is a dense contraction (R rows
// padded to 16-row MFMA tiles), not because they bound the time.
//
// bf16 path: v_mfma_f32_16x16x32_bf16.  A workgroup of 8 waves owns 16 output columns
// (16 rows of W) and up to 64 rows of A; the waves split K in 128-wide super-steps,
// round-robin, and the 8 fp32 partials are summed in LDS in a fixed order.  In a
// super-step, MFMA s (s = 0..3) covers k in [128i + 32s, 128i + 32s + 32) and lane l
// holds W row (l % 16), elements 8(l / 16) .. +8 of that range, so one load
// instruction reads 64 contiguous bytes of each of 16 rows.  Each wave keeps PF
// super-steps of W loads in flight (a register ring, statically indexed).
//
// Epilogues (selected per launch):
//   STORE      Y -> fp32 C (rows past a sequence's token count stored as 0): LM head
//   QKV_ROPE   columns paired (i, i + hd/2) inside a head; RoPE at the row's absolute
//              position (angle pos * theta^(-2i/hd), fp64), q -> bf16 buffer, k and v ->
//              the KV cache at the row's position
//   SWIGLU     columns paired (gate n, up n): a = bf16(silu(g) * u)
//   GELU       a = bf16(gelu(y)), erf form
//   RESID      x += Y (fp32 residual stream) and per-workgroup row sums of squares of
//              the new x (fp64), from which k_rownorm forms h = bf16(RMSNorm(x) * g), the
//              next matrix's input
//
// fp32 path (small fp32 models): separate simple kernels, one wave per output column.
#include <hip/hip_ext.h>
#include <math.h>

#include "common.h"
#include "internal.h"

namespace specdec {

constexpr int GW = 8;        // waves per workgroup
constexpr int GT = GW * 64;  // threads per workgroup
constexpr int PF = 4;        // super-steps of W in flight per wave

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

// Global column of local column c (0..15) of workgroup bx.
__device__ __forceinline__ int gemm_col(const GemmArgs& g, int bx, int c) {
  switch (g.mode) {
    case EPI_QKV_ROPE: {
      const int half = g.hd >> 1, per_head = half / 8, per_sec = g.d / 16;
      const int sec = bx / per_sec, rem = bx % per_sec;
      const int h = rem / per_head, i0 = 8 * (rem % per_head);
      return sec * g.d + h * g.hd + i0 + (c < 8 ? c : half + c - 8);
    }
    case EPI_SWIGLU:
      return (c < 8 ? 0 : g.N1) + 8 * bx + (c & 7);
    default:
      return bx * 16 + c;
  }
}

__device__ __forceinline__ const u16* gemm_wrow(const GemmArgs& g, int col) {
  return col < g.N1 ? g.W + (size_t)col * g.K : g.W2 + (size_t)(col - g.N1) * g.K;
}

template <int MT>
__global__ __launch_bounds__(GT) void k_gemm_bf16(GemmArgs g) {
  constexpr int P = MT <= 2 ? 4 : 2;  // super-steps of W and A in flight per wave
  __shared__ float red[GW][MT * 16][17];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bx = blockIdx.x;
  const int r0 = blockIdx.y * (MT * 16);
  const int nl = lane & 15, gq = lane >> 4;
  const int K = g.K, R = g.R;
  const u16* wrow = gemm_wrow(g, gemm_col(g, bx, nl)) + 8 * gq;
  const u16* arow[MT];
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = r0 + mt * 16 + nl;
    aok[mt] = r < R;
    arow[mt] = g.A + (size_t)(aok[mt] ? r : 0) * g.lda + 8 * gq;
  }
  floatx4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // K is a multiple of 128.  Wave wv owns super-steps wv, wv + GW, ...; every wave runs
  // the same trip count S = ceil(nsuper / GW) so the loop body has no branches (the
  // compiler then keeps every slot of the ring in flight across iterations).  A step
  // past the wave's last one re-reads the wave's last W segment (already in cache, no
  // HBM traffic) and multiplies it by a zero A fragment.
  const int nsuper = K >> 7;
  const int S = (nsuper + GW - 1) / GW;
  const int last_step = nsuper > wv ? (nsuper - 1 - wv) / GW : 0;
  bf16x8 wf[P][4];
  bf16x8 af[P][MT][4];
  // invalid A fragments are read from a zeroed 16-byte block (an address select, so the
  // loaded data is never waited on before the MFMA that uses it)
  const u16* zblk = g.zeros;
  auto issue = [&](int slot, int step) {
    const bool valid = step <= last_step && wv < nsuper;
    // waves without any step of their own read the first segment (in bounds) times 0
    const int kb = wv < nsuper ? (wv + (valid ? step : last_step) * GW) * 128 : 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) wf[slot][s] = ld8_nt(wrow + kb + 32 * s, true);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        af[slot][mt][s] = ld8((valid && aok[mt]) ? arow[mt] + kb + 32 * s : zblk, true);
  };
  auto consume = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[slot][mt][s], wf[slot][s],
                                                          acc[mt], 0, 0, 0);
  };
  const int T = (S + P - 1) / P;  // rounds of P steps
#pragma unroll
  for (int u = 0; u < P; ++u) issue(u, u);
  for (int t = 0; t + 1 < T; ++t) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      consume(u);
      issue(u, (t + 1) * P + u);
      // keep each refill right behind the use of its slot (no drain per round)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < P; ++u) consume(u);
  // D layout: lane holds rows 4*gq .. 4*gq+3 of each tile, column nl
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wv][mt * 16 + 4 * gq + e][nl] = acc[mt][e];
  __syncthreads();
  // sum the wave partials in place (fixed order) into red[0]
  for (int idx = threadIdx.x; idx < MT * 16 * 16; idx += GT) {
    const int rr = idx >> 4, c = idx & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < GW; ++w) v += red[w][rr][c];
    red[0][rr][c] = v;
  }
  __syncthreads();

  const int mode = g.mode;
  if (mode == EPI_QKV_ROPE || mode == EPI_SWIGLU) {
    // pairs: local columns c and c + 8
    for (int idx = threadIdx.x; idx < MT * 16 * 8; idx += GT) {
      const int rr = idx >> 3, c = idx & 7;
      const int r = r0 + rr;
      if (r >= R) continue;
      const float lo = red[0][rr][c], hi = red[0][rr][c + 8];
      if (mode == EPI_SWIGLU) {
        const int col = 8 * bx + c;
        const float v = lo / (1.f + expf(-lo)) * hi;
        g.act_out[(size_t)r * g.N1 + col] = f32_to_bf16(v);
        continue;
      }
      const int half = g.hd >> 1, per_head = half / 8, per_sec = g.d / 16;
      const int sec = bx / per_sec, rem = bx % per_sec;
      const int h = rem / per_head, i = 8 * (rem % per_head) + c;
      const int b = r / g.M, j = r % g.M;
      const int pos = g.pos0[b] + j;
      u16 o0, o1;
      if (sec < 2) {
        const double inv_freq = pow((double)g.theta, -2.0 * (double)i / (double)g.hd);
        double sn, cs;
        sincos((double)pos * inv_freq, &sn, &cs);
        o0 = f32_to_bf16((float)((double)lo * cs - (double)hi * sn));
        o1 = f32_to_bf16((float)((double)hi * cs + (double)lo * sn));
      } else {
        o0 = f32_to_bf16(lo);
        o1 = f32_to_bf16(hi);
      }
      if (sec == 0) {
        u16* qo = g.q_out + (size_t)r * g.d + h * g.hd;
        qo[i] = o0;
        qo[i + half] = o1;
      } else if (j < g.ntok_eff[b] && pos < g.max_len) {
        u16* cp = (sec == 1 ? g.kc : g.vc) + (size_t)b * g.row_stride +
                  (size_t)h * g.head_stride + (size_t)pos * g.hd;
        cp[i] = o0;
        cp[i + half] = o1;
      }
    }
    return;
  }
  if (mode != EPI_RESID) {
    for (int idx = threadIdx.x; idx < MT * 16 * 16; idx += GT) {
      const int rr = idx >> 4, c = idx & 15;
      const int r = r0 + rr;
      if (r >= R) continue;
      const int col = bx * 16 + c;
      const float v = red[0][rr][c];
      if (mode == EPI_STORE) {
        const bool pad = g.ntok_eff && (r % g.M) >= g.ntok_eff[r / g.M];
        g.C[(size_t)r * g.ldc + col] = pad ? 0.f : v;
      } else {  // EPI_GELU
        g.act_out[(size_t)r * g.N + col] =
            f32_to_bf16(0.5f * v * (1.f + erff(v * 0.70710678118654752f)));
      }
    }
    return;
  }
  // EPI_RESID: x += Y, plus this workgroup's share of each row's sum of squares of the
  // new x (one wave per row, lanes 0..15 over the 16 columns) in ss_part[bx][r] (fp64);
  // the row-norm kernel that follows turns them into the next matrix's input.
  for (int rr = wv; rr < MT * 16; rr += GW) {
    const int r = r0 + rr;
    if (r >= R) continue;
    double sq = 0.0;
    if (lane < 16) {
      float* p = g.C + (size_t)r * g.ldc + bx * 16 + lane;
      const float nv = *p + red[0][rr][lane];
      *p = nv;
      sq = (double)nv * nv;
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
    if (lane == 0) g.ss_part[(size_t)bx * R + r] = sq;
  }
}

// h[r] = bf16(x[r] * rsqrt(sum_sq[r] / d + eps) * g): one 256-thread block per row; the
// row's sum of squares is the fixed-order sum of the GEMM workgroups' partials.
__global__ __launch_bounds__(256) void k_rownorm(const float* __restrict__ x,
                                                 const double* __restrict__ ss_part, int nparts,
                                                 int R, int d, const float* __restrict__ gain,
                                                 float eps, u16* __restrict__ h) {
  __shared__ double red[4];
  const int r = blockIdx.x;
  double sq = 0.0;
  for (int j = threadIdx.x; j < nparts; j += 256) sq += ss_part[(size_t)j * R + r];
  sq = block_sum(sq, red);
  const double inv = 1.0 / sqrt(sq / d + (double)eps);
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)r * d);
  const float4* gr = reinterpret_cast<const float4*>(gain);
  uint2* hr = reinterpret_cast<uint2*>(h + (size_t)r * d);
  for (int i = threadIdx.x; i < d / 4; i += 256) {
    const float4 v = xr[i], gg = gr[i];
    const uint32_t a = f32_to_bf16((float)((double)v.x * inv * (double)gg.x)) |
                       ((uint32_t)f32_to_bf16((float)((double)v.y * inv * (double)gg.y)) << 16);
    const uint32_t b = f32_to_bf16((float)((double)v.z * inv * (double)gg.z)) |
                       ((uint32_t)f32_to_bf16((float)((double)v.w * inv * (double)gg.w)) << 16);
    hr[i] = uint2{a, b};
  }
}

hipError_t launch_rownorm(const float* x, const double* ss_part, int nparts, int R, int d,
                          const float* gain, float eps, uint16_t* h, hipStream_t s) {
  k_rownorm<<<R, 256, 0, s>>>(x, ss_part, nparts, R, d, gain, eps, h);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32 path -----

// fp32: one wave per output column n, lanes stride K; rows looped.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, const float* __restrict__ W,
                                                  const float* __restrict__ W2, int N1, int N,
                                                  int R, int K, float* __restrict__ C, int ldc,
                                                  int accumulate, const int32_t* __restrict__ ntok_eff,
                                                  int M) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* wrow = n < N1 ? W + (size_t)n * K : W2 + (size_t)(n - N1) * K;
  for (int r = 0; r < R; ++r) {
    const float* arow = A + (size_t)r * K;
    float s = 0.f;
    for (int k = lane; k < K; k += 64) s = fmaf(arow[k], wrow[k], s);
    s = wave_sum(s);
    if (lane == 0) {
      float* p = C + (size_t)r * ldc + n;
      if (ntok_eff && (r % M) >= ntok_eff[r / M]) s = 0.f;
      if (accumulate) *p += s;
      else *p = s;
    }
  }
}

hipError_t launch_gemm_f32(const float* A, const float* W, const float* W2, int N1, int R,
                           int N, int K, float* C, int accumulate, const int32_t* ntok_eff,
                           int M, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (!W2) { W2 = W; N1 = N; }
  hipExtLaunchKernelGGL(k_gemm_f32, dim3(cdiv(N, 4)), dim3(256), 0, s, e0, e1, 0, A, W, W2,
                        N1, N, R, K, C, N, accumulate, ntok_eff, M);
  return hipGetLastError();
}

int gemm_blocks_x(const GemmArgs& g) {
  switch (g.mode) {
    case EPI_QKV_ROPE: return 3 * g.d / 16;
    case EPI_SWIGLU: return g.N1 / 8;
    default: return g.N / 16;
  }
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int tiles = cdiv(g.R, 16);
  const int bx = gemm_blocks_x(g);
  if (tiles <= 1) {
    hipExtLaunchKernelGGL(k_gemm_bf16<1>, dim3(bx, 1), dim3(GT), 0, s, e0, e1, 0, g);
  } else if (tiles <= 2) {
    hipExtLaunchKernelGGL(k_gemm_bf16<2>, dim3(bx, 1), dim3(GT), 0, s, e0, e1, 0, g);
  } else if (tiles <= 3) {
    hipExtLaunchKernelGGL(k_gemm_bf16<3>, dim3(bx, 1), dim3(GT), 0, s, e0, e1, 0, g);
  } else {
    hipExtLaunchKernelGGL(k_gemm_bf16<4>, dim3(bx, cdiv(g.R, 64)), dim3(GT), 0, s, e0, e1, 0, g);
  }
  return hipGetLastError();
}

}  // namespace specdec
