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
//   RESID      partial Y of the workgroup's K split -> fp32 buffer; k_resid_norm then
//              adds the splits to the residual stream x in split order and forms
//              h = bf16(RMSNorm(x) * g), the next matrix's input
//
// fp32 path (small fp32 models): separate simple kernels, one wave per output column.
#include <hip/hip_ext.h>

#include <algorithm>
#include <math.h>

#include "common.h"
#include "internal.h"

namespace specdec {

#ifndef SPEC_GEMM_WAVES
#define SPEC_GEMM_WAVES 4  // streaming waves per workgroup (plus one epilogue wave)
#endif
#ifndef SPEC_GEMM_RING
#define SPEC_GEMM_RING 2
#endif
#ifndef SPEC_GEMM_WPC
#define SPEC_GEMM_WPC 2  // resident workgroups per compute unit the grid is sized for
#endif
constexpr int GW = SPEC_GEMM_WAVES;  // streaming waves per workgroup
constexpr int GT = (GW + 1) * 64;    // threads per workgroup

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

// Packed weight layout.  A matrix is stored as a sequence of column tiles, each the
// 16 weight rows behind 16 output columns; tile t, super-step j (k in [128j, 128j+128)),
// MFMA slice s (k in [128j + 32s, +32)) and lane l hold, contiguously,
//   row(t, l % 16)[128j + 32s + 8(l / 16) .. +8]
// at element offset (((t * K/128 + j) * 4 + s) * 64 + l) * 8, i.e. exactly the B operand
// of v_mfma_f32_16x16x32_bf16 for that slice.  Every wave load is then 1 KB contiguous
// and a tile is one contiguous 32*K-byte block.  Which weight row sits behind local
// column c of tile t depends on the epilogue that consumes the tile:
//   QKV_ROPE  c < 8: row base + c, c >= 8: row base + hd/2 + c - 8 of the fused [3d, d]
//             matrix, base = sec*d + h*hd + i0 (RoPE pairs (i, i + hd/2) meet in a tile)
//   SWIGLU    c < 8: gate row 8t + c, c >= 8: up row 8t + c - 8 (silu(g) * u meets)
//   others    row 16t + c
struct QkvTile {
  int sec, h, i0;  // section (0 q, 1 k, 2 v), head, first rotation index of the tile
};
__device__ __forceinline__ QkvTile qkv_tile(int t, int d, int hd) {
  const int half = hd >> 1, per_head = half / 8, per_sec = d / 16;
  QkvTile q;
  q.sec = t / per_sec;
  const int rem = t - q.sec * per_sec;
  q.h = rem / per_head;
  q.i0 = 8 * (rem - q.h * per_head);
  return q;
}

// Pack src [rows, K] (row-major bf16) into the tile layout above.  mode: PACK_PLAIN,
// PACK_QKV (src is the fused [3d, d] matrix), PACK_PAIR_LO / PACK_PAIR_HI (src fills the
// c < 8 / c >= 8 half of tiles of 8 rows).  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void k_pack_bf16(const u16* __restrict__ src, int K, int mode,
                                                   int d, int hd, int ntiles,
                                                   u16* __restrict__ dst) {
  const int J = K >> 7;
  const size_t chunks = (size_t)ntiles * J * 256;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks;
       q += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(q & 63), s = (int)((q >> 6) & 3);
    const size_t tj = q >> 8;
    const int j = (int)(tj % J), t = (int)(tj / J);
    const int c = l & 15;
    int row;
    if (mode == PACK_QKV) {
      const QkvTile qt = qkv_tile(t, d, hd);
      const int base = qt.sec * d + qt.h * hd + qt.i0;
      row = c < 8 ? base + c : base + (hd >> 1) + c - 8;
    } else if (mode == PACK_PAIR_LO) {
      if (c >= 8) continue;
      row = 8 * t + c;
    } else if (mode == PACK_PAIR_HI) {
      if (c < 8) continue;
      row = 8 * t + c - 8;
    } else {
      row = 16 * t + c;
    }
    const int k = 128 * j + 32 * s + 8 * (l >> 4);
    *reinterpret_cast<uint4*>(dst + q * 8) =
        *reinterpret_cast<const uint4*>(src + (size_t)row * K + k);
  }
}

hipError_t launch_pack_bf16(const uint16_t* src, int K, int mode, int d, int hd, int ntiles,
                            uint16_t* dst, hipStream_t s) {
  if (K % 128 || ntiles < 1) return hipErrorInvalidValue;
  const size_t chunks = (size_t)ntiles * (K >> 7) * 256;
  const int blocks = (int)std::min<size_t>((chunks + 255) / 256, 8192);
  k_pack_bf16<<<blocks, 256, 0, s>>>(src, K, mode, d, hd, ntiles, dst);
  return hipGetLastError();
}

// Per-tile epilogue, run by the workgroup's epilogue wave.  part[w][mt][lane] holds
// wave w's MFMA accumulator fragment of row tile mt: lane l has rows 4(l/16)+e
// (e = 0..3) of local column l%16.  The GW partials are summed in wave order.
// rowinfo[rr] = (absolute position, flags) of row r0 + rr: flag 1 = a real token of its
// sequence, flag 2 = its K/V may be written (real token and position < max_len).
template <int MT>
__device__ __forceinline__ void gemm_tile_epilogue(const GemmArgs& g, int t, int r0,
                                                   const floatx4 (*part)[MT][64],
                                                   const int2* rowinfo, int lane) {
  const int nl = lane & 15, gq = lane >> 4, R = g.R, mode = g.mode;
  const bool is_hi = nl >= 8;
  int sec = 0, h = 0, i = 0;
  const int half = g.hd >> 1;
  if (mode == EPI_QKV_ROPE) {
    const QkvTile qt = qkv_tile(t, g.d, g.hd);
    sec = qt.sec;
    h = qt.h;
    i = qt.i0 + (nl & 7);
  }
#pragma unroll 1
  for (int mt = 0; mt < MT; ++mt) {
    // rotation factors of this lane's four rows, loaded together (one latency)
    double cs[4], sn[4];
    if (mode == EPI_QKV_ROPE && sec < 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // rows past a sequence's tokens may sit past max_len: their q is never used
        const int pos = min(rowinfo[mt * 16 + 4 * gq + e].x, g.max_len - 1);
        const double2 c2 = *reinterpret_cast<const double2*>(g.rope_cs +
                                                             ((size_t)pos * half + i) * 2);
        cs[e] = c2.x;
        sn[e] = c2.y;
      }
    }
    floatx4 v = part[0][mt][lane];
#pragma unroll
    for (int w = 1; w < GW; ++w) {
      const floatx4 p = part[w][mt][lane];
      v[0] += p[0]; v[1] += p[1]; v[2] += p[2]; v[3] += p[3];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = mt * 16 + 4 * gq + e, r = r0 + rr;
      const float y = v[e];
      const float yp = __shfl_xor(y, 8);  // the paired column c ^ 8 of the same row
      if (r >= R) continue;
      switch (mode) {
        case EPI_QKV_ROPE: {
          const float lo = is_hi ? yp : y, hi = is_hi ? y : yp;
          u16 o;
          if (sec < 2) {
            o = is_hi ? f32_to_bf16((float)((double)hi * cs[e] + (double)lo * sn[e]))
                      : f32_to_bf16((float)((double)lo * cs[e] - (double)hi * sn[e]));
          } else {
            o = f32_to_bf16(y);
          }
          const int ii = is_hi ? i + half : i;
          if (sec == 0) {
            g.q_out[(size_t)r * g.d + h * g.hd + ii] = o;
          } else {
            const int2 info = rowinfo[rr];
            if (info.y & 2) {
              const int b = r / g.M;
              ((sec == 1) ? g.kc : g.vc)[(size_t)b * g.row_stride + (size_t)h * g.head_stride +
                                         (sec == 1 ? kv_k_offset(info.x, ii, g.hd)
                                                   : kv_v_offset(info.x, ii, g.hd))] = o;
            }
          }
          break;
        }
        case EPI_SWIGLU:
          if (!is_hi)
            g.act_out[(size_t)r * g.N1 + 8 * t + nl] = f32_to_bf16(y / (1.f + expf(-y)) * yp);
          break;
        case EPI_GELU:
          g.act_out[(size_t)r * g.N + 16 * t + nl] =
              f32_to_bf16(0.5f * y * (1.f + erff(y * 0.70710678118654752f)));
          break;
        case EPI_STORE:
          g.C[(size_t)r * g.ldc + 16 * t + nl] = (rowinfo[rr].y & 1) ? y : 0.f;
          break;
        default:  // EPI_RESID: Y -> C; the row-norm kernel adds it to x
          g.C[(size_t)r * g.ldc + 16 * t + nl] = y;
          break;
      }
    }
  }
}

// Persistent weight-streaming GEMM.  Workgroup (bx, by) owns row block by (MT*16 rows
// of A) and the column tiles bx, bx + G, bx + 2G, ... (G = gridDim.x).  It has GW
// streaming waves and one epilogue wave.  The streaming waves split K: wave wv takes
// 128-wide super-steps wv, wv + GW, ... of every tile, so its steps form one flat
// stream over (tile, step) and its register ring of P steps runs across tile
// boundaries.  At the end of a tile each streaming wave parks its accumulator in LDS
// (double-buffered by tile parity) and meets the others at one barrier; the epilogue
// wave then sums the partials and runs the epilogue (with its own global loads and
// stores) while the streaming waves go on with the next tile.  A streaming wave thus
// never waits on anything but its own weight loads.
template <int MT>
__global__ __launch_bounds__(GT) void k_gemm_bf16(GemmArgs g) {
  constexpr int P = MT <= 2 ? SPEC_GEMM_RING : (SPEC_GEMM_RING > 2 ? 2 : SPEC_GEMM_RING);
  __shared__ floatx4 part[2][GW][MT][64];
  __shared__ int2 rowinfo[MT * 16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bx = blockIdx.x, G = gridDim.x;
  const int r0 = blockIdx.y * (MT * 16);
  const int nt = (g.ntiles - bx + G - 1) / G;  // tiles of this workgroup (>= 1)
  if (wv == GW) {
    for (int rr = lane; rr < MT * 16; rr += 64) {
      const int r = r0 + rr;
      int2 info{0, 0};
      if (r < g.R) {
        const int b = r / g.M, j = r - b * g.M;
        const int n = g.ntok_eff ? g.ntok_eff[b] : g.M;
        const int pos = (g.pos0 ? g.pos0[b] : 0) + j;
        info = int2{pos, (j < n ? 1 : 0) | (j < n && pos < g.max_len ? 2 : 0)};
      }
      rowinfo[rr] = info;
    }
    wave_lds_sync();
    for (int ct = 0; ct < nt; ++ct) {
      __syncthreads();
      gemm_tile_epilogue<MT>(g, bx + ct * G, r0, part[ct & 1], rowinfo, lane);
    }
    return;
  }
  const int nl = lane & 15, gq = lane >> 4;
  const int R = g.R, nsuper = g.K >> 7;
  const int S = (nsuper + GW - 1) / GW;  // steps per tile, the same for every wave
  const bool wact = wv < nsuper;
  const int last_step = wact ? (nsuper - 1 - wv) / GW : 0;
  const size_t tile_elems = (size_t)nsuper * 2048;  // one packed tile
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

  bf16x8 wf[P][4];
  bf16x8 af[P][MT][4];
  const u16* zblk = g.zeros;
  // issue stream: tile iteration it, step is; a step past the wave's last one in a tile,
  // or past the workgroup's last tile, re-reads an in-bounds W segment (cache hit) and
  // pairs it with zero A fragments, so every wave runs the same branch-free schedule.
  int it = 0, is = 0;
  const u16* wp = g.W + (size_t)bx * tile_elems + 8 * lane;
  auto issue = [&](int slot) {
    const bool valid = is <= last_step && wact && it < nt;
    const int js = wact ? wv + (is <= last_step ? is : last_step) * GW : 0;  // super-step
    const int kb = js * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) wf[slot][s] = ld8_nt(wp + js * 2048 + 512 * s, true);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        af[slot][mt][s] = ld8((valid && aok[mt]) ? arow[mt] + kb + 32 * s : zblk, true);
    if (++is == S) {
      is = 0;
      ++it;
      if (it < nt) wp += (size_t)G * tile_elems;
    }
  };
  int ct = 0, cs = 0;  // consume stream: tile iteration, step
  auto consume = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[slot][mt][s], wf[slot][s],
                                                          acc[mt], 0, 0, 0);
    if (++cs == S) {
      cs = 0;
      if (ct < nt) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) part[ct & 1][wv][mt][lane] = acc[mt];
        __syncthreads();
      }
      ++ct;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Rounds of P steps; the last round's refills read in-bounds W past the end (cache
  // hits, never consumed) so that the loop body is the only copy of the tile code.
  const int F = nt * S;  // steps of this wave
  const int T = (F + P - 1) / P;
#pragma unroll
  for (int u = 0; u < P; ++u) issue(u);
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      consume(u);
      issue(u);
      // keep each refill right behind the use of its slot (no drain per round)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Residual update and RMSNorm of the next matrix's input, one 256-thread block per row:
//   x[r] += y[r];  h[r] = bf16(x[r] * g / rms(x[r]))
// with the sum of squares and the scaling in fp64.
__global__ __launch_bounds__(256) void k_resid_norm(float* __restrict__ x,
                                                    const float* __restrict__ y, int R, int d,
                                                    const float* __restrict__ gain, float eps,
                                                    u16* __restrict__ h) {
  __shared__ double red[4];
  const int r = blockIdx.x;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)r * d);
  const float4* yr = reinterpret_cast<const float4*>(y + (size_t)r * d);
  double sq = 0.0;
  for (int i = threadIdx.x; i < d / 4; i += 256) {
    float4 v = xr[i];
    const float4 p = yr[i];
    v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
    xr[i] = v;
    sq += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
  }
  sq = block_sum(sq, red);
  const double inv = 1.0 / sqrt(sq / d + (double)eps);
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

hipError_t launch_resid_norm(float* x, const float* y, int R, int d, const float* gain,
                             float eps, uint16_t* h, hipStream_t s) {
  k_resid_norm<<<R, 256, 0, s>>>(x, y, R, d, gain, eps, h);
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

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Grid: G persistent workgroups per row block, G chosen so that the tiles divide as
// evenly as possible (every workgroup gets ceil(tiles / G) or one fewer).
hipError_t launch_gemm_bf16(const GemmArgs& g0, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  GemmArgs g = g0;
  g.ntiles = gemm_blocks_x(g);
  const int tiles = cdiv(g.R, 16);
  const int rowblocks = tiles <= 3 ? 1 : cdiv(g.R, 64);
  const int gmax = std::max(1, device_cus() * SPEC_GEMM_WPC / rowblocks);
  const int per = cdiv(g.ntiles, gmax);
  const int G = cdiv(g.ntiles, per);
  if (tiles <= 1) {
    hipExtLaunchKernelGGL(k_gemm_bf16<1>, dim3(G), dim3(GT), 0, s, e0, e1, 0, g);
  } else if (tiles <= 2) {
    hipExtLaunchKernelGGL(k_gemm_bf16<2>, dim3(G), dim3(GT), 0, s, e0, e1, 0, g);
  } else if (tiles <= 3) {
    hipExtLaunchKernelGGL(k_gemm_bf16<3>, dim3(G), dim3(GT), 0, s, e0, e1, 0, g);
  } else {
    hipExtLaunchKernelGGL(k_gemm_bf16<4>, dim3(G, rowblocks), dim3(GT), 0, s, e0, e1, 0, g);
  }
  return hipGetLastError();
}


}  // namespace specdec
