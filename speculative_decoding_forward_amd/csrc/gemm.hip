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
// bf16 path: v_mfma_f32_16x16x32_bf16.  A workgroup has 4 streaming waves and one
// epilogue wave; it owns column tiles of 16 output columns (16 rows of W) and up to 64
// rows of A.  The streaming waves split K in 128-wide super-steps, round-robin, and
// their fp32 partials are summed in LDS in a fixed order.  In a super-step, MFMA s
// (s = 0..3) covers k in [128i + 32s, 128i + 32s + 32) and lane l holds W row (l % 16),
// elements 8(l / 16) .. +8 of that range; with the packed layout below one load
// instruction reads 1 KB contiguous.  Each wave requests the super-step ahead before
// multiplying the current one (a register ring, statically indexed).
//
// Epilogues (selected per launch):
//   STORE      Y -> fp32 C (rows past a sequence's token count stored as 0): LM head
//   QKV_ROPE   columns paired (i, i + hd/2) inside a head; RoPE at the row's absolute
//              position (angle pos * theta^(-2i/hd), fp64), q -> bf16 buffer, k and v ->
//              the KV cache at the row's position
//   SWIGLU     columns paired (gate n, up n): a = bf16(silu(g) * u)
//   GELU       a = bf16(gelu(y)), erf form
//   RESID      x += Y on the residual stream (each column belongs to one tile, so the
//              update is race-free), h = bf16(x * g) for the next normalised product and
//              the tile's partial sums of x^2 per row (16 columns each, summed in fp64,
//              stored as fp32); before the final norm x * g is written in fp32 instead
//              (xg_out), for the exact normalise pass of the LM head's input
// A normalised product inside the layers (QKV_ROPE, SWIGLU, GELU) takes A = bf16(x * g)
// and scales output row r by s_r = 1 / sqrt(mean(x_r^2) + eps), summed from those
// partials in a fixed order: RMSNorm(x) * g = s * (x * g), with the row factor taken out
// of the product, so no separate normalisation pass runs between GEMMs (the one bf16
// rounding of the input falls before the row factor instead of after it).  The LM head
// takes bf16(RMSNorm(x) * g) from launch_norm_pack, the rounding after the row factor.
//
// Kernels by row count: k_gemm_bf16 (one row tile; and several row tiles with one tile
// group per workgroup), k_gemm_bf16_ko (2-4 row tiles, several tiles per workgroup: A loaded
// once per step for a chunk of tiles), k_gemm_sk (residual products at 2-4 row tiles that
// would own one tile per workgroup, and at 5-8 row tiles: four tiles per workgroup, split by
// wave slot).  All
// three accumulate every output element over the same steps in the same order, so a verify
// call equals single-token calls bit for bit.
//
// fp32 path (small fp32 models): separate simple kernels, one wave per output column.
#include <hip/hip_ext.h>

#include <algorithm>
#include <math.h>

#include "act_layout.h"
#include "common.h"
#include "gemm.h"
#include "kv_layout.h"

namespace specdec {

#ifndef SPEC_GEMM_WAVES
#define SPEC_GEMM_WAVES 4  // streaming waves per workgroup (plus one epilogue wave)
#endif
#ifndef SPEC_GEMM_RING
#define SPEC_GEMM_RING 1  // steps requested ahead of the one being multiplied
#endif
#ifndef SPEC_GEMM_WPC
#define SPEC_GEMM_WPC 1  // workgroups per compute unit the grid is sized for
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

// Exact quotient a / b for 0 <= a < 2^22, 1 <= b < 2^12 from a float reciprocal plus one
// correction step each way (a few instructions instead of the ~25 of an integer
// division), for index math on the epilogue wave's path to its first memory requests.
__device__ __forceinline__ int qdiv(int a, int b) {
  int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
  q -= (q * b > a) ? 1 : 0;
  q += ((q + 1) * b <= a) ? 1 : 0;
  return q;
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
  q.sec = qdiv(t, per_sec);
  const int rem = t - q.sec * per_sec;
  q.h = qdiv(rem, per_head);
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

// LDS the epilogue wave stages its inputs in.  With one row tile (MT = 1) every input
// of the epilogue comes from LDS, copied there by direct global-to-LDS loads that the
// epilogue wave issues first thing, so they are in flight early and need no registers
// (once the weight stream saturates HBM a load waits several microseconds, and an
// epilogue waiting for one would hold the streaming waves at the next tile barrier):
// the row factors' partial sums, the RoPE factors of the block's rows and, for RESID,
// the residual values and norm gains of the current tile.  With more row tiles only the
// partial sums are staged (16 rows at a time) and the other inputs are read from global
// memory.
constexpr int SS_NP_MAX = 512;     // partial sums per row (d_model <= 8192)
constexpr int ROPE_HALF_MAX = 64;  // rotation pairs per head (head_dim <= 128)

// Dynamic LDS of the epilogue wave, sized per launch (epi_lds_bytes): the partial sums
// of squares of the block's rows (all of them, or 16 at a time when they do not fit),
// and the inputs of the tile group being finished: RoPE factors (QKV_ROPE; with one row
// tile those of every row, else the group's 8 pairs per tile) or residual values and
// gains (RESID).  Everything is requested ahead of use by direct global-to-LDS loads.
struct EpiLds {
  float* ss;       // [ss rows][np]
  double2* rope;   // MT == 1: [rows][hd/2]; MT > 1: [NT][MT*16][8]
  float* xres;     // [NT][MT*16][16]
  float* gain;     // [NT][16]
};

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

__host__ __device__ inline int epi_lds_bytes(int mt, int nt, int mode, int ss_rows, int np,
                                             int half, int rows, bool norm_in) {
  int b = norm_in ? align16(ss_rows * np * 4) : 0;
  if (mode == EPI_QKV_ROPE) b += mt == 1 ? align16(rows * half * 16) : nt * mt * 16 * 8 * 16;
  if (mode == EPI_RESID) b += nt * (mt * 16 * 16 * 4 + 16 * 4);
  return b;
}

// Copy `bytes` (a multiple of 16) from global `src` to LDS `dst` with direct loads: lane l
// of pass k moves bytes [1024 k + 16 l, +16).
__device__ __forceinline__ void lds_copy(const void* src, void* dst, int bytes, int lane) {
  for (int off = 0; off < bytes; off += 1024) {
    if (off + 16 * lane < bytes)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)((const char*)src + off + 16 * lane),
          (__attribute__((address_space(3))) void*)((char*)dst + off), 16, 0, 0);
  }
}

// Residual values x[r0 + row][16 t .. 16 t + 15] (row < rows) and gains of tile t:
// 16 rows per pass, four lanes per row.
__device__ __forceinline__ void lds_copy_resid(const GemmArgs& g, int t, int r0, int rows,
                                               float* xres, float* gain, int lane) {
  const int q = lane & 3;
  for (int rb = 0; rb < rows; rb += 16) {
    const int row = rb + (lane >> 2);
    if (row < rows)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(g.x + (size_t)(r0 + row) * g.N +
                                                          16 * t + 4 * q),
          (__attribute__((address_space(3))) void*)(xres + rb * 16), 16, 0, 0);
  }
  if (lane < 4)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(g.gain + 16 * t + 4 * lane),
        (__attribute__((address_space(3))) void*)gain, 16, 0, 0);
}

// RoPE factors of the 8 rotation pairs of QKV tile t (q and k sections) for rows
// r0 .. r0 + rows - 1: [rows][8] (cos, sin), 8 rows per pass, 8 lanes per row.
__device__ __forceinline__ void lds_copy_rope_tile(const GemmArgs& g, int t, int r0, int rows,
                                                   double2* rope, int lane) {
  const QkvTile qt = qkv_tile(t, g.d, g.hd);
  if (qt.sec >= 2) return;
  const int half = g.hd >> 1, j = lane & 7;
  for (int rb = 0; rb < rows; rb += 8) {
    const int row = rb + (lane >> 3);
    if (row < rows)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(g.rope_rows +
                                                          ((size_t)(r0 + row) * half + qt.i0 + j) * 2),
          (__attribute__((address_space(3))) void*)(rope + rb * 8), 16, 0, 0);
  }
}

// 16 bytes per lane from a buffer (byte offset voff + soff; zeros past its end) straight
// to LDS at lds + 16 * lane.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                                uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

// Cross-lane moves inside a row of 16 lanes by DPP (a vector ALU operation of a few
// cycles) instead of the LDS crossbar of __shfl (ds_bpermute, an LDS round trip).
// CTRL: 0xB1 lane ^ 1 and 0x4E lane ^ 2 (quad permutes), 0x141 mirror within each half row
// of 8, 0x140 mirror within the row, 0x128 rotate the row by 8 (lane ^ 8).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const unsigned hi =
      (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Sum over the 16 lanes of a row, bitwise the xor butterfly (^1, ^2, ^4, ^8): after the two
// quad steps every lane of a quad holds the same sum, so pairing each lane with any lane of
// the other quad of its half row (the half-row mirror), then with any lane of the other
// half (the row mirror), adds the same two values as ^4 and ^8 do.
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return v;
}

// Wait for this wave's outstanding global loads, direct-to-LDS ones included.
__device__ __forceinline__ void wait_vm() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row factors s_r = 1 / sqrt(sum_p ss[r][p] / K + eps) of `rows` (<= 16) rows whose np
// partial sums sit in LDS: four lanes per row add contiguous quarters in column order
// (fp64, four at a time as ((a + b) + (c + d))) and combine them by a fixed butterfly,
// the same order for every row count and on every path that normalises a row.
__device__ __forceinline__ void row_factors(const float* ss, int rows, int np, int K, float eps,
                                            int lane, double* rowscale) {
  const int row = lane >> 2, qq = lane & 3, per = np >> 2;  // np is a multiple of 8
  double part = 0.0;
  if (row < rows) {
    const float* src = ss + row * np + qq * per;
    for (int c = 0; c + 4 <= per; c += 4)
      part += ((double)src[c] + (double)src[c + 1]) + ((double)src[c + 2] + (double)src[c + 3]);
    for (int c = per & ~3; c < per; ++c) part += (double)src[c];
  }
  part += dpp_f64<0xB1>(part);  // lane ^ 1
  part += dpp_f64<0x4E>(part);  // lane ^ 2
  if (qq == 0 && row < rows) rowscale[row] = 1.0 / sqrt(part / K + (double)eps);
}

template <int MT, int NP = GW>
__device__ __forceinline__ floatx4 sum_partials(const floatx4 (*part)[MT][64], int mt, int lane) {
  floatx4 v = part[0][mt][lane];
#pragma unroll
  for (int w = 1; w < NP; ++w) {
    const floatx4 p = part[w][mt][lane];
    v[0] += p[0]; v[1] += p[1]; v[2] += p[2]; v[3] += p[3];
  }
  return v;
}

// Per-tile epilogue, run by the workgroup's epilogue wave.  part[w][mt][lane] holds
// wave w's MFMA accumulator fragment of row tile mt: lane l has rows 4(l/16)+e
// (e = 0..3) of local column l%16.  The NP partials are summed in wave order (NP = 1: a
// fragment the caller has already summed in that order).
// rowinfo[rr] = (absolute position, flags) of row r0 + rr: flag 1 = a real token of its
// sequence, flag 2 = its K/V may be written (real token and position < max_len).
// One loop per mode, so each mode's registers are allocated on its own.
template <int MT, int NP = GW>
__device__ __forceinline__ void gemm_tile_epilogue(const GemmArgs& g, int t, int r0,
                                                   const floatx4 (*part)[MT][64],
                                                   const int2* rowinfo, const double* rowscale,
                                                   const EpiLds& L, int lane, int mt0 = 0,
                                                   int mt1 = MT) {
  const int nl = lane & 15, gq = lane >> 4, R = g.R, mode = g.mode;
  const bool is_hi = nl >= 8;
  if (mode == EPI_RESID) {
    // residual update, next input bf16(x * g) (or x * g in fp32) and the tile's sums of
    // squares per row
    const int col = 16 * t + nl, np = g.N >> 4;
    const float gc = L.gain[nl];
#pragma unroll 1
    for (int mt = mt0; mt < mt1; ++mt) {
      const floatx4 v = sum_partials<MT, NP>(part, mt, lane);
      double sq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = mt * 16 + 4 * gq + e, r = r0 + rr;
        float xn = 0.f;
        if (r < R) {
          const float xo = L.xres[rr * 16 + nl];
          xn = xo + v[e];
          g.x[(size_t)r * g.N + col] = xn;
          if (g.h_out)
            g.h_out[act_index(r, col, g.N)] = f32_to_bf16(xn * gc);
          else
            g.xg_out[act32_index(r, col, g.N)] = xn * gc;
        }
        sq[e] = (double)xn * xn;
      }
      // sum over the 16 columns of the tile (the 16 lanes of this row group), fixed order
#pragma unroll
      for (int e = 0; e < 4; ++e) sq[e] = row16_sum(sq[e]);
      if (nl == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = r0 + mt * 16 + 4 * gq + e;
          if (r < R) g.ss_out[(size_t)r * np + t] = (float)sq[e];
        }
      }
    }
    return;
  }
  // normalised products: the row factor first
#pragma unroll 1
  for (int mt = mt0; mt < mt1; ++mt) {
    floatx4 v = sum_partials<MT, NP>(part, mt, lane);
    if (g.ss_in) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (float)((double)v[e] * rowscale[mt * 16 + 4 * gq + e]);
    }
    if (mode == EPI_QKV_ROPE) {
      const QkvTile qt = qkv_tile(t, g.d, g.hd);
      const int half = g.hd >> 1, i = qt.i0 + (nl & 7), ii = is_hi ? i + half : i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = mt * 16 + 4 * gq + e, r = r0 + rr;
        const float y = v[e];
        const float yp = dpp_f32<0x128>(y);  // the paired column c ^ 8 of the same row
        if (r >= R) continue;
        u16 o;
        if (qt.sec < 2) {
          // rotation of the pair (i, i + hd/2) at the row's position, in fp64
          const double2 c2 = MT == 1 ? L.rope[rr * half + i] : L.rope[rr * 8 + (nl & 7)];
          const float lo = is_hi ? yp : y, hi = is_hi ? y : yp;
          o = is_hi ? f32_to_bf16((float)((double)hi * c2.x + (double)lo * c2.y))
                    : f32_to_bf16((float)((double)lo * c2.x - (double)hi * c2.y));
        } else {
          o = f32_to_bf16(y);
        }
        if (qt.sec == 0) {
          g.q_out[(size_t)r * g.d + qt.h * g.hd + ii] = o;
        } else {
          const int2 info = rowinfo[rr];
          if (info.y & 2) {
            const int b = r / g.M;
            ((qt.sec == 1) ? g.kc : g.vc)[(size_t)b * g.row_stride + (size_t)qt.h * g.head_stride +
                                          (qt.sec == 1 ? kv_k_offset(info.x, ii, g.hd)
                                                       : kv_v_offset(info.x, ii, g.hd))] = o;
          }
        }
      }
    } else if (mode == EPI_SWIGLU) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + mt * 16 + 4 * gq + e;
        const float y = v[e];
        const float yp = dpp_f32<0x128>(y);  // the up column paired with gate column nl
        if (r < R && !is_hi)
          g.act_out[act_index(r, 8 * t + nl, g.N1)] = f32_to_bf16(y / (1.f + expf(-y)) * yp);
      }
    } else if (mode == EPI_GELU) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + mt * 16 + 4 * gq + e;
        if (r < R)
          g.act_out[act_index(r, 16 * t + nl, g.N)] =
              f32_to_bf16(0.5f * v[e] * (1.f + erff(v[e] * 0.70710678118654752f)));
      }
    } else {  // EPI_STORE
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = mt * 16 + 4 * gq + e, r = r0 + rr;
        if (r < R) g.C[(size_t)r * g.ldc + 16 * t + nl] = (rowinfo[rr].y & 1) ? v[e] : 0.f;
      }
    }
  }
}

// The epilogue wave's side of the per-tile barrier.  It shares only LDS with the
// streaming waves, so it waits for its own LDS accesses and nothing else: its global
// stores and the loads it has issued for the next tile stay in flight across the
// barrier (__syncthreads would also wait for those).
__device__ __forceinline__ void epi_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Persistent weight-streaming GEMM.  Workgroup (bx, by) owns row block by (MT*16 rows
// of A) and the column-tile groups bx, bx + G, bx + 2G, ... (G = gridDim.x; a group is
// NT consecutive 16-column tiles, see below).  It has GW
// streaming waves and one epilogue wave.  The streaming waves split K: wave wv takes
// 128-wide super-steps wv, wv + GW, ... of every tile, so its steps form one flat
// stream over (tile, step) and its register ring of P steps runs across tile
// boundaries.  At the end of a tile each streaming wave parks its accumulator in LDS
// (double-buffered by tile parity) and meets the others at one barrier; the epilogue
// wave then sums the partials and runs the epilogue while the streaming waves go on with
// the next tile.
// Residency: the grid is sized for one workgroup per compute unit (a CU holding two
// streams both shares through one memory pipeline and finishes last).  Were it sized
// for two, two workgroups of GW + 1 waves put two waves of each on one SIMD, and the
// kernel would have to fit four waves per SIMD (<= 128 VGPRs) to be resident at once.
// NT: column tiles multiplied per step.  With 32 or more rows every A fragment is used
// for NT tiles at once, which divides the A reads per weight byte (with three or four
// row tiles the A reads through L1, not HBM, bound the kernel).  Every output element
// still accumulates its K steps in the same order as with NT = 1.
template <int MT, int NT>
__global__ __launch_bounds__(GT) void k_gemm_bf16(GemmArgs g) {
  constexpr int P = SPEC_GEMM_RING;
  static_assert(MT > 1 || NT == 1, "one row tile uses single column tiles");
  __shared__ floatx4 part[2][NT][GW][MT][64];
  __shared__ int2 rowinfo[MT * 16];
  __shared__ double rowscale[MT * 16];
  extern __shared__ float4 epi_dyn[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bx = blockIdx.x, G = gridDim.x;
  const int r0 = blockIdx.y * (MT * 16);
  const int ngroups = g.ntiles / NT;
  const int nt = (ngroups - bx + G - 1) / G;  // tile groups of this workgroup (>= 1)
  if (wv == GW) {
    const int rows = min(MT * 16, g.R - r0);  // >= 1
    const int np = g.ss_np, half = g.hd >> 1;
    EpiLds L;
    const int ss_rows = min(g.ss_rows, g.R);  // partial-sum rows the LDS holds at once
    {
      char* p = reinterpret_cast<char*>(epi_dyn);
      L.ss = reinterpret_cast<float*>(p);
      if (g.ss_in) p += align16(ss_rows * np * 4);
      L.rope = reinterpret_cast<double2*>(p);
      if (g.mode == EPI_QKV_ROPE) p += MT == 1 ? align16(g.R * half * 16) : NT * MT * 16 * 8 * 16;
      L.xres = reinterpret_cast<float*>(p);
      L.gain = L.xres + NT * MT * 16 * 16;
    }
    // the inputs of tile group `grp` into the per-tile slots (RESID; QKV_ROPE with
    // several row tiles -- one row tile keeps every row's factors from the start)
    auto stage_group = [&](int grp) {
#pragma unroll 1
      for (int n = 0; n < NT; ++n) {
        const int t = grp * NT + n;
        if (g.mode == EPI_RESID)
          lds_copy_resid(g, t, r0, rows, L.xres + n * MT * 16 * 16, L.gain + n * 16, lane);
        else if (MT > 1 && g.mode == EPI_QKV_ROPE)
          lds_copy_rope_tile(g, t, r0, rows, L.rope + n * MT * 16 * 8, lane);
      }
    };
    // requests first: the rows' token counts and start positions, direct-to-LDS copies of
    // the row factors' partial sums and the first group's inputs
    int ntok[(MT * 16 + 63) / 64], p0v[(MT * 16 + 63) / 64];
#pragma unroll
    for (int k = 0; k < (MT * 16 + 63) / 64; ++k) {
      const int r = min(r0 + lane + 64 * k, g.R - 1), b = qdiv(r, g.M);
      ntok[k] = g.ntok_eff ? g.ntok_eff[b] : g.M;
      p0v[k] = g.pos0 ? g.pos0[b] : 0;
    }
    const bool ss_all = ss_rows >= rows;
    if (g.ss_in)
      lds_copy(g.ss_in + (size_t)r0 * np, L.ss, (ss_all ? rows : min(16, rows)) * np * 4, lane);
    if (MT == 1 && g.mode == EPI_QKV_ROPE)
      lds_copy(g.rope_rows + (size_t)r0 * half * 2, L.rope, rows * half * 16, lane);
    stage_group(bx);
    if constexpr (MT > 1) {
      // Several row tiles: the streaming waves' A requests are then many, and a request
      // queued behind them returns after 5-20 us; the streaming waves start once these
      // are on their way (the matching barrier opens their code).
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k = 0; k < (MT * 16 + 63) / 64; ++k) {
      const int rr = lane + 64 * k, r = r0 + rr;
      int2 info{0, 0};
      if (r < g.R) {
        const int j = r - qdiv(r, g.M) * g.M, pos = p0v[k] + j;
        info = int2{pos, (j < ntok[k] ? 1 : 0) | (j < ntok[k] && pos < g.max_len ? 2 : 0)};
      }
      if (rr < MT * 16) rowinfo[rr] = info;
    }
    wait_vm();
    if (g.ss_in) {
      for (int rb = 0; rb < MT && 16 * rb < rows; ++rb) {
        const float* src = L.ss + (ss_all ? rb * 16 * np : 0);
        if (!ss_all && rb > 0) {  // 16 rows at a time: the next batch (requested late)
          wave_lds_sync();
          lds_copy(g.ss_in + (size_t)(r0 + 16 * rb) * np, L.ss, min(16, rows - 16 * rb) * np * 4,
                   lane);
          wait_vm();
        }
        row_factors(src, min(16, rows - 16 * rb), np, g.K, g.eps, lane, rowscale + 16 * rb);
      }
    }
    wave_lds_sync();
    for (int ct = 0; ct < nt; ++ct) {
      epi_barrier();
#pragma unroll 1
      for (int n = 0; n < NT; ++n) {
        EpiLds Ln = L;
        if (MT > 1) Ln.rope = L.rope + n * MT * 16 * 8;
        Ln.xres = L.xres + n * MT * 16 * 16;
        Ln.gain = L.gain + n * 16;
        gemm_tile_epilogue<MT>(g, (bx + ct * G) * NT + n, r0, part[ct & 1][n], rowinfo, rowscale,
                               Ln, lane);
      }
      if (ct + 1 < nt && (g.mode == EPI_RESID || (MT > 1 && g.mode == EPI_QKV_ROPE))) {
        wave_lds_sync();  // this group's slots are read
        stage_group(bx + (ct + 1) * G);
        wait_vm();
      }
    }
    return;
  }
  if constexpr (MT > 1) {
    __builtin_amdgcn_s_barrier();  // the epilogue wave's requests go first
    __builtin_amdgcn_sched_barrier(0);
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
    // packed activations (act_layout.h): this lane's 16 bytes of step js, slice s sit at
    // arow[mt] + js * 2048 + s * 512
    arow[mt] = g.A + (size_t)(blockIdx.y * MT + mt) * (size_t)nsuper * 2048 + 8 * (4 * nl + gq);
  }
  floatx4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  constexpr int Q = P + 1;  // register buffers: P steps in flight while one is multiplied
  bf16x8 wf[Q][NT][4];
  bf16x8 af[Q][MT][4];
  const u16* zblk = g.zeros;
  // issue stream: tile iteration it, step is; a step past the wave's last one in a tile,
  // or past the workgroup's last tile, re-reads an in-bounds W segment (cache hit) and
  // pairs it with zero A fragments, so every wave runs the same branch-free schedule.
  int it = 0, is = 0;
  const u16* wp = g.W + (size_t)bx * NT * tile_elems + 8 * lane;
  auto issue = [&](int slot) {
    const bool valid = is <= last_step && wact && it < nt;
    const int js = wact ? wv + (is <= last_step ? is : last_step) * GW : 0;  // super-step
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        wf[slot][n][s] = ld8_nt(wp + n * tile_elems + js * 2048 + 512 * s, true);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        af[slot][mt][s] = ld8((valid && aok[mt]) ? arow[mt] + (size_t)js * 2048 + 512 * s : zblk,
                              true);
    if (++is == S) {
      is = 0;
      ++it;
      if (it < nt) wp += (size_t)G * NT * tile_elems;
    }
  };
  int ct = 0, cs = 0;  // consume stream: tile iteration, step
  auto consume = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[mt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[slot][mt][s], wf[slot][n][s],
                                                               acc[mt][n], 0, 0, 0);
    if (++cs == S) {
      cs = 0;
      if (ct < nt) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) part[ct & 1][n][wv][mt][lane] = acc[mt][n];
        __syncthreads();
      }
      ++ct;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[mt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Rounds of Q steps.  Each step first requests the step P ahead (into the buffer
  // multiplied last) and then multiplies its own buffer, so the requests never wait
  // behind the MFMA chain.  The last round's requests read in-bounds W past the end
  // (cache hits, never multiplied), so the loop body is the only copy of the tile code.
  const int F = nt * S;  // steps of this wave
  const int T = (F + Q - 1) / Q;
#pragma unroll
  for (int u = 0; u < P; ++u) issue(u);
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int u = 0; u < Q; ++u) {
      issue((u + P) % Q);
      __builtin_amdgcn_sched_barrier(0);
      consume(u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// K-outer variant for several row tiles (R > 16) and several tiles per workgroup.
// Workgroup bx owns the tiles bx + G j (j < per, G = gridDim.x) and takes them in chunks
// of TPW.  Each streaming wave walks its K super-steps once per chunk; per step it loads
// the A fragments of all row tiles once and multiplies them into every tile of the chunk
// (accumulators in registers), so A is requested once per step instead of once per tile
// and step -- at 48 rows the loads per tile and step fall from 10-16 to 4 + 12/TPW, and
// load instructions, not bytes, bound the tile-at-a-time kernel there.  The partials meet
// in LDS at the end of a chunk and all five waves share the chunk's epilogues.  Every
// output element accumulates its K steps in the same order as in k_gemm_bf16 (the same
// per-wave step sequence, waves summed in order), so results are bitwise the same.
// Tiles past the end are computed on the last tile (in bounds) and dropped.
// (register budget, 256 VGPRs: TPW accumulators, one step of A fragments -- the next
// step's wait in LDS -- and two steps of W)
template <int MT> constexpr int ko_tpw_max() { return MT == 4 ? 5 : 8; }

// WAUX: the cache policy of the weight loads (an immediate of each load).  Non-temporal (2)
// by default.  A launch with several 64-row blocks takes ordinary loads (0): its row blocks
// of one column group run side by side on one XCD (the launcher makes the grid's x extent
// a multiple of 8 where the grid allows) and stream the same tiles in the same order, so
// the later request finds the line in L2.  With non-temporal loads a 96-row verify's qkv, gate/up and LM head fetched 1.7-2.1x
// their weight bytes from HBM.
template <int MT, int TPW, int WAUX = 2>
__global__ __launch_bounds__(GT) void k_gemm_bf16_ko(GemmArgs g, int per) {
  static_assert(MT >= 2 && MT <= 4 && TPW >= 2 && TPW <= ko_tpw_max<MT>(), "K-outer shape");
  // the chunk's partials; while the chunk streams, the same LDS holds each streaming
  // wave's A staging slot ([GW][MT][4][64] 16-byte fragments, at most TPW >= 4 times
  // smaller than the partials, hence the max)
  constexpr int PT = TPW > 4 ? TPW : 4;
  __shared__ floatx4 part[PT][GW][MT][64];
  __shared__ int2 rowinfo[MT * 16];
  __shared__ double rowscale[MT * 16];
  extern __shared__ float4 epi_dyn[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bx = blockIdx.x, G = gridDim.x;
  const int r0 = blockIdx.y * (MT * 16);
  const int rows = min(MT * 16, g.R - r0);  // >= 1
  const int np = g.ss_np;
  EpiLds L;
  {
    char* p = reinterpret_cast<char*>(epi_dyn);
    L.ss = reinterpret_cast<float*>(p);
    if (g.ss_in) p += align16(16 * np * 4);
    L.rope = reinterpret_cast<double2*>(p);
    if (g.mode == EPI_QKV_ROPE) p += TPW * MT * 16 * 8 * 16;
    L.xres = reinterpret_cast<float*>(p);
    L.gain = L.xres + TPW * MT * 16 * 16;
  }
  const int nchunks = (per + TPW - 1) / TPW;
  auto tile_of = [&](int c, int j) { return min(bx + G * (c * TPW + j), g.ntiles - 1); };
  auto stage_chunk = [&](int c) {
#pragma unroll 1
    for (int j = 0; j < TPW; ++j) {
      const int t = tile_of(c, j);
      if (g.mode == EPI_RESID)
        lds_copy_resid(g, t, r0, rows, L.xres + j * MT * 16 * 16, L.gain + j * 16, lane);
      else if (g.mode == EPI_QKV_ROPE)
        lds_copy_rope_tile(g, t, r0, rows, L.rope + j * MT * 16 * 8, lane);
    }
  };
  // streaming state
  const int nl = lane & 15, gq = lane >> 4;
  const int nsuper = g.K >> 7;
  const int S = (nsuper + GW - 1) / GW;  // steps per wave
  const size_t tile_elems = (size_t)nsuper * 2048;

#pragma unroll 1
  for (int c = 0; c < nchunks; ++c) {
    if (wv == GW) {
      if (c == 0) {
        // counts and start positions, the first 16 rows' sums of squares and the chunk's
        // epilogue inputs.  Up to three row tiles they are requested beside the streaming
        // waves' first steps (needed only at the chunk's end; holding the streams back
        // behind them cost about 1 us per 48-row launch).  At four row tiles the streams
        // wait for them: the four batches of row sums must be back before the stream ends.
        int ntok[(MT * 16 + 63) / 64], p0v[(MT * 16 + 63) / 64];
#pragma unroll
        for (int k = 0; k < (MT * 16 + 63) / 64; ++k) {
          const int r = min(r0 + lane + 64 * k, g.R - 1), b = qdiv(r, g.M);
          ntok[k] = g.ntok_eff ? g.ntok_eff[b] : g.M;
          p0v[k] = g.pos0 ? g.pos0[b] : 0;
        }
        if (g.ss_in) lds_copy(g.ss_in + (size_t)r0 * np, L.ss, min(16, rows) * np * 4, lane);
        stage_chunk(0);
        if constexpr (MT == 4) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < (MT * 16 + 63) / 64; ++k) {
          const int rr = lane + 64 * k, r = r0 + rr;
          int2 info{0, 0};
          if (r < g.R) {
            const int j = r - qdiv(r, g.M) * g.M, pos = p0v[k] + j;
            info = int2{pos, (j < ntok[k] ? 1 : 0) | (j < ntok[k] && pos < g.max_len ? 2 : 0)};
          }
          if (rr < MT * 16) rowinfo[rr] = info;
        }
        wait_vm();
        if (g.ss_in) {
          // later 16-row batches are requested behind the weight stream; the results are
          // needed only at the end of the chunk
          for (int rb = 0; rb < MT && 16 * rb < rows; ++rb) {
            if (rb > 0) {
              wave_lds_sync();
              lds_copy(g.ss_in + (size_t)(r0 + 16 * rb) * np, L.ss,
                       min(16, rows - 16 * rb) * np * 4, lane);
              wait_vm();
            }
            row_factors(L.ss, min(16, rows - 16 * rb), np, g.K, g.eps, lane, rowscale + 16 * rb);
          }
        }
      } else {
        stage_chunk(c);
        wait_vm();
      }
    } else {
      if constexpr (MT == 4) {
        if (c == 0) {
          __builtin_amdgcn_s_barrier();  // the epilogue wave's requests go first
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      floatx4 acc[TPW][MT];
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[j][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      bf16x8 af[MT][4];
      bf16x8 wf[2][4];
      // Buffer loads: a 32-bit lane offset and a scalar step / tile offset per request,
      // and requests past the buffer's end read zeros, so rows past R and steps past the
      // wave's last one need no selects (steps past the last re-read an in-bounds weight
      // segment and pair it with zero A fragments).  The next step's A fragments go
      // straight to this wave's LDS slot and are read into registers at the step's start.
      const int wvu = __builtin_amdgcn_readfirstlane(wv);
      const bool wactu = wvu < nsuper;
      const int lastu = wactu ? (nsuper - 1 - wvu) / GW : 0;
      // packed activations (act_layout.h): row tile mt_abs, step js, slice s of this lane
      // at byte mt_abs * nsuper * 4096 + js * 4096 + s * 1024 + 16 * (4 * nl + gq); the
      // direct-to-LDS load still lands lane l's 16 bytes at 16 * l of the slot
      const uint32_t a_bytes = (uint32_t)act_rows(g.R) * (uint32_t)g.K * 2u;
      const __amdgpu_buffer_rsrc_t ra = coherent_rsrc(g.A, a_bytes);
      const __amdgpu_buffer_rsrc_t rw = coherent_rsrc(g.W, (size_t)g.ntiles * tile_elems * 2);
      uint32_t aoff[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = r0 + mt * 16 + nl;
        aoff[mt] = r < g.R ? ((uint32_t)(r0 / 16 + mt) * (uint32_t)nsuper * 4096u +
                              16u * (uint32_t)(4 * nl + gq))
                           : a_bytes;
      }
      const uint32_t woff = 16u * lane;
      uint32_t wtile[TPW];  // byte offset of each tile of the chunk (uniform)
#pragma unroll
      for (int j = 0; j < TPW; ++j) wtile[j] = (uint32_t)tile_of(c, j) * (uint32_t)tile_elems * 2u;
      char* aslot = reinterpret_cast<char*>(&part[0][0][0][0]) + (size_t)wvu * MT * 4 * 1024;
      auto dmaA = [&](int i) {
        const uint32_t so = (wactu && i <= lastu) ? (uint32_t)(wvu + i * GW) * 4096u : a_bytes;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            buffer_to_lds16(ra, aslot + (mt * 4 + s) * 1024, aoff[mt] + 1024u * s, so);
      };
      auto readA = [&]() {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            af[mt][s] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4*>(aslot + (mt * 4 + s) * 1024 + 16 * lane));
      };
      auto loadW = [&](int buf, int i, int j) {
        const uint32_t js = wactu ? (uint32_t)(wvu + (i <= lastu ? i : lastu) * GW) : 0u;
        const uint32_t so = wtile[j] + js * 4096u;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          wf[buf][s] = __builtin_bit_cast(
              bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rw, woff + 1024u * s, so, WAUX));
      };
      dmaA(0);
      loadW(0, 0, 0);
      // two steps per round so both W register buffers are addressed statically
      for (int i0 = 0; i0 < S; i0 += 2) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = i0 + ii;
          // step i's A is in the slot once only the last W request (4 loads, issued after
          // it) may still be outstanding; reading it frees the slot for step i + 1
          __builtin_amdgcn_sched_barrier(0);
          __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory");
          readA();
          __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          dmaA(i + 1);
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            const int f = ii * TPW + j;
            if (j + 1 < TPW) loadW((f + 1) & 1, i, j + 1);
            else loadW((f + 1) & 1, i + 1, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int s = 0; s < 4; ++s)
                acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt][s], wf[f & 1][s],
                                                                     acc[j][mt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // the partials overwrite the A slots: every wave's requests have landed and every
      // wave is past its last read of its slot
      wait_vm();
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) part[j][wv][mt][lane] = acc[j][mt];
    }
    if (wv == GW) __builtin_amdgcn_s_barrier();  // the streaming waves' slot barrier
    __syncthreads();  // partials, row factors and the chunk's staged inputs are complete
    // the chunk's (tile, row tile) epilogues, spread over all five waves
#pragma unroll 1
    for (int it = wv; it < TPW * MT; it += GW + 1) {
      const int j = it / MT, mt = it - j * MT;
      const int t = bx + G * (c * TPW + j);
      if (t >= g.ntiles) break;
      EpiLds Lj = L;
      Lj.rope = L.rope + j * MT * 16 * 8;
      Lj.xres = L.xres + j * MT * 16 * 16;
      Lj.gain = L.gain + j * 16;
      gemm_tile_epilogue<MT>(g, t, r0, part[j], rowinfo, rowscale, Lj, lane, mt, mt + 1);
    }
    __syncthreads();  // the chunk's partials and input slots may be reused
  }
}

__host__ __device__ inline int ko_lds_bytes(int mt, int tpw, int mode, int np, bool norm_in) {
  int b = norm_in ? align16(16 * np * 4) : 0;
  if (mode == EPI_QKV_ROPE) b += tpw * mt * 16 * 8 * 16;
  if (mode == EPI_RESID) b += tpw * (mt * 16 * 16 * 4 + 16 * 4);
  return b;
}

// ------------------------------------------------------ split by wave slot (RESID) --
//
// The residual GEMMs (O-projection, down) of a 2-4-row-tile launch on a grid where every
// workgroup would own a single 16-column tile: the tile-at-a-time kernel then reads the
// whole A operand (all rows, all K) once per tile, 3 KB of A per KB of weights at 48 rows,
// and that A traffic from L2 -- not the weight stream -- set its time (with A read from a
// cached zero block instead, wo + down took 0.95 instead of 1.52 ms per 48-row pass).  At
// 5-8 row tiles (up to 128 rows) it takes every row in one pass where the other kernels
// stream the weights once per 64 rows (96-row verify GEMMs 6.94 -> 6.35 ms).
//
// Here a workgroup owns four tiles (one per streaming wave) and ONE of the four wave
// slots of k_gemm_bf16: slot q accumulates super-steps q, q + 4, ... of each tile in
// increasing order, exactly the sequence wave q of k_gemm_bf16 accumulates.  A step's A
// fragments (all row tiles) are loaded once into LDS, by direct loads split over the
// waves, and shared by the four tiles -- a quarter of the A traffic per weight byte.  The
// four slot workgroups of a tile group store their fp32 partials (device-coherent); the
// last to finish (completion counter, reset by it) sums the slots in order 0..3 and runs
// the residual epilogue, so every output is bitwise that of k_gemm_bf16.
constexpr int SK_SLOTS = GW;  // wave slots of the reference summation order
constexpr int SK_MT_MAX = 8;  // row tiles of the split-by-slot kernel (128 rows)

#ifndef SPEC_SK_DEPTH
#define SPEC_SK_DEPTH 2  // steps requested ahead of the one being multiplied
#endif
template <int MT>
__global__ __launch_bounds__(GT) void k_gemm_sk(GemmArgs g) {
  static_assert(MT >= 2 && MT <= SK_MT_MAX, "2-8 row tiles");
  constexpr int P = SPEC_SK_DEPTH;  // steps in flight ahead of the multiplied one
  constexpr int NB = P + 1;         // A buffers (LDS) and W buffers (registers)
  __shared__ uint4 abuf[NB][MT][4][64];               // A fragments of NB steps
  // merger, up to 4 row tiles: [tile of wave][slot][mt][lane]; from 5 on the four slots
  // are summed in registers and the sums reuse the A ring (the stream has ended)
  __shared__ floatx4 part[MT <= 4 ? GW : 1][MT <= 4 ? SK_SLOTS : 1][MT <= 4 ? MT : 1][64];
  __shared__ int2 rowinfo[MT * 16];
  __shared__ double rowscale[MT * 16];
  __shared__ int is_last;
  extern __shared__ float4 epi_dyn[];                 // [4 tiles] residual slices + gains
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int grp = blockIdx.x / SK_SLOTS, q = blockIdx.x % SK_SLOTS;
  const int nsuper = g.K >> 7;
  const int S = q < nsuper ? (nsuper - 1 - q) / SK_SLOTS + 1 : 0;  // this slot's steps
  const int rows = min(MT * 16, g.R);
  float* xres = reinterpret_cast<float*>(epi_dyn);
  float* gain = xres + GW * MT * 16 * 16;
  floatx4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (wv == GW) {
    // the residual slices and gains of the group's tiles, in case this workgroup merges
    for (int w = 0; w < GW; ++w)
      lds_copy_resid(g, grp * GW + w, 0, rows, xres + w * MT * 16 * 16, gain + w * 16, lane);
    for (int i = 0; i < S; ++i) __builtin_amdgcn_s_barrier();  // the streaming waves' steps
    wait_vm();
  } else if (S > 0) {
    const int t = grp * GW + wv;
    const size_t tile_bytes = (size_t)nsuper * 4096;
    const uint32_t a_bytes = (uint32_t)act_rows(g.R) * (uint32_t)g.K * 2u;
    const __amdgpu_buffer_rsrc_t ra = coherent_rsrc(g.A, a_bytes);
    const __amdgpu_buffer_rsrc_t rw = coherent_rsrc(g.W, (size_t)g.ntiles * tile_bytes);
    const int nl = lane & 15, gq = lane >> 4;
    bf16x8 wf[NB][4];
    // Requests of step i (clamped to the last step: the tail re-reads in-bounds data that
    // is never multiplied, so every step issues the same MT + 4 loads and one vmcnt value
    // fits all): this wave's slice (wv) of every row tile's A fragment into LDS buffer
    // i % NB -- lane l's 16 bytes land at 16 l of the slice, the MFMA A-operand lane order
    // -- then the tile's 4 weight loads into register buffer i % NB.
    auto request = [&](int b, int i) {
      const int js = q + SK_SLOTS * min(i, S - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        buffer_to_lds16(ra, &abuf[b][mt][wv][0],
                        (uint32_t)(mt * nsuper + js) * 4096u + 1024u * wv + 16u * (4 * nl + gq), 0);
      const uint32_t so = (uint32_t)((size_t)t * tile_bytes) + (uint32_t)js * 4096u;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        wf[b][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rw, 16u * lane + 1024u * s, so, 2));
    };
    auto step = [&](int b, int i) {
      // step i's A slice and weights have landed once only the P - 1 later steps' loads
      // may be outstanding; the barrier then makes every wave's slice of A(i) visible and
      // proves that step i - 1's buffer, (i + P) % NB, has been read by every wave
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (P == 1) __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if constexpr (P == 2) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(MT + 4) : "memory");
      else __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (MT + 4)) : "memory");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      request((b + P) % NB, i + P);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 af[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          af[mt][s] = __builtin_bit_cast(bf16x8, abuf[b][mt][s][lane]);
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt][s], wf[b][s], acc[mt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int i = 0; i < P; ++i) request(i, i);
    for (int i0 = 0; i0 < S; i0 += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (i0 + u < S) step(u, i0 + u);
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  if (wv < GW) {
    const int t = grp * GW + wv;
    // this slot's partial of the wave's tile (zeros for a slot without steps)
    const __amdgpu_buffer_rsrc_t rp =
        coherent_rsrc(g.sk_part, (size_t)g.ntiles * SK_SLOTS * MT * 1024);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      __builtin_amdgcn_raw_buffer_store_b128(
          acc[mt], rp, (uint32_t)(((t * SK_SLOTS + q) * MT + mt) * 1024 + 16 * lane), 0,
          kCoherentSc1);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();  // partials stored, residual slices staged
  if (threadIdx.x == 0)
    is_last = atomicAdd(&g.sk_counters[grp * kSkCounterStride], 1u) == SK_SLOTS - 1;
  __syncthreads();
  if (!is_last) return;
  if (wv == GW) {
    if (lane == 0) g.sk_counters[grp * kSkCounterStride] = 0u;
    return;
  }
  // merge: each streaming wave finishes its own tile from the four slot partials
  const int t = grp * GW + wv;
  const __amdgpu_buffer_rsrc_t rp =
      coherent_rsrc(g.sk_part, (size_t)g.ntiles * SK_SLOTS * MT * 1024);
  EpiLds L{};
  L.xres = xres + wv * MT * 16 * 16;
  L.gain = gain + wv * 16;
  if constexpr (MT <= 4) {
#pragma unroll
    for (int qq = 0; qq < SK_SLOTS; ++qq)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        part[wv][qq][mt][lane] =
            qq == q ? acc[mt]
                    : __builtin_amdgcn_raw_buffer_load_b128(
                          rp, (uint32_t)(((t * SK_SLOTS + qq) * MT + mt) * 1024 + 16 * lane), 0,
                          kCoherentSc1);
    wave_lds_sync();
    gemm_tile_epilogue<MT>(g, t, 0, part[wv], rowinfo, rowscale, L, lane);
  } else {
    // every slot's partial from the stores above (this one's included, bit for bit), all
    // requested at once, then summed in slot order 0..3 -- the order the epilogue's own
    // sum of slot partials uses -- into this wave's region of the A ring
    floatx4 ps[SK_SLOTS][MT];
#pragma unroll
    for (int qq = 0; qq < SK_SLOTS; ++qq)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        ps[qq][mt] = __builtin_amdgcn_raw_buffer_load_b128(
            rp, (uint32_t)(((t * SK_SLOTS + qq) * MT + mt) * 1024 + 16 * lane), 0, kCoherentSc1);
    floatx4(*sums)[MT][64] = reinterpret_cast<floatx4(*)[MT][64]>(&abuf[0][0][0][0]);
    static_assert(sizeof(abuf) >= sizeof(floatx4) * GW * MT * 64, "sums fit the A ring");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      floatx4 v = ps[0][mt];
#pragma unroll
      for (int qq = 1; qq < SK_SLOTS; ++qq) {
        v[0] += ps[qq][mt][0]; v[1] += ps[qq][mt][1]; v[2] += ps[qq][mt][2]; v[3] += ps[qq][mt][3];
      }
      sums[wv][mt][lane] = v;
    }
    wave_lds_sync();
    gemm_tile_epilogue<MT, 1>(g, t, 0, &sums[wv], rowinfo, rowscale, L, lane);
  }
}

// ------------------------------------------------------------------ normalise pass --

// h = bf16(xg * s_r): the LM head's input, RMSNorm(x) * g rounded once after the row
// factor.  One 256-thread workgroup per row; the first wave forms the row factor from the
// staged partial sums with row_factors (the order the products inside the layers use),
// then every thread rounds 8-column groups into the packed bf16 order.
__global__ __launch_bounds__(256) void k_norm_pack(const float* __restrict__ xg,
                                                   const float* __restrict__ ss, int K, float eps,
                                                   u16* __restrict__ h, int32_t* __restrict__ len,
                                                   const int32_t* __restrict__ ntok_eff, int M) {
  __shared__ float ssl[SS_NP_MAX];
  __shared__ double rs;
  const int r = blockIdx.x, np = K >> 4;
  // the length update of the forward's row bookkeeping: every earlier kernel of the forward
  // has read the old length (the embedding pass) or the start positions derived from it
  if (len && threadIdx.x == 0 && r % M == 0) len[r / M] += ntok_eff[r / M];
  for (int i = threadIdx.x; i < np; i += 256) ssl[i] = ss[(size_t)r * np + i];
  __syncthreads();
  if (threadIdx.x < 64) row_factors(ssl, 1, np, K, eps, threadIdx.x, &rs);
  __syncthreads();
  const float sv = (float)rs;
  for (int c8 = threadIdx.x; c8 < (K >> 3); c8 += 256) {
    const int k = 8 * c8;
    const float4v lo = *reinterpret_cast<const float4v*>(xg + act32_index(r, k, K));
    const float4v hi = *reinterpret_cast<const float4v*>(xg + act32_index(r, k + 4, K));
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      o[e] = f32_to_bf16(lo[2 * e] * sv) | ((uint32_t)f32_to_bf16(lo[2 * e + 1] * sv) << 16);
      o[2 + e] = f32_to_bf16(hi[2 * e] * sv) | ((uint32_t)f32_to_bf16(hi[2 * e + 1] * sv) << 16);
    }
    *reinterpret_cast<uint4*>(h + act_index(r, k, K)) = uint4{o[0], o[1], o[2], o[3]};
  }
}

hipError_t launch_norm_pack(const float* xg, const float* ss, int R, int K, float eps, u16* h,
                            int32_t* len, const int32_t* ntok_eff, int M, hipStream_t s) {
  if (R < 1 || K % 128 || K / 16 > SS_NP_MAX || M < 1 || R % M) return hipErrorInvalidValue;
  k_norm_pack<<<R, 256, 0, s>>>(xg, ss, K, eps, h, len, ntok_eff, M);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32 path -----

// fp32: one wave per output column n, lanes stride K; rows looped.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, const float* __restrict__ W,
                                                  const float* __restrict__ W2, int N1, int N,
                                                  int R, int K, float* __restrict__ C, int ldc,
                                                  int accumulate, const float* __restrict__ rowscale,
                                                  const int32_t* __restrict__ ntok_eff, int M) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* wrow = n < N1 ? W + (size_t)n * K : W2 + (size_t)(n - N1) * K;
  for (int r = 0; r < R; ++r) {
    const float* arow = A + (size_t)r * K;
    float s = 0.f;
    for (int k = lane; k < K; k += 64) s = fmaf(arow[k], wrow[k], s);
    s = wave_sum(s);
    if (rowscale) s *= rowscale[r];
    if (lane == 0) {
      float* p = C + (size_t)r * ldc + n;
      if (ntok_eff && (r % M) >= ntok_eff[r / M]) s = 0.f;
      if (accumulate) *p += s;
      else *p = s;
    }
  }
}

hipError_t launch_gemm_f32(const float* A, const float* W, const float* W2, int N1, int R,
                           int N, int K, float* C, int accumulate, const float* rowscale,
                           const int32_t* ntok_eff, int M, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  if (!W2) { W2 = W; N1 = N; }
  hipExtLaunchKernelGGL(k_gemm_f32, dim3(cdiv(N, 4)), dim3(256), 0, s, e0, e1, 0, A, W, W2,
                        N1, N, R, K, C, N, accumulate, rowscale, ntok_eff, M);
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

// Grid: G persistent workgroups per row block, at most one per compute unit, G chosen
// so that the tiles divide as evenly as possible (every workgroup gets ceil(tiles / G)
// or one fewer).
template <int MT, int TPW>
static void launch_ko_one(dim3 grid, unsigned lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                          const GemmArgs& g, int per) {
  if constexpr (TPW <= ko_tpw_max<MT>()) {  // the dispatcher never asks for more
    // several row blocks (only at four row tiles): ordinary weight loads, shared in L2
    if constexpr (MT == 4) {
      if (grid.y > 1) {
        hipExtLaunchKernelGGL(k_gemm_bf16_ko<MT, TPW, 0>, grid, dim3(GT), lds, s, e0, e1, 0, g,
                              per);
        return;
      }
    }
    hipExtLaunchKernelGGL(k_gemm_bf16_ko<MT, TPW>, grid, dim3(GT), lds, s, e0, e1, 0, g, per);
  }
}

template <int MT>
static void launch_ko(int tpw, dim3 grid, unsigned lds, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1, const GemmArgs& g, int per) {
  switch (tpw) {
    case 2: launch_ko_one<MT, 2>(grid, lds, s, e0, e1, g, per); break;
    case 3: launch_ko_one<MT, 3>(grid, lds, s, e0, e1, g, per); break;
    case 4: launch_ko_one<MT, 4>(grid, lds, s, e0, e1, g, per); break;
    case 5: launch_ko_one<MT, 5>(grid, lds, s, e0, e1, g, per); break;
    case 6: launch_ko_one<MT, 6>(grid, lds, s, e0, e1, g, per); break;
    case 7: launch_ko_one<MT, 7>(grid, lds, s, e0, e1, g, per); break;
    default: launch_ko_one<MT, 8>(grid, lds, s, e0, e1, g, per); break;
  }
}

hipError_t launch_gemm_bf16(const GemmArgs& g0, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  GemmArgs g = g0;
  g.ntiles = gemm_blocks_x(g);
  const int tiles = cdiv(g.R, 16);
  const int rowblocks = tiles <= 3 ? 1 : cdiv(g.R, 64);
  const int gmax = std::max(1, device_cus() * SPEC_GEMM_WPC / rowblocks);
  // Column tiles per step.  With 32+ rows a pair of tiles streamed together takes about
  // 1.5 times as long as one tile (measured at 48 rows: the A fragments are read once
  // for both), so pairs are used when the busiest workgroup's time in tile units,
  // 1.5 * ceil(pairs / gmax), is below ceil(tiles / gmax).
  int NTc = 1;
  if (tiles >= 2 && g.ntiles % 2 == 0 && 3 * cdiv(g.ntiles / 2, gmax) < 2 * cdiv(g.ntiles, gmax))
    NTc = 2;
  const int ngroups = g.ntiles / NTc;
  const int per = cdiv(ngroups, gmax);
  const int G = cdiv(ngroups, per);
  if (g.ss_in && (g.ss_np > SS_NP_MAX || g.ss_np % 8)) return hipErrorInvalidValue;
  if (g.mode == EPI_QKV_ROPE && g.hd > 2 * ROPE_HALF_MAX) return hipErrorInvalidValue;
  const int mt = std::min(tiles, 4);
  if (g.mode == EPI_RESID && tiles >= 2 && tiles <= SK_MT_MAX && g.ntiles % SK_SLOTS == 0 &&
      g.ntiles <= device_cus() * SPEC_GEMM_WPC && g.sk_part && g.sk_counters) {
    // residual products owning one tile per workgroup (2-4 row tiles), and every residual
    // product of 5-8 row tiles: four tiles per workgroup, one wave slot each, A shared
    // across the tiles -- up to 128 rows, so the weights stream once (the other kernels
    // stream them once per 64 rows)
    const unsigned lds = (unsigned)(GW * (tiles * 16 * 16 * 4 + 16 * 4));
#define SPEC_SK_LAUNCH(MT_) \
  hipExtLaunchKernelGGL(k_gemm_sk<MT_>, dim3(g.ntiles), dim3(GT), lds, s, e0, e1, 0, g)
    switch (tiles) {
      case 2: SPEC_SK_LAUNCH(2); break;
      case 3: SPEC_SK_LAUNCH(3); break;
      case 4: SPEC_SK_LAUNCH(4); break;
      case 5: SPEC_SK_LAUNCH(5); break;
      case 6: SPEC_SK_LAUNCH(6); break;
      case 7: SPEC_SK_LAUNCH(7); break;
      default: SPEC_SK_LAUNCH(8); break;
    }
#undef SPEC_SK_LAUNCH
    return hipGetLastError();
  }
  {
    // several row tiles and several tiles per workgroup: the K-outer kernel, in chunks
    // of equal size, at most ko_tpw_max tiles and as many as its LDS allows
    int kper = cdiv(g.ntiles, gmax);
    int kG = cdiv(g.ntiles, kper);
    if (rowblocks > 1) {
      // row blocks of one column group on one XCD (dispatch places workgroup i on XCD
      // i mod 8): an x extent that is a multiple of 8, within the one-round grid
      const int kg8 = std::min((kG + 7) / 8 * 8, gmax / 8 * 8);
      if (kg8 >= 8 && kg8 <= g.ntiles) {
        kG = kg8;
        kper = cdiv(g.ntiles, kG);
      }
    }
    if (mt >= 2 && kper >= 2) {
      const int tmax = mt == 4 ? ko_tpw_max<4>() : ko_tpw_max<2>();
      for (int tcap = tmax; tcap >= 2; --tcap) {
        const int tpw = cdiv(kper, cdiv(kper, tcap));
        const int kstatic = std::max(tpw, 4) * GW * mt * 1024 + mt * 16 * (8 + 8);
        const int kdyn = ko_lds_bytes(mt, tpw, g.mode, g.ss_np, g.ss_in != nullptr);
        if (kstatic + kdyn > 160 * 1024) continue;
        const dim3 grid(kG, rowblocks);
        if (mt == 2) launch_ko<2>(tpw, grid, (unsigned)kdyn, s, e0, e1, g, kper);
        else if (mt == 3) launch_ko<3>(tpw, grid, (unsigned)kdyn, s, e0, e1, g, kper);
        else launch_ko<4>(tpw, grid, (unsigned)kdyn, s, e0, e1, g, kper);
        return hipGetLastError();
      }
    }
  }
  // stage every row's partial sums of squares at once when the LDS holds them next to
  // the tile partials (static LDS of the kernel), else 16 rows at a time
  const int static_lds = 2 * NTc * GW * mt * 1024 + mt * 16 * (8 + 8);
  g.ss_rows = mt * 16;
  if (static_lds + epi_lds_bytes(mt, NTc, g.mode, std::min(g.ss_rows, g.R), g.ss_np, g.hd / 2,
                                 g.R, g.ss_in != nullptr) > 160 * 1024)
    g.ss_rows = 16;
  const unsigned lds = (unsigned)epi_lds_bytes(mt, NTc, g.mode, std::min(g.ss_rows, g.R),
                                               g.ss_np, g.hd / 2, g.R, g.ss_in != nullptr);
  if (static_lds + (int)lds > 160 * 1024) return hipErrorInvalidValue;
#define SPEC_GEMM_LAUNCH(MT_, NT_, GY)                                                     \
  hipExtLaunchKernelGGL(k_gemm_bf16<MT_, NT_>, dim3(G, GY), dim3(GT), lds, s, e0, e1, 0, g)
  if (tiles <= 1) {
    SPEC_GEMM_LAUNCH(1, 1, 1);
  } else if (tiles <= 2) {
    if (NTc == 2) SPEC_GEMM_LAUNCH(2, 2, 1);
    else SPEC_GEMM_LAUNCH(2, 1, 1);
  } else if (tiles <= 3) {
    if (NTc == 2) SPEC_GEMM_LAUNCH(3, 2, 1);
    else SPEC_GEMM_LAUNCH(3, 1, 1);
  } else {
    if (NTc == 2) SPEC_GEMM_LAUNCH(4, 2, rowblocks);
    else SPEC_GEMM_LAUNCH(4, 1, rowblocks);
  }
#undef SPEC_GEMM_LAUNCH
  return hipGetLastError();
}


}  // namespace specdec
