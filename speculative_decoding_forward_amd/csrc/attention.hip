// KV-cache attention of the verify pass (bf16 models): the K+1 query rows of each
// sequence attend causally over its cache ([LENS] §2.1 step 2: one target call scores
// every drafted position; [GC] "How It Works": the verify pass runs the draft tokens
// through the target in parallel).  A query at cache position p sees positions t <= p.
//
// Cache layout (per layer, row b, head h; the arrangement inside a head region of
// cap = roundup(max_len, 32) positions x hd elements):
//   K: blocks of 16 positions; block k, slice s (dims 32s .. 32s+31) and lane l hold
//      K[16k + l%16][32s + 8(l/16) .. +8] -- the A operand of v_mfma_f32_16x16x32_bf16
//      for S^T = K Q^T;
//   V: blocks of 32 positions; block k, dim tile u (dims 16u .. 16u+15) and lane l hold
//      V[32k + key(l/16, e)][16u + l%16] for e = 0..7 with key(g, e) = 4g + e (e < 4)
//      or 16 + 4g + e - 4 -- the B operand of O = P V, in the key order in which the
//      S^T fragments leave the first product (so P never moves between lanes).
// Every wave load is therefore 1 KB contiguous.  K and V are read with non-temporal loads
// except for the later layers of a model whose K/V fits the memory-side cache
// (kAttnCacheBudget).
//
// Split-KV: workgroup (split, h, b*NG + qg) owns `bps` consecutive 32-key blocks of
// (b, h) and one group of up to 16 queries.  The split count (the grid) is fixed per
// launch shape -- at most one workgroup per compute unit, about 1.5 blocks per wave over
// the cache capacity (attn_nsplit) -- and each row divides its ACTUAL blocks over it:
// bps = max(ceil(blocks / splits), waves), read on the device from the row's length, so
// a row far shorter than the capacity still spreads over every split (a split count
// taken from the capacity left 3 of 8 splits idle at 2048 of 3456 positions: 15.6 against
// 13.5 us per launch), and no split has less than one block per wave.  Its waves (8 for
// head_dim 128) take the blocks
// round-robin, keep two blocks of K and V in flight each -- with a split's blocks thus
// all requested at once -- and run an online softmax per query.  The
// wave states merge in LDS; with more than one split the workgroup partial goes to
// global memory and the last workgroup of (b, h, qg) to finish -- found by a
// completion counter, one per (b, h, qg), 128 bytes apart -- merges them in split order
// and writes the bf16 output.  P enters the second product as bf16 hi + lo
// parts (two MFMAs), which keeps its value to ~16 bits.
#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "act_layout.h"
#include "common.h"
#include "internal.h"

namespace specdec {

// Waves per workgroup and blocks each wave keeps in flight (ring depth).  With one
// workgroup per compute unit the ring can be deep: a split's blocks are then all
// requested at once.
#ifndef SPEC_ATTN_WAVES
#define SPEC_ATTN_WAVES 8
#endif
#ifndef SPEC_ATTN_RING
#define SPEC_ATTN_RING 2
#endif
template <int HD> constexpr int attn_waves() { return HD == 128 ? SPEC_ATTN_WAVES : 4; }
template <int HD> constexpr int attn_ring() { return HD == 128 ? SPEC_ATTN_RING : 2; }
constexpr int AQ = 16;   // queries per group
constexpr int AKB = 32;  // keys per block

__device__ __forceinline__ bf16x8 ldfrag(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Buffer resource over `bytes` bytes of a K or V head region (offsets past it read zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kv_rsrc(const u16* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(base), 0,
                                           (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                           0x00020000);
}

// One 16-byte K/V fragment at byte offset `off` of a head region, with the cache policy an
// immediate of the instruction (AUX 2: non-temporal), so that the two policies of the
// kernel's branch stay distinct instructions.
template <int AUX>
__device__ __forceinline__ bf16x8 ldkv(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

// K/V bytes of all layers of a model that the memory-side cache (256 MB on MI355X) is left
// to hold across forwards: the cache policy of the K/V loads below.  Whole 7B-shape rounds
// took 6.27-6.28 ms with 200, 224 or 240 MB and 6.30 ms with 256 MB.
constexpr size_t kAttnCacheBudget = (size_t)224 << 20;

template <int HD, int AW = attn_waves<HD>(), int RING = attn_ring<HD>()>
__global__ __launch_bounds__(AW * 64) void k_attn_bf16(
    const u16* __restrict__ q, int M, int H, const u16* __restrict__ kc,
    const u16* __restrict__ vc, size_t row_stride, size_t head_stride,
    const int32_t* __restrict__ pos0, const int32_t* __restrict__ ntok_eff,
    float* __restrict__ part, unsigned* __restrict__ counters, int nsplit,
    u16* __restrict__ out, int layer, int n_layers) {
  constexpr int NS = HD / 32;  // K slices (MFMAs per 16-key tile)
  constexpr int NT = HD / 16;  // dim tiles of O
  __shared__ float wm[AW][AQ], wl[AW][AQ];
  __shared__ float wo[AW][AQ][HD + 1];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int NG = cdiv(M, AQ);
  const int b = blockIdx.z / NG, qg = blockIdx.z % NG;
  const int h = blockIdx.y, split = blockIdx.x;
  const int nq = ntok_eff[b];
  const int p0 = pos0[b];
  const int len_end = p0 + nq;
  const int nblk = cdiv(len_end, AKB);
  const int bps = max(cdiv(nblk, nsplit), AW);  // blocks per split of this row
  // blocks of this wave in its split: wv, wv + AW, ... below bps
  const int nmine = wv < bps ? (bps - 1 - wv) / AW + 1 : 0;
  const int n_active = cdiv(nblk, bps);
  const int d = H * HD;
  const int jend = min(M, qg * AQ + AQ);  // rows of this query group
  if (qg * AQ >= nq) {
    // no query of this row in this group: the first split writes the padding rows
    if (split == 0)
      for (int idx = threadIdx.x; idx < (jend - qg * AQ) * HD; idx += AW * 64)
        out[act_index(b * M + qg * AQ + idx / HD, h * HD + idx % HD, d)] = 0;
    return;
  }
  if (split >= n_active) return;  // uniform over the workgroup
  // Cache policy of the K/V loads (a hint: results do not depend on it).  A model whose K/V
  // at this length fits about twice the budget (a draft, a small model) keeps its later
  // layers in the memory-side cache, where the next forward finds them, and streams its
  // first layers with non-temporal loads: a K/V stream larger than the cache, read in the
  // same order every forward, would otherwise evict itself before reuse.  Larger ones (a
  // 7B or 70B target, any batch of drafts) stream every layer.
  const size_t layer_bytes = (size_t)(gridDim.z / NG) * 4u * (size_t)H * (size_t)len_end * HD;
  const bool stream = (size_t)n_layers * layer_bytes > 2 * kAttnCacheBudget ||
                      layer < n_layers - (int)(kAttnCacheBudget / layer_bytes);
  const u16* kh = kc + (size_t)b * row_stride + (size_t)h * head_stride;
  const u16* vh = vc + (size_t)b * row_stride + (size_t)h * head_stride;
  const float scale = 1.0f / sqrtf((float)HD);

  // query fragments (B operand of S^T = K Q^T): query column nl, dims 32s + 8g .. +8;
  // columns without a query read row 0 (finite) and are masked
  const int jq = qg * AQ + nl;
  const bool qok = jq < nq;
  const u16* qrow = q + (size_t)(b * M + (qok ? jq : 0)) * d + h * HD + 8 * g;
  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = ldfrag(qrow + 32 * s);
  const int qpos = p0 + jq;  // the query's cache position

  // Ring of RING blocks.  Block i of this wave is split*bps + wv + AW*i (i < nmine); a
  // block past the row's end is clamped to its last block (in bounds) and masked.
  bf16x8 kf[RING][2][NS];
  bf16x8 vf[RING][NT];
  const int blk0 = split * bps + wv;
  // buffer resources over this (row, head)'s K and V regions (head_stride elements each)
  const __amdgpu_buffer_rsrc_t rk = kv_rsrc(kh, head_stride * 2);
  const __amdgpu_buffer_rsrc_t rv = kv_rsrc(vh, head_stride * 2);
  auto load_policy = [&](auto aux, int slot, int blk) {
    constexpr int A = decltype(aux)::value;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        kf[slot][kt][s] =
            ldkv<A>(rk, (uint32_t)((((2 * blk + kt) * NS + s) * 512 + 8 * lane) * 2));
#pragma unroll
    for (int u = 0; u < NT; ++u)
      vf[slot][u] = ldkv<A>(rv, (uint32_t)(((blk * NT + u) * 512 + 8 * lane) * 2));
  };
  auto load = [&](int slot, int i) {
    const int blk = min(blk0 + AW * min(i, max(nmine - 1, 0)), nblk - 1);
    if (stream) load_policy(std::integral_constant<int, 2>{}, slot, blk);
    else load_policy(std::integral_constant<int, 0>{}, slot, blk);
  };
  float m = -INFINITY, l = 0.f;  // running max / sum of query nl (replicated over g)
  floatx4 o[NT];                 // O[query 4g + e][dim 16u + nl]
#pragma unroll
  for (int u = 0; u < NT; ++u) o[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot, int i) {
    const bool in_share = i < nmine;
    const int kb = (blk0 + AW * i) * AKB;  // first key position of the block
    if (kb + AKB > len_end) {
      // the block holding the row's end: positions from len_end on were never written
      // by this row (the arena is caller memory), and P = 0 there does not cancel a
      // NaN in the P V product, so those V elements are zeroed (K needs no care: masked
      // scores are replaced, not multiplied)
      typedef unsigned short u16x8v __attribute__((ext_vector_type(8)));
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        u16x8v w = __builtin_bit_cast(u16x8v, vf[slot][u]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kb + (e < 4 ? 4 * g + e : 12 + 4 * g + e) >= len_end) w[e] = 0;
        vf[slot][u] = __builtin_bit_cast(bf16x8, w);
      }
    }
    float sc[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[slot][kt][s], qf[s], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kp = kb + 16 * kt + 4 * g + e;
        sc[kt][e] = (in_share && qok && kp <= qpos) ? acc[e] * scale : -INFINITY;
      }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mb = fmaxf(mb, sc[kt][e]);
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mn = fmaxf(m, mb);
    const float alpha = (mn == -INFINITY) ? 1.f : expf(m - mn);
    float p[2][4], ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[kt][e] = (sc[kt][e] == -INFINITY) ? 0.f : expf(sc[kt][e] - mn);
        ps += p[kt][e];
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
    m = mn;
    // O rows are queries 4g + e; their factors sit in lanes 4g + e
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ae = __shfl(alpha, 4 * g + e, 64);
#pragma unroll
      for (int u = 0; u < NT; ++u) o[u][e] *= ae;
    }
    // O += P V with P split into bf16 hi + lo parts (two MFMAs per dim tile): query nl,
    // keys (4g + e | 16 + 4g + e) = the V key order, so P never moves between lanes;
    // the split keeps P's value to ~16 bits, and the result matched an fp32-P evaluation
    // to the last digit of its error statistics against an fp64 reference
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    u16x8 hi8, lo8;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float pv = p[t >> 2][t & 3];
      const u16 hb = f32_to_bf16(pv);
      hi8[t] = hb;
      lo8[t] = f32_to_bf16(pv - bf16_to_f32(hb));
    }
    const bf16x8 phi = __builtin_bit_cast(bf16x8, hi8), plo = __builtin_bit_cast(bf16x8, lo8);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vf[slot][u], o[u], 0, 0, 0);
      o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vf[slot][u], o[u], 0, 0, 0);
    }
  };
  // Loads are only issued for the wave's own blocks (a uniform branch per wave); the
  // scheduling fences keep a slot's refill right behind its use, so RING blocks stay
  // in flight.
#pragma unroll
  for (int r = 0; r < RING; ++r) {
    if (r < nmine) load(r, r);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int i0 = 0; i0 < nmine; i0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      if (i0 + r < nmine) {
        compute(r, i0 + r);
        __builtin_amdgcn_sched_barrier(0);
        if (i0 + r + RING < nmine) load(r, i0 + r + RING);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // wave states -> LDS; merge the waves: thread -> (query jj, dims)
  if (lane < AQ) {
    wm[wv][lane] = m;
    wl[wv][lane] = l;
  }
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) wo[wv][4 * g + e][16 * u + nl] = o[u][e];
  __syncthreads();
  constexpr int TPQ = AW * 64 / AQ;  // threads per query (16 or 32)
  constexpr int DPT = HD / TPQ;      // dims per thread (4)
  static_assert(DPT == 4 || DPT == 8, "merge layout");
  const int jj = threadIdx.x / TPQ, tt = threadIdx.x % TPQ;
  const int j = qg * AQ + jj;
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < AW; ++w) mx = fmaxf(mx, wm[w][jj]);
  float f[AW];
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < AW; ++w) {
    f[w] = (wm[w][jj] == -INFINITY) ? 0.f : expf(wm[w][jj] - mx);
    lsum += f[w] * wl[w][jj];
  }
  float v[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < AW; ++w) a += f[w] * wo[w][jj][tt * DPT + k];
    v[k] = a;
  }
  if (n_active == 1) {
    // one split: this workgroup has the whole row; padding rows of the group are zeros
    if (j < jend) {
      uint32_t ov[DPT / 2];
#pragma unroll
      for (int k = 0; k < DPT / 2; ++k)
        ov[k] = j < nq ? (f32_to_bf16(v[2 * k] / lsum) |
                          ((uint32_t)f32_to_bf16(v[2 * k + 1] / lsum) << 16))
                       : 0u;
      u16* dst = out + act_index(b * M + j, h * HD + tt * DPT, d);  // DPT columns contiguous
      if constexpr (DPT == 8)
        *reinterpret_cast<uint4*>(dst) = uint4{ov[0], ov[1], ov[2], ov[3]};
      else
        *reinterpret_cast<uint2*>(dst) = uint2{ov[0], ov[1]};
    }
    return;
  }
  // partials of (b, h): O rows [nsplit][M][HD], then (max, sum) pairs [nsplit][M][2]
  const int Bt = gridDim.z / NG;
  const size_t obytes = (size_t)nsplit * M * HD * 4, mlbytes = (size_t)nsplit * M * 8;
  const float* po = part + (((size_t)b * H + h) * nsplit) * M * HD;
  const float* pml = part + (size_t)Bt * H * nsplit * M * HD + (((size_t)b * H + h) * nsplit) * M * 2;
  const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(po, obytes), rml = coherent_rsrc(pml, mlbytes);
  if (j < nq) {
    const size_t row = (size_t)split * M + j;
#pragma unroll
    for (int k = 0; k < DPT; k += 4)
      __builtin_amdgcn_raw_buffer_store_b128(float4v{v[k], v[k + 1], v[k + 2], v[k + 3]}, ro,
                                             (int)((row * HD + tt * DPT + k) * 4), 0,
                                             kCoherentSc1);
    if (tt == 0)
      __builtin_amdgcn_raw_buffer_store_b64(float2v{mx, lsum}, rml, (int)(row * 8), 0,
                                            kCoherentSc1);
  }
  // count this workgroup in once its partial is written
  const int cidx = ((b * H + h) * NG + qg) * kAttnCounterStride;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last_flag = atomicAdd(&counters[cidx], 1u) == (unsigned)(n_active - 1);
  __syncthreads();
  if (!last_flag) return;
  // The last workgroup merges the splits in split order: a thread takes 4 dims of one
  // query and issues the loads of up to SM splits at once (one memory round trip per SM
  // splits; clamped indices, no branches around the loads).
  constexpr int NQD = HD / 4, SM = 16;
  for (int item = threadIdx.x; item < (jend - qg * AQ) * NQD; item += AW * 64) {
    const int jr = qg * AQ + item / NQD, c4 = 4 * (item % NQD);
    float r[4] = {0.f, 0.f, 0.f, 0.f};  // padding rows of this group are written as zeros
    if (jr < nq) {
      float mm = -INFINITY, den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
      for (int cb = 0; cb < n_active; cb += SM) {
        float2v ml[SM];
        float4v oc[SM];
#pragma unroll
        for (int u = 0; u < SM; ++u) {
          const size_t row = (size_t)min(cb + u, n_active - 1) * M + jr;
          ml[u] = __builtin_amdgcn_raw_buffer_load_b64(rml, (int)(row * 8), 0, kCoherentSc1);
          oc[u] = __builtin_amdgcn_raw_buffer_load_b128(ro, (int)((row * HD + c4) * 4), 0,
                                                        kCoherentSc1);
        }
#pragma unroll
        for (int u = 0; u < SM; ++u) {
          if (cb + u >= n_active || ml[u].x == -INFINITY) continue;
          const float nm = fmaxf(mm, ml[u].x);
          const float s0 = mm == -INFINITY ? 0.f : expf(mm - nm);
          const float s1 = expf(ml[u].x - nm);
          den = den * s0 + ml[u].y * s1;
#pragma unroll
          for (int k = 0; k < 4; ++k) num[k] = num[k] * s0 + oc[u][k] * s1;
          mm = nm;
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = num[k] / den;
    }
    const uint32_t lo = f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
    const uint32_t hi = f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
    *reinterpret_cast<uint2*>(out + act_index(b * M + jr, h * HD + c4, d)) = uint2{lo, hi};
  }
  if (threadIdx.x == 0) counters[cidx] = 0u;
}

// Upper bound of attn_nsplit for any device (workspace sizing): one split per block and
// at most kAttnMaxCUs workgroups.
int attn_max_splits(int B, int H, int M, int max_len) {
  const int groups = B * H * cdiv(M, AQ);
  return std::max(1, std::min(cdiv(max_len, AKB), cdiv(kAttnMaxCUs, groups)));
}

// Splits per (row, head, query group): as many as make the grid one workgroup per
// compute unit (a CU holding two workgroups streams its two shares at half the rate
// and finishes last), but no more than give each split about 1.5 blocks per wave of the
// capacity (kAttnBlocksPerSplit): more, smaller splits only lengthen the merge.  Over a
// 69-block capacity, 8 or 14 splits (9 or 5 blocks) took 14.2 / 11.1 us at 6 / 1
// queries per row, 6 splits of 12 blocks 13.6 / 10.6 us, 5 of 16 and 3 of 24 longer
// again.  The kernel divides each row's actual blocks over these splits.
constexpr int kAttnBlocksPerSplit = 3 * SPEC_ATTN_WAVES / 2;
int attn_nsplit(int B, int H, int M, int max_len) {
  const int blocks = cdiv(max_len, AKB), groups = B * H * cdiv(M, AQ);
  int ns = std::max(1, std::min(device_cus(), kAttnMaxCUs) / groups);
  ns = std::min(ns, cdiv(blocks, kAttnBlocksPerSplit));
  ns = std::min(ns, attn_max_splits(B, H, M, max_len));
  // the same split count with fewer blocks per split would leave splits empty: shrink
  // it to the number that the per-split block count really needs
  const int bps = cdiv(blocks, ns);
  return cdiv(blocks, bps);
}

int attn_groups(int M) { return cdiv(M, AQ); }

hipError_t launch_attention_bf16(const u16* q, const u16* kc, const u16* vc, size_t row_stride,
                                 size_t head_stride, int B, int M, int H, int hd,
                                 const int32_t* pos0, const int32_t* ntok_eff, float* part,
                                 unsigned* counters, int max_len, u16* out, int layer,
                                 int n_layers, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int nsplit = attn_nsplit(B, H, M, max_len);
  const dim3 grid(nsplit, H, B * attn_groups(M));
  // The kernel picks the K/V cache policy per layer (kAttnCacheBudget).  Measured per launch
  // at the 7B shape and 2048 positions, non-temporal against ordinary loads: 8 rows of 6
  // queries 50.7 -> 45.7 us, 4 rows 29.8 -> 28.2, 16 rows of one query 49.3 -> 44.5, and the
  // one-row verify pass 2.833 -> 2.805 ms in replayed rounds; the one-row draft (about
  // 270 MB of K/V over 16 layers) 10.9 -> 12.5 us with every layer streamed, and 10.8 ->
  // 10.3 us on average with only the layers past the budget streamed (6.39 -> 6.29 ms per
  // 7B-shape round).
#define SPEC_ATTN_LAUNCH(HD_)                                                                 \
  hipExtLaunchKernelGGL(k_attn_bf16<HD_>, grid, dim3(attn_waves<HD_>() * 64), 0, s, e0, e1, 0, \
                        q, M, H, kc, vc, row_stride, head_stride, pos0, ntok_eff, part,        \
                        counters, nsplit, out, layer, n_layers)
  if (hd == 128)
    SPEC_ATTN_LAUNCH(128);
  else if (hd == 64)
    SPEC_ATTN_LAUNCH(64);
  else
    return hipErrorInvalidValue;
#undef SPEC_ATTN_LAUNCH
  return hipGetLastError();
}

// ------------------------------------------------------------ layout conversion -----

// Natural [L][B][2][H][n][hd] block <-> the cache's packed head regions (positions
// [0, n) of every row, layer and head).  One thread per element.
__global__ void k_kv_convert(u16* __restrict__ cache, u16* __restrict__ nat, int L, int B,
                             int H, int hd, int n, size_t layer_stride, size_t row_stride,
                             size_t kv_stride, size_t head_stride, int to_cache) {
  const size_t total = (size_t)L * B * 2 * H * n * hd;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    size_t r = idx;
    const int i = (int)(r % hd); r /= hd;
    const int p = (int)(r % n); r /= n;
    const int hh = (int)(r % H); r /= H;
    const int kv = (int)(r % 2); r /= 2;
    const int bb = (int)(r % B);
    const int ll = (int)(r / B);
    u16* head = cache + (size_t)ll * layer_stride + (size_t)bb * row_stride +
                (size_t)kv * kv_stride + (size_t)hh * head_stride;
    const size_t off = kv == 0 ? kv_k_offset(p, i, hd) : kv_v_offset(p, i, hd);
    if (to_cache)
      head[off] = nat[idx];
    else
      nat[idx] = head[off];
  }
}

hipError_t launch_kv_convert(u16* cache, u16* nat, int L, int B, int H, int hd, int n,
                             size_t layer_stride, size_t row_stride, size_t kv_stride,
                             size_t head_stride, int to_cache, hipStream_t s) {
  const size_t total = (size_t)L * B * 2 * H * n * hd;
  if (total == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  k_kv_convert<<<blocks, 256, 0, s>>>(cache, nat, L, B, H, hd, n, layer_stride, row_stride,
                                      kv_stride, head_stride, to_cache);
  return hipGetLastError();
}

}  // namespace specdec
