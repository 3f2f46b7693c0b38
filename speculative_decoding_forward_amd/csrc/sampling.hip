// Fused vocab kernels: knob transform (temperature -> top-k -> top-p -> softmax) of
// target and draft logit rows, the accept test against Philox uniforms, the residual
// max(0, p - q) and its inverse-CDF sample, the bonus sample, first-rejection select,
// and the draft-step sampler.
//
// Method ([ZSM] "The algorithm"; [CANON] "Acceptance, and why the distribution is NOT
// distorted"; [LENS] §2.1 and §2.3; [GC] "How It Works" steps 3-4; knobs before the
// rule: [NOTE] "Key results" and Recommendation R3):
//   accept x~_j  <=>  u_acc * q_j(x~_j) < p_j(x~_j)
//   first rejection a: y ~ norm(max(0, p_a - q_a)); all accepted: bonus y ~ p_K.
// The K+1 positions of a row are evaluated in parallel, one workgroup each; because
// the uniforms are counter-based on (round, j, b, purpose), the data-parallel result
// equals the left-to-right walk the pages describe.
//
// Layout: a workgroup of 1024 threads (16 waves) owns one logit row of V <= 32768
// values, VPT = ceil(V/1024) per thread in registers, element i = t*1024 + tid
// (coalesced loads).  Each row is read from HBM exactly once.
//
// Numerics: exponentials in fp32, computed once per element; all sums (softmax
// normaliser, kept mass, the residual mass and the inverse-CDF running sums) in fp64
// or exact integers with a fixed reduction order.  Thresholds are found by radix
// select on an order-preserving 32-bit key with integer histograms, so the selection
// is deterministic: top-k on the key of the logit (ties are equal logits), top-p on
// the key of the unnormalised probability e = exp((l - max) / T) with each element's
// mass e/S as a 2^-52 fixed-point integer (ties are equal probabilities, the rule
// "keep every token whose probability reaches the threshold's").  Temperature 0 is
// argmax decoding: the processed row is one-hot at the lowest index holding the
// largest logit, and the rule then runs unchanged (the draft proposes argmax q, a
// draft is accepted iff it is argmax p, the resample and the bonus are argmax p).
#include <float.h>
#include <limits.h>

#include "common.h"
#include "internal.h"

namespace specdec {

constexpr int VT = 1024;   // threads per vocab workgroup
constexpr int NWV = VT / 64;
constexpr int MAXVPT = 32;  // V <= 32768
constexpr int RBINS = 2048;  // radix digit bins (11-bit digits)

struct VocabLDS {
  double dred[NWV];
  float fred[NWV];
  int ired[NWV];
  unsigned long long hist[RBINS];
  unsigned long long wsuf[NWV];
  double scan[NWV];
  float w[MAXVPT * VT];  // inverse-CDF weights in token-id order
  unsigned long long bcast_ull[3];
  int bcast_i[4];
  float px, qx;
  float zero;  // always 0; read inside loops so per-element work is not hoisted
};

// Lane shuffles whose address is computed from a lane id read afresh each time (the
// asm is volatile): the compiler would otherwise keep one address register per
// shuffle pattern live through the whole kernel, and with a 32-value row in registers
// those spill.
__device__ __forceinline__ int lane_fresh() {
  int l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
__device__ __forceinline__ uint64_t shfl_src_u64(uint64_t v, int src) {
  const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)v);
  const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)(v >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ double shfl_src_d(double v, int src) {
  return __longlong_as_double((long long)shfl_src_u64((uint64_t)__double_as_longlong(v), src));
}
__device__ __forceinline__ float shfl_xor_f(float v, int o) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane_fresh() ^ o) << 2, __float_as_int(v)));
}
// value of lane - o (lanes below o read a wrapped lane; callers mask those)
__device__ __forceinline__ double shfl_up_d(double v, int o) {
  return shfl_src_d(v, (lane_fresh() - o) & 63);
}
// value of lane + o (wrapped; callers mask)
__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t v, int o) {
  return shfl_src_u64(v, (lane_fresh() + o) & 63);
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    v = min(v, __builtin_amdgcn_ds_bpermute((lane_fresh() ^ o) << 2, v));
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_src_d(v, lane_fresh() ^ o);
  return v;
}
__device__ __forceinline__ double block_sum_d(double v, double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum_d(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < NWV; ++i) t += red[i];
  return t;
}

// order-preserving key of a float (-0 folded onto +0)
__device__ __forceinline__ uint32_t okey(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct RadixResult {
  uint32_t t;                // threshold key: keep key >= t
  unsigned long long kept;   // total weight of the kept elements
  bool all;                  // the target was not reached: keep everything
};

// Largest key t such that the total weight of the participating elements with key
// >= t reaches `target` (> 0).  kf(x, key) says whether element x takes part and gives
// its key, whose bits from KB up are zero; wf(x) its integer weight (evaluated only for
// elements a pass counts).  Three passes over digits of 11, 11 and KB - 22 bits (high to
// low), each an LDS histogram of the elements whose key matches the digits chosen so far,
// a block-wide suffix scan over the 2048 bins, and the unique bin where the running
// weight crosses the target.  Keys with fewer significant bits (KB < 32) spread the
// first pass over all of its bins, which divides the LDS atomics that collide on a bin.
template <int VPT, int KB, typename KF, typename WF>
__device__ __forceinline__ RadixResult radix_select(const float (&v)[VPT], KF kf, WF wf,
                                                    unsigned long long target, VocabLDS& sh) {
  static_assert(KB > 22 && KB <= 32, "key bits");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t prefix = 0;
  unsigned long long above = 0, kept = 0;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    // digit bits [shift, hs); bits [hs, KB) were fixed by the earlier passes
    const int shift = pass == 0 ? KB - 11 : (pass == 1 ? KB - 22 : 0);
    const int hs = pass == 0 ? KB : (pass == 1 ? KB - 11 : KB - 22);
    const uint32_t dmask = pass == 2 ? (1u << (KB - 22)) - 1u : 2047u;
    sh.hist[2 * tid] = 0ull;
    sh.hist[2 * tid + 1] = 0ull;
    if (tid == 0) sh.bcast_i[0] = -1;
    __syncthreads();
    const float zero = sh.zero;
#pragma unroll
    for (int t = 0; t < VPT; ++t) {
      const float x = v[t] + zero;
      uint32_t k;
      if (kf(x, k) && (pass == 0 || (k >> hs) == (prefix >> hs)))
        atomicAdd(&sh.hist[(k >> shift) & dmask], wf(x));
      __builtin_amdgcn_sched_barrier(0);  // one element at a time: bounded register use
    }
    __syncthreads();
    // thread tid owns bins 2tid, 2tid+1; suffix sums from the top bin down
    const unsigned long long b0 = sh.hist[2 * tid], b1 = sh.hist[2 * tid + 1];
    const unsigned long long mine = b0 + b1;
    unsigned long long suf = mine;  // sum over lanes >= lane of this wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long y = shfl_down_u64(suf, o);
      if (lane + o < 64) suf += y;
    }
    if (lane == 0) sh.wsuf[wv] = suf;
    __syncthreads();
    unsigned long long after = suf - mine;  // bins >= 2tid + 2
#pragma unroll 1
    for (int i0 = wv + 1; i0 < NWV; i0 += 4) {  // later waves' totals, four reads at a time
      unsigned long long y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = i0 + k < NWV ? sh.wsuf[i0 + k] : 0ull;
#pragma unroll
      for (int k = 0; k < 4; ++k) after += y[k];
    }
    const unsigned long long n2 = above + after, n1 = n2 + b1, n0 = n1 + b0;
    // the largest digit d whose weight at or above it (plus `above`) reaches the target
    if (n1 >= target && n2 < target) {
      sh.bcast_i[0] = 2 * tid + 1;
      sh.bcast_ull[0] = n2;
      sh.bcast_ull[1] = n1;
    } else if (n0 >= target && n1 < target) {
      sh.bcast_i[0] = 2 * tid;
      sh.bcast_ull[0] = n1;
      sh.bcast_ull[1] = n0;
    }
    if (pass == 0 && tid == 0) sh.bcast_ull[2] = n0;  // the total weight
    __syncthreads();
    const int d = sh.bcast_i[0];
    if (d < 0) {  // first pass only: all elements together do not reach the target
      const unsigned long long total = sh.bcast_ull[2];
      __syncthreads();
      return RadixResult{0u, total, true};
    }
    above = sh.bcast_ull[0];
    kept = sh.bcast_ull[1];
    prefix |= ((uint32_t)d) << shift;
    __syncthreads();
  }
  return RadixResult{prefix, kept, false};
}

// In place: v holds a logit row on entry (-inf past the row's end) and the processed
// probability row on exit (0 outside the kept set).  Returns false (row zeroed) if a
// logit of the row is not finite.
template <int VPT>
__device__ __forceinline__ bool process_row(float (&v)[VPT], int V, const SamplingKnobs& kn,
                                            VocabLDS& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) sh.zero = 0.f;  // published by the barrier below
  // finiteness and the maximum in one block reduction
  int bad = 0;
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < VPT; ++t) {
    if (t * VT + tid < V && !isfinite(v[t])) bad = 1;
    m = fmaxf(m, v[t]);
  }
  m = wave_max_f(m);
  const bool wbad = __ballot(bad) != 0ull;
  if (lane == 0) {
    sh.fred[wv] = m;
    sh.ired[wv] = wbad;
  }
  __syncthreads();
  m = -INFINITY;
  bad = 0;
  for (int i = 0; i < NWV; ++i) {
    m = fmaxf(m, sh.fred[i]);
    bad |= sh.ired[i];
  }
  if (bad) {
#pragma unroll
    for (int t = 0; t < VPT; ++t) v[t] = 0.f;
    __syncthreads();
    return false;
  }
  if (kn.greedy) {
    // T = 0, argmax decoding: one-hot at the lowest index holding the maximum (the
    // maximum survives any top-k or top-p cut, so those knobs change nothing here)
    int first = INT_MAX;
#pragma unroll
    for (int t = VPT - 1; t >= 0; --t)
      if (t * VT + tid < V && v[t] == m) first = t * VT + tid;
    first = wave_min_i(first);
    __syncthreads();  // every thread has read sh.ired above
    if (lane == 0) sh.ired[wv] = first;
    __syncthreads();
    first = INT_MAX;
    for (int i = 0; i < NWV; ++i) first = min(first, sh.ired[i]);
#pragma unroll
    for (int t = 0; t < VPT; ++t) v[t] = t * VT + tid == first ? 1.f : 0.f;
    return true;
  }
  // top-k on the logit (the order of l/T is the order of l for T > 0); dropped
  // elements become -inf.  The maximum is always kept.
  if (kn.top_k > 0 && kn.top_k < V) {
    const RadixResult r = radix_select<VPT, 32>(
        v,
        [](float x, uint32_t& k) {
          k = okey(x);
          return x != -INFINITY;
        },
        [](float) { return 1ull; }, (unsigned long long)kn.top_k, sh);
    const float zero = sh.zero;
#pragma unroll
    for (int t = 0; t < VPT; ++t)
      if (okey(v[t] + zero) < r.t) v[t] = -INFINITY;
  }
  // e = exp((l - max) / T) = 2^((l - max) * log2(e) / T), once per element, with the
  // hardware base-2 exponential (about 1 ulp; the rounding of the fp32 multiplier adds
  // at most ~4e-6 relative on e values below 2^-100 and ~1e-7 near the maximum); 0 for
  // dropped and padding elements (argument -inf)
  const float itl = kn.inv_t * 1.44269504088896340736f;
  double s = 0.0;
#pragma unroll
  for (int t = 0; t < VPT; ++t) {
    v[t] = __builtin_amdgcn_exp2f((v[t] - m) * itl);
    s += (double)v[t];
    __builtin_amdgcn_sched_barrier(0);
  }
  const double S = block_sum_d(s, sh.dred);
  const double invS = 1.0 / S;
  double norm = invS;
  uint32_t tkeep = 0u;  // keep e with bits >= tkeep (e >= 0: bit order is value order)
  if (kn.top_p < 1.0f) {
    // mass of element i: round(e_i / S * 2^52), from one fma (adding 2^52 leaves the
    // rounded integer in the low mantissa bits; e_i / S <= 1 keeps it below 2^53)
    const double ws = invS * 4503599627370496.0;  // 2^52 / S
    const unsigned long long target =
        (unsigned long long)((double)kn.top_p * 4503599627370496.0);
    const RadixResult r = radix_select<VPT, 30>(
        v,
        [](float e, uint32_t& k) {
          // 0 <= e <= 1: the bit pattern is order-preserving, with bits 30 and 31 zero
          k = __float_as_uint(e);
          return e > 0.f;
        },
        [=](float e) {
          return (unsigned long long)__double_as_longlong(
                     __builtin_fma((double)e, ws, 4503599627370496.0)) -
                 0x4330000000000000ull;
        },
        target, sh);
    tkeep = r.all ? 0u : r.t;
    norm = ws / (double)r.kept;  // 1 / (kept sum of e), the kept sum from exact integers
  }
  // e + zero (zero re-read from LDS) keeps the compiler from reusing the e pass's
  // fp64 conversions, which would hold 2 * VPT registers across the top-p passes
  __syncthreads();
  const float zero = sh.zero;
#pragma unroll
  for (int t = 0; t < VPT; ++t) {
    const float e = __float_as_uint(v[t]) >= tkeep ? v[t] + zero : 0.f;
    v[t] = (float)((double)e * norm);
    __builtin_amdgcn_sched_barrier(0);
  }
  return true;
}

// Inverse CDF in token-id order over the weights in sh.w[0..V): smallest i whose
// running sum exceeds u*S, S the total.  Running sums in fp64: thread c sums the 32
// consecutive tokens of chunk c (in a rotated but fixed order, so LDS banks do not
// collide), a block scan over the 1024 chunk sums locates the chunk holding the
// crossing -- the one thread whose inclusive sum exceeds u*S while its predecessor's
// does not -- and that thread's wave walks the chunk with a 32-lane prefix sum.
// Returns -1 if S == 0.
__device__ __forceinline__ int inverse_cdf_lds(int V, double u, VocabLDS& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int CH = MAXVPT;  // tokens per chunk; chunk c = [c*CH, c*CH + CH)
  constexpr int NONE = 0x7fffffff;
  if (tid == 0) sh.bcast_i[2] = NONE;
  __syncthreads();  // sh.w complete
  double c = 0.0;
  const int c0 = tid * CH;
  if (c0 < V) {
#pragma unroll
    for (int e0 = 0; e0 < CH; e0 += 8) {  // 8 independent reads, then their additions in order
      float xs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = c0 + ((e0 + e + tid) & (CH - 1));
        xs[e] = i < V ? sh.w[i] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) c += (double)xs[e];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // inclusive block scan of the chunk sums
  double inc = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = shfl_up_d(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh.scan[wv] = inc;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < wv; ++i) off += sh.scan[i];
  inc += off;
  double S = 0.0;
  for (int i = 0; i < NWV; ++i) S += sh.scan[i];
  if (!(S > 0.0)) {
    __syncthreads();
    return -1;
  }
  const double T = u * S;
  // the predecessor's inclusive sum, as that thread holds it (the wave's offset is the
  // previous wave's last inclusive sum: the same additions in the same order)
  const double up = shfl_up_d(inc, 1);
  const double prev = lane == 0 ? off : up;
  // Exactly one owner when the running sums are monotone; should rounding in the
  // scan tree ever break that, the smallest token found wins (atomicMin), which is the
  // first owner's.
  const bool owner = inc > T && prev <= T;
  const unsigned long long ob = __ballot(owner);
  if (ob) {
    const int ol = __ffsll((long long)ob) - 1;
    const int base = (wv * 64 + ol) * CH;
    const double run = __longlong_as_double(
        ((long long)__builtin_amdgcn_readlane((int)(__double_as_longlong(prev) >> 32), ol) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)__double_as_longlong(prev), ol));
    const int i = base + lane;
    const float x = (lane < CH && i < V) ? sh.w[i] : 0.f;
    double ps = (double)x;  // inclusive prefix over lanes 0..lane
#pragma unroll
    for (int o = 1; o < CH; o <<= 1) {
      const double y = shfl_up_d(ps, o);
      if (lane >= o) ps += y;
    }
    const unsigned long long crossed = __ballot(lane < CH && run + ps > T);
    const unsigned long long pos = __ballot(x > 0.f);
    if (lane == 0) {
      int tok;
      if (crossed) tok = base + __ffsll((long long)crossed) - 1;
      else tok = pos ? base + 63 - __clzll(pos) : -1;  // rounding: last positive of the chunk
      if (tok >= 0) atomicMin(&sh.bcast_i[2], tok);
    }
  }
  __syncthreads();
  if (sh.bcast_i[2] == NONE && tid == 0) {
    // rounding put u*S at or past the end: the last token with positive weight
    int last_pos = -1;
    for (int i = V - 1; i >= 0; --i)
      if (sh.w[i] > 0.f) { last_pos = i; break; }
    sh.bcast_i[2] = last_pos;
  }
  __syncthreads();
  const int r = sh.bcast_i[2];
  __syncthreads();
  return r;
}

template <int VPT>
__device__ __forceinline__ void store_w(const float (&v)[VPT], int V, VocabLDS& sh) {
  __syncthreads();  // previous readers of sh.w are done
#pragma unroll
  for (int t = 0; t < VPT; ++t) {
    const int i = t * VT + threadIdx.x;
    if (i < V) sh.w[i] = v[t];
  }
}

template <int VPT>
__device__ __forceinline__ void load_row(float (&v)[VPT], const float* row, int V) {
#pragma unroll
  for (int t = 0; t < VPT; ++t) {
    const int i = t * VT + threadIdx.x;
    v[t] = i < V ? __builtin_nontemporal_load(row + i) : -INFINITY;
  }
}

// One workgroup per (b, j), j = 0..K.  Writes res_acc[b*K + j] (j < K), res_cand[b*(K+1)+j]
// and res_status[b*(K+1)+j].  While the draft row is processed, the processed target
// row waits in the LDS weight buffer (one row in registers at a time).  Workgroups
// 0 .. B*K-1 take the positions with a draft row (b = id / K, j = id % K) and the last B
// the bonus rows (j = K): with more workgroups than compute units, those that start
// late are then the bonus rows, which process one row instead of two.
template <int VPT>
__global__ __launch_bounds__(VT) void k_accept_rows(
    const float* __restrict__ p_logits, const float* __restrict__ q_logits,
    const int32_t* __restrict__ x_tilde, int K, int V, SamplingKnobs kn, uint64_t seed,
    uint64_t round, const uint64_t* __restrict__ round_dev, int32_t* __restrict__ res_acc,
    int32_t* __restrict__ res_cand, int32_t* __restrict__ res_status, float* __restrict__ dbg_p,
    float* __restrict__ dbg_q) {
  __shared__ VocabLDS sh;
  if (round_dev) round = *round_dev;
  const int nbk = (int)(gridDim.x / (K + 1)) * K, id = blockIdx.x;
  const int b = id < nbk ? id / K : id - nbk, j = id < nbk ? id % K : K, tid = threadIdx.x;
  const bool has_q = j < K;
  const float* prow = p_logits + ((size_t)b * (K + 1) + j) * V;
  int status = 0;
  int cand = -1;
  {
    float pv[VPT];
    load_row<VPT>(pv, prow, V);
    if (!process_row<VPT>(pv, V, kn, sh)) status |= SPEC_ROW_NONFINITE;
    if (dbg_p) {
      float* d = dbg_p + ((size_t)b * (K + 1) + j) * V;
#pragma unroll
      for (int t = 0; t < VPT; ++t)
        if (t * VT + tid < V) d[t * VT + tid] = pv[t];
    }
    store_w<VPT>(pv, V, sh);  // P -> sh.w (the bonus row samples from it directly)
  }
  if (!has_q) {
    if (!(status & SPEC_ROW_NONFINITE)) {
      const double u = philox_uniform(seed, round, j, b, 2);
      cand = inverse_cdf_lds(V, u, sh);
    }
  } else {
    float qv[VPT];
    load_row<VPT>(qv, q_logits + ((size_t)b * K + j) * V, V);
    if (!process_row<VPT>(qv, V, kn, sh)) status |= SPEC_ROW_NONFINITE;  // publishes sh.w
    if (dbg_q) {
      float* d = dbg_q + ((size_t)b * K + j) * V;
#pragma unroll
      for (int t = 0; t < VPT; ++t)
        if (t * VT + tid < V) d[t * VT + tid] = qv[t];
    }
    const int x = x_tilde[b * K + j];
    int accept = 0;
    if (x < 0 || x >= V) {
      status |= SPEC_ROW_BAD_TOKEN;
    } else {
#pragma unroll
      for (int t = 0; t < VPT; ++t)
        if (t * VT + tid == x) sh.qx = qv[t];
      __syncthreads();
      const float px = sh.w[x], qx = sh.qx;
      if (qx == 0.f) status |= SPEC_ROW_Q_ZERO;
      const double u = philox_uniform(seed, round, j, b, 1);
      accept = (u * (double)qx < (double)px) ? 1 : 0;
    }
    if (!(status & (SPEC_ROW_NONFINITE | SPEC_ROW_BAD_TOKEN)) && !accept) {
      // residual max(0, p - q), kept in the q registers
#pragma unroll
      for (int t = 0; t < VPT; ++t) {
        const int i = t * VT + tid;
        qv[t] = i < V ? fmaxf(sh.w[i] - qv[t], 0.f) : 0.f;
      }
      const double u = philox_uniform(seed, round, j, b, 2);
      store_w<VPT>(qv, V, sh);
      cand = inverse_cdf_lds(V, u, sh);
      if (cand < 0) {
        // empty residual (p <= q everywhere): sample P, processed again from its logits
        status |= SPEC_ROW_RESIDUAL_EMPTY;
        float pv[VPT];
        load_row<VPT>(pv, prow, V);
        process_row<VPT>(pv, V, kn, sh);
        store_w<VPT>(pv, V, sh);
        cand = inverse_cdf_lds(V, u, sh);
      }
    }
    if (tid == 0) res_acc[b * K + j] = accept;
  }
  if (tid == 0) {
    res_cand[b * (K + 1) + j] = cand;
    res_status[b * (K + 1) + j] = status;
  }
}

// One thread per row: first rejection, outputs, cache lengths, pending tokens.
__global__ void k_select(const int32_t* __restrict__ x_tilde, int B, int K,
                         const int32_t* __restrict__ res_acc, const int32_t* __restrict__ res_cand,
                         const int32_t* __restrict__ res_status, int32_t* __restrict__ out_tok,
                         int32_t* __restrict__ n_out, int32_t* __restrict__ row_status,
                         int32_t* t_len, const int32_t* t_base, int32_t* d_len,
                         const int32_t* d_base, int32_t* pending, int32_t* n_pending,
                         uint64_t* round_dev) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (round_dev && b == 0) *round_dev += 1;  // the rows of this round were decided
  if (b >= B) return;
  int fatal = 0;
  for (int j = 0; j <= K; ++j)
    fatal |= res_status[b * (K + 1) + j] & (SPEC_ROW_NONFINITE | SPEC_ROW_BAD_TOKEN);
  if (t_len && t_base && (t_len[b] - t_base[b]) != K + 1) fatal |= SPEC_ROW_KV_OVERFLOW;
  if (d_len && d_base && n_pending && (d_len[b] - d_base[b]) != n_pending[b] + K - 1)
    fatal |= SPEC_ROW_KV_OVERFLOW;
  int a = K;
  for (int j = 0; j < K; ++j)
    if (!res_acc[b * K + j]) { a = j; break; }
  int st = fatal;
  for (int j = 0; j <= a; ++j) st |= res_status[b * (K + 1) + j] & ~(SPEC_ROW_NONFINITE | SPEC_ROW_BAD_TOKEN);
  int32_t* o = out_tok + (size_t)b * (K + 1);
  if (fatal) {
    for (int j = 0; j <= K; ++j) o[j] = -1;
    n_out[b] = 0;
    row_status[b] = st;
    if (t_len && t_base) t_len[b] = t_base[b];
    if (d_len && d_base) d_len[b] = d_base[b];
    return;
  }
  const int y = res_cand[b * (K + 1) + a];
  for (int j = 0; j < a; ++j) o[j] = x_tilde[b * K + j];
  o[a] = y;
  for (int j = a + 1; j <= K; ++j) o[j] = -1;
  n_out[b] = a + 1;
  row_status[b] = st;
  int new_t = -1;
  if (t_len && t_base) {
    new_t = t_base[b] + a + 1;
    t_len[b] = new_t;
  }
  if (d_len && a < K) {
    // the draft cache holds every committed token but the newest one
    if (new_t >= 0) d_len[b] = new_t;
    else if (d_base) d_len[b] = min(d_len[b], d_base[b] + (n_pending ? n_pending[b] : 1) + a);
  }
  if (pending && n_pending) {
    if (a < K) {
      pending[2 * b] = y;
      pending[2 * b + 1] = -1;
      n_pending[b] = 1;
    } else {
      pending[2 * b] = x_tilde[b * K + K - 1];
      pending[2 * b + 1] = y;
      n_pending[b] = 2;
    }
  }
}

// Draft step sampler: one workgroup per row b.  Copies the logits of the row's last
// input position into q_logits[b, step], processes them and draws x~_step.  A row whose
// logits are not all finite gets SPEC_ROW_NONFINITE in row_status (when given) and the
// placeholder token 0, which keeps the next steps' inputs in range; the accept step
// then emits nothing for the row (its q row is non-finite too).
template <int VPT>
__global__ __launch_bounds__(VT) void k_draft_sample(
    const float* __restrict__ logits, int M, const int32_t* __restrict__ n_in, int step,
    int K, int V, SamplingKnobs kn, uint64_t seed, uint64_t round,
    const uint64_t* __restrict__ round_dev, int32_t* __restrict__ x_tilde,
    float* __restrict__ q_logits, int32_t* __restrict__ row_status) {
  __shared__ VocabLDS sh;
  if (round_dev) round = *round_dev;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int last = step == 0 ? max(0, min(n_in[b], M) - 1) : 0;
  const float* row = logits + ((size_t)b * M + last) * V;
  float* qrow = q_logits + ((size_t)b * K + step) * V;
  float v[VPT];
  load_row<VPT>(v, row, V);
#pragma unroll
  for (int t = 0; t < VPT; ++t)
    if (t * VT + tid < V) qrow[t * VT + tid] = v[t];
  int x = 0;
  if (process_row<VPT>(v, V, kn, sh)) {
    const double u = philox_uniform(seed, round, step, b, 0);
    store_w<VPT>(v, V, sh);
    x = inverse_cdf_lds(V, u, sh);
    if (x < 0) x = 0;
  } else if (tid == 0 && row_status) {
    row_status[b] |= SPEC_ROW_NONFINITE;
  }
  if (tid == 0) x_tilde[b * K + step] = x;
}

// tokens[b] = [pending[b, n_pending[b] - 1], x~_0 .. x~_{K-1}]
__global__ void k_verify_tokens(const int32_t* __restrict__ pending,
                                const int32_t* __restrict__ n_pending,
                                const int32_t* __restrict__ x_tilde, int B, int K,
                                int32_t* __restrict__ tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int np = min(max(n_pending[b], 1), 2);
  tokens[(size_t)b * (K + 1)] = pending[2 * b + np - 1];
  for (int j = 0; j < K; ++j) tokens[(size_t)b * (K + 1) + 1 + j] = x_tilde[b * K + j];
}

__global__ void k_rollback(int32_t* __restrict__ len, const int32_t* __restrict__ new_len, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) len[b] = min(len[b], max(new_len[b], 0));
}

#define VPT_DISPATCH(V, CALL)                      \
  do {                                             \
    const int vpt_ = cdiv((V), VT);                \
    if (vpt_ <= 1) { constexpr int P = 1; CALL; }  \
    else if (vpt_ <= 2) { constexpr int P = 2; CALL; } \
    else if (vpt_ <= 4) { constexpr int P = 4; CALL; } \
    else if (vpt_ <= 8) { constexpr int P = 8; CALL; } \
    else if (vpt_ <= 16) { constexpr int P = 16; CALL; } \
    else { constexpr int P = 32; CALL; }           \
  } while (0)

hipError_t launch_accept_rows(const float* p_logits, const float* q_logits,
                              const int32_t* x_tilde, int B, int K, int V, SamplingKnobs kn,
                              uint64_t seed, uint64_t round, const uint64_t* round_dev,
                              int32_t* res_acc, int32_t* res_cand, int32_t* res_status,
                              float* dbg_p, float* dbg_q, hipStream_t s) {
  VPT_DISPATCH(V, (k_accept_rows<P><<<B * (K + 1), VT, 0, s>>>(
                       p_logits, q_logits, x_tilde, K, V, kn, seed, round, round_dev, res_acc,
                       res_cand, res_status, dbg_p, dbg_q)));
  return hipGetLastError();
}

hipError_t launch_select(const int32_t* x_tilde, int B, int K, const int32_t* res_acc,
                         const int32_t* res_cand, const int32_t* res_status,
                         int32_t* out_tok, int32_t* n_out, int32_t* row_status,
                         int32_t* t_len, const int32_t* t_base, int32_t* d_len,
                         const int32_t* d_base, int32_t* pending, int32_t* n_pending,
                         uint64_t* round_dev, hipStream_t s) {
  k_select<<<cdiv(B, 64), 64, 0, s>>>(x_tilde, B, K, res_acc, res_cand, res_status, out_tok,
                                      n_out, row_status, t_len, t_base, d_len, d_base,
                                      pending, n_pending, round_dev);
  return hipGetLastError();
}

hipError_t launch_draft_sample(const float* logits, int B, int M, const int32_t* n_in,
                               int step, int K, int V, SamplingKnobs kn, uint64_t seed,
                               uint64_t round, const uint64_t* round_dev, int32_t* x_tilde,
                               float* q_logits, int32_t* row_status, hipStream_t s) {
  VPT_DISPATCH(V, (k_draft_sample<P><<<B, VT, 0, s>>>(logits, M, n_in, step, K, V, kn, seed,
                                                     round, round_dev, x_tilde, q_logits,
                                                     row_status)));
  return hipGetLastError();
}

hipError_t launch_verify_tokens(const int32_t* pending, const int32_t* n_pending,
                                const int32_t* x_tilde, int B, int K, int32_t* tokens,
                                hipStream_t s) {
  k_verify_tokens<<<cdiv(B, 64), 64, 0, s>>>(pending, n_pending, x_tilde, B, K, tokens);
  return hipGetLastError();
}

hipError_t launch_rollback(int32_t* len, const int32_t* new_len, int B, hipStream_t s) {
  k_rollback<<<cdiv(B, 64), 64, 0, s>>>(len, new_len, B);
  return hipGetLastError();
}

}  // namespace specdec
