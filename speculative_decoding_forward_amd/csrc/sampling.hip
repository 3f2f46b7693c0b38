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
// Numerics: exponentials in fp32, all sums (softmax normaliser, top-p masses, the
// residual mass and the inverse-CDF running sums) in fp64 with a fixed reduction
// order; top-k / top-p thresholds are found by radix select on an order-preserving
// key of the LOGIT (so ties are exactly the equal logits), with integer (count or
// 2^52 fixed-point mass) histograms, so the selection is deterministic.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace specdec {

constexpr int VT = 1024;   // threads per vocab workgroup
constexpr int NWV = VT / 64;
constexpr int MAXVPT = 32;  // V <= 32768

struct VocabLDS {
  double dred[NWV];
  float fred[NWV];
  int ired[NWV];
  unsigned long long hist[256];
  double scan[NWV];
  float w[MAXVPT * VT];  // inverse-CDF weights in token-id order
  double bcast_d[4];
  int bcast_i[4];
  unsigned long long bcast_ull;
  float px, qx;
  float zero;  // always 0; read inside loops so per-element work is not hoisted
};

// order-preserving key of a float (-0 folded onto +0)
__device__ __forceinline__ uint32_t okey(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest key t such that the total weight of kept elements (logit > -inf) with
// key >= t reaches `target` (4 passes of 8-bit digits, integer histograms in LDS).
// Returns 0 (keep everything) if all kept elements together do not reach it.
template <int VPT, typename WeightF>
__device__ __forceinline__ uint32_t radix_select(const float (&v)[VPT], WeightF wf,
                                                 unsigned long long target, VocabLDS& sh) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  unsigned long long above = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += VT) sh.hist[i] = 0ull;
    __syncthreads();
    // keys and weights are recomputed every pass (x = v + 0 read from LDS) rather
    // than kept live across passes, which would not fit the register budget
    const float zero = sh.zero;
#pragma unroll
    for (int t = 0; t < VPT; ++t) {
      const float x = v[t] + zero;
      if (x == -INFINITY) continue;
      const uint32_t k = okey(x);
      const bool match = pass == 0 ? true : ((k >> (shift + 8)) == (prefix >> (shift + 8)));
      if (match) atomicAdd(&sh.hist[(k >> shift) & 255u], wf(x));
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4l..4l+3; suffix sums from the top bin down
      const unsigned long long b0 = sh.hist[4 * tid], b1 = sh.hist[4 * tid + 1],
                               b2 = sh.hist[4 * tid + 2], b3 = sh.hist[4 * tid + 3];
      const unsigned long long mine = b0 + b1 + b2 + b3;
      // inclusive suffix scan over lanes (lane l gets the sum over lanes >= l)
      unsigned long long suf = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_down(suf, o, 64);
        if (tid + o < 64) suf += y;
      }
      const unsigned long long after = suf - mine;  // lanes > l
      // largest digit d with above + sum_{bins >= d} >= target
      int d = -1;
      const unsigned long long s3 = above + after + b3, s2 = s3 + b2, s1 = s2 + b1,
                               s0 = s1 + b0;
      if (s3 >= target) d = 4 * tid + 3;
      else if (s2 >= target) d = 4 * tid + 2;
      else if (s1 >= target) d = 4 * tid + 1;
      else if (s0 >= target) d = 4 * tid;
      // the largest lane with a hit holds the answer
      const unsigned long long hit = __ballot(d >= 0);
      const int hl = hit ? (63 - (int)__clzll(hit)) : -1;
      if (tid == 0) sh.bcast_i[0] = hl;
      if (hl >= 0 && tid == hl) {
        // weight above the chosen digit = above + (sum of bins > d)
        unsigned long long ab = above + after;
        if (d < 4 * tid + 3) ab += b3;
        if (d < 4 * tid + 2) ab += b2;
        if (d < 4 * tid + 1) ab += b1;
        sh.bcast_i[1] = d;
        sh.bcast_ull = ab;
      }
    }
    __syncthreads();
    if (sh.bcast_i[0] < 0) {
      __syncthreads();
      return 0u;  // nothing reaches the target: keep all
    }
    const int d = sh.bcast_i[1];
    above = sh.bcast_ull;
    prefix |= ((uint32_t)d) << shift;
    __syncthreads();
  }
  return prefix;
}

// In place: v holds a logit row on entry (-inf past the row's end) and the processed
// probability row on exit (0 outside the kept set).  Returns false (row zeroed) if a
// logit of the row is not finite.
template <int VPT>
__device__ __forceinline__ bool process_row(float (&v)[VPT], int V, const SamplingKnobs& kn,
                                            VocabLDS& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.zero = 0.f;  // published by the barrier inside block_or
  int bad = 0;
#pragma unroll
  for (int t = 0; t < VPT; ++t)
    if (t * VT + tid < V && !isfinite(v[t])) bad = 1;
  bad = block_or(bad, sh.ired);
  if (bad) {
#pragma unroll
    for (int t = 0; t < VPT; ++t) v[t] = 0.f;
    return false;
  }
  // top-k on the logit (the order of l/T is the order of l for T > 0); dropped
  // elements become -inf
  if (kn.top_k > 0 && kn.top_k < V) {
    const uint32_t tk = radix_select<VPT>(v, [](float) { return 1ull; },
                                          (unsigned long long)kn.top_k, sh);
    const float zero = sh.zero;
#pragma unroll
    for (int t = 0; t < VPT; ++t)
      if (okey(v[t] + zero) < tk) v[t] = -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < VPT; ++t) m = fmaxf(m, v[t]);
  m = block_max(m, sh.fred);
  const float it = kn.inv_t;
  double s = 0.0;
  {
    const float zero = sh.zero;
#pragma unroll
    for (int t = 0; t < VPT; ++t) {
      s += (double)expf((v[t] + zero - m) * it);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const double S = block_sum(s, sh.dred);
  const double invS = 1.0 / S;
  double S2 = 1.0;
  if (kn.top_p < 1.0f) {
    const double scale = 4503599627370496.0;  // 2^52
    const unsigned long long target = (unsigned long long)((double)kn.top_p * scale);
    const uint32_t tp = radix_select<VPT>(
        v,
        [=](float x) {
          const double p1 = (double)expf((x - m) * it) * invS;
          return (unsigned long long)(p1 * scale + 0.5);
        },
        target, sh);
    double s2 = 0.0;
    const float zero = sh.zero;
#pragma unroll
    for (int t = 0; t < VPT; ++t) {
      if (okey(v[t] + zero) < tp) v[t] = -INFINITY;
      s2 += (double)expf((v[t] - m) * it) * invS;
      __builtin_amdgcn_sched_barrier(0);
    }
    S2 = block_sum(s2, sh.dred);
  }
  const double norm = invS / S2;
  __syncthreads();
  const float zero = sh.zero;
#pragma unroll
  for (int t = 0; t < VPT; ++t) {
    v[t] = (float)((double)expf((v[t] + zero - m) * it) * norm);
    __builtin_amdgcn_sched_barrier(0);
  }
  return true;
}

// Inverse CDF in token-id order over the weights in sh.w[0..V): smallest i whose
// running sum exceeds u*S, S the total.  Running sums in fp64: thread c sums the 32
// consecutive tokens of chunk c (in a rotated but fixed order, so LDS banks do not
// collide), a block scan over the 1024 chunk sums locates the chunk holding the
// crossing, and one thread walks that chunk in token order.  Returns -1 if S == 0.
__device__ __forceinline__ int inverse_cdf_lds(int V, double u, VocabLDS& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int CH = MAXVPT;  // tokens per chunk; chunk c = [c*CH, c*CH + CH)
  __syncthreads();            // sh.w complete
  double c = 0.0;
  const int c0 = tid * CH;
  if (c0 < V) {
    for (int e = 0; e < CH; ++e) {
      const int i = c0 + ((e + tid) & (CH - 1));
      if (i < V) c += (double)sh.w[i];
    }
  }
  // inclusive block scan of the chunk sums
  double inc = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o, 64);
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
  const int hit = block_min_int(inc > T ? tid : 0x7fffffff, sh.ired);
  // the owner of the crossing chunk walks it (its exclusive prefix is inc - c)
  if (hit != 0x7fffffff && tid == hit) {
    double run = inc - c;
    int tok = -1, last_pos = -1;
    for (int e = 0; e < CH; ++e) {
      const int i = c0 + e;
      if (i >= V) break;
      const float x = sh.w[i];
      if (x > 0.f) last_pos = i;
      run += (double)x;
      if (run > T) { tok = i; break; }
    }
    sh.bcast_i[2] = tok >= 0 ? tok : last_pos;
  }
  if (hit == 0x7fffffff && tid == 0) {
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
// and res_status[b*(K+1)+j].
template <int VPT>
__global__ __launch_bounds__(VT) void k_accept_rows(
    const float* __restrict__ p_logits, const float* __restrict__ q_logits,
    const int32_t* __restrict__ x_tilde, int K, int V, SamplingKnobs kn, uint64_t seed,
    uint64_t round, const uint64_t* __restrict__ round_dev, int32_t* __restrict__ res_acc,
    int32_t* __restrict__ res_cand, int32_t* __restrict__ res_status, float* __restrict__ dbg_p,
    float* __restrict__ dbg_q) {
  __shared__ VocabLDS sh;
  if (round_dev) round = *round_dev;
  const int b = blockIdx.x / (K + 1), j = blockIdx.x % (K + 1), tid = threadIdx.x;
  const bool has_q = j < K;
  float pv[VPT], qv[VPT];
  load_row<VPT>(pv, p_logits + ((size_t)b * (K + 1) + j) * V, V);
  int status = 0;
  if (!process_row<VPT>(pv, V, kn, sh)) status |= SPEC_ROW_NONFINITE;
  if (dbg_p) {
    float* d = dbg_p + ((size_t)b * (K + 1) + j) * V;
#pragma unroll
    for (int t = 0; t < VPT; ++t)
      if (t * VT + tid < V) d[t * VT + tid] = pv[t];
  }
  int cand = -1;
  if (has_q) {
    load_row<VPT>(qv, q_logits + ((size_t)b * K + j) * V, V);
    if (!process_row<VPT>(qv, V, kn, sh)) status |= SPEC_ROW_NONFINITE;
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
        if (t * VT + tid == x) { sh.px = pv[t]; sh.qx = qv[t]; }
      __syncthreads();
      const float px = sh.px, qx = sh.qx;
      if (qx == 0.f) status |= SPEC_ROW_Q_ZERO;
      const double u = philox_uniform(seed, round, j, b, 1);
      accept = (u * (double)qx < (double)px) ? 1 : 0;
    }
    if (!(status & (SPEC_ROW_NONFINITE | SPEC_ROW_BAD_TOKEN)) && !accept) {
      // residual max(0, p - q), kept in the q registers
#pragma unroll
      for (int t = 0; t < VPT; ++t) qv[t] = fmaxf(pv[t] - qv[t], 0.f);
      const double u = philox_uniform(seed, round, j, b, 2);
      store_w<VPT>(qv, V, sh);
      cand = inverse_cdf_lds(V, u, sh);
      if (cand < 0) {
        status |= SPEC_ROW_RESIDUAL_EMPTY;
        store_w<VPT>(pv, V, sh);
        cand = inverse_cdf_lds(V, u, sh);
      }
    }
    if (tid == 0) res_acc[b * K + j] = accept;
  } else if (!(status & SPEC_ROW_NONFINITE)) {
    const double u = philox_uniform(seed, round, j, b, 2);
    store_w<VPT>(pv, V, sh);
    cand = inverse_cdf_lds(V, u, sh);
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
// input position into q_logits[b, step], processes them and draws x~_step.
template <int VPT>
__global__ __launch_bounds__(VT) void k_draft_sample(
    const float* __restrict__ logits, int M, const int32_t* __restrict__ n_in, int step,
    int K, int V, SamplingKnobs kn, uint64_t seed, uint64_t round,
    const uint64_t* __restrict__ round_dev, int32_t* __restrict__ x_tilde,
    float* __restrict__ q_logits) {
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
  }
  if (tid == 0) x_tilde[b * K + step] = x;
}

// Builds the token matrix [B, 2] / counts for a draft step.
__global__ void k_draft_tokens(const int32_t* __restrict__ in_tok, const int32_t* __restrict__ n_in,
                               const int32_t* __restrict__ x_tilde, int B, int K, int step,
                               int32_t* __restrict__ tokens, int32_t* __restrict__ n_tok) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  if (step == 0) {
    const int n = min(max(n_in[b], 0), 2);
    tokens[2 * b] = in_tok[2 * b];
    tokens[2 * b + 1] = n > 1 ? in_tok[2 * b + 1] : 0;
    n_tok[b] = n;
  } else {
    tokens[b] = x_tilde[b * K + step - 1];
    n_tok[b] = 1;
  }
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
                               float* q_logits, hipStream_t s) {
  VPT_DISPATCH(V, (k_draft_sample<P><<<B, VT, 0, s>>>(logits, M, n_in, step, K, V, kn, seed,
                                                     round, round_dev, x_tilde, q_logits)));
  return hipGetLastError();
}

hipError_t launch_draft_tokens(const int32_t* in_tok, const int32_t* n_in,
                               const int32_t* x_tilde, int B, int K, int step,
                               int32_t* tokens, int32_t* n_tok, hipStream_t s) {
  k_draft_tokens<<<cdiv(B, 64), 64, 0, s>>>(in_tok, n_in, x_tilde, B, K, step, tokens, n_tok);
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
