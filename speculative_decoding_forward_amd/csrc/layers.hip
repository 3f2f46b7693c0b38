// Per-layer pieces of the verify pass other than the weight GEMMs: row bookkeeping,
// embedding gather, RMSNorm (+ cast to the activation type), RoPE + KV append, the
// FFN activation, and attention of the new rows over the KV cache.
//
// The verify pass scores the context plus the K drafts, K+1 positions in one call
// ([ZSM] "The algorithm"; [LENS] §2.1 step 2); keys and values of the new positions
// are appended to the cache and all weights and cache entries are read once per call
// ([LENS] §3.4).  The layer definition (pre-norm, RMSNorm, RoPE with half-split
// pairs, causal MHA, GELU or SwiGLU FFN) is the library's own spec: the pages only
// say "transformer".
#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace specdec {

// ------------------------------------------------------------------ bookkeeping ----

// One thread per row b: effective token count (0 on cache overflow), start position,
// validated token ids, and the length update.
__global__ void k_prep(const int32_t* __restrict__ tokens, const int32_t* __restrict__ n_tok,
                       int B, int M, int V, int32_t* __restrict__ len,
                       int32_t* __restrict__ base, int record_base, int max_len,
                       int32_t* __restrict__ pos0, int32_t* __restrict__ ntok_eff,
                       int32_t* __restrict__ tok_eff, int32_t* __restrict__ row_status,
                       unsigned* __restrict__ counters, int n_counters) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  // completion counters of the fused kernels start each forward at zero
  for (int i = b; i < n_counters; i += gridDim.x * blockDim.x) counters[i] = 0u;
  if (b >= B) return;
  int n = n_tok ? n_tok[b] : M;
  n = min(max(n, 0), M);
  const int L = len[b];
  int flags = 0;
  if (L < 0 || L + n > max_len) {
    flags |= SPEC_ROW_KV_OVERFLOW;
    n = 0;
  }
  for (int j = 0; j < M; ++j) {
    int t = 0;
    if (j < n) {
      t = tokens[(size_t)b * M + j];
      if (t < 0 || t >= V) {
        flags |= SPEC_ROW_BAD_TOKEN;
        t = 0;
      }
    }
    tok_eff[(size_t)b * M + j] = t;
  }
  pos0[b] = max(L, 0);
  ntok_eff[b] = n;
  if (record_base) base[b] = L;
  len[b] = L + n;
  if (row_status && flags) row_status[b] |= flags;
}

// x[r, :] = E[tok_eff[r], :] as fp32.  One block per row.
template <typename T>
__global__ void k_embed(const T* __restrict__ E, const int32_t* __restrict__ tok, int d,
                        float* __restrict__ x) {
  const int r = blockIdx.x;
  const T* e = E + (size_t)tok[r] * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) x[(size_t)r * d + i] = Act<T>::load(e + i);
}

// bf16 models: x[r, :] = E[tok[r], :] (fp32) and h = bf16(RMSNorm(x) * g) of the first
// layer in one pass; also the row's RoPE rotation table rope_cs[r][i] = (cos, sin) of
// pos * theta^(-2i/hd), i < hd/2, in fp64, which every layer's QKV epilogue reads (the
// position of row r = b*M + j is pos0[b] + j).  One block (256 threads) per row.
__global__ __launch_bounds__(256) void k_embed_norm(const u16* __restrict__ E,
                                                    const int32_t* __restrict__ tok, int d,
                                                    const float* __restrict__ g, float eps,
                                                    float* __restrict__ x, u16* __restrict__ h,
                                                    const int32_t* __restrict__ pos0, int M,
                                                    int hd, float theta,
                                                    double* __restrict__ rope_cs) {
  __shared__ double red[4];
  const int r = blockIdx.x;
  const u16* e = E + (size_t)tok[r] * d;
  const int half = hd >> 1;
  if (threadIdx.x < half) {
    const int i = threadIdx.x;
    const double pos = (double)(pos0[r / M] + r % M);
    const double inv_freq = pow((double)theta, -2.0 * (double)i / (double)hd);
    double sn, cs;
    sincos(pos * inv_freq, &sn, &cs);
    rope_cs[((size_t)r * half + i) * 2] = cs;
    rope_cs[((size_t)r * half + i) * 2 + 1] = sn;
  }
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) {
    const float v = bf16_to_f32(e[i]);
    x[(size_t)r * d + i] = v;
    s += (double)v * v;
  }
  s = block_sum(s, red);
  const double inv = 1.0 / sqrt(s / d + (double)eps);
  for (int i = threadIdx.x; i < d; i += 256)
    h[(size_t)r * d + i] = f32_to_bf16((float)((double)bf16_to_f32(e[i]) * inv * (double)g[i]));
}

// h = act(x / sqrt(mean(x^2) + eps) * g).  One block (256 threads) per row; the
// sum of squares and the scaling are done in fp64.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x,
                                                 const float* __restrict__ g, int d, float eps,
                                                 T* __restrict__ h) {
  __shared__ double red[4];
  const int r = blockIdx.x;
  const float* xr = x + (size_t)r * d;
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) {
    const double v = xr[i];
    s += v * v;
  }
  s = block_sum(s, red);
  const double inv = 1.0 / sqrt(s / d + (double)eps);
  for (int i = threadIdx.x; i < d; i += 256)
    h[(size_t)r * d + i] = Act<T>::cvt((float)((double)xr[i] * inv * (double)g[i]));
}

// RoPE on q and k of the new rows (half-split pairs (i, i + hd/2), angle =
// pos * theta^(-2i/hd), evaluated in fp64), q written to q_out in the activation type,
// k and v appended to the cache at position pos0[b] + j.  Grid (R, H), hd/2 threads.
template <typename T>
__global__ void k_rope_append(const float* __restrict__ qkv, int M, int H, int hd, float theta,
                              const int32_t* __restrict__ pos0, const int32_t* __restrict__ ntok_eff,
                              T* __restrict__ q_out, T* __restrict__ kc, T* __restrict__ vc,
                              size_t row_stride, size_t head_stride, int max_len) {
  const int r = blockIdx.x, h = blockIdx.y, i = threadIdx.x, half = hd >> 1;
  if (i >= half) return;
  const int b = r / M, j = r % M;
  const int d = H * hd;
  const float* row = qkv + (size_t)r * 3 * d;
  const int pos = pos0[b] + j;
  const double inv_freq = pow((double)theta, -2.0 * (double)i / (double)hd);
  const double ang = (double)pos * inv_freq;
  double sn, cs;
  sincos(ang, &sn, &cs);
  const int c0 = h * hd + i, c1 = h * hd + i + half;
  const double q0 = row[c0], q1 = row[c1];
  T* qo = q_out + (size_t)r * d;
  qo[c0] = Act<T>::cvt((float)(q0 * cs - q1 * sn));
  qo[c1] = Act<T>::cvt((float)(q1 * cs + q0 * sn));
  if (j < ntok_eff[b] && pos < max_len) {
    const double k0 = row[d + c0], k1 = row[d + c1];
    T* kp = kc + (size_t)b * row_stride + (size_t)h * head_stride + (size_t)pos * hd;
    T* vp = vc + (size_t)b * row_stride + (size_t)h * head_stride + (size_t)pos * hd;
    kp[i] = Act<T>::cvt((float)(k0 * cs - k1 * sn));
    kp[i + half] = Act<T>::cvt((float)(k1 * cs + k0 * sn));
    vp[i] = Act<T>::cvt(row[2 * d + c0]);
    vp[i + half] = Act<T>::cvt(row[2 * d + c1]);
  }
}

// FFN activation.  SwiGLU: a = silu(y[:, :F]) * y[:, F:], y [R, 2F];
// GELU (erf form): a = gelu(y), y [R, F].
template <typename T>
__global__ void k_act(const float* __restrict__ y, int R, int F, int swiglu, T* __restrict__ a) {
  const size_t n = (size_t)R * F;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t r = idx / F, c = idx % F;
    float v;
    if (swiglu) {
      const float gt = y[r * 2 * F + c], up = y[r * 2 * F + F + c];
      v = gt / (1.f + expf(-gt)) * up;
    } else {
      const float t = y[idx];
      v = 0.5f * t * (1.f + erff(t * 0.70710678118654752f));
    }
    a[idx] = Act<T>::cvt(v);
  }
}

// ------------------------------------------------------------------ attention ------
//
// bf16 path, head_dim 128 (or 64).  Split-KV: a workgroup of 4 waves owns 256
// consecutive cache positions of one (row b, head h) and one group of up to 8 queries
// (more groups only in prefill chunks); each wave owns 64 positions.  Per wave: S^T = K q^T on the
// matrix cores (v_mfma_f32_16x16x32_bf16, the K tile as the A operand, so each load
// reads 64 contiguous bytes of 16 key rows), an exact softmax over the wave's 64 keys,
// O = P V on the vector units (lanes = 4 key groups x 16 column groups).  The 4 wave
// partials are merged in LDS; the workgroup partial goes to global memory and the last
// workgroup of the (b, h) pair to finish merges all of them and writes the bf16
// output.  A query at cache position p sees positions t <= p.

constexpr int AW = 4;             // waves per workgroup
constexpr int ACH = 64;           // keys per wave
constexpr int ASPLIT = AW * ACH;  // keys per workgroup
constexpr int AQG = 8;            // queries per group

template <int HD>
__global__ __launch_bounds__(AW * 64) void k_attn_bf16(
    const u16* __restrict__ q, int M, int H, const u16* __restrict__ kc,
    const u16* __restrict__ vc, size_t row_stride, size_t head_stride,
    const int32_t* __restrict__ pos0, const int32_t* __restrict__ ntok_eff,
    float* __restrict__ part, unsigned* __restrict__ counters, int nsplit,
    u16* __restrict__ out) {
  constexpr int NS = HD / 32;  // MFMAs per 16-key tile
  constexpr int DL = HD / 16;  // dims per lane in O = P V
  __shared__ float P[AW][AQG][ACH + 1];
  __shared__ float wm[AW][AQG], wl[AW][AQG];
  __shared__ float wo[AW][AQG][HD];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int NG = cdiv(M, AQG);  // query groups per row
  const int b = blockIdx.z / NG, qg = blockIdx.z % NG;
  const int h = blockIdx.y, split = blockIdx.x;
  const int nq = ntok_eff[b];
  const int p0 = pos0[b];
  const int len_end = p0 + nq;
  const int n_active = cdiv(len_end, ASPLIT);
  const int d = H * HD;
  const int cidx = (b * H + h) * NG + qg;  // completion counter of this (b, h, group)
  if (qg * AQG >= nq) {
    // no query of this row in this group: the first split writes the padding rows
    if (split == 0)
      for (int jj = qg * AQG + threadIdx.x / HD; jj < min(M, qg * AQG + AQG);
           jj += (AW * 64) / HD)
        out[((size_t)b * M + jj) * d + h * HD + threadIdx.x % HD] = 0;
    return;
  }
  if (split >= n_active) return;  // uniform over the workgroup
  const u16* kh = kc + (size_t)b * row_stride + (size_t)h * head_stride;
  const u16* vh = vc + (size_t)b * row_stride + (size_t)h * head_stride;
  const int nl = lane & 15, gq = lane >> 4;
  const int t0 = split * ASPLIT + wv * ACH;
  const float scale = 1.0f / sqrtf((float)HD);

  // Loads are unconditional: a position past the row's end reads the last valid
  // position instead (in bounds, finite) and is removed by the causal mask (its score
  // is -inf, its probability 0), so no load sits behind a branch.
  // K fragments: tile kt, MFMA s: key t0 + 16kt + nl, dims 32s + 8gq .. +8
  bf16x8 kf[4][NS];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int t = min(t0 + kt * 16 + nl, len_end - 1);
    const u16* kr = kh + (size_t)t * HD + 8 * gq;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kf[kt][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kr + 32 * s));
  }
  // q fragment (B operand): column nl = query qg*8 + nl; columns without a query read
  // row 0 (finite) and are masked
  const int jq = qg * AQG + nl;
  const bool qok = nl < AQG && jq < nq;
  const u16* qrow = q + (size_t)(b * M + (qok ? jq : 0)) * d + h * HD + 8 * gq;
  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 32 * s));
  // V fragments, issued right behind K and q: key t0 + 4i + gq, dims DL*nl .. +DL
  typedef uint32_t vfrag[DL / 2];
  vfrag vf[ACH / 4];
#pragma unroll
  for (int i = 0; i < ACH / 4; ++i) {
    const int t = min(t0 + 4 * i + gq, len_end - 1);
    const u16* vr = vh + (size_t)t * HD + DL * nl;
    if constexpr (DL == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(vr);
      vf[i][0] = u.x; vf[i][1] = u.y; vf[i][2] = u.z; vf[i][3] = u.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(vr);
      vf[i][0] = u.x; vf[i][1] = u.y;
    }
  }
  // lane holds S^T[key 16kt + 4gq + e][query nl]
  float sc[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][s], qf[s], acc, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tk = t0 + kt * 16 + 4 * gq + e;
      sc[kt][e] = (qok && tk <= p0 + jq) ? acc[e] * scale : -INFINITY;
    }
  }
  // exact softmax over this wave's 64 positions for query nl (lanes nl + 16k)
  float m = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, sc[kt][e]);
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  float l = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = (m == -INFINITY) ? 0.f : expf(sc[kt][e] - m);
      l += p;
      if (nl < AQG) P[wv][nl][kt * 16 + 4 * gq + e] = p;
    }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  wave_lds_sync();
  // O = P V: lane (key group gq, column group nl) over keys 4i + gq
  float o[AQG][DL];
#pragma unroll
  for (int jj = 0; jj < AQG; ++jj)
#pragma unroll
    for (int e = 0; e < DL; ++e) o[jj][e] = 0.f;
#pragma unroll
  for (int i = 0; i < ACH / 4; ++i) {
    const int kk = 4 * i + gq;
    float vv[DL];
#pragma unroll
    for (int e = 0; e < DL / 2; ++e) {
      vv[2 * e] = __uint_as_float(vf[i][e] << 16);
      vv[2 * e + 1] = __uint_as_float(vf[i][e] & 0xffff0000u);
    }
#pragma unroll
    for (int jj = 0; jj < AQG; ++jj) {
      const float p = P[wv][jj][kk];
#pragma unroll
      for (int e = 0; e < DL; ++e) o[jj][e] = fmaf(p, vv[e], o[jj][e]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < AQG; ++jj)
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      float v = o[jj][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      o[jj][e] = v;
    }
  // wave partial -> LDS, then the 4 waves are merged: thread -> (query jj, dims)
  if (gq == 0) {
#pragma unroll
    for (int jj = 0; jj < AQG; ++jj)
#pragma unroll
      for (int e = 0; e < DL; ++e) wo[wv][jj][DL * nl + e] = o[jj][e];
  }
  if (lane < AQG) {
    wm[wv][lane] = m;
    wl[wv][lane] = l;
  }
  __syncthreads();
  constexpr int TPQ = AW * 64 / AQG;  // threads per query (32)
  {
    const int jj = threadIdx.x / TPQ, tt = threadIdx.x % TPQ;
    const int j = qg * AQG + jj;
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
    if (j < nq) {
      // device-coherent stores: read by the last workgroup, maybe on another XCD
      float* dst = part + ((((size_t)b * H + h) * nsplit + split) * M + j) * (HD + 2);
      for (int dd = tt; dd < HD; dd += TPQ) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < AW; ++w) v += f[w] * wo[w][jj][dd];
        coherent_store(dst + dd, v);
      }
      if (tt == 0) {
        coherent_store(dst + HD, mx);
        coherent_store(dst + HD + 1, lsum);
      }
    }
  }
  // the last workgroup of (b, h, group) merges every split (partials were written
  // with device-coherent stores; wait for them before counting this workgroup in)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last_flag = atomicAdd(&counters[cidx], 1u) == (unsigned)(n_active - 1);
  __syncthreads();
  if (!last_flag) return;
  const size_t cstride = (size_t)M * (HD + 2);
  const int jend = min(M, qg * AQG + AQG);
  for (int jj = qg * AQG + threadIdx.x / HD; jj < jend; jj += (AW * 64) / HD) {
    const int dd = threadIdx.x % HD;
    u16 res = 0;  // padding rows of this group are written as zeros
    if (jj < nq) {
      const float* base = part + (((size_t)b * H + h) * nsplit) * cstride + (size_t)jj * (HD + 2);
      // online merge over the splits, 8 at a time; the 8 splits' values are loaded
      // together (clamped indices, no branches) before any of them is used
      float mx = -INFINITY, num = 0.f, den = 0.f;
      for (int cb = 0; cb < n_active; cb += 8) {
        float mc[8], lc[8], oc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float* pc = base + (size_t)min(cb + u, n_active - 1) * cstride;
          mc[u] = coherent_load(pc + HD);
          lc[u] = coherent_load(pc + HD + 1);
          oc[u] = coherent_load(pc + dd);
        }
        float nm = mx;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (cb + u < n_active) nm = fmaxf(nm, mc[u]);
        if (nm == -INFINITY) continue;
        const float sc0 = mx == -INFINITY ? 0.f : expf(mx - nm);
        num *= sc0;
        den *= sc0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (cb + u < n_active && mc[u] != -INFINITY) {
            const float w = expf(mc[u] - nm);
            den += w * lc[u];
            num += w * oc[u];
          }
        }
        mx = nm;
      }
      res = f32_to_bf16(num / den);
    }
    out[((size_t)b * M + jj) * d + h * HD + dd] = res;
  }
  if (threadIdx.x == 0) counters[cidx] = 0u;
}

// fp32 path (small fp32 models): one 64-thread block per (query j, head h, row b);
// scores of all visible positions in dynamic LDS, exact softmax, then P V.
__global__ void k_attn_f32(const float* __restrict__ q, int M, int H, int HD,
                           const float* __restrict__ kc, const float* __restrict__ vc,
                           size_t row_stride, size_t head_stride,
                           const int32_t* __restrict__ pos0, const int32_t* __restrict__ ntok_eff,
                           float* __restrict__ out) {
  extern __shared__ float sc[];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int d = H * HD;
  const size_t r = (size_t)b * M + j;
  if (j >= ntok_eff[b]) {
    for (int dd = lane; dd < HD; dd += 64) out[r * d + h * HD + dd] = 0.f;
    return;
  }
  const int P = pos0[b] + j + 1;  // visible positions 0..pos
  const float* qr = q + r * d + h * HD;
  const float* kh = kc + (size_t)b * row_stride + (size_t)h * head_stride;
  const float* vh = vc + (size_t)b * row_stride + (size_t)h * head_stride;
  const float scale = 1.0f / sqrtf((float)HD);
  for (int t = lane; t < P; t += 64) {
    float s = 0.f;
    for (int dd = 0; dd < HD; ++dd) s = fmaf(qr[dd], kh[(size_t)t * HD + dd], s);
    sc[t] = s * scale;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int t = lane; t < P; t += 64) m = fmaxf(m, sc[t]);
  m = wave_max(m);
  float l = 0.f;
  for (int t = lane; t < P; t += 64) {
    const float p = expf(sc[t] - m);
    sc[t] = p;
    l += p;
  }
  l = wave_sum(l);
  __syncthreads();
  for (int dd = lane; dd < HD; dd += 64) {
    float o = 0.f;
    for (int t = 0; t < P; ++t) o = fmaf(sc[t], vh[(size_t)t * HD + dd], o);
    out[r * d + h * HD + dd] = o / l;
  }
}

// ------------------------------------------------------------------ launchers -----

hipError_t launch_prep(const int32_t* tokens, const int32_t* n_tok, int B, int M, int V,
                       int32_t* len, int32_t* base, int record_base, int max_len,
                       int32_t* pos0, int32_t* ntok_eff, int32_t* tok_eff,
                       int32_t* row_status, unsigned* counters, int n_counters,
                       hipStream_t s) {
  const int threads = std::max(B, n_counters);
  k_prep<<<cdiv(threads, 256), 256, 0, s>>>(tokens, n_tok, B, M, V, len, base, record_base,
                                            max_len, pos0, ntok_eff, tok_eff, row_status,
                                            counters, n_counters);
  return hipGetLastError();
}

hipError_t launch_embed(const void* embed, int dtype, const int32_t* tok_eff, int R, int d,
                        float* x, hipStream_t s) {
  if (dtype == SPEC_DT_BF16)
    k_embed<u16><<<R, 256, 0, s>>>((const u16*)embed, tok_eff, d, x);
  else
    k_embed<float><<<R, 256, 0, s>>>((const float*)embed, tok_eff, d, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, const float* g, int R, int d, float eps, int dtype,
                          void* h, hipStream_t s) {
  if (dtype == SPEC_DT_BF16)
    k_rmsnorm<u16><<<R, 256, 0, s>>>(x, g, d, eps, (u16*)h);
  else
    k_rmsnorm<float><<<R, 256, 0, s>>>(x, g, d, eps, (float*)h);
  return hipGetLastError();
}

hipError_t launch_rope_append(int dtype, const float* qkv, int B, int M, int H, int hd,
                              float theta, const int32_t* pos0, const int32_t* ntok_eff,
                              void* q_out, void* kcache, void* vcache, size_t row_stride,
                              size_t head_stride, int max_len, hipStream_t s) {
  const dim3 grid(B * M, H);
  const int threads = max(64, hd / 2);
  if (dtype == SPEC_DT_BF16)
    k_rope_append<u16><<<grid, threads, 0, s>>>(qkv, M, H, hd, theta, pos0, ntok_eff,
                                                (u16*)q_out, (u16*)kcache, (u16*)vcache,
                                                row_stride, head_stride, max_len);
  else
    k_rope_append<float><<<grid, threads, 0, s>>>(qkv, M, H, hd, theta, pos0, ntok_eff,
                                                  (float*)q_out, (float*)kcache,
                                                  (float*)vcache, row_stride, head_stride,
                                                  max_len);
  return hipGetLastError();
}

hipError_t launch_attention_f32(const float* q, const float* kcache, const float* vcache,
                                size_t row_stride, size_t head_stride, int B, int M, int H,
                                int hd, const int32_t* pos0, const int32_t* ntok_eff,
                                int max_len, float* out, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1) {
  const size_t lds = (size_t)max_len * sizeof(float);
  hipExtLaunchKernelGGL(k_attn_f32, dim3(M, H, B), dim3(64), (uint32_t)lds, s, e0, e1, 0, q, M,
                        H, hd, kcache, vcache, row_stride, head_stride, pos0, ntok_eff, out);
  return hipGetLastError();
}

hipError_t launch_attention_bf16(const u16* q, const u16* kc, const u16* vc, size_t row_stride,
                                 size_t head_stride, int B, int M, int H, int hd,
                                 const int32_t* pos0, const int32_t* ntok_eff, float* part,
                                 unsigned* counters, int max_len, u16* out, hipStream_t s,
                                 hipEvent_t e0, hipEvent_t e1) {
  const int nsplit = cdiv(max_len, ASPLIT);
  const dim3 grid(nsplit, H, B * cdiv(M, AQG));
  if (hd == 128)
    hipExtLaunchKernelGGL(k_attn_bf16<128>, grid, dim3(AW * 64), 0, s, e0, e1, 0, q, M, H, kc,
                          vc, row_stride, head_stride, pos0, ntok_eff, part, counters, nsplit,
                          out);
  else
    hipExtLaunchKernelGGL(k_attn_bf16<64>, grid, dim3(AW * 64), 0, s, e0, e1, 0, q, M, H, kc,
                          vc, row_stride, head_stride, pos0, ntok_eff, part, counters, nsplit,
                          out);
  return hipGetLastError();
}

int attn_split() { return ASPLIT; }

hipError_t launch_embed_norm(const void* embed, const int32_t* tok_eff, int R, int d,
                             const float* g, float eps, float* x, void* h,
                             const int32_t* pos0, int M, int hd, float theta, double* rope_cs,
                             hipStream_t s) {
  if (hd / 2 > 256) return hipErrorInvalidValue;
  k_embed_norm<<<R, 256, 0, s>>>((const u16*)embed, tok_eff, d, g, eps, x, (u16*)h, pos0, M, hd,
                                 theta, rope_cs);
  return hipGetLastError();
}

hipError_t launch_act(int dtype, int ffn_kind, const float* y, int R, int F, void* a,
                      hipStream_t s) {
  const size_t n = (size_t)R * F;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  if (dtype == SPEC_DT_BF16)
    k_act<u16><<<blocks, 256, 0, s>>>(y, R, F, ffn_kind == SPEC_FFN_SWIGLU, (u16*)a);
  else
    k_act<float><<<blocks, 256, 0, s>>>(y, R, F, ffn_kind == SPEC_FFN_SWIGLU, (float*)a);
  return hipGetLastError();
}

}  // namespace specdec
