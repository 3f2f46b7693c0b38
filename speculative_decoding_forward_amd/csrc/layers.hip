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
#include <math.h>

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
                       int32_t* __restrict__ tok_eff, int32_t* __restrict__ row_status) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
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
// bf16 path, head_dim 128 (or 64).  Split-KV: a wave owns 64 consecutive cache
// positions of one (row b, head h) and up to 8 queries of that row (query groups loop
// for more).  S^T = K q^T on the matrix cores (v_mfma_f32_16x16x32_bf16, the K tile
// as the A operand so each lane reads 64 contiguous bytes of a key row), an exact
// softmax over the wave's 64 keys, then O = P V on the vector units with lanes over
// (4 key groups x 16 column groups of 8), each V load instruction reading 4
// consecutive 256-byte key rows.  Partials (O, max, sum) per chunk are merged by
// k_attn_combine.  A query at position p sees cache positions t <= p.

constexpr int ACH = 64;  // keys per wave chunk
constexpr int AQG = 8;   // queries per group

template <int HD>
__global__ __launch_bounds__(256) void k_attn_bf16(
    const u16* __restrict__ q, int M, int H, const u16* __restrict__ kc,
    const u16* __restrict__ vc, size_t row_stride, size_t head_stride,
    const int32_t* __restrict__ pos0, const int32_t* __restrict__ ntok_eff,
    float* __restrict__ part, int nsplit) {
  constexpr int CW = HD / 4;     // elements per lane chunk of a key row (32 or 16)
  constexpr int NS = CW / 8;     // MFMAs per 16-key tile (4 or 2)
  constexpr int DL = HD / 16;    // dims per lane in PV (8 or 4)
  __shared__ float P[4][AQG][ACH + 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const int c = blockIdx.x * 4 + wv;
  const int nq = ntok_eff[b];
  const int p0 = pos0[b];
  const int len_end = p0 + nq;
  const int t0 = c * ACH;
  if (nq == 0 || t0 >= len_end) return;
  const int d = H * HD;
  const u16* kh = kc + (size_t)b * row_stride + (size_t)h * head_stride;
  const u16* vh = vc + (size_t)b * row_stride + (size_t)h * head_stride;
  const int nl = lane & 15, g = lane >> 4;
  const float scale = 1.0f / sqrtf((float)HD);

  for (int qg = 0; qg * AQG < nq; ++qg) {
    // q fragment (B operand): column = query qg*8 + nl (zero for nl >= 8 or past nq)
    const int jq = qg * AQG + nl;
    const bool qok = nl < AQG && jq < nq;
    const u16* qrow = q + (size_t)(b * M + (qok ? jq : 0)) * d + h * HD + g * CW;
    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (qok) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 8 * s));
      else qf[s] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    // scores: 4 tiles of 16 keys; lane holds S^T[key 16kt + 4g + e][query nl]
    float sc[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int t = t0 + kt * 16 + nl;
      const bool kok = t < len_end;
      const u16* krow = kh + (size_t)(kok ? t : 0) * HD + g * CW;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8 kf = kok ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + 8 * s))
                        : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tk = t0 + kt * 16 + 4 * g + e;
        const bool vis = qok && tk <= p0 + jq;
        sc[kt][e] = vis ? acc[e] * scale : -INFINITY;
      }
    }
    // softmax over this chunk for query nl (lanes nl, nl+16, nl+32, nl+48)
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
        if (nl < AQG) P[wv][nl][kt * 16 + 4 * g + e] = p;
      }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    wave_lds_sync();  // P[wv] is private to this wave
    // O = P V: lane (kg = g, column group nl) handles keys 4i + kg, dims DL*nl..+DL
    float o[AQG][DL];
#pragma unroll
    for (int jj = 0; jj < AQG; ++jj)
#pragma unroll
      for (int e = 0; e < DL; ++e) o[jj][e] = 0.f;
#pragma unroll 4
    for (int i = 0; i < ACH / 4; ++i) {
      const int kk = 4 * i + g;
      const int t = t0 + kk;
      if (t < len_end) {
        float vv[DL];
        const u16* vrow = vh + (size_t)t * HD + DL * nl;
        if constexpr (DL == 8) {
          const uint4 u = *reinterpret_cast<const uint4*>(vrow);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vv[2 * e] = __uint_as_float(w[e] << 16);
            vv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
          }
        } else {
          const uint2 u = *reinterpret_cast<const uint2*>(vrow);
          const uint32_t w[2] = {u.x, u.y};
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            vv[2 * e] = __uint_as_float(w[e] << 16);
            vv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
          }
        }
#pragma unroll
        for (int jj = 0; jj < AQG; ++jj) {
          const float p = P[wv][jj][kk];
#pragma unroll
          for (int e = 0; e < DL; ++e) o[jj][e] = fmaf(p, vv[e], o[jj][e]);
        }
      }
    }
    // sum the 4 key groups (lanes nl, nl+16, nl+32, nl+48)
#pragma unroll
    for (int jj = 0; jj < AQG; ++jj)
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        float v = o[jj][e];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        o[jj][e] = v;
      }
    // write partials: part[((b*H + h)*nsplit + c)*M + j][HD + 2]
    if (g == 0) {
#pragma unroll
      for (int jj = 0; jj < AQG; ++jj) {
        const int j = qg * AQG + jj;
        if (j < nq) {
          float* dst = part + ((((size_t)b * H + h) * nsplit + c) * M + j) * (HD + 2);
#pragma unroll
          for (int e = 0; e < DL; ++e) dst[DL * nl + e] = o[jj][e];
        }
      }
    }
    // m and l of query nl live on lanes nl (< 8)
    if (lane < AQG) {
      const int j = qg * AQG + lane;
      if (j < nq) {
        float* dst = part + ((((size_t)b * H + h) * nsplit + c) * M + j) * (HD + 2);
        dst[HD] = m;
        dst[HD + 1] = l;
      }
    }
    wave_lds_sync();  // P[wv] is reused by the next query group
  }
}

// Merge the chunk partials of one (b, h, query j): block of HD threads.
template <typename T>
__global__ void k_attn_combine(const float* __restrict__ part, int M, int H, int HD,
                               const int32_t* __restrict__ pos0,
                               const int32_t* __restrict__ ntok_eff, int nsplit, int chunk,
                               T* __restrict__ out) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, dd = threadIdx.x;
  const int nq = ntok_eff[b];
  const size_t r = (size_t)b * M + j;
  const int d = H * HD;
  if (j >= nq) {
    if (dd < HD) out[r * d + h * HD + dd] = Act<T>::cvt(0.f);
    return;
  }
  const int nchunks = min(nsplit, cdiv(pos0[b] + nq, chunk));
  const float* base = part + (((size_t)b * H + h) * nsplit) * M * (HD + 2) + (size_t)j * (HD + 2);
  const size_t cstride = (size_t)M * (HD + 2);
  float mx = -INFINITY;
  for (int c = 0; c < nchunks; ++c) mx = fmaxf(mx, base[c * cstride + HD]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const float* pc = base + c * cstride;
    const float mc = pc[HD];
    if (mc == -INFINITY) continue;
    const float w = expf(mc - mx);
    den += w * pc[HD + 1];
    if (dd < HD) num += w * pc[dd];
  }
  if (dd < HD) out[r * d + h * HD + dd] = Act<T>::cvt(num / den);
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
                       int32_t* row_status, hipStream_t s) {
  k_prep<<<cdiv(B, 64), 64, 0, s>>>(tokens, n_tok, B, M, V, len, base, record_base, max_len,
                                    pos0, ntok_eff, tok_eff, row_status);
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

hipError_t launch_attention(int dtype, const void* q, const void* kcache, const void* vcache,
                            size_t row_stride, size_t head_stride, int B, int M, int H, int hd,
                            const int32_t* pos0, const int32_t* ntok_eff, float* part,
                            int n_split_max, int max_len, void* out, hipStream_t s) {
  if (dtype == SPEC_DT_F32) {
    const size_t lds = (size_t)max_len * sizeof(float);
    k_attn_f32<<<dim3(M, H, B), 64, lds, s>>>((const float*)q, M, H, hd, (const float*)kcache,
                                              (const float*)vcache, row_stride, head_stride,
                                              pos0, ntok_eff, (float*)out);
    return hipGetLastError();
  }
  const int nsplit = n_split_max;  // = ceil(max_len / ACH)
  const dim3 grid(cdiv(nsplit, 4), H, B);
  if (hd == 128)
    k_attn_bf16<128><<<grid, 256, 0, s>>>((const u16*)q, M, H, (const u16*)kcache,
                                          (const u16*)vcache, row_stride, head_stride, pos0,
                                          ntok_eff, part, nsplit);
  else
    k_attn_bf16<64><<<grid, 256, 0, s>>>((const u16*)q, M, H, (const u16*)kcache,
                                         (const u16*)vcache, row_stride, head_stride, pos0,
                                         ntok_eff, part, nsplit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_attn_combine<u16><<<dim3(M, H, B), max(64, hd), 0, s>>>(part, M, H, hd, pos0, ntok_eff,
                                                            nsplit, ACH, (u16*)out);
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

int attn_chunk() { return ACH; }

}  // namespace specdec
