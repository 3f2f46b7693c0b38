// Per-layer pieces of the verify pass other than the weight GEMMs: row bookkeeping,
// embedding gather, the normalised-product input (x * g and the RMS row factor), RoPE
// + KV append, the FFN activation, and attention of the new rows over the KV cache.
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

#include "act_layout.h"
#include "common.h"
#include "internal.h"

namespace specdec {

// ------------------------------------------------------------------ bookkeeping ----

// One thread per row b: effective token count (0 on cache overflow), start position,
// validated token ids, and the length update.  A draft step (draft != 0) takes its
// tokens from the DraftSrc instead of tokens / n_tok.
__global__ void k_prep(const int32_t* __restrict__ tokens, const int32_t* __restrict__ n_tok,
                       int B, int M, int V, int32_t* __restrict__ len,
                       int32_t* __restrict__ base, int record_base, int max_len,
                       int32_t* __restrict__ pos0, int32_t* __restrict__ ntok_eff,
                       int32_t* __restrict__ tok_eff, int32_t* __restrict__ row_status,
                       unsigned* __restrict__ counters, int n_counters, DraftSrc ds,
                       int draft) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  // completion counters of the fused kernels start each forward at zero
  for (int i = b; i < n_counters; i += gridDim.x * blockDim.x) counters[i] = 0u;
  if (b >= B) return;
  int n;
  if (draft) {
    n = ds.step == 0 ? min(max(ds.n_in[b], 0), 2) : 1;
    ds.n_tok_out[b] = n;
  } else {
    n = n_tok ? n_tok[b] : M;
  }
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
      t = !draft ? tokens[(size_t)b * M + j]
                 : (ds.step == 0 ? ds.in_tok[2 * b + j] : ds.x_tilde[b * ds.K + ds.step - 1]);
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

// bf16 models: x[r, :] = E[tok[r], :] (fp32), the first layer's normalised-product input
// h = bf16(x * g) and the partial sums of x^2 over each 16-column group (summed in
// fp64, stored as fp32: ss[r][c], in column order), from which the QKV product takes its row factor
// 1 / sqrt(mean(x^2) + eps); also the row's RoPE factors for all layers.  One block (256
// threads) per row; a thread takes one 16-column group at a time (two 16-byte loads; d is
// a multiple of 128).
//
// The same kernel does the row bookkeeping of k_prep (bf16 models have no pass of their
// own for it): every block computes its sequence's token count, start position and
// overflow flag from the length, which nothing writes during the forward; block j = 0 of a
// sequence publishes them, each block its own row's token, and the length update itself
// is left to the LM head's normalise pass (k_norm_pack), after every reader of the old
// length.
__global__ __launch_bounds__(256) void k_embed_norm(
    const u16* __restrict__ E, const PrepArgs pa, int d, const float* __restrict__ g,
    float* __restrict__ x, u16* __restrict__ h, float* __restrict__ ss,
    const double* __restrict__ rope, int M, int hd, int max_len,
    double* __restrict__ rope_rows) {
  const int r = blockIdx.x, b = r / M, j = r - b * M;
  for (int i = r * 256 + threadIdx.x; i < pa.n_counters; i += gridDim.x * 256)
    pa.counters[i] = 0u;
  // the row's token is requested together with the counts and length (an in-bounds read
  // either way; it is used only for a row below the sequence's count), so the embedding
  // row waits for one round trip, not two
  const int tok_in = !pa.draft ? pa.tokens[(size_t)b * M + j]
                               : (pa.ds.step == 0 ? pa.ds.in_tok[2 * b + min(j, 1)]
                                                  : pa.ds.x_tilde[b * pa.ds.K + pa.ds.step - 1]);
  int n;
  if (pa.draft) {
    n = pa.ds.step == 0 ? min(max(pa.ds.n_in[b], 0), 2) : 1;
  } else {
    n = pa.n_tok ? pa.n_tok[b] : M;
  }
  const int n_req = n;
  n = min(max(n, 0), M);
  const int L = pa.len[b];
  int flags = 0;
  if (L < 0 || L + n > max_len) {
    flags |= SPEC_ROW_KV_OVERFLOW;
    n = 0;
  }
  const int p0 = max(L, 0);
  int tok = 0;
  if (j < n) {
    tok = tok_in;
    if (tok < 0 || tok >= pa.V) {
      flags |= SPEC_ROW_BAD_TOKEN;
      tok = 0;
    }
  }
  if (threadIdx.x == 0) {
    pa.tok_eff[r] = tok;
    if (j == 0) {
      pa.pos0[b] = p0;
      pa.ntok_eff[b] = n;
      if (pa.record_base) pa.base[b] = L;
      if (pa.draft) pa.ds.n_tok_out[b] = n_req;
    }
    if (pa.row_status && flags) atomicOr(&pa.row_status[b], flags);
  }
  {
    // the row's RoPE factors for every layer of this forward: (cos, sin) at the row's
    // absolute position, copied from the cache's table (rows past a sequence's tokens may
    // sit past max_len; their q and k are never used)
    const int half = hd >> 1;
    const int pos = min(p0 + j, max_len - 1);
    const double2* src = reinterpret_cast<const double2*>(rope) + (size_t)pos * half;
    double2* dst = reinterpret_cast<double2*>(rope_rows) + (size_t)r * half;
    for (int i = threadIdx.x; i < half; i += 256) dst[i] = src[i];
  }
  const uint4* e = reinterpret_cast<const uint4*>(E + (size_t)tok * d);
  float4* xr = reinterpret_cast<float4*>(x + (size_t)r * d);
  const float4* gr = reinterpret_cast<const float4*>(g);
  // h in the packed activation order (act_layout.h): 8 consecutive columns stay contiguous
  const int np = d / 16;
  for (int c = threadIdx.x; c < np; c += 256) {
    double sq = 0.0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c8 = 2 * c + half;  // 8-element chunk
      const uint4 u = e[c8];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      float v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
      xr[2 * c8] = float4{v[0], v[1], v[2], v[3]};
      xr[2 * c8 + 1] = float4{v[4], v[5], v[6], v[7]};
      const float4 g0 = gr[2 * c8], g1 = gr[2 * c8 + 1];
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = f32_to_bf16(v[2 * k] * gg[2 * k]) |
               ((uint32_t)f32_to_bf16(v[2 * k + 1] * gg[2 * k + 1]) << 16);
      *reinterpret_cast<uint4*>(h + act_index(r, 8 * c8, d)) = uint4{o[0], o[1], o[2], o[3]};
#pragma unroll
      for (int k = 0; k < 8; ++k) sq += (double)v[k] * v[k];
    }
    ss[(size_t)r * np + c] = (float)sq;
  }
}

// fp32 models: h = x * g and rowscale[r] = 1 / sqrt(mean(x^2) + eps), the normalised
// product's input and row factor.  One block (256 threads) per row; the sum of squares
// in fp64.
__global__ __launch_bounds__(256) void k_norm_input(const float* __restrict__ x,
                                                    const float* __restrict__ g, int d, float eps,
                                                    float* __restrict__ h,
                                                    float* __restrict__ rowscale) {
  __shared__ double red[4];
  const int r = blockIdx.x;
  const float* xr = x + (size_t)r * d;
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) {
    const double v = xr[i];
    s += v * v;
    h[(size_t)r * d + i] = xr[i] * g[i];
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) rowscale[r] = (float)(1.0 / sqrt(s / d + (double)eps));
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

// RoPE table of a bf16 cache: (cos, sin) of pos * theta^(-2i/hd) for every position pos
// < max_len and pair i < hd/2, in fp64, [max_len][hd/2][2].
__global__ void k_rope_table(double* __restrict__ tab, int max_len, int hd, double theta) {
  const int half = hd >> 1;
  const size_t n = (size_t)max_len * half;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx % half), p = (int)(idx / half);
    const double a = (double)p * pow(theta, -2.0 * (double)i / (double)hd);
    double sn, cs;
    sincos(a, &sn, &cs);
    tab[2 * idx] = cs;
    tab[2 * idx + 1] = sn;
  }
}

// ------------------------------------------------------------------ launchers -----

hipError_t launch_prep(const int32_t* tokens, const int32_t* n_tok, int B, int M, int V,
                       int32_t* len, int32_t* base, int record_base, int max_len,
                       int32_t* pos0, int32_t* ntok_eff, int32_t* tok_eff,
                       int32_t* row_status, unsigned* counters, int n_counters,
                       const DraftSrc* ds, hipStream_t s) {
  const int threads = std::max(B, n_counters);
  if (ds && (ds->step < 0 || (ds->step == 0 ? M < 2 : M < 1))) return hipErrorInvalidValue;
  k_prep<<<cdiv(threads, 256), 256, 0, s>>>(tokens, n_tok, B, M, V, len, base, record_base,
                                            max_len, pos0, ntok_eff, tok_eff, row_status,
                                            counters, n_counters, ds ? *ds : DraftSrc{},
                                            ds ? 1 : 0);
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

hipError_t launch_norm_input(const float* x, const float* g, int R, int d, float eps,
                             float* h, float* rowscale, hipStream_t s) {
  k_norm_input<<<R, 256, 0, s>>>(x, g, d, eps, h, rowscale);
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


hipError_t launch_embed_norm(const void* embed, const PrepArgs& pa, int R, int d, const float* g,
                             float* x, void* h, float* ss, const double* rope, int M, int hd,
                             int max_len, double* rope_rows, hipStream_t s) {
  if (pa.draft && (pa.ds.step < 0 || (pa.ds.step == 0 ? M < 2 : M < 1)))
    return hipErrorInvalidValue;
  k_embed_norm<<<R, 256, 0, s>>>((const u16*)embed, pa, d, g, x, (u16*)h, ss, rope, M, hd,
                                 max_len, rope_rows);
  return hipGetLastError();
}

hipError_t launch_rope_table(double* tab, int max_len, int hd, double theta, hipStream_t s) {
  const size_t n = (size_t)max_len * (hd / 2);
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  k_rope_table<<<blocks, 256, 0, s>>>(tab, max_len, hd, theta);
  return hipGetLastError();
}

// Packed bf16 activations (act_layout.h) -> natural [R][K].
__global__ void k_unpack_act(const u16* __restrict__ src, int R, int K, u16* __restrict__ dst) {
  const size_t n = (size_t)R * K;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * blockDim.x)
    dst[idx] = src[act_index((int)(idx / K), (int)(idx % K), K)];
}

hipError_t launch_trace_act(int dtype, const void* src, int R, int K, void* dst, hipStream_t s) {
  const size_t n = (size_t)R * K;
  if (dtype != SPEC_DT_BF16)
    return hipMemcpyAsync(dst, src, n * 4, hipMemcpyDeviceToDevice, s);
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 8192);
  k_unpack_act<<<blocks, 256, 0, s>>>((const u16*)src, R, K, (u16*)dst);
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
