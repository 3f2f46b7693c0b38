// C ABI of the library (declared in include/specdec.h): argument checks, workspace
// layout, and the launch sequence of the verify pass, the draft step and the rule.
// Host code only; every step of the computation runs in the kernels of gemm.hip,
// layers.hip and sampling.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "internal.h"

using namespace specdec;

namespace {

std::atomic<int> g_last_hip_error{0};

spec_status hip_fail(hipError_t e) {
  g_last_hip_error.store((int)e);
  return SPEC_E_HIP;
}

#define SPEC_LAUNCH(expr)                     \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return hip_fail(e_); \
  } while (0)

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

inline size_t elt_bytes(const spec_model_cfg& c) { return c.dtype == SPEC_DT_BF16 ? 2 : 4; }

bool cfg_valid(const spec_model_cfg* c) {
  if (!c) return false;
  if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->head_dim < 2 ||
      c->d_ffn < 1 || c->vocab < 1)
    return false;
  if (c->n_heads * c->head_dim != c->d_model) return false;
  if (c->ffn_kind != SPEC_FFN_GELU && c->ffn_kind != SPEC_FFN_SWIGLU) return false;
  if (c->dtype != SPEC_DT_F32 && c->dtype != SPEC_DT_BF16) return false;
  if (!(c->norm_eps >= 0.f) || !(c->rope_theta > 0.f)) return false;
  return true;
}

bool cfg_supported(const spec_model_cfg* c) {
  if (c->dtype == SPEC_DT_BF16) {
    // GEMM contraction dims in 128-wide super-steps, output dims in 16-column tiles
    if (c->head_dim != 64 && c->head_dim != 128) return false;
    if (c->d_model % 128 || c->d_ffn % 128 || c->vocab % 16) return false;
  } else {
    if (c->head_dim % 2 || c->head_dim > 128) return false;
  }
  return true;
}

int g_device_ok = -1;  // -1 unknown, 0 no, 1 yes
bool device_is_gfx950() {
  if (g_device_ok >= 0) return g_device_ok == 1;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    g_device_ok = 0;
    return false;
  }
  g_device_ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  return g_device_ok == 1;
}

bool knobs_valid(const spec_sampling* k) {
  if (!k) return false;
  if (!(k->temperature >= 0.f) || !std::isfinite(k->temperature)) return false;
  if (k->top_k < 0) return false;
  if (!(k->top_p > 0.f && k->top_p <= 1.f)) return false;
  return true;
}

SamplingKnobs to_knobs(const spec_sampling* k) {
  const bool greedy = k->temperature == 0.f;
  return SamplingKnobs{greedy ? 0.f : 1.0f / k->temperature, k->top_k, k->top_p, greedy ? 1 : 0};
}

// Workspace of the forward: regions carved from the caller's buffer.
struct FwdWS {
  int32_t* pos0;
  int32_t* ntok_eff;
  int32_t* tok_eff;
  int32_t* ntok2;     // draft-step counts [B]
  unsigned* counters; // completion counters: attention, residual GEMM groups, zeros
  int n_counters;
  int n_sk;           // residual GEMM group counters
  float* sk_part;     // residual GEMM slot partials
  float* x;           // residual stream [R, d] fp32
  float* xg;          // bf16: x * g_f after the last layer (act32_index order)
  void* h;            // normed activations [R, d]
  void* a;            // FFN activations [R, F]
  float* y;           // fp32 models: GEMM outputs [R, max(3d, 2F)]
  void* q;            // rotated queries [R, d]
  void* att;          // attention output [R, d]
  float* part;        // attention partials
  float* ss;          // bf16: partial sums of x^2 per row and 16-column group [R, d/16]
  float* rowscale;    // fp32 models: RMS row factor of the normalised input [R]
  double* rope_rows;  // bf16: (cos, sin) of each row's RoPE angles [R, hd/2, 2]
  float* logits;      // draft-step logits [R, V]
  size_t total;
};

FwdWS fwd_layout(const spec_model_cfg& c, int B, int M, int max_len, char* base) {
  FwdWS w{};
  const size_t R = (size_t)B * M;
  const size_t e = elt_bytes(c);
  const size_t d = c.d_model, F = c.d_ffn, V = c.vocab;
  const size_t ffn_out = c.ffn_kind == SPEC_FFN_SWIGLU ? 2 * F : F;
  // attention splits: the bound of the split count for this call shape
  const size_t nsplit = (size_t)attn_max_splits(B, c.n_heads, M, max_len);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.pos0 = (int32_t*)take(B * 4);
  w.ntok_eff = (int32_t*)take(B * 4);
  w.tok_eff = (int32_t*)take(R * 4);
  w.ntok2 = (int32_t*)take(B * 4);
  // attention completion counters (one per (row, head, query group), kAttnCounterStride
  // words apart), the residual GEMMs' group counters (one per 4 column tiles,
  // kSkCounterStride apart) and 64 zero words; prep clears all of them at the start of
  // every forward
  w.n_sk = c.dtype == SPEC_DT_BF16 ? c.d_model / 64 : 0;
  w.n_counters = B * c.n_heads * attn_groups(M) * kAttnCounterStride +
                 w.n_sk * kSkCounterStride + 64;
  w.counters = (unsigned*)take((size_t)w.n_counters * 4);
  w.x = (float*)take(R * d * 4);
  w.xg = (float*)take(c.dtype == SPEC_DT_BF16 ? (size_t)act_rows(R) * d * 4 : 0);
  // the GEMMs' bf16 inputs in the packed activation order (whole 16-row tiles)
  w.h = take((size_t)act_rows(R) * d * e);
  w.a = take((size_t)act_rows(R) * F * e);
  w.y = (float*)take(c.dtype == SPEC_DT_F32 ? R * std::max(3 * d, ffn_out) * 4 : 0);
  w.q = take(R * d * e);
  w.att = take((size_t)act_rows(R) * d * e);
  w.part = (float*)take(c.dtype == SPEC_DT_BF16
                            ? (size_t)B * c.n_heads * nsplit * M * (c.head_dim + 2) * 4
                            : 0);
  w.logits = (float*)take(R * V * 4);
  w.ss = (float*)take(c.dtype == SPEC_DT_BF16 ? R * (d / 16) * 4 : 0);
  // slot partials of the residual GEMMs at 2-4 row tiles: [d/16 tiles][4 slots][4][1 KB]
  w.sk_part = (float*)take(c.dtype == SPEC_DT_BF16 ? (d / 16) * 4 * 8 * 1024 : 0);
  w.rowscale = (float*)take(c.dtype == SPEC_DT_F32 ? R * 4 : 0);
  w.rope_rows = (double*)take(c.dtype == SPEC_DT_BF16 ? R * c.head_dim * 8 : 0);
  w.total = off;
  return w;
}

// Parity-check exports of a traced forward (spec_verify_forward_trace).
struct Trace {
  float* resid;    // [2L+1][R][d]
  void* q;         // [L][R][d] activation type, or NULL
  void* attn_out;  // [L][R][d] activation type, or NULL
  void* ffn_act;   // [L][R][F] activation type, or NULL
};

// Kernel timing (measurement only): start/stop events attached to the dispatch packets
// of GEMM and attention launches (hipExtLaunchKernelGGL), so no extra commands are
// queued between kernels.
struct Timing {
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<std::pair<int, int>> gemm, attn;  // indices into pool (start, stop)
  size_t used = 0;
  int next() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return -1;
      pool.push_back(e);
    }
    return (int)used++;
  }
};
Timing g_timing;
std::mutex g_timing_mu;

struct Ev {
  hipEvent_t e0 = nullptr, e1 = nullptr;
};

Ev timed(std::vector<std::pair<int, int>>& list) {
  Ev ev;
  if (!g_timing.on) return ev;
  const int a = g_timing.next(), b = g_timing.next();
  if (a < 0 || b < 0) return ev;
  list.push_back({a, b});
  ev.e0 = g_timing.pool[a];
  ev.e1 = g_timing.pool[b];
  return ev;
}

// Residual-stream trace (parity checks): copies of x [R, d] after the embedding and after
// each half of every layer, trace[0 .. 2L].
#define SPEC_TRACE(idx)                                                                    \
  do {                                                                                     \
    if (trace)                                                                             \
      SPEC_LAUNCH(hipMemcpyAsync(trace->resid + (size_t)(idx) * R * d, w.x,                \
                                 (size_t)R * d * 4, hipMemcpyDeviceToDevice, s));          \
  } while (0)
// the layer's rotated queries (natural order already)
#define SPEC_TRACE_Q(l)                                                                    \
  do {                                                                                     \
    if (trace && trace->q)                                                                 \
      SPEC_LAUNCH(hipMemcpyAsync((char*)trace->q + (size_t)(l) * R * d * e, w.q,           \
                                 (size_t)R * d * e, hipMemcpyDeviceToDevice, s));          \
  } while (0)
// the layer's rounded attention output / FFN activation in natural row order
#define SPEC_TRACE_ACT(dst, l, src, width)                                                  \
  do {                                                                                     \
    if (trace && trace->dst)                                                               \
      SPEC_LAUNCH(launch_trace_act(c.dtype, src, R, width,                                 \
                                   (char*)trace->dst + (size_t)(l) * R * (width) * e, s)); \
  } while (0)

spec_status forward_f32(const spec_model* m, spec_kv* kv, int B, int M, float* logits,
                        const FwdWS& w, hipStream_t s, const Trace* trace) {
  const spec_model_cfg& c = m->cfg;
  const int dt = c.dtype;
  const int R = B * M, d = c.d_model, F = c.d_ffn, V = c.vocab, H = c.n_heads,
            hd = c.head_dim;
  const size_t e = elt_bytes(c);
  SPEC_LAUNCH(launch_embed(m->embed, dt, w.tok_eff, R, d, w.x, s));
  SPEC_TRACE(0);
  const int swiglu = c.ffn_kind == SPEC_FFN_SWIGLU;
  for (int l = 0; l < c.n_layers; ++l) {
    const spec_model::Layer& L = m->layers[l];
    char* kl = (char*)kv->data + (size_t)l * kv->layer_stride * e;
    char* vl = kl + kv->kv_stride * e;
    SPEC_LAUNCH(launch_norm_input(w.x, L.norm1, R, d, c.norm_eps, (float*)w.h, w.rowscale, s));
    Ev e1 = timed(g_timing.gemm);
    SPEC_LAUNCH(launch_gemm_f32((const float*)w.h, (const float*)L.wqkv, nullptr, 3 * d, R,
                                3 * d, d, w.y, 0, w.rowscale, nullptr, M, s, e1.e0, e1.e1));
    SPEC_LAUNCH(launch_rope_append(dt, w.y, B, M, H, hd, c.rope_theta, w.pos0, w.ntok_eff, w.q,
                                   kl, vl, kv->row_stride, kv->head_stride, kv->max_len, s));
    SPEC_TRACE_Q(l);
    Ev e2 = timed(g_timing.attn);
    SPEC_LAUNCH(launch_attention_f32((const float*)w.q, (const float*)kl, (const float*)vl,
                                     kv->row_stride, kv->head_stride, B, M, H, hd, w.pos0,
                                     w.ntok_eff, kv->max_len, (float*)w.att, s, e2.e0, e2.e1));
    SPEC_TRACE_ACT(attn_out, l, w.att, d);
    Ev e3 = timed(g_timing.gemm);
    SPEC_LAUNCH(launch_gemm_f32((const float*)w.att, (const float*)L.wo, nullptr, d, R, d, d,
                                w.x, 1, nullptr, nullptr, M, s, e3.e0, e3.e1));
    SPEC_TRACE(2 * l + 1);
    SPEC_LAUNCH(launch_norm_input(w.x, L.norm2, R, d, c.norm_eps, (float*)w.h, w.rowscale, s));
    Ev e4 = timed(g_timing.gemm);
    if (swiglu)
      SPEC_LAUNCH(launch_gemm_f32((const float*)w.h, (const float*)L.w_up,
                                  (const float*)L.w_up2, F, R, 2 * F, d, w.y, 0, w.rowscale,
                                  nullptr, M, s, e4.e0, e4.e1));
    else
      SPEC_LAUNCH(launch_gemm_f32((const float*)w.h, (const float*)L.w_up, nullptr, F, R, F, d,
                                  w.y, 0, w.rowscale, nullptr, M, s, e4.e0, e4.e1));
    SPEC_LAUNCH(launch_act(dt, c.ffn_kind, w.y, R, F, w.a, s));
    SPEC_TRACE_ACT(ffn_act, l, w.a, F);
    Ev e5 = timed(g_timing.gemm);
    SPEC_LAUNCH(launch_gemm_f32((const float*)w.a, (const float*)L.w_down, nullptr, d, R, d, F,
                                w.x, 1, nullptr, nullptr, M, s, e5.e0, e5.e1));
    SPEC_TRACE(2 * l + 2);
  }
  SPEC_LAUNCH(launch_norm_input(w.x, m->norm_f, R, d, c.norm_eps, (float*)w.h, w.rowscale, s));
  Ev e6 = timed(g_timing.gemm);
  SPEC_LAUNCH(launch_gemm_f32((const float*)w.h, (const float*)m->head, nullptr, V, R, V, d,
                              logits, 0, w.rowscale, w.ntok_eff, M, s, e6.e0, e6.e1));
  return SPEC_OK;
}

// bf16 models: 5 kernels per layer.
//   QKV GEMM (row factor, RoPE, q out, K/V append) -> attention (+ split merge) ->
//   O GEMM (x += y, next input bf16(x * g2) and its sums of squares) ->
//   up GEMM (row factor, SwiGLU / GELU) -> down GEMM (x += y, next input and sums of
//   squares for the next layer's QKV; after the last layer x * g_f in fp32) ->
//   after the layers: normalise pass (bf16(RMSNorm(x) * g_f)) -> LM head GEMM.
spec_status forward_bf16(const spec_model* m, spec_kv* kv, int B, int M, float* logits,
                         const FwdWS& w, hipStream_t s, const Trace* trace, const PrepArgs& pa) {
  const spec_model_cfg& c = m->cfg;
  const int R = B * M, d = c.d_model, F = c.d_ffn, V = c.vocab, H = c.n_heads,
            hd = c.head_dim;
  const size_t e = elt_bytes(c);
  unsigned* attn_counters = w.counters;
  SPEC_LAUNCH(launch_embed_norm(m->embed, pa, R, d, m->layers[0].norm1, w.x, w.h, w.ss,
                                kv->rope, M, hd, kv->max_len, w.rope_rows, s));
  SPEC_TRACE(0);
  GemmArgs base{};
  base.R = R;
  base.M = M;
  base.ntok_eff = w.ntok_eff;
  base.pos0 = w.pos0;
  base.d = d;
  base.hd = hd;
  base.rope_rows = w.rope_rows;
  base.row_stride = kv->row_stride;
  base.head_stride = kv->head_stride;
  base.max_len = kv->max_len;
  base.zeros = (const uint16_t*)(w.counters + w.n_counters - 64);
  base.sk_part = w.sk_part;
  base.sk_counters = w.counters + (w.n_counters - 64 - w.n_sk * kSkCounterStride);
  base.ss_np = d / 16;
  base.eps = c.norm_eps;
  for (int l = 0; l < c.n_layers; ++l) {
    const spec_model::Layer& L = m->layers[l];
    const bool last = l + 1 == c.n_layers;
    uint16_t* kl = (uint16_t*)((char*)kv->data + (size_t)l * kv->layer_stride * e);
    uint16_t* vl = kl + kv->kv_stride;
    {
      GemmArgs g = base;
      g.mode = EPI_QKV_ROPE;
      g.A = (const uint16_t*)w.h;
      g.lda = d;
      g.W = (const uint16_t*)L.wqkv;
      g.N = g.N1 = 3 * d;
      g.K = d;
      g.q_out = (uint16_t*)w.q;
      g.kc = kl;
      g.vc = vl;
      g.ss_in = w.ss;
      Ev ev = timed(g_timing.gemm);
      SPEC_LAUNCH(launch_gemm_bf16(g, s, ev.e0, ev.e1));
    }
    SPEC_TRACE_Q(l);
    {
      Ev ev = timed(g_timing.attn);
      SPEC_LAUNCH(launch_attention_bf16((const uint16_t*)w.q, kl, vl, kv->row_stride,
                                        kv->head_stride, B, M, H, hd, w.pos0, w.ntok_eff,
                                        w.part, attn_counters, kv->max_len,
                                        (uint16_t*)w.att, l, c.n_layers, s, ev.e0, ev.e1));
    }
    SPEC_TRACE_ACT(attn_out, l, w.att, d);
    {
      GemmArgs g = base;
      g.mode = EPI_RESID;
      g.A = (const uint16_t*)w.att;
      g.lda = d;
      g.W = (const uint16_t*)L.wo;
      g.N = g.N1 = d;
      g.K = d;
      g.x = w.x;
      g.gain = L.norm2;
      g.h_out = (uint16_t*)w.h;
      g.ss_out = w.ss;
      Ev ev = timed(g_timing.gemm);
      SPEC_LAUNCH(launch_gemm_bf16(g, s, ev.e0, ev.e1));
    }
    SPEC_TRACE(2 * l + 1);
    {
      GemmArgs g = base;
      g.A = (const uint16_t*)w.h;
      g.lda = d;
      g.K = d;
      g.act_out = (uint16_t*)w.a;
      g.ss_in = w.ss;
      g.W = (const uint16_t*)L.w_up;
      if (c.ffn_kind == SPEC_FFN_SWIGLU) {
        g.mode = EPI_SWIGLU;
        g.N1 = F;
        g.N = 2 * F;
      } else {
        g.mode = EPI_GELU;
        g.N = g.N1 = F;
      }
      Ev ev = timed(g_timing.gemm);
      SPEC_LAUNCH(launch_gemm_bf16(g, s, ev.e0, ev.e1));
    }
    SPEC_TRACE_ACT(ffn_act, l, w.a, F);
    {
      GemmArgs g = base;
      g.mode = EPI_RESID;
      g.A = (const uint16_t*)w.a;
      g.lda = F;
      g.W = (const uint16_t*)L.w_down;
      g.N = g.N1 = d;
      g.K = F;
      g.x = w.x;
      g.gain = last ? m->norm_f : m->layers[l + 1].norm1;
      // the last layer hands x * g_f in fp32 to the normalise pass of the LM head's input
      g.h_out = last ? nullptr : (uint16_t*)w.h;
      g.xg_out = last ? w.xg : nullptr;
      g.ss_out = w.ss;
      Ev ev = timed(g_timing.gemm);
      SPEC_LAUNCH(launch_gemm_bf16(g, s, ev.e0, ev.e1));
    }
    SPEC_TRACE(2 * l + 2);
  }
  // the LM head's input bf16(RMSNorm(x) * g_f), rounded once after the row factor
  SPEC_LAUNCH(launch_norm_pack(w.xg, w.ss, R, d, c.norm_eps, (uint16_t*)w.h, kv->len,
                               w.ntok_eff, M, s));
  GemmArgs g = base;
  g.mode = EPI_STORE;
  g.A = (const uint16_t*)w.h;
  g.lda = d;
  g.W = (const uint16_t*)m->head;
  g.N = g.N1 = V;
  g.K = d;
  g.C = logits;
  g.ldc = V;
  Ev ev = timed(g_timing.gemm);
  SPEC_LAUNCH(launch_gemm_bf16(g, s, ev.e0, ev.e1));
  return SPEC_OK;
}
#undef SPEC_TRACE
#undef SPEC_TRACE_ACT
#undef SPEC_TRACE_Q

// The forward pass shared by the verify call, draft steps and prefill chunks.
spec_status forward(const spec_model* m, spec_kv* kv, const int32_t* tokens,
                    const int32_t* n_tok, int B, int M, float* logits, int32_t* row_status,
                    int record_base, const FwdWS& w, hipStream_t s,
                    const DraftSrc* ds = nullptr, const Trace* trace = nullptr) {
  if (m->cfg.dtype == SPEC_DT_BF16) {
    // the row bookkeeping runs inside the embedding kernel (k_embed_norm)
    const PrepArgs pa{tokens,    n_tok,      m->cfg.vocab,       kv->len,
                      kv->base,  record_base, w.pos0,            w.ntok_eff,
                      w.tok_eff, row_status, w.counters,         w.n_counters,
                      ds ? *ds : DraftSrc{}, ds ? 1 : 0};
    return forward_bf16(m, kv, B, M, logits, w, s, trace, pa);
  }
  SPEC_LAUNCH(launch_prep(tokens, n_tok, B, M, m->cfg.vocab, kv->len, kv->base, record_base,
                          kv->max_len, w.pos0, w.ntok_eff, w.tok_eff, row_status, w.counters,
                          w.n_counters, ds, s));
  return forward_f32(m, kv, B, M, logits, w, s, trace);
}

bool kv_matches(const spec_model* m, const spec_kv* kv) {
  const spec_model_cfg &a = m->cfg, &b = kv->cfg;
  return a.n_layers == b.n_layers && a.n_heads == b.n_heads && a.head_dim == b.head_dim &&
         a.dtype == b.dtype;
}

}  // namespace

extern "C" {

int spec_abi_version(void) { return 2; }

int spec_last_hip_error(void) { return g_last_hip_error.load(); }

const char* spec_status_str(int st) {
  switch (st) {
    case SPEC_OK: return "ok";
    case SPEC_E_INVALID: return "invalid argument";
    case SPEC_E_UNSUPPORTED: return "unsupported";
    case SPEC_E_CAPACITY: return "buffer too small";
    case SPEC_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int spec_model_n_weights(const spec_model_cfg* cfg) {
  if (!cfg_valid(cfg)) return -1;
  return 3 + cfg->n_layers * (cfg->ffn_kind == SPEC_FFN_SWIGLU ? 7 : 6);
}

namespace {

// Tensor i of the canonical order: its shape, where it lives in the model's store and
// how it is written there.
struct TensorSlot {
  int rows, cols;   // source shape [rows, cols] (norm gains: [1, d])
  bool fp32;        // stored as fp32 (norm gains, and every tensor of an fp32 model)
  int pack;         // -1 plain copy, else a PACK_* mode
  int ntiles;       // packed tiles (pack >= 0)
  size_t offset;    // byte offset of the tensor's storage in the store
  size_t bytes;     // storage bytes (for a pair half: the whole pair)
};

// Lay the model out; returns the store size and fills slots (canonical order) if given.
size_t model_layout(const spec_model_cfg& c, TensorSlot* slots) {
  const int d = c.d_model, F = c.d_ffn, V = c.vocab, L = c.n_layers;
  const bool bf = c.dtype == SPEC_DT_BF16, swiglu = c.ffn_kind == SPEC_FFN_SWIGLU;
  const size_t e = bf ? 2 : 4;
  size_t off = 0;
  int i = 0;
  auto put = [&](int rows, int cols, bool gain, int pack, int ntiles) {
    TensorSlot t{rows, cols, gain || !bf, bf && !gain ? pack : -1, ntiles, off, 0};
    t.bytes = (size_t)rows * cols * (t.fp32 ? 4 : e);
    off += align_up(t.bytes);
    if (slots) slots[i] = t;
    ++i;
  };
  put(V, d, false, -1, 0);               // embed (gathered by token, kept as given)
  put(V, d, false, PACK_PLAIN, V / 16);  // head
  put(1, d, true, -1, 0);                // norm_f
  for (int l = 0; l < L; ++l) {
    put(1, d, true, -1, 0);                         // norm1
    put(3 * d, d, false, PACK_QKV, 3 * d / 16);     // wqkv
    put(d, d, false, PACK_PLAIN, d / 16);           // wo
    put(1, d, true, -1, 0);                         // norm2
    if (swiglu && bf) {
      // gate and up share one packed block of F/8 tiles
      TensorSlot g{F, d, false, PACK_PAIR_LO, F / 8, off, (size_t)2 * F * d * e};
      TensorSlot u = g;
      u.pack = PACK_PAIR_HI;
      off += align_up(g.bytes);
      if (slots) {
        slots[i] = g;
        slots[i + 1] = u;
      }
      i += 2;
    } else if (swiglu) {
      put(F, d, false, -1, 0);  // wgate
      put(F, d, false, -1, 0);  // wup
    } else {
      put(F, d, false, PACK_PLAIN, F / 16);  // w1
    }
    put(d, F, false, PACK_PLAIN, d / 16);   // wdown / w2
  }
  return off;
}

}  // namespace

size_t spec_model_bytes(const spec_model_cfg* cfg) {
  if (!cfg_valid(cfg)) return 0;
  return model_layout(*cfg, nullptr);
}

spec_status spec_model_create(const spec_model_cfg* cfg, void* store, size_t store_bytes,
                              spec_model** out) {
  if (!cfg_valid(cfg) || !store || !out) return SPEC_E_INVALID;
  if (((uintptr_t)store) % kAlign) return SPEC_E_INVALID;
  if (!cfg_supported(cfg)) return SPEC_E_UNSUPPORTED;
  const int n = spec_model_n_weights(cfg);
  std::vector<TensorSlot> slots(n);
  const size_t bytes = model_layout(*cfg, slots.data());
  if (store_bytes < bytes) return SPEC_E_CAPACITY;
  if (!device_is_gfx950()) return SPEC_E_UNSUPPORTED;
  spec_model* m = new (std::nothrow) spec_model;
  if (!m) return SPEC_E_INVALID;
  m->cfg = *cfg;
  m->layers = new (std::nothrow) spec_model::Layer[cfg->n_layers];
  m->store = store;
  m->store_bytes = bytes;
  if (!m->layers) {
    delete m;
    return SPEC_E_INVALID;
  }
  char* base = (char*)m->store;
  int i = 0;
  auto at = [&]() { return (const void*)(base + slots[i++].offset); };
  m->embed = at();
  m->head = at();
  m->norm_f = (const float*)at();
  for (int l = 0; l < cfg->n_layers; ++l) {
    spec_model::Layer& L = m->layers[l];
    L.norm1 = (const float*)at();
    L.wqkv = at();
    L.wo = at();
    L.norm2 = (const float*)at();
    L.w_up = at();
    L.w_up2 = nullptr;
    if (cfg->ffn_kind == SPEC_FFN_SWIGLU) {
      const void* up = at();
      if (cfg->dtype != SPEC_DT_BF16) L.w_up2 = up;
    }
    L.w_down = at();
  }
  *out = m;
  return SPEC_OK;
}

spec_status spec_model_load_weight(spec_model* m, int index, const void* src, void* stream) {
  if (!m || !src) return SPEC_E_INVALID;
  const int n = spec_model_n_weights(&m->cfg);
  if (index < 0 || index >= n) return SPEC_E_INVALID;
  std::vector<TensorSlot> slots(n);
  model_layout(m->cfg, slots.data());
  const TensorSlot& t = slots[index];
  hipStream_t s = (hipStream_t)stream;
  char* dst = (char*)m->store + t.offset;
  hipError_t err;
  if (t.pack < 0) {
    err = hipMemcpyAsync(dst, src, t.bytes, hipMemcpyDeviceToDevice, s);
  } else {
    err = launch_pack_bf16((const uint16_t*)src, t.cols, t.pack, m->cfg.d_model,
                           m->cfg.head_dim, t.ntiles, (uint16_t*)dst, s);
  }
  if (err != hipSuccess) {
    g_last_hip_error.store((int)err);
    return SPEC_E_HIP;
  }
  return SPEC_OK;
}

spec_status spec_model_destroy(spec_model* m) {
  if (!m) return SPEC_E_INVALID;
  delete[] m->layers;
  delete m;
  return SPEC_OK;
}

// RoPE table of a bf16 cache: (cos, sin) of pos * theta^(-2i/hd) for every position.
size_t rope_table_bytes(const spec_model_cfg& c, int max_len) {
  return c.dtype == SPEC_DT_BF16 ? (size_t)max_len * (c.head_dim / 2) * 16 : 0;
}

size_t spec_kv_bytes(const spec_model_cfg* cfg, int batch, int max_len) {
  if (!cfg_valid(cfg) || batch < 1 || max_len < 1) return 0;
  const size_t cap = cfg->dtype == SPEC_DT_BF16 ? kv_capacity(max_len) : max_len;
  const size_t n = (size_t)cfg->n_layers * batch * 2 * cfg->n_heads * cap * cfg->head_dim;
  return align_up(n * elt_bytes(*cfg)) + align_up((size_t)batch * 4) +
         align_up(rope_table_bytes(*cfg, max_len));
}

spec_status spec_kv_create(const spec_model_cfg* cfg, int batch, int max_len, void* arena,
                           size_t arena_bytes, int32_t* len, void* stream, spec_kv** out) {
  if (!cfg_valid(cfg) || batch < 1 || max_len < 1 || !arena || !len || !out)
    return SPEC_E_INVALID;
  if (((uintptr_t)arena) % 256) return SPEC_E_INVALID;
  if (arena_bytes < spec_kv_bytes(cfg, batch, max_len)) return SPEC_E_CAPACITY;
  spec_kv* kv = new (std::nothrow) spec_kv;
  if (!kv) return SPEC_E_INVALID;
  kv->cfg = *cfg;
  kv->batch = batch;
  kv->max_len = max_len;
  kv->data = arena;
  kv->len = len;
  const size_t hd = cfg->head_dim, H = cfg->n_heads;
  kv->head_stride =
      (size_t)(cfg->dtype == SPEC_DT_BF16 ? kv_capacity(max_len) : max_len) * hd;
  kv->kv_stride = H * kv->head_stride;
  kv->row_stride = 2 * kv->kv_stride;
  kv->layer_stride = (size_t)batch * kv->row_stride;
  const size_t n = (size_t)cfg->n_layers * kv->layer_stride;
  kv->base = (int32_t*)((char*)arena + align_up(n * elt_bytes(*cfg)));
  kv->rope = nullptr;
  if (cfg->dtype == SPEC_DT_BF16) {
    // rotation factors in fp64, written into the arena tail on the caller's stream
    kv->rope = (double*)((char*)kv->base + align_up((size_t)batch * 4));
    const hipError_t err = launch_rope_table(kv->rope, max_len, cfg->head_dim,
                                             (double)cfg->rope_theta, (hipStream_t)stream);
    if (err != hipSuccess) {
      g_last_hip_error.store((int)err);
      delete kv;
      return SPEC_E_HIP;
    }
  }
  *out = kv;
  return SPEC_OK;
}

spec_status spec_kv_destroy(spec_kv* kv) {
  if (!kv) return SPEC_E_INVALID;
  delete kv;
  return SPEC_OK;
}

void* spec_kv_data(spec_kv* kv) { return kv ? kv->data : nullptr; }

namespace {
spec_status kv_transfer(spec_kv* kv, void* nat, int n_pos, void* stream, int to_cache) {
  if (!kv || !nat || n_pos < 0 || n_pos > kv->max_len) return SPEC_E_INVALID;
  const spec_model_cfg& c = kv->cfg;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err;
  if (c.dtype == SPEC_DT_BF16) {
    err = launch_kv_convert((uint16_t*)kv->data, (uint16_t*)nat, c.n_layers, kv->batch,
                            c.n_heads, c.head_dim, n_pos, kv->layer_stride, kv->row_stride,
                            kv->kv_stride, kv->head_stride, to_cache, s);
  } else {
    // fp32 caches keep the natural layout: one strided copy
    const size_t w = (size_t)n_pos * c.head_dim * 4;
    const size_t heads = (size_t)c.n_layers * kv->batch * 2 * c.n_heads;
    if (w == 0) return SPEC_OK;
    err = to_cache ? hipMemcpy2DAsync(kv->data, kv->head_stride * 4, nat, w, w, heads,
                                      hipMemcpyDeviceToDevice, s)
                   : hipMemcpy2DAsync(nat, w, kv->data, kv->head_stride * 4, w, heads,
                                      hipMemcpyDeviceToDevice, s);
  }
  if (err != hipSuccess) return hip_fail(err);
  return SPEC_OK;
}
}  // namespace

spec_status spec_kv_import(spec_kv* kv, const void* src, int n_pos, void* stream) {
  return kv_transfer(kv, const_cast<void*>(src), n_pos, stream, 1);
}

spec_status spec_kv_export(spec_kv* kv, void* dst, int n_pos, void* stream) {
  return kv_transfer(kv, dst, n_pos, stream, 0);
}

spec_status spec_kv_rollback(spec_kv* kv, const int32_t* new_len, void* stream) {
  if (!kv || !new_len) return SPEC_E_INVALID;
  SPEC_LAUNCH(launch_rollback(kv->len, new_len, kv->batch, (hipStream_t)stream));
  return SPEC_OK;
}

size_t spec_workspace_bytes(const spec_model_cfg* cfg, int batch, int max_rows, int max_len) {
  if (!cfg_valid(cfg) || batch < 1 || max_rows < 1 || max_len < 1) return 0;
  return fwd_layout(*cfg, batch, std::max(max_rows, 2), max_len, nullptr).total;
}

spec_status spec_verify_forward(const spec_model* m, spec_kv* kv, const int32_t* tokens,
                                const int32_t* n_tok, int B, int M, float* logits,
                                int32_t* row_status, void* ws, size_t ws_bytes, void* stream) {
  if (!m || !kv || !tokens || !logits || !ws) return SPEC_E_INVALID;
  if (B < 1 || B > kv->batch || M < 1 || M > 64) return SPEC_E_INVALID;
  if (!kv_matches(m, kv)) return SPEC_E_INVALID;
  if (((uintptr_t)ws) % 256) return SPEC_E_INVALID;
  const FwdWS w = fwd_layout(m->cfg, B, M, kv->max_len, (char*)ws);
  if (ws_bytes < w.total) return SPEC_E_CAPACITY;
  return forward(m, kv, tokens, n_tok, B, M, logits, row_status, 1, w, (hipStream_t)stream);
}

spec_status spec_verify_forward_trace(const spec_model* m, spec_kv* kv, const int32_t* tokens,
                                      const int32_t* n_tok, int B, int M, float* logits,
                                      int32_t* row_status, float* resid, void* q,
                                      void* attn_out, void* ffn_act, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!m || !kv || !tokens || !logits || !ws || !resid) return SPEC_E_INVALID;
  if (B < 1 || B > kv->batch || M < 1 || M > 64) return SPEC_E_INVALID;
  if (!kv_matches(m, kv)) return SPEC_E_INVALID;
  if (((uintptr_t)ws) % 256) return SPEC_E_INVALID;
  const FwdWS w = fwd_layout(m->cfg, B, M, kv->max_len, (char*)ws);
  if (ws_bytes < w.total) return SPEC_E_CAPACITY;
  const Trace tr{resid, q, attn_out, ffn_act};
  return forward(m, kv, tokens, n_tok, B, M, logits, row_status, 1, w, (hipStream_t)stream,
                 nullptr, &tr);
}

spec_status spec_draft_step(const spec_model* draft, spec_kv* dkv, const int32_t* in_tok,
                            const int32_t* n_in, int B, int K, int step,
                            const spec_sampling* knobs, uint64_t seed, uint64_t round,
                            const uint64_t* round_dev, int32_t* x_tilde, float* q_logits,
                            int32_t* row_status, void* ws, size_t ws_bytes, void* stream) {
  if (!draft || !dkv || !x_tilde || !q_logits || !ws || !knobs_valid(knobs))
    return SPEC_E_INVALID;
  if (B < 1 || B > dkv->batch || K < 1 || K > 16 || step < 0 || step >= K)
    return SPEC_E_INVALID;
  if (step == 0 && (!in_tok || !n_in)) return SPEC_E_INVALID;
  if (!kv_matches(draft, dkv)) return SPEC_E_INVALID;
  if (draft->cfg.vocab > 32768) return SPEC_E_UNSUPPORTED;
  if (((uintptr_t)ws) % 256) return SPEC_E_INVALID;
  const int M = step == 0 ? 2 : 1;
  const FwdWS w = fwd_layout(draft->cfg, B, M, dkv->max_len, (char*)ws);
  if (ws_bytes < w.total) return SPEC_E_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  const DraftSrc ds{in_tok, n_in, x_tilde, K, step, w.ntok2};
  spec_status st = forward(draft, dkv, nullptr, nullptr, B, M, w.logits, row_status,
                           step == 0 ? 1 : 0, w, s, &ds);
  if (st != SPEC_OK) return st;
  SPEC_LAUNCH(launch_draft_sample(w.logits, B, M, w.ntok2, step, K, draft->cfg.vocab,
                                  to_knobs(knobs), seed, round, round_dev, x_tilde, q_logits,
                                  row_status, s));
  return SPEC_OK;
}

spec_status spec_verify_tokens(const int32_t* pending, const int32_t* n_pending,
                               const int32_t* x_tilde, int B, int K, int32_t* tokens,
                               void* stream) {
  if (!pending || !n_pending || !x_tilde || !tokens || B < 1 || K < 1) return SPEC_E_INVALID;
  SPEC_LAUNCH(launch_verify_tokens(pending, n_pending, x_tilde, B, K, tokens,
                                   (hipStream_t)stream));
  return SPEC_OK;
}

size_t spec_accept_workspace_bytes(int B, int K) {
  if (B < 1 || K < 1) return 0;
  return align_up((size_t)B * K * 4) + 2 * align_up((size_t)B * (K + 1) * 4);
}

spec_status spec_accept_resample(const float* p_logits, const float* q_logits,
                                 const int32_t* x_tilde, int B, int K, int V,
                                 const spec_sampling* knobs, uint64_t seed, uint64_t round,
                                 uint64_t* round_dev, int32_t* out_tok, int32_t* n_out,
                                 int32_t* row_status,
                                 spec_kv* tkv, spec_kv* dkv, int32_t* pending,
                                 int32_t* n_pending, void* const* debug, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!p_logits || !q_logits || !x_tilde || !out_tok || !n_out || !row_status || !ws)
    return SPEC_E_INVALID;
  if (B < 1 || K < 1 || K > 16 || V < 1 || !knobs_valid(knobs)) return SPEC_E_INVALID;
  if ((pending == nullptr) != (n_pending == nullptr)) return SPEC_E_INVALID;
  if (tkv && tkv->batch < B) return SPEC_E_INVALID;
  if (dkv && dkv->batch < B) return SPEC_E_INVALID;
  if (V > 32768) return SPEC_E_UNSUPPORTED;
  if (ws_bytes < spec_accept_workspace_bytes(B, K)) return SPEC_E_CAPACITY;
  char* p = (char*)ws;
  int32_t* res_acc = (int32_t*)p;
  p += align_up((size_t)B * K * 4);
  int32_t* res_cand = (int32_t*)p;
  p += align_up((size_t)B * (K + 1) * 4);
  int32_t* res_status = (int32_t*)p;
  float* dbg_p = debug ? (float*)debug[0] : nullptr;
  float* dbg_q = debug ? (float*)debug[1] : nullptr;
  hipStream_t s = (hipStream_t)stream;
  SPEC_LAUNCH(launch_accept_rows(p_logits, q_logits, x_tilde, B, K, V, to_knobs(knobs), seed,
                                 round, round_dev, res_acc, res_cand, res_status, dbg_p, dbg_q,
                                 s));
  SPEC_LAUNCH(launch_select(x_tilde, B, K, res_acc, res_cand, res_status, out_tok, n_out,
                            row_status, tkv ? tkv->len : nullptr, tkv ? tkv->base : nullptr,
                            dkv ? dkv->len : nullptr, dkv ? dkv->base : nullptr, pending,
                            n_pending, round_dev, s));
  if (debug && debug[2])
    SPEC_LAUNCH(hipMemcpyAsync(debug[2], res_acc, (size_t)B * K * 4, hipMemcpyDeviceToDevice, s));
  if (debug && debug[3])
    SPEC_LAUNCH(hipMemcpyAsync(debug[3], res_cand, (size_t)B * (K + 1) * 4,
                               hipMemcpyDeviceToDevice, s));
  return SPEC_OK;
}

}  // extern "C"

namespace {

// Scratch of spec_accept_resample_static: a file-scope device array (each GPU the library
// runs on holds its own copy until the process ends).  In host code `scratch` only names
// the symbol; its device address comes from hipGetSymbolAddress, once per device, with
// that device current.
constexpr size_t kStaticScratchBytes = 64 * 1024;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// This device's address of `scratch`, resolved on first use; nullptr on failure.
void* static_scratch(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

spec_status spec_accept_resample_static(const float* p_logits, const float* q_logits,
                                        const int32_t* x_tilde, int B, int K, int V,
                                        const spec_sampling* knobs, uint64_t seed,
                                        uint64_t round, uint64_t* round_dev, int32_t* out_tok,
                                        int32_t* n_out, int32_t* row_status, spec_kv* tkv,
                                        spec_kv* dkv, int32_t* pending, int32_t* n_pending,
                                        void* stream) {
  if (B < 1 || K < 1) return SPEC_E_INVALID;
  if (spec_accept_workspace_bytes(B, K) > kStaticScratchBytes) return SPEC_E_CAPACITY;
  hipError_t err = hipSuccess;
  void* ws = static_scratch(&err);
  if (!ws) return hip_fail(err);
  // every slot the kernels read is written earlier in the same call: nothing to clear
  return spec_accept_resample(p_logits, q_logits, x_tilde, B, K, V, knobs, seed, round,
                              round_dev, out_tok, n_out, row_status, tkv, dkv, pending,
                              n_pending, nullptr, ws, kStaticScratchBytes, stream);
}

spec_status spec_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing.on = on != 0;
  return SPEC_OK;
}

spec_status spec_timing_read(double* gemm_ms, int* gemm_launches, double* attn_ms,
                             int* attn_launches) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  auto total = [](const std::vector<std::pair<int, int>>& l, double* ms, int* n) -> hipError_t {
    double t = 0.0;
    for (auto& pr : l) {
      hipError_t e = hipEventSynchronize(g_timing.pool[pr.second]);
      if (e != hipSuccess) return e;
      float x = 0.f;
      e = hipEventElapsedTime(&x, g_timing.pool[pr.first], g_timing.pool[pr.second]);
      if (e != hipSuccess) return e;
      t += x;
    }
    if (ms) *ms = t;
    if (n) *n = (int)l.size();
    return hipSuccess;
  };
  hipError_t e = total(g_timing.gemm, gemm_ms, gemm_launches);
  if (e == hipSuccess) e = total(g_timing.attn, attn_ms, attn_launches);
  g_timing.gemm.clear();
  g_timing.attn.clear();
  g_timing.used = 0;
  if (e != hipSuccess) return hip_fail(e);
  return SPEC_OK;
}

}  // extern "C"
