// Host-side structures shared by the C ABI implementation and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specdec.h"
#include "act_layout.h"
#include "gemm.h"
#include "kv_layout.h"

struct spec_model {
  spec_model_cfg cfg;
  // The caller's device store (spec_model_bytes) holds the model's copy of every tensor:
  // bf16 matrices packed into GEMM tiles, the rest (embedding, norm gains, fp32
  // matrices) stored as given.
  void* store;
  size_t store_bytes;
  const void* embed;   // [V, d] as given
  const void* head;    // bf16: packed tiles of 16 vocabulary rows; f32: [V, d]
  const float* norm_f;
  struct Layer {
    const float* norm1;
    const void* wqkv;    // bf16: packed (RoPE-paired tiles); f32: [3d, d]
    const void* wo;
    const float* norm2;
    const void* w_up;    // bf16 SwiGLU: packed gate/up pair tiles; GELU: w1.  f32: wgate / w1
    const void* w_up2;   // f32 SwiGLU: wup; otherwise unused
    const void* w_down;  // wdown / w2
  };
  Layer* layers;
};

struct spec_kv {
  spec_model_cfg cfg;
  int batch, max_len;
  void* data;        // [L][B][2][H][max_len][hd]
  int32_t* len;      // [B] caller-owned
  int32_t* base;     // [B] length before the last recorded append (in the arena tail)
  double* rope;      // bf16 models: [max_len][hd/2][2] RoPE (cos, sin) (in the arena tail)
  size_t layer_stride, row_stride, kv_stride, head_stride;  // in elements
};

struct SamplingKnobs {
  float inv_t;  // 1 / temperature (unused when greedy)
  int top_k;
  float top_p;
  int greedy;   // temperature 0: argmax decoding
};

// kernel launchers (defined in the .hip files)
namespace specdec {


hipError_t launch_attention_bf16(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                                 size_t row_stride, size_t head_stride, int B, int M, int H,
                                 int hd, const int32_t* pos0, const int32_t* ntok_eff,
                                 float* part, unsigned* counters, int max_len, uint16_t* out,
                                 int layer, int n_layers, hipStream_t s, hipEvent_t e0,
                                 hipEvent_t e1);
constexpr int kAttnMaxCUs = 1024;                     // bound on the CUs a split grid uses
// completion counters of the split attention sit 128 bytes apart: the atomics of
// different (row, head, group) units then do not queue on one cache line
constexpr int kAttnCounterStride = 32;
int attn_nsplit(int B, int H, int M, int max_len);  // splits per (row, head, group)
int attn_max_splits(int B, int H, int M, int max_len);  // bound of attn_nsplit (workspace)
int attn_groups(int M);                               // query groups per row
hipError_t launch_kv_convert(uint16_t* cache, uint16_t* nat, int L, int B, int H, int hd, int n,
                             size_t layer_stride, size_t row_stride, size_t kv_stride,
                             size_t head_stride, int to_cache, hipStream_t s);


// forward pieces
// Input tokens of a draft step, assembled by the prep kernel itself: step 0 takes the
// n_in[b] (1 or 2) pending tokens in_tok[b, 0..1], step s > 0 the draft token
// x_tilde[b, s - 1]; the per-row count also goes to n_tok_out (the sampler reads it).
struct DraftSrc {
  const int32_t* in_tok;
  const int32_t* n_in;
  const int32_t* x_tilde;
  int K, step;
  int32_t* n_tok_out;
};
// Row bookkeeping of a forward (k_prep; for bf16 models folded into k_embed_norm).
struct PrepArgs {
  const int32_t* tokens;
  const int32_t* n_tok;
  int V;
  int32_t* len;
  int32_t* base;
  int record_base;
  int32_t* pos0;
  int32_t* ntok_eff;
  int32_t* tok_eff;
  int32_t* row_status;
  unsigned* counters;
  int n_counters;
  DraftSrc ds;
  int draft;
};
hipError_t launch_embed_norm(const void* embed, const PrepArgs& pa, int R, int d, const float* g,
                             float* x, void* h, float* ss, const double* rope, int M, int hd,
                             int max_len, double* rope_rows, hipStream_t s);
hipError_t launch_prep(const int32_t* tokens, const int32_t* n_tok, int B, int M, int V,
                       int32_t* len, int32_t* base, int record_base, int max_len,
                       int32_t* pos0, int32_t* ntok_eff, int32_t* tok_eff,
                       int32_t* row_status, unsigned* counters, int n_counters,
                       const DraftSrc* ds, hipStream_t s);
hipError_t launch_embed(const void* embed, int dtype, const int32_t* tok_eff, int R, int d,
                        float* x, hipStream_t s);
hipError_t launch_norm_input(const float* x, const float* g, int R, int d, float eps,
                             float* h, float* rowscale, hipStream_t s);
hipError_t launch_rope_append(int dtype, const float* qkv, int B, int M, int H, int hd,
                              float theta, const int32_t* pos0, const int32_t* ntok_eff,
                              void* q_out, void* kcache, void* vcache, size_t row_stride,
                              size_t head_stride, int max_len, hipStream_t s);
hipError_t launch_attention_f32(const float* q, const float* kcache, const float* vcache,
                                size_t row_stride, size_t head_stride, int B, int M, int H,
                                int hd, const int32_t* pos0, const int32_t* ntok_eff,
                                int max_len, float* out, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1);
hipError_t launch_act(int dtype, int ffn_kind, const float* y, int R, int F, void* a,
                      hipStream_t s);

// sampling
hipError_t launch_accept_rows(const float* p_logits, const float* q_logits,
                              const int32_t* x_tilde, int B, int K, int V, SamplingKnobs kn,
                              uint64_t seed, uint64_t round, const uint64_t* round_dev,
                              int32_t* res_acc, int32_t* res_cand, int32_t* res_status,
                              float* dbg_p, float* dbg_q, hipStream_t s);
hipError_t launch_select(const int32_t* x_tilde, int B, int K, const int32_t* res_acc,
                         const int32_t* res_cand, const int32_t* res_status,
                         int32_t* out_tok, int32_t* n_out, int32_t* row_status,
                         int32_t* t_len, const int32_t* t_base, int32_t* d_len,
                         const int32_t* d_base, int32_t* pending, int32_t* n_pending,
                         uint64_t* round_dev, hipStream_t s);
hipError_t launch_draft_sample(const float* logits, int B, int M, const int32_t* n_in,
                               int step, int K, int V, SamplingKnobs kn, uint64_t seed,
                               uint64_t round, const uint64_t* round_dev, int32_t* x_tilde,
                               float* q_logits, int32_t* row_status, hipStream_t s);
hipError_t launch_rollback(int32_t* len, const int32_t* new_len, int B, hipStream_t s);
hipError_t launch_rope_table(double* tab, int max_len, int hd, double theta, hipStream_t s);
// R rows of width K of an activation buffer (bf16: the packed order; fp32: natural) into
// natural row-major order (parity-check exports)
hipError_t launch_trace_act(int dtype, const void* src, int R, int K, void* dst, hipStream_t s);
hipError_t launch_verify_tokens(const int32_t* pending, const int32_t* n_pending,
                                const int32_t* x_tilde, int B, int K, int32_t* tokens,
                                hipStream_t s);

}  // namespace specdec
