/*
 * specdec.h -- C ABI of the speculative-sampling hot path on MI355X (gfx950).
 *
 * The library computes one speculative round's GPU work: the target model's single
 * verify pass over the K+1 drafted positions, the draft model's steps, and the
 * modified rejection-sampling step (accept with min(1, p/q), resample the first
 * rejection from norm(max(0, p - q)), bonus token when all K are accepted), plus the
 * KV-cache append / roll-back that goes with them.
 *
 * Sources (web pages describing the method):
 *   [ZSM]   "Accelerating Large Language Model Decoding with Speculative Sampling"
 *           (zeroshotmind.com explainer of Chen et al.)
 *   [CANON] "57 Speculative Decoding" (ml-canon)
 *   [LENS]  "Speculative Decoding from Scratch -- How a Tiny Draft Model Speeds Up an
 *           LLM Without Changing a Single Output" (ta-paperlens)
 *   [GC]    "Speculative Decoding: Getting 3x Speedups Without Changing the Model"
 *           (General Compute blog)
 *   [NOTE]  "NOTE-159: Accelerating Large Language Model Decoding with Speculative
 *           Sampling" (anthology-of-the-sota)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates and
 *     frees every device buffer (model store, KV arena, lengths, logits, tokens,
 *     outputs, workspace); no call allocates device memory or throws, and no call
 *     waits for the device except spec_timing_read (a measurement aid).
 *   - Calls that launch work are asynchronous on `stream` (a hipStream_t; NULL = the
 *     null stream).  The caller keeps buffers alive until the stream work has finished.
 *   - A handle (spec_model, spec_kv) is an opaque host object owned by the library;
 *     use one handle from one stream at a time.
 *   - Arguments the host can check are checked before anything is launched; a bad
 *     call returns a negative spec_status and launches nothing.  Conditions only the
 *     device can see (lengths, token ids, non-finite logits) are reported per row in
 *     `row_status` bits (SPEC_ROW_*), and such a row is left well-defined.
 *   - Indices are 0-based: drafts x~_0..x~_{K-1}; target logit rows P_0..P_K (row j
 *     scores draft j, row K is the bonus row); draft rows Q_0..Q_{K-1}.
 *   - Layouts are row-major, innermost index last.
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_E_INVALID = -1,      /* null pointer, bad shape, bad knob value              */
  SPEC_E_UNSUPPORTED = -2,  /* valid but not built: e.g. V > 32768, no gfx950 */
  SPEC_E_CAPACITY = -3,     /* workspace or arena smaller than the size query says  */
  SPEC_E_HIP = -4           /* a HIP launch failed; see spec_last_hip_error()        */
} spec_status;

/* row_status bits (int32 per sequence row) */
#define SPEC_ROW_NONFINITE 1        /* a logit row of this sequence held NaN/Inf: nothing emitted  */
#define SPEC_ROW_Q_ZERO 2           /* q(x~_j) == 0 at an evaluated position (rule still total)   */
#define SPEC_ROW_RESIDUAL_EMPTY 4   /* max(0, p - q) summed to 0 at the rejection: sampled P_a    */
#define SPEC_ROW_KV_OVERFLOW 8      /* cache could not take the tokens: row skipped               */
#define SPEC_ROW_BAD_TOKEN 16       /* token id outside [0, V): nothing emitted                   */

enum { SPEC_FFN_GELU = 0, SPEC_FFN_SWIGLU = 1 };
enum { SPEC_DT_F32 = 0, SPEC_DT_BF16 = 1 };

/* Model shape (host).  Decoder-only, pre-norm, no biases, untied embedding and LM
 * head, RMSNorm (eps), RoPE (theta, half-split pairs (i, i + hd/2)), causal MHA with
 * 1/sqrt(hd) scaling.  GELU FFN: W1 [F,d], W2 [d,F]; SwiGLU: Wg, Wu [F,d], Wd [d,F].
 * bf16 models: bf16 weights and activations into every matrix product, fp32
 * accumulation, fp32 residual stream / norms / softmax / logits.  f32: all fp32. */
typedef struct {
  int n_layers, d_model, n_heads, head_dim, d_ffn, vocab;
  int ffn_kind; /* SPEC_FFN_* */
  int dtype;    /* SPEC_DT_*  */
  float norm_eps, rope_theta;
} spec_model_cfg;

/* Sampling knobs applied to BOTH p and q before the rule ([NOTE] "Key results",
 * robust-to-knobs item, and Recommendation R3), in the order temperature -> top-k ->
 * top-p -> renormalise.  temperature >= 0; 0 is argmax decoding ([LENS] "How much faster
 * in practice?", the argmax column of Table 2): each processed row is one-hot at the
 * lowest token id holding the largest logit, top_k and top_p change nothing, and the rule
 * emits the target's own argmax continuation;
 * top_k = 0 means off (0 <= top_k); top_p = 1 means off (0 < top_p <= 1).  Ties at a
 * top-k or top-p threshold are all kept. */
typedef struct {
  float temperature;
  int top_k;
  float top_p;
} spec_sampling;

typedef struct spec_model spec_model; /* opaque */
typedef struct spec_kv spec_kv;       /* opaque */

/* ------------------------------------------------------------------ model --------- */

/* Number of tensors of a model of `cfg` (the canonical order of spec_model_load_weight). */
int spec_model_n_weights(const spec_model_cfg* cfg);

/* Bytes of the device store a model of `cfg` keeps its copy of the weights in (0 for an
 * invalid cfg). */
size_t spec_model_bytes(const spec_model_cfg* cfg);

/* Create a model handle over a caller-owned device store of store_bytes >=
 * spec_model_bytes(cfg) bytes (256-byte aligned; the caller frees it after
 * spec_model_destroy).  Nothing is allocated or launched: fill the store with
 * spec_model_load_weight, one call per tensor.  The store holds every tensor, the bf16
 * matrices rearranged into the tile order the verify GEMM streams (column tiles of 16
 * weight rows, each tile one contiguous block in MFMA operand order), so each weight byte
 * is read from HBM once in fully used 1 KB wave loads ([ZSM] "The cost of one token is
 * the cost of reading the weights"; [GC] "Why Standard Decoding Is Slow").
 * Returns SPEC_E_INVALID for a bad shape, a null or misaligned pointer;
 * SPEC_E_CAPACITY for a store smaller than spec_model_bytes; SPEC_E_UNSUPPORTED for a
 * shape the kernels are not built for (bf16: head_dim 64 or 128, d_model and d_ffn
 * multiples of 128, vocab a multiple of 16; f32: even head_dim <= 128) or a device that
 * is not gfx950.  *out receives the handle. */
spec_status spec_model_create(const spec_model_cfg* cfg, void* store, size_t store_bytes,
                              spec_model** out);

/* Copy tensor `index` into the model's store, asynchronously on `stream`: `src` (device,
 * the layout below) must stay valid until the stream has passed this call.  Canonical
 * order of the spec_model_n_weights(cfg) tensors:
 *   embed [V,d], head [V,d], norm_f [d] (fp32),
 *   then per layer: norm1 [d] (fp32), wqkv [3d,d] (rows: q heads | k heads | v heads),
 *   wo [d,d], norm2 [d] (fp32), then SwiGLU: wgate [F,d], wup [F,d], wdown [d,F]
 *   or GELU: w1 [F,d], w2 [d,F].
 * Matrices and embeddings are bf16 for SPEC_DT_BF16 and fp32 for SPEC_DT_F32, row-major
 * [out, in].  A loader can stage one tensor at a time (peak memory: the store plus one
 * tensor).  SPEC_E_INVALID for a bad index or null pointer, SPEC_E_HIP if the copy cannot
 * be queued. */
spec_status spec_model_load_weight(spec_model* m, int index, const void* src, void* stream);

/* Free the handle (host memory only; the store stays the caller's). */
spec_status spec_model_destroy(spec_model* m);

/* ------------------------------------------------------------------ KV cache ------ */

/* Bytes of the KV arena for `batch` rows of up to `max_len` positions.  Layout:
 * [n_layers][batch][2 (K,V)][n_heads] head regions, then 256-byte aligned per-row
 * bookkeeping and, for bf16 models, the RoPE table (cos, sin of every position's
 * angles, fp64).  fp32 models: a head region is [max_len][head_dim] (natural order).
 * bf16 models: a head region holds roundup(max_len, 32) positions in the order the
 * attention's matrix-core products read them (K in blocks of 16 positions, V
 * transposed in blocks of 32); use spec_kv_import / spec_kv_export to move positions
 * in natural order. */
size_t spec_kv_bytes(const spec_model_cfg* cfg, int batch, int max_len);

/* Bind a cache to a caller-owned arena of at least spec_kv_bytes() (256-byte aligned)
 * and to a caller-owned int32 length vector len[batch] (device; the number of valid
 * positions of each row; the caller initialises it, usually to 0).  For bf16 models one
 * kernel is queued on `stream` that writes the RoPE table into the arena tail; the cache
 * is usable by later work on that stream (other streams must wait for it). */
spec_status spec_kv_create(const spec_model_cfg* cfg, int batch, int max_len, void* arena,
                           size_t arena_bytes, int32_t* len, void* stream, spec_kv** out);
spec_status spec_kv_destroy(spec_kv* kv);

/* Device pointer to the start of the arena's K/V element block. */
void* spec_kv_data(spec_kv* kv);

/* Write positions [0, n_pos) of every row, layer and head from `src` (device, natural
 * order [n_layers][batch][2][n_heads][n_pos][head_dim], the model's element type),
 * asynchronously on `stream`; for seeding a cache with precomputed contents, e.g. a
 * long prefilled context.  Lengths are not changed.  SPEC_E_INVALID for a null pointer
 * or n_pos outside [0, max_len]. */
spec_status spec_kv_import(spec_kv* kv, const void* src, int n_pos, void* stream);

/* Read positions [0, n_pos) into `dst` in the natural order of spec_kv_import. */
spec_status spec_kv_export(spec_kv* kv, void* dst, int n_pos, void* stream);

/* Roll back: len[b] <- min(len[b], max(new_len[b], 0)).  Entries past the new length
 * become stale and are overwritten by the next append.  [LENS] §2.1: drafts after the
 * first rejection are discarded. */
spec_status spec_kv_rollback(spec_kv* kv, const int32_t* new_len, void* stream);

/* ------------------------------------------------------------------ forward ------- */

/* Workspace bytes for spec_verify_forward / spec_draft_step with `batch` rows of up to
 * `max_rows` new tokens each, over a cache of `max_len` positions. */
size_t spec_workspace_bytes(const spec_model_cfg* cfg, int batch, int max_rows, int max_len);

/* The verify pass ([ZSM] "One pass can score many tokens" and "The algorithm"; [LENS]
 * §2.1 step 2; [GC] "How It Works" step 2): score n_tok[b] <= M new tokens per row at
 * positions len[b] .. len[b]+n_tok[b]-1 in ONE pass over the weights and the cache,
 * append their K/V and advance len[b] by n_tok[b].
 *   tokens  [B, M] int32 (row b uses its first n_tok[b] entries)
 *   n_tok   [B] int32 or NULL (= M for every row)
 *   logits  [B, M, V] fp32 out (rows j >= n_tok[b] are written as 0)
 *   row_status [B] int32 or NULL: OR-ed with SPEC_ROW_KV_OVERFLOW when
 *           len[b] + n_tok[b] > max_len (the row is then not appended and its logits
 *           are 0) and SPEC_ROW_BAD_TOKEN for a token id outside [0, V) (embedded as 0)
 *   ws      workspace of ws_bytes >= spec_workspace_bytes(cfg, B, M, kv max_len)
 * Used for the verify (n_tok = K+1), for draft steps (1 or 2) and for chunked prefill.
 * B <= the cache's batch, 1 <= M <= 64. */
spec_status spec_verify_forward(const spec_model* m, spec_kv* kv, const int32_t* tokens,
                                const int32_t* n_tok, int B, int M, float* logits,
                                int32_t* row_status, void* ws, size_t ws_bytes,
                                void* stream);

/* spec_verify_forward that also exports the residual stream and the rounded activations
 * that enter the residual updates, for parity checks of each half-layer against a
 * reference fed the same rows:
 *   resid    [2 * n_layers + 1, B * M, d] fp32 out: entry 0 the embedded rows, entry
 *            2l + 1 the rows after layer l's attention half (x + o W_o^T), entry 2l + 2
 *            after its FFN half (x + a W_down^T);
 *   q        [n_layers, B * M, d] out or NULL: each layer's rotated queries as attention
 *            takes them (bf16 for bf16 models, fp32 for f32 models);
 *   attn_out [n_layers, B * M, d] out or NULL: o of each layer (the attention output as
 *            the O product takes it: bf16 for bf16 models, fp32 for f32 models);
 *   ffn_act  [n_layers, B * M, d_ffn] out or NULL: a of each layer (the FFN activation as
 *            the down product takes it, same element type);
 *   rows j >= n_tok[b] of a sequence hold unspecified values.
 * Same arguments, results and errors as spec_verify_forward otherwise (resid NULL:
 * SPEC_E_INVALID). */
spec_status spec_verify_forward_trace(const spec_model* m, spec_kv* kv, const int32_t* tokens,
                                      const int32_t* n_tok, int B, int M, float* logits,
                                      int32_t* row_status, float* resid, void* q,
                                      void* attn_out, void* ffn_act, void* ws, size_t ws_bytes,
                                      void* stream);

/* One draft step ([ZSM] "The algorithm": the draft generates K tokens autoregressively;
 * [CANON] listing, draft loop; [LENS] §2.1 step 1): a forward of the draft model over
 * this step's input tokens, then x~_step ~ q_step drawn by inverse CDF with the
 * uniform U(seed, round, step, b, purpose 0) after the knobs (same transform as the
 * rule).  Input tokens: step 0 takes in_tok[b, 0..n_in[b]-1] (in_tok [B,2], n_in [B]
 * in {1,2}: the draft's pending tokens); step s > 0 takes x_tilde[b, s-1].
 *   x_tilde  [B, K] int32, column `step` written
 *   q_logits [B, K, V] fp32, row `step` written (the draft logits at the last input)
 * row_status [B] int32 or NULL: OR-ed with SPEC_ROW_KV_OVERFLOW / SPEC_ROW_BAD_TOKEN as in
 * spec_verify_forward, and with SPEC_ROW_NONFINITE when the step's draft logits are not
 * all finite (x~_step is then the placeholder 0; the accept step emits nothing for the
 * row).
 * A step-0 call records the row's pre-round cache length for spec_accept_resample.
 * round_dev (device, NULL = use `round`): when set, the round number is read from
 * *round_dev at execution time, so a captured HIP graph of a whole round can be
 * replayed round after round (spec_accept_resample advances the counter). */
spec_status spec_draft_step(const spec_model* draft, spec_kv* dkv, const int32_t* in_tok,
                            const int32_t* n_in, int B, int K, int step,
                            const spec_sampling* knobs, uint64_t seed, uint64_t round,
                            const uint64_t* round_dev, int32_t* x_tilde, float* q_logits,
                            int32_t* row_status, void* ws, size_t ws_bytes, void* stream);

/* Verify-input assembly ([ZSM] "The algorithm": the target scores the context followed
 * by the drafts; [CANON] listing, target call over ctx and xs): tokens[b] =
 * [y_prev, x~_0 .. x~_{K-1}] with y_prev = pending[b, n_pending[b] - 1], the newest
 * committed token, which the target cache does not hold yet.
 *   pending [B, 2], n_pending [B] in {1, 2}, x_tilde [B, K]  ->  tokens [B, K+1] int32 */
spec_status spec_verify_tokens(const int32_t* pending, const int32_t* n_pending,
                               const int32_t* x_tilde, int B, int K, int32_t* tokens,
                               void* stream);

/* ------------------------------------------------------------------ the rule ------ */

/* Workspace bytes for spec_accept_resample with B rows and K drafts. */
size_t spec_accept_workspace_bytes(int B, int K);

/* The modified rejection-sampling step for every row, evaluated data-parallel over
 * positions with counter-based uniforms so that it equals the left-to-right walk:
 *   accept x~_j  <=>  U(seed,round,j,b,1) * q_j(x~_j) < p_j(x~_j)
 *     ([ZSM] "The algorithm", acceptance eq.; [CANON] eq. alpha(x); [LENS] §2.3;
 *      written without division, equal to u < min(1, p/q) whenever q > 0)
 *   a = number of leading accepts;
 *   a < K : y ~ norm(max(0, p_a - q_a)) by inverse CDF with U(seed,round,a,b,2)
 *     ([CANON] residual eq.; [LENS] §2.3 eq. p'); an all-zero residual samples p_a
 *     instead (SPEC_ROW_RESIDUAL_EMPTY)
 *   a = K : bonus y ~ p_K with U(seed,round,K,b,2) ([LENS] §2.1 step 3; [GC] step 4)
 *   out_tok[b] = x~_0..x~_{a-1}, y (then -1 padding); n_out[b] = a + 1 in [1, K+1]
 *     ([LENS] §2.1; [NOTE] "At least one token per loop").
 * Uniforms: Philox4x64-10 (Salmon et al., SC'11), key (seed, 0), counter
 * (round, j, b, purpose), u = top 24 bits of word 0 times 2^-24.
 * Inverse CDF: smallest token id i whose running sum (token-id order) exceeds u * S.
 *   p_logits [B, K+1, V] fp32, q_logits [B, K, V] fp32, x_tilde [B, K] int32
 *   out_tok [B, K+1] int32 out, n_out [B] int32 out, row_status [B] int32 out (set)
 * Optional state updates (NULL = skip):
 *   tkv: target cache after the verify appended K+1 rows: len <- pre-verify len + a+1
 *   dkv: draft cache after K draft steps: len <- target's new len if a < K, unchanged
 *        if a = K
 *   pending [B, 2] / n_pending [B]: the draft's pending tokens for the next round:
 *        [y] if a < K, [x~_{K-1}, y] if a = K
 * round_dev (device, NULL = use `round`): when set, the round number is read from
 *   *round_dev and *round_dev is incremented by one after the rows are decided.
 * A row with NONFINITE, BAD_TOKEN or KV_OVERFLOW emits nothing (n_out = 0) and its
 * caches are restored to their pre-round lengths.
 * V <= 32768 (else SPEC_E_UNSUPPORTED); 1 <= K <= 16.
 * `debug` (NULL = none) exports intermediate values for parity checks:
 *   debug[0] float* p_probs [B, K+1, V], debug[1] float* q_probs [B, K, V],
 *   debug[2] int32_t* accept [B, K], debug[3] int32_t* cand [B, K+1]
 *   (cand[j] = the token position j would emit if it were the first rejection, or the
 *   bonus token for j = K; -1 where not evaluated). */
spec_status spec_accept_resample(const float* p_logits, const float* q_logits,
                                 const int32_t* x_tilde, int B, int K, int V,
                                 const spec_sampling* knobs, uint64_t seed, uint64_t round,
                                 uint64_t* round_dev, int32_t* out_tok, int32_t* n_out,
                                 int32_t* row_status,
                                 spec_kv* tkv, spec_kv* dkv, int32_t* pending,
                                 int32_t* n_pending, void* const* debug, void* ws,
                                 size_t ws_bytes, void* stream);

/* spec_accept_resample for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and results without debug exports or workspace.  Its scratch is a 64 KB
 * device array inside the library (each GPU holds its own copy until the process ends),
 * so spec_accept_workspace_bytes(B, K) must not exceed 65536 (else SPEC_E_CAPACITY; e.g.
 * B <= 256 at K <= 16).  Calls that overlap on one GPU (concurrent streams) share that
 * array and race: issue them on one stream.  The first call on a device looks up the
 * array's device address (SPEC_E_HIP if that fails). */
spec_status spec_accept_resample_static(const float* p_logits, const float* q_logits,
                                        const int32_t* x_tilde, int B, int K, int V,
                                        const spec_sampling* knobs, uint64_t seed,
                                        uint64_t round, uint64_t* round_dev, int32_t* out_tok,
                                        int32_t* n_out, int32_t* row_status, spec_kv* tkv,
                                        spec_kv* dkv, int32_t* pending, int32_t* n_pending,
                                        void* stream);

/* ------------------------------------------------------------------ measurement --- */

/* Kernel timing for measurement.  While enabled, HIP events are recorded on the launch
 * stream immediately before and after every weight-GEMM launch and every attention
 * launch (split-KV kernel + merge) of spec_verify_forward / spec_draft_step.
 * spec_timing_read waits for the recorded events (the one call that waits for the
 * device), returns the summed elapsed times (ms) and launch counts since the last read,
 * and clears them.  Events are created on first use and reused; timing adds the event
 * records to the stream. */
spec_status spec_timing_enable(int on);
spec_status spec_timing_read(double* gemm_ms, int* gemm_launches, double* attn_ms,
                             int* attn_launches);

/* ------------------------------------------------------------------ misc ---------- */

const char* spec_status_str(int status);
int spec_last_hip_error(void); /* hipError_t of the last failed launch (0 = none) */
int spec_abi_version(void);    /* bumped on any incompatible change to this header  */

#ifdef __cplusplus
}
#endif
#endif /* SPECDEC_H */
