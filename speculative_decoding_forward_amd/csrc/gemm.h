// Argument block and launchers of the weight GEMMs (defined in gemm.hip).  The GEMM
// kernels compile from gemm.hip, this header and common.h alone.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specdec {

// fused bf16 GEMM epilogues
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_QKV_ROPE = 2, EPI_SWIGLU = 3, EPI_GELU = 4 };

struct GemmArgs {
  const uint16_t* A;  // [R, K] bf16 activations
  int lda;
  const uint16_t* W;  // packed column tiles (see the packed layout in gemm.hip)
  int N1;             // SWIGLU: gate/up width F (output row stride); else N
  int R, N, K, mode;
  int ntiles;  // column tiles (set by the launcher)
  float* C;  // STORE: logits [R, N]; RESID: Y [R, N], added to the residual stream later
  int ldc;
  const int32_t* ntok_eff;  // [B] tokens per sequence (rows past it are padding)
  int M;                    // rows per sequence
  // QKV_ROPE
  const int32_t* pos0;
  int d, hd;
  const double* rope_rows;  // [R][hd/2][2] (cos, sin) of each row's rotation angles
  uint16_t* q_out;
  uint16_t* kc;
  uint16_t* vc;
  size_t row_stride, head_stride;
  int max_len;
  // SWIGLU / GELU
  uint16_t* act_out;
  const uint16_t* zeros;  // >= 16 zero bytes (device)
  // RMS-normalised input (QKV_ROPE, SWIGLU, GELU, STORE): A = bf16(x * g) of the rows and
  // ss_in [R][ss_np] the partial sums of x^2 over 16-column groups; the product row r is
  // scaled by 1 / sqrt(sum_p ss_in[r][p] / K + eps).  NULL: no scaling.
  const float* ss_in;
  int ss_np;
  float eps;
  int ss_rows;  // rows of ss_in the epilogue stages in LDS at once (set by the launcher)
  // RESID: x [R, N] += Y; h_out [R, N] = bf16(x * gain) (the next normalised product's
  // input) or, when h_out is NULL, xg_out = x * gain in fp32 (act32_index order: the
  // input of launch_norm_pack), and ss_out [R][N/16] the partial sums of squares per
  // 16-column tile
  float* x;
  const float* gain;
  uint16_t* h_out;
  float* xg_out;
  float* ss_out;
  // RESID at 2-8 row tiles (k_gemm_sk): fp32 slot partials [ntiles][4][row tiles][64
  // lanes][4] and completion counters [ntiles / 4] kSkCounterStride words apart, zero at
  // launch (the last workgroup of a group resets its counter); NULL: that kernel is not used
  float* sk_part;
  unsigned* sk_counters;
};
constexpr int kSkCounterStride = 32;  // 128 bytes between completion counters

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
// h = bf16(xg * s_r) in the packed bf16 order for R rows of width K (xg in act32_index
// order, s_r = 1 / sqrt(sum of the partial sums ss [R][K/16] / K + eps)).  With len, the
// pass also ends the forward's row bookkeeping: len[b] += ntok_eff[b] for each sequence b
// of M rows.
hipError_t launch_norm_pack(const float* xg, const float* ss, int R, int K, float eps,
                            uint16_t* h, int32_t* len, const int32_t* ntok_eff, int M,
                            hipStream_t s);
enum { PACK_PLAIN = 0, PACK_QKV = 1, PACK_PAIR_LO = 2, PACK_PAIR_HI = 3 };
hipError_t launch_pack_bf16(const uint16_t* src, int K, int mode, int d, int hd, int ntiles,
                            uint16_t* dst, hipStream_t s);
hipError_t launch_gemm_f32(const float* A, const float* W, const float* W2, int N1, int R,
                           int N, int K, float* C, int accumulate, const float* rowscale,
                           const int32_t* ntok_eff, int M, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1);
int device_cus();  // compute units of the device

}  // namespace specdec
