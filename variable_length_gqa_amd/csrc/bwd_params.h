// Launch parameters shared by the C ABI (host) and the backward kernels.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "fwd_params.h"

namespace vlgqa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;     // workspace: rowsum(dout * o) per (row, head), f32, same layout as lse
  void* dq;
  void* dk;
  void* dv;
  // packed layout: sequence b spans rows cu[b] .. cu[b+1]; null for dense
  const int32_t* cu_q;
  const int32_t* cu_k;
  // strides in elements: batch, row (token), head
  int64_t q_bs, q_rs, q_hs;  // q, o, dout, dq
  int64_t k_bs, k_rs, k_hs;  // k, v, dk, dv
  int64_t l_bs, l_rs, l_hs;  // lse, delta
  int32_t batch, heads, kv_heads, group;
  int32_t seqlen_q, seqlen_k;  // dense extents (per-sequence lengths come from cu_* when given)
  int32_t causal, window;
  int32_t max_seqlen_q, max_seqlen_k;
  // rowsum kernel: rows are (b, r, h) with b < d_batch, r < d_rows
  int32_t d_batch, d_rows;
  // dK/dV partial sums (f32) when the query heads of a group are split over
  // n_split workgroups: [2 (dk, dv)][n_split][kp_rows][kv_heads][D], summed by
  // the reduction kernel; kp_rows = total_k (packed) or batch * seqlen_k
  float* part;
  int32_t kp_rows;
  // filled by plan_bwd:
  int32_t n_split;    // workgroups per (kv head, key tile): 1 or 2
  int32_t n_ktiles;   // ceil(max_seqlen_k / 128): key tiles of the dK/dV kernel
  int32_t stream_major;  // dK/dV block order: one stream's key tiles together (1) or
                         // the streams' first key tiles first (0)
  int32_t n_qtiles;   // ceil(max_seqlen_q / 128): query tiles of the dQ kernel
  float score_mul;    // log2(e) / sqrt(D): scores into the log2 domain
  float scale;        // 1 / sqrt(D)
  // multipliers of dP = dO.V^T and of the stored dq, dk, dv (16-bit inputs:
  // 1, 1/sqrt(D), 1/sqrt(D), 1; E4M3 inputs: the per-tensor scales folded in)
  float dp_mul, dq_mul, dk_mul, dv_mul;
  // E4M3 path: q8, k8, v8, do8 are the codes, the operands of the products
  // S = Q K^T and dP = dO V^T on the FP8 matrix cores; q, k and dout point at
  // bf16 copies of the codes (exact, unscaled, made by the widening kernel)
  // for the transposed operands of the dK, dQ and dV accumulations; delta is
  // taken from the codes of dout and o times delta_mul; dq, dk, dv are E4M3
  // codes (dk, dv always through the f32 partials)
  int32_t e4m3;
  float delta_mul;
  const void* q8;
  const void* k8;
  const void* v8;
  const void* do8;
  // bf16 copies (in the workspace) and their element counts
  void* wq;
  void* wk;
  void* wdo;
  int64_t n_q, n_k;   // elements of q (= dout) and of k
};

// float32 workspace of the backward: the row planes (LSE log2 e, delta), the
// dk / dv partials, and for E4M3 inputs the bf16 copies of q, dout and k;
// returns the offsets of the parts in floats
struct BwdWorkspace {
  int64_t part, wide, total;
};
BwdWorkspace bwd_workspace(int64_t rows, int64_t keys, int64_t heads, int64_t kv_heads,
                           int64_t head_dim, bool e4m3);

bool plan_bwd(BwdParams& p, int head_dim);

hipError_t launch_bwd(const BwdParams& p, int elem, int head_dim, hipStream_t stream);

}  // namespace vlgqa
