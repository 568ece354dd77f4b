// Launch parameters shared by the C ABI (host) and the forward kernels.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace vlgqa {

// storage element kinds of q/k/v/out
enum Elem : int { E_F32 = 0, E_F16 = 1, E_BF16 = 2, E_E4M3 = 3 };

// keys per K/V tile and threads (4 waves) per workgroup
constexpr int kBlockN = 64;
constexpr int kThreads = 256;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  // packed layout: sequence b spans rows cu[b] .. cu[b+1]; null for dense
  const int32_t* cu_q;
  const int32_t* cu_k;
  // strides in elements: batch, row (token), head
  int64_t q_bs, q_rs, q_hs;
  int64_t k_bs, k_rs, k_hs;  // shared by v
  int64_t o_bs, o_rs, o_hs;
  int64_t l_bs, l_rs, l_hs;
  int32_t batch, heads, kv_heads, group;
  int32_t seqlen_q, seqlen_k;  // dense extents (per-sequence lengths come from cu_* when given)
  int32_t causal, window;
  int32_t max_seqlen_q;
  // filled by plan_fwd for the kernel that runs:
  int32_t heads_per_wg;  // query heads of one KV group handled by a workgroup (1 or 2)
  int32_t rows_per_wg;   // query rows per head per workgroup
  int32_t n_qtiles;      // ceil(max_seqlen_q / rows_per_wg)
  int32_t n_groups;      // n_qtiles * batch * kv_heads
  float score_mul;   // multiplies q.k into the log2 domain: scale * log2(e) [* q_scale * k_scale]
  float out_mul;     // multiplies the normalised output: 1, or v_scale / o_scale for E4M3
  // run-time hand-out of the last items of a launch (filled by launch_fwd):
  unsigned* ticket;    // this stream's claim counter, or null: every block's item by its index
  unsigned ticket_base;  // the counter's value when this launch starts
  int32_t n_static;    // slots per XCD handed out by block index
  int32_t n_tail;      // items after them (8 per remaining slot), claimed in order
  int32_t n_claim;     // blocks that claim one (the tail items plus spares)
};

// Number of workgroups the forward launch uses for these parameters.
inline int64_t fwd_grid_size(const FwdParams& p) {
  if (p.ticket) return 8 * (int64_t)p.n_static + p.n_claim;
  int64_t groups8 = ((int64_t)p.n_groups + 7) / 8 * 8;
  return groups8 * (p.group / p.heads_per_wg);
}

// Fills the launch-shape fields for the kernel that serves (elem, head_dim).
// Returns false when the problem does not fit one launch.
bool plan_fwd(FwdParams& p, int elem, int head_dim);

hipError_t launch_fwd(const FwdParams& p, int elem, int head_dim, hipStream_t stream);

}  // namespace vlgqa
