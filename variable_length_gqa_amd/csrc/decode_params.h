// Launch parameters of the split-KV decode path (decode.hip).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "fwd_params.h"

namespace vlgqa {

struct DecParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* ws;   // partials: [n_bk][n_parts][32][D] O, then [n_bk][n_parts][32][2] (m, l)
  // dense strides in elements: batch, head, row
  int64_t q_bs, q_hs, q_rs;  // q and out
  int64_t k_bs, k_hs, k_rs;  // k and v (head stride = capacity * D)
  int64_t l_bs, l_hs, l_rs;
  int32_t kv_heads, group, seqlen_q, kv_len;
  int32_t causal, window;
  int32_t n_bk;     // batch * kv_heads
  int32_t n_parts;  // key slices (one wave each) per (batch, kv head)
  float score_mul;  // log2(e) / sqrt(D)
  float out_mul;
};

// key slices per (batch, kv head), and the workspace they need (floats)
int64_t decode_parts(int64_t batch, int64_t kv_heads, int64_t head_dim, int64_t kv_len);
int64_t decode_workspace_floats(int64_t batch, int64_t kv_heads, int64_t head_dim,
                                int64_t kv_len);
hipError_t launch_decode(const DecParams& p, int elem, int head_dim, hipStream_t stream);

// floats in the library-owned decode scratch (16 MiB per GPU)
constexpr int64_t kDecodeScratchFloats = (int64_t)4 << 20;
// device address of the current GPU's copy of that scratch (looked up once per
// device); no allocation
hipError_t decode_scratch(float** ptr);

}  // namespace vlgqa
