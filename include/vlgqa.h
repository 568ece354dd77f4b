/*
 * vlgqa.h -- C ABI of the MI355X (gfx950) attention library.
 *
 * Forward entry points: the packed variable-length forward, the dense forward
 * with a KV-capacity stride and sliding window, and the FP8 dense forward; and
 * the packed and dense backward passes (declared further down).  The
 * forwards compute, for every query row i of every (sequence, query head h):
 *
 *     kv_head = h / (num_heads / num_kv_heads)              (GQA, no repeat)
 *     s_j     = scale * <q_i, k_j>,   scale = 1/sqrt(head_dim)
 *     O_i     = sum_{j visible} softmax(s)_j v_j,   LSE_i = ln sum_{j visible} exp(s_j)
 *
 * visible: causal -> j <= i + (Lk - Lq)  (queries are the newest Lq positions);
 *          window W > 0 -> additionally j >= i + (Lk - Lq) - W + 1 (the W most
 *          recent keys; a window implies the causal bound).
 * A row that sees no key gets O = 0 and LSE = -inf.
 *
 * Conventions shared by all entry points
 *   - Every tensor pointer is DEVICE memory owned by the caller; inputs are
 *     only read.  out and lse are written for every valid row and nothing
 *     else (rows of other sequences, padding and capacity tails are left
 *     untouched).
 *   - Tensors are contiguous in the layouts stated per entry point; extents
 *     that a tensor's shape would carry are passed as scalars.
 *   - The library never synchronises: kernels are enqueued on `hip_stream`
 *     (a hipStream_t; NULL = the null stream) and the call returns at once.
 *     Buffers must stay alive until the stream work completes.  It allocates
 *     and frees nothing, except the FP8 forward's stream-ordered scratch block
 *     (see flash_attention_fwd_fp8).
 *   - The launch runs on the device `hip_stream` belongs to (the current
 *     device for the null, legacy and per-thread streams), and the pointers
 *     must be that device's memory.  While a call runs it makes that device
 *     current and restores the caller's current device before returning, so
 *     the library's per-device state (claim counters, the decode's static
 *     scratch, the FP8 scratch pool) is always the launch device's.
 *   - Forward launches hand out their last items at run time (faster XCDs
 *     take more of them) from a claim counter the library owns: one 4-byte
 *     device counter per (device, stream) a forward has been launched on, zero
 *     when the library loads, for up to 64 streams per device.  Launches on
 *     one stream run in order and so never use a counter at the same time;
 *     the host keeps each counter's running value (a mutex orders the
 *     launches of several host threads on one stream).  A launch on a stream
 *     that is being captured into a graph, on hipStreamPerThread, or on a
 *     65th stream uses the static order instead; results are identical
 *     either way.  A new stream that receives a destroyed stream's handle
 *     continues its counter: hipStreamDestroy waits for the stream's pending
 *     work, so no earlier launch is still claiming.
 *   - Base pointers must be 16-byte aligned.
 *   - Return value: VLGQA_OK, or an error code; no exception crosses the ABI.
 *     vlgqa_last_error() then gives "argument: reason" (thread-local, valid
 *     until the next call on the same thread).  Argument errors are detected
 *     on the host before any HIP call is made.
 *   - Empty problems (no batch, no query rows, no heads' work) return VLGQA_OK
 *     without launching anything.
 *   - Size limit: the kernels address one sequence's rows (of one head, in
 *     the dense layouts) through 32-bit byte offsets, so (length + 128) x
 *     (row stride in bytes) must stay below 4 GiB for q and for k/v (packed:
 *     the row stride is heads x head_dim elements, e.g. 262,016 tokens at 64
 *     bf16 heads of 128); longer sequences return EINVAL.  The FP8 entry
 *     points count k/v (forward: v) at 2 bytes per element: they read 16-bit
 *     copies of the codes.
 */
#ifndef VLGQA_H
#define VLGQA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vlgqa_status {
  VLGQA_OK = 0,
  VLGQA_EINVAL = 1,        /* a bad argument (mirrors InvalidArgument / InvalidShape) */
  VLGQA_EUNSUPPORTED = 2,  /* head_dim or dtype not compiled (mirrors UnsupportedOperation) */
  VLGQA_EHIP = 3           /* the HIP runtime reported a launch failure */
};

/* storage dtypes of q, k, v and out (LSE is always float32) */
enum vlgqa_dtype { VLGQA_F32 = 0, VLGQA_F16 = 1, VLGQA_BF16 = 2 };

/*
 * Packed variable-length forward.
 * boostr 0.2.0, src/ops/traits/attention/varlen_attention.rs,
 * VarLenAttentionOps::varlen_attention_fwd (layout contract, GQA key/value
 * head mapping, cumulative sequence lengths; returns output and logsumexp).
 *
 *   q            [total_q, num_heads, head_dim]      dtype
 *   k, v         [total_k, num_kv_heads, head_dim]   dtype
 *   cu_seqlens_q [batch_size + 1] int32, device: sequence b owns query rows
 *                cu_seqlens_q[b] .. cu_seqlens_q[b+1]; cu[0] = 0, non-decreasing,
 *                cu[batch_size] = total_q.  Likewise cu_seqlens_k for k/v.
 *                The contents are trusted (they are device memory).
 *   max_seqlen_q / max_seqlen_k  upper bounds of the per-sequence lengths
 *                (they size the launch).  EINVAL when total_q > batch_size *
 *                max_seqlen_q (or likewise for k): some sequence must be longer.
 *                A sequence longer than max_seqlen_q that this test cannot see
 *                gets its rows beyond ceil(max_seqlen_q / 128) * 128 written as
 *                NaN (O and LSE), never left unwritten.
 *   causal       0/1.  There is no window on this entry point.
 *   out          [total_q, num_heads, head_dim]      dtype
 *   lse          [total_q, num_heads]                float32, natural log
 *
 * Errors: EINVAL for num_heads % num_kv_heads != 0, negative extents, null or
 * misaligned pointers with non-empty extents; EUNSUPPORTED for head_dim not in
 * {64, 128} or an unknown dtype.
 */
int varlen_attention_fwd(const void* q, const void* k, const void* v,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int64_t total_q, int64_t total_k, int64_t batch_size,
                         int64_t num_heads, int64_t num_kv_heads,
                         int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t head_dim,
                         int causal, int dtype,
                         void* out, float* lse, void* hip_stream);

/*
 * Dense forward over a KV buffer that may be longer than the attended part.
 * boostr, src/ops/traits/attention/flash.rs, FlashAttentionOps::flash_attention_fwd
 * (layout contract, GQA support, sliding window, kv_seq_len).
 *
 *   q      [batch, num_heads, seqlen_q, head_dim]        dtype
 *   k, v   [batch, num_kv_heads, kv_capacity, head_dim]  dtype; kv_capacity is
 *          the dim-2 memory stride
 *   kv_seq_len  number of leading key positions attended (0 <= n <= kv_capacity),
 *          or < 0 for "None" = kv_capacity.  Positions n .. kv_capacity-1 are
 *          never read.
 *   causal 0/1;  window_size 0 = off, W > 0 = only the W most recent keys.
 *   out    [batch, num_heads, seqlen_q, head_dim]        dtype
 *   lse    [batch, num_heads, seqlen_q]                  float32
 *
 * Errors: EINVAL as above, plus kv_seq_len > kv_capacity and window_size < 0;
 * EUNSUPPORTED as above.
 */
int flash_attention_fwd(const void* q, const void* k, const void* v,
                        int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                        int64_t seqlen_q, int64_t kv_capacity, int64_t head_dim,
                        int causal, int64_t window_size, int64_t kv_seq_len,
                        int dtype, void* out, float* lse, void* hip_stream);

/*
 * Decode-shaped dense forward over a KV cache (split-KV).  Same operation,
 * layouts, masks and results as flash_attention_fwd (boostr, src/ops/traits/
 * attention/flash.rs, FlashAttentionOps::flash_attention_fwd, "kv_seq_len":
 * a full-capacity cache buffer is attended up to n positions without
 * narrowing), for a few new queries per sequence: it requires
 * seqlen_q * (num_heads / num_kv_heads) <= 32.  The keys of each (batch, kv
 * head) are split into slices that run in parallel; each slice writes an
 * unnormalised partial output with its softmax maximum and denominator to the
 * workspace, and a second kernel merges the slices by their log-sum-exp.
 *
 *   workspace  caller-allocated float32 scratch, 16-byte aligned, of at least
 *              vlgqa_decode_workspace_floats(batch, num_kv_heads, head_dim, n)
 *              floats, n = the attended length.  That size never decreases
 *              as n grows, so a workspace sized for kv_capacity serves every
 *              n.  Contents on return are unspecified; calls sharing one
 *              workspace are ordered by their stream, concurrent calls need
 *              separate workspaces.
 *   workspace_floats  its size in floats.
 *   dtype      VLGQA_BF16 or VLGQA_F16 (f32: EUNSUPPORTED).
 *
 * Errors: as flash_attention_fwd, plus EINVAL for seqlen_q * group > 32 or a
 * workspace that is too small or null / misaligned.
 */
int flash_attention_decode(const void* q, const void* k, const void* v,
                           int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                           int64_t seqlen_q, int64_t kv_capacity, int64_t head_dim,
                           int causal, int64_t window_size, int64_t kv_seq_len,
                           int dtype, void* out, float* lse, float* workspace,
                           int64_t workspace_floats, void* hip_stream);

/*
 * flash_attention_decode without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (minus the workspace),
 * kernels, results and errors as flash_attention_decode; the slices' partials
 * go to a library-owned static device array of 4194304 floats (16 MiB) per
 * GPU, held until the process ends.  The call allocates nothing (no hipMalloc,
 * no library routine that allocates): the array's device address is looked up
 * once per device on the first call there.
 *
 *   Limit: vlgqa_decode_workspace_floats(batch, num_kv_heads, head_dim, n)
 *   must not exceed 4194304; beyond it the call returns EINVAL ("batch: ...")
 *   without launching.  (About 2.7 M floats for any batch * num_kv_heads up to
 *   640 at head_dim 128, 1280 at 64.)
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (different streams, or different host threads) race and must be
 *   ordered by the caller, e.g. on one stream.  EHIP if the array's address
 *   cannot be found on the launch device (the device of hip_stream).
 */
int flash_attention_decode_noalloc(const void* q, const void* k, const void* v,
                                   int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                                   int64_t seqlen_q, int64_t kv_capacity, int64_t head_dim,
                                   int causal, int64_t window_size, int64_t kv_seq_len,
                                   int dtype, void* out, float* lse, void* hip_stream);

/* Workspace floats flash_attention_decode needs for an attended length kv_len
 * (-1 for a negative argument).  Host-only arithmetic. */
int64_t vlgqa_decode_workspace_floats(int64_t batch, int64_t num_kv_heads, int64_t head_dim,
                                      int64_t kv_len);

/*
 * FP8 (OCP E4M3, "e4m3fn": max 448, no infinities) dense forward.
 * boostr, src/ops/traits/attention/flash.rs,
 * FlashAttentionOps::flash_attention_fwd_fp8 (per-tensor scales, FP32
 * accumulation).
 *
 *   q      [batch, num_heads, seqlen_q, head_dim]     uint8 E4M3 codes
 *   k, v   [batch, num_kv_heads, seqlen_k, head_dim]  uint8 E4M3 codes
 *   q_scale, k_scale, v_scale  dequantisation: real value = code value * scale
 *   o_scale                    output quantisation: out = E4M3(O / o_scale),
 *                              round to nearest even, saturating at +-448
 *   out    [batch, num_heads, seqlen_q, head_dim]     uint8 E4M3 codes
 *   lse    [batch, num_heads, seqlen_q]               float32, over the scaled
 *                              scores q_scale*k_scale*<q8,k8>/sqrt(head_dim)
 *
 * Two launches on hip_stream: an exact bf16 copy of the V codes (every E4M3
 * value is a bf16 value), then the attention kernel.  The copy lives in a
 * block of 2 * batch * num_kv_heads * seqlen_k * head_dim bytes taken, in
 * stream order, from a device memory pool the library creates per device and
 * keeps until the process ends (it holds on to what it has reserved, so only
 * a first call, or a larger one, reserves device memory); the block is given
 * back on hip_stream after the kernel.
 *
 * Errors: EINVAL as above, plus any scale that is not finite and positive;
 * EUNSUPPORTED for head_dim not in {64, 128}; EHIP when the scratch block
 * cannot be had.
 */
int flash_attention_fwd_fp8(const void* q, const void* k, const void* v,
                            int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                            int64_t seqlen_q, int64_t seqlen_k, int64_t head_dim,
                            int causal, float q_scale, float k_scale, float v_scale,
                            float o_scale, void* out, float* lse, void* hip_stream);

/*
 * Backward passes.  Gradients of the forward above for a loss whose gradient
 * with respect to O is dout:
 *
 *     P_ij  = exp(scale q_i.k_j - LSE_i)          (visible pairs; recomputed)
 *     dv_j  = sum_i P_ij dout_i,   dS_ij = P_ij (dout_i.v_j - delta_i),
 *     delta_i = dout_i.out_i,      dq_i = scale sum_j dS_ij k_j,
 *     dk_j  = scale sum_i dS_ij q_i,
 *
 * with dk and dv of a kv head summed over the num_heads / num_kv_heads query
 * heads that share it.  out and lse are the forward's results for the same
 * inputs (lse natural log, -inf for a row with no visible key).  The masks
 * are those of the forward.  dtype: VLGQA_BF16 or VLGQA_F16 (f32 and FP8 are
 * not compiled: EUNSUPPORTED); f32 accumulation, gradients stored in dtype.
 *
 * workspace: caller-allocated float32 scratch, 16-byte aligned, of
 *     vlgqa_bwd_workspace_floats(rows, keys, num_heads, num_kv_heads, head_dim, 0)
 *   = round_up(2 * rows * num_heads, 4) + 4 * keys * num_kv_heads * head_dim
 * floats, rows = total_q, keys = total_k (packed) or rows = batch * seqlen_q,
 * keys = batch * seqlen_k (dense).  On return its first part holds
 * LSE * log2(e) (+inf for rows with no visible key) and then delta,
 * head-major ([num_heads][total_q], dense [batch][num_heads][seqlen_q]); the
 * rest holds f32 partial sums of dk and dv.  It is required whenever the call has work.
 * Calls that share a workspace on one stream are ordered by the stream;
 * concurrent calls need separate workspaces.
 * dq, dk, dv are written in full (zero for rows / keys that take part in no
 * visible pair); padding outside the sequences is not written.
 */

/*
 * Packed variable-length backward.
 * boostr 0.2.0, src/ops/traits/attention/varlen_attention.rs,
 * VarLenAttentionOps::varlen_attention_bwd (full GQA: dk, dv shaped like k, v;
 * returns dq, dk, dv).
 *
 *   dout, out, q, dq  [total_q, num_heads, head_dim]      dtype
 *   k, v, dk, dv      [total_k, num_kv_heads, head_dim]   dtype
 *   lse               [total_q, num_heads]                float32
 *   cu_seqlens_q/k, max_seqlen_q/k, causal: as in varlen_attention_fwd
 *   (the same EINVAL when total_q / total_k exceed batch_size times the bound;
 *   a sequence longer than its bound that the check cannot see leaves its
 *   gradient rows beyond the bound unwritten: a broken caller promise).
 *
 * Errors: as varlen_attention_fwd, plus EUNSUPPORTED for a dtype other than
 * VLGQA_BF16 / VLGQA_F16.
 */
int varlen_attention_bwd(const void* dout, const void* q, const void* k, const void* v,
                         const void* out, const float* lse,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int64_t total_q, int64_t total_k, int64_t batch_size,
                         int64_t num_heads, int64_t num_kv_heads,
                         int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t head_dim,
                         int causal, int dtype, void* dq, void* dk, void* dv,
                         float* workspace, void* hip_stream);

/*
 * Dense backward.  boostr, src/ops/traits/attention/flash.rs,
 * FlashAttentionOps::flash_attention_bwd (gradients with the shapes of the
 * inputs; causal and sliding window as in the forward).  The method takes no
 * kv_seq_len: all seqlen_k keys of k and v are attended.
 *
 *   dout, out, q, dq  [batch, num_heads, seqlen_q, head_dim]     dtype
 *   k, v, dk, dv      [batch, num_kv_heads, seqlen_k, head_dim]  dtype
 *   lse               [batch, num_heads, seqlen_q]               float32
 *
 * Errors: as flash_attention_fwd, plus EUNSUPPORTED for a dtype other than
 * VLGQA_BF16 / VLGQA_F16.
 */
int flash_attention_bwd(const void* dout, const void* q, const void* k, const void* v,
                        const void* out, const float* lse,
                        int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                        int64_t seqlen_q, int64_t seqlen_k, int64_t head_dim,
                        int causal, int64_t window_size, int dtype,
                        void* dq, void* dk, void* dv, float* workspace, void* hip_stream);

/*
 * FP8 (OCP E4M3) dense backward.  boostr, src/ops/traits/attention/flash.rs,
 * FlashAttentionOps::flash_attention_bwd_fp8 (per-tensor dequantisation scales
 * for the inputs and for the forward output, which serves the preprocessing
 * step; quantisation scales for the gradients).
 *
 *   dout, out, q  [batch, num_heads, seqlen_q, head_dim]      uint8 E4M3 codes
 *   k, v          [batch, num_kv_heads, seqlen_k, head_dim]   uint8 E4M3 codes
 *   lse           [batch, num_heads, seqlen_q]                float32, natural
 *                 log, over the scaled scores (flash_attention_fwd_fp8's lse)
 *   q/k/v/do/o_scale  real value = code value * scale
 *   dq/dk/dv_scale    gradient codes = E4M3(g / scale), round to nearest even,
 *                     saturating at +-448
 *   dq [.., seqlen_q, ..], dk, dv [.., seqlen_k, ..]          uint8 E4M3 codes
 *
 * The gradients are those of flash_attention_bwd on the dequantised inputs
 * (scale 1/sqrt(head_dim); causal or no mask: this method takes no window),
 * with delta_i = dout_i . out_i taken from the stored output.  S = q k^T and
 * dP = dout v^T run on the FP8 matrix cores from the codes; P and dS are
 * rounded to bf16 for the dv, dk and dq products; f32 accumulation.
 *
 * workspace: float32, 16-byte aligned, workspace_floats >=
 * vlgqa_bwd_workspace_floats(batch * seqlen_q, batch * seqlen_k, num_heads,
 * num_kv_heads, head_dim, 1): the 16-bit layout followed by bf16 copies of the
 * codes of q, dout and k.  Contents on return are unspecified.
 *
 * Errors: EINVAL for a scale that is not finite and positive, scale products
 * outside the f32 range, a workspace that is too small, and as
 * flash_attention_bwd; EUNSUPPORTED for head_dim not in {64, 128}.
 */
int flash_attention_bwd_fp8(const void* dout, const void* q, const void* k, const void* v,
                            const void* out, const float* lse,
                            int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                            int64_t seqlen_q, int64_t seqlen_k, int64_t head_dim, int causal,
                            float q_scale, float k_scale, float v_scale, float do_scale,
                            float o_scale, float dq_scale, float dk_scale, float dv_scale,
                            void* dq, void* dk, void* dv, float* workspace,
                            int64_t workspace_floats, void* hip_stream);

/* Workspace floats of the backward entry points (e4m3 = 1: the FP8 form),
 * for rows query rows and keys key rows in total (-1 for a negative
 * argument).  Host-only arithmetic. */
int64_t vlgqa_bwd_workspace_floats(int64_t rows, int64_t keys, int64_t num_heads,
                                   int64_t num_kv_heads, int64_t head_dim, int e4m3);

/*
 * Packing of padded batches into the varlen layout.
 * boostr 0.2.0, src/ops/traits/attention/varlen_attention.rs: sequences of
 * different lengths are packed into one buffer instead of being padded, and
 * "Cumulative sequence lengths": cu_seqlens[0] = 0, cu_seqlens[i] = sum of
 * the lengths of sequences 0..i-1 (the CSR offsets that boostr's MoE dispatch
 * builds as a cumulative sum with a leading zero).  Pure data movement; rows
 * are opaque bytes, so any dtype and head layout works.
 */

/*
 * cu_seqlens [batch_size + 1] int32 (device) from lengths [batch_size] int32
 * (device): the exclusive prefix sum followed by the total.  The lengths are
 * trusted device memory: they must be non-negative with a sum that fits
 * int32.  Errors: EINVAL for a negative batch_size or a null / misaligned
 * pointer (lengths may be null when batch_size is 0).
 */
int vlgqa_cu_seqlens(const int32_t* lengths, int64_t batch_size, int32_t* cu_seqlens,
                     void* hip_stream);

/*
 * Pack: packed row cu_seqlens[b] + s  <-  padded row (b, s), for every s <
 * length_b = cu_seqlens[b+1] - cu_seqlens[b].
 *   padded   [batch_size, max_seqlen, row_bytes]  (a row = one token's heads x
 *            head_dim elements; row_bytes a multiple of 16)
 *   packed   [total, row_bytes], total = cu_seqlens[batch_size]
 *   cu_seqlens  device int32, trusted: non-decreasing, cu[0] = 0, each length
 *            <= max_seqlen.
 * Padding rows are not read; rows of packed past total are not written.
 * Errors: EINVAL for negative extents, total > INT32_MAX, row_bytes not a
 * positive multiple of 16, null or misaligned pointers with work to do.
 */
int vlgqa_pack(const void* padded, const int32_t* cu_seqlens, int64_t batch_size,
               int64_t max_seqlen, int64_t row_bytes, int64_t total, void* packed,
               void* hip_stream);

/*
 * Unpack: padded row (b, s) <- packed row cu_seqlens[b] + s for s < length_b,
 * zero bytes for length_b <= s < max_seqlen.  Every padded row is written.
 * Same layouts and errors as vlgqa_pack.
 */
int vlgqa_unpack(const void* packed, const int32_t* cu_seqlens, int64_t batch_size,
                 int64_t max_seqlen, int64_t row_bytes, void* padded, void* hip_stream);

/* "argument: reason" for the last non-OK return on this thread ("" if none). */
const char* vlgqa_last_error(void);

/* Library version string. */
const char* vlgqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VLGQA_H */
