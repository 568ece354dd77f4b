// C ABI of the attention forward library: argument validation, layout
// description and dispatch.  The contract of every entry point is documented
// in include/vlgqa.h.  All checks run on the host before any HIP call, so a
// rejected call never touches the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <cstdint>
#include <string>

#include "bwd_params.h"
#include "decode_params.h"
#include "fwd_params.h"
#include "pack_api.h"
#include "vlgqa.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* arg, const std::string& reason) {
  g_last_error = std::string(arg) + ": " + reason;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// non-null and 16-byte aligned
int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(VLGQA_EINVAL, name, "null pointer");
  if (!aligned16(p)) return fail(VLGQA_EINVAL, name, "not 16-byte aligned");
  return VLGQA_OK;
}

int check_heads(int64_t num_heads, int64_t num_kv_heads) {
  if (num_heads <= 0) return fail(VLGQA_EINVAL, "num_heads", "must be positive");
  if (num_kv_heads <= 0) return fail(VLGQA_EINVAL, "num_kv_heads", "must be positive");
  if (num_heads % num_kv_heads != 0)
    return fail(VLGQA_EINVAL, "num_heads", "must be a multiple of num_kv_heads (GQA)");
  if (num_heads > (1 << 20)) return fail(VLGQA_EINVAL, "num_heads", "too large");
  return VLGQA_OK;
}

int check_head_dim(int64_t head_dim) {
  if (head_dim != 64 && head_dim != 128)
    return fail(VLGQA_EUNSUPPORTED, "head_dim", "only 64 and 128 are compiled");
  return VLGQA_OK;
}

// The kernels address the rows of one sequence (and head) through a buffer
// descriptor with 32-bit byte offsets, reading up to a tile past its end:
// rows + 128 rows of row_bytes each must stay below 4 GiB.
int check_span(int64_t rows, int64_t row_bytes, const char* name) {
  if (rows > 0 && (rows + 128) * row_bytes > (int64_t)UINT32_MAX)
    return fail(VLGQA_EINVAL, name,
                "one sequence's rows span 4 GiB or more (32-bit buffer offsets)");
  return VLGQA_OK;
}

// Makes the device that `stream` belongs to current for the guard's lifetime
// and restores the caller's current device afterwards.  The library's
// per-device state (the forward's claim counters, the decode's static scratch,
// the FP8 scratch pool) is looked up on the current device, so it must be the
// device the launch runs on.  The null, legacy and per-thread default streams
// belong to the current device.
class StreamDeviceGuard {
 public:
  explicit StreamDeviceGuard(hipStream_t stream) {
    int cur = -1;
    if ((err_ = hipGetDevice(&cur)) != hipSuccess) return;
    if (stream == nullptr || stream == hipStreamLegacy || stream == hipStreamPerThread) return;
    hipDevice_t dev = 0;
    if ((err_ = hipStreamGetDevice(stream, &dev)) != hipSuccess) return;
    if ((int)dev == cur) return;
    if ((err_ = hipSetDevice((int)dev)) != hipSuccess) return;
    prev_ = cur;
  }
  ~StreamDeviceGuard() {
    if (prev_ >= 0) (void)hipSetDevice(prev_);  // the device was current when the call began
  }
  StreamDeviceGuard(const StreamDeviceGuard&) = delete;
  StreamDeviceGuard& operator=(const StreamDeviceGuard&) = delete;
  hipError_t error() const { return err_; }

 private:
  int prev_ = -1;
  hipError_t err_ = hipSuccess;
};

int elem_bytes(int elem) { return elem == vlgqa::E_F32 ? 4 : elem == vlgqa::E_E4M3 ? 1 : 2; }

int elem_of_dtype(int dtype, int* elem) {
  switch (dtype) {
    case VLGQA_F32: *elem = vlgqa::E_F32; return VLGQA_OK;
    case VLGQA_F16: *elem = vlgqa::E_F16; return VLGQA_OK;
    case VLGQA_BF16: *elem = vlgqa::E_BF16; return VLGQA_OK;
    default: return fail(VLGQA_EUNSUPPORTED, "dtype", "unknown dtype code");
  }
}

// host part of a forward launch: the grid plan (no HIP call)
int plan_launch(vlgqa::FwdParams& p, int64_t max_seqlen_q, int elem, int64_t head_dim) {
  if (max_seqlen_q > INT32_MAX) return fail(VLGQA_EINVAL, "max_seqlen_q", "too large");
  p.max_seqlen_q = (int32_t)max_seqlen_q;
  if (!vlgqa::plan_fwd(p, elem, (int)head_dim))
    return fail(VLGQA_EINVAL, "max_seqlen_q", "problem too large for one launch");
  return VLGQA_OK;
}

int launch_planned(const vlgqa::FwdParams& p, int elem, int64_t head_dim, hipStream_t stream) {
  const StreamDeviceGuard guard(stream);
  if (guard.error() != hipSuccess) return fail(VLGQA_EHIP, "hip_stream", hipGetErrorString(guard.error()));
  hipError_t e = vlgqa::launch_fwd(p, elem, (int)head_dim, stream);
  if (e != hipSuccess) return fail(VLGQA_EHIP, "launch", hipGetErrorString(e));
  return VLGQA_OK;
}

int finish_and_launch(vlgqa::FwdParams& p, int64_t max_seqlen_q, int elem, int64_t head_dim,
                      void* hip_stream) {
  int rc;
  if ((rc = plan_launch(p, max_seqlen_q, elem, head_dim))) return rc;
  return launch_planned(p, elem, head_dim, reinterpret_cast<hipStream_t>(hip_stream));
}

}  // namespace

extern "C" {

const char* vlgqa_last_error(void) { return g_last_error.c_str(); }

const char* vlgqa_version(void) { return "vlgqa 0.1.0 gfx950"; }

int varlen_attention_fwd(const void* q, const void* k, const void* v,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int64_t total_q, int64_t total_k, int64_t batch_size,
                         int64_t num_heads, int64_t num_kv_heads,
                         int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t head_dim,
                         int causal, int dtype, void* out, float* lse, void* hip_stream) {
  g_last_error.clear();
  int rc, elem = 0;
  if ((rc = elem_of_dtype(dtype, &elem))) return rc;
  if ((rc = check_head_dim(head_dim))) return rc;
  if ((rc = check_heads(num_heads, num_kv_heads))) return rc;
  if (total_q < 0) return fail(VLGQA_EINVAL, "total_q", "must be non-negative");
  if (total_k < 0) return fail(VLGQA_EINVAL, "total_k", "must be non-negative");
  if (batch_size < 0) return fail(VLGQA_EINVAL, "batch_size", "must be non-negative");
  if (max_seqlen_q < 0) return fail(VLGQA_EINVAL, "max_seqlen_q", "must be non-negative");
  if (max_seqlen_k < 0) return fail(VLGQA_EINVAL, "max_seqlen_k", "must be non-negative");
  if (causal != 0 && causal != 1) return fail(VLGQA_EINVAL, "causal", "must be 0 or 1");
  if (total_q > INT32_MAX || total_k > INT32_MAX)
    return fail(VLGQA_EINVAL, "total_q", "token counts must fit I32 cu_seqlens");
  if (batch_size > INT32_MAX - 1) return fail(VLGQA_EINVAL, "batch_size", "too large");
  if (batch_size == 0 || total_q == 0) return VLGQA_OK;
  // lengths at most max_seqlen add up to at most batch_size * max_seqlen
  if (total_q > batch_size * max_seqlen_q)
    return fail(VLGQA_EINVAL, "max_seqlen_q", "below total_q / batch_size: a sequence is longer");
  if (total_k > batch_size * max_seqlen_k)
    return fail(VLGQA_EINVAL, "max_seqlen_k", "below total_k / batch_size: a sequence is longer");
  if ((rc = check_span(max_seqlen_q, num_heads * head_dim * elem_bytes(elem), "max_seqlen_q")))
    return rc;
  if ((rc = check_span(max_seqlen_k, num_kv_heads * head_dim * elem_bytes(elem),
                       "max_seqlen_k")))
    return rc;
  if ((rc = check_ptr(q, "q"))) return rc;
  if (total_k > 0) {
    if ((rc = check_ptr(k, "k"))) return rc;
    if ((rc = check_ptr(v, "v"))) return rc;
  }
  if ((rc = check_ptr(cu_seqlens_q, "cu_seqlens_q"))) return rc;
  if ((rc = check_ptr(cu_seqlens_k, "cu_seqlens_k"))) return rc;
  if ((rc = check_ptr(out, "out"))) return rc;
  if ((rc = check_ptr(lse, "lse"))) return rc;

  vlgqa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.q_bs = 0; p.q_rs = num_heads * head_dim; p.q_hs = head_dim;
  p.k_bs = 0; p.k_rs = num_kv_heads * head_dim; p.k_hs = head_dim;
  p.o_bs = 0; p.o_rs = num_heads * head_dim; p.o_hs = head_dim;
  p.l_bs = 0; p.l_rs = num_heads; p.l_hs = 1;
  p.batch = (int32_t)batch_size;
  p.heads = (int32_t)num_heads;
  p.kv_heads = (int32_t)num_kv_heads;
  p.group = (int32_t)(num_heads / num_kv_heads);
  p.seqlen_q = 0; p.seqlen_k = 0;
  p.causal = causal; p.window = 0;
  p.score_mul = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  p.out_mul = 1.0f;
  return finish_and_launch(p, max_seqlen_q, elem, head_dim, hip_stream);
}

// Stream-ordered scratch for the FP8 forward's bf16 copy of V: a memory pool
// per device, owned by the library, that keeps what it has reserved (release
// threshold at its maximum), so after the first call of a given size the
// allocation is bookkeeping on the stream, not a device allocation.  Each
// block lives from its allocation to its free on the caller's stream, so
// concurrent calls on different streams get different blocks.
namespace {
constexpr int kMaxPoolDevices = 64;
std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxPoolDevices] = {};

hipError_t scratch_pool(hipMemPool_t* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxPoolDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mutex);
  if (g_pools[dev] == nullptr) {
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if ((e = hipMemPoolCreate(&pool, &props)) != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    if ((e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
      (void)hipMemPoolDestroy(pool);  // the attribute error is the one reported
      return e;
    }
    g_pools[dev] = pool;
  }
  *out = g_pools[dev];
  return hipSuccess;
}
}  // namespace

static int dense_common(const void* q, const void* k, const void* v, int64_t batch,
                        int64_t num_heads, int64_t num_kv_heads, int64_t seqlen_q,
                        int64_t kv_capacity, int64_t head_dim, int causal, int64_t window_size,
                        int64_t kv_seq_len, int elem, double score_mul, double out_mul,
                        void* out, float* lse, void* hip_stream) {
  int rc;
  if ((rc = check_head_dim(head_dim))) return rc;
  if ((rc = check_heads(num_heads, num_kv_heads))) return rc;
  if (batch < 0) return fail(VLGQA_EINVAL, "batch", "must be non-negative");
  if (seqlen_q < 0) return fail(VLGQA_EINVAL, "seqlen_q", "must be non-negative");
  if (kv_capacity < 0) return fail(VLGQA_EINVAL, "kv_capacity", "must be non-negative");
  if (window_size < 0) return fail(VLGQA_EINVAL, "window_size", "must be non-negative");
  if (causal != 0 && causal != 1) return fail(VLGQA_EINVAL, "causal", "must be 0 or 1");
  const int64_t n = kv_seq_len < 0 ? kv_capacity : kv_seq_len;
  if (n > kv_capacity) return fail(VLGQA_EINVAL, "kv_seq_len", "exceeds the K/V buffer capacity");
  if (seqlen_q > INT32_MAX || kv_capacity > INT32_MAX || batch > INT32_MAX)
    return fail(VLGQA_EINVAL, "seqlen_q", "extents must fit 32 bits");
  if (window_size > INT32_MAX) window_size = INT32_MAX;
  if (batch == 0 || seqlen_q == 0) return VLGQA_OK;
  if ((rc = check_span(seqlen_q, head_dim * elem_bytes(elem), "seqlen_q"))) return rc;
  // E4M3: the kernel reads V as its 16-bit copy
  const int64_t v_bytes = elem == vlgqa::E_E4M3 ? 2 : elem_bytes(elem);
  if ((rc = check_span(n, head_dim * v_bytes, "kv_seq_len"))) return rc;
  if ((rc = check_ptr(q, "q"))) return rc;
  if (n > 0) {
    if ((rc = check_ptr(k, "k"))) return rc;
    if ((rc = check_ptr(v, "v"))) return rc;
  }
  if ((rc = check_ptr(out, "out"))) return rc;
  if ((rc = check_ptr(lse, "lse"))) return rc;

  vlgqa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
  p.cu_q = nullptr; p.cu_k = nullptr;
  p.q_bs = num_heads * seqlen_q * head_dim; p.q_rs = head_dim; p.q_hs = seqlen_q * head_dim;
  p.k_bs = num_kv_heads * kv_capacity * head_dim; p.k_rs = head_dim; p.k_hs = kv_capacity * head_dim;
  p.o_bs = p.q_bs; p.o_rs = p.q_rs; p.o_hs = p.q_hs;
  p.l_bs = num_heads * seqlen_q; p.l_rs = 1; p.l_hs = seqlen_q;
  p.batch = (int32_t)batch;
  p.heads = (int32_t)num_heads;
  p.kv_heads = (int32_t)num_kv_heads;
  p.group = (int32_t)(num_heads / num_kv_heads);
  p.seqlen_q = (int32_t)seqlen_q;
  p.seqlen_k = (int32_t)n;
  p.causal = causal;
  p.window = (int32_t)window_size;
  p.score_mul = (float)score_mul;
  p.out_mul = (float)out_mul;
  if (elem != vlgqa::E_E4M3 || n == 0) return finish_and_launch(p, seqlen_q, elem, head_dim, hip_stream);

  // E4M3: the kernel takes V as its exact bf16 copy (same element strides),
  // made here on the caller's stream into a stream-ordered scratch block
  if ((rc = plan_launch(p, seqlen_q, elem, head_dim))) return rc;
  const hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const StreamDeviceGuard guard(stream);  // the pool is the stream's device's
  if (guard.error() != hipSuccess) return fail(VLGQA_EHIP, "hip_stream", hipGetErrorString(guard.error()));
  const int64_t codes = batch * num_kv_heads * kv_capacity * head_dim;
  hipMemPool_t pool = nullptr;
  void* wide = nullptr;
  hipError_t e = scratch_pool(&pool);
  if (e == hipSuccess) e = hipMallocFromPoolAsync(&wide, (size_t)codes * 2, pool, stream);
  if (e != hipSuccess) return fail(VLGQA_EHIP, "scratch", hipGetErrorString(e));
  e = vlgqa::launch_widen_e4m3(v, wide, codes, stream);
  if (e == hipSuccess) {
    p.v = wide;
    rc = launch_planned(p, elem, head_dim, stream);
  } else {
    rc = fail(VLGQA_EHIP, "launch", hipGetErrorString(e));
  }
  e = hipFreeAsync(wide, stream);
  if (e != hipSuccess && rc == VLGQA_OK) rc = fail(VLGQA_EHIP, "scratch", hipGetErrorString(e));
  return rc;
}

int flash_attention_fwd(const void* q, const void* k, const void* v, int64_t batch,
                        int64_t num_heads, int64_t num_kv_heads, int64_t seqlen_q,
                        int64_t kv_capacity, int64_t head_dim, int causal, int64_t window_size,
                        int64_t kv_seq_len, int dtype, void* out, float* lse, void* hip_stream) {
  g_last_error.clear();
  int rc, elem = 0;
  if ((rc = elem_of_dtype(dtype, &elem))) return rc;
  const double mul = 1.4426950408889634 / std::sqrt((double)(head_dim > 0 ? head_dim : 1));
  return dense_common(q, k, v, batch, num_heads, num_kv_heads, seqlen_q, kv_capacity, head_dim,
                      causal, window_size, kv_seq_len, elem, mul, 1.0, out, lse, hip_stream);
}

int flash_attention_fwd_fp8(const void* q, const void* k, const void* v, int64_t batch,
                            int64_t num_heads, int64_t num_kv_heads, int64_t seqlen_q,
                            int64_t seqlen_k, int64_t head_dim, int causal, float q_scale,
                            float k_scale, float v_scale, float o_scale, void* out, float* lse,
                            void* hip_stream) {
  g_last_error.clear();
  const struct { const char* name; float value; } scales[] = {
      {"q_scale", q_scale}, {"k_scale", k_scale}, {"v_scale", v_scale}, {"o_scale", o_scale}};
  for (const auto& s : scales)
    if (!std::isfinite(s.value) || !(s.value > 0.0f))
      return fail(VLGQA_EINVAL, s.name, "must be finite and positive");
  const double mul = (double)q_scale * (double)k_scale * 1.4426950408889634 /
                     std::sqrt((double)(head_dim > 0 ? head_dim : 1));
  const double omul = (double)v_scale / (double)o_scale;
  if (!std::isfinite(mul) || !std::isfinite(omul) || mul == 0.0 || omul == 0.0 ||
      (float)mul == 0.0f || std::isinf((float)mul) || std::isinf((float)omul))
    return fail(VLGQA_EINVAL, "q_scale", "scale products overflow or underflow f32");
  return dense_common(q, k, v, batch, num_heads, num_kv_heads, seqlen_q, seqlen_k, head_dim,
                      causal, 0, -1, vlgqa::E_E4M3, mul, omul, out, lse, hip_stream);
}

int64_t vlgqa_decode_workspace_floats(int64_t batch, int64_t num_kv_heads, int64_t head_dim,
                                      int64_t kv_len) {
  if (batch < 0 || num_kv_heads < 0 || head_dim < 0 || kv_len < 0) return -1;
  return vlgqa::decode_workspace_floats(batch, num_kv_heads, head_dim, kv_len);
}

// The decode path behind flash_attention_decode (caller workspace) and
// flash_attention_decode_noalloc (workspace == nullptr: the library's static
// scratch, no allocation).
static int decode_common(const void* q, const void* k, const void* v, int64_t batch,
                         int64_t num_heads, int64_t num_kv_heads, int64_t seqlen_q,
                         int64_t kv_capacity, int64_t head_dim, int causal, int64_t window_size,
                         int64_t kv_seq_len, int dtype, void* out, float* lse, float* workspace,
                         int64_t workspace_floats, bool static_scratch, void* hip_stream) {
  int rc, elem = 0;
  if ((rc = elem_of_dtype(dtype, &elem))) return rc;
  if (elem == vlgqa::E_F32)
    return fail(VLGQA_EUNSUPPORTED, "dtype", "the decode path is compiled for bf16 and f16");
  if ((rc = check_head_dim(head_dim))) return rc;
  if ((rc = check_heads(num_heads, num_kv_heads))) return rc;
  if (batch < 0) return fail(VLGQA_EINVAL, "batch", "must be non-negative");
  if (seqlen_q < 0) return fail(VLGQA_EINVAL, "seqlen_q", "must be non-negative");
  if (kv_capacity < 0) return fail(VLGQA_EINVAL, "kv_capacity", "must be non-negative");
  if (window_size < 0) return fail(VLGQA_EINVAL, "window_size", "must be non-negative");
  if (causal != 0 && causal != 1) return fail(VLGQA_EINVAL, "causal", "must be 0 or 1");
  const int64_t group = num_heads / num_kv_heads;
  if (seqlen_q > 32 || seqlen_q * group > 32)
    return fail(VLGQA_EINVAL, "seqlen_q",
                "seqlen_q * num_heads / num_kv_heads must be at most 32 (use flash_attention_fwd)");
  const int64_t n = kv_seq_len < 0 ? kv_capacity : kv_seq_len;
  if (n > kv_capacity) return fail(VLGQA_EINVAL, "kv_seq_len", "exceeds the K/V buffer capacity");
  if (kv_capacity > INT32_MAX || batch > INT32_MAX)
    return fail(VLGQA_EINVAL, "kv_capacity", "extents must fit 32 bits");
  if (window_size > INT32_MAX) window_size = INT32_MAX;
  if (batch == 0 || seqlen_q == 0) return VLGQA_OK;
  if ((rc = check_span(n, head_dim * 2, "kv_seq_len"))) return rc;
  const int64_t need = vlgqa::decode_workspace_floats(batch, num_kv_heads, head_dim, n);
  const int64_t parts = vlgqa::decode_parts(batch, num_kv_heads, head_dim, n);
  if (batch * num_kv_heads * parts > INT32_MAX)
    return fail(VLGQA_EINVAL, "batch", "batch * num_kv_heads too large for one launch");
  if (static_scratch) {
    if (need > vlgqa::kDecodeScratchFloats)
      return fail(VLGQA_EINVAL, "batch",
                  "the slices' partials exceed the library's static decode scratch of 4194304 "
                  "floats (use flash_attention_decode with a workspace)");
  } else if (workspace_floats < need) {
    return fail(VLGQA_EINVAL, "workspace_floats",
                "smaller than vlgqa_decode_workspace_floats(batch, num_kv_heads, head_dim, n)");
  }
  if ((rc = check_ptr(q, "q"))) return rc;
  if (n > 0) {
    if ((rc = check_ptr(k, "k"))) return rc;
    if ((rc = check_ptr(v, "v"))) return rc;
  }
  if ((rc = check_ptr(out, "out"))) return rc;
  if ((rc = check_ptr(lse, "lse"))) return rc;
  if (!static_scratch && (rc = check_ptr(workspace, "workspace"))) return rc;
  const hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const StreamDeviceGuard guard(stream);  // the static scratch is the stream's device's
  if (guard.error() != hipSuccess) return fail(VLGQA_EHIP, "hip_stream", hipGetErrorString(guard.error()));
  if (static_scratch) {
    hipError_t se = vlgqa::decode_scratch(&workspace);
    if (se != hipSuccess) return fail(VLGQA_EHIP, "scratch", hipGetErrorString(se));
  }

  vlgqa::DecParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse; p.ws = workspace;
  p.q_bs = num_heads * seqlen_q * head_dim; p.q_hs = seqlen_q * head_dim; p.q_rs = head_dim;
  p.k_bs = num_kv_heads * kv_capacity * head_dim; p.k_hs = kv_capacity * head_dim;
  p.k_rs = head_dim;
  p.l_bs = num_heads * seqlen_q; p.l_hs = seqlen_q; p.l_rs = 1;
  p.kv_heads = (int32_t)num_kv_heads;
  p.group = (int32_t)group;
  p.seqlen_q = (int32_t)seqlen_q;
  p.kv_len = (int32_t)n;
  p.causal = causal;
  p.window = (int32_t)window_size;
  p.n_bk = (int32_t)(batch * num_kv_heads);
  p.n_parts = (int32_t)parts;
  p.score_mul = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  p.out_mul = 1.0f;
  hipError_t e = vlgqa::launch_decode(p, elem, (int)head_dim, stream);
  if (e != hipSuccess) return fail(VLGQA_EHIP, "launch", hipGetErrorString(e));
  return VLGQA_OK;
}

int flash_attention_decode(const void* q, const void* k, const void* v, int64_t batch,
                           int64_t num_heads, int64_t num_kv_heads, int64_t seqlen_q,
                           int64_t kv_capacity, int64_t head_dim, int causal, int64_t window_size,
                           int64_t kv_seq_len, int dtype, void* out, float* lse, float* workspace,
                           int64_t workspace_floats, void* hip_stream) {
  g_last_error.clear();
  return decode_common(q, k, v, batch, num_heads, num_kv_heads, seqlen_q, kv_capacity, head_dim,
                       causal, window_size, kv_seq_len, dtype, out, lse, workspace,
                       workspace_floats, false, hip_stream);
}

int flash_attention_decode_noalloc(const void* q, const void* k, const void* v, int64_t batch,
                                   int64_t num_heads, int64_t num_kv_heads, int64_t seqlen_q,
                                   int64_t kv_capacity, int64_t head_dim, int causal,
                                   int64_t window_size, int64_t kv_seq_len, int dtype, void* out,
                                   float* lse, void* hip_stream) {
  g_last_error.clear();
  return decode_common(q, k, v, batch, num_heads, num_kv_heads, seqlen_q, kv_capacity, head_dim,
                       causal, window_size, kv_seq_len, dtype, out, lse, nullptr, 0, true,
                       hip_stream);
}

static int bwd_common(vlgqa::BwdParams& p, int dtype, int64_t head_dim, int64_t rows,
                      void* hip_stream) {
  int rc;
  if (p.e4m3) {
    dtype = VLGQA_BF16;  // the kernels run on the bf16 copies of the codes
  } else if (dtype != VLGQA_BF16 && dtype != VLGQA_F16) {
    if (dtype == VLGQA_F32) return fail(VLGQA_EUNSUPPORTED, "dtype", "the backward is compiled for bf16 and f16 only");
    return fail(VLGQA_EUNSUPPORTED, "dtype", "unknown dtype code");
  }
  if ((rc = check_ptr(p.delta, "workspace"))) return rc;
  if (rows > 0) {  // with no query rows only dk = dv = 0 are written
    if ((rc = check_ptr(p.dout, "dout"))) return rc;
    if ((rc = check_ptr(p.q, "q"))) return rc;
    if ((rc = check_ptr(p.o, "out"))) return rc;
    if ((rc = check_ptr(p.lse, "lse"))) return rc;
    if ((rc = check_ptr(p.dq, "dq"))) return rc;
  }
  if (!p.e4m3) {
    p.score_mul = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    p.scale = (float)(1.0 / std::sqrt((double)head_dim));
    p.dp_mul = 1.0f;
    p.dq_mul = p.scale;
    p.dk_mul = p.scale;
    p.dv_mul = 1.0f;
  }
  if (!vlgqa::plan_bwd(p, (int)head_dim))
    return fail(VLGQA_EINVAL, "max_seqlen_q", "problem too large for one launch");
  const int elem = dtype == VLGQA_F16 ? vlgqa::E_F16 : vlgqa::E_BF16;
  hipError_t e = vlgqa::launch_bwd(p, elem, (int)head_dim, reinterpret_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(VLGQA_EHIP, "launch", hipGetErrorString(e));
  return VLGQA_OK;
}

int varlen_attention_bwd(const void* dout, const void* q, const void* k, const void* v,
                         const void* out, const float* lse, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int64_t total_q, int64_t total_k,
                         int64_t batch_size, int64_t num_heads, int64_t num_kv_heads,
                         int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t head_dim,
                         int causal, int dtype, void* dq, void* dk, void* dv, float* workspace,
                         void* hip_stream) {
  g_last_error.clear();
  int rc;
  if (dtype != VLGQA_BF16 && dtype != VLGQA_F16 && dtype != VLGQA_F32)
    return fail(VLGQA_EUNSUPPORTED, "dtype", "unknown dtype code");
  if ((rc = check_head_dim(head_dim))) return rc;
  if ((rc = check_heads(num_heads, num_kv_heads))) return rc;
  if (total_q < 0) return fail(VLGQA_EINVAL, "total_q", "must be non-negative");
  if (total_k < 0) return fail(VLGQA_EINVAL, "total_k", "must be non-negative");
  if (batch_size < 0) return fail(VLGQA_EINVAL, "batch_size", "must be non-negative");
  if (max_seqlen_q < 0) return fail(VLGQA_EINVAL, "max_seqlen_q", "must be non-negative");
  if (max_seqlen_k < 0) return fail(VLGQA_EINVAL, "max_seqlen_k", "must be non-negative");
  if (causal != 0 && causal != 1) return fail(VLGQA_EINVAL, "causal", "must be 0 or 1");
  if (total_q > INT32_MAX || total_k > INT32_MAX)
    return fail(VLGQA_EINVAL, "total_q", "token counts must fit I32 cu_seqlens");
  if (max_seqlen_q > INT32_MAX || max_seqlen_k > INT32_MAX)
    return fail(VLGQA_EINVAL, "max_seqlen_q", "too large");
  if (batch_size > INT32_MAX - 1) return fail(VLGQA_EINVAL, "batch_size", "too large");
  if (batch_size == 0 || (total_q == 0 && total_k == 0)) return VLGQA_OK;
  if (total_q > batch_size * max_seqlen_q)
    return fail(VLGQA_EINVAL, "max_seqlen_q", "below total_q / batch_size: a sequence is longer");
  if (total_k > batch_size * max_seqlen_k)
    return fail(VLGQA_EINVAL, "max_seqlen_k", "below total_k / batch_size: a sequence is longer");
  if (dtype == VLGQA_F32)
    return fail(VLGQA_EUNSUPPORTED, "dtype", "the backward is compiled for bf16 and f16 only");
  if ((rc = check_span(max_seqlen_q, num_heads * head_dim * 2, "max_seqlen_q"))) return rc;
  if ((rc = check_span(max_seqlen_k, num_kv_heads * head_dim * 2, "max_seqlen_k"))) return rc;
  if ((rc = check_ptr(cu_seqlens_q, "cu_seqlens_q"))) return rc;
  if ((rc = check_ptr(cu_seqlens_k, "cu_seqlens_k"))) return rc;
  if (total_k > 0) {
    if ((rc = check_ptr(k, "k"))) return rc;
    if ((rc = check_ptr(v, "v"))) return rc;
    if ((rc = check_ptr(dk, "dk"))) return rc;
    if ((rc = check_ptr(dv, "dv"))) return rc;
  }
  vlgqa::BwdParams p{};
  p.dout = dout; p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse; p.delta = workspace;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.q_bs = 0; p.q_rs = num_heads * head_dim; p.q_hs = head_dim;
  p.k_bs = 0; p.k_rs = num_kv_heads * head_dim; p.k_hs = head_dim;
  p.l_bs = 0; p.l_rs = num_heads; p.l_hs = 1;
  p.batch = (int32_t)batch_size;
  p.heads = (int32_t)num_heads;
  p.kv_heads = (int32_t)num_kv_heads;
  p.group = (int32_t)(num_heads / num_kv_heads);
  p.seqlen_q = 0; p.seqlen_k = 0;
  p.causal = causal; p.window = 0;
  p.max_seqlen_q = (int32_t)max_seqlen_q;
  p.max_seqlen_k = (int32_t)max_seqlen_k;
  p.d_batch = 1; p.d_rows = (int32_t)total_q;
  p.kp_rows = (int32_t)total_k;
  p.part = workspace ? workspace + vlgqa::bwd_workspace(total_q, total_k, num_heads,
                                                       num_kv_heads, head_dim, false).part
                     : nullptr;
  return bwd_common(p, dtype, head_dim, total_q, hip_stream);
}

int flash_attention_bwd(const void* dout, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, int64_t batch, int64_t num_heads,
                        int64_t num_kv_heads, int64_t seqlen_q, int64_t seqlen_k,
                        int64_t head_dim, int causal, int64_t window_size, int dtype, void* dq,
                        void* dk, void* dv, float* workspace, void* hip_stream) {
  g_last_error.clear();
  int rc;
  if (dtype != VLGQA_BF16 && dtype != VLGQA_F16 && dtype != VLGQA_F32)
    return fail(VLGQA_EUNSUPPORTED, "dtype", "unknown dtype code");
  if ((rc = check_head_dim(head_dim))) return rc;
  if ((rc = check_heads(num_heads, num_kv_heads))) return rc;
  if (batch < 0) return fail(VLGQA_EINVAL, "batch", "must be non-negative");
  if (seqlen_q < 0) return fail(VLGQA_EINVAL, "seqlen_q", "must be non-negative");
  if (seqlen_k < 0) return fail(VLGQA_EINVAL, "seqlen_k", "must be non-negative");
  if (window_size < 0) return fail(VLGQA_EINVAL, "window_size", "must be non-negative");
  if (causal != 0 && causal != 1) return fail(VLGQA_EINVAL, "causal", "must be 0 or 1");
  if (seqlen_q > INT32_MAX || seqlen_k > INT32_MAX || batch > INT32_MAX)
    return fail(VLGQA_EINVAL, "seqlen_q", "extents must fit 32 bits");
  if (window_size > INT32_MAX) window_size = INT32_MAX;
  if (batch == 0 || (seqlen_q == 0 && seqlen_k == 0)) return VLGQA_OK;
  if (dtype == VLGQA_F32)
    return fail(VLGQA_EUNSUPPORTED, "dtype", "the backward is compiled for bf16 and f16 only");
  if ((rc = check_span(seqlen_q, head_dim * 2, "seqlen_q"))) return rc;
  if ((rc = check_span(seqlen_k, head_dim * 2, "seqlen_k"))) return rc;
  if (seqlen_k > 0) {
    if ((rc = check_ptr(k, "k"))) return rc;
    if ((rc = check_ptr(v, "v"))) return rc;
    if ((rc = check_ptr(dk, "dk"))) return rc;
    if ((rc = check_ptr(dv, "dv"))) return rc;
  }
  vlgqa::BwdParams p{};
  p.dout = dout; p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse; p.delta = workspace;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.cu_q = nullptr; p.cu_k = nullptr;
  p.q_bs = num_heads * seqlen_q * head_dim; p.q_rs = head_dim; p.q_hs = seqlen_q * head_dim;
  p.k_bs = num_kv_heads * seqlen_k * head_dim; p.k_rs = head_dim; p.k_hs = seqlen_k * head_dim;
  p.l_bs = num_heads * seqlen_q; p.l_rs = 1; p.l_hs = seqlen_q;
  p.batch = (int32_t)batch;
  p.heads = (int32_t)num_heads;
  p.kv_heads = (int32_t)num_kv_heads;
  p.group = (int32_t)(num_heads / num_kv_heads);
  p.seqlen_q = (int32_t)seqlen_q;
  p.seqlen_k = (int32_t)seqlen_k;
  p.causal = causal;
  p.window = (int32_t)window_size;
  p.max_seqlen_q = (int32_t)seqlen_q;
  p.max_seqlen_k = (int32_t)seqlen_k;
  p.d_batch = (int32_t)batch; p.d_rows = (int32_t)seqlen_q;
  if (batch * seqlen_k > INT32_MAX) return fail(VLGQA_EINVAL, "seqlen_k", "batch * seqlen_k must fit 32 bits");
  p.kp_rows = (int32_t)(batch * seqlen_k);
  p.part = workspace ? workspace + vlgqa::bwd_workspace(batch * seqlen_q, batch * seqlen_k,
                                                       num_heads, num_kv_heads, head_dim,
                                                       false).part
                     : nullptr;
  return bwd_common(p, dtype, head_dim, batch * seqlen_q, hip_stream);
}

int64_t vlgqa_bwd_workspace_floats(int64_t rows, int64_t keys, int64_t num_heads,
                                   int64_t num_kv_heads, int64_t head_dim, int e4m3) {
  if (rows < 0 || keys < 0 || num_heads < 0 || num_kv_heads < 0 || head_dim < 0) return -1;
  return vlgqa::bwd_workspace(rows, keys, num_heads, num_kv_heads, head_dim, e4m3 != 0).total;
}

int flash_attention_bwd_fp8(const void* dout, const void* q, const void* k, const void* v,
                            const void* out, const float* lse, int64_t batch, int64_t num_heads,
                            int64_t num_kv_heads, int64_t seqlen_q, int64_t seqlen_k,
                            int64_t head_dim, int causal, float q_scale, float k_scale,
                            float v_scale, float do_scale, float o_scale, float dq_scale,
                            float dk_scale, float dv_scale, void* dq, void* dk, void* dv,
                            float* workspace, int64_t workspace_floats, void* hip_stream) {
  g_last_error.clear();
  int rc;
  const struct { const char* name; float value; } scales[] = {
      {"q_scale", q_scale},   {"k_scale", k_scale},   {"v_scale", v_scale},
      {"do_scale", do_scale}, {"o_scale", o_scale},   {"dq_scale", dq_scale},
      {"dk_scale", dk_scale}, {"dv_scale", dv_scale}};
  for (const auto& s : scales)
    if (!std::isfinite(s.value) || !(s.value > 0.0f))
      return fail(VLGQA_EINVAL, s.name, "must be finite and positive");
  if ((rc = check_head_dim(head_dim))) return rc;
  if ((rc = check_heads(num_heads, num_kv_heads))) return rc;
  if (batch < 0) return fail(VLGQA_EINVAL, "batch", "must be non-negative");
  if (seqlen_q < 0) return fail(VLGQA_EINVAL, "seqlen_q", "must be non-negative");
  if (seqlen_k < 0) return fail(VLGQA_EINVAL, "seqlen_k", "must be non-negative");
  if (causal != 0 && causal != 1) return fail(VLGQA_EINVAL, "causal", "must be 0 or 1");
  if (seqlen_q > INT32_MAX || seqlen_k > INT32_MAX || batch > INT32_MAX)
    return fail(VLGQA_EINVAL, "seqlen_q", "extents must fit 32 bits");
  if (batch * seqlen_k > INT32_MAX)
    return fail(VLGQA_EINVAL, "seqlen_k", "batch * seqlen_k must fit 32 bits");
  const double rs = 1.0 / std::sqrt((double)head_dim);
  const double m[6] = {(double)q_scale * k_scale * 1.4426950408889634 * rs,
                       (double)do_scale * v_scale,
                       (double)k_scale * rs / dq_scale,
                       (double)q_scale * rs / dk_scale,
                       (double)do_scale / dv_scale,
                       (double)do_scale * o_scale};
  for (double x : m)
    if (!std::isfinite(x) || x == 0.0 || (float)x == 0.0f || std::isinf((float)x))
      return fail(VLGQA_EINVAL, "q_scale", "scale products overflow or underflow f32");
  if (batch == 0 || (seqlen_q == 0 && seqlen_k == 0)) return VLGQA_OK;
  if ((rc = check_span(seqlen_q, head_dim * 2, "seqlen_q"))) return rc;
  if ((rc = check_span(seqlen_k, head_dim * 2, "seqlen_k"))) return rc;
  const int64_t rows = batch * seqlen_q, keys = batch * seqlen_k;
  const vlgqa::BwdWorkspace w =
      vlgqa::bwd_workspace(rows, keys, num_heads, num_kv_heads, head_dim, true);
  if (workspace_floats < w.total)
    return fail(VLGQA_EINVAL, "workspace_floats",
                "smaller than vlgqa_bwd_workspace_floats(rows, keys, H, Hkv, D, 1)");
  if ((rc = check_ptr(workspace, "workspace"))) return rc;
  if (seqlen_k > 0) {
    if ((rc = check_ptr(k, "k"))) return rc;
    if ((rc = check_ptr(v, "v"))) return rc;
    if ((rc = check_ptr(dk, "dk"))) return rc;
    if ((rc = check_ptr(dv, "dv"))) return rc;
  }
  if (rows > 0) {  // the copies are checked again as q / dout below
    if ((rc = check_ptr(dout, "dout"))) return rc;
    if ((rc = check_ptr(q, "q"))) return rc;
  }
  vlgqa::BwdParams p{};
  p.e4m3 = 1;
  p.q8 = q; p.k8 = k; p.v8 = v; p.do8 = dout;
  p.wq = workspace + w.wide;
  p.wdo = workspace + w.wide + rows * num_heads * head_dim / 2;
  p.wk = workspace + w.wide + rows * num_heads * head_dim;
  p.n_q = rows * num_heads * head_dim;
  p.n_k = keys * num_kv_heads * head_dim;
  p.dout = p.wdo; p.q = p.wq; p.k = p.wk; p.v = nullptr; p.o = out; p.lse = lse;
  p.delta = workspace;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.cu_q = nullptr; p.cu_k = nullptr;
  p.q_bs = num_heads * seqlen_q * head_dim; p.q_rs = head_dim; p.q_hs = seqlen_q * head_dim;
  p.k_bs = num_kv_heads * seqlen_k * head_dim; p.k_rs = head_dim; p.k_hs = seqlen_k * head_dim;
  p.l_bs = num_heads * seqlen_q; p.l_rs = 1; p.l_hs = seqlen_q;
  p.batch = (int32_t)batch;
  p.heads = (int32_t)num_heads;
  p.kv_heads = (int32_t)num_kv_heads;
  p.group = (int32_t)(num_heads / num_kv_heads);
  p.seqlen_q = (int32_t)seqlen_q;
  p.seqlen_k = (int32_t)seqlen_k;
  p.causal = causal;
  p.window = 0;
  p.max_seqlen_q = (int32_t)seqlen_q;
  p.max_seqlen_k = (int32_t)seqlen_k;
  p.d_batch = (int32_t)batch; p.d_rows = (int32_t)seqlen_q;
  p.kp_rows = (int32_t)keys;
  p.part = workspace + w.part;
  p.scale = (float)rs;
  p.score_mul = (float)m[0];
  p.dp_mul = (float)m[1];
  p.dq_mul = (float)m[2];
  p.dk_mul = (float)m[3];
  p.dv_mul = (float)m[4];
  p.delta_mul = (float)m[5];
  return bwd_common(p, VLGQA_BF16, head_dim, rows, hip_stream);
}

static int check_pack_common(const int32_t* cu_seqlens, int64_t batch_size, int64_t max_seqlen,
                             int64_t row_bytes) {
  int rc;
  if (batch_size < 0) return fail(VLGQA_EINVAL, "batch_size", "must be non-negative");
  if (batch_size > INT32_MAX - 1) return fail(VLGQA_EINVAL, "batch_size", "too large");
  if (max_seqlen < 0) return fail(VLGQA_EINVAL, "max_seqlen", "must be non-negative");
  if (max_seqlen > INT32_MAX) return fail(VLGQA_EINVAL, "max_seqlen", "too large");
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(VLGQA_EINVAL, "row_bytes", "must be a positive multiple of 16");
  if (row_bytes > ((int64_t)1 << 40) / (max_seqlen > 0 ? max_seqlen : 1) / (batch_size > 0 ? batch_size : 1))
    return fail(VLGQA_EINVAL, "row_bytes", "padded buffer too large");
  if (batch_size > 0 && (rc = check_ptr(cu_seqlens, "cu_seqlens"))) return rc;
  return VLGQA_OK;
}

int vlgqa_cu_seqlens(const int32_t* lengths, int64_t batch_size, int32_t* cu_seqlens,
                     void* hip_stream) {
  g_last_error.clear();
  int rc;
  if (batch_size < 0) return fail(VLGQA_EINVAL, "batch_size", "must be non-negative");
  if (batch_size > INT32_MAX - 1) return fail(VLGQA_EINVAL, "batch_size", "too large");
  if ((rc = check_ptr(cu_seqlens, "cu_seqlens"))) return rc;
  if (batch_size > 0 && (rc = check_ptr(lengths, "lengths"))) return rc;
  hipError_t e = vlgqa::launch_cu_seqlens(lengths, batch_size, cu_seqlens,
                                          reinterpret_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(VLGQA_EHIP, "launch", hipGetErrorString(e));
  return VLGQA_OK;
}

int vlgqa_pack(const void* padded, const int32_t* cu_seqlens, int64_t batch_size,
               int64_t max_seqlen, int64_t row_bytes, int64_t total, void* packed,
               void* hip_stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pack_common(cu_seqlens, batch_size, max_seqlen, row_bytes))) return rc;
  if (total < 0) return fail(VLGQA_EINVAL, "total", "must be non-negative");
  if (total > INT32_MAX) return fail(VLGQA_EINVAL, "total", "must fit I32 cu_seqlens");
  if (batch_size == 0 || total == 0) return VLGQA_OK;
  if ((rc = check_ptr(padded, "padded"))) return rc;
  if ((rc = check_ptr(packed, "packed"))) return rc;
  hipError_t e = vlgqa::launch_pack(padded, cu_seqlens, batch_size, max_seqlen, row_bytes, total,
                                    packed, reinterpret_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(VLGQA_EHIP, "launch", hipGetErrorString(e));
  return VLGQA_OK;
}

int vlgqa_unpack(const void* packed, const int32_t* cu_seqlens, int64_t batch_size,
                 int64_t max_seqlen, int64_t row_bytes, void* padded, void* hip_stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pack_common(cu_seqlens, batch_size, max_seqlen, row_bytes))) return rc;
  if (batch_size == 0 || max_seqlen == 0) return VLGQA_OK;
  if ((rc = check_ptr(packed, "packed"))) return rc;
  if ((rc = check_ptr(padded, "padded"))) return rc;
  hipError_t e = vlgqa::launch_unpack(packed, cu_seqlens, batch_size, max_seqlen, row_bytes,
                                      padded, reinterpret_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(VLGQA_EHIP, "launch", hipGetErrorString(e));
  return VLGQA_OK;
}

}  // extern "C"
