// Packing of padded batches into the varlen layout (gfx950): the exclusive
// prefix sum of the sequence lengths (cu_seqlens) and the row copies padded
// [B, S, row] <-> packed [total, row]; and the E4M3 -> bf16 widening copy the
// FP8 paths use.  boostr 0.2.0 varlen_attention.rs:
// sequences of different lengths are packed into one buffer instead of being
// padded; cu_seqlens[0] = 0, cu_seqlens[i] = sum of lengths 0..i-1.  Rows are
// opaque bytes (a multiple of 16), moved as 16-byte vectors.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pack_api.h"

namespace vlgqa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kScanThreads = 1024;

// One workgroup: chunks of 1024 lengths, a workgroup-wide inclusive scan per
// chunk (wave prefix by shuffles, then the wave totals), plus the carry of
// the chunks before.
__global__ __launch_bounds__(kScanThreads) void cu_seqlens_kernel(const int32_t* lengths,
                                                                  int64_t batch, int32_t* cu) {
  __shared__ int32_t wave_sum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) cu[0] = 0;
  int32_t carry = 0;
  for (int64_t base = 0; base < batch; base += kScanThreads) {
    const int64_t i = base + tid;
    int32_t x = i < batch ? lengths[i] : 0;
    // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_sum[wid] = x;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wid; ++w) before += wave_sum[w];
    int32_t total = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) total += wave_sum[w];
    if (i < batch) cu[i + 1] = carry + before + x;
    carry += total;
    __syncthreads();  // wave_sum is rewritten by the next chunk
  }
}

// Pack: one wave per packed row (grid-stride over rows, wave-uniform, so the
// sequence lookup runs on the scalar unit once per row); the lanes copy the
// row's 16-byte chunks with four loads in flight each.  (The same scheme for
// unpack measured 10% slower than its one-chunk-per-thread form below.)
__device__ __forceinline__ int64_t wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
}

__device__ __forceinline__ void copy_row(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                         int64_t row16, int lane) {
  for (int64_t c = lane; c < row16; c += 256) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c + 64 * j < row16) v[j] = src[c + 64 * j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c + 64 * j < row16) dst[c + 64 * j] = v[j];
  }
}

// packed row t <- padded row (b, t - cu[b]) with cu[b] <= t < cu[b+1]
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ padded,
                                                   const int32_t* __restrict__ cu, int64_t batch,
                                                   int64_t S, int64_t row16, int64_t total,
                                                   uint8_t* __restrict__ packed) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = wave_id(); t < total; t += nwaves) {
    int64_t lo = 0, hi = batch;  // largest b with cu[b] <= t
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    const int64_t s = t - cu[lo];
    copy_row(reinterpret_cast<const u32x4*>(padded + (lo * S + s) * row16 * 16),
             reinterpret_cast<u32x4*>(packed + t * row16 * 16), row16, lane);
  }
}

// padded row (b, s) <- packed row cu[b] + s for s < length_b, else zeros: one
// thread per 16-byte chunk (IDX uint32_t when every chunk index fits)
template <typename IDX>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* packed, const int32_t* cu,
                                                     int64_t batch, int64_t S_, int64_t row16_,
                                                     uint8_t* padded) {
  const IDX row16 = (IDX)row16_, S = (IDX)S_;
  const IDX n = (IDX)(batch * S_ * row16_);
  for (IDX i = (IDX)blockIdx.x * 256 + threadIdx.x; i < n; i += (IDX)gridDim.x * 256) {
    const IDX r = i / row16, c = i - r * row16;
    const IDX b = r / S, s = r - b * S;
    const int64_t start = cu[b], len = (int64_t)cu[b + 1] - start;
    u32x4 v = {0u, 0u, 0u, 0u};
    if ((int64_t)s < len)
      v = *reinterpret_cast<const u32x4*>(packed + ((start + (int64_t)s) * (int64_t)row16 +
                                                    (int64_t)c) * 16);
    *reinterpret_cast<u32x4*>(padded + (int64_t)i * 16) = v;
  }
}

unsigned grid_for(int64_t n) {
  const int64_t blocks = (n + 255) / 256;
  return (unsigned)(blocks < 65536 ? blocks : 65536);  // grid-stride beyond
}

// workgroups of 4 one-row waves: enough to cover the rows, at most 8 per CU
unsigned grid_for_rows(int64_t rows) {
  const int64_t blocks = (rows + 3) / 4;
  return (unsigned)(blocks < 2048 ? blocks : 2048);
}

// E4M3 codes -> bf16 (exact: every E4M3 value is a bf16 value), 16 codes per
// thread (n16 = codes / 16)
__global__ __launch_bounds__(256) void widen_e4m3_kernel(const uint8_t* __restrict__ src,
                                                         uint16_t* __restrict__ dst, int64_t n16) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 c = *reinterpret_cast<const u32x4*>(src + i * 16);
  u32x4 w[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[k], 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[k], 1.0f, true);
    w[k >> 1][2 * (k & 1)] = __builtin_bit_cast(uint32_t, lo);
    w[k >> 1][2 * (k & 1) + 1] = __builtin_bit_cast(uint32_t, hi);
  }
  *reinterpret_cast<u32x4*>(dst + i * 16) = w[0];
  *reinterpret_cast<u32x4*>(dst + i * 16 + 8) = w[1];
}

}  // namespace

hipError_t launch_widen_e4m3(const void* codes, void* bf16, int64_t n, hipStream_t stream) {
  if (n % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = n / 16;
  if (n16 > 0)
    hipLaunchKernelGGL(widen_e4m3_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0,
                       stream, reinterpret_cast<const uint8_t*>(codes),
                       reinterpret_cast<uint16_t*>(bf16), n16);
  return hipGetLastError();
}

hipError_t launch_cu_seqlens(const int32_t* lengths, int64_t batch, int32_t* cu,
                             hipStream_t stream) {
  hipLaunchKernelGGL(cu_seqlens_kernel, dim3(1), dim3(kScanThreads), 0, stream, lengths, batch,
                     cu);
  return hipGetLastError();
}

hipError_t launch_pack(const void* padded, const int32_t* cu, int64_t batch, int64_t S,
                       int64_t row_bytes, int64_t total, void* packed, hipStream_t stream) {
  if (total > 0)
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for_rows(total)), dim3(256), 0, stream,
                       reinterpret_cast<const uint8_t*>(padded), cu, batch, S, row_bytes / 16,
                       total, reinterpret_cast<uint8_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack(const void* packed, const int32_t* cu, int64_t batch, int64_t S,
                         int64_t row_bytes, void* padded, hipStream_t stream) {
  const int64_t row16 = row_bytes / 16;
  const int64_t n = batch * S * row16;
  const bool small = n + (int64_t)65536 * 256 < ((int64_t)1 << 32);
  if (n > 0) {
    if (small)
      hipLaunchKernelGGL(unpack_kernel<uint32_t>, dim3(grid_for(n)), dim3(256), 0, stream,
                         reinterpret_cast<const uint8_t*>(packed), cu, batch, S, row16,
                         reinterpret_cast<uint8_t*>(padded));
    else
      hipLaunchKernelGGL(unpack_kernel<int64_t>, dim3(grid_for(n)), dim3(256), 0, stream,
                         reinterpret_cast<const uint8_t*>(packed), cu, batch, S, row16,
                         reinterpret_cast<uint8_t*>(padded));
  }
  return hipGetLastError();
}

}  // namespace vlgqa
