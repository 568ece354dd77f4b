// Device-side building blocks shared by the attention kernels (gfx950):
// vector types, matrix-core and conversion wrappers (16-bit and E4M3),
// range-checked buffer loads, LDS DMA, the LDS-only workgroup barrier, the
// 16-byte chunk swizzles of 16-bit and E4M3 rows and the transposing V^T
// operand read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_params.h"

namespace vlgqa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

template <int ELEM>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (ELEM == E_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {  // bf16, and E4M3 widened to bf16
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// two floats -> packed 16-bit pair (round to nearest even), one v_cvt_pk_*
template <int ELEM>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  if constexpr (ELEM == E_F16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
}

// four floats -> four OCP E4M3 codes in one register (v_cvt_pk_fp8_f32: round
// to nearest even).  Callers keep |x| <= 448 (the largest finite code).
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// clamp to the finite E4M3 range (saturating encode: never a NaN code)
__device__ __forceinline__ float sat448(float x) {
  return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f);
}

// Range-checked loads: a buffer resource covering [base, base + bytes) returns
// zeros for any access at or beyond `bytes` (rows past a sequence's end).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t sat_bytes(int64_t b) {
  return b > 0xFFFFFFFFll ? 0xFFFFFFFFu : (b < 0 ? 0u : (uint32_t)b);
}

// chunk swizzle of an LDS row: physical chunk = logical chunk ^ swz(row)
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);  // 16 chunks per row
  else return (row >> 1) & 7;                                       // 8 chunks per row
}

// chunk swizzle of an E4M3 row (K, Q or dO codes) in LDS: the 16 lanes of a K read cover 16
// consecutive rows of one logical chunk; the swizzle is a bijection on the
// rows of equal parity (D=128, 8 chunks a row) or equal residue mod 4 (D=64,
// 4 chunks), so the 16 reads fall in distinct banks.
template <int D>
__device__ __forceinline__ int swz8(int row) {
  if constexpr (D == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(const u32x4 (&a)[2], const u32x4 (&b)[2], f32x16 c) {
  const i32x8 av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                    (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
  const i32x8 bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                    (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
  // format selectors 0/0: both operands OCP E4M3; zero block scales = no scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
}

// two E4M3 codes (bytes 0-1 or 2-3 of w) -> two bf16 in one register, exact
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// Scheduling hint for the run of N matrix products just emitted, each fed by R
// LDS reads: keep the reads of AHEAD products in flight ahead of the products
// (the default interleave issues them just in time).  Only instructions of
// the current scheduling region take part.
template <int N, int R, int AHEAD>
__device__ __forceinline__ void sched_lds_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one product
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);        // its successor's reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// (lgkmcnt) but lets global loads and LDS DMA stay in flight across it.  A
// __syncthreads(), and even an LDS-scoped fence, drains every outstanding
// vector-memory request (DMA writes count as LDS stores).  DMA into LDS is
// published by an explicit vmcnt wait before this.  The empty asm statements
// with a memory clobber keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait until no vector-memory request of this wave is outstanding
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Request one 16-byte chunk per lane from global memory (buffer descriptor
// rsrc, byte offset voff) straight into LDS: lane i writes LDS bytes
// lds_dst + 16 i .. + 16 (lds_dst is wave-uniform: it goes to m0, which the
// compiler sets).  No register results; completion is awaited with an explicit
// vmcnt wait before the barrier that publishes the tile.  The compiler tracks
// the LDS write per __shared__ array, so reads of the other buffers of a
// double-buffered pair are not held up by it.
__device__ __forceinline__ void dma16(const void* lds_dst, uint32_t voff,
                                      __amdgpu_buffer_rsrc_t rsrc, uint32_t soff = 0) {
  // soff: a wave-uniform byte offset added in the scalar unit
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_dst, 16, (int)voff, (int)soff, 0,
                                           0);
}

// one V^T operand (32 d x 16 keys) by two transposing reads
__device__ __forceinline__ u32x4 vt_operand(const uint8_t* p0, const uint8_t* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

}  // namespace vlgqa
