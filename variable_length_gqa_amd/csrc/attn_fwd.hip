// Fused attention forward for gfx950 (CDNA4): packed varlen and dense layouts,
// GQA, causal / sliding-window masks, bf16 / f16 / f32 / E4M3 storage.
//
// What is computed (boostr varlen_attention.rs "VarLenAttentionOps" and boostr
// flash.rs "FlashAttentionOps"): for each (sequence, query head h, query row i)
// O_i = softmax(scale * q_i K^T restricted to the visible keys) V with
// kv_head = h / (H / Hkv), plus LSE_i = ln sum exp(scores) in f32.  The
// evaluation is the tiled online softmax of realizar attention.rs IMP-111
// ("tiled_single_head_attention"): per query row a running maximum, running
// denominator and running weighted sum, rescaled when the maximum grows.
//
// Work decomposition: one workgroup = 4 waves x 32 query rows of one sequence:
// a 128-row query tile of one query head, or (16-bit kernel, long sequences,
// an even group) a 64-row tile of two query heads of the group.  K/V tiles of
// 32 keys are staged through LDS (double buffered, one barrier per tile) and
// shared by the 4 waves.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_{bf16,f16}, wave64):
//   S^T = K Q^T   A = K tile (32 keys x 16 d, from LDS), B = Q^T (registers)
//                 -> lane l holds query (l % 32) and 16 of the tile's 32 keys,
//                    so a row's max / sum is an in-lane reduction plus one
//                    permlane32 swap.
//   O^T = V^T P^T A = V^T (32 d x 16 keys, transposing LDS reads of the
//                 row-major V tile), B = P^T taken straight from the S^T
//                 accumulator registers (converted to 16 bit) -> O^T keeps
//                 query (l % 32) per lane, so the per-row rescale factor is a
//                 per-lane scalar.
// The P registers cover keys {0-3, 8-11} (lanes 0-31) and {4-7, 12-15}
// (lanes 32-63) of each 16-key step; the transposing V reads gather the keys
// in that order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <type_traits>

#include "fwd_params.h"
#include "kernel_common.h"
#include "ticket.h"

namespace vlgqa {

// a row's reference maximum is only moved when a tile raises it by more than
// this (log2 units); until then probabilities may reach 2^kRescaleSlack.  The
// result is exact either way: numerator and denominator use the same reference.
constexpr float kRescaleSlack = 8.0f;
// bf16/f16 kernels: a lane's partial sum of a tile's probabilities may reach
// this before the reference maximum is moved.  It also bounds each probability,
// and 2^15 keeps every one finite in f16 (largest finite value 65504).
constexpr float kPartialSumBound = 32768.0f;

// ---------------------------------------------------------------------------
// work decode: XCD-aware, longest query tiles first
// ---------------------------------------------------------------------------
//
// Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8).  A
// "group" is (query tile, sequence, kv head); the workgroups of a group cover
// its G query heads (heads_per_wg at a time) and read the same K/V, so they
// are placed on consecutive slots of ONE XCD and share its L2.  Groups are
// ordered by descending query tile: under a causal mask later tiles see more
// keys, so the longest work is dispatched first.  The XCDs run the same work
// at different speeds (their finishing times spread by ~9%), so the last
// slots of every XCD (about a fifth, the shortest items) are not tied to a
// block: the blocks after the statically assigned ones claim them in order
// from a counter, and fast XCDs take more of them.  Under a sliding window the
// tiles of one sequence come together instead (sequence-major, descending
// within it): nearby tiles read nearly the same window of K/V, and the
// windows of the sequences interleaved would not fit an XCD's L2 together.
struct Work {
  int b, kvh, h0, r0;
  int q_start, Lq, k_start, Lk;
};

__device__ __forceinline__ bool decode_work(const FwdParams& p, Work& w) {
  const int G2 = p.group / p.heads_per_wg;  // workgroups per group
  const int pid = blockIdx.x;
  int xcd = pid & 7;
  int slot = pid >> 3;
  if (p.ticket != nullptr && pid >= 8 * p.n_static) {
    // a claiming block: its item is the next unclaimed tail item (slot by
    // slot, XCD by XCD: descending work), so XCDs that run faster take more
    // of the end of the launch.  A relaxed atomic: only the counter's
    // atomicity matters (an ordering fence here would write back the L2).
    __shared__ unsigned claimed;
    if (threadIdx.x == 0)
      claimed = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) - p.ticket_base;
    __syncthreads();
    const unsigned j = __builtin_amdgcn_readfirstlane(claimed);
    if (j >= (unsigned)p.n_tail) return false;
    xcd = (int)(j & 7);
    slot = p.n_static + (int)(j >> 3);
  }
  const int gq = slot / G2;
  const int g2 = slot - gq * G2;
  const int grp = gq * 8 + xcd;
  if (grp >= p.n_groups) return false;
  w.kvh = grp % p.kv_heads;
  const int t2 = grp / p.kv_heads;
  int tidx;
  if (p.window > 0) {  // a sequence's tiles together: they share their K/V windows
    w.b = t2 / p.n_qtiles;
    tidx = t2 % p.n_qtiles;
  } else {
    w.b = t2 % p.batch;
    tidx = t2 / p.batch;
  }
  w.r0 = (p.n_qtiles - 1 - tidx) * p.rows_per_wg;
  w.h0 = w.kvh * p.group + g2 * p.heads_per_wg;
  w.q_start = 0;
  w.Lq = p.seqlen_q;
  w.k_start = 0;
  w.Lk = p.seqlen_k;
  if (p.cu_q) {
    w.q_start = p.cu_q[w.b];
    w.Lq = p.cu_q[w.b + 1] - w.q_start;
  }
  if (p.cu_k) {
    w.k_start = p.cu_k[w.b];
    w.Lk = p.cu_k[w.b + 1] - w.k_start;
  }
  return w.r0 < w.Lq;
}

// Key range [lo, hi) visible to query rows [qa, qb] of a sequence.
__device__ __forceinline__ void key_range(const FwdParams& p, const Work& w, int qa, int qb,
                                          int& lo, int& hi) {
  const int off = w.Lk - w.Lq;
  const bool upper = p.causal || p.window > 0;
  hi = upper ? min(w.Lk, qb + off + 1) : w.Lk;
  lo = p.window > 0 ? max(0, qa + off - p.window + 1) : 0;
}

// The BN-key tiles a wave of 32 query rows (rows rw .. rw + 31 of the
// workgroup's tile) works on, [tv0, tv1) (empty when the wave has no rows),
// and which of them need element masks: tiles below tm_lo the window's lower
// bound, tiles from tm_hi on the causal bound or the sequence end.  Computed
// once, so a tile's tests are two integer compares each.
__device__ __forceinline__ void wave_tiles(const FwdParams& p, const Work& w, int rw, int BN,
                                           int& tv0, int& tv1, int& tm_lo, int& tm_hi) {
  const int wa = w.r0 + rw, wb = min(wa + 31, w.Lq - 1);
  const int off = w.Lk - w.Lq;
  const bool upper = p.causal || p.window > 0;
  tv0 = tv1 = 0;
  if (wa <= wb) {
    int lo, hi;
    key_range(p, w, wa, wb, lo, hi);
    if (hi > lo) {
      tv0 = lo / BN;
      tv1 = (hi + BN - 1) / BN;
    }
  }
  // key c of a tile is unmasked for every row of the wave iff c <= lim (the
  // first row's causal bound, or the last key) and c >= wlim (the last row's
  // window start)
  const int lim = upper ? min(w.Lk - 1, wa + off) : w.Lk - 1;
  tm_hi = lim >= 0 ? (lim + 1) / BN : 0;
  const int wlim = wb + off - p.window + 1;
  tm_lo = p.window > 0 && wlim > 0 ? (wlim + BN - 1) / BN : 0;
}

// ---------------------------------------------------------------------------
// shared softmax / epilogue pieces
// ---------------------------------------------------------------------------

// Mask the S^T accumulators of a 64-key tile starting at key c0 for the
// lane's query row q.  Key of register r in block kb: c0 + 32 kb + 8 (r / 4)
// + 4 (lane / 32) + r % 4.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int c0, int hl, int q, int off, int Lk,
                                          bool upper, int window) {
  const int hi = upper ? min(Lk - 1, q + off) : Lk - 1;
  const int lo = window > 0 ? q + off - window + 1 : 0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = c0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (key > hi || key < lo) s[kb][r] = -INFINITY;
    }
  }
}

// max over the 64 scores of the lane's row in one tile (32 here, 32 in lane ^ 32)
__device__ __forceinline__ float tile_row_max(const f32x16 (&s)[2]) {
  float a = fmaxf(s[0][0], s[1][0]), b = fmaxf(s[0][1], s[1][1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) {
    a = fmaxf(a, fmaxf(s[0][r], s[1][r]));
    b = fmaxf(b, fmaxf(s[0][r + 1], s[1][r + 1]));
  }
  return swap_halves_max(fmaxf(a, b));
}

// Move the reference maximum m of a row to mx (log2 domain) when the tile
// raises it by more than kRescaleSlack; rescale l and o to match.  The caller
// has the wave-uniform "any lane moves" test around it.
template <int NOB>
__device__ __forceinline__ void rescale_row(float mx, float& m, float& l, f32x16 (&o)[NOB]) {
  const bool up = mx > m + kRescaleSlack;
  const float alpha = up ? __builtin_amdgcn_exp2f(m - mx) : 1.0f;
  m = up ? mx : m;
  l *= alpha;
#pragma unroll
  for (int i = 0; i < NOB; ++i) o[i] *= alpha;
}

template <int NOB>
struct RowState {
  float m;         // reference maximum, log2 domain (score * score_mul)
  float l;         // this lane's half of the running denominator
  f32x16 o[NOB];   // O^T accumulators: query (lane % 32), 16 d values per block
};

// Normalise and store one query row's O (4 consecutive d per store) and LSE.
template <int OUT_ELEM, int D>
__device__ __forceinline__ void store_row(const FwdParams& p, const Work& w, int h, int qrow,
                                          int hl, float m, float l, const f32x16 (&o)[D / 32]) {
  const float ltot = swap_halves_sum(l);
  if (qrow >= w.Lq) return;
  const float inv = ltot > 0.0f ? p.out_mul / ltot : 0.0f;
  const int64_t orow = (int64_t)w.b * p.o_bs + (int64_t)(w.q_start + qrow) * p.o_rs +
                       (int64_t)h * p.o_hs;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + g * 8 + 4 * hl;
      const float x0 = o[db][4 * g + 0] * inv, x1 = o[db][4 * g + 1] * inv;
      const float x2 = o[db][4 * g + 2] * inv, x3 = o[db][4 * g + 3] * inv;
      if constexpr (OUT_ELEM == E_F32) {
        f32x4 v = {x0, x1, x2, x3};
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + orow + d0) = v;
      } else if constexpr (OUT_ELEM == E_E4M3) {
        const uint32_t v = pack4_fp8(sat448(x0), sat448(x1), sat448(x2), sat448(x3));
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(p.o) + orow + d0) = v;
      } else {
        u32x2 v = {pack2<OUT_ELEM>(x0, x1), pack2<OUT_ELEM>(x2, x3)};
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o) + orow + d0) = v;
      }
    }
  }
  if (hl == 0) {
    const float lse = ltot > 0.0f ? (m + __builtin_log2f(ltot)) * kLn2 : -INFINITY;
    p.lse[(int64_t)w.b * p.l_bs + (int64_t)(w.q_start + qrow) * p.l_rs + (int64_t)h * p.l_hs] = lse;
  }
}

// 16-bit output through LDS: the wave writes its normalised 32 x D tile of O
// into `stage` (its own 32 * 2D bytes, rows with their 16-byte chunks
// XOR-swizzled by row as in the K/V tiles), then reads it back a row chunk
// per lane and stores whole rows: 16-byte stores covering 64 / (D / 8) rows
// each, in place of 8-byte stores scattered over 32 rows.  LSE as store_row.
template <int OUT_ELEM, int D>
__device__ __forceinline__ void store_row_staged(const FwdParams& p, const Work& w, int h,
                                                 int r0w, int ql, int hl, float m, float l,
                                                 const f32x16 (&o)[D / 32], uint8_t* stage) {
  static_assert(OUT_ELEM == E_BF16 || OUT_ELEM == E_F16, "16-bit output");
  constexpr int ROWB = 2 * D, CPR = ROWB / 16;
  const float ltot = swap_halves_sum(l);
  const float inv = ltot > 0.0f ? p.out_mul / ltot : 0.0f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // d = 32 db + 8 g + 4 hl .. +4: half of logical chunk 4 db + g
      const int c = 4 * db + g;
      const u32x2 v = {pack2<OUT_ELEM>(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                       pack2<OUT_ELEM>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
      *reinterpret_cast<u32x2*>(stage + ql * ROWB + ((c ^ swz<D>(ql)) * 16) + 8 * hl) = v;
    }
  }
  const int qrow = r0w + ql;
  if (hl == 0 && qrow < w.Lq) {
    const float lse = ltot > 0.0f ? (m + __builtin_log2f(ltot)) * kLn2 : -INFINITY;
    p.lse[(int64_t)w.b * p.l_bs + (int64_t)(w.q_start + qrow) * p.l_rs + (int64_t)h * p.l_hs] = lse;
  }
  const int lane = ql + 32 * hl;
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = RPI * k + lane / CPR, c = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * ROWB + ((c ^ swz<D>(row)) * 16));
    if (r0w + row < w.Lq) {
      const int64_t orow = (int64_t)w.b * p.o_bs + (int64_t)(w.q_start + r0w + row) * p.o_rs +
                           (int64_t)h * p.o_hs;
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.o) + orow + 8 * c) = v;
    }
  }
}

// The same for E4M3 output: the wave's 32 x D tile of codes (rows of D bytes,
// 16-byte chunks XOR-swizzled by swz8) goes through `stage` (32 * D bytes),
// and whole rows are stored with 16-byte stores.
template <int D>
__device__ __forceinline__ void store_row_staged8(const FwdParams& p, const Work& w, int h,
                                                  int r0w, int ql, int hl, float m, float l,
                                                  const f32x16 (&o)[D / 32], uint8_t* stage) {
  constexpr int CPR = D / 16;
  const float ltot = swap_halves_sum(l);
  const float inv = ltot > 0.0f ? p.out_mul / ltot : 0.0f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // codes d = 32 db + 8 g + 4 hl .. +4: bytes 8 (g % 2) + 4 hl of chunk 2 db + g / 2
      const int c = 2 * db + (g >> 1);
      const uint32_t v = pack4_fp8(sat448(o[db][4 * g + 0] * inv), sat448(o[db][4 * g + 1] * inv),
                                   sat448(o[db][4 * g + 2] * inv), sat448(o[db][4 * g + 3] * inv));
      *reinterpret_cast<uint32_t*>(stage + ql * D + ((c ^ swz8<D>(ql)) * 16) + 8 * (g & 1) +
                                   4 * hl) = v;
    }
  }
  const int qrow = r0w + ql;
  if (hl == 0 && qrow < w.Lq) {
    const float lse = ltot > 0.0f ? (m + __builtin_log2f(ltot)) * kLn2 : -INFINITY;
    p.lse[(int64_t)w.b * p.l_bs + (int64_t)(w.q_start + qrow) * p.l_rs + (int64_t)h * p.l_hs] = lse;
  }
  const int lane = ql + 32 * hl;
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = RPI * k + lane / CPR, c = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * D + ((c ^ swz8<D>(row)) * 16));
    if (r0w + row < w.Lq) {
      const int64_t orow = (int64_t)w.b * p.o_bs + (int64_t)(w.q_start + r0w + row) * p.o_rs +
                           (int64_t)h * p.o_hs;
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(p.o) + orow + 16 * c) = v;
    }
  }
}

// Packed layout: the launch covers n_qtiles * rows_per_wg rows of every
// sequence (max_seqlen_q, which the caller promises bounds every length).  A
// longer sequence breaks that promise; its rows beyond the reach are written
// as NaN (O and LSE) by the workgroup of its first tile, so the broken promise
// shows in the result instead of leaving whatever the buffers held.
template <int OUT_ELEM, int D>
__device__ __forceinline__ void poison_beyond_reach(const FwdParams& p, const Work& w, int h) {
  const int reach = p.n_qtiles * p.rows_per_wg;
  if (p.cu_q == nullptr || w.r0 != 0 || w.Lq <= reach) return;
  const int n = (w.Lq - reach) * D;
  const int nt = kThreads / p.heads_per_wg;  // the threads of head h
  for (int e = threadIdx.x % nt; e < n; e += nt) {
    const int r = reach + e / D, d = e % D;
    const int64_t i = (int64_t)(w.q_start + r) * p.o_rs + (int64_t)h * p.o_hs + d;
    if constexpr (OUT_ELEM == E_F32) reinterpret_cast<float*>(p.o)[i] = __builtin_nanf("");
    else if constexpr (OUT_ELEM == E_E4M3) reinterpret_cast<uint8_t*>(p.o)[i] = 0x7F;
    else if constexpr (OUT_ELEM == E_F16) reinterpret_cast<uint16_t*>(p.o)[i] = 0x7E00;
    else reinterpret_cast<uint16_t*>(p.o)[i] = 0x7FC0;
    if (d == 0) p.lse[(int64_t)(w.q_start + r) * p.l_rs + (int64_t)h * p.l_hs] = __builtin_nanf("");
  }
}

// ---------------------------------------------------------------------------
// bf16 / f16 kernel
// ---------------------------------------------------------------------------
//
// One workgroup = 4 waves x 32 query rows (128 rows of one head, or 64 rows of
// two heads); three workgroups share a CU at D = 128 (four at D = 64), so the
// waves on a SIMD belong to independent workgroups and one's vector work
// (softmax) overlaps another's matrix work.  Per tile of BN keys a wave does
// BN/4 MFMAs for S^T = K Q^T, the softmax of its 32 x BN scores, and BN/4
// MFMAs for O^T += V^T P^T.
//
// K and V tiles reach LDS by DMA (buffer loads that write LDS directly: no
// staging registers, no vector instructions), double-buffered: the next tile
// is requested at the start of a tile and awaited at its end, and one
// workgroup barrier per tile publishes it.  That barrier orders LDS only, so
// it does not drain other requests.  The DMA is the compiler's buffer-to-LDS
// builtin; the two buffers of each pair are separate __shared__ arrays and the
// tile loop is unrolled by two, so the compiler relates every LDS read to the
// DMA into its own buffer and does not hold it for the other one.  Ordering
// is by the explicit vmcnt wait before each barrier.  V is stored
// row-major and read as the V^T operand with the transposing
// ds_read_b64_tr_b16.  Rows are stored unpadded with their 16-byte chunks
// XOR-swizzled by the row index, which keeps both read patterns free of bank
// conflicts: K fragments (16 rows x one chunk per 16 lanes) and V^T fragments
// (4 rows x 4 chunks per 32 lanes of a transposing read).  All LDS read
// addresses are computed once; tile-to-tile they differ by immediate offsets.
// The buffer range of a (sequence, kv head) ends at its last key, so rows past
// it arrive as zeros.

template <int ELEM, int D, int NKB>
struct Cfg5 {
  static constexpr int BN = 32 * NKB;                // keys per tile (NKB blocks of 32)
  static constexpr int NS = D / 16;                  // MFMA k-steps over d
  static constexpr int NOB = D / 32;                 // O^T accumulator blocks
  static constexpr int ROWB = D * 2;                 // bytes per K/V row in LDS
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;             // bytes of one K (or V) tile
  static constexpr int CPT = TILE / 16 / kThreads;   // DMA chunks per thread per tensor
  static_assert(CPT >= 1 && (TILE / 16) % kThreads == 0, "tile shape");
};

// Request one tile of K or V (BN rows from byte offset `base`) into an LDS
// tile buffer: this thread's chunk n goes to LDS chunk (wid*CPT + n)*64 + lane,
// from tile offset voff[n].  The instruction writes LDS only (no register
// results).
template <int ELEM, int D, int NKB>
__device__ __forceinline__ void dma_tile(uint8_t* buf, __amdgpu_buffer_rsrc_t rsrc, uint32_t base,
                                         int wid,
                                         const uint32_t (&voff)[Cfg5<ELEM, D, NKB>::CPT]) {
  using C = Cfg5<ELEM, D, NKB>;
  // the tile's base goes in the scalar offset: no per-tile vector add
  const uint32_t sb = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int n = 0; n < C::CPT; ++n) dma16(buf + (wid * C::CPT + n) * 1024, voff[n], rsrc, sb);
}

// Mask the S^T accumulators of the NKB 32-key blocks of a tile starting at key
// c0 for the lane's query row q.  Key of register r in block kb: c0 + 32 kb +
// kk(r) + 4 (lane / 32) with kk(r) = 8 (r / 4) + r % 4, so each test is one
// compare of a constant against a per-lane bound.
template <int NKB>
__device__ __forceinline__ void mask_blocks(f32x16 (&s)[NKB], int c0, int hl, int q, int off,
                                            int Lk, bool upper, int window) {
  const int base = c0 + 4 * hl;
  const int a = (upper ? min(Lk - 1, q + off) : Lk - 1) - base;  // visible iff key' <= a
  if (window > 0) {
    const int b = q + off - window + 1 - base;                   // ... and key' >= b
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * kb + 8 * (r >> 2) + (r & 3);
        if (kk > a || kk < b) s[kb][r] = -INFINITY;
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * kb + 8 * (r >> 2) + (r & 3);
        if (kk > a) s[kb][r] = -INFINITY;
      }
  }
}

template <int ELEM, int D, int NKB, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(WPE, WPE)))
void fwd16_kernel(FwdParams p) {
  using C = Cfg5<ELEM, D, NKB>;
  constexpr int BN = C::BN;
  constexpr int OUT = ELEM;
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lk1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv1[C::TILE];

  Work w;
  if (!decode_work(p, w)) return;

  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  // with two heads per workgroup, waves 0-1 take rows r0 .. r0+63 of head h0
  // and waves 2-3 the same rows of head h0+1
  const int wrow = p.heads_per_wg == 2 ? (wid & 1) : wid;  // the wave's 32-row block
  const int h = w.h0 + (p.heads_per_wg == 2 ? (wid >> 1) : 0);
  const int qrow = w.r0 + 32 * wrow + ql;  // this lane's query row within the sequence
  const float mul = p.score_mul;

  // Q^T fragments: lane holds q[qrow][16 ks + 8 hl .. +8]
  u32x4 qf[C::NS];
  {
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(p.q) +
                           ((int64_t)w.b * p.q_bs + (int64_t)w.q_start * p.q_rs +
                            (int64_t)h * p.q_hs) * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qbase, sat_bytes((int64_t)w.Lq * p.q_rs * 2));
    const uint32_t roff = (uint32_t)qrow * (uint32_t)(p.q_rs * 2);
#pragma unroll
    for (int ks = 0; ks < C::NS; ++ks) qf[ks] = bload16(qr, roff + (16 * ks + 8 * hl) * 2);
  }

  // K/V of this (sequence, kv head): descriptors and per-thread tile offsets
  __amdgpu_buffer_rsrc_t krs, vrs;
  uint32_t rs;
  {
    const int64_t koff = ((int64_t)w.b * p.k_bs + (int64_t)w.k_start * p.k_rs +
                          (int64_t)w.kvh * p.k_hs) * 2;
    const uint32_t bytes = sat_bytes((int64_t)w.Lk * p.k_rs * 2);
    krs = make_rsrc(reinterpret_cast<const uint8_t*>(p.k) + koff, bytes);
    vrs = make_rsrc(reinterpret_cast<const uint8_t*>(p.v) + koff, bytes);
    rs = (uint32_t)(p.k_rs * 2);
  }
  uint32_t voff[C::CPT];
#pragma unroll
  for (int n = 0; n < C::CPT; ++n) {
    const int P = (wid * C::CPT + n) * 64 + lane;
    const int row = P / C::CPR, ch = (P % C::CPR) ^ swz<D>(row);
    voff[n] = (uint32_t)row * rs + ch * 16;
  }
  // LDS read offsets (tile-relative), fixed for the whole loop:
  //  K fragment (kb, ks): row 32 kb + ql, logical chunk 2 ks + hl  (kb via +32 rows)
  //  (offset of step ks = koff0 ^ (ks << 5): the swizzled chunk index 2 ks + hl
  //  XOR swz(ql) differs from step 0's in chunk bits 1.. only)
  const uint32_t koff0 = (uint32_t)ql * C::ROWB + (uint32_t)((hl ^ swz<D>(ql)) * 16);
  //  V^T operand (t2, db), transposing read c: this lane supplies row
  //  16 t2 + 8 c + 4 (g / 2) + e, d = 32 db + 16 (g % 2) + 4 j, where g is the
  //  16-lane group, e = (lane % 16) / 4, j = lane % 4  (t2 via +16 rows)
  uint32_t voffs[C::NOB][2];
  {
    const int g = lane >> 4, e = (lane & 15) >> 2, j = lane & 3;
#pragma unroll
    for (int db = 0; db < C::NOB; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 8 * c + 4 * (g >> 1) + e;
        const int ch = 4 * db + 2 * (g & 1) + (j >> 1);
        voffs[db][c] = (uint32_t)row * C::ROWB + (uint32_t)((ch ^ swz<D>(row)) * 16) + (j & 1) * 8;
      }
  }

  const int off = w.Lk - w.Lq;
  const bool upper = p.causal || p.window > 0;
  int kv_lo, kv_hi;
  key_range(p, w, w.r0, min(w.r0 + p.rows_per_wg, w.Lq) - 1, kv_lo, kv_hi);
  const int t0 = kv_lo / BN;
  const int t1 = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : t0;
  int tv0, tv1, tm_lo, tm_hi;
  wave_tiles(p, w, 32 * wrow, BN, tv0, tv1, tm_lo, tm_hi);

  RowState<C::NOB> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int i = 0; i < C::NOB; ++i) st.o[i] = f32x16{};

  if (t0 < t1) {
    dma_tile<ELEM, D, NKB>(lk0, krs, (uint32_t)(t0 * BN) * rs, wid, voff);
    dma_tile<ELEM, D, NKB>(lv0, vrs, (uint32_t)(t0 * BN) * rs, wid, voff);
  }
  wait_vm_all();
  lds_barrier();

  auto tile = [&](int t, const uint8_t* kb_, const uint8_t* vb_, uint8_t* knext,
                  uint8_t* vnext) __attribute__((always_inline)) {
    if (t + 1 < t1) {
      const uint32_t base = (uint32_t)((t + 1) * BN) * rs;
      dma_tile<ELEM, D, NKB>(knext, krs, base, wid, voff);
      dma_tile<ELEM, D, NKB>(vnext, vrs, base, wid, voff);
    }
    const int c0 = t * BN;
    if (t >= tv0 && t < tv1) {
      // S^T = K Q^T for the two 32-key blocks
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::NS; ++ks) {
        const uint32_t ko = koff0 ^ (uint32_t)(ks << 5);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(kb_ + ko + kb * 32 * C::ROWB);
          s[kb] = mfma16<ELEM>(a, qf[ks], s[kb]);
        }
      }
      // four K fragment reads in flight ahead of the products (+1% measured)
      if constexpr (NKB == 1) sched_lds_ahead<C::NS, 1, 4>();
      if (t >= tm_hi || t < tm_lo) mask_blocks<NKB>(s, c0, hl, qrow, off, w.Lk, upper, p.window);

      // Online softmax over the row's BN scores (half here, half in lane ^ 32).
      // Optimistic: exponentiate against the current reference maximum and
      // move the reference only when some lane's partial sum exceeds 2^15
      // (or is not finite) -- the first tile of a row, or a large jump.  Then
      // the true tile maximum is taken, O and l are rescaled and the tile is
      // exponentiated again.  Any reference gives the exact result (numerator
      // and denominator share it); the bound only keeps P, l and O in range.
      u32x4 pk[2 * NKB];
      float part;
      auto exp_tile = [&](float ref) __attribute__((always_inline)) {
        float sum0 = 0.0f, sum1 = 0.0f;
#pragma unroll
        for (int t2 = 0; t2 < 2 * NKB; ++t2) {
          const f32x16& sb = s[t2 >> 1];
          const int r = 8 * (t2 & 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[r + 2 * i], mul, -ref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[r + 2 * i + 1], mul, -ref));
            sum0 = (t2 == 0 && i == 0) ? p0 : sum0 + p0;
            sum1 = (t2 == 0 && i == 0) ? p1 : sum1 + p1;
            pk[t2][i] = pack2<ELEM>(p0, p1);
          }
        }
        part = sum0 + sum1;
      };
      exp_tile(st.m);  // a row's first tile (m = -inf) gives a non-finite sum
      if (wave_any(!(part <= kPartialSumBound))) {
        float a = s[0][0], b = s[0][1];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = kb == 0 ? 2 : 0; r < 16; r += 2) {
            a = __builtin_elementwise_maximum(a, s[kb][r]);
            b = __builtin_elementwise_maximum(b, s[kb][r + 1]);
          }
        }
        const float mx = swap_halves_max(__builtin_elementwise_maximum(a, b)) * mul;
        const bool up = mx > st.m;  // -inf stays -inf
        const float alpha = up ? __builtin_amdgcn_exp2f(st.m - mx) : 1.0f;
        st.m = up ? mx : st.m;
        st.l *= alpha;
#pragma unroll
        for (int i = 0; i < C::NOB; ++i) st.o[i] *= alpha;
        exp_tile(st.m == -INFINITY ? 0.0f : st.m);
      }
      st.l += part;

      // O^T += V^T P^T
#pragma unroll
      for (int t2 = 0; t2 < 2 * NKB; ++t2) {
#pragma unroll
        for (int db = 0; db < C::NOB; ++db) {
          const u32x4 a = vt_operand(vb_ + voffs[db][0] + t2 * 16 * C::ROWB,
                                     vb_ + voffs[db][1] + t2 * 16 * C::ROWB);
          st.o[db] = mfma16<ELEM>(a, pk[t2], st.o[db]);
        }
      }
      // two V^T operands (two transposing reads each) in flight ahead of the
      // products (+1% measured)
      if constexpr (NKB == 1) sched_lds_ahead<2 * C::NOB, 2, 2>();
    }
    wait_vm_all();  // tile t+1 has landed (this wave's part)
    lds_barrier();  // ... and everyone's
  };

  int t = t0;
  for (; t + 1 < t1; t += 2) {
    tile(t, lk0, lv0, lk1, lv1);
    tile(t + 1, lk1, lv1, lk0, lv0);
  }
  if (t < t1) tile(t, lk0, lv0, lk1, lv1);

  // every wave has passed the last tile's barrier (or the prologue's): the
  // four K/V buffers are free, one per wave, each the size of its O tile
  static_assert(C::TILE >= 32 * 2 * D, "a K/V buffer holds one wave's O tile");
  uint8_t* stage = wid == 0 ? lk0 : wid == 1 ? lk1 : wid == 2 ? lv0 : lv1;
  store_row_staged<OUT, D>(p, w, h, w.r0 + 32 * wrow, ql, hl, st.m, st.l, st.o, stage);
  poison_beyond_reach<OUT, D>(p, w, h);
}

// ---------------------------------------------------------------------------
// E4M3 kernel: S^T on the FP8 matrix cores, P V in bf16
// ---------------------------------------------------------------------------
//
// The structure of the 16-bit kernel (128 query rows per workgroup, 4 waves x
// 32 rows, 32-key tiles, double-buffered LDS, one LDS-only barrier per tile),
// with two changes:
//   S^T = K Q^T runs on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, f32
//     accumulation; a lane holds row l % 32 and the 32 consecutive k elements
//     from 32 (l / 32)): A = K codes from LDS (two 16-byte reads), B = Q^T codes
//     kept in registers.  The per-tensor scales q_scale k_scale / sqrt(D) (times
//     log2 e) multiply the f32 scores.  K reaches LDS by DMA, unconverted.
//   P V stays on the bf16 matrix cores with P rounded to bf16: rounding P to
//     E4M3 instead (3 mantissa bits) moves O by up to ~2.5% of max|O| on
//     long, flat rows, which with the E4M3 rounding of the output exceeds the
//     6e-2 * max|O| tolerance.  V arrives as its bf16 copy (exact: every E4M3
//     value is a bf16 value), made by a widening launch on the same stream just
//     before, and reaches LDS by DMA in the 16-bit kernel's swizzled row layout,
//     so the same transposing reads build V^T.  (Widening each V tile inside
//     every workgroup that reads it cost ~16 vector instructions per tile and
//     wave, about a fifth of the kernel's time.)
// The epilogue multiplies by v_scale / o_scale and encodes E4M3 with round to
// nearest even, saturating at +-448.

template <int D>
struct Cfg8 {
  static constexpr int BN = 32;                      // keys per tile
  static constexpr int NS = D / 64;                  // 64-deep k-steps of S^T over d
  static constexpr int NOB = D / 32;                 // O^T accumulator blocks
  static constexpr int KROWB = D;                    // bytes per E4M3 K row in LDS
  static constexpr int KCPR = KROWB / 16;            // 16-byte chunks per K row
  static constexpr int KTILE = BN * KROWB;           // bytes of one K tile
  static constexpr int NCH = KTILE / 16;             // 16-byte chunks per K tile
  static constexpr int VROWB = 2 * D;                // bytes per bf16 V row in LDS
  static constexpr int VTILE = BN * VROWB;           // bytes of one bf16 V tile
  static_assert(NCH <= kThreads && NCH % 64 == 0, "tile shape");
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(D == 64 ? 4 : 3, D == 64 ? 4 : 3)))
void fwd8_kernel(FwdParams p) {
  using C = Cfg8<D>;
  using V16 = Cfg5<E_BF16, D, 1>;  // the bf16 V tile layout of the 16-bit kernel
  constexpr int BN = C::BN;
  static_assert(V16::TILE == C::VTILE, "V tile");
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[C::KTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lk1[C::KTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv0[C::VTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv1[C::VTILE];

  Work w;
  if (!decode_work(p, w)) return;

  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  const int h = w.h0;
  const int qrow = w.r0 + 32 * wid + ql;
  const float mul = p.score_mul;

  // Q^T codes: lane holds q[qrow][64 ks + 32 hl .. +32]
  u32x4 qf[C::NS][2];
  {
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(p.q) +
                           ((int64_t)w.b * p.q_bs + (int64_t)w.q_start * p.q_rs +
                            (int64_t)h * p.q_hs);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qbase, sat_bytes((int64_t)w.Lq * p.q_rs));
    const uint32_t roff = (uint32_t)qrow * (uint32_t)p.q_rs;
#pragma unroll
    for (int ks = 0; ks < C::NS; ++ks) {
      qf[ks][0] = bload16(qr, roff + 64 * ks + 32 * hl);
      qf[ks][1] = bload16(qr, roff + 64 * ks + 32 * hl + 16);
    }
  }

  // K codes and V of this (sequence, kv head).  p.v is the bf16 copy of the V
  // codes (exact, made by the launch before this one), with the codes'
  // element strides: V tiles reach LDS by DMA in the 16-bit kernel's layout,
  // with no vector work.
  __amdgpu_buffer_rsrc_t krs, vrs;
  uint32_t rs;  // bytes per K row; a V row has twice as many
  {
    const int64_t koff = (int64_t)w.b * p.k_bs + (int64_t)w.k_start * p.k_rs +
                         (int64_t)w.kvh * p.k_hs;
    const int64_t bytes = (int64_t)w.Lk * p.k_rs;
    krs = make_rsrc(reinterpret_cast<const uint8_t*>(p.k) + koff, sat_bytes(bytes));
    vrs = make_rsrc(reinterpret_cast<const uint8_t*>(p.v) + 2 * koff, sat_bytes(2 * bytes));
    rs = (uint32_t)p.k_rs;
  }
  // this thread's 16-byte chunk of a K tile, if any (wave-uniform)
  const bool has_chunk = wid * 64 < C::NCH;
  const int crow = tid / C::KCPR, cch = tid % C::KCPR;
  const uint32_t kdma = (uint32_t)crow * rs + (uint32_t)((cch ^ swz8<D>(crow)) * 16);
  auto dma_k = [&](uint8_t* buf, uint32_t base) __attribute__((always_inline)) {
    if (has_chunk) {
      dma16(buf + wid * 1024, kdma, krs, __builtin_amdgcn_readfirstlane(base));
    }
  };
  // ... and its chunks of a bf16 V tile
  uint32_t vdma[V16::CPT];
#pragma unroll
  for (int n = 0; n < V16::CPT; ++n) {
    const int P = (wid * V16::CPT + n) * 64 + lane;
    const int row = P / V16::CPR, ch = (P % V16::CPR) ^ swz<D>(row);
    vdma[n] = (uint32_t)row * (2 * rs) + ch * 16;
  }
  // LDS read offsets (tile-relative):
  //  K for step ks: row ql, chunks 4 ks + 2 hl and 4 ks + 2 hl + 1
  uint32_t koffs[C::NS][2];
#pragma unroll
  for (int ks = 0; ks < C::NS; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      koffs[ks][c] = (uint32_t)ql * C::KROWB + (uint32_t)(((4 * ks + 2 * hl + c) ^ swz8<D>(ql)) * 16);
  //  V^T operands: as in the 16-bit kernel
  uint32_t voffs[C::NOB][2];
  {
    const int g = lane >> 4, e = (lane & 15) >> 2, j = lane & 3;
#pragma unroll
    for (int db = 0; db < C::NOB; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 8 * c + 4 * (g >> 1) + e;
        const int ch = 4 * db + 2 * (g & 1) + (j >> 1);
        voffs[db][c] = (uint32_t)row * C::VROWB + (uint32_t)((ch ^ swz<D>(row)) * 16) + (j & 1) * 8;
      }
  }

  const int off = w.Lk - w.Lq;
  const bool upper = p.causal || p.window > 0;
  int kv_lo, kv_hi;
  key_range(p, w, w.r0, min(w.r0 + p.rows_per_wg, w.Lq) - 1, kv_lo, kv_hi);
  const int t0 = kv_lo / BN;
  const int t1 = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : t0;
  int tv0, tv1, tm_lo, tm_hi;
  wave_tiles(p, w, 32 * wid, BN, tv0, tv1, tm_lo, tm_hi);

  RowState<C::NOB> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int i = 0; i < C::NOB; ++i) st.o[i] = f32x16{};

  if (t0 < t1) {
    dma_k(lk0, (uint32_t)(t0 * BN) * rs);
    dma_tile<E_BF16, D, 1>(lv0, vrs, (uint32_t)(t0 * BN) * 2 * rs, wid, vdma);
  }
  // on every path (with no tile too), so that no load, the Q codes included,
  // is in flight when the tile loop starts: otherwise the compiler's wait
  // insertion carries the Q code loads into the loop as pending and waits for
  // each tile's prefetch before the tile's second score MFMA
  wait_vm_all();
  lds_barrier();

  auto tile = [&](int t, const uint8_t* kb_, const uint8_t* vb_, uint8_t* knext,
                  uint8_t* vnext) __attribute__((always_inline)) {
    if (t + 1 < t1) {
      const uint32_t base = (uint32_t)((t + 1) * BN) * rs;
      dma_k(knext, base);
      dma_tile<E_BF16, D, 1>(vnext, vrs, 2 * base, wid, vdma);
    }
    const int c0 = t * BN;
    if (t >= tv0 && t < tv1) {
      f32x16 s[1] = {f32x16{}};
#pragma unroll
      for (int ks = 0; ks < C::NS; ++ks) {
        const u32x4 a[2] = {*reinterpret_cast<const u32x4*>(kb_ + koffs[ks][0]),
                            *reinterpret_cast<const u32x4*>(kb_ + koffs[ks][1])};
        s[0] = mfma_fp8(a, qf[ks], s[0]);
      }
      if (t >= tm_hi || t < tm_lo) mask_blocks<1>(s, c0, hl, qrow, off, w.Lk, upper, p.window);

      // optimistic softmax, exactly as in the 16-bit kernel
      u32x4 pk[2];
      float part;
      auto exp_tile = [&](float ref) __attribute__((always_inline)) {
        float sum0 = 0.0f, sum1 = 0.0f;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int r = 8 * t2;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][r + 2 * i], mul, -ref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][r + 2 * i + 1], mul, -ref));
            sum0 = (t2 == 0 && i == 0) ? p0 : sum0 + p0;
            sum1 = (t2 == 0 && i == 0) ? p1 : sum1 + p1;
            pk[t2][i] = pack2<E_BF16>(p0, p1);
          }
        }
        part = sum0 + sum1;
      };
      exp_tile(st.m);  // a row's first tile (m = -inf) gives a non-finite sum
      if (wave_any(!(part <= kPartialSumBound))) {
        float a = s[0][0], b = s[0][1];
#pragma unroll
        for (int r = 2; r < 16; r += 2) {
          a = __builtin_elementwise_maximum(a, s[0][r]);
          b = __builtin_elementwise_maximum(b, s[0][r + 1]);
        }
        const float mx = swap_halves_max(__builtin_elementwise_maximum(a, b)) * mul;
        const bool up = mx > st.m;  // -inf stays -inf
        const float alpha = up ? __builtin_amdgcn_exp2f(st.m - mx) : 1.0f;
        st.m = up ? mx : st.m;
        st.l *= alpha;
#pragma unroll
        for (int i = 0; i < C::NOB; ++i) st.o[i] *= alpha;
        exp_tile(st.m == -INFINITY ? 0.0f : st.m);
      }
      st.l += part;

      // O^T += V^T P^T (bf16)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int db = 0; db < C::NOB; ++db) {
          const u32x4 a = vt_operand(vb_ + voffs[db][0] + t2 * 16 * C::VROWB,
                                     vb_ + voffs[db][1] + t2 * 16 * C::VROWB);
          st.o[db] = mfma16<E_BF16>(a, pk[t2], st.o[db]);
        }
      }
      sched_lds_ahead<2 * C::NOB, 2, 2>();
    }
    wait_vm_all();  // the K and V DMA of tile t+1 have landed (this wave's part)
    lds_barrier();  // ... and everyone's
  };

  int t = t0;
  for (; t + 1 < t1; t += 2) {
    tile(t, lk0, lv0, lk1, lv1);
    tile(t + 1, lk1, lv1, lk0, lv0);
  }
  if (t < t1) tile(t, lk0, lv0, lk1, lv1);

  // every wave has passed the last tile's barrier: the K (32 D bytes each)
  // and V (64 D bytes each) buffers are free, one per wave
  static_assert(C::KTILE >= 32 * D && C::VTILE >= 32 * D, "a buffer holds a wave's O codes");
  uint8_t* stage = wid == 0 ? lk0 : wid == 1 ? lk1 : wid == 2 ? lv0 : lv1;
  store_row_staged8<D>(p, w, h, w.r0 + 32 * wid, ql, hl, st.m, st.l, st.o, stage);
  poison_beyond_reach<E_E4M3, D>(p, w, h);
}
// ---------------------------------------------------------------------------
// f32 kernel (v_mfma_f32_32x32x2_f32: exact products, f32 accumulation)
// ---------------------------------------------------------------------------
//
// 4 waves x 32 query rows of one head per workgroup.  The d contraction order
// is permuted consistently for Q and K: MFMA step s, lane half h <-> d =
// (D/2) h + s, so each lane reads contiguous d values.  P.V: step r of key
// block kb pairs the keys 32 kb + 8 (r/4) + 4 h + r%4 (h = lane half), which
// is exactly what accumulator register r holds, so P needs no movement and V
// stays row-major in LDS.

// One online-softmax step over the 64 scores of this lane's row, exact for the
// row maximum: score * mul is rounded on its own before the reference is
// subtracted, so the maximal score maps to exactly exp2(0) = 1.
template <int NOB>
__device__ __forceinline__ void softmax_step_exact(f32x16 (&s)[2], RowState<NOB>& st, float mul) {
  const float mx = tile_row_max(s) * mul;  // -inf stays -inf
  if (wave_any(mx > st.m + kRescaleSlack)) rescale_row<NOB>(mx, st.m, st.l, st.o);
  const float ref = st.m == -INFINITY ? 0.0f : st.m;
  float sum = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float arg;
      {
#pragma clang fp contract(off)
        const float t = s[kb][r] * mul;  // rounded on its own, not fused into the subtraction
        arg = t - ref;
      }
      const float pr = __builtin_amdgcn_exp2f(arg);
      s[kb][r] = pr;
      sum += pr;
    }
  }
  st.l += sum;
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 2)))
void fwd32_kernel(FwdParams p) {
  constexpr int P32 = D + 4;  // LDS row pitch (floats)
  constexpr int NOB = D / 32;
  constexpr int CPR = D / 4;                      // 16-byte chunks per row
  constexpr int CPT = kBlockN * CPR / kThreads;   // per thread, per tensor
  __shared__ __attribute__((aligned(16))) float sK[2][kBlockN * P32];
  __shared__ __attribute__((aligned(16))) float sV[2][kBlockN * P32];

  Work w;
  if (!decode_work(p, w)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  const int h = w.h0;
  const int qrow = w.r0 + wid * 32 + ql;

  float qf[D / 2];
  {
    const float* qb = reinterpret_cast<const float*>(p.q) + (int64_t)w.b * p.q_bs +
                      (int64_t)(w.q_start + qrow) * p.q_rs + (int64_t)h * p.q_hs + (D / 2) * hl;
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      if (qrow < w.Lq) z = *reinterpret_cast<const f32x4*>(qb + s);
      qf[s] = z[0]; qf[s + 1] = z[1]; qf[s + 2] = z[2]; qf[s + 3] = z[3];
    }
  }

  RowState<NOB> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int i = 0; i < NOB; ++i) st.o[i] = f32x16{};

  const int rlast = min(w.r0 + p.rows_per_wg, w.Lq) - 1;
  int kv_lo, kv_hi;
  key_range(p, w, w.r0, rlast, kv_lo, kv_hi);
  const int wa = w.r0 + wid * 32, wb = min(w.r0 + wid * 32 + 31, w.Lq - 1);
  int wlo, whi;
  key_range(p, w, wa, wb, wlo, whi);
  const bool wave_live = wa <= wb;
  const int off = w.Lk - w.Lq;
  const bool upper = p.causal || p.window > 0;
  const int t0 = kv_lo / kBlockN;
  const int t1 = kv_hi > kv_lo ? (kv_hi + kBlockN - 1) / kBlockN : t0;

  const float* kbase = reinterpret_cast<const float*>(p.k) + (int64_t)w.b * p.k_bs +
                       (int64_t)w.k_start * p.k_rs + (int64_t)w.kvh * p.k_hs;
  const float* vbase = reinterpret_cast<const float*>(p.v) + (int64_t)w.b * p.k_bs +
                       (int64_t)w.k_start * p.k_rs + (int64_t)w.kvh * p.k_hs;
  f32x4 rk[CPT], rv[CPT];
  auto load = [&](int c0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = c * kThreads + tid, row = idx / CPR, col = idx % CPR;
      const int key = c0 + row;
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, bb = {0.f, 0.f, 0.f, 0.f};
      if (key < w.Lk) {
        a = *reinterpret_cast<const f32x4*>(kbase + (int64_t)key * p.k_rs + col * 4);
        bb = *reinterpret_cast<const f32x4*>(vbase + (int64_t)key * p.k_rs + col * 4);
      }
      rk[c] = a;
      rv[c] = bb;
    }
  };
  if (t0 < t1) load(t0 * kBlockN);

  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    float* k_s = sK[buf];
    float* v_s = sV[buf];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = c * kThreads + tid, row = idx / CPR, col = idx % CPR;
      *reinterpret_cast<f32x4*>(k_s + row * P32 + col * 4) = rk[c];
      *reinterpret_cast<f32x4*>(v_s + row * P32 + col * 4) = rv[c];
    }
    __syncthreads();
    if (t + 1 < t1) load((t + 1) * kBlockN);

    const int c0 = t * kBlockN;
    if (!wave_live || c0 >= whi || c0 + kBlockN <= wlo) continue;

    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < D / 2; ks += 4) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(k_s + ql * P32 + (D / 2) * hl + ks);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(k_s + (32 + ql) * P32 + (D / 2) * hl + ks);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[e], qf[ks + e], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[e], qf[ks + e], s[1], 0, 0, 0);
      }
    }

    const bool need_mask = (c0 + kBlockN > w.Lk) || (upper && c0 + kBlockN - 1 > wa + off) ||
                           (p.window > 0 && c0 < wb + off - p.window + 1);
    if (need_mask) mask_tile(s, c0, hl, qrow, off, w.Lk, upper, p.window);

    softmax_step_exact<NOB>(s, st, p.score_mul);

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
#pragma unroll
        for (int db = 0; db < NOB; ++db) {
          const float a = v_s[key * P32 + db * 32 + ql];
          st.o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][r], st.o[db], 0, 0, 0);
        }
      }
    }
  }

  store_row<E_F32, D>(p, w, h, qrow, hl, st.m, st.l, st.o);
  poison_beyond_reach<E_F32, D>(p, w, h);
}

// ---------------------------------------------------------------------------
// host planning and launch
// ---------------------------------------------------------------------------

constexpr int kTwoHeadMinRows = 4096;  // max_seqlen_q from which the 16-bit kernel takes two heads

bool plan_fwd(FwdParams& p, int elem, int head_dim) {
  // 4 waves x 32 query rows per workgroup: 128 rows of one head, or for the
  // 16-bit kernel on long sequences (an even group) 64 rows of two heads of
  // the group, whose waves then see the same keys (measured +0.5% on the
  // long-context and +1% on the window workload, -1 to -3% on sequences of
  // 128-2048 tokens)
  const bool two = (elem == E_BF16 || elem == E_F16) && p.group % 2 == 0 &&
                   p.max_seqlen_q >= kTwoHeadMinRows;
  p.heads_per_wg = two ? 2 : 1;
  p.rows_per_wg = two ? 64 : 128;
  const int64_t n_qtiles = ((int64_t)p.max_seqlen_q + p.rows_per_wg - 1) / p.rows_per_wg;
  const int64_t n_groups = n_qtiles * p.batch * p.kv_heads;
  if (n_groups > INT32_MAX / 8) return false;
  p.n_qtiles = (int32_t)n_qtiles;
  p.n_groups = (int32_t)n_groups;
  return fwd_grid_size(p) <= (int64_t)UINT32_MAX / 2 && head_dim > 0;
}

#ifndef VLGQA_NKB
#define VLGQA_NKB 1
#endif
#ifndef VLGQA_WPE
#define VLGQA_WPE 3
#endif
constexpr int kTicketSlots = 64;    // streams per device with run-time hand-out
constexpr int kTicketDevices = 64;
constexpr int kNkb = VLGQA_NKB;  // 32-key blocks per tile of the bf16/f16 kernel
constexpr int kWpe = VLGQA_WPE;  // its waves per SIMD (D = 128)
constexpr int kWpe64 = 4;        // at D = 64 (about 100 VGPRs, 16 KB of LDS a workgroup)

// Claim counters of the run-time hand-out, 128 bytes apart: one per
// (device, stream) the forward has launched on.
static __device__ unsigned run_ticket[kTicketSlots * 32];

namespace {
std::mutex g_ticket_mutex;
unsigned* g_ticket_base_ptr[kTicketDevices] = {};
struct TicketSlot {
  int index;
  unsigned next;  // the counter's value once the launches enqueued so far have run
};
std::map<std::pair<int, hipStream_t>, TicketSlot> g_ticket_slots;
int g_ticket_used[kTicketDevices] = {};
}  // namespace

TicketLease ticket_lease(hipStream_t stream) {
  TicketLease l;
  l.lock = std::unique_lock<std::mutex>(g_ticket_mutex);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  int dev = -1;
  if (stream == hipStreamPerThread ||
      hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone ||
      hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kTicketDevices) {
    l.lock.unlock();
    return l;
  }
  if (!g_ticket_base_ptr[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(run_ticket)) != hipSuccess) {
      l.lock.unlock();
      return l;
    }
    g_ticket_base_ptr[dev] = static_cast<unsigned*>(a);
  }
  auto key = std::make_pair(dev, stream);
  auto it = g_ticket_slots.find(key);
  if (it == g_ticket_slots.end()) {
    if (g_ticket_used[dev] >= kTicketSlots) {
      l.lock.unlock();
      return l;
    }
    it = g_ticket_slots.emplace(key, TicketSlot{g_ticket_used[dev]++, 0u}).first;
  }
  l.counter = g_ticket_base_ptr[dev] + 32 * it->second.index;
  l.next = &it->second.next;
  return l;
}

hipError_t launch_fwd(const FwdParams& p0, int elem, int head_dim, hipStream_t stream) {
  FwdParams p = p0;
  TicketLease lease;
  {
    const int G2 = p.group / p.heads_per_wg;
    const int64_t slots = ((int64_t)p.n_groups + 7) / 8 * G2;  // per XCD
    const int64_t tail = tail_slots(slots);
    if (tail > 0) {
      lease = ticket_lease(stream);
      if (lease.counter) {
        p.ticket = lease.counter;
        p.ticket_base = lease.base();
        p.n_static = (int32_t)(slots - tail);
        p.n_tail = (int32_t)(8 * tail);
        p.n_claim = (int32_t)claim_blocks(tail);
      }
    }
  }
  const int64_t grid = fwd_grid_size(p);
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), b(kThreads);
#define VLGQA_LAUNCH(KERNEL) hipLaunchKernelGGL((KERNEL), g, b, 0, stream, p)
  if (head_dim == 128) {
    switch (elem) {
      case E_BF16: VLGQA_LAUNCH((fwd16_kernel<E_BF16, 128, kNkb, kWpe>)); break;
      case E_F16: VLGQA_LAUNCH((fwd16_kernel<E_F16, 128, kNkb, kWpe>)); break;
      case E_E4M3: VLGQA_LAUNCH((fwd8_kernel<128>)); break;
      case E_F32: VLGQA_LAUNCH((fwd32_kernel<128>)); break;
      default: return hipErrorInvalidValue;
    }
  } else if (head_dim == 64) {
    switch (elem) {
      case E_BF16: VLGQA_LAUNCH((fwd16_kernel<E_BF16, 64, kNkb, kWpe64>)); break;
      case E_F16: VLGQA_LAUNCH((fwd16_kernel<E_F16, 64, kNkb, kWpe64>)); break;
      case E_E4M3: VLGQA_LAUNCH((fwd8_kernel<64>)); break;
      case E_F32: VLGQA_LAUNCH((fwd32_kernel<64>)); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef VLGQA_LAUNCH
  const hipError_t e = hipGetLastError();
  // the counter moves only for a launch that was enqueued
  if (p.ticket && e == hipSuccess) lease.advance((unsigned)p.n_claim);
  return e;
}

}  // namespace vlgqa
