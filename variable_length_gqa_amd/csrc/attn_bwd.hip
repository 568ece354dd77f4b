// Fused attention backward for gfx950 (CDNA4): packed varlen and dense layouts,
// GQA, causal / sliding-window masks, bf16 / f16 / E4M3 storage, f32
// accumulation.
//
// What is computed (the gradient of the forward, for the interface of boostr
// varlen_attention.rs ``varlen_attention_bwd`` and boostr flash.rs
// ``flash_attention_bwd``: dout, q, k, v, the forward output and its
// logsumexp in, dq / dk / dv out, dk and dv shaped like k and v under GQA):
//   P_ij  = exp(scale q_i.k_j - LSE_i)            (recomputed from the LSE)
//   dv_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i.v_j - delta_i),   delta_i = dO_i.O_i
//   dq_i  = scale sum_j dS_ij k_j,       dk_j = scale sum_i dS_ij q_i
// with dk / dv of a kv head summed over its G query heads.
//
// Two launches (three with the dK / dV reduction, more for E4M3 inputs):
//   bwd_dq_kernel      one workgroup per (sequence, 128-row query tile, query
//                      head), the forward's structure: K/V tiles of 32 keys by
//                      DMA into LDS, Q^T and dO^T in registers, dQ^T in
//                      registers.  It first computes the row terms of its rows,
//                      delta_i = dO_i.O_i and LSE_i log2(e), and writes them
//                      head-major into the caller's workspace (so a query
//                      tile's values are contiguous) for the next launch.
//   bwd_kv_kernel      dK and dV in one pass (E4M3: dV, then dK, two
//                      launches of one body): one workgroup per (sequence,
//                      kv head, 128-key tile), 4 waves x 32 keys; K of the
//                      wave's keys stays in registers, V in LDS (E4M3: both
//                      in registers); the loop runs over the group's query
//                      heads and the 32-row query tiles that see the keys,
//                      with Q, dO and the tile's LSE / delta brought to LDS by
//                      DMA (double buffered).  dV / dK accumulate in
//                      registers: no atomics, deterministic.  On long loops
//                      the group's heads are split in two halves, one
//                      workgroup each, whose f32 partial sums
//   bwd_reduce_kernel  adds in a fixed order before storing dk and dv.
// Matrix-core formulation (v_mfma_f32_32x32x16_{bf16,f16}): every product has
// the operand layouts of the forward kernel.  In dK/dV the lane owns a key:
//   S  = Q K^T     A = Q rows (LDS), B = K^T (registers)  -> lane: key l % 32,
//   dP = dO V^T    A = dO rows (LDS), B = V^T (LDS rows)     16 query rows
//   dV^T += dO^T P     A = dO^T by transposing LDS reads, B = P (bf16)
//   dK^T += Q^T dS     A = Q^T by transposing LDS reads,  B = dS (bf16)
// In dQ the lane owns a query:
//   S^T = K Q^T, dP^T = V dO^T   A = K / V rows (LDS), B = Q^T / dO^T (registers)
//   dQ^T += K^T dS^T             A = K^T by transposing LDS reads, B = dS^T
//
// E4M3 inputs (boostr flash.rs ``flash_attention_bwd_fp8``: per-tensor
// dequantisation scales for q, k, v, dout and the forward output, quantisation
// scales for dq, dk, dv): the codes of q, k, v and dout are first widened to
// bf16 (exact: every E4M3 value is a bf16 value) into the workspace, and the
// same kernels run on those copies with the scales folded into their
// multipliers: scores q_scale k_scale / sqrt(D), dP do_scale v_scale, delta
// do_scale o_scale (taken from the codes of dout and of the output), stored
// gradients dq k_scale / (sqrt(D) dq_scale), dk q_scale / (sqrt(D) dk_scale),
// dv do_scale / dv_scale, encoded as E4M3 with round to nearest even,
// saturating at +-448.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bwd_params.h"
#include "kernel_common.h"
#include "pack_api.h"

namespace vlgqa {

constexpr int kTileB = 128;  // keys per dK/dV workgroup, query rows per dQ workgroup

template <int ELEM>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (ELEM == E_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  } else {
    return __uint_as_float(w << 16);
  }
}
template <int ELEM>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (ELEM == E_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  } else {
    return __uint_as_float(w & 0xFFFF0000u);
  }
}

// Workspace layout (f32): [2][B][H][rows]: plane 0 = LSE * log2(e) (+inf for a
// row with no visible key, so its weights are exp2(-inf) = 0), plane 1 = delta.
// Dense: rows = S_q per batch; packed: B = 1 and rows = total_q.
__device__ __forceinline__ int64_t ws_index(const BwdParams& p, int b, int64_t r, int h) {
  return ((int64_t)b * p.heads + h) * p.d_rows + r;
}
__device__ __forceinline__ int64_t ws_plane(const BwdParams& p) {
  return (int64_t)p.d_batch * p.heads * p.d_rows;
}

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------

struct SeqBounds {
  int q_start, Lq, k_start, Lk;
};

__device__ __forceinline__ SeqBounds seq_bounds(const BwdParams& p, int b) {
  SeqBounds s{0, p.seqlen_q, 0, p.seqlen_k};
  if (p.cu_q) {
    s.q_start = p.cu_q[b];
    s.Lq = p.cu_q[b + 1] - s.q_start;
  }
  if (p.cu_k) {
    s.k_start = p.cu_k[b];
    s.Lk = p.cu_k[b + 1] - s.k_start;
  }
  return s;
}

// the 16-bit tile layout of the forward kernel: 32 rows of D elements, rows
// unpadded, 16-byte chunks XOR-swizzled by swz<D>(row)
template <int D>
struct T16 {
  static constexpr int ROWB = 2 * D;
  static constexpr int CPR = ROWB / 16;
  static constexpr int TILE = 32 * ROWB;
  static constexpr int CPT = TILE / 16 / kThreads;   // DMA chunks per thread
  static constexpr int NS = D / 16;
  static constexpr int NOB = D / 32;
  static_assert(CPT >= 1 && (TILE / 16) % kThreads == 0, "tile shape");
};

// per-thread DMA offsets of a 32-row tile whose rows are rs bytes apart
template <int D>
__device__ __forceinline__ void tile_dma_offsets(uint32_t (&voff)[T16<D>::CPT], int wid, int lane,
                                                 uint32_t rs) {
  using C = T16<D>;
#pragma unroll
  for (int n = 0; n < C::CPT; ++n) {
    const int P = (wid * C::CPT + n) * 64 + lane;
    const int row = P / C::CPR, ch = (P % C::CPR) ^ swz<D>(row);
    voff[n] = (uint32_t)row * rs + ch * 16;
  }
}

template <int D>
__device__ __forceinline__ void dma_tile16(const uint8_t* buf, __amdgpu_buffer_rsrc_t rsrc,
                                           uint32_t base, int wid,
                                           const uint32_t (&voff)[T16<D>::CPT]) {
  using C = T16<D>;
#pragma unroll
  for (int n = 0; n < C::CPT; ++n) dma16(buf + (wid * C::CPT + n) * 1024, base + voff[n], rsrc);
}

// row-operand read offset of lane (row ql, half hl) for k-step 0: the
// offset of step ks is this ^ (ks << 5) (as in the forward)
template <int D>
__device__ __forceinline__ uint32_t row_read_off(int ql, int hl) {
  return (uint32_t)ql * T16<D>::ROWB + (uint32_t)((hl ^ swz<D>(ql)) * 16);
}

// E4M3 tiles (32 rows of D codes, 16-byte chunks XOR-swizzled by swz8): the
// DMA chunk of thread tid (row tid / (D/16)); false for threads past the
// tile's 2 D chunks (D = 64: waves 2 and 3)
template <int D>
__device__ __forceinline__ bool tile8_dma_offset(uint32_t& voff, int tid, uint32_t rs) {
  const int crow = tid / (D / 16), cch = tid % (D / 16);
  voff = (uint32_t)crow * rs + (uint32_t)((cch ^ swz8<D>(crow)) * 16);
  return tid < 2 * D;
}

// the A (or B) operand of v_mfma_f32_32x32x64_f8f6f4 for k-step ks: row ql,
// codes 64 ks + 32 hl .. +32, as two 16-byte LDS reads
template <int D>
__device__ __forceinline__ void tile8_read(const uint8_t* t, int ql, int hl, int ks, u32x4 (&a)[2]) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
    a[c] = *reinterpret_cast<const u32x4*>(
        t + (uint32_t)ql * D + (uint32_t)(((4 * ks + 2 * hl + c) ^ swz8<D>(ql)) * 16));
}

// transposing-read offsets (the forward's V^T operand)
template <int D>
__device__ __forceinline__ void tr_read_offsets(uint32_t (&o)[T16<D>::NOB][2], int lane) {
  const int g = lane >> 4, e = (lane & 15) >> 2, j = lane & 3;
#pragma unroll
  for (int db = 0; db < T16<D>::NOB; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 8 * c + 4 * (g >> 1) + e;
      const int ch = 4 * db + 2 * (g & 1) + (j >> 1);
      o[db][c] = (uint32_t)row * T16<D>::ROWB + (uint32_t)((ch ^ swz<D>(row)) * 16) + (j & 1) * 8;
    }
}

// store a [key or query][d] row block held as 32-row accumulators (lane: row
// l % 32, d = 32 db + 8 (r / 4) + 4 (l / 32) + r % 4), times mul
template <int ELEM, int D>
__device__ __forceinline__ void store_rows(void* base, int64_t row_off, int hl,
                                           const f32x16 (&acc)[D / 32], float mul) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + g * 8 + 4 * hl;
      const u32x2 v = {pack2<ELEM>(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul),
                       pack2<ELEM>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + row_off + d0) = v;
    }
  }
}

// The same row block through LDS: the wave writes its 32 x D tile (times
// mul, 16-bit or E4M3) into `stage` (32 rows of D elements, 16-byte chunks
// XOR-swizzled by row), reads it back a row chunk per lane and stores whole
// rows with 16-byte stores: rows first + i * rs (in elements) for i < nrows.
template <int OUT, int D>
__device__ __forceinline__ void store_rows_staged(void* base, int64_t first, int64_t rs, int nrows,
                                                  int ql, int hl, const f32x16 (&acc)[D / 32],
                                                  float mul, uint8_t* stage) {
  constexpr int EB = OUT == E_E4M3 ? 1 : 2;  // bytes per element
  constexpr int ROWB = D * EB, CPR = ROWB / 16;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // elements d = 32 db + 8 g + 4 hl .. +4
      const float x0 = acc[db][4 * g + 0] * mul, x1 = acc[db][4 * g + 1] * mul;
      const float x2 = acc[db][4 * g + 2] * mul, x3 = acc[db][4 * g + 3] * mul;
      if constexpr (OUT == E_E4M3) {
        const int c = 2 * db + (g >> 1);
        *reinterpret_cast<uint32_t*>(stage + ql * ROWB + ((c ^ swz8<D>(ql)) * 16) + 8 * (g & 1) +
                                     4 * hl) =
            pack4_fp8(sat448(x0), sat448(x1), sat448(x2), sat448(x3));
      } else {
        const int c = 4 * db + g;
        const u32x2 v = {pack2<OUT>(x0, x1), pack2<OUT>(x2, x3)};
        *reinterpret_cast<u32x2*>(stage + ql * ROWB + ((c ^ swz<D>(ql)) * 16) + 8 * hl) = v;
      }
    }
  }
  const int lane = ql + 32 * hl;
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = RPI * k + lane / CPR, c = lane % CPR;
    const int pc = OUT == E_E4M3 ? (c ^ swz8<D>(row)) : (c ^ swz<D>(row));
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * ROWB + pc * 16);
    if (row < nrows)
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(base) + (first + row * rs) * EB +
                                16 * c) = v;
  }
}

// ---------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------
//
// One kernel body, three modes.  MODE_DKV (16-bit inputs) computes S, dP ->
// P, dS -> dV^T += dO^T P and dK^T += Q^T dS in one pass: K^T of the lane's
// key in registers, V of the workgroup's 128 keys in LDS (read as the B
// operand of dP each stage), both accumulators in registers (two waves per
// SIMD at D = 128).  MODE_DV (S -> P -> dV^T) and MODE_DK (S, dP -> dS ->
// dK^T, K^T and V^T in registers) are two launches of the E4M3 path, whose
// FP8 operands do not leave room for the fused body.
enum : int { MODE_DV = 0, MODE_DK = 1, MODE_DKV = 2 };

// E8: E4M3 inputs.  S = Q K^T (and dP = dO V^T) run on the FP8 matrix cores
// from the codes (K^T / V^T codes in registers, Q / dO code tiles in LDS); the
// accumulation products keep the bf16 copies (dO tile for dV, Q tile for dK).
template <int ELEM, int D, int MODE, int E8>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(MODE == MODE_DV || E8 || D == 64 ? 3 : 2,
                                              MODE == MODE_DV || E8 || D == 64 ? 3 : 2)))
void bwd_kv_kernel(BwdParams p) {
  using C = T16<D>;
  constexpr bool FUSED = MODE == MODE_DKV;
  static_assert(!(FUSED && E8), "the fused body takes 16-bit inputs");
  constexpr int T8 = 32 * D;  // bytes of an E4M3 tile
  // stage buffer (byte offsets): the S operand tile, the dP operand tile (dK),
  // the transposed-read tile of the accumulation, then 32 lse2 + 32 delta
  // floats.  16-bit: Q, dO (both roles); E8 dV: Q8, dO; E8 dK: Q8, dO8, Q.
  constexpr int OFF_S = 0;
  constexpr int OFF_DP = E8 ? T8 : C::TILE;
  constexpr int OFF_T = !E8 ? (MODE == MODE_DV ? C::TILE : 0) : (MODE == MODE_DV ? T8 : 2 * T8);
  constexpr int OFF_W = !E8 ? 2 * C::TILE : (MODE == MODE_DV ? T8 + C::TILE : 2 * T8 + C::TILE);
  constexpr int STAGE = OFF_W + 256;
  // fused: V rows of the workgroup's keys (4 tiles) in an array of their own
  // The two stage buffers and the V tiles are arrays of their own and the
  // stage loop is unrolled by two, so every DMA and every read names its
  // buffer at compile time: the compiler holds a read back only for the DMA
  // into that same buffer, not for the next stage's DMA into the other one.
  __shared__ __attribute__((aligned(1024))) uint8_t lst0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lst1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lvk[FUSED ? 4 * C::TILE : 16];
  auto stage_buf = [&](auto U) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(U)::value == 0) return lst0;
    else return lst1;
  };

  // work: a "stream" is (batch, kv head, split) -- the query heads whose Q /
  // dO it reads; one split covers group / n_split query heads.  Blocks go to
  // the 8 XCDs round-robin and stream i always lands on XCD i % 8.  When a
  // stream's Q / dO exceed an XCD's L2 (stream_major), an XCD runs one
  // stream's key tiles on consecutive slots, so that they are resident
  // together and read each Q / dO tile from L2 at about the same time;
  // otherwise it runs the streams' first key tiles first (longest work
  // first under a causal mask).  Key tiles ascend in both orders.
  const int nstream = p.batch * p.kv_heads * p.n_split;
  const int per_xcd = (nstream + 7) / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int kt = p.stream_major ? slot % p.n_ktiles : slot / per_xcd;
  const int stream = (p.stream_major ? slot / p.n_ktiles : slot % per_xcd) * 8 + xcd;
  if (stream >= nstream) return;
  const int sp = stream % p.n_split;
  const int kvh = (stream / p.n_split) % p.kv_heads;
  const int b = stream / (p.n_split * p.kv_heads);
  const SeqBounds sb = seq_bounds(p, b);
  const int k0 = kt * kTileB;
  if (k0 >= sb.Lk) return;
  const int gsplit = p.group / p.n_split;  // query heads of this workgroup
  const int hbase = kvh * p.group + sp * gsplit;

  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  const int kw = k0 + 32 * wid;           // the wave's first key
  const int key = kw + ql;                // this lane's key
  const int off = sb.Lk - sb.Lq;
  const bool upper = p.causal || p.window > 0;
  const float mul = p.score_mul;
  const float dpm = p.dp_mul;

  // K^T (and for dK V^T) B operands of the lane's key: 16-bit k[key][16 ks +
  // 8 hl .. +8]; E8 codes k8[key][64 ks + 32 hl .. +32]
  constexpr int NSB = E8 ? D / 64 : C::NS;
  u32x4 kf[NSB][E8 ? 2 : 1], vf[MODE == MODE_DK ? NSB : 1][E8 ? 2 : 1];
  {
    const int eb = E8 ? 1 : 2;
    const int64_t koff = ((int64_t)b * p.k_bs + (int64_t)sb.k_start * p.k_rs +
                          (int64_t)kvh * p.k_hs) * eb;
    const uint32_t bytes = sat_bytes((int64_t)sb.Lk * p.k_rs * eb);
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(E8 ? p.k8 : p.k);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(E8 ? p.v8 : p.v);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + koff, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + koff, bytes);
    const uint32_t roff = (uint32_t)key * (uint32_t)(p.k_rs * eb);
#pragma unroll
    for (int ks = 0; ks < NSB; ++ks) {
#pragma unroll
      for (int c = 0; c < (E8 ? 2 : 1); ++c) {
        const uint32_t o = E8 ? roff + 64 * ks + 32 * hl + 16 * c : roff + (16 * ks + 8 * hl) * 2;
        kf[ks][c] = bload16(kr, o);
        if constexpr (MODE == MODE_DK) vf[ks][c] = bload16(vr, o);
      }
    }
    if constexpr (FUSED) {
      // V rows k0 .. k0 + 127 into LDS in the tile layout (rows past the
      // sequence arrive as zeros); awaited with the first stage
      uint32_t voffk[C::CPT];
      tile_dma_offsets<D>(voffk, wid, lane, (uint32_t)(p.k_rs * 2));
      const __amdgpu_buffer_rsrc_t vrw = make_rsrc(vbase + koff, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dma_tile16<D>(lvk + i * C::TILE, vrw, (uint32_t)(k0 + 32 * i) * (uint32_t)(p.k_rs * 2),
                      wid, voffk);
    }
  }
  // accumulators: dV^T (MODE_DV), dK^T (MODE_DK), both (fused: acc = dK^T)
  f32x16 acc[C::NOB], accv[FUSED ? C::NOB : 1];
#pragma unroll
  for (int i = 0; i < C::NOB; ++i) acc[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < (FUSED ? C::NOB : 1); ++i) accv[i] = f32x16{};

  // query rows that see any key of the workgroup / of this wave
  const int k1 = min(k0 + kTileB, sb.Lk);
  const int qa = upper ? max(0, k0 - off) : 0;
  const int qb = p.window > 0 ? min(sb.Lq, k1 - 1 - off + p.window) : sb.Lq;
  const int ta = qa / 32, tb = qb > qa ? (qb + 31) / 32 : ta;
  const int nt = tb - ta;
  // stages: (query tile, query head), the tiles from the last one down and
  // the heads inside a tile, so that the workgroups of one stream (whose
  // tile ranges differ at the low end under a causal mask) read the same
  // Q / dO tiles at the same stage index for as long as they run
  const int nst = nt * gsplit;
  const int kw1 = min(kw + 32, sb.Lk);
  const bool wave_keys = kw < sb.Lk;
  const int wqa = upper ? max(0, kw - off) : 0;
  const int wqb = p.window > 0 ? min(sb.Lq, kw1 - 1 - off + p.window) : sb.Lq;

  uint32_t voff[C::CPT];
  tile_dma_offsets<D>(voff, wid, lane, (uint32_t)(p.q_rs * 2));
  uint32_t voff8 = 0;
  const bool has8 = E8 ? tile8_dma_offset<D>(voff8, tid, (uint32_t)p.q_rs) : false;
  const uint32_t roff0 = row_read_off<D>(ql, hl);
  uint32_t troff[C::NOB][2];
  tr_read_offsets<D>(troff, lane);
  const int64_t plane = ws_plane(p);

  // DMA of the next stage into buffer U: the tiles of its (head, query tile)
  // and their lse2 / delta.  The stage's query tile and the row offsets of its
  // head in Q / dO and in the workspace are carried from stage to stage (no
  // division by the head count in the loop).
  const int64_t qhead0 = (int64_t)b * p.q_bs + (int64_t)sb.q_start * p.q_rs + (int64_t)hbase * p.q_hs;
  const int64_t whead0 = ws_index(p, p.cu_q ? 0 : b, p.cu_q ? (int64_t)sb.q_start : 0, hbase);
  int iss_h = 0, iss_t = tb - 1;
  int64_t iss_q = qhead0, iss_w = whead0;
  auto issue = [&](auto U) __attribute__((always_inline)) {
    const int t = iss_t;
    const int64_t qrow0 = iss_q;
    const uint32_t bytes = sat_bytes((int64_t)sb.Lq * p.q_rs * 2);
    const uint32_t base = (uint32_t)(t * 32) * (uint32_t)(p.q_rs * 2);
    const uint8_t* buf = stage_buf(U);
    const __amdgpu_buffer_rsrc_t q16 = make_rsrc(reinterpret_cast<const uint8_t*>(p.q) + qrow0 * 2,
                                                 bytes);
    const __amdgpu_buffer_rsrc_t d16 = make_rsrc(
        reinterpret_cast<const uint8_t*>(p.dout) + qrow0 * 2, bytes);
    if constexpr (!E8) {
      dma_tile16<D>(buf, q16, base, wid, voff);
      dma_tile16<D>(buf + C::TILE, d16, base, wid, voff);
    } else {
      const uint32_t bytes8 = sat_bytes((int64_t)sb.Lq * p.q_rs);
      const uint32_t base8 = (uint32_t)(t * 32) * (uint32_t)p.q_rs;
      const uint8_t* l8 = buf + wid * 1024;
      if (has8) {
        dma16(l8 + OFF_S, base8 + voff8,
              make_rsrc(reinterpret_cast<const uint8_t*>(p.q8) + qrow0, bytes8));
        if constexpr (MODE == MODE_DK)
          dma16(l8 + OFF_DP, base8 + voff8,
                make_rsrc(reinterpret_cast<const uint8_t*>(p.do8) + qrow0, bytes8));
      }
      dma_tile16<D>(buf + OFF_T, MODE == MODE_DV ? d16 : q16, base, wid, voff);
    }
    if (wid < 2 && lane < 8) {
      // wave 0: lse2 of rows 32 t .. +32 (4 per lane), wave 1: delta; rows past
      // the sequence arrive as zeros
      const float* src = p.delta + iss_w + (wid == 1 ? plane : 0);
      dma16(buf + OFF_W + wid * 128, (uint32_t)(t * 32 * 4 + lane * 16),
            make_rsrc(src, sat_bytes((int64_t)sb.Lq * 4)));
    }
    if (++iss_h == gsplit) {
      iss_h = 0;
      --iss_t;
      iss_q = qhead0;
      iss_w = whead0;
    } else {
      iss_q += p.q_hs;
      iss_w += p.d_rows;
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (nst > 0) issue(S0{});
  wait_vm_all();
  lds_barrier();

  // stage s sits in buffer s % 2
  int cur_h = 0, cur_t = tb - 1;  // the stage computed next
  auto stage = [&](int s, auto U) __attribute__((always_inline)) {
    if (s + 1 < nst) issue(std::integral_constant<int, 1 - decltype(U)::value>{});
    const int q0 = cur_t * 32;
    if (++cur_h == gsplit) {
      cur_h = 0;
      --cur_t;
    }
    if (wave_keys && q0 < wqb && q0 + 32 > wqa) {
      const uint8_t* sbuf = stage_buf(U);
      const uint8_t* st_ = sbuf + OFF_S;    // A operand of S (Q rows)
      const uint8_t* dpt = sbuf + OFF_DP;   // A operand of dP (dO rows)
      const float* wsv = reinterpret_cast<const float*>(sbuf + OFF_W);
      f32x16 sc = {}, dp = {};
      if constexpr (FUSED) {
        // B operand of dP: V^T of the wave's keys, the same row reads as Q
        const uint8_t* vk = lvk + wid * C::TILE;
#pragma unroll
        for (int ks = 0; ks < C::NS; ++ks) {
          const uint32_t ro = roff0 ^ (uint32_t)(ks << 5);
          sc = mfma16<ELEM>(*reinterpret_cast<const u32x4*>(st_ + ro), kf[ks][0], sc);
          dp = mfma16<ELEM>(*reinterpret_cast<const u32x4*>(dpt + ro),
                            *reinterpret_cast<const u32x4*>(vk + ro), dp);
        }
      } else if constexpr (!E8) {
#pragma unroll
        for (int ks = 0; ks < C::NS; ++ks) {
          const uint32_t ro = roff0 ^ (uint32_t)(ks << 5);
          sc = mfma16<ELEM>(*reinterpret_cast<const u32x4*>(st_ + ro), kf[ks][0], sc);
          if constexpr (MODE == MODE_DK)
            dp = mfma16<ELEM>(*reinterpret_cast<const u32x4*>(dpt + ro), vf[ks][0], dp);
        }
        sched_lds_ahead<(MODE == MODE_DK ? 2 : 1) * C::NS, 1, 4>();
      } else {
#pragma unroll
        for (int ks = 0; ks < NSB; ++ks) {
          u32x4 a[2];
          tile8_read<D>(st_, ql, hl, ks, a);
          sc = mfma_fp8(a, kf[ks], sc);
          if constexpr (MODE == MODE_DK) {
            tile8_read<D>(dpt, ql, hl, ks, a);
            dp = mfma_fp8(a, vf[ks], dp);
          }
        }
        sched_lds_ahead<(MODE == MODE_DK ? 2 : 1) * NSB, 2, 2>();
      }
      // register r holds query row q0 + qq(r) + 4 hl, qq(r) = 8 (r / 4) + r % 4

      const bool need_mask = key >= sb.Lk || q0 + 32 > sb.Lq ||
                             (upper && kw + 31 > q0 + off) ||
                             (p.window > 0 && kw < q0 + 31 + off - p.window + 1);
      if (need_mask) {
        // visible iff key <= q + off (causal), key >= q + off - W + 1 (window),
        // q < Lq, key < Lk; with q = q0 + 4 hl + qq:
        const int base = q0 + 4 * hl;
        const int lo = upper ? key - off - base : INT32_MIN / 2;       // qq >= lo
        const int hi = min(sb.Lq - 1 - base,
                           p.window > 0 ? key - off + p.window - 1 - base : INT32_MAX / 2);
        const bool kin = key < sb.Lk;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = 8 * (r >> 2) + (r & 3);
          if (!kin || qq < lo || qq > hi) sc[r] = -INFINITY;
        }
      }
      // B operand of the accumulation: P (dV) or dS (dK), 16-bit; fused: dS
      // in bk, P in bp
      u32x4 bk[2], bp[FUSED ? 2 : 1];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        // lse2 / delta of rows j = 2 t2, 2 t2 + 1 (read when needed: fewer live
        // registers)
        f32x4 l2[4], dl[4];
#pragma unroll
        for (int j = 2 * t2; j < 2 * t2 + 2; ++j) {
          l2[j] = *reinterpret_cast<const f32x4*>(wsv + 8 * j + 4 * hl);
          if constexpr (MODE != MODE_DV)
            dl[j] = *reinterpret_cast<const f32x4*>(wsv + 32 + 8 * j + 4 * hl);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * t2 + 2 * i;
          const int j = r >> 2, e = r & 3;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], mul, -l2[j][e]));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r + 1], mul, -l2[j][e + 1]));
          if constexpr (MODE == MODE_DV)
            bk[t2][i] = pack2<ELEM>(p0, p1);
          else
            bk[t2][i] = pack2<ELEM>(p0 * __builtin_fmaf(dp[r], dpm, -dl[j][e]),
                                    p1 * __builtin_fmaf(dp[r + 1], dpm, -dl[j][e + 1]));
          if constexpr (FUSED) bp[t2][i] = pack2<ELEM>(p0, p1);
        }
      }
      // dV^T += dO^T P  or  dK^T += Q^T dS  (A by transposing reads)
      const uint8_t* at = sbuf + OFF_T;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int db = 0; db < C::NOB; ++db) {
          const uint32_t o0 = troff[db][0] + t2 * 16 * C::ROWB, o1 = troff[db][1] + t2 * 16 * C::ROWB;
          acc[db] = mfma16<ELEM>(vt_operand(at + o0, at + o1), bk[t2], acc[db]);
          if constexpr (FUSED)  // dV^T from the dO tile
            accv[db] = mfma16<ELEM>(vt_operand(dpt + o0, dpt + o1), bp[t2], accv[db]);
        }
      }
    }
    wait_vm_all();
    lds_barrier();
  };
  for (int s = 0; s < nst; s += 2) {
    stage(s, S0{});
    if (s + 1 < nst) stage(s + 1, S1{});
  }

  if (key < sb.Lk) {
    if (p.n_split == 1 && !p.e4m3) {
      const int64_t row = (int64_t)b * p.k_bs + (int64_t)(sb.k_start + key) * p.k_rs +
                          (int64_t)kvh * p.k_hs;
      if constexpr (MODE == MODE_DV)
        store_rows<ELEM, D>(p.dv, row, hl, acc, p.dv_mul);
      else
        store_rows<ELEM, D>(p.dk, row, hl, acc, p.dk_mul);
      if constexpr (FUSED) store_rows<ELEM, D>(p.dv, row, hl, accv, p.dv_mul);
    } else {
      // f32 partials of this split: [mode][sp][kp_row][kvh][d], mode 0 dK, 1 dV
      const int64_t kp = (p.cu_k ? 0 : (int64_t)b * p.seqlen_k) + sb.k_start + key;
      auto put = [&](int mode, const f32x16 (&a)[C::NOB]) __attribute__((always_inline)) {
        float* dst = p.part + ((((int64_t)mode * p.n_split + sp) * p.kp_rows + kp) *
                               p.kv_heads + kvh) * D;
#pragma unroll
        for (int db = 0; db < C::NOB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v4 = {a[db][4 * g], a[db][4 * g + 1], a[db][4 * g + 2], a[db][4 * g + 3]};
            *reinterpret_cast<f32x4*>(dst + db * 32 + g * 8 + 4 * hl) = v4;
          }
      };
      put(MODE == MODE_DV ? 1 : 0, acc);
      if constexpr (FUSED) put(1, accv);
    }
  }
}

// Sum the n_split partials of dK and dV, apply their multipliers and store
// them in the input dtype, or as E4M3 codes: one thread per (key row, kv head,
// 8 d).
template <int ELEM, int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p) {
  const int64_t n = (int64_t)p.kp_rows * p.kv_heads * (D / 8);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % (D / 8));
  const int64_t rk = i / (D / 8);           // kp_row * kv_heads + kvh
  const int kvh = (int)(rk % p.kv_heads);
  const int64_t kp = rk / p.kv_heads;
  const int64_t plane = (int64_t)p.kp_rows * p.kv_heads * D;
  float sk[8] = {}, sv[8] = {};
  for (int sp = 0; sp < p.n_split; ++sp) {
    const float* a = p.part + (int64_t)sp * plane + rk * D + c * 8;
    const float* v = p.part + (int64_t)(p.n_split + sp) * plane + rk * D + c * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(a + 4 * h);
      const f32x4 y = *reinterpret_cast<const f32x4*>(v + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sk[4 * h + j] += x[j];
        sv[4 * h + j] += y[j];
      }
    }
  }
  // packed: kp is the token row; dense: kp = b * seqlen_k + key
  const int64_t b = p.cu_k ? 0 : kp / p.seqlen_k;
  const int64_t key = p.cu_k ? kp : kp % p.seqlen_k;
  const int64_t off = b * p.k_bs + key * p.k_rs + (int64_t)kvh * p.k_hs + c * 8;
  const float km = p.dk_mul, vm = p.dv_mul;
  if (p.e4m3) {
    const u32x2 ok = {pack4_fp8(sat448(sk[0] * km), sat448(sk[1] * km), sat448(sk[2] * km),
                                sat448(sk[3] * km)),
                      pack4_fp8(sat448(sk[4] * km), sat448(sk[5] * km), sat448(sk[6] * km),
                                sat448(sk[7] * km))};
    const u32x2 ov = {pack4_fp8(sat448(sv[0] * vm), sat448(sv[1] * vm), sat448(sv[2] * vm),
                                sat448(sv[3] * vm)),
                      pack4_fp8(sat448(sv[4] * vm), sat448(sv[5] * vm), sat448(sv[6] * vm),
                                sat448(sv[7] * vm))};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(p.dk) + off) = ok;
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(p.dv) + off) = ov;
    return;
  }
  u32x4 ok, ov;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ok[j] = pack2<ELEM>(sk[2 * j] * km, sk[2 * j + 1] * km);
    ov[j] = pack2<ELEM>(sv[2 * j] * vm, sv[2 * j + 1] * vm);
  }
  *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.dk) + off) = ok;
  *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.dv) + off) = ov;
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

// E8: E4M3 inputs.  S^T = K Q^T and dP^T = V dO^T run on the FP8 matrix cores
// (Q^T / dO^T codes in registers, K / V code tiles in LDS, in the second half
// of the lv buffers); dQ^T += K^T dS^T keeps the bf16 copy of the K tile.
template <int ELEM, int D, int E8>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
void bwd_dq_kernel(BwdParams p) {
  using C = T16<D>;
  constexpr int T8 = 32 * D;  // bytes of an E4M3 tile
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lk1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv1[C::TILE];

  // work, as in the forward: a group is (query tile, batch, kv head); its G
  // query heads read the same K/V and sit on consecutive slots of one XCD
  // (blocks go to the 8 XCDs round-robin); query tiles in descending order
  // (under a causal mask later tiles see more keys: longest first)
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int gq = slot / p.group, hh = slot - gq * p.group;
  const int grp = gq * 8 + xcd;
  if (grp >= p.n_qtiles * p.batch * p.kv_heads) return;
  const int kvh = grp % p.kv_heads;
  const int b = (grp / p.kv_heads) % p.batch;
  const int tq = p.n_qtiles - 1 - grp / (p.kv_heads * p.batch);
  const int h = kvh * p.group + hh;
  const SeqBounds sb = seq_bounds(p, b);
  const int r0 = tq * kTileB;
  if (r0 >= sb.Lq) return;

  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  const int qrow = r0 + 32 * wid + ql;
  const float mul = p.score_mul;
  const float dpm = p.dp_mul;
  const int off = sb.Lk - sb.Lq;
  const bool upper = p.causal || p.window > 0;

  // Q^T and dO^T B operands of the lane's row (16-bit: [16 ks + 8 hl .. +8];
  // E8 codes: [64 ks + 32 hl .. +32]), and its lse2 / delta
  constexpr int NSB = E8 ? D / 64 : C::NS;
  u32x4 qf[NSB][E8 ? 2 : 1], of[NSB][E8 ? 2 : 1];
  {
    const int eb = E8 ? 1 : 2;
    const int64_t qoff = ((int64_t)b * p.q_bs + (int64_t)sb.q_start * p.q_rs +
                          (int64_t)h * p.q_hs) * eb;
    const uint32_t bytes = sat_bytes((int64_t)sb.Lq * p.q_rs * eb);
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(E8 ? p.q8 : p.q);
    const uint8_t* dbase = reinterpret_cast<const uint8_t*>(E8 ? p.do8 : p.dout);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qbase + qoff, bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dbase + qoff, bytes);
    const uint32_t roff = (uint32_t)qrow * (uint32_t)(p.q_rs * eb);
#pragma unroll
    for (int ks = 0; ks < NSB; ++ks) {
#pragma unroll
      for (int c = 0; c < (E8 ? 2 : 1); ++c) {
        const uint32_t o = E8 ? roff + 64 * ks + 32 * hl + 16 * c : roff + (16 * ks + 8 * hl) * 2;
        qf[ks][c] = bload16(qr, o);
        of[ks][c] = bload16(dr, o);
      }
    }
  }
  // The row terms of the lane's row, written to the workspace for the
  // dK / dV kernel (which runs after this one): delta = dO . O (E4M3: from
  // the codes, times do_scale o_scale) over the row's two lane halves, and
  // LSE log2(e) (+inf for a row that sees no key, so its weights are 0).
  float lse2 = INFINITY, dlt = 0.0f;
  {
    const int eb = E8 ? 1 : 2;
    const int64_t ooff = ((int64_t)b * p.q_bs + (int64_t)sb.q_start * p.q_rs +
                          (int64_t)h * p.q_hs) * eb;
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(reinterpret_cast<const uint8_t*>(p.o) + ooff,
                                                 sat_bytes((int64_t)sb.Lq * p.q_rs * eb));
    const uint32_t roff = (uint32_t)qrow * (uint32_t)(p.q_rs * eb);
    float acc = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NSB; ++ks) {
#pragma unroll
      for (int c = 0; c < (E8 ? 2 : 1); ++c) {
        const uint32_t o = E8 ? roff + 64 * ks + 32 * hl + 16 * c : roff + (16 * ks + 8 * hl) * 2;
        const u32x4 ov = bload16(orr, o), dv = of[ks][c];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (E8) {
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
              const uint32_t x = fp8x2_to_bf16x2(dv[i], hi), y = fp8x2_to_bf16x2(ov[i], hi);
              acc += lo16<E_BF16>(x) * lo16<E_BF16>(y) + hi16<E_BF16>(x) * hi16<E_BF16>(y);
            }
          } else {
            acc += lo16<ELEM>(dv[i]) * lo16<ELEM>(ov[i]) + hi16<ELEM>(dv[i]) * hi16<ELEM>(ov[i]);
          }
        }
      }
    }
    acc = swap_halves_sum(acc);
    if (qrow < sb.Lq) {
      const float lse = p.lse[(int64_t)b * p.l_bs + (int64_t)(sb.q_start + qrow) * p.l_rs +
                              (int64_t)h * p.l_hs];
      lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
      dlt = E8 ? acc * p.delta_mul : acc;
      if (hl == 0) {
        const int64_t wi = ws_index(p, p.cu_q ? 0 : b, p.cu_q ? (int64_t)sb.q_start + qrow : qrow, h);
        p.delta[wi] = lse2;
        p.delta[ws_plane(p) + wi] = dlt;
      }
    }
  }

  // descriptors: 16-bit K and V tiles; E8: the bf16 K copy and the K / V codes
  __amdgpu_buffer_rsrc_t krs, vrs = make_rsrc(nullptr, 0), k8rs = make_rsrc(nullptr, 0),
                         v8rs = make_rsrc(nullptr, 0);
  uint32_t rs;
  {
    const int64_t krow0 = (int64_t)b * p.k_bs + (int64_t)sb.k_start * p.k_rs +
                          (int64_t)kvh * p.k_hs;
    const uint32_t bytes = sat_bytes((int64_t)sb.Lk * p.k_rs * 2);
    krs = make_rsrc(reinterpret_cast<const uint8_t*>(p.k) + krow0 * 2, bytes);
    if constexpr (!E8) vrs = make_rsrc(reinterpret_cast<const uint8_t*>(p.v) + krow0 * 2, bytes);
    rs = (uint32_t)(p.k_rs * 2);
    if constexpr (E8) {
      const uint32_t bytes8 = sat_bytes((int64_t)sb.Lk * p.k_rs);
      k8rs = make_rsrc(reinterpret_cast<const uint8_t*>(p.k8) + krow0, bytes8);
      v8rs = make_rsrc(reinterpret_cast<const uint8_t*>(p.v8) + krow0, bytes8);
    }
  }
  uint32_t voff[C::CPT];
  tile_dma_offsets<D>(voff, wid, lane, rs);
  uint32_t voff8 = 0;
  const bool has8 = E8 ? tile8_dma_offset<D>(voff8, tid, (uint32_t)p.k_rs) : false;
  // one key tile into (kbuf, vbuf): 16-bit K and V; E8: bf16 K, K codes and
  // V codes (the two code tiles in vbuf)
  auto dma_kv = [&](const uint8_t* kbuf, const uint8_t* vbuf, int t) __attribute__((always_inline)) {
    dma_tile16<D>(kbuf, krs, (uint32_t)(t * 32) * rs, wid, voff);
    if constexpr (!E8) {
      dma_tile16<D>(vbuf, vrs, (uint32_t)(t * 32) * rs, wid, voff);
    } else if (has8) {
      const uint32_t base8 = (uint32_t)(t * 32) * (uint32_t)p.k_rs;
      const uint8_t* l8 = vbuf + wid * 1024;
      dma16(l8, base8 + voff8, k8rs);
      dma16(l8 + T8, base8 + voff8, v8rs);
    }
  };
  const uint32_t roff0 = row_read_off<D>(ql, hl);
  uint32_t troff[C::NOB][2];
  tr_read_offsets<D>(troff, lane);

  // key range of the workgroup and of this wave
  const int qa = r0, qb = min(r0 + kTileB, sb.Lq) - 1;
  const int kv_hi = upper ? min(sb.Lk, qb + off + 1) : sb.Lk;
  const int kv_lo = p.window > 0 ? max(0, qa + off - p.window + 1) : 0;
  const int t0 = kv_lo / 32;
  const int t1 = kv_hi > kv_lo ? (kv_hi + 31) / 32 : t0;
  const int wa = r0 + 32 * wid, wb = min(wa + 31, sb.Lq - 1);
  int whi = 0, wlo = 0;
  if (wa <= wb) {
    whi = upper ? min(sb.Lk, wb + off + 1) : sb.Lk;
    wlo = p.window > 0 ? max(0, wa + off - p.window + 1) : 0;
  }

  f32x16 dq[C::NOB];
#pragma unroll
  for (int i = 0; i < C::NOB; ++i) dq[i] = f32x16{};

  if (t0 < t1) dma_kv(lk0, lv0, t0);
  wait_vm_all();
  lds_barrier();

  auto tile = [&](int t, const uint8_t* kb_, const uint8_t* vb_, const uint8_t* knext,
                  const uint8_t* vnext) __attribute__((always_inline)) {
    if (t + 1 < t1) dma_kv(knext, vnext, t + 1);
    const int c0 = t * 32;
    if (wa <= wb && c0 < whi && c0 + 32 > wlo) {
      f32x16 sc = {}, dp = {};
      if constexpr (!E8) {
#pragma unroll
        for (int ks = 0; ks < C::NS; ++ks) {
          const uint32_t ro = roff0 ^ (uint32_t)(ks << 5);
          sc = mfma16<ELEM>(*reinterpret_cast<const u32x4*>(kb_ + ro), qf[ks][0], sc);
          dp = mfma16<ELEM>(*reinterpret_cast<const u32x4*>(vb_ + ro), of[ks][0], dp);
        }
        sched_lds_ahead<2 * C::NS, 1, 4>();
      } else {
#pragma unroll
        for (int ks = 0; ks < NSB; ++ks) {
          u32x4 a[2];
          tile8_read<D>(vb_, ql, hl, ks, a);
          sc = mfma_fp8(a, qf[ks], sc);
          tile8_read<D>(vb_ + T8, ql, hl, ks, a);
          dp = mfma_fp8(a, of[ks], dp);
        }
        sched_lds_ahead<2 * NSB, 2, 2>();
      }
      // register r holds key c0 + kk(r) + 4 hl, kk(r) = 8 (r / 4) + r % 4
      const bool need_mask = (c0 + 32 > sb.Lk) || (upper && c0 + 31 > wa + off) ||
                             (p.window > 0 && c0 < wb + off - p.window + 1);
      if (need_mask) {
        const int base = c0 + 4 * hl;
        const int a = (upper ? min(sb.Lk - 1, qrow + off) : sb.Lk - 1) - base;
        const int lo = p.window > 0 ? qrow + off - p.window + 1 - base : INT32_MIN / 2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + (r & 3);
          if (kk > a || kk < lo) sc[r] = -INFINITY;
        }
      }
      u32x4 dsk[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * t2 + 2 * i;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], mul, -lse2));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r + 1], mul, -lse2));
          dsk[t2][i] = pack2<ELEM>(p0 * __builtin_fmaf(dp[r], dpm, -dlt),
                                   p1 * __builtin_fmaf(dp[r + 1], dpm, -dlt));
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int db = 0; db < C::NOB; ++db) {
          const uint32_t o0 = troff[db][0] + t2 * 16 * C::ROWB, o1 = troff[db][1] + t2 * 16 * C::ROWB;
          dq[db] = mfma16<ELEM>(vt_operand(kb_ + o0, kb_ + o1), dsk[t2], dq[db]);
        }
      }
      // two K^T operands (two transposing reads each) in flight ahead of the
      // dQ products, as in the forward's P V (+0.6 to +0.9% on the backward)
      sched_lds_ahead<2 * C::NOB, 2, 2>();
    }
    wait_vm_all();
    lds_barrier();
  };

  int t = t0;
  for (; t + 1 < t1; t += 2) {
    tile(t, lk0, lv0, lk1, lv1);
    tile(t + 1, lk1, lv1, lk0, lv0);
  }
  if (t < t1) tile(t, lk0, lv0, lk1, lv1);

  // every wave has passed the last tile's barrier: the four K/V buffers are
  // free, one per wave, each at least the size of its dQ tile
  static_assert(C::TILE >= 32 * 2 * D, "a buffer holds a wave's dQ tile");
  {
    uint8_t* stage = wid == 0 ? lk0 : wid == 1 ? lk1 : wid == 2 ? lv0 : lv1;
    const int r0w = r0 + 32 * wid;
    const int64_t first = (int64_t)b * p.q_bs + (int64_t)(sb.q_start + r0w) * p.q_rs +
                          (int64_t)h * p.q_hs;
    const int nrows = min(32, sb.Lq - r0w);
    if (p.e4m3)
      store_rows_staged<E_E4M3, D>(p.dq, first, p.q_rs, nrows, ql, hl, dq, p.dq_mul, stage);
    else
      store_rows_staged<ELEM, D>(p.dq, first, p.q_rs, nrows, ql, hl, dq, p.dq_mul, stage);
  }
}

// ---------------------------------------------------------------------------
// host planning and launch
// ---------------------------------------------------------------------------

bool plan_bwd(BwdParams& p, int head_dim) {
  const int64_t nk = ((int64_t)p.max_seqlen_k + kTileB - 1) / kTileB;
  const int64_t nq = ((int64_t)p.max_seqlen_q + kTileB - 1) / kTileB;
  // Two workgroups per (kv head, key tile), each over half of the group's
  // query heads (the group must have an even size), when one workgroup's loop
  // would be long or the grid small.  Under a causal mask or a window the
  // first key tiles carry the most work: ceil(max_seqlen_q / 32) * group
  // stages for the longest sequence (fewer under a window); past 256 stages,
  // halving that loop brings the longest workgroup down to about the average
  // load of a CU slot.  A grid of fewer than two workgroups per CU (256 CUs)
  // is split for parallelism.  Otherwise the split costs more than it gains:
  // its reduction pass reads and writes f32 partials of dK and dV.
  const int64_t wg1 = ((int64_t)p.kp_rows + kTileB - 1) / kTileB * p.kv_heads;
  int64_t seen = p.max_seqlen_q;
  if (p.window > 0 && (int64_t)p.window + kTileB < seen) seen = (int64_t)p.window + kTileB;
  const bool long_loop = (p.causal || p.window > 0) && (seen + 31) / 32 * p.group > 256;
  p.n_split = (p.group % 2 == 0 && p.part != nullptr && (wg1 < 512 || long_loop)) ? 2 : 1;
  if (nk * ((int64_t)p.batch * p.kv_heads * p.n_split + 8) > INT32_MAX / 2) return false;
  if ((nq * p.batch * p.kv_heads + 8) * p.group > INT32_MAX / 2) return false;
  p.n_ktiles = (int32_t)nk;
  p.n_qtiles = (int32_t)nq;
  // the Q and dO bytes one dK/dV stream reads, against the 4 MiB L2 of an XCD
  const int64_t stream_bytes = (int64_t)p.max_seqlen_q * (p.group / p.n_split) * head_dim * 2 * 2;
  p.stream_major = stream_bytes >= ((int64_t)4 << 20) ? 1 : 0;
  return head_dim > 0;
}

BwdWorkspace bwd_workspace(int64_t rows, int64_t keys, int64_t heads, int64_t kv_heads,
                           int64_t head_dim, bool e4m3) {
  BwdWorkspace w;
  w.part = (2 * rows * heads + 3) / 4 * 4;  // 16-byte aligned parts
  w.wide = w.part + 4 * keys * kv_heads * head_dim;
  // E4M3: bf16 copies of q and dout (rows x heads), and of k (keys x kv heads)
  w.total = w.wide + (e4m3 ? rows * heads * head_dim + keys * kv_heads * head_dim / 2 : 0);
  return w;
}

// dK and dV: one fused launch for 16-bit inputs, dV then dK for E4M3
template <int E, int D, int E8>
void launch_kv(dim3 grid, dim3 blk, hipStream_t stream, const BwdParams& p) {
  if constexpr (E8) {
    hipLaunchKernelGGL((bwd_kv_kernel<E, D, MODE_DV, 1>), grid, blk, 0, stream, p);
    hipLaunchKernelGGL((bwd_kv_kernel<E, D, MODE_DK, 1>), grid, blk, 0, stream, p);
  } else {
    hipLaunchKernelGGL((bwd_kv_kernel<E, D, MODE_DKV, 0>), grid, blk, 0, stream, p);
  }
}

hipError_t launch_bwd(const BwdParams& p, int elem, int head_dim, hipStream_t stream) {
  const int64_t nred = (int64_t)p.kp_rows * p.kv_heads * (head_dim / 8);
  const int64_t streams8 = ((int64_t)p.batch * p.kv_heads * p.n_split + 7) / 8 * 8;
  const int64_t groups8 = ((int64_t)p.n_qtiles * p.batch * p.kv_heads + 7) / 8 * 8;
  const dim3 g1((unsigned)(p.n_ktiles * streams8)),
      g2((unsigned)(groups8 * p.group)), g3((unsigned)((nred + 255) / 256)), blk(kThreads);
  const bool reduce = p.n_split > 1 || p.e4m3;
  if (p.e4m3) {
    // bf16 copies of the codes (V is only an operand of dP, which runs on the
    // codes)
    const struct { const void* src; void* dst; int64_t n; } w[3] = {
        {p.q8, p.wq, p.n_q}, {p.do8, p.wdo, p.n_q}, {p.k8, p.wk, p.n_k}};
    for (const auto& t : w) {
      const hipError_t e = launch_widen_e4m3(t.src, t.dst, t.n, stream);
      if (e != hipSuccess) return e;
    }
  }
#define VLGQA_BWD(E, D, E8)                                                    \
  do {                                                                         \
    /* dQ first: it also writes the row terms the dK / dV kernel reads */      \
    if (g2.x > 0) hipLaunchKernelGGL((bwd_dq_kernel<E, D, E8>), g2, blk, 0, stream, p);     \
    if (g1.x > 0) launch_kv<E, D, E8>(g1, blk, stream, p);                    \
    if (reduce && g3.x > 0)                                                              \
      hipLaunchKernelGGL((bwd_reduce_kernel<E, D>), g3, blk, 0, stream, p);              \
  } while (0)
  if (p.e4m3 && head_dim == 128) VLGQA_BWD(E_BF16, 128, 1);
  else if (p.e4m3 && head_dim == 64) VLGQA_BWD(E_BF16, 64, 1);
  else if (head_dim == 128 && elem == E_BF16) VLGQA_BWD(E_BF16, 128, 0);
  else if (head_dim == 128 && elem == E_F16) VLGQA_BWD(E_F16, 128, 0);
  else if (head_dim == 64 && elem == E_BF16) VLGQA_BWD(E_BF16, 64, 0);
  else if (head_dim == 64 && elem == E_F16) VLGQA_BWD(E_F16, 64, 0);
  else return hipErrorInvalidValue;
#undef VLGQA_BWD
  return hipGetLastError();
}

}  // namespace vlgqa
