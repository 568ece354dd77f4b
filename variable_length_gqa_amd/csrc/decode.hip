// Split-KV attention forward for decode-shaped problems on gfx950: a few new
// queries per sequence (seqlen_q * G <= 32) against a long KV cache in a
// capacity buffer (boostr flash.rs, FlashAttentionOps: dense layout, GQA
// without repeat_kv, causal / sliding window, kv_seq_len shorter than the
// dim-2 stride).  The work is bound by reading K and V once from HBM, so:
//   * the rows of one (batch, kv head) are all its query heads times all its
//     queries (row r = (head r / S_q, query r % S_q)), padded to the 32 rows of
//     one MFMA tile: K and V are read once for the whole GQA group;
//   * the keys are split into NP contiguous slices, one wave each (a workgroup
//     is one wave): each wave streams its slice through a private LDS ring of
//     three K/V tile pairs by DMA (32-key tiles, no barriers) and keeps the
//     online-softmax state of the forward kernel (S^T = K Q^T and
//     O^T += V^T P^T on v_mfma_f32_32x32x16, optimistic reference maximum);
//   * each wave writes its partial (unnormalised O, reference maximum m,
//     denominator l) to the caller's workspace, and a merge kernel combines
//     the NP partials of a row: M = max m_p, L = sum l_p 2^(m_p - M),
//     O = sum O_p 2^(m_p - M) / L, LSE = (M + log2 L) ln 2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "decode_params.h"
#include "kernel_common.h"

namespace vlgqa {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// a lane's partial sum of a tile's probabilities may reach this before the
// reference maximum is moved; it also bounds each probability, and 2^15 keeps
// every one finite in f16 (largest finite value 65504)
constexpr float kDecPartialBound = 32768.0f;
constexpr int kMaxDecodeParts = 256;

// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left at their maxima
// (vmcnt is split over bits 3:0 and 15:14)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

template <int D>
struct CfgD {
  static constexpr int NS = D / 16;
  static constexpr int NOB = D / 32;
  static constexpr int ROWB = 2 * D;
  static constexpr int CPR = ROWB / 16;
  static constexpr int TILE = 32 * ROWB;       // one 32-key K (or V) tile
  static constexpr int CPL = TILE / 16 / 64;   // DMA chunks per lane per tensor
  static constexpr int NBUF = 3;               // K/V tile pairs in the ring
};

template <int ELEM, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64))) void decode_kernel(DecParams p) {
  using C = CfgD<D>;
  // ring of three (K, V) tile pairs: two tiles stream in while one is used.
  // Each buffer is an array of its own and the loop is unrolled over the ring,
  // so every DMA and every read names its buffer at compile time and the
  // compiler holds a read back only for the DMA into that same buffer.
  static_assert(C::NBUF == 3, "the ring is unrolled for three slots");
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lk1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lk2[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv2[C::TILE];
  auto kbuf = [&](auto U) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(U)::value == 0) return lk0;
    else if constexpr (decltype(U)::value == 1) return lk1;
    else return lk2;
  };
  auto vbuf = [&](auto U) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(U)::value == 0) return lv0;
    else if constexpr (decltype(U)::value == 1) return lv1;
    else return lv2;
  };

  const int np = p.n_parts;
  const int part = blockIdx.x % np;
  const int bk = blockIdx.x / np;
  const int kvh = bk % p.kv_heads, b = bk / p.kv_heads;
  const int lane = threadIdx.x, hl = lane >> 5, ql = lane & 31;
  const int n = p.kv_len;
  const int off = n - p.seqlen_q;
  const bool upper = p.causal || p.window > 0;
  const float mul = p.score_mul;

  // this lane's row: query head kvh * G + r / S_q, query r % S_q (rows past
  // G * S_q are padding: zero queries, never stored)
  const int rows = p.group * p.seqlen_q;
  const bool live = ql < rows;
  const int hh = live ? ql / p.seqlen_q : 0, qi = live ? ql % p.seqlen_q : 0;
  const int h = kvh * p.group + hh;
  u32x4 qf[C::NS];
  {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q) +
                        ((int64_t)b * p.q_bs + (int64_t)h * p.q_hs + (int64_t)qi * p.q_rs) * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qb, live ? (uint32_t)(p.q_rs * 2) : 0u);
#pragma unroll
    for (int ks = 0; ks < C::NS; ++ks) qf[ks] = bload16(qr, (16 * ks + 8 * hl) * 2);
  }

  // this wave's key tiles [t0, t1): a contiguous slice of the keys any row
  // sees (the last query sits at key n - 1, so the causal bound is n itself)
  const int kv_hi = n;
  const int kv_lo = p.window > 0 ? max(0, off - p.window + 1) : 0;
  const int tiles_lo = kv_lo / 32, tiles_hi = kv_hi > kv_lo ? (kv_hi + 31) / 32 : tiles_lo;
  const int nt = tiles_hi - tiles_lo;
  const int t0 = tiles_lo + (int)((int64_t)nt * part / np);
  const int t1 = tiles_lo + (int)((int64_t)nt * (part + 1) / np);

  const int64_t koff = ((int64_t)b * p.k_bs + (int64_t)kvh * p.k_hs) * 2;
  const uint32_t bytes = sat_bytes((int64_t)n * p.k_rs * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const uint8_t*>(p.k) + koff, bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const uint8_t*>(p.v) + koff, bytes);
  const uint32_t rs = (uint32_t)(p.k_rs * 2);
  uint32_t voff[C::CPL];
#pragma unroll
  for (int c = 0; c < C::CPL; ++c) {
    const int P = c * 64 + lane;
    const int row = P / C::CPR, ch = (P % C::CPR) ^ swz<D>(row);
    voff[c] = (uint32_t)row * rs + ch * 16;
  }
  auto dma = [&](int t, auto U) __attribute__((always_inline)) {
    // the tile's base in the scalar offset: no per-tile vector adds
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(t * 32) * rs);
    uint8_t* kb = kbuf(U);
    uint8_t* vb = vbuf(U);
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
      dma16(kb + c * 1024, voff[c], krs, base);
      dma16(vb + c * 1024, voff[c], vrs, base);
    }
  };
  const uint32_t koff0 = (uint32_t)ql * C::ROWB + (uint32_t)((hl ^ swz<D>(ql)) * 16);
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

  float m = -INFINITY, l = 0.0f;
  f32x16 o[C::NOB];
#pragma unroll
  for (int i = 0; i < C::NOB; ++i) o[i] = f32x16{};

  constexpr int NB = C::NBUF;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  if (t0 < t1) dma(t0, S0{});
  if (t0 + 1 < t1) dma(t0 + 1, S1{});
  // tile t sits in slot U = (t - t0) % 3
  auto step = [&](int t, auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    // refill the slot used by tile t - 1; then tile t is the oldest of the
    // (up to) NB DMA batches in flight
    if (t + NB - 1 < t1) {
      dma(t + NB - 1, std::integral_constant<int, (u + NB - 1) % NB>{});
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * 2 * C::CPL));
    } else {
      wait_vm_all();
    }
    asm volatile("" ::: "memory");
    const uint8_t* kb_ = kbuf(U);
    const uint8_t* vb_ = vbuf(U);
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < C::NS; ++ks)
      s = mfma16<ELEM>(*reinterpret_cast<const u32x4*>(kb_ + (koff0 ^ (uint32_t)(ks << 5))), qf[ks], s);
    const int c0 = t * 32;
    // key of register r: c0 + 8 (r / 4) + 4 hl + r % 4
    // (padding rows have zero queries: their scores are 0, never masked away
    // entirely, so they cannot force the rescaling path)
    const bool need_mask = c0 + 32 > n || (upper && c0 + 31 > off) ||
                           (p.window > 0 && c0 < off + p.seqlen_q - 1 - p.window + 1);
    if (need_mask) {
      const int base = c0 + 4 * hl;
      const int a = (upper ? min(n - 1, qi + off) : n - 1) - base;
      const int lo = p.window > 0 ? qi + off - p.window + 1 - base : INT32_MIN / 2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        if (kk > a || kk < lo) s[r] = -INFINITY;
      }
    }
    u32x4 pk[2];
    float part_sum;
    auto exp_tile = [&](float ref) __attribute__((always_inline)) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * t2 + 2 * i;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], mul, -ref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], mul, -ref));
          s0 = (t2 == 0 && i == 0) ? p0 : s0 + p0;
          s1 = (t2 == 0 && i == 0) ? p1 : s1 + p1;
          pk[t2][i] = pack2<ELEM>(p0, p1);
        }
      part_sum = s0 + s1;
    };
    exp_tile(m);
    if (wave_any(!(part_sum <= kDecPartialBound))) {
      float a = s[0], bb = s[1];
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        a = __builtin_elementwise_maximum(a, s[r]);
        bb = __builtin_elementwise_maximum(bb, s[r + 1]);
      }
      const float mx = swap_halves_max(__builtin_elementwise_maximum(a, bb)) * mul;
      const bool up = mx > m;
      const float alpha = up ? __builtin_amdgcn_exp2f(m - mx) : 1.0f;
      m = up ? mx : m;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < C::NOB; ++i) o[i] *= alpha;
      exp_tile(m == -INFINITY ? 0.0f : m);
    }
    l += part_sum;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int db = 0; db < C::NOB; ++db)
        o[db] = mfma16<ELEM>(vt_operand(vb_ + voffs[db][0] + t2 * 16 * C::ROWB,
                                        vb_ + voffs[db][1] + t2 * 16 * C::ROWB),
                             pk[t2], o[db]);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads of slot u done before its refill
  };
  int t = t0;
  for (; t + 2 < t1; t += NB) {
    step(t, S0{});
    step(t + 1, S1{});
    step(t + 2, S2{});
  }
  if (t < t1) step(t, S0{});
  if (t + 1 < t1) step(t + 1, S1{});

  // partial of this wave: unnormalised O (f32), reference max m (log2), l
  l = swap_halves_sum(l);
  if (live) {
    const int64_t pr = ((int64_t)bk * np + part) * 32 + ql;
    float* dst = p.ws + pr * D;
#pragma unroll
    for (int db = 0; db < C::NOB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v4 = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(dst + db * 32 + g * 8 + 4 * hl) = v4;
      }
    if (hl == 0) {
      float* st = p.ws + (int64_t)p.n_bk * np * 32 * D + pr * 2;
      st[0] = m;
      st[1] = l;
    }
  }
}

// one wave per (batch, kv head, row): combine the row's NP partials.  Lane q
// (and q + 64, ...) holds partial q's (m, l); the weights 2^(m_q - M) are
// broadcast from their lanes while every lane sums D / 64 output columns, with
// the partial loads of eight slices in flight at once.
template <int ELEM, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecParams p) {
  constexpr int PER = D / 64;
  constexpr int CH = kMaxDecodeParts / 64;
  const int rows = p.group * p.seqlen_q;
  const int r = blockIdx.x % rows;
  const int bk = blockIdx.x / rows;
  const int lane = threadIdx.x;
  const int np = p.n_parts;
  const float* stats = p.ws + (int64_t)p.n_bk * np * 32 * D;
  const int64_t pr0 = (int64_t)bk * np * 32 + r;  // partial q of the row: pr0 + 32 q

  float mq[CH], lq[CH];
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    // (clamped index: every lane loads, lanes past np then drop the value)
    const int q = 64 * c + lane;
    const f32x2 st = *reinterpret_cast<const f32x2*>(stats + (pr0 + 32 * min(q, np - 1)) * 2);
    mq[c] = q < np ? st[0] : -INFINITY;
    lq[c] = q < np ? st[1] : 0.0f;
    M = fmaxf(M, mq[c]);
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
  float L = 0.0f;
  float w[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    w[c] = mq[c] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mq[c] - M);
    L += lq[c] * w[c];
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) L += __shfl_xor(L, s);

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  const float* part = p.ws + pr0 * D + lane * PER;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int nq = min(64, np - 64 * c);
    // eight slices per batch: their loads are issued before any is used
    for (int j0 = 0; j0 < nq; j0 += 8) {
      float v[8][PER];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float* src = part + (int64_t)(64 * c + min(j0 + i, nq - 1)) * 32 * D;
        if constexpr (PER == 2) {
          const f32x2 t = *reinterpret_cast<const f32x2*>(src);
          v[i][0] = t[0];
          v[i][1] = t[1];
        } else {
          v[i][0] = src[0];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = min(j0 + i, nq - 1);
        const float wq = j0 + i < nq
                             ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[c]), j))
                             : 0.0f;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += v[i][e] * wq;
      }
    }
  }

  const int kvh = bk % p.kv_heads, b = bk / p.kv_heads;
  const int h = kvh * p.group + r / p.seqlen_q, qi = r % p.seqlen_q;
  const float inv = L > 0.0f ? p.out_mul / L : 0.0f;
  const int64_t orow = (int64_t)b * p.q_bs + (int64_t)h * p.q_hs + (int64_t)qi * p.q_rs;
  uint16_t* dst = reinterpret_cast<uint16_t*>(p.o) + orow + lane * PER;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack2<ELEM>(acc[0] * inv, acc[1] * inv);
  } else {
    *dst = (uint16_t)(pack2<ELEM>(acc[0] * inv, 0.0f) & 0xFFFFu);
  }
  if (lane == 0)
    p.lse[(int64_t)b * p.l_bs + (int64_t)h * p.l_hs + (int64_t)qi * p.l_rs] =
        L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

int64_t decode_parts(int64_t batch, int64_t kv_heads, int64_t head_dim, int64_t kv_len) {
  // About 2.5 one-wave workgroups per CU at D = 128 (their 48 KB LDS rings
  // allow 3 per CU; 2.5 measured best on the 8192-key cache), twice that at
  // D = 64; at least 4 key tiles per slice.
  const int64_t target = head_dim == 64 ? 1280 : 640;
  const int64_t bk = batch * kv_heads > 0 ? batch * kv_heads : 1;
  int64_t np = target / bk;
  const int64_t max_np = (kv_len / 32 + 3) / 4;
  if (np > max_np) np = max_np;
  if (np < 1) np = 1;
  if (np > kMaxDecodeParts) np = kMaxDecodeParts;
  return np;
}

int64_t decode_workspace_floats(int64_t batch, int64_t kv_heads, int64_t head_dim,
                                int64_t kv_len) {
  const int64_t np = decode_parts(batch, kv_heads, head_dim, kv_len);
  return batch * kv_heads * np * 32 * (head_dim + 2);
}

// ---------------------------------------------------------------------------
// library-owned scratch for callers that cannot allocate
// ---------------------------------------------------------------------------
//
// The allocation-free decode entry point keeps the slices' partials here
// instead of in a caller workspace: a file-scope device array, one copy per
// GPU, alive until the process ends.  Its host-side name is not a device
// address; the device address is looked up once per device (with that device
// current) and kept.  Every call on a GPU shares that GPU's copy, so calls
// that overlap on one GPU race.  Nothing in it needs clearing: the merge reads
// only partials the same call's slices wrote.
static __device__ __align__(256) float scratch[kDecodeScratchFloats];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t decode_scratch(float** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(a);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecParams& p, int elem, int head_dim, hipStream_t stream) {
  const dim3 g1((unsigned)(p.n_bk * p.n_parts)), b1(64);
  const dim3 g2((unsigned)(p.n_bk * p.group * p.seqlen_q)), b2(64);
#define VLGQA_DEC(E, D)                                                          \
  do {                                                                           \
    hipLaunchKernelGGL((decode_kernel<E, D>), g1, b1, 0, stream, p);             \
    hipLaunchKernelGGL((decode_merge_kernel<E, D>), g2, b2, 0, stream, p);       \
  } while (0)
  if (head_dim == 128 && elem == E_BF16) VLGQA_DEC(E_BF16, 128);
  else if (head_dim == 128 && elem == E_F16) VLGQA_DEC(E_F16, 128);
  else if (head_dim == 64 && elem == E_BF16) VLGQA_DEC(E_BF16, 64);
  else if (head_dim == 64 && elem == E_F16) VLGQA_DEC(E_F16, 64);
  else return hipErrorInvalidValue;
#undef VLGQA_DEC
  return hipGetLastError();
}

}  // namespace vlgqa
