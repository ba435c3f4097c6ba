// Fused variable-length attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup = 4 wave64s = BM = 128 query rows of one (sequence, query
// head); each wave owns 32 rows.  The workgroup walks the key tiles of its
// sequence that hold at least one visible key for its rows (diagonal skip
// and window-band jump), staging K and V through LDS (double-buffered, or
// four buffers where they fit, the next tiles' HBM loads in flight while
// the current tile is computed).  Key tiles are 64 keys (32 for the 192-wide
// head and the biased 128-wide head, 128 for the bias-free 64-wide head).
// Per tile and wave:
//   S^T = K Q^T           on MFMA 32x32x16 (bf16/fp16) or 32x32x2 (fp32),
//                         fp32 accumulate; keys on the M axis, queries on N,
//                         so each lane holds one query column;
//   mask / bias / scale   fp32, masks only on boundary tiles;
//   online softmax        fp32 running max and sum per row (the row max is
//                         an in-lane reduction plus one exchange with the
//                         lane 32 away, so all 64 lanes work); the running
//                         max is raised (and O, l rescaled) only when a row's
//                         max grows by more than 2^8;
//   O^T += V^T P^T        on MFMA, P rounded to the input type (RNE); on
//                         tiles after which some row's sum l is still small
//                         (a few keys carry the row) the rounding residue
//                         P - round(P) is rounded and multiplied in too.
// The method is the streaming-softmax forward described on the triton-msl
// part-1 post (section "What works, and where the edges are": Q staged once,
// one loop over K/V tiles doing QK^T, online softmax with running max and
// sum and a rescale, then P.V, output accumulator resident throughout) with
// the masking conventions of the mtlattn 0.3.0 project page (section "Use").
// The exact diagonal skip follows the triton-msl part-2 post (section
// "FlashAttention: faster than PyTorch, competitive with MLX").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_fwd.h"

// Schedule switches for the LDS race check (the shipping build uses the
// defaults): MI_ATTN_MAX_SLOTS=2 gives every 16-bit kernel two K/V slots;
// MI_ATTN_SYNC_COPIES=1 makes each step wait for its tile copies behind a
// barrier before it reads anything; MI_ATTN_DEEP_COPIES=0 runs the
// four-slot kernels' copies one step less ahead, with a barrier every
// second step.
#ifndef MI_ATTN_MAX_SLOTS
#define MI_ATTN_MAX_SLOTS 4
#endif
#ifndef MI_ATTN_SYNC_COPIES
#define MI_ATTN_SYNC_COPIES 0
#endif
// Four-slot kernels: each tile copy starts three steps before its first
// read and every step ends with a barrier (see step()).
#ifndef MI_ATTN_DEEP_COPIES
#define MI_ATTN_DEEP_COPIES 1
#endif

namespace mi_attn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt in 6:4, lgkmcnt in 11:8): wait for vmcnt == 0 / lgkmcnt == 0 only.
constexpr int kWaitVm0 = 0x0F70;
// vmcnt <= n (n < 64), expcnt and lgkmcnt not waited for
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkm0 = 0xC07F;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// A running max is only raised when a tile's max exceeds it by more than
// this many powers of two; until then p = exp2(t - m) stays below 2^8, which
// fp32 sums and 16-bit P (5 exponent bits or more) hold without overflow.
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x, x of the lane 32 away).  v_permlane32_swap exchanges lanes 32-63 of
// its first operand with lanes 0-31 of its second; given two copies of x it
// leaves (low half of x in both halves, high half of x in both halves), whose
// elementwise max is the pairwise max on every lane.  It is written as
// inline assembly (with the two wait states a VALU write needs before the
// swap reads it): the compiler builtin's second result was dropped from the
// max by the optimiser.
__device__ __forceinline__ float max_with_other_half(float x) {
  float lo = x, hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
  return __builtin_fmaxf(lo, hi);
}

// x + (x of the lane 32 away), by the same exchange.
__device__ __forceinline__ float sum_with_other_half(float x) {
  float lo = x, hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
  return lo + hi;
}

// Minimum / maximum of an int over the 64 lanes of a wave.
__device__ __forceinline__ int wave_min_i32(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i32(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Where the logits' additive bias comes from (the kernels' BSRC parameter):
// an fp32 tensor, ALiBi slopes, or a byte mask (nonzero = visible, 0 = -inf).
enum : int { kBiasTensor = 0, kBiasAlibi = 1, kBiasMask = 2 };

// The four bias values of four consecutive keys of a byte-mask row.
__device__ __forceinline__ f32x4_t mask_bias4(uint32_t w) {
  return (f32x4_t){(w & 0xffu) ? 0.0f : kNegInf, (w & 0xff00u) ? 0.0f : kNegInf,
                   (w & 0xff0000u) ? 0.0f : kNegInf, (w & 0xff000000u) ? 0.0f : kNegInf};
}

// ALiBi bias of query position pos (in key coordinates) for key `key`:
// minus the head's slope times their distance.  The distance is an exact
// integer below 2^24, so the value is the product rounded once.
__device__ __forceinline__ float alibi_bias(float neg_slope, int pos, int key) {
  return neg_slope * __builtin_fabsf((float)(pos - key));
}

// Key hull of the bias rows [r0, r0 + rows) of one sequence and head: the
// smallest lo and largest hi over the rows' ranges [lo, hi) of keys whose
// bias is not -inf (empty ranges count for nothing), and the largest hi over
// the rows [w0, w0 + wrows).  Every lane of the wave returns the same values.
struct KeyHull {
  int lo, hi, wave_hi;
};
__device__ __forceinline__ KeyHull bias_key_hull(const int32_t* rg, int r0, int rows, int lq, int w0,
                                                 int wrows, int lane) {
  int lo = 0x7fffffff, hi = 0, whi = 0;
  for (int r = r0 + lane; r < min(lq, r0 + rows); r += 64) {
    const int2 v = *reinterpret_cast<const int2*>(rg + 2 * (int64_t)r);
    if (v.y > v.x) {
      lo = min(lo, v.x);
      hi = max(hi, v.y);
      if (r >= w0 && r < w0 + wrows) whi = max(whi, v.y);
    }
  }
  return KeyHull{__builtin_amdgcn_readfirstlane(wave_min_i32(lo)),
                 __builtin_amdgcn_readfirstlane(wave_max_i32(hi)),
                 __builtin_amdgcn_readfirstlane(wave_max_i32(whi))};
}

// Rows of a sequence's span [cu[s], cu[s+1]) that it uses: the first
// seqused[s] (clamped to the span), or all of them without seqused.
__device__ __forceinline__ int used_rows(int span, const int32_t* seqused, int seq) {
  return seqused != nullptr ? max(0, min(span, seqused[seq])) : span;
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Max of the 16 entries of one accumulator block as a tree (depth 3).
__device__ __forceinline__ float max16(const f32x16_t& v) {
  const float a0 = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
  const float a1 = __builtin_fmaxf(__builtin_fmaxf(v[3], v[4]), v[5]);
  const float a2 = __builtin_fmaxf(__builtin_fmaxf(v[6], v[7]), v[8]);
  const float a3 = __builtin_fmaxf(__builtin_fmaxf(v[9], v[10]), v[11]);
  const float a4 = __builtin_fmaxf(__builtin_fmaxf(v[12], v[13]), v[14]);
  const float b0 = __builtin_fmaxf(__builtin_fmaxf(a0, a1), a2);
  const float b1 = __builtin_fmaxf(__builtin_fmaxf(a3, a4), v[15]);
  return __builtin_fmaxf(b0, b1);
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  static constexpr bool kWide = false;  // 16-bit operands
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // Two fp32 -> two bf16 (round to nearest even), low half = lo.
  __device__ static uint32_t pack(float lo, float hi) {
    bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static float round_trip(float x) {
    return (float)(__bf16)x;
  }
  // The two values of a packed pair, exactly, as fp32 (low half first).
  __device__ static void unpack(uint32_t w, float& lo, float& hi) {
    lo = __builtin_bit_cast(float, w << 16);
    hi = __builtin_bit_cast(float, w & 0xffff0000u);
  }
};

template <>
struct Elem<_Float16> {
  static constexpr bool kWide = false;
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float lo, float hi) {
    f16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t);
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static float round_trip(float x) { return (float)(_Float16)x; }
  __device__ static void unpack(uint32_t w, float& lo, float& hi) {
    const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
    lo = (float)v[0];
    hi = (float)v[1];
  }
};

template <>
struct Elem<float> {
  static constexpr bool kWide = true;  // 32-bit operands, 32x32x2 MFMA
  __device__ static f32x16_t mma(float a, float b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Output stores: four consecutive head-dim values of one row.
template <typename OutT>
__device__ __forceinline__ void store4(OutT* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4_t*>(p) = (f32x4_t){a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  u32x2_t w = {Elem<__bf16>::pack(a, b), Elem<__bf16>::pack(c, d)};
  *reinterpret_cast<u32x2_t*>(p) = w;
}
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* p, float a, float b, float c, float d) {
  u32x2_t w = {Elem<_Float16>::pack(a, b), Elem<_Float16>::pack(c, d)};
  *reinterpret_cast<u32x2_t*>(p) = w;
}

// Compile-time tile geometry.
template <typename T, int DQK, int DV>
struct Geo {
  static constexpr bool kWide = Elem<T>::kWide;
  static constexpr int BN = kWide ? 32 : 64;   // keys per tile
  static constexpr int NMB = BN / 32;          // 32-key blocks of S^T
  static constexpr int PAD = kWide ? 4 : 8;    // LDS row padding (elements)
  static constexpr int KSTR = DQK + PAD;       // K tile row stride in LDS
  // 16-bit: V is stored transposed (d rows, key positions); fp32: row-major.
  static constexpr int VSTR = kWide ? DV + PAD : BN + PAD;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = kWide ? BN * VSTR : DV * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk
  static constexpr int KCPR = DQK / EPC;       // 16-byte chunks per K row
  static constexpr int KPT = BN * KCPR / kThreads;  // K chunks per thread
  static constexpr int VCPR = DV / EPC;
  static constexpr int VPT_WIDE = BN * VCPR / kThreads;  // fp32 V chunks per thread
  static constexpr int VOCT = DV / 8;          // 16-bit: d-octets per V row
  static constexpr int VUNITS = 16 * VOCT;     // 16-bit: (key quad, d octet) units
  static constexpr int KSTEPS = kWide ? DQK / 2 : DQK / 16;  // MFMA k-steps of QK^T
  static constexpr int NDB = DV / 32;          // 32-row blocks of O^T
  static_assert(BN * KCPR % kThreads == 0, "K staging must divide evenly");
  static_assert(kWide ? (BN * VCPR % kThreads == 0) : (VUNITS <= kThreads), "V staging");
};

// ----------------------------------------------------------------------------
// The kernel.
// ----------------------------------------------------------------------------
// BSRC: where the bias comes from when BIAS is set (kBiasTensor, kBiasAlibi:
// computed from per-head slopes, kBiasMask: a byte mask).
template <typename T, int DQK, int DV, bool BIAS, typename OutT, int BSRC = kBiasTensor>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const KernelArgs a) {
  using G = Geo<T, DQK, DV>;
  using E = Elem<T>;
  constexpr int BN = G::BN;
  constexpr int NMB = G::NMB;
  constexpr bool kWide = G::kWide;
  typedef typename std::conditional<kWide, float, uint16_t>::type Raw;

  __shared__ __attribute__((aligned(16))) Raw smem[2 * G::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is made a scalar so that every per-wave condition below
  // (rows, tile range, masking, P split) is a uniform scalar branch.  MFMA
  // writes all 64 lanes whatever EXEC holds, so an MFMA must never sit in a
  // branch the compiler could execute with a partial or empty EXEC mask.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;   // which half of the wave
  const int l32 = lane & 31;  // column (query) index inside a 32-wide block

  // ---- work decode: (q-tile counted from the end, sequence, head)
  const int head = blockIdx.x % a.hq;
  const int seq = blockIdx.x / a.hq;
  const int cq0 = a.cu_q[seq];
  const int ck0 = a.cu_kv[seq];
  // rows used (lq) and written (span_q: rows past lq get out 0, lse -inf)
  const int span_q = a.cu_q[seq + 1] - cq0;
  const int lq = used_rows(span_q, a.seqused_q, seq);
  const int lk = used_rows(a.cu_kv[seq + 1] - ck0, a.seqused_kv, seq);
  const int n_qtiles = (span_q + kBM - 1) / kBM;
  const int qtile = n_qtiles - 1 - (int)blockIdx.y;  // heaviest causal tiles first
  if (qtile < 0) return;

  const int r0 = qtile * kBM;
  const int r1 = min(lq, r0 + kBM);
  const int off = lk - lq;  // end-aligned diagonal offset
  const int g = head / a.group;
  const bool causal = a.causal != 0;
  const int W = a.window;

  // Key range holding at least one visible key for rows [r0, r1).
  int kv_hi = lk;
  if (causal) kv_hi = min(lk, r1 - 1 + off + 1);
  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, r0 + off - W + 1);
  if constexpr (BIAS && BSRC != kBiasAlibi) {
    // keys outside the hull of the rows' bias ranges have a -inf bias
    if (a.bias_ranges != nullptr) {
      const int32_t* rg = a.bias_ranges +
          ((int64_t)(a.bias_heads == 1 ? 0 : head) * a.total_q + cq0) * 2;
      const KeyHull h = bias_key_hull(rg, r0, kBM, lq, r0, kBM, tid & 63);
      kv_lo = max(kv_lo, h.lo);
      kv_hi = min(kv_hi, h.hi);
    }
  }
  const int t_begin = kv_lo / BN;
  int t_end = kv_hi > 0 ? (kv_hi + BN - 1) / BN : 0;
  if (t_end < t_begin || r0 >= lq) t_end = t_begin;  // (no used row here: zeros only)

  if (a.tile_counts != nullptr && tid == 0 && qtile < (int)gridDim.y)
    a.tile_counts[((int64_t)qtile * a.num_seqs + seq) * a.hq + head] = t_end - t_begin;

  // ---- per-wave rows
  const int w0 = r0 + wave * 32;
  const int w1 = min(lq, w0 + 32);
  const bool wave_active = w0 < lq;
  const int my_row = w0 + l32;
  const bool row_ok = my_row < lq;
  int wkv_hi = lk;
  if (causal) wkv_hi = min(lk, w1 - 1 + off + 1);
  int wkv_lo = 0;
  if (W > 0) wkv_lo = max(0, w0 + off - W + 1);


  const T* __restrict__ kbase = reinterpret_cast<const T*>(a.k) + (int64_t)ck0 * a.k_st +
                                (int64_t)g * a.k_sh;
  const T* __restrict__ vbase = reinterpret_cast<const T*>(a.v) + (int64_t)ck0 * a.v_st +
                                (int64_t)g * a.v_sh;

  // ---- Q fragments (MFMA B operand), loaded once.
  typedef typename std::conditional<kWide, float, u32x4_t>::type QFrag;
  QFrag qf[G::KSTEPS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)(cq0 + my_row) * a.q_st +
                  (int64_t)head * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
      if constexpr (kWide) {
        qf[ks] = row_ok ? reinterpret_cast<const float*>(qp)[2 * ks + hf] : 0.0f;
      } else {
        qf[ks] = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + 16 * ks + 8 * hf)
                        : (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
  }

  // ---- staging registers for one K/V tile
  u32x4_t kreg[G::KPT];
  constexpr int VREG = kWide ? G::VPT_WIDE : 4;
  u32x4_t vreg[VREG];
  const bool v_stager = kWide || tid < G::VUNITS;

  auto load_tile = [&](int t) {
    const int kb = t * BN;
#pragma unroll
    for (int i = 0; i < G::KPT; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / G::KCPR;
      const int c = idx % G::KCPR;
      const int key = kb + row;
      kreg[i] = key < lk ? *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)key * a.k_st +
                                                              G::EPC * c)
                         : (u32x4_t){0u, 0u, 0u, 0u};
    }
    if constexpr (kWide) {
#pragma unroll
      for (int i = 0; i < VREG; ++i) {
        const int idx = tid + kThreads * i;
        const int row = idx / G::VCPR;
        const int c = idx % G::VCPR;
        const int key = kb + row;
        vreg[i] = key < lk ? *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)key * a.v_st +
                                                                G::EPC * c)
                           : (u32x4_t){0u, 0u, 0u, 0u};
      }
    } else {
      if (v_stager) {
        const int oc = tid % G::VOCT;
        const int kq = tid / G::VOCT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 4 * kq + r;
          vreg[r] = key < lk ? *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)key * a.v_st +
                                                                  8 * oc)
                             : (u32x4_t){0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    Raw* ks = smem + buf * G::STAGE;
    Raw* vs = ks + G::K_ELEMS;
#pragma unroll
    for (int i = 0; i < G::KPT; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / G::KCPR;
      const int c = idx % G::KCPR;
      *reinterpret_cast<u32x4_t*>(ks + row * G::KSTR + G::EPC * c) = kreg[i];
    }
    if constexpr (kWide) {
#pragma unroll
      for (int i = 0; i < VREG; ++i) {
        const int idx = tid + kThreads * i;
        const int row = idx / G::VCPR;
        const int c = idx % G::VCPR;
        *reinterpret_cast<u32x4_t*>(vs + row * G::VSTR + G::EPC * c) = vreg[i];
      }
    } else {
      if (v_stager) {
        // 4 keys x 8 head-dims in registers -> 8 rows of V^T, 4 keys each.
        const int oc = tid % G::VOCT;
        const int kq = tid / G::VOCT;
        const int quad = kq & 3;
        // Key positions inside each 16-key group follow the order in which
        // the S^T accumulator hands keys to the P operand (see PV below):
        // keys 0-3, 8-11, 4-7, 12-15.
        const int pos = 16 * (kq >> 2) + 4 * (((quad & 1) << 1) | (quad >> 1));
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int w = dd >> 1;
          const int sh = (dd & 1) * 16;
          const uint32_t e0 = (vreg[0][w] >> sh) & 0xffffu;
          const uint32_t e1 = (vreg[1][w] >> sh) & 0xffffu;
          const uint32_t e2 = (vreg[2][w] >> sh) & 0xffffu;
          const uint32_t e3 = (vreg[3][w] >> sh) & 0xffffu;
          u32x2_t pk = {e0 | (e1 << 16), e2 | (e3 << 16)};
          *reinterpret_cast<u32x2_t*>(vs + (8 * oc + dd) * G::VSTR + pos) = pk;
        }
      }
    }
  };

  // ---- accumulators
  f32x16_t o[G::NDB];
#pragma unroll
  for (int i = 0; i < G::NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m_run = kNegInf;  // running max, log2 units (scale folded in)
  float l_run = 0.0f;     // this lane's share of the running sum

  const float c_scale = a.scale_log2;
  const float* brow = nullptr;
  const uint8_t* mrow = nullptr;
  const float neg_slope = BSRC == kBiasAlibi ? -a.alibi[(int64_t)seq * a.alibi_ss + head] : 0.0f;
  if constexpr (BIAS && BSRC == kBiasTensor) {
    brow = a.bias + (int64_t)(cq0 + (row_ok ? my_row : 0)) * a.b_st +
           (int64_t)(a.bias_heads == 1 ? 0 : head) * a.b_sh;
  }
  if constexpr (BIAS && BSRC == kBiasMask) {
    mrow = a.mask + (int64_t)(cq0 + (row_ok ? my_row : 0)) * a.b_st +
           (int64_t)(a.bias_heads == 1 ? 0 : head) * a.b_sh;
  }

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool has_next = t + 1 < t_end;
    if (has_next) load_tile(t + 1);

    const int kb = t * BN;
    const bool wave_tile = wave_active && kb < wkv_hi && kb + BN > wkv_lo;
    if (wave_tile) {
      const Raw* ks = smem + buf * G::STAGE;
      const Raw* vs = ks + G::K_ELEMS;

      // ---- S^T = K Q^T (keys x queries), fp32
      f32x16_t s[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mb][e] = 0.0f;
#pragma unroll
      for (int ks_ = 0; ks_ < G::KSTEPS; ++ks_) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          if constexpr (kWide) {
            const float kf = ks[(32 * mb + l32) * G::KSTR + 2 * ks_ + hf];
            s[mb] = E::mma(kf, qf[ks_], s[mb]);
          } else {
            const u32x4_t kf =
                *reinterpret_cast<const u32x4_t*>(ks + (32 * mb + l32) * G::KSTR + 16 * ks_ + 8 * hf);
            s[mb] = E::mma(kf, qf[ks_], s[mb]);
          }
        }
      }

      // ---- mask (boundary tiles only): sequence end, causal diagonal, window
      const bool need_mask = (kb + BN > lk) || (causal && kb + BN - 1 > w0 + off) ||
                             (W > 0 && kb <= w1 - 1 + off - W);
      if (need_mask) {
        const int lim_hi = causal ? my_row + off : lk - 1;
        const int lim_lo = W > 0 ? my_row + off - W : -1;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb + 32 * mb + 8 * (e >> 2) + 4 * hf + (e & 3);
            const bool ok = key < lk && key <= lim_hi && key > lim_lo;
            s[mb][e] = ok ? s[mb][e] : kNegInf;
          }
      }

      // ---- logits in log2 units; bias added here
      if constexpr (BIAS) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int key0 = kb + 32 * mb + 8 * qd + 4 * hf;
            f32x4_t bv;
            const int blim = min(lk, a.bias_cols);  // bias columns read: below both
            if constexpr (BSRC == kBiasAlibi) {
#pragma unroll
              for (int e = 0; e < 4; ++e) bv[e] = alibi_bias(neg_slope, my_row + off, key0 + e);
            } else if constexpr (BSRC == kBiasMask) {
              uint32_t w = 0xffffffffu;  // past the mask's columns: visible (bias 0)
              if (row_ok && key0 + 3 < blim) {
                w = *reinterpret_cast<const uint32_t*>(mrow + key0);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (row_ok && key0 + e < blim && mrow[key0 + e] == 0) w &= ~(0xffu << (8 * e));
              }
              bv = mask_bias4(w);
            } else if (row_ok && key0 + 3 < blim) {
              bv = *reinterpret_cast<const f32x4_t*>(brow + key0);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) bv[e] = (row_ok && key0 + e < blim) ? brow[key0 + e] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[mb][4 * qd + e] = __builtin_fmaf(s[mb][4 * qd + e], c_scale, bv[e] * kLog2e);
          }
      }

      // ---- row max: in-lane over this lane's keys, then with the lane 32 away
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_tile = BIAS ? mx : mx * c_scale;

      // ---- online rescale.  Each row decides for itself (alpha = 1, an
      // exact no-op, for rows whose max did not grow past the threshold), so
      // a row's result never depends on the other rows of its wave; the
      // wave only skips the work when no row needs it.
      const bool grow = m_tile > m_run + kRescaleThreshold;
      if (__ballot(grow) != 0ull) {
        const float m_new = grow ? m_tile : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < G::NDB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == kNegInf) ? 0.0f : m_run;

      // ---- p = exp2(t - m); fp32 partial row sum from the unrounded p
      float lsum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = BIAS ? s[mb][e] - m_use : __builtin_fmaf(s[mb][e], c_scale, -m_use);
          const float p = fast_exp2(x);
          s[mb][e] = p;
          lsum += p;
        }
      l_run += lsum;

      // ---- O^T += V^T P^T
      if constexpr (kWide) {
        // fp32: one key per MFMA k-step.  S^T entry e of block mb is key
        // 32 mb + 8 (e/4) + 4 hf + e%4 for this lane; V is row-major in LDS.
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = 32 * mb + 8 * (e >> 2) + 4 * hf + (e & 3);
#pragma unroll
            for (int db = 0; db < G::NDB; ++db) {
              const float vf = vs[key * G::VSTR + 32 * db + l32];
              o[db] = E::mma(vf, s[mb][e], o[db]);
            }
          }
      } else {
        static_assert(kWide, "the register-staged kernel runs fp32 inputs only");
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: out = O / l, lse = (m + log2 l) ln 2 (rows of the span
  // past the used ones: 0 and -inf)
  if (w0 >= span_q) return;
  const float l_all = l_run + __shfl_xor(l_run, 32);
  const float l_tot = row_ok ? l_all : 0.0f;
  if (my_row >= span_q) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  OutT* op = reinterpret_cast<OutT*>(a.out) + (int64_t)(cq0 + my_row) * a.o_st +
             (int64_t)head * a.o_sh;
#pragma unroll
  for (int db = 0; db < G::NDB; ++db)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = 32 * db + 8 * qd + 4 * hf;
      store4<OutT>(op + d0, o[db][4 * qd] * inv, o[db][4 * qd + 1] * inv, o[db][4 * qd + 2] * inv,
                   o[db][4 * qd + 3] * inv);
    }
  if (a.lse != nullptr && hf == 0) {
    const float m_use = (m_run == kNegInf) ? 0.0f : m_run;
    a.lse[(int64_t)head * a.total_q + cq0 + my_row] =
        l_tot > 0.0f ? (m_use + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

// ----------------------------------------------------------------------------
// 16-bit kernel with direct HBM -> LDS staging.
//
// K and V tiles are copied by buffer_load ... lds: lane i of each wave-wide
// load writes 16 bytes at LDS base + 16 i, so the tile layout in LDS is
// chosen by which (key, 16-byte chunk) each lane fetches.  Loads past the
// end of the sequence fall outside the buffer's byte range and come back as
// zeros.  Chunks are XOR-swizzled per key so that the MFMA operand reads
// (K as 16-byte rows, V through the transposing 8-byte read) hit 16
// different 16-byte bank groups.
// ----------------------------------------------------------------------------
template <int D>
struct KSwz {
  // 16-byte-chunk swizzle of K rows: D=128 rows are 256 B (all 64 banks), so
  // 16 consecutive keys take 16 distinct chunk slots; 128 B / 384 B rows
  // alternate bank halves with key parity, so pairs of keys share a pattern.
  __device__ static int f(int key) { return D % 128 == 0 ? (key & 15) : ((key >> 1) & 7); }
};
template <int D>
struct VSwz {
  // V rows are read four keys at a time by the transposing read; the four
  // keys must land in four different 4-chunk groups.
  __device__ static int f(int key) { return D % 128 == 0 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2); }
};

// A pointer the compiler cannot prove wave-uniform, made uniform (every lane
// must hold the same value): keeps buffer descriptors in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) dword access, no swizzle, no stride.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// Copy rows [kb, kb + rows) of one tensor's 64-key tile into LDS at dst
// (this wave's 1 KB slice); rows past `rows` read as zeros.
template <int D, int LOADS>
__device__ __forceinline__ void load_tile_part(const char* base, int64_t st_b, int kb, int rows,
                                               lds_char* dst, const uint32_t* off) {
  // rows <= 0 (a tile past the sequence end): an empty window, all zeros
  const uint32_t bytes = rows > 0 ? (uint32_t)((rows - 1) * st_b + D * 2) : 0u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base + kb * st_b, bytes);
#pragma unroll
  for (int i = 0; i < LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * kThreads * 16), 16, off[i], 0, 0, 0);
}

// ----------------------------------------------------------------------------
// Software-pipelined 16-bit kernel.
//
// A wave owns NB blocks of 32 query rows (BM = 4 waves x 32 NB).  Every K
// and V^T fragment read from LDS feeds NB MFMAs, one per query block.  Each
// wave runs its key loop one tile ahead: the MFMAs of tile t+1's scores, the
// PV MFMAs of tile t and tile t's softmax form one interleaved instruction
// stream, with operand reads issued ahead of their MFMAs.  K and V have
// separate double buffers so K(t+2) and V(t+1) stream in while tile t is
// consumed.  Whether a tile's P also needs its low half multiplied in is
// decided per wave after the tile's row sums are known.
// ----------------------------------------------------------------------------

// Compile-time order of one tile's stream: QK^T MFMAs of the next tile
// (after the first kHead), PV MFMAs of this tile, the softmax chunks (one
// chunk = one pair of scores of one query block) and, when MAXOPS, the next
// tile's masking and row max in small pieces: kMaxPieces per (query block,
// key block) once that block's last QK^T MFMA is two MFMAs old, then two
// that combine the blocks and exchange with the other half of the wave.
// Chunk q covers k-step q / (4 NB), query block (q / 4) % NB, P word q % 4,
// so the P operand of (k-step kk, block n) is complete after chunk
// (kk NB + n) 4 + 3.  PV MFMA p uses V fragment p / NB (k-step (p / NB) /
// NDB, d-block (p / NB) % NDB) for block p % NB; QK MFMA i uses K fragment
// i / NB (d-step (i / NB) / NMB, key block (i / NB) % NMB) for block i % NB.
// MFMAs alternate between QK and PV where possible; one chunk (else one max
// op) follows each MFMA.
enum : int { kOpQK = 0, kOpPV = 1, kOpChunk = 2, kOpMax = 3, kOpMaxEnd = 4 };
constexpr int kMaxPieces = 3;  // max-tree pieces per 16-entry accumulator block
constexpr int kMaxEndPieces = 2;

template <int NQK, int NPV, int NB, int NDB, int NKS, int NMB, bool MAXOPS>
struct StreamPlan {
  static constexpr int kHead = NQK < 4 ? NQK : 4;
  static constexpr int kChunks = 4 * NKS * NB;
  static constexpr int kBlockMaxOps = NB * NMB * kMaxPieces;
  static constexpr int kMaxOps = MAXOPS ? kBlockMaxOps + kMaxEndPieces : 0;
  static constexpr int kOps = (NQK - kHead) + NPV + kChunks + kMaxOps;
  struct Table {
    int8_t op[kOps];
    int8_t ix[kOps];
  };
  static constexpr int pv_needs(int p) {
    return (((p / NB) / NDB) * NB + (p % NB)) * 4 + 4;
  }
  // QK MFMA index after which block (n, mb) of the next tile's scores is final
  static constexpr int qk_last(int n, int mb) {
    return ((NQK / NB / NMB - 1) * NMB + mb) * NB + n;
  }
  static constexpr Table build() {
    Table t{};
    int n = 0, qk = kHead, pv = 0, ch = 0, mx = 0, mfmas = 0;
    int qk_pos[NQK > 0 ? NQK : 1] = {};  // MFMA ordinal of each QK MFMA
    for (int i = 0; i < kHead; ++i) qk_pos[i] = i - kHead;
    bool last_pv = false;
    auto max_ready = [&](int m) {
      if (m >= kBlockMaxOps) return true;  // combine ops: after all block ops
      const int b = m / kMaxPieces;
      const int i = qk_last(b / NMB, b % NMB);
      return i < qk && mfmas - qk_pos[i] >= 3;
    };
    while (qk < NQK || pv < NPV || ch < kChunks || mx < kMaxOps) {
      const bool pv_ready = pv < NPV && ch >= pv_needs(pv);
      bool mfma = false;
      if (pv_ready && (qk >= NQK || !last_pv)) {
        t.op[n] = kOpPV; t.ix[n] = (int8_t)pv++; ++n; last_pv = true; mfma = true; ++mfmas;
      } else if (qk < NQK) {
        qk_pos[qk] = mfmas;
        t.op[n] = kOpQK; t.ix[n] = (int8_t)qk++; ++n; last_pv = false; mfma = true; ++mfmas;
      }
      if (ch < kChunks) {
        t.op[n] = kOpChunk; t.ix[n] = (int8_t)ch++; ++n;
      } else if (mx < kMaxOps && (max_ready(mx) || (!mfma && qk >= NQK))) {
        t.op[n] = mx >= kBlockMaxOps ? kOpMaxEnd : kOpMax;
        t.ix[n] = (int8_t)(mx >= kBlockMaxOps ? mx - kBlockMaxOps : mx);
        ++mx; ++n;
      } else if (!mfma && qk >= NQK && pv >= NPV && mx >= kMaxOps) {
        break;
      }
    }
    return t;
  }
  static constexpr Table kTable = build();
  static constexpr int op(int n) { return kTable.op[n]; }
  static constexpr int index(int n) { return kTable.ix[n]; }
};

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Row width (elements) of a head dim's K / V rows in LDS: the 96-wide head
// is laid out like the 128-wide one (16 chunk slots per row, 12 used), so
// that its rows keep the power-of-two swizzles of the 128-wide layout.
constexpr int lds_dim(int d) { return d == 96 ? 128 : d; }

// Per head-dim pair: NB query blocks of 32 rows per wave, NMB key blocks
// of 32 keys per tile, OCC workgroups per CU (the register budget).  The
// 192-wide contraction keeps 32-key tiles: its Q fragments need 48
// registers, and 64-key tiles would push two workgroups per CU into spills.
template <int DQK, int DV, bool BIAS = false>
struct WaveBlocks {
  static constexpr int NB = 1;
  // 32-key tiles where 64 would not fit the registers: the 192-wide head,
  // and the 128-wide head with a bias (whose next tile's bias values are
  // held in registers through a step).  The 64-wide head without a bias
  // has room for 128-key tiles, which halves its per-tile overheads (barrier,
  // max exchange, copy issue) per key.
  static constexpr int NMB = (DQK > 128 || (BIAS && DQK == 128)) ? 1 : (DQK == 64 && !BIAS) ? 4 : 2;
  // Workgroups per CU: two, except for the 256-wide head, whose output
  // block and Q fragments need the registers of a whole SIMD per wave.
  static constexpr int OCC = DV == 256 ? 1 : 2;
  // K/V buffer slots.  Where four of each fit the LDS share of a workgroup
  // (80 KB with two per CU) copies run further ahead (step()).
  static constexpr int NSLOT =
      MI_ATTN_MAX_SLOTS >= 4 &&
              4 * 32 * NMB * (lds_dim(DQK) + lds_dim(DV)) * 2 <= (OCC == 1 ? 152 : 80) * 1024
          ? 4 : 2;
  // keys per tile as reported by mi_attn_tile_shape (tile counts are given
  // in these units): the bias-free tile
  static constexpr int kReportBN = 32 * (DQK > 128 ? 1 : DQK == 64 ? 4 : 2);
};

// ROPE: the query-key contraction's last 64 dims come from separate q_rope /
// k_rope tensors (the latent-attention head without concatenation); the K
// tile then holds a 128-wide "nope" part and a 64-wide "rope" part.
template <typename T, int DQK, int DV, bool BIAS, typename OutT, bool ROPE = false,
          int BSRC = kBiasTensor>
__global__ __launch_bounds__(kThreads, (WaveBlocks<DQK, DV, BIAS>::OCC)) void attn_fwd16p_kernel(
    const KernelArgs a) {
  using E = Elem<T>;
  static_assert(!ROPE || DQK == 192, "split nope / rope operands only for the 192-wide head");
  static_assert(BSRC == kBiasTensor || BIAS, "ALiBi and masks take the biased path");
  constexpr int DN = ROPE ? DQK - 64 : DQK;  // width of the q / k operand (the nope part)
  // A row's running max m lags the true row max by less than
  // 2^kRescaleThreshold: O and l are rescaled between tiles only when a row's
  // max grows by more than that, so most steps skip the O rescale.  The
  // largest p of a row is then some 2^f rather than exactly 1, and its
  // 16-bit rounding lands on the dominant term of P V; where that matters
  // (rows whose sum l is small against their largest p) the tile's P is
  // carried to 16 bits by the low-half pass of step().
  constexpr int NB = WaveBlocks<DQK, DV, BIAS>::NB;
  constexpr int NMB = WaveBlocks<DQK, DV, BIAS>::NMB;
  constexpr int RW = 32 * NB;  // query rows per wave
  constexpr int BM = 4 * RW;   // query rows per workgroup
  constexpr int BN = 32 * NMB; // keys per tile
  constexpr int NKS = BN / 16; // PV k-steps per tile
  constexpr int DQK_L = lds_dim(DQK);  // K row width in LDS
  constexpr int DV_L = lds_dim(DV);    // V row width in LDS
  constexpr int KRB = DQK_L * 2;
  constexpr int VRB = DV_L * 2;
  constexpr int VCPR = DV_L / 8;
  constexpr int K_BYTES = BN * KRB;
  constexpr int V_BYTES = BN * VRB;
  constexpr int KLOADS = K_BYTES / (kThreads * 16);
  constexpr int VLOADS = V_BYTES / (kThreads * 16);
  constexpr int KSTEPS = DQK / 16;
  constexpr int NDB = DV / 32;
  constexpr int OUT_RB = DV * (int)sizeof(OutT);       // bytes of an output row
  constexpr int OUT_CPR = OUT_RB / 16;
  constexpr int OUT_RBL = DV_L * (int)sizeof(OutT);    // its staging row in LDS
  constexpr int OUT_CPRL = OUT_RBL / 16;               // (a power of two)
  static_assert(K_BYTES % (kThreads * 16) == 0 && V_BYTES % (kThreads * 16) == 0, "tile loads");
  // output rows staged per pass (a wave stages in one K or V buffer)
  constexpr int STAGE_BYTES = K_BYTES < V_BYTES ? K_BYTES : V_BYTES;
  constexpr int STAGE_ROWS = 32 * OUT_RBL <= STAGE_BYTES ? 32 : STAGE_BYTES / OUT_RBL;
  static_assert(STAGE_ROWS >= 1 && 32 % STAGE_ROWS == 0, "output staging");

  // K and V buffers (NSLOT of each) as separate LDS objects.  Each access
  // names its buffer at compile time, so the compiler can tell that reads of
  // the current tiles do not overlap the copies in flight into the other
  // buffers and does not wait for those copies before reading.
  constexpr int NSLOT = WaveBlocks<DQK, DV, BIAS>::NSLOT;
  // deep copies: K copies four and V copies three tiles ahead, a barrier
  // after every step (four slots only)
  constexpr bool DEEP = MI_ATTN_DEEP_COPIES && NSLOT == 4;
  constexpr int K_BYTES_HI = NSLOT == 4 ? K_BYTES : 16;  // slots 2 and 3
  constexpr int V_BYTES_HI = NSLOT == 4 ? V_BYTES : 16;
  __shared__ __attribute__((aligned(1024))) char kbuf_0[K_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf_1[K_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf_0[V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf_1[V_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf_2[K_BYTES_HI];
  __shared__ __attribute__((aligned(1024))) char kbuf_3[K_BYTES_HI];
  __shared__ __attribute__((aligned(1024))) char vbuf_2[V_BYTES_HI];
  __shared__ __attribute__((aligned(1024))) char vbuf_3[V_BYTES_HI];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Scalar wave index: every per-wave condition below is a uniform scalar
  // branch.  MFMA writes all 64 lanes whatever EXEC holds, so an MFMA must
  // never sit in a branch the compiler could run with a partial EXEC mask.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;

  // ---- work decode.  blockIdx.y counts query tiles down from the last tile
  // of the longest sequence: tile index gridDim.y - 1 - blockIdx.y from the
  // start of every sequence, so workgroups are dispatched roughly by
  // decreasing row position, i.e. (for causal rows) decreasing work, and
  // the last ones to start are the lightest.  Within one (sequence, tile) slab
  // the query heads are ordered so that the heads dispatched to one XCD
  // (consecutive workgroups go round-robin over 8 XCDs) are neighbours and
  // mostly share their kv head, i.e. hit the same L2.
  //
  // With a bias shared by all query heads (head_major, one-dimensional
  // grid) the order is different: XCD c (workgroups c, c + 8, ...) takes the
  // (sequence, tile) groups c, c + 8, c + 16, ... in turn, all query heads of
  // a group back to back, so that the group's bias rows are fetched from HBM
  // into that XCD's L2 once and read there by every head.  Groups are
  // numbered tile-major (sequence fastest), counting tiles down from the
  // last as above; with a few sequences the groups an XCD holds at one time
  // are tiles of the same sequence and share its K/V.
  //
  // With many heads and no kv sharing between them (kv_rows = R > 0, one-
  // dimensional grid), one row holds more items per XCD than the XCD runs at
  // once, so concurrent items would all read different K/V.  Instead XCD c
  // takes its (sequence, head) slots R rows at a time: slot 0 for rows
  // 0..R-1, slot 1 for rows 0..R-1, ..., then rows R..2R-1, so the R query
  // tiles of one head that run together share their K/V through L2.  Rows
  // still count down from the last tile, R at a time.
  int seq, head, by;
  if (a.kv_rows > 0) {
    const int R = a.kv_rows;
    const int per_xcd = (a.hq * a.num_seqs) >> 3;  // (sequence, head) slots per XCD
    const int k = (int)(blockIdx.x >> 3);
    const int sr = k / (per_xcd * R);
    const int rem = k - sr * (per_xcd * R);
    const int slot = rem / R;
    by = sr * R + (rem - slot * R);
    if (by >= a.n_qtiles) return;  // padding rows of the last group of R
    const int bx = slot * 8 + (int)(blockIdx.x & 7);
    const int hx = bx % a.hq;
    seq = bx / a.hq;
    head = hx;
    if ((a.hq & 7) == 0) head = (hx & 7) * (a.hq >> 3) + (hx >> 3);
  } else if (a.head_major) {
    const int k = (int)(blockIdx.x >> 3);
    const int kg = k / a.hq;
    head = k - kg * a.hq;
    const int gb = kg * 8 + (int)(blockIdx.x & 7);
    by = gb / a.num_seqs;
    seq = gb - by * a.num_seqs;
    if (by >= a.n_qtiles) return;  // padding of the last round of 8 groups
  } else {
    const int hx = blockIdx.x % a.hq;
    seq = blockIdx.x / a.hq;
    by = blockIdx.y;
    head = hx;
    if ((a.hq & 7) == 0) {
      const int per_xcd = a.hq >> 3;
      head = (hx & 7) * per_xcd + (hx >> 3);
    }
  }
  // The sequence bounds and the arguments the set-up needs are fetched in
  // one round trip: the empty asm keeps the compiler from deferring loads
  // past the early exit, one dependent wait at a time.
  int cq0 = a.cu_q[seq], cq1 = a.cu_q[seq + 1];
  int ck0 = a.cu_kv[seq], ck1 = a.cu_kv[seq + 1];
  int uq = a.seqused_q != nullptr ? a.seqused_q[seq] : 0x7fffffff;
  int uk = a.seqused_kv != nullptr ? a.seqused_kv[seq] : 0x7fffffff;
  asm volatile("" : "+s"(cq0), "+s"(cq1), "+s"(ck0), "+s"(ck1), "+s"(uq), "+s"(uk)
               : "s"(a.q_st), "s"(a.q_sh), "s"(a.k_st), "s"(a.k_sh), "s"(a.v_st), "s"(a.v_sh),
                 "s"(a.group), "s"(a.causal), "s"(a.window), "s"(a.n_qtiles));
  // rows of the sequence's spans that it uses (all of them without seqused);
  // the output rows of the span past lq are written as 0 (lse -inf)
  const int span_q = cq1 - cq0;
  const int lq = max(0, min(span_q, uq));
  const int lk = max(0, min(ck1 - ck0, uk));
  const int n_qtiles = (span_q + BM - 1) / BM;
  const int qtile = a.n_qtiles - 1 - by;
  if (qtile >= n_qtiles) return;

  const int r0 = qtile * BM;
  const int r1 = min(lq, r0 + BM);
  const int off = lk - lq;
  const int g = head / a.group;
  const bool causal = a.causal != 0;
  const int W = a.window;

  // Key range holding at least one visible key for rows [r0, r1).
  int kv_hi = lk;
  if (causal) kv_hi = min(lk, r1 - 1 + off + 1);
  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, r0 + off - W + 1);
  // With the bias rows' key ranges given: keys outside the hull of the
  // workgroup's rows have a -inf bias for every row, so their tiles are
  // skipped exactly as masked tiles are; a wave also stops after the last
  // tile its own rows can see.
  int wave_bias_hi = lk;
  if constexpr (BIAS && BSRC != kBiasAlibi) {
    if (a.bias_ranges != nullptr) {
      const int32_t* rg = a.bias_ranges +
          ((int64_t)(a.bias_heads == 1 ? 0 : head) * a.total_q + cq0) * 2;
      const KeyHull h = bias_key_hull(rg, r0, BM, lq, r0 + wave * RW, RW, lane);
      kv_lo = max(kv_lo, h.lo);
      kv_hi = min(kv_hi, h.hi);
      wave_bias_hi = h.wave_hi;
    }
  }
  const int t_begin = kv_lo / BN;
  int t_end = kv_hi > 0 ? (kv_hi + BN - 1) / BN : 0;
  if (t_end < t_begin || r0 >= lq) t_end = t_begin;  // (no used row here: zeros only)

  if (a.tile_counts != nullptr && tid == 0) {
    // in units of the reported tile width (a multiple of BN)
    constexpr int RBN = WaveBlocks<DQK, DV, BIAS>::kReportBN;
    a.tile_counts[((int64_t)qtile * a.num_seqs + seq) * a.hq + head] =
        t_end > t_begin ? (t_end * BN + RBN - 1) / RBN - (t_begin * BN) / RBN : 0;
  }

  const int w0 = r0 + wave * RW;
  const int w1 = min(lq, w0 + RW);
  const bool wave_active = w0 < lq;
  int my_row[NB];
  bool row_ok[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    my_row[n] = w0 + 32 * n + l32;
    row_ok[n] = my_row[n] < lq;
  }
  // Rows whose bias is exactly 0 on their key range [rlo, rhi) and -inf
  // elsewhere (bias_pure, from the key-range pass): when every row of the
  // wave is such a row, the wave reads no bias at all.  It adds a bias of 0
  // instead (the same arithmetic, so the same results) and masks keys
  // outside each row's range on the tiles that cross a range end, as it
  // masks the causal diagonal.
  int rlo[NB], rhi[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    rlo[n] = 0;
    rhi[n] = lk;
  }
  bool pure_w = false;
  int pure_lo_max = 0, pure_hi_min = lk;  // over the wave's rows
  if constexpr (BIAS && BSRC != kBiasAlibi) {
    if (a.bias_pure != nullptr && wave_active) {
      const int64_t rb = (int64_t)(a.bias_heads == 1 ? 0 : head) * a.total_q + cq0;
      bool all = true;
#pragma unroll
      for (int n = 0; n < NB; ++n)
        if (row_ok[n]) {
          const int2 v = *reinterpret_cast<const int2*>(a.bias_ranges + 2 * (rb + my_row[n]));
          rlo[n] = v.x;
          rhi[n] = v.y;
          all = all && a.bias_pure[rb + my_row[n]] != 0;
          pure_lo_max = max(pure_lo_max, v.x);
          pure_hi_min = min(pure_hi_min, v.y);
        }
      pure_w = __ballot(!all) == 0ull;
      pure_lo_max = __builtin_amdgcn_readfirstlane(wave_max_i32(pure_lo_max));
      pure_hi_min = __builtin_amdgcn_readfirstlane(wave_min_i32(pure_hi_min));
    }
  }
  // Tiles from wt_end on hold no key visible to any row of this wave (causal
  // rows that end before the workgroup's last diagonal; no rows at all past
  // the sequence end): the wave skips their work but still does its share of
  // the copies and the barriers.
  const int wt_end = max(t_begin, min(!wave_active ? t_begin
                                      : causal    ? (min(lk, w1 - 1 + off + 1) + BN - 1) / BN
                                                  : t_end,
                                      (wave_bias_hi + BN - 1) / BN));

  const int64_t k_st_b = a.k_st * 2;
  const int64_t v_st_b = a.v_st * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)ck0 * a.k_st + (int64_t)g * a.k_sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v) + ((int64_t)ck0 * a.v_st + (int64_t)g * a.v_sh) * 2;

  // Per-lane byte offsets (within a tile, from its first key) of the chunks
  // this lane copies; the same for every tile.  With ROPE the first KN
  // copies fill the nope part of the tile and the rest the rope part, so
  // that every copy reads from one tensor.
  constexpr int KN = ROPE ? BN * DN * 2 / (kThreads * 16) : KLOADS;
  const int64_t kr_st_b = a.kr_st * 2;
  uint32_t koff[KLOADS];
  uint32_t voff[VLOADS];
#pragma unroll
  for (int i = 0; i < KLOADS; ++i) {
    if (i < KN) {
      constexpr int DL = ROPE ? DN : DQK_L;
      const int pos = i * kThreads + tid;  // 16-byte slot in the LDS tile
      const int key = pos / (DL / 8);
      const int c = (pos % (DL / 8)) ^ KSwz<DL>::f(key);
      // slots past the row's DN / 8 chunks (96-wide head) read past the
      // buffer window: zeros, never read back
      koff[i] = c < DN / 8 ? (uint32_t)(key * k_st_b + c * 16) : 0x80000000u;
    } else {
      const int pos = (i - KN) * kThreads + tid;
      const int key = pos / 8;
      const int c = (pos % 8) ^ KSwz<64>::f(key);
      koff[i] = (uint32_t)(key * kr_st_b + c * 16);
    }
  }
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) {
    const int pos = i * kThreads + tid;
    const int key = pos / VCPR;
    const int c = (pos % VCPR) ^ VSwz<DV_L>::f(key);
    voff[i] = c < DV / 8 ? (uint32_t)(key * v_st_b + c * 16) : 0x80000000u;
  }
  // buffer of compile-time slot S
  auto kbuf = [&](auto S) __attribute__((device)) -> lds_char* {
    constexpr int i = decltype(S)::value;
    static_assert(i < NSLOT, "K slot");
    if constexpr (i == 0) return (lds_char*)kbuf_0;
    else if constexpr (i == 1) return (lds_char*)kbuf_1;
    else if constexpr (i == 2) return (lds_char*)kbuf_2;
    else return (lds_char*)kbuf_3;
  };
  auto vbuf = [&](auto S) __attribute__((device)) -> lds_char* {
    constexpr int i = decltype(S)::value;
    static_assert(i < NSLOT, "V slot");
    if constexpr (i == 0) return (lds_char*)vbuf_0;
    else if constexpr (i == 1) return (lds_char*)vbuf_1;
    else if constexpr (i == 2) return (lds_char*)vbuf_2;
    else return (lds_char*)vbuf_3;
  };
  const char* krbase = nullptr;
  if constexpr (ROPE)
    krbase = reinterpret_cast<const char*>(a.k_rope) + ((int64_t)ck0 * a.kr_st + (int64_t)g * a.kr_sh) * 2;
  // Keys copied: those of the tile range (a tile at or past t_end copies
  // nothing and reads as zeros).
  const int kcopy_end = (int)min((int64_t)lk, (int64_t)t_end * BN);
  auto load_k = [&](int t, auto S) __attribute__((device)) {
    load_tile_part<DN, KN>(kbase, k_st_b, t * BN, min(kcopy_end - t * BN, BN), kbuf(S) + wave * 1024, koff);
    if constexpr (ROPE)
      load_tile_part<64, KLOADS - KN>(krbase, kr_st_b, t * BN, min(kcopy_end - t * BN, BN),
                                      kbuf(S) + KN * kThreads * 16 + wave * 1024, koff + KN);
  };
  // LDS address of K fragment (k-step kk: head dims 16 kk .. 16 kk + 15) of key
  auto kaddr = [&](const lds_char* kt, int key, int kk) __attribute__((device)) -> const lds_char* {
    if constexpr (ROPE) {
      if (kk < DN / 16) {
        const int c = (2 * kk + hf) ^ KSwz<DN>::f(key);
        return kt + key * (DN * 2) + c * 16;
      }
      const int c = (2 * (kk - DN / 16) + hf) ^ KSwz<64>::f(key);
      return kt + BN * DN * 2 + key * 128 + c * 16;
    } else {
      const int c = (2 * kk + hf) ^ KSwz<DQK_L>::f(key);
      return kt + key * KRB + c * 16;
    }
  };
  auto load_v = [&](int t, auto S) __attribute__((device)) {
    load_tile_part<DV, VLOADS>(vbase, v_st_b, t * BN, min(kcopy_end - t * BN, BN), vbuf(S) + wave * 1024, voff);
  };

  // ---- Q fragments (B operand of S^T = K Q^T), loaded once.
  // Rows past the sequence end fall outside the buffer window and read as 0.
  u32x4_t qf[NB][KSTEPS];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int64_t q_st_b = a.q_st * 2;
    const int rows = min(32, lq - (w0 + 32 * n));  // valid rows of this block (may be <= 0)
    const char* qb = uniform_ptr(reinterpret_cast<const char*>(a.q) +
                                 ((int64_t)(cq0 + w0 + 32 * n) * a.q_st + (int64_t)head * a.q_sh) * 2);
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(qb, rows > 0 ? (uint32_t)((rows - 1) * q_st_b + DN * 2) : 0u);
    const int qoff = (int)(l32 * q_st_b) + 16 * hf;
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks)
      qf[n][ks] = __builtin_amdgcn_raw_buffer_load_b128(r, qoff + 32 * ks, 0, 0);
    if constexpr (ROPE) {
      const int64_t qr_st_b = a.qr_st * 2;
      const char* qrb = uniform_ptr(reinterpret_cast<const char*>(a.q_rope) +
                                    ((int64_t)(cq0 + w0 + 32 * n) * a.qr_st + (int64_t)head * a.qr_sh) * 2);
      const __amdgpu_buffer_rsrc_t rr =
          make_rsrc(qrb, rows > 0 ? (uint32_t)((rows - 1) * qr_st_b + 128) : 0u);
      const int qroff = (int)(l32 * qr_st_b) + 16 * hf;
#pragma unroll
      for (int ks = DN / 16; ks < KSTEPS; ++ks)
        qf[n][ks] = __builtin_amdgcn_raw_buffer_load_b128(rr, qroff + 32 * (ks - DN / 16), 0, 0);
    }
  }

  // V^T fragment (A operand of O^T += V^T P^T): two transposing reads of the
  // row-major V tile.  Read h of k-step kk, d-block db gives this lane keys
  // 16 kk + 8 h + 4 hf + k (k = 0..3) at head dim 32 db + lane % 32.
  const int vkey_lane = 4 * hf + ((lane & 15) >> 2);
  const int vchunk_lane = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vbyte_lane = (lane & 1) * 8;
  auto vfrag = [&](const lds_char* vt, int kk, int db) __attribute__((device)) -> u32x4_t {
    u32x4_t r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = 16 * kk + 8 * h + vkey_lane;
      const int c = (4 * db + vchunk_lane) ^ VSwz<DV_L>::f(key);
      const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(vt + key * VRB + c * 16 + vbyte_lane));
      const u32x2_t xw = __builtin_bit_cast(u32x2_t, x);
      r[2 * h] = xw[0];
      r[2 * h + 1] = xw[1];
    }
    return r;
  };

  f32x16_t o[NB][NDB];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[n][i][e] = 0.0f;
  float m_run[NB];
  float l_run[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    m_run[n] = kNegInf;  // running max, log2 units (scale folded in)
    l_run[n] = 0.0f;     // this lane's share of the running sum
  }
  const float c_scale = a.scale_log2;
  // With a bias, logits stay in natural units (scale s + b, one fma) until
  // the exponent's argument multiplies them by log2(e).
  const float c_nat = a.scale_log2 * (1.0f / kLog2e);
  const float* brow[NB];
  const uint8_t* mrow[NB];
  const float neg_slope = BSRC == kBiasAlibi ? -a.alibi[(int64_t)seq * a.alibi_ss + head] : 0.0f;
  if constexpr (BIAS && BSRC == kBiasTensor) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      brow[n] = a.bias + (int64_t)(cq0 + (row_ok[n] ? my_row[n] : 0)) * a.b_st +
                (int64_t)(a.bias_heads == 1 ? 0 : head) * a.b_sh;
  }
  if constexpr (BIAS && BSRC == kBiasMask) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      mrow[n] = a.mask + (int64_t)(cq0 + (row_ok[n] ? my_row[n] : 0)) * a.b_st +
                (int64_t)(a.bias_heads == 1 ? 0 : head) * a.b_sh;
  }

  // S^T = K Q^T for the whole K tile at kt (prologue only).
  auto qk_all = [&](const lds_char* kt, f32x16_t (&s)[NB][NMB]) __attribute__((device)) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[n][mb][e] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const u32x4_t kf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
            kaddr(kt, 32 * mb + l32, kk));
#pragma unroll
        for (int n = 0; n < NB; ++n) s[n][mb] = E::mma(kf, qf[n][kk], s[n][mb]);
      }
  };

  // Mask (boundary tiles only) and bias the raw scores of tile t, then take
  // each row's max; returns true when some row's max exceeds its running max
  // by more than the growth bound (m_pend holds the new maxima).  A row whose
  // running max is still -inf (nothing visible yet: O and l are zero) simply
  // adopts the new max.
  // Tile t holds keys that some row of this wave must not see (sequence
  // end, causal diagonal, window start).
  auto tile_needs_mask = [&](int t) __attribute__((device)) -> bool {
    const int kb = t * BN;
    return (kb + BN > lk) || (causal && kb + BN - 1 > w0 + off) || (W > 0 && kb <= w1 - 1 + off - W) ||
           (pure_w && (kb < pure_lo_max || kb + BN > pure_hi_min));
  };
  // Masks key block mb of query block n of tile t: entry e of the lane holds
  // key kb + 32 mb + 8 (e / 4) + 4 hf + e % 4, visible iff lo < key <= hi
  // (one unsigned compare per entry).
  auto mask_block = [&](int t, f32x16_t& sc, int n, int mb) __attribute__((device)) {
    const int key0 = t * BN + 32 * mb + 4 * hf;
    // (rlo, rhi: the row's bias key range, or all keys)
    const int hi = min(min(lk, rhi[n]) - 1, causal ? my_row[n] + off : lk - 1);
    const int lo = max(W > 0 ? my_row[n] + off - W : -1, rlo[n] - 1);
    const int base = lo + 1 - key0;         // first visible entry offset
    const uint32_t span = (uint32_t)max(hi - lo, 0);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 8 * (e >> 2) + (e & 3);
      sc[e] = (uint32_t)(c - base) < span ? sc[e] : kNegInf;
    }
  };
  // Given the row max of tile t's (masked) scores for each query block, set
  // the pending max; returns true when some row's max exceeds its running
  // max by more than the growth bound (2^kRescaleThreshold).  A row whose running max is still
  // -inf (nothing visible yet: O and l are zero) adopts the new max.
  // mx holds the maxima over both halves of the wave (max_with_other_half).
  auto finish_max = [&](float (&mx)[NB], float (&m_pend)[NB]) __attribute__((device)) -> bool {
    bool grow = false;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const float m_all = mx[n];
      const float m_tile = BIAS ? m_all * kLog2e : m_all * c_scale;
      if (m_run[n] == kNegInf) m_run[n] = m_tile;
      m_pend[n] = m_tile;
      grow = grow || (m_tile > m_run[n] + kRescaleThreshold);
    }
    return __ballot(grow) != 0ull;
  };
  // This lane's bias values of tile t (the entries of its S^T registers);
  // keys past the sequence end read as 0 (they are masked).  They are loaded
  // at the start of the step whose end consumes them (prep_tile of the next
  // tile), so the loads' latency is hidden behind that step's stream.
  const int blim = BIAS ? min(lk, a.bias_cols) : 0;  // bias columns read: below both
  auto load_bias = [&](int t, f32x4_t (&bv)[NB][NMB][4]) __attribute__((device)) {
    const int kb = t * BN;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int key0 = kb + 32 * mb + 8 * qd + 4 * hf;
          if constexpr (BSRC == kBiasAlibi) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              bv[n][mb][qd][e] = alibi_bias(neg_slope, my_row[n] + off, key0 + e);
          } else if constexpr (BSRC == kBiasMask) {
            uint32_t w = 0xffffffffu;  // past the mask's columns: visible (bias 0)
            if (row_ok[n] && key0 + 3 < blim) {
              w = *reinterpret_cast<const uint32_t*>(mrow[n] + key0);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (row_ok[n] && key0 + e < blim && mrow[n][key0 + e] == 0) w &= ~(0xffu << (8 * e));
            }
            bv[n][mb][qd] = mask_bias4(w);
          } else if (row_ok[n] && key0 + 3 < blim) {
            bv[n][mb][qd] = *reinterpret_cast<const f32x4_t*>(brow[n] + key0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              bv[n][mb][qd][e] = (row_ok[n] && key0 + e < blim) ? brow[n][key0 + e] : 0.0f;
          }
        }
  };
  auto prep_tile = [&](int t, f32x16_t (&sc)[NB][NMB], float (&m_pend)[NB],
                       const f32x4_t (&bv)[NB][NMB][4]) __attribute__((device)) -> bool {
    if (tile_needs_mask(t)) {
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) mask_block(t, sc[n][mb], n, mb);
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sc[n][mb][4 * qd + e] =
                  __builtin_fmaf(sc[n][mb][4 * qd + e], c_nat, bv[n][mb][qd][e]);
    }
    float mx[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      mx[n] = max16(sc[n][0]);
#pragma unroll
      for (int mb = 1; mb < NMB; ++mb) mx[n] = __builtin_fmaxf(mx[n], max16(sc[n][mb]));
      mx[n] = max_with_other_half(mx[n]);
    }
    return finish_max(mx, m_pend);
  };

  // Rows whose max grew past the bound: move their running max and rescale
  // O and l (kept outside the interleaved stream so that O needs no VALU
  // work there).  Every other row multiplies by exactly 1, so a row's
  // result never depends on the other rows of its wave.
  auto rescale = [&](const float (&m_pend)[NB]) __attribute__((device)) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const bool g = m_pend[n] > m_run[n] + kRescaleThreshold;
      const float alpha = g ? fast_exp2(m_run[n] - m_pend[n]) : 1.0f;
      if (g) m_run[n] = m_pend[n];
      l_run[n] *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[n][i][e] *= alpha;
    }
  };

  // One loop step for tile t.  Entry: s_cur holds tile t's masked, biased
  // scores and m_run is final for them.  One interleaved stream (StreamPlan):
  // QK^T MFMAs of tile t+1, PV MFMAs of tile t as soon as their slice of P
  // is packed, and tile t's softmax in pairs of scores, with operand reads
  // issued ahead.  Then tile t+1's scores are prepared; the return value says
  // whether a rescale is due before tile t+1.
  auto step = [&](auto slot_tag, int j, f32x16_t (&s_cur)[NB][NMB],
                  f32x16_t (&s_nxt)[NB][NMB], float (&m_pend)[NB],
                  f32x4_t (&bpre)[NB][NMB][4]) __attribute__((device)) -> bool {
    constexpr int NKF = NMB * KSTEPS;     // K fragments per tile
    constexpr int NQK = NKF * NB;         // QK^T MFMAs per tile
    constexpr int NVF = NKS * NDB;        // V^T fragments per tile
    constexpr int NPV = NVF * NB;         // PV MFMAs per tile
    // The next tile's masking, bias and row max run inside the stream, in
    // pieces after each key block's last QK^T MFMA.
    constexpr bool MAXOPS = true;
    using Plan = StreamPlan<NQK, NPV, NB, NDB, NKS, NMB, MAXOPS>;
    const int nt = t_end - t_begin;
    const int t = t_begin + j;
    // slot = j % NSLOT (the caller's loop is unrolled NSLOT times).  K(t+u)
    // lives in K slot (slot + u) % NSLOT and V(t+u) in V slot
    // (slot + u) % NSLOT.  This step reads K(t+1) and V(t) and starts the
    // copies of K(t+LK) and V(t+LV), into the slots of the tiles read
    // NSLOT - LK + 1 steps earlier.  With two slots every step ends with a
    // barrier.  With four (MI_ATTN_DEEP_COPIES=0), copies start one step
    // further ahead and only odd steps end with one.  Either way a barrier
    // separates the last read of a slot from the copy that refills it, and
    // the end of a copy (each wave's vmcnt wait at its step's end) from the
    // first read of its tile.
    //
    // Deep copies (four slots, a barrier after every step): K(t+4) goes to
    // the slot of K(t), last read in step t-1, and V(t+3) to that of V(t-1),
    // also last read in step t-1.  A step's copies are first read three
    // steps later, so each step waits only for the copies of two steps
    // earlier: they overlap two whole steps of work instead of one.  The
    // copies are issued whether or not their tile exists (past the end they
    // read an empty window), so that every step has the same count of
    // memory operations in flight; the bias loads of the next tile are
    // issued before them, so that their own wait leaves the copies in flight.
    constexpr int slot = decltype(slot_tag)::value;
    constexpr int LK = DEEP ? 4 : NSLOT == 4 ? 3 : 2;  // K copies run LK tiles ahead
    constexpr int LV = LK - 1;                         // V copies LV tiles ahead
    using KR = std::integral_constant<int, (slot + 1) % NSLOT>;
    using VR = std::integral_constant<int, slot>;
    using KW = std::integral_constant<int, (slot + LK) % NSLOT>;
    using VW = std::integral_constant<int, (slot + LV) % NSLOT>;
    constexpr bool BAR = DEEP || NSLOT == 2 || (slot & 1) != 0;
    if constexpr (DEEP) {
      if constexpr (BIAS) {
        if (!pure_w && t < wt_end && j + 1 < nt) load_bias(t + 1, bpre);
      }
      load_v(t + LV, VW{});
      load_k(t + LK, KW{});
    } else {
      if (j + LV < nt) load_v(t + LV, VW{});
      if (j + LK < nt) load_k(t + LK, KW{});
    }
    if constexpr (MI_ATTN_SYNC_COPIES) {  // schedule check: copies land before any read
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    }
    if (t >= wt_end) {  // nothing visible to this wave from here on
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if constexpr (BAR) __syncthreads();
      return false;
    }
    if constexpr (BIAS && !DEEP) {
      if (!pure_w && j + 1 < nt) load_bias(t + 1, bpre);
    }

    const lds_char* kt = kbuf(KR{});
    const lds_char* vt = vbuf(VR{});
    // K fragment fi: d-step fi / NMB, key block fi % NMB
    auto kread = [&](int fi) __attribute__((device)) -> u32x4_t {
      const int kk = fi / NMB, mb = fi % NMB;
      return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(kaddr(kt, 32 * mb + l32, kk));
    };
    u32x4_t kf[3];
    u32x4_t vf[3];
    // QK MFMA i: K fragment i / NB, query block i % NB
    auto do_qk = [&](int i) __attribute__((device)) {
      const int fi = i / NB, n = i % NB;
      if (n == 0 && fi + 2 < NKF) kf[(fi + 2) % 3] = kread(fi + 2);
      s_nxt[n][fi % NMB] = E::mma(kf[fi % 3], qf[n][fi / NMB], s_nxt[n][fi % NMB]);
    };
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_nxt[n][mb][e] = 0.0f;
    kf[0] = kread(0);
    if (NKF > 1) kf[1] = kread(1);
    float neg_m[NB];
    float m_cur[NB];  // this tile's row max (-inf: nothing visible to the row here)
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      neg_m[n] = (m_run[n] == kNegInf) ? 0.0f : -m_run[n];
      m_cur[n] = m_pend[n];
    }

    u32x4_t ph[NB][NKS];
    float lsum[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) lsum[n] = 0.0f;
    const bool has_next = j + 1 < nt;
    const bool mask_next = has_next && tile_needs_mask(t + 1);
    float mxp[NB];
    float mpart[NB][NMB][5];  // leaf maxima of the max tree of each block
    bool grow = false;
    auto vread = [&](int vi) __attribute__((device)) -> u32x4_t { return vfrag(vt, vi / NDB, vi % NDB); };
#pragma unroll
    for (int i = 0; i < Plan::kHead; ++i) do_qk(i);
    vf[0] = vread(0);
    if (NVF > 1) vf[1] = vread(1);
    __builtin_amdgcn_sched_barrier(0);
    // The two waves of a SIMD come from different workgroups and drift
    // apart.  A wave inside its stream (MFMAs with VALU between them) takes
    // issue priority over one in the VALU-only parts around it (low-half
    // pass, waits, rescale, the next step's set-up): the matrix pipe idles
    // less (+0.5 to 1.7% across the workloads).
    __builtin_amdgcn_s_setprio(1);
    static_for<0, Plan::kOps>([&](auto qc) __attribute__((device)) {
      constexpr int op = Plan::op(decltype(qc)::value);
      constexpr int ix = Plan::index(decltype(qc)::value);
      if constexpr (op == kOpQK) {
        do_qk(ix);
      } else if constexpr (op == kOpPV) {
        const int vi = ix / NB, n = ix % NB;
        if (n == 0 && vi + 2 < NVF) vf[(vi + 2) % 3] = vread(vi + 2);
        const int kk = vi / NDB, db = vi % NDB;
        o[n][db] = E::mma(vf[vi % 3], ph[n][kk], o[n][db]);
      } else if constexpr (op == kOpMax) {
        // next tile, query block n, key block mb: masking, then the max tree
        // (leaves of three entries, then two levels), in kMaxPieces pieces.
        // On the last tile the scores are stale and the result is unused.
        constexpr int b = ix / kMaxPieces, piece = ix % kMaxPieces;
        constexpr int n = b / NMB, mb = b % NMB;
        f32x16_t& v = s_nxt[n][mb];
        float* mp = mpart[n][mb];
        // (empty asm fences keep each piece at its slot, as in the chunks)
        // With a bias the entries become logits (natural units) first.
        auto add_bias = [&](int e0, int e1) __attribute__((device)) {
          if constexpr (BIAS) {
#pragma unroll
            for (int e = e0; e < e1; ++e)
              v[e] = __builtin_fmaf(v[e], c_nat, bpre[n][mb][e / 4][e % 4]);
          }
        };
        if constexpr (piece == 0) {
          if (mask_next) mask_block(t + 1, v, n, mb);
          add_bias(0, 6);
          mp[0] = max3f(v[0], v[1], v[2]);
          mp[1] = max3f(v[3], v[4], v[5]);
          asm volatile("" : "+v"(mp[0]), "+v"(mp[1]));
        } else if constexpr (piece == 1) {
          add_bias(6, 15);
          mp[2] = max3f(v[6], v[7], v[8]);
          mp[3] = max3f(v[9], v[10], v[11]);
          mp[4] = max3f(v[12], v[13], v[14]);
          asm volatile("" : "+v"(mp[2]), "+v"(mp[3]), "+v"(mp[4]));
        } else {
          add_bias(15, 16);
          const float m = __builtin_fmaxf(max3f(mp[0], mp[1], mp[2]), max3f(mp[3], mp[4], v[15]));
          mxp[n] = mb == 0 ? m : __builtin_fmaxf(mxp[n], m);
          asm volatile("" : "+v"(mxp[n]));
        }
      } else if constexpr (op == kOpMaxEnd) {
        if constexpr (ix == 0) {
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            mxp[n] = max_with_other_half(mxp[n]);
            asm volatile("" : "+v"(mxp[n]));
          }
        } else {
          if (has_next) grow = finish_max(mxp, m_pend);
        }
      } else {
        static_assert(op == kOpChunk, "stream op");
        // chunk ix: k-step kk, query block n, P word w -> S^T block kk / 2,
        // entries 8 (kk % 2) + 2 w, +1 (keys 16 kk + {2w, 2w+1 | +8} + 4 hf)
        const int kk = ix / (4 * NB), n = (ix / 4) % NB, w = ix % 4;
        const int mb = kk >> 1, e0 = 8 * (kk & 1) + 2 * w;
        const float cx = BIAS ? kLog2e : c_scale;
        const float x0 = __builtin_fmaf(s_cur[n][mb][e0], cx, neg_m[n]);
        const float x1 = __builtin_fmaf(s_cur[n][mb][e0 + 1], cx, neg_m[n]);
        const float p0 = fast_exp2(x0);
        const float p1 = fast_exp2(x1);
        lsum[n] += p0;
        lsum[n] += p1;
        uint32_t hw = E::pack(p0, p1);
        // Empty asm with in/out register operands: an optimisation fence
        // that keeps this pair's VALU work at its slot in the stream (pure
        // arithmetic would otherwise be sunk below the MFMAs).
        asm volatile("" : "+v"(hw), "+v"(lsum[n]));
        ph[n][kk][w] = hw;
        // p stays in the score registers for a possible low-half pass
        s_cur[n][mb][e0] = p0;
        s_cur[n][mb][e0 + 1] = p1;
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    // Low halves of P.  The stream multiplied V by P rounded to 16 bits,
    // which errs by up to 2^-9 (bf16) or 2^-12 (fp16) of each p.  Relative
    // to the row's sum l those errors are at most about sqrt(p_max / l) of
    // the rounding unit, p_max being this tile's largest p: they count only
    // while l is small against p_max (a few keys of this tile carry the
    // row).  So when a row has l < split_l * p_max after this tile, this
    // tile's P - round(P) is rounded too and multiplied in: P is then carried
    // to about 16 bits.  Each row decides for itself (the other rows of the
    // wave multiply in zeros, an exact no-op), so that a row's result never
    // depends on the other rows; rows that saw nothing in this tile skip it.
    bool lo_row[NB];
    bool lo_pass = false;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      l_run[n] += lsum[n];
      const float l_row = sum_with_other_half(l_run[n]);
      // this tile's largest p is exp2(m_cur - m_run) (below 2^kRescaleThreshold)
      lo_row[n] = m_cur[n] != kNegInf && l_row < a.split_l * fast_exp2(m_cur[n] - m_run[n]);
      lo_pass = lo_pass || lo_row[n];
    }
    if (__ballot(lo_pass) != 0ull) {
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        u32x4_t pl[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int mb = kk >> 1, e0 = 8 * (kk & 1) + 2 * w;
            const float p0 = s_cur[n][mb][e0], p1 = s_cur[n][mb][e0 + 1];
            float h0, h1;  // the rounded values the stream multiplied
            E::unpack(E::pack(p0, p1), h0, h1);
            pl[n][w] = lo_row[n] ? E::pack(p0 - h0, p1 - h1) : 0u;
          }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4_t v = vfrag(vt, kk, db);
#pragma unroll
          for (int n = 0; n < NB; ++n) o[n][db] = E::mma(v, pl[n], o[n][db]);
        }
      }
    }
    if constexpr (DEEP) {
      // this wave's copies of two steps earlier (read next step) have landed;
      // this step's and the previous step's may still be in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (KLOADS + VLOADS)));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies of V(t+LV), K(t+LK) have landed
    }
    if constexpr (BAR) __syncthreads();
    return grow;
  };

  auto run = [&]() __attribute__((device)) {
    const int nt = t_end - t_begin;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    load_k(t_begin, S0{});
    load_v(t_begin, S0{});
    if (nt > 1) load_k(t_begin + 1, S1{});
    if constexpr (NSLOT == 4) {  // copies run a step further ahead
      using S2 = std::integral_constant<int, 2>;
      if (nt > 1) load_v(t_begin + 1, S1{});
      if (nt > 2) load_k(t_begin + 2, S2{});
      if constexpr (DEEP) {  // and deep copies one more
        using S3 = std::integral_constant<int, 3>;
        if (nt > 2) load_v(t_begin + 2, S2{});
        if (nt > 3) load_k(t_begin + 3, S3{});
      }
    }
    // bias of the first tile: in flight together with the first copies
    f32x4_t bpre[NB][NMB][4];
    if constexpr (BIAS) {
      if (pure_w) {  // a bias of 0 for every tile
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) bpre[n][mb][qd] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
      } else {
        load_bias(t_begin, bpre);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    f32x16_t sa[NB][NMB], sb[NB][NMB];
    float m_pend[NB];
    qk_all(kbuf(S0{}), sa);
    bool need = prep_tile(t_begin, sa, m_pend, bpre);
    __syncthreads();  // every wave is done with K buffer 0 before it is refilled
    if constexpr (NSLOT == 2) {
      for (int j = 0; j < nt; j += 2) {
        need = step(S0{}, j, sa, sb, m_pend, bpre);
        if (need) rescale(m_pend);
        if (j + 1 < nt) {
          need = step(S1{}, j + 1, sb, sa, m_pend, bpre);
          if (need) rescale(m_pend);
        }
      }
    } else {
      using S2 = std::integral_constant<int, 2>;
      using S3 = std::integral_constant<int, 3>;
      for (int j = 0; j < nt; j += 4) {
        need = step(S0{}, j, sa, sb, m_pend, bpre);
        if (need) rescale(m_pend);
        if (j + 1 < nt) {
          need = step(S1{}, j + 1, sb, sa, m_pend, bpre);
          if (need) rescale(m_pend);
        }
        if (j + 2 < nt) {
          need = step(S2{}, j + 2, sa, sb, m_pend, bpre);
          if (need) rescale(m_pend);
        }
        if (j + 3 < nt) {
          need = step(S3{}, j + 3, sb, sa, m_pend, bpre);
          if (need) rescale(m_pend);
        }
      }
      // the epilogue reuses the buffers as staging: every copy (deep copies
      // run past the last tile) has landed and the last step ended with a
      // barrier (without deep copies an even step ends without one)
      if constexpr (DEEP) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
      } else {
        if (nt & 1) __syncthreads();
      }
    }
  };
  if (t_begin < t_end) run();

  // ---- epilogue: O / l staged through LDS (the K/V buffers are free after
  // the loop's last barrier), STAGE_ROWS rows of a 32-row query block at a
  // time, so that every output row is written as contiguous 16-byte stores.
  if (w0 >= span_q) return;
  // each wave stages its rows in one of the four (now free) buffers
  lds_char* ostage = wave == 0 ? (lds_char*)kbuf_0 : wave == 1 ? (lds_char*)kbuf_1
                   : wave == 2 ? (lds_char*)vbuf_0 : (lds_char*)vbuf_1;
  // this lane's rows, recomputed here rather than kept through the loop
  int lane_e = (int)threadIdx.x & 31;
  asm volatile("" : "+v"(lane_e));
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int row_e = w0 + 32 * n + lane_e;
    const float l_all = l_run[n] + __shfl_xor(l_run[n], 32);
    const float l_tot = row_e < lq ? l_all : 0.0f;  // rows of the span past lq: 0
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int pass = 0; pass < 32 / STAGE_ROWS; ++pass) {
      if (n > 0 || pass > 0) __builtin_amdgcn_wave_barrier();
      const int sr = l32 - pass * STAGE_ROWS;  // this lane's row within the pass
      if (sr >= 0 && sr < STAGE_ROWS) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int d0 = 32 * db + 8 * qd + 4 * hf;
            const float v0 = o[n][db][4 * qd] * inv, v1 = o[n][db][4 * qd + 1] * inv;
            const float v2 = o[n][db][4 * qd + 2] * inv, v3 = o[n][db][4 * qd + 3] * inv;
            const int byte = d0 * (int)sizeof(OutT);
            const int c = (byte >> 4) ^ (sr & (OUT_CPRL - 1));
            lds_char* dst = ostage + sr * OUT_RBL + c * 16 + (byte & 15);
            if constexpr (sizeof(OutT) == 4) {
              *(__attribute__((address_space(3))) f32x4_t*)dst = (f32x4_t){v0, v1, v2, v3};
            } else {
              *(__attribute__((address_space(3))) u32x2_t*)dst =
                  (u32x2_t){Elem<OutT>::pack(v0, v1), Elem<OutT>::pack(v2, v3)};
            }
          }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
      constexpr int RPI = 64 / OUT_CPR;  // rows per wave-wide pass
      const int cc = lane % OUT_CPR;
      const bool store_lane = lane < RPI * OUT_CPR;  // (12-chunk rows leave 4 lanes idle)
      const int qb = w0 + 32 * n + pass * STAGE_ROWS;  // first row of this pass
      // The pass's rows through one buffer window: rows past the sequence
      // end fall outside it and their stores are dropped.
      const int o_rows = min(max(span_q - qb, 0), STAGE_ROWS);
      const int64_t o_st_b = a.o_st * (int64_t)sizeof(OutT);
      const char* obase = uniform_ptr(reinterpret_cast<const char*>(a.out) +
                                      ((int64_t)(cq0 + qb) * a.o_st + (int64_t)head * a.o_sh) *
                                          (int64_t)sizeof(OutT));
      const __amdgpu_buffer_rsrc_t orsrc =
          make_rsrc(obase, o_rows > 0 ? (uint32_t)((o_rows - 1) * o_st_b + OUT_RB) : 0u);
#pragma unroll
      for (int it = 0; it < (STAGE_ROWS + RPI - 1) / RPI; ++it) {
        const int q = it * RPI + lane / OUT_CPR;
        const int c = cc ^ (q & (OUT_CPRL - 1));
        if (store_lane && q < STAGE_ROWS) {
          const u32x4_t val =
              *(const __attribute__((address_space(3))) u32x4_t*)(ostage + q * OUT_RBL + c * 16);
          __builtin_amdgcn_raw_buffer_store_b128(val, orsrc, (int)(q * o_st_b) + cc * 16, 0, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
    if (a.lse != nullptr && hf == 0 && row_e < span_q) {
      const float m_use = (m_run[n] == kNegInf) ? 0.0f : m_run[n];
      a.lse[(int64_t)head * a.total_q + cq0 + row_e] =
          l_tot > 0.0f ? (m_use + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <typename T, int DQK, int DV, bool BIAS, typename OutT, bool ROPE, int BSRC = kBiasTensor>
hipError_t launch_one(const KernelArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (Elem<T>::kWide) {
    hipLaunchKernelGGL((attn_fwd_kernel<T, DQK, DV, BIAS, OutT, BSRC>), grid, dim3(kThreads), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((attn_fwd16p_kernel<T, DQK, DV, BIAS, OutT, ROPE, BSRC>), grid,
                       dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

// a.alibi / a.mask set: the bias comes from the slopes / the byte mask (the
// host refuses them together with each other or with a bias tensor)
template <typename T, int DQK, int DV, bool ROPE>
hipError_t launch_rope(const KernelArgs& a, bool bias, bool out_f32, dim3 grid, hipStream_t s) {
  if (a.alibi != nullptr) {
    return out_f32 ? launch_one<T, DQK, DV, true, float, ROPE, kBiasAlibi>(a, grid, s)
                   : launch_one<T, DQK, DV, true, T, ROPE, kBiasAlibi>(a, grid, s);
  }
  if (a.mask != nullptr) {
    return out_f32 ? launch_one<T, DQK, DV, true, float, ROPE, kBiasMask>(a, grid, s)
                   : launch_one<T, DQK, DV, true, T, ROPE, kBiasMask>(a, grid, s);
  }
  if (bias) {
    return out_f32 ? launch_one<T, DQK, DV, true, float, ROPE>(a, grid, s)
                   : launch_one<T, DQK, DV, true, T, ROPE>(a, grid, s);
  }
  return out_f32 ? launch_one<T, DQK, DV, false, float, ROPE>(a, grid, s)
                 : launch_one<T, DQK, DV, false, T, ROPE>(a, grid, s);
}

// rope: q / k hold the nope part and a.q_rope / a.k_rope the last 64 dims
// (16-bit types, the 192-wide head only)
template <typename T, int DQK, int DV>
hipError_t launch_dims(const KernelArgs& a, bool bias, bool out_f32, dim3 grid, hipStream_t s) {
  if constexpr (!Elem<T>::kWide && DQK == 192) {
    if (a.q_rope != nullptr) return launch_rope<T, DQK, DV, true>(a, bias, out_f32, grid, s);
  }
  return launch_rope<T, DQK, DV, false>(a, bias, out_f32, grid, s);
}

}  // namespace
}  // namespace mi_attn
