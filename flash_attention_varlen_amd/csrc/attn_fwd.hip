// Fused variable-length attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup = 4 wave64s = BM = 128 query rows of one (sequence, query
// head); each wave owns 32 rows.  The workgroup walks the key tiles of its
// sequence that hold at least one visible key for its rows (diagonal skip
// and window-band jump), staging K and V through LDS (double-buffered, the
// next tile's HBM loads in flight while the current tile is computed).
// Per tile and wave:
//   S^T = K Q^T           on MFMA 32x32x16 (bf16/fp16) or 32x32x2 (fp32),
//                         fp32 accumulate; keys on the M axis, queries on N,
//                         so each lane holds one query column;
//   mask / bias / scale   fp32, masks only on boundary tiles;
//   online softmax        fp32 running max and sum per row (the row max is
//                         an in-lane reduction plus one exchange with the
//                         lane 32 away, so all 64 lanes work);
//   O^T += V^T P^T        on MFMA, P rounded to the input type (RNE), with
//                         a hi/lo split of P on tiles of rows that see few
//                         keys.
// The method is the streaming-softmax forward described on the triton-msl
// part-1 post (section "What works, and where the edges are": Q staged once,
// one loop over K/V tiles doing QK^T, online softmax with running max and
// sum and a rescale, then P.V, output accumulator resident throughout) with
// the masking conventions of the mtlattn 0.3.0 project page (section "Use").
// The exact diagonal skip follows the triton-msl part-2 post (section
// "FlashAttention: faster than PyTorch, competitive with MLX").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_fwd.h"

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
constexpr int kWaitLgkm0 = 0xC07F;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// A running max is only raised when a tile's max exceeds it by more than
// this many powers of two; until then p = exp2(t - m) stays below 2^8, which
// fp32 sums and 16-bit P (8 exponent bits or more) hold without loss.
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
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
template <typename T, int DQK, int DV, bool BIAS, typename OutT>
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
  const int lq = a.cu_q[seq + 1] - cq0;
  const int ck0 = a.cu_kv[seq];
  const int lk = a.cu_kv[seq + 1] - ck0;
  const int n_qtiles = (lq + kBM - 1) / kBM;
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
  const int t_begin = kv_lo / BN;
  int t_end = kv_hi > 0 ? (kv_hi + BN - 1) / BN : 0;
  if (t_end < t_begin) t_end = t_begin;

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

  // Few visible keys for the wave's first row -> hi/lo split of P.
  bool split = false;
  if constexpr (!kWide) {
    int nvis = (causal ? min(lk, w0 + off + 1) : lk) - wkv_lo;
    split = (nvis < a.split_keys) || (BIAS && a.split_bias != 0);
  }

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
  if constexpr (BIAS) {
    brow = a.bias + (int64_t)(cq0 + (row_ok ? my_row : 0)) * a.b_st +
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
            if (row_ok && key0 + 3 < lk) {
              bv = *reinterpret_cast<const f32x4_t*>(brow + key0);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) bv[e] = (row_ok && key0 + e < lk) ? brow[key0 + e] : 0.0f;
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
        // 16-bit: k-step kk covers keys 16kk..16kk+15.  The B operand of a
        // lane is 8 consecutive S^T entries of its own column, i.e. keys
        // 16kk + {0,1,2,3,8,9,10,11} + 4 hf; V^T rows in LDS store the keys
        // of every 16-key group in exactly that order, so the A operand is
        // one 16-byte read.
        constexpr int PK = BN / 16;
        u32x4_t ph[PK];
        u32x4_t pl[PK];
#pragma unroll
        for (int kk = 0; kk < PK; ++kk) {
          const int mb = kk >> 1;
          const int b8 = 8 * (kk & 1);
#pragma unroll
          for (int w = 0; w < 4; ++w)
            ph[kk][w] = E::pack(s[mb][b8 + 2 * w], s[mb][b8 + 2 * w + 1]);
        }
        if (split) {
#pragma unroll
          for (int kk = 0; kk < PK; ++kk) {
            const int mb = kk >> 1;
            const int b8 = 8 * (kk & 1);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float x0 = s[mb][b8 + 2 * w], x1 = s[mb][b8 + 2 * w + 1];
              pl[kk][w] = E::pack(x0 - E::round_trip(x0), x1 - E::round_trip(x1));
            }
          }
        }
        if (split) {
#pragma unroll
          for (int kk = 0; kk < PK; ++kk) {
#pragma unroll
            for (int db = 0; db < G::NDB; ++db) {
              const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(
                  vs + (32 * db + l32) * G::VSTR + 16 * kk + 8 * hf);
              o[db] = E::mma(vf, ph[kk], o[db]);
              o[db] = E::mma(vf, pl[kk], o[db]);
            }
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < PK; ++kk) {
#pragma unroll
            for (int db = 0; db < G::NDB; ++db) {
              const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(
                  vs + (32 * db + l32) * G::VSTR + 16 * kk + 8 * hf);
              o[db] = E::mma(vf, ph[kk], o[db]);
            }
          }
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: out = O / l, lse = (m + log2 l) ln 2
  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
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
  __device__ static int f(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
};
template <int D>
struct VSwz {
  // V rows are read four keys at a time by the transposing read; the four
  // keys must land in four different 4-chunk groups.
  __device__ static int f(int key) { return D == 128 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2); }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) dword access, no swizzle, no stride.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// Copy one 64-key tile of K and V (rows [kb, kb + rows) of this sequence
// and kv head) into LDS at kdst (this wave's 1 KB slice of the K tile; the
// V tile follows K_BYTES later).  Device-only: the buffer-resource builtins
// have no host form.
template <int DQK, int DV, int KLOADS, int VLOADS>
__device__ __forceinline__ void load_kv_tile(const char* kbase, const char* vbase, int64_t k_st_b,
                                             int64_t v_st_b, int kb, int rows, lds_char* kdst,
                                             int k_bytes, const uint32_t* koff,
                                             const uint32_t* voff) {
  const __amdgpu_buffer_rsrc_t kr =
      make_rsrc(kbase + kb * k_st_b, (uint32_t)((rows - 1) * k_st_b + DQK * 2));
  const __amdgpu_buffer_rsrc_t vr =
      make_rsrc(vbase + kb * v_st_b, (uint32_t)((rows - 1) * v_st_b + DV * 2));
  lds_char* vdst = kdst + k_bytes;
#pragma unroll
  for (int i = 0; i < KLOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kdst + i * kThreads * 16), 16, koff[i],
                                             0, 0, 0);
#pragma unroll
  for (int i = 0; i < VLOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vdst + i * kThreads * 16), 16, voff[i],
                                             0, 0, 0);
}

template <typename T, int DQK, int DV, bool BIAS, typename OutT>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd16_kernel(const KernelArgs a) {
  using E = Elem<T>;
  constexpr int BN = 64;            // keys per tile
  constexpr int KRB = DQK * 2;      // K row bytes in LDS
  constexpr int VRB = DV * 2;       // V row bytes in LDS (row-major, keys x d)
  constexpr int KCPR = DQK / 8;     // 16-byte chunks per K row
  constexpr int VCPR = DV / 8;
  constexpr int K_BYTES = BN * KRB;
  constexpr int V_BYTES = BN * VRB;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int KLOADS = K_BYTES / (kThreads * 16);  // direct loads per thread per tile
  constexpr int VLOADS = V_BYTES / (kThreads * 16);
  constexpr int KSTEPS = DQK / 16;  // MFMA k-steps of S^T = K Q^T
  constexpr int NDB = DV / 32;      // 32-row blocks of O^T
  constexpr int OUT_RB = DV * (int)sizeof(OutT);  // epilogue row bytes
  constexpr int OUT_CPR = OUT_RB / 16;
  static_assert(K_BYTES % (kThreads * 16) == 0 && V_BYTES % (kThreads * 16) == 0, "tile loads");
  static_assert(4 * 32 * OUT_RB <= 2 * STAGE, "epilogue staging must fit in the K/V buffers");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Scalar wave index: every per-wave condition below is a uniform scalar
  // branch.  MFMA writes all 64 lanes whatever EXEC holds, so an MFMA must
  // never sit in a branch the compiler could run with a partial EXEC mask.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;

  // ---- work decode.  blockIdx.y counts query tiles from the end of each
  // sequence (longest causal rows first).  Within one (sequence, tile) slab
  // the query heads are ordered so that the heads dispatched to one XCD
  // (consecutive workgroups go round-robin over 8 XCDs) are neighbours, i.e.
  // mostly share their kv head and hit the same L2.
  const int hx = blockIdx.x % a.hq;
  const int seq = blockIdx.x / a.hq;
  int head = hx;
  if ((a.hq & 7) == 0) {
    const int per_xcd = a.hq >> 3;
    head = (hx & 7) * per_xcd + (hx >> 3);
  }
  const int cq0 = a.cu_q[seq];
  const int lq = a.cu_q[seq + 1] - cq0;
  const int ck0 = a.cu_kv[seq];
  const int lk = a.cu_kv[seq + 1] - ck0;
  const int n_qtiles = (lq + kBM - 1) / kBM;
  const int qtile = n_qtiles - 1 - (int)blockIdx.y;
  if (qtile < 0) return;

  const int r0 = qtile * kBM;
  const int r1 = min(lq, r0 + kBM);
  const int off = lk - lq;
  const int g = head / a.group;
  const bool causal = a.causal != 0;
  const int W = a.window;

  int kv_hi = lk;
  if (causal) kv_hi = min(lk, r1 - 1 + off + 1);
  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, r0 + off - W + 1);
  const int t_begin = kv_lo / BN;
  int t_end = kv_hi > 0 ? (kv_hi + BN - 1) / BN : 0;
  if (t_end < t_begin) t_end = t_begin;

  if (a.tile_counts != nullptr && tid == 0 && qtile < (int)gridDim.y)
    a.tile_counts[((int64_t)qtile * a.num_seqs + seq) * a.hq + head] = t_end - t_begin;

  const int w0 = r0 + wave * 32;
  const int w1 = min(lq, w0 + 32);
  const bool wave_active = w0 < lq;
  const int my_row = w0 + l32;
  const bool row_ok = my_row < lq;
  int wkv_hi = lk;
  if (causal) wkv_hi = min(lk, w1 - 1 + off + 1);
  int wkv_lo = 0;
  if (W > 0) wkv_lo = max(0, w0 + off - W + 1);
  bool split;
  {
    const int nvis = (causal ? min(lk, w0 + off + 1) : lk) - wkv_lo;
    split = (nvis < a.split_keys) || (BIAS && a.split_bias != 0);
  }

  const int64_t k_st_b = a.k_st * 2;
  const int64_t v_st_b = a.v_st * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)ck0 * a.k_st + (int64_t)g * a.k_sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v) + ((int64_t)ck0 * a.v_st + (int64_t)g * a.v_sh) * 2;

  // Per-lane byte offsets (within a tile, from its first key) of the chunks
  // this lane copies; the same for every tile.
  uint32_t koff[KLOADS];
  uint32_t voff[VLOADS];
#pragma unroll
  for (int i = 0; i < KLOADS; ++i) {
    const int pos = i * kThreads + tid;  // 16-byte slot in the LDS tile
    const int key = pos / KCPR;
    const int c = (pos % KCPR) ^ KSwz<DQK>::f(key);
    koff[i] = (uint32_t)(key * k_st_b + c * 16);
  }
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) {
    const int pos = i * kThreads + tid;
    const int key = pos / VCPR;
    const int c = (pos % VCPR) ^ VSwz<DV>::f(key);
    voff[i] = (uint32_t)(key * v_st_b + c * 16);
  }

  auto load_tile = [&](int t, int buf) __attribute__((device)) {
    load_kv_tile<DQK, DV, KLOADS, VLOADS>(kbase, vbase, k_st_b, v_st_b, t * BN, min(lk - t * BN, BN),
                                         (lds_char*)smem + buf * STAGE + wave * 1024, K_BYTES, koff,
                                         voff);
  };

  // ---- Q fragments (B operand of S^T = K Q^T), loaded once.
  u32x4_t qf[KSTEPS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)(cq0 + my_row) * a.q_st +
                  (int64_t)head * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + 16 * ks + 8 * hf)
                      : (u32x4_t){0u, 0u, 0u, 0u};
  }

  // LDS byte offsets of this lane's operand reads (tile-relative).
  // K: key 32 mb + l32, chunk 2 ks + hf.
  // V (transposing read r of k-step kk, d-block db): key 16 kk + 8 r + 4 hf +
  // (lane % 16) / 4, head dims 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4) .. +3.
  const int vkey_lane = 4 * hf + ((lane & 15) >> 2);
  const int vchunk_lane = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vbyte_lane = (lane & 1) * 8;

  f32x16_t o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m_run = kNegInf;
  float l_run = 0.0f;
  const float c_scale = a.scale_log2;
  const float* brow = nullptr;
  if constexpr (BIAS) {
    brow = a.bias + (int64_t)(cq0 + (row_ok ? my_row : 0)) * a.b_st +
           (int64_t)(a.bias_heads == 1 ? 0 : head) * a.b_sh;
  }

  if (t_begin < t_end) load_tile(t_begin, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    if (t + 1 < t_end) load_tile(t + 1, buf ^ 1);

    const int kb = t * BN;
    const bool wave_tile = wave_active && kb < wkv_hi && kb + BN > wkv_lo;
    if (wave_tile) {
      const lds_char* ks = (const lds_char*)smem + buf * STAGE;
      const lds_char* vs = ks + K_BYTES;

      f32x16_t s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mb][e] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int key = 32 * mb + l32;
          const int c = (2 * kk + hf) ^ KSwz<DQK>::f(key);
          const u32x4_t kf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
              ks + key * KRB + c * 16);
          s[mb] = E::mma(kf, qf[kk], s[mb]);
        }
      }

      const bool need_mask = (kb + BN > lk) || (causal && kb + BN - 1 > w0 + off) ||
                             (W > 0 && kb <= w1 - 1 + off - W);
      if (need_mask) {
        const int lim_hi = causal ? my_row + off : lk - 1;
        const int lim_lo = W > 0 ? my_row + off - W : -1;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb + 32 * mb + 8 * (e >> 2) + 4 * hf + (e & 3);
            const bool ok = key < lk && key <= lim_hi && key > lim_lo;
            s[mb][e] = ok ? s[mb][e] : kNegInf;
          }
      }

      if constexpr (BIAS) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int key0 = kb + 32 * mb + 8 * qd + 4 * hf;
            f32x4_t bv;
            if (row_ok && key0 + 3 < lk) {
              bv = *reinterpret_cast<const f32x4_t*>(brow + key0);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) bv[e] = (row_ok && key0 + e < lk) ? brow[key0 + e] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[mb][4 * qd + e] = __builtin_fmaf(s[mb][4 * qd + e], c_scale, bv[e] * kLog2e);
          }
      }

      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_tile = BIAS ? mx : mx * c_scale;

      // Per-row lazy rescale (alpha = 1 for rows whose max stayed within the
      // threshold: exact, so a row never depends on its wave neighbours).
      const bool grow = m_tile > m_run + kRescaleThreshold;
      if (__ballot(grow) != 0ull) {
        const float m_new = grow ? m_tile : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == kNegInf) ? 0.0f : m_run;

      float lsum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = BIAS ? s[mb][e] - m_use : __builtin_fmaf(s[mb][e], c_scale, -m_use);
          const float p = fast_exp2(x);
          s[mb][e] = p;
          lsum += p;
        }
      l_run += lsum;

      // P as the B operand: k-step kk takes S^T entries 8 (kk % 2) .. +7 of
      // block kk / 2, i.e. keys 16 kk + {0..3, 8..11} + 4 hf; the transposing
      // V reads fetch the same keys in the same order.
      u32x4_t ph[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int mb = kk >> 1, b8 = 8 * (kk & 1);
#pragma unroll
        for (int w = 0; w < 4; ++w) ph[kk][w] = E::pack(s[mb][b8 + 2 * w], s[mb][b8 + 2 * w + 1]);
      }
      auto vfrag = [&](int kk, int db) -> u32x4_t {
        u32x4_t r;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int key = 16 * kk + 8 * h + vkey_lane;
          const int c = (4 * db + vchunk_lane) ^ VSwz<DV>::f(key);
          const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(vs + key * VRB + c * 16 + vbyte_lane));
          const u32x2_t xw = __builtin_bit_cast(u32x2_t, x);
          r[2 * h] = xw[0];
          r[2 * h + 1] = xw[1];
        }
        return r;
      };
      if (split) {
        u32x4_t pl[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int mb = kk >> 1, b8 = 8 * (kk & 1);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float x0 = s[mb][b8 + 2 * w], x1 = s[mb][b8 + 2 * w + 1];
            pl[kk][w] = E::pack(x0 - E::round_trip(x0), x1 - E::round_trip(x1));
          }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x4_t vf = vfrag(kk, db);
            o[db] = E::mma(vf, ph[kk], o[db]);
            o[db] = E::mma(vf, pl[kk], o[db]);
          }
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db] = E::mma(vfrag(kk, db), ph[kk], o[db]);
      }
    }

    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies of tile t+1 have landed
    __syncthreads();
  }

  // ---- epilogue: O / l staged through LDS (the K/V buffers are free after
  // the loop's last barrier) so that every output row is written as
  // contiguous 16-byte stores.
  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  lds_char* ostage = (lds_char*)smem + wave * 32 * OUT_RB;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = 32 * db + 8 * qd + 4 * hf;
      const float v0 = o[db][4 * qd] * inv, v1 = o[db][4 * qd + 1] * inv;
      const float v2 = o[db][4 * qd + 2] * inv, v3 = o[db][4 * qd + 3] * inv;
      const int byte = d0 * (int)sizeof(OutT);
      const int c = (byte >> 4) ^ (l32 & (OUT_CPR - 1));
      lds_char* dst = ostage + l32 * OUT_RB + c * 16 + (byte & 15);
      if constexpr (sizeof(OutT) == 4) {
        *(__attribute__((address_space(3))) f32x4_t*)dst = (f32x4_t){v0, v1, v2, v3};
      } else {
        *(__attribute__((address_space(3))) u32x2_t*)dst =
            (u32x2_t){Elem<OutT>::pack(v0, v1), Elem<OutT>::pack(v2, v3)};
      }
    }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_wave_barrier();
  {
    constexpr int RPI = 64 / OUT_CPR;  // rows per wave-wide pass
    const int cc = lane % OUT_CPR;
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int q = it * RPI + lane / OUT_CPR;
      const int c = cc ^ (q & (OUT_CPR - 1));
      const u32x4_t val = *(const __attribute__((address_space(3))) u32x4_t*)(ostage + q * OUT_RB + c * 16);
      if (w0 + q < lq) {
        char* dst = reinterpret_cast<char*>(a.out) +
                    ((int64_t)(cq0 + w0 + q) * a.o_st + (int64_t)head * a.o_sh) * (int64_t)sizeof(OutT) +
                    cc * 16;
        *reinterpret_cast<u32x4_t*>(dst) = val;
      }
    }
  }
  if (a.lse != nullptr && hf == 0 && row_ok) {
    const float m_use = (m_run == kNegInf) ? 0.0f : m_run;
    a.lse[(int64_t)head * a.total_q + cq0 + my_row] =
        l_tot > 0.0f ? (m_use + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

template <typename T, int DQK, int DV, bool BIAS, typename OutT>
hipError_t launch_one(const KernelArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (Elem<T>::kWide) {
    hipLaunchKernelGGL((attn_fwd_kernel<T, DQK, DV, BIAS, OutT>), grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_fwd16_kernel<T, DQK, DV, BIAS, OutT>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, int DQK, int DV>
hipError_t launch_dims(const KernelArgs& a, bool bias, bool out_f32, dim3 grid, hipStream_t s) {
  if (bias) {
    return out_f32 ? launch_one<T, DQK, DV, true, float>(a, grid, s)
                   : launch_one<T, DQK, DV, true, T>(a, grid, s);
  }
  return out_f32 ? launch_one<T, DQK, DV, false, float>(a, grid, s)
                 : launch_one<T, DQK, DV, false, T>(a, grid, s);
}

template <typename T>
hipError_t launch_type(const KernelArgs& a, int dqk, int dv, bool bias, bool out_f32, dim3 grid,
                       hipStream_t s) {
  if (dqk == 64 && dv == 64) return launch_dims<T, 64, 64>(a, bias, out_f32, grid, s);
  if (dqk == 128 && dv == 128) return launch_dims<T, 128, 128>(a, bias, out_f32, grid, s);
  if constexpr (!Elem<T>::kWide) {
    if (dqk == 192 && dv == 128) return launch_dims<T, 192, 128>(a, bias, out_f32, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int tile_bn(int in_dtype) { return in_dtype == kF32 ? Geo<float, 64, 64>::BN : Geo<__bf16, 64, 64>::BN; }

hipError_t launch_attn_fwd(const KernelArgs& a, int in_dtype, int out_dtype, int dqk, int dv,
                           bool bias, dim3 grid, hipStream_t stream) {
  (void)hipGetLastError();  // clear a stale error so the check below is about this launch
  const bool out_f32 = out_dtype == kF32;
  switch (in_dtype) {
    case kBF16: return launch_type<__bf16>(a, dqk, dv, bias, out_f32, grid, stream);
    case kF16: return launch_type<_Float16>(a, dqk, dv, bias, out_f32, grid, stream);
    case kF32: return launch_type<float>(a, dqk, dv, bias, true, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mi_attn
