// Backward of the fused variable-length attention for gfx950 (MI355X, CDNA4):
// dq, dk, dv from q, k, v, the forward's lse and the output gradient dout.
//
// The gradients follow from the forward's definition (out = softmax(z) v,
// z = scale q k^T, masked): with p the forward's probabilities,
//   dv_j = sum_i p_ij dout_i,   dp_ij = dout_i . v_j,   D_i = dout_i . out_i,
//   ds_ij = p_ij (dp_ij - D_i),  dq_i = scale sum_j ds_ij k_j,
//   dk_j = scale sum_i ds_ij q_i,
// dk and dv summed over the query heads that share a kv head.  This is the
// tiled FlashAttention-2 backward that the triton-msl part-2 post (section
// "Beyond softmax: linear attention and a trainable backward") ships for its
// forward; p is recomputed tile by tile from the saved lse, never stored.
//
// Three kernels, no atomics (every output element has one writer, so the
// result is bitwise deterministic):
//   delta_kernel  D = rowsum(dout * out) per (row, head), fp32;
//   dkdv_kernel   one workgroup per (sequence, kv head, 128 keys): each wave
//                 owns 32 keys (one key per lane column) and loops over the
//                 query heads of its kv head's group and the 64-row query
//                 tiles that see its keys.  S = Q K^T and dP = dO V^T on MFMA
//                 with keys on the N axis, so each lane's accumulator column
//                 is one key and P, dS feed the dV^T = dO^T P and
//                 dK^T = Q^T dS products directly as B operands; dO^T and Q^T
//                 come from the row-major LDS tiles through the transposing
//                 LDS read;
//   dq_kernel     one workgroup per (sequence, query head, 128 rows), laid
//                 out like the forward: S^T = K Q^T and dP^T = V dO^T with
//                 one query per lane column, dQ^T = K^T dS^T with K^T from the
//                 transposing LDS read of the row-major K tile.
// P and dS are rounded to the input type (RNE) for the MFMAs, which
// accumulate in fp32.
#pragma once

#include "attn_bwd.h"
#include "attn_fwd_kernels.h"
#include "tile_lds.h"

namespace mi_attn {
namespace {

// ----------------------------------------------------------------------------
// delta_kernel: D[h][t] = sum_d dout[t][h][d] * out[t][h][d], fp32.  DV / 8
// lanes per (row, head), 16-byte loads.
// ----------------------------------------------------------------------------
template <typename OutT, int DV>
__global__ __launch_bounds__(256) void delta_kernel(const BwdArgs a) {
  // out and dout in the input type (the forward's default output type)
  constexpr int EPL = 16 / (int)sizeof(OutT);  // elements per 16-byte load
  constexpr int LPR_D = DV / EPL;              // lanes holding a row's elements
  // lanes per (row, head): a power of two for the reduction (the 96-wide
  // head's 12 loads use 16 lanes; the other 4 add 0)
  constexpr int LPR = LPR_D <= 8 ? 8 : LPR_D <= 16 ? 16 : 32;
  static_assert(LPR >= LPR_D && 64 % LPR == 0, "lanes per row");
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  const int64_t total = a.total_q * a.hq;
  const bool ok = item < total && sub < LPR_D;
  const int64_t t = ok ? item / a.hq : 0;
  const int h = ok ? (int)(item % a.hq) : 0;
  float acc = 0.0f;
  if (ok) {
    const OutT* o = reinterpret_cast<const OutT*>(a.out) + t * a.o_st + (int64_t)h * a.o_sh + sub * EPL;
    const OutT* g = reinterpret_cast<const OutT*>(a.dout) + t * a.do_st + (int64_t)h * a.do_sh + sub * EPL;
    typedef __attribute__((__vector_size__(16))) char c16;
    const c16 ov = *reinterpret_cast<const c16*>(o);
    const c16 gv = *reinterpret_cast<const c16*>(g);
    const OutT* oe = reinterpret_cast<const OutT*>(&ov);
    const OutT* ge = reinterpret_cast<const OutT*>(&gv);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf((float)oe[e], (float)ge[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (ok && sub == 0) a.delta[(int64_t)h * a.total_q + t] = acc;
}

// Four consecutive gradient values of one row.
template <typename T>
__device__ __forceinline__ void store_grad4(T* p, float a, float b, float c, float d) {
  store4<T>(p, a, b, c, d);
}

// ----------------------------------------------------------------------------
// dkdv_kernel
// ----------------------------------------------------------------------------
// ALIBI: the bias is -slope * |query position - key|, computed (BIAS set too).
// MFMA operands of the dK / dV kernel are read this many MFMAs ahead.
#ifndef MI_ATTN_BWD_AHEAD
#define MI_ATTN_BWD_AHEAD 4
#endif

template <typename T, int D, typename GradT, bool BIAS, bool ALIBI = false>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(const BwdArgs a) {
  constexpr int BK = 128;              // keys per workgroup (32 per wave)
  constexpr int BQ = 64;               // query rows per step (two 32-row blocks)
  constexpr int KS = D / 16;           // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;          // 32-wide d blocks of dK^T / dV^T
  // LDS rows are DL wide: the 96-wide head is laid out like the 128-wide one
  // (its 4 pad chunks are copied, beyond the row, and never read), so that
  // the power-of-two swizzle holds
  constexpr int DL = lds_dim(D);
  constexpr int TILE = BQ * DL * 2;    // bytes of one Q or dO tile
  constexpr int LOADS = TILE / (kThreads * 16);
  using E = Elem<T>;

  __shared__ __attribute__((aligned(1024))) char qt_0[TILE];
  __shared__ __attribute__((aligned(1024))) char qt_1[TILE];
  __shared__ __attribute__((aligned(1024))) char gt_0[TILE];
  __shared__ __attribute__((aligned(1024))) char gt_1[TILE];
  __shared__ __attribute__((aligned(16))) float ls_0[BQ], ls_1[BQ], dl_0[BQ], dl_1[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;

  const int g = blockIdx.x % a.hkv;
  const int seq = blockIdx.x / a.hkv;
  const int ktile = blockIdx.y;  // key tiles in order: the first ones see the most queries
  int cq0 = a.cu_q[seq], cq1 = a.cu_q[seq + 1];
  int ck0 = a.cu_kv[seq], ck1 = a.cu_kv[seq + 1];
  asm volatile("" : "+s"(cq0), "+s"(cq1), "+s"(ck0), "+s"(ck1));
  const int lq = cq1 - cq0;
  const int lk = ck1 - ck0;
  const int kb0 = ktile * BK;
  if (kb0 >= lk) return;
  const int kb1 = min(lk, kb0 + BK);
  const int off = lk - lq;
  const bool causal = a.causal != 0;
  const int W = a.window;

  // Query rows that see at least one of the workgroup's keys.
  int q_lo = 0, q_hi = lq;
  if (causal) q_lo = max(0, kb0 - off);
  if (W > 0) q_hi = min(lq, kb1 - 1 - off + W);
  q_lo = q_lo / BQ * BQ;
  const int n_qt = q_hi > q_lo ? (q_hi - q_lo + BQ - 1) / BQ : 0;
  const int n_it = n_qt * a.group;  // (query head of the group, query tile) pairs

  // This wave's keys and the rows that see them.
  const int kw0 = kb0 + 32 * wave;
  const int kw1 = min(lk, kw0 + 32);
  const bool wave_keys = kw0 < lk;
  const int my_key = kw0 + l32;
  int wq_lo = 0, wq_hi = lq;
  if (causal) wq_lo = max(0, kw0 - off);
  if (W > 0) wq_hi = min(lq, kw1 - 1 - off + W);

  // K and V fragments of the wave's keys (B operands: key = lane column,
  // 8 consecutive d), loaded once.  Keys past the sequence end read as 0.
  u32x4_t kf[KS], vf[KS];
  {
    const int64_t k_st_b = a.k_st * 2, v_st_b = a.v_st * 2;
    const char* kb = uniform_ptr(reinterpret_cast<const char*>(a.k) +
                                 ((int64_t)(ck0 + kw0) * a.k_st + (int64_t)g * a.k_sh) * 2);
    const char* vb = uniform_ptr(reinterpret_cast<const char*>(a.v) +
                                 ((int64_t)(ck0 + kw0) * a.v_st + (int64_t)g * a.v_sh) * 2);
    const int rows = kw1 - kw0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, rows > 0 ? (uint32_t)((rows - 1) * k_st_b + D * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, rows > 0 ? (uint32_t)((rows - 1) * v_st_b + D * 2) : 0u);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(l32 * k_st_b) + 32 * ks + 16 * hf, 0, 0);
      vf[ks] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(l32 * v_st_b) + 32 * ks + 16 * hf, 0, 0);
    }
  }

  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[i][e] = dv[i][e] = 0.0f;

  uint32_t qoff[LOADS], goff[LOADS];
  tile_offsets<DL, LOADS>(qoff, a.q_st * 2, tid);
  tile_offsets<DL, LOADS>(goff, a.do_st * 2, tid);
  const float c_scale = a.scale_log2;

  // Stage iteration `it` (query head h = g * group + it % group, tile it / group):
  // the Q and dO tiles go to LDS by direct copies; the rows' lse and delta
  // are loaded into registers (first wave) and written to LDS by stage_lds
  // once the step's copies have landed, so no wave waits for a load in the
  // middle of a step.
  float st_l = 0.0f, st_d = 0.0f;
  bool st_row = false;
  auto stage = [&](int it, auto S) __attribute__((device)) {
    constexpr int s = decltype(S)::value;
    const int h = g * a.group + it % a.group;
    const int q0 = q_lo + (it / a.group) * BQ;
    const int rows = min(BQ, lq - q0);
    const char* qb = reinterpret_cast<const char*>(a.q) + ((int64_t)(cq0 + q0) * a.q_st + (int64_t)h * a.q_sh) * 2;
    const char* gb = reinterpret_cast<const char*>(a.dout) + ((int64_t)(cq0 + q0) * a.do_st + (int64_t)h * a.do_sh) * 2;
    load_tile<D, LOADS>(qb, a.q_st * 2, rows, (lds_char*)(s == 0 ? qt_0 : qt_1), qoff, wave);
    load_tile<D, LOADS>(gb, a.do_st * 2, rows, (lds_char*)(s == 0 ? gt_0 : gt_1), goff, wave);
    st_row = tid < rows;
    if (st_row) {
      st_l = a.lse[(int64_t)h * a.total_q + cq0 + q0 + tid];
      st_d = a.delta[(int64_t)h * a.total_q + cq0 + q0 + tid];
    }
  };
  auto stage_lds = [&](auto S) __attribute__((device)) {
    constexpr int s = decltype(S)::value;
    if (tid < BQ) {
      // log2-domain lse (+inf where the row does not exist or sees nothing:
      // its p is then exactly 0) and delta
      const float l2 = !st_row || st_l == -__builtin_inff() ? __builtin_inff() : st_l * kLog2e;
      (s == 0 ? ls_0 : ls_1)[tid] = l2;
      (s == 0 ? dl_0 : dl_1)[tid] = st_row ? st_d : 0.0f;
    }
  };

  auto compute = [&](int it, auto S) __attribute__((device)) {
    constexpr int s = decltype(S)::value;
    const int q0 = q_lo + (it / a.group) * BQ;
    const int h = g * a.group + it % a.group;
    // bias column of this lane's key (keys at or past the bias columns read 0)
    const float* bcol = nullptr;
    const bool bkey = BIAS && !ALIBI && my_key < min(lk, a.bias_cols);
    if constexpr (BIAS && !ALIBI)
      bcol = a.bias + (int64_t)(a.bias_heads == 1 ? 0 : h) * a.b_sh + (bkey ? my_key : 0);
    const float neg_slope = ALIBI ? -a.alibi[(int64_t)seq * a.alibi_ss + h] : 0.0f;
    if (!wave_keys || q0 >= wq_hi || q0 + BQ <= wq_lo) return;  // no visible pair for this wave
    const lds_char* qt = (const lds_char*)(s == 0 ? qt_0 : qt_1);
    const lds_char* gt = (const lds_char*)(s == 0 ? gt_0 : gt_1);
    const float* ls = s == 0 ? ls_0 : ls_1;
    const float* dl = s == 0 ? dl_0 : dl_1;
    // Entry e of block qb is query row q0 + 32 qb + 8 (e/4) + 4 hf + e%4 and key my_key.
    const bool need_mask = (causal && kw1 - 1 > q0 + off) || (W > 0 && kw0 <= q0 + BQ - 1 + off - W);
    u32x4_t pb[2][2], sb[2][2];
    // P and dS of one 32-row block from its scores sc and dP values dp; the
    // causal / window mask (MASK) only where the step's tile crosses it.
    auto probs = [&](int qb, f32x16_t& sc, f32x16_t& dp, auto MASK) __attribute__((device)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 32 * qb + 8 * j + 4 * hf;  // tile row of entries 4j .. 4j + 3
        const f32x4_t l2 = *reinterpret_cast<const f32x4_t*>(ls + r);
        const f32x4_t dd = *reinterpret_cast<const f32x4_t*>(dl + r);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * j + i;
          float x = sc[e] * c_scale;
          if constexpr (BIAS) {
            // logit = scale s + bias, in log2 units
            const int row = q0 + r + i;
            float b;
            if constexpr (ALIBI)
              b = neg_slope * __builtin_fabsf((float)(row + off - my_key));
            else
              b = (bkey && row < lq) ? bcol[(int64_t)(cq0 + row) * a.b_st] : 0.0f;
            x = __builtin_fmaf(b, kLog2e, x);
          }
          float p = fast_exp2(x - l2[i]);
          if constexpr (decltype(MASK)::value) {
            const int row = q0 + r + i;
            const bool vis = (!causal || my_key <= row + off) && (W == 0 || my_key > row + off - W);
            p = vis ? p : 0.0f;
          }
          sc[e] = p;
          dp[e] = p * (dp[e] - dd[i]);
        }
      }
    };
    // With one wave per SIMD nothing hides an LDS read's latency but the
    // wave's own work: every MFMA's operand is read MI_ATTN_BWD_AHEAD MFMAs
    // before it (a ring of fragments), and scheduling fences keep that order.
    constexpr int AH = MI_ATTN_BWD_AHEAD;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t sc, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.0f;
      // S = Q K^T, dP = dO V^T: MFMA i takes a Q (even i) or dO (odd i)
      // fragment of k-step i / 2
      auto rd_s = [&](int i) __attribute__((device)) -> u32x4_t {
        return row_frag<DL>((i & 1) ? gt : qt, 32 * qb + l32, i >> 1, hf);
      };
      u32x4_t fr[AH + 1];
#pragma unroll
      for (int i = 0; i < AH; ++i) fr[i] = rd_s(i);
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        if (i + AH < 2 * KS) fr[(i + AH) % (AH + 1)] = rd_s(i + AH);
        if (i & 1)
          dp = E::mma(fr[i % (AH + 1)], vf[i >> 1], dp);
        else
          sc = E::mma(fr[i % (AH + 1)], kf[i >> 1], sc);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (need_mask)
        probs(qb, sc, dp, std::true_type{});
      else
        probs(qb, sc, dp, std::false_type{});
      pb[qb][0] = pack_b<T>(sc, 0);
      pb[qb][1] = pack_b<T>(sc, 1);
      sb[qb][0] = pack_b<T>(dp, 0);
      sb[qb][1] = pack_b<T>(dp, 1);
    }
    // dV^T += dO^T P, dK^T += Q^T dS (reduction over the 64 query rows):
    // MFMA i is (block, k-step, d block) = i / (4 NDB), (i / (2 NDB)) % 2,
    // (i / 2) % NDB, dV (even i) or dK (odd i)
    constexpr int NT = 8 * NDB;
    auto rd_t = [&](int i) __attribute__((device)) -> u32x4_t {
      const int qb = i / (4 * NDB), kk = (i / (2 * NDB)) % 2, db = (i / 2) % NDB;
      return tr_frag<DL>((i & 1) ? qt : gt, 2 * qb + kk, db, lane);
    };
    u32x4_t tf[AH + 1];
#pragma unroll
    for (int i = 0; i < AH; ++i) tf[i] = rd_t(i);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (i + AH < NT) tf[(i + AH) % (AH + 1)] = rd_t(i + AH);
      const int qb = i / (4 * NDB), kk = (i / (2 * NDB)) % 2, db = (i / 2) % NDB;
      if (i & 1)
        dk[db] = E::mma(tf[i % (AH + 1)], sb[qb][kk], dk[db]);
      else
        dv[db] = E::mma(tf[i % (AH + 1)], pb[qb][kk], dv[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_it > 0) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    stage(0, S0{});
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stage_lds(S0{});
    __syncthreads();
    for (int it = 0; it < n_it; it += 2) {
      if (it + 1 < n_it) stage(it + 1, S1{});
      compute(it, S0{});
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if (it + 1 < n_it) stage_lds(S1{});
      __syncthreads();
      if (it + 1 < n_it) {
        if (it + 2 < n_it) stage(it + 2, S0{});
        compute(it + 1, S1{});
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (it + 2 < n_it) stage_lds(S0{});
        __syncthreads();
      }
    }
  }

  // dK = scale dK^T, dV = dV^T: lane column = key, entries = d rows.
  if (!wave_keys || my_key >= lk) return;
  GradT* dkp = reinterpret_cast<GradT*>(a.dk) + (int64_t)(ck0 + my_key) * a.dk_st + (int64_t)g * a.dk_sh;
  GradT* dvp = reinterpret_cast<GradT*>(a.dv) + (int64_t)(ck0 + my_key) * a.dv_st + (int64_t)g * a.dv_sh;
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hf;
      store_grad4<GradT>(dkp + d0, dk[db][4 * j] * sc, dk[db][4 * j + 1] * sc, dk[db][4 * j + 2] * sc,
                         dk[db][4 * j + 3] * sc);
      store_grad4<GradT>(dvp + d0, dv[db][4 * j], dv[db][4 * j + 1], dv[db][4 * j + 2],
                         dv[db][4 * j + 3]);
    }
}

// ----------------------------------------------------------------------------
// dq_kernel
// ----------------------------------------------------------------------------
template <typename T, int D, typename GradT, bool BIAS, bool ALIBI = false>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(const BwdArgs a) {
  constexpr int BM = 128;              // query rows per workgroup (32 per wave)
  constexpr int BN = 32;               // keys per tile
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int DL = lds_dim(D);  // LDS row width (as in dkdv_kernel)
  constexpr int TILE = BN * DL * 2;
  constexpr int LOADS = TILE / (kThreads * 16);
  using E = Elem<T>;

  __shared__ __attribute__((aligned(1024))) char kt_0[TILE];
  __shared__ __attribute__((aligned(1024))) char kt_1[TILE];
  __shared__ __attribute__((aligned(1024))) char vt_0[TILE];
  __shared__ __attribute__((aligned(1024))) char vt_1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;

  const int head = blockIdx.x % a.hq;
  const int seq = blockIdx.x / a.hq;
  int cq0 = a.cu_q[seq], cq1 = a.cu_q[seq + 1];
  int ck0 = a.cu_kv[seq], ck1 = a.cu_kv[seq + 1];
  asm volatile("" : "+s"(cq0), "+s"(cq1), "+s"(ck0), "+s"(ck1));
  const int lq = cq1 - cq0;
  const int lk = ck1 - ck0;
  const int n_qtiles = (lq + BM - 1) / BM;
  const int qtile = (int)gridDim.y - 1 - (int)blockIdx.y;  // heaviest causal tiles first
  if (qtile >= n_qtiles) return;
  const int r0 = qtile * BM;
  const int r1 = min(lq, r0 + BM);
  const int off = lk - lq;
  const int g = head / a.group;
  const bool causal = a.causal != 0;
  const int W = a.window;

  int kv_hi = lk;
  if (causal) kv_hi = min(lk, r1 - 1 + off + 1);
  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, r0 + off - W + 1);
  const int t_begin = kv_lo / BN;
  const int t_end = kv_hi > t_begin * BN ? (kv_hi + BN - 1) / BN : t_begin;

  const int w0 = r0 + 32 * wave;
  const int w1 = min(lq, w0 + 32);
  const bool wave_rows = w0 < lq;
  const int my_row = w0 + l32;
  const bool row_ok = my_row < lq;
  int wk_hi = lk, wk_lo = 0;
  if (causal) wk_hi = min(lk, w1 - 1 + off + 1);
  if (W > 0) wk_lo = max(0, w0 + off - W + 1);

  // Q and dO fragments of the wave's rows (B operands: query = lane column).
  u32x4_t qf[KS], gf[KS];
  {
    const int64_t q_st_b = a.q_st * 2, g_st_b = a.do_st * 2;
    const int rows = w1 - w0;
    const char* qb = uniform_ptr(reinterpret_cast<const char*>(a.q) +
                                 ((int64_t)(cq0 + w0) * a.q_st + (int64_t)head * a.q_sh) * 2);
    const char* gb = uniform_ptr(reinterpret_cast<const char*>(a.dout) +
                                 ((int64_t)(cq0 + w0) * a.do_st + (int64_t)head * a.do_sh) * 2);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, rows > 0 ? (uint32_t)((rows - 1) * q_st_b + D * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gb, rows > 0 ? (uint32_t)((rows - 1) * g_st_b + D * 2) : 0u);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(l32 * q_st_b) + 32 * ks + 16 * hf, 0, 0);
      gf[ks] = __builtin_amdgcn_raw_buffer_load_b128(rg, (int)(l32 * g_st_b) + 32 * ks + 16 * hf, 0, 0);
    }
  }
  const float* brow = nullptr;
  if constexpr (BIAS && !ALIBI)
    brow = a.bias + (int64_t)(cq0 + (row_ok ? my_row : 0)) * a.b_st +
           (int64_t)(a.bias_heads == 1 ? 0 : head) * a.b_sh;
  const int blim = BIAS ? min(lk, a.bias_cols) : 0;
  const float neg_slope = ALIBI ? -a.alibi[(int64_t)seq * a.alibi_ss + head] : 0.0f;
  float l2 = __builtin_inff(), dd = 0.0f;
  if (row_ok) {
    const float l = a.lse[(int64_t)head * a.total_q + cq0 + my_row];
    l2 = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
    dd = a.delta[(int64_t)head * a.total_q + cq0 + my_row];
  }

  f32x16_t dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.0f;

  uint32_t koff[LOADS], voff[LOADS];
  tile_offsets<DL, LOADS>(koff, a.k_st * 2, tid);
  tile_offsets<DL, LOADS>(voff, a.v_st * 2, tid);
  const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)ck0 * a.k_st + (int64_t)g * a.k_sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v) + ((int64_t)ck0 * a.v_st + (int64_t)g * a.v_sh) * 2;
  const float c_scale = a.scale_log2;

  auto stage = [&](int t, auto S) __attribute__((device)) {
    constexpr int s = decltype(S)::value;
    const int kb = t * BN;
    load_tile<D, LOADS>(kbase + (int64_t)kb * a.k_st * 2, a.k_st * 2, min(BN, lk - kb),
                        (lds_char*)(s == 0 ? kt_0 : kt_1), koff, wave);
    load_tile<D, LOADS>(vbase + (int64_t)kb * a.v_st * 2, a.v_st * 2, min(BN, lk - kb),
                        (lds_char*)(s == 0 ? vt_0 : vt_1), voff, wave);
  };

  auto compute = [&](int t, auto S) __attribute__((device)) {
    constexpr int s = decltype(S)::value;
    const int kb = t * BN;
    if (!wave_rows || kb >= wk_hi || kb + BN <= wk_lo) return;
    const lds_char* kt = (const lds_char*)(s == 0 ? kt_0 : kt_1);
    const lds_char* vt = (const lds_char*)(s == 0 ? vt_0 : vt_1);
    f32x16_t sc, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc = E::mma(row_frag<DL>(kt, l32, ks, hf), qf[ks], sc);
      dp = E::mma(row_frag<DL>(vt, l32, ks, hf), gf[ks], dp);
    }
    // entry e: key kb + 8 (e/4) + 4 hf + e%4, query my_row
    const bool need_mask = (kb + BN > lk) || (causal && kb + BN - 1 > w0 + off) ||
                           (W > 0 && kb <= w1 - 1 + off - W);
    const int hi = causal ? my_row + off : lk - 1;
    const int lo = W > 0 ? my_row + off - W : -1;
    f32x4_t bv[4];
    if constexpr (BIAS) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key0 = kb + 8 * j + 4 * hf;
        if constexpr (ALIBI) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            bv[j][i] = neg_slope * __builtin_fabsf((float)(my_row + off - (key0 + i)));
        } else if (row_ok && key0 + 3 < blim) {
          bv[j] = *reinterpret_cast<const f32x4_t*>(brow + key0);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) bv[j][i] = (row_ok && key0 + i < blim) ? brow[key0 + i] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = sc[e] * c_scale;
      if constexpr (BIAS) x = __builtin_fmaf(bv[e >> 2][e & 3], kLog2e, x);
      float p = fast_exp2(x - l2);
      if (need_mask) {
        const int key = kb + 8 * (e >> 2) + 4 * hf + (e & 3);
        p = (key < lk && key <= hi && key > lo) ? p : 0.0f;
      }
      dp[e] = p * (dp[e] - dd);
    }
    const u32x4_t s0 = pack_b<T>(dp, 0), s1 = pack_b<T>(dp, 1);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dq[db] = E::mma(tr_frag<DL>(kt, 0, db, lane), s0, dq[db]);
      dq[db] = E::mma(tr_frag<DL>(kt, 1, db, lane), s1, dq[db]);
    }
  };

  if (t_begin < t_end) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    stage(t_begin, S0{});
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (int t = t_begin; t < t_end; t += 2) {
      if (t + 1 < t_end) stage(t + 1, S1{});
      compute(t, S0{});
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (t + 1 < t_end) {
        if (t + 2 < t_end) stage(t + 2, S0{});
        compute(t + 1, S1{});
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
      }
    }
  }

  if (!row_ok) return;
  GradT* dqp = reinterpret_cast<GradT*>(a.dq) + (int64_t)(cq0 + my_row) * a.dq_st + (int64_t)head * a.dq_sh;
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hf;
      store_grad4<GradT>(dqp + d0, dq[db][4 * j] * sc, dq[db][4 * j + 1] * sc, dq[db][4 * j + 2] * sc,
                         dq[db][4 * j + 3] * sc);
    }
}

template <typename T, int D, typename GradT, bool BIAS, bool ALIBI = false>
hipError_t launch_bwd_grad(const BwdArgs& a, int max_seqlen_q, int max_seqlen_kv, hipStream_t stream) {
  // delta
  const int64_t items = a.total_q * a.hq;
  {
    constexpr int LPR = D / 8 <= 8 ? 8 : D / 8 <= 16 ? 16 : 32;  // as in delta_kernel
    const int64_t blocks = (items * LPR + 255) / 256;
    hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned n_kt = (unsigned)((max_seqlen_kv + 127) / 128);
  const unsigned n_qt = (unsigned)((max_seqlen_q + 127) / 128);
  hipLaunchKernelGGL((dkdv_kernel<T, D, GradT, BIAS, ALIBI>), dim3((unsigned)(a.hkv * a.num_seqs), n_kt),
                     dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_kernel<T, D, GradT, BIAS, ALIBI>), dim3((unsigned)(a.hq * a.num_seqs), n_qt),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// grad_f32: dq, dk, dv stored as fp32 instead of the input type; bias: a
// constant additive bias enters the logits
template <typename T, int D>
hipError_t launch_bwd_dims(const BwdArgs& a, bool grad_f32, bool bias, int max_seqlen_q,
                           int max_seqlen_kv, hipStream_t stream) {
  if (a.alibi != nullptr)
    return grad_f32 ? launch_bwd_grad<T, D, float, true, true>(a, max_seqlen_q, max_seqlen_kv, stream)
                    : launch_bwd_grad<T, D, T, true, true>(a, max_seqlen_q, max_seqlen_kv, stream);
  if (bias)
    return grad_f32 ? launch_bwd_grad<T, D, float, true>(a, max_seqlen_q, max_seqlen_kv, stream)
                    : launch_bwd_grad<T, D, T, true>(a, max_seqlen_q, max_seqlen_kv, stream);
  return grad_f32 ? launch_bwd_grad<T, D, float, false>(a, max_seqlen_q, max_seqlen_kv, stream)
                  : launch_bwd_grad<T, D, T, false>(a, max_seqlen_q, max_seqlen_kv, stream);
}

}  // namespace
}  // namespace mi_attn
