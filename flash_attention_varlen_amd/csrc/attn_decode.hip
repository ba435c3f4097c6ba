// Split-KV decode for gfx950: few query rows per sequence against a long
// key/value cache, the end-aligned causal convention of the mtlattn 0.3.0
// project page (section "Use": self-attention and cached decode both hold).
//
// With a handful of query rows one workgroup per (sequence, head) would use a
// sliver of the chip.  Here the key range of each (sequence, kv head) is cut
// into chunks, and each chunk is one workgroup of one wave:
//   * the rows of every query head that reads this kv head (GQA group) and
//     every query row of the sequence are packed onto the MFMA N axis (one
//     row per lane column, up to 64 rows), so each K/V element is read from
//     HBM once per chunk, not once per query head;
//   * the wave streams its chunk's K/V tiles (32 keys) through LDS (two
//     slots, buffer_load ... lds) and runs the forward's online softmax:
//     S^T = K Q^T and O^T += V^T P^T on MFMA, fp32 running max and sum, the
//     rescale only when a row's max grows past 2^8, and the low half of P
//     multiplied in while a row's sum is small against its largest p;
//   * the chunk's unnormalised output, running max and sum go to a
//     caller-provided fp32 workspace.
// A second kernel merges the chunks of every (row, head) with the LSE rule:
// M = max_c m_c, L = sum_c l_c 2^(m_c - M), out = sum_c O_c 2^(m_c - M) / L,
// lse = (M + log2 L) ln 2.  Decode is bound by HBM bandwidth: every K/V byte
// of the visible range is read once.
#include "attn_decode.h"
#include "tile_lds.h"

namespace mi_attn {
namespace {

// s_waitcnt immediate waiting until at most n vector-memory operations of
// this wave are outstanding (vmcnt bits 3:0 and 15:14; expcnt, lgkmcnt left
// at their maxima, i.e. not waited for).
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

constexpr int kDecodeBN = 32;  // keys per tile

template <typename T, int D, int NB>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeArgs a) {
  constexpr int BN = kDecodeBN;
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = BN * D * 2;
  constexpr int LOADS = TILE / (64 * 16);
  using E = Elem<T>;

  __shared__ __attribute__((aligned(1024))) char kt_0[TILE];
  __shared__ __attribute__((aligned(1024))) char kt_1[TILE];
  __shared__ __attribute__((aligned(1024))) char vt_0[TILE];
  __shared__ __attribute__((aligned(1024))) char vt_1[TILE];

  const int lane = threadIdx.x;
  const int hf = lane >> 5;
  const int l32 = lane & 31;
  const int g = blockIdx.x % a.hkv;
  const int seq = blockIdx.x / a.hkv;
  const int chunk = blockIdx.y;
  int cq0 = a.cu_q[seq], cq1 = a.cu_q[seq + 1];
  int ck0 = a.cu_kv[seq], ck1 = a.cu_kv[seq + 1];
  int uk = a.seqused_kv != nullptr ? a.seqused_kv[seq] : 0x7fffffff;
  asm volatile("" : "+s"(cq0), "+s"(cq1), "+s"(ck0), "+s"(ck1), "+s"(uk));
  const int lq = cq1 - cq0;
  const int lk = max(0, min(ck1 - ck0, uk));  // the cache keys in use
  const int off = lk - lq;
  const bool causal = a.causal != 0;
  const int W = a.window;
  const int R = a.group * lq;  // packed rows: (query head of the group, query row)

  // This lane's rows: r = 32 nb + l32 -> head g * group + r / lq, row r % lq.
  int row_i[NB], row_h[NB];
  bool row_ok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 32 * nb + l32;
    row_ok[nb] = r < R;
    row_i[nb] = row_ok[nb] ? r % lq : 0;
    row_h[nb] = g * a.group + (row_ok[nb] ? r / lq : 0);
  }

  // Keys any row sees: [lo, hi); this chunk's tiles.
  const int lo = W > 0 ? max(0, off - W + 1) : 0;
  const int hi = causal ? min(lk, lq - 1 + off + 1) : lk;
  const int t_begin = lo / BN + chunk * a.chunk_tiles;
  const int t_end = min((hi + BN - 1) / BN, t_begin + a.chunk_tiles);

  float m_run[NB], l_run[NB];
  f32x16_t o[NB][NDB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nb][db][e] = 0.0f;
  }

  if (R > 0 && hi > lo && t_begin < t_end) {
    // Q fragments (B operand, row = lane column); rows past R read as 0.
    u32x4_t qf[NB][KS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)(cq0 + row_i[nb]) * a.q_st +
                    (int64_t)row_h[nb] * a.q_sh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[nb][ks] = row_ok[nb] ? *reinterpret_cast<const u32x4_t*>(qp + 16 * ks + 8 * hf)
                                : (u32x4_t){0u, 0u, 0u, 0u};
    }
    uint32_t koff[LOADS], voff[LOADS];
    tile_offsets<D, LOADS, 64>(koff, a.k_st * 2, lane);
    tile_offsets<D, LOADS, 64>(voff, a.v_st * 2, lane);
    const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)ck0 * a.k_st + (int64_t)g * a.k_sh) * 2;
    const char* vbase = reinterpret_cast<const char*>(a.v) + ((int64_t)ck0 * a.v_st + (int64_t)g * a.v_sh) * 2;
    auto stage = [&](int t, lds_char* kd, lds_char* vd) __attribute__((device)) {
      const int kb = t * BN;
      load_tile<D, LOADS, 64>(kbase + (int64_t)kb * a.k_st * 2, a.k_st * 2, min(BN, lk - kb), kd, koff, 0);
      load_tile<D, LOADS, 64>(vbase + (int64_t)kb * a.v_st * 2, a.v_st * 2, min(BN, lk - kb), vd, voff, 0);
    };
    const float c_scale = a.scale_log2;

    auto compute = [&](int t, const lds_char* kt, const lds_char* vt) __attribute__((device)) {
      const int kb = t * BN;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x16_t s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = E::mma(row_frag<D>(kt, l32, ks, hf), qf[nb][ks], s);
        // mask: entry e is key kb + 8 (e/4) + 4 hf + e%4 of row row_i[nb]
        const int rhi = row_ok[nb] ? (causal ? min(lk - 1, row_i[nb] + off) : lk - 1) : -1;
        const int rlo = W > 0 ? row_i[nb] + off - W : -1;
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + 8 * (e >> 2) + 4 * hf + (e & 3);
          s[e] = (key <= rhi && key > rlo) ? s[e] * c_scale : kNegInf;
          mx = __builtin_fmaxf(mx, s[e]);
        }
        const float m_tile = max_with_other_half(mx);
        // lazy rescale: only past 2^kRescaleThreshold growth (or the first visible key)
        if (__ballot(m_tile > m_run[nb] + kRescaleThreshold) != 0ull) {
          const bool grow = m_tile > m_run[nb] + kRescaleThreshold;
          const float alpha = grow ? (m_run[nb] == kNegInf ? 0.0f : fast_exp2(m_run[nb] - m_tile)) : 1.0f;
          if (grow) m_run[nb] = m_tile;
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[nb][db][e] *= alpha;
        }
        const float m_use = m_run[nb] == kNegInf ? 0.0f : m_run[nb];
        float lsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[e] = fast_exp2(s[e] - m_use);
          lsum += s[e];
        }
        l_run[nb] += lsum;
        const u32x4_t p0 = pack_b<T>(s, 0), p1 = pack_b<T>(s, 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          o[nb][db] = E::mma(tr_frag<D>(vt, 0, db, lane), p0, o[nb][db]);
          o[nb][db] = E::mma(tr_frag<D>(vt, 1, db, lane), p1, o[nb][db]);
        }
        // low halves of P while the row's sum is small against this tile's
        // largest p (exp2(m_tile - m_run)); other rows add zeros
        const float l_row = sum_with_other_half(l_run[nb]);
        const bool lo_row = m_tile != kNegInf && l_row < a.split_l * fast_exp2(m_tile - m_use);
        if (__ballot(lo_row) != 0ull) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            u32x4_t pl;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float x0 = s[8 * kk + 2 * w], x1 = s[8 * kk + 2 * w + 1];
              float h0, h1;
              E::unpack(E::pack(x0, x1), h0, h1);
              pl[w] = lo_row ? E::pack(x0 - h0, x1 - h1) : 0u;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              o[nb][db] = E::mma(tr_frag<D>(vt, kk, db, lane), pl, o[nb][db]);
          }
        }
      }
    };

    lds_char* k0 = (lds_char*)kt_0;
    lds_char* k1 = (lds_char*)kt_1;
    lds_char* v0 = (lds_char*)vt_0;
    lds_char* v1 = (lds_char*)vt_1;
    stage(t_begin, k0, v0);
    for (int t = t_begin; t < t_end; t += 2) {
      // tile t is in slot 0, t + 1 goes to slot 1 (the slot's last reads
      // were consumed by the previous step's MFMAs)
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      if (t + 1 < t_end) {
        stage(t + 1, k1, v1);
        __builtin_amdgcn_s_waitcnt(wait_vm(2 * LOADS));
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      }
      compute(t, k0, v0);
      if (t + 1 < t_end) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        if (t + 2 < t_end) {
          stage(t + 2, k0, v0);
          __builtin_amdgcn_s_waitcnt(wait_vm(2 * LOADS));
        } else {
          __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
        compute(t + 1, k1, v1);
      }
    }
  }

  // partial results of this chunk
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l_tot = l_run[nb] + __shfl_xor(l_run[nb], 32);
    if (!row_ok[nb]) continue;
    const int64_t w = ((int64_t)chunk * a.total_q + cq0 + row_i[nb]) * a.hq + row_h[nb];
    if (hf == 0) {
      a.ws_ml[2 * w] = m_run[nb];
      a.ws_ml[2 * w + 1] = l_tot;
    }
    if (m_run[nb] == kNegInf) continue;  // nothing visible: the merge skips this chunk
    float* op = a.ws_o + w * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * hf;
        *reinterpret_cast<f32x4_t*>(op + d0) =
            (f32x4_t){o[nb][db][4 * j], o[nb][db][4 * j + 1], o[nb][db][4 * j + 2], o[nb][db][4 * j + 3]};
      }
  }
}

// One workgroup per (row, head): merge the chunks.  Wave 0 finds the max M
// of the chunks' running maxima and the merged sum L; then every thread
// takes 4 consecutive dims of a strided subset of the chunks, and the
// partial sums meet in LDS (fixed order: the result does not depend on
// timing).
template <typename OutT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeArgs a) {
  constexpr int DG = D / 4;            // 4-dim groups per row
  constexpr int CL = 256 / DG;         // chunk lanes: threads per dim group
  __shared__ float s_ml[2];
  __shared__ __attribute__((aligned(16))) float s_part[CL][D];
  const int tid = threadIdx.x;
  const int64_t pairs = a.total_q * a.hq;
  const int64_t pair = blockIdx.x;
  const int64_t t = pair / a.hq;
  const int h = (int)(pair % a.hq);
  if (tid < 64) {
    float m = kNegInf;
    for (int c = tid; c < a.n_chunks; c += 64) m = __builtin_fmaxf(m, a.ws_ml[2 * ((int64_t)c * pairs + pair)]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
    float l = 0.0f;
    if (m != kNegInf) {
      for (int c = tid; c < a.n_chunks; c += 64) {
        const int64_t w = (int64_t)c * pairs + pair;
        const float mc = a.ws_ml[2 * w];
        if (mc != kNegInf) l += a.ws_ml[2 * w + 1] * fast_exp2(mc - m);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (tid == 0) {
      s_ml[0] = m;
      s_ml[1] = l;
    }
  }
  __syncthreads();
  const float M = s_ml[0], L = s_ml[1];
  const int dg = tid % DG, cl = tid / DG;
  const int d0 = 4 * dg;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (M != kNegInf) {
    for (int c = cl; c < a.n_chunks; c += CL) {
      const int64_t w = (int64_t)c * pairs + pair;
      const float m = a.ws_ml[2 * w];
      if (m == kNegInf) continue;
      const float f = fast_exp2(m - M);
      const f32x4_t ov = *reinterpret_cast<const f32x4_t*>(a.ws_o + w * D + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += ov[e] * f;
    }
  }
  *reinterpret_cast<f32x4_t*>(&s_part[cl][d0]) = (f32x4_t){acc[0], acc[1], acc[2], acc[3]};
  __syncthreads();
  if (cl == 0) {
#pragma unroll
    for (int j = 1; j < CL; ++j) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&s_part[j][d0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    OutT* op = reinterpret_cast<OutT*>(a.out) + t * a.o_st + (int64_t)h * a.o_sh + d0;
    store4<OutT>(op, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    if (d0 == 0 && a.lse != nullptr)
      a.lse[(int64_t)h * a.total_q + t] = L > 0.0f ? (M + fast_log2(L)) * kLn2 : kNegInf;
  }
}

template <typename T, int D>
hipError_t launch_decode_dims(const DecodeArgs& a, bool out_f32, int nb, unsigned units,
                              hipStream_t stream) {
  const dim3 grid(units, (unsigned)a.n_chunks);
  if (nb == 1)
    hipLaunchKernelGGL((decode_kernel<T, D, 1>), grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, 2>), grid, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid((unsigned)(a.total_q * a.hq));  // one workgroup per (row, head)
  if (out_f32)
    hipLaunchKernelGGL((decode_merge_kernel<float, D>), mgrid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), mgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_decode(const DecodeArgs& a, int in_dtype, bool out_f32, int d, int nb,
                              hipStream_t stream) {
  (void)hipGetLastError();
  const unsigned units = (unsigned)(a.num_seqs * a.hkv);
  if (in_dtype == kBF16 && d == 64) return launch_decode_dims<__bf16, 64>(a, out_f32, nb, units, stream);
  if (in_dtype == kBF16 && d == 128) return launch_decode_dims<__bf16, 128>(a, out_f32, nb, units, stream);
  if (in_dtype == kF16 && d == 64) return launch_decode_dims<_Float16, 64>(a, out_f32, nb, units, stream);
  if (in_dtype == kF16 && d == 128) return launch_decode_dims<_Float16, 128>(a, out_f32, nb, units, stream);
  return hipErrorInvalidValue;
}

}  // namespace mi_attn
