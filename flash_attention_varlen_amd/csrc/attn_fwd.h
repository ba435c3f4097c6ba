// Internal interface between the C-ABI front end (mi_attn.cpp) and the
// gfx950 kernels (attn_fwd.hip).  Not installed; see include/mi_attn.h for
// the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

constexpr int kThreads = 256;  // 4 wave64s per workgroup
constexpr int kBM = 128;       // query rows per workgroup of the fp32 kernel (32 per wave)

// Element type codes (same values as the public MI_ATTN_F32 / F16 / BF16).
constexpr int kF32 = 0;
constexpr int kF16 = 1;
constexpr int kBF16 = 2;

// Kernel arguments, passed by value.  Strides are in elements.
struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  // optional [num_seqs]: sequence s uses the first seqused[s] rows of its span
  const int32_t* seqused_q;
  const int32_t* seqused_kv;
  const float* bias;
  const int32_t* bias_ranges;  // optional [bias_heads, total_q, 2] key ranges of the bias rows
  const void* q_rope;  // optional: last 64 dims of the 192-wide q / k (q, k then hold 128)
  const void* k_rope;
  const float* alibi;  // optional ALiBi slopes, alibi[seq * alibi_ss + head]
  const uint8_t* mask;  // optional byte mask [total_q, bias_heads, bias_cols] (strides b_st, b_sh)
  // optional [bias_heads, total_q]: 1 where the row's bias is exactly 0 on
  // its whole key range (bias_ranges) and -inf elsewhere
  const uint8_t* bias_pure;
  int32_t* tile_counts;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  int64_t b_st, b_sh;
  int64_t qr_st, qr_sh, kr_st, kr_sh;  // q_rope / k_rope strides
  int64_t alibi_ss;
  int64_t total_q;
  int32_t num_seqs;
  int32_t hq;
  int32_t group;  // hq / hkv
  int32_t bias_heads;
  int32_t bias_cols;   // bias columns; keys at or past it read a bias of 0 (never out of bounds)
  int32_t causal;
  int32_t window;
  float scale_log2;    // softmax scale * log2(e)
  float split_l;       // 16-bit kernels: low half of P multiplied in while a row's sum is below this
  int32_t n_qtiles;    // query tiles of the longest sequence (grid.y unless head_major)
  int32_t head_major;  // 16-bit kernels: 1-D grid, all heads of a (sequence, tile) on one XCD
  int32_t kv_rows;     // 16-bit kernels: > 0 = 1-D grid, this many rows of one head run together
};

// Keys per tile for an input type and head dims.
int tile_bn(int in_dtype, int dqk, int dv);

// Query rows per workgroup for an input type and head dims.
int tile_bm(int in_dtype, int dqk, int dv);

// The kernel instances, one per (element type, head dims) pair.  Each is
// compiled in its own translation unit (attn_fwd_inst.hip, built once per
// pair) and launches the template for (bias, out type) on `stream`.
#define MI_ATTN_FWD_INSTANCES(X)                                                        \
  X(bf16, __bf16, 64, 64) X(bf16, __bf16, 128, 128) X(bf16, __bf16, 192, 128)           \
  X(bf16, __bf16, 96, 96) X(bf16, __bf16, 256, 256)                                     \
  X(f16, _Float16, 64, 64) X(f16, _Float16, 128, 128) X(f16, _Float16, 192, 128)        \
  X(f16, _Float16, 96, 96) X(f16, _Float16, 256, 256)                                   \
  X(f32, float, 64, 64) X(f32, float, 128, 128)
#define MI_ATTN_FWD_INSTANCE_NAME(tag, dqk, dv) launch_fwd_##tag##_##dqk##_##dv
#define MI_ATTN_FWD_DECLARE(tag, T, dqk, dv)                                            \
  hipError_t MI_ATTN_FWD_INSTANCE_NAME(tag, dqk, dv)(const KernelArgs& a, bool bias,   \
                                                     bool out_f32, dim3 grid, hipStream_t s);
MI_ATTN_FWD_INSTANCES(MI_ATTN_FWD_DECLARE)

// Launch on `stream`; grid = (hq * num_seqs, n_qtiles), or with head_major
// (hq * (num_seqs * n_qtiles rounded up to a multiple of 8), 1), or with
// kv_rows = R (hq * num_seqs * (n_qtiles rounded up to a multiple of R), 1).
hipError_t launch_attn_fwd(const KernelArgs& a, int in_dtype, int out_dtype, int dqk, int dv,
                           bool bias, dim3 grid, hipStream_t stream);

}  // namespace mi_attn
