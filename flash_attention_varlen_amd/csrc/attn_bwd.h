// Internal interface between the C-ABI front end (mi_attn.cpp) and the
// backward kernels (attn_bwd_kernels.h).  Not installed; the public
// interface is include/mi_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

// Backward kernel arguments, passed by value.  Strides are in elements.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [hq, total_q] workspace: rowsum(dout * out)
  const int32_t* cu_q;
  const int32_t* cu_kv;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh, do_st, do_sh;
  int64_t dq_st, dq_sh, dk_st, dk_sh, dv_st, dv_sh;
  int64_t total_q;
  int32_t num_seqs;
  int32_t hq, hkv;
  int32_t group;  // hq / hkv
  int32_t causal;
  int32_t window;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  // optional constant additive bias [total_q, bias_heads, bias_cols] (fp32)
  const float* bias;
  int64_t b_st, b_sh;
  int32_t bias_heads;  // 1 or hq
  int32_t bias_cols;   // keys at or past it read a bias of 0
  // optional ALiBi slopes alibi[seq * alibi_ss + head] (no bias tensor then)
  const float* alibi;
  int64_t alibi_ss;
};

// The backward instances, one per (element type, head dim), compiled in
// their own translation units (attn_bwd_inst.hip).
#define MI_ATTN_BWD_INSTANCES(X)                                                     \
  X(bf16, __bf16, 64) X(bf16, __bf16, 96) X(bf16, __bf16, 128) X(f16, _Float16, 64) \
  X(f16, _Float16, 96) X(f16, _Float16, 128)
#define MI_ATTN_BWD_INSTANCE_NAME(tag, d) launch_bwd_##tag##_##d
#define MI_ATTN_BWD_DECLARE(tag, T, d)                                                         \
  hipError_t MI_ATTN_BWD_INSTANCE_NAME(tag, d)(const BwdArgs& a, bool grad_f32, bool bias,     \
                                               int max_seqlen_q, int max_seqlen_kv, hipStream_t s);
MI_ATTN_BWD_INSTANCES(MI_ATTN_BWD_DECLARE)

// delta, then dK/dV, then dQ, all on `stream`; grad_f32: fp32 gradients.
hipError_t launch_attn_bwd(const BwdArgs& a, int in_dtype, bool grad_f32, bool bias, int d,
                           int max_seqlen_q, int max_seqlen_kv, hipStream_t stream);

}  // namespace mi_attn
