// Host-side dispatch of the backward kernels to the compiled instance for
// (element type, head dim).
#include "attn_bwd.h"

namespace mi_attn {

constexpr int kBwdF16 = 1, kBwdBF16 = 2;  // MI_ATTN_F16 / MI_ATTN_BF16

hipError_t launch_attn_bwd(const BwdArgs& a, int in_dtype, bool grad_f32, bool bias, int d,
                           int max_seqlen_q, int max_seqlen_kv, hipStream_t stream) {
  (void)hipGetLastError();  // clear a stale error so the checks are about these launches
  constexpr int kTag_bf16 = kBwdBF16, kTag_f16 = kBwdF16;
#define MI_ATTN_BWD_DISPATCH(t, T, D)                                                          \
  if (in_dtype == kTag_##t && d == D)                                                          \
    return MI_ATTN_BWD_INSTANCE_NAME(t, D)(a, grad_f32, bias, max_seqlen_q, max_seqlen_kv, stream);
  MI_ATTN_BWD_INSTANCES(MI_ATTN_BWD_DISPATCH)
#undef MI_ATTN_BWD_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace mi_attn
