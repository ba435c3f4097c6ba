// One instantiation unit of the backward kernels, compiled once per
// (element type, head dim) pair listed in MI_ATTN_BWD_INSTANCES, selected by
// -DMI_ATTN_INST_TAG / _T / _D.
#include "attn_bwd_kernels.h"

#if !defined(MI_ATTN_INST_TAG) || !defined(MI_ATTN_INST_T) || !defined(MI_ATTN_INST_D)
#error "compile with -DMI_ATTN_INST_TAG=<bf16|f16> -DMI_ATTN_INST_T=<type> -DMI_ATTN_INST_D=<64|128>"
#endif

#define MI_ATTN_EXPAND_BWD_NAME(tag, d) MI_ATTN_BWD_INSTANCE_NAME(tag, d)

namespace mi_attn {

hipError_t MI_ATTN_EXPAND_BWD_NAME(MI_ATTN_INST_TAG, MI_ATTN_INST_D)(const BwdArgs& a, bool grad_f32,
                                                                    bool bias, int max_seqlen_q,
                                                                    int max_seqlen_kv, hipStream_t s) {
  return launch_bwd_dims<MI_ATTN_INST_T, MI_ATTN_INST_D>(a, grad_f32, bias, max_seqlen_q, max_seqlen_kv,
                                                         s);
}

}  // namespace mi_attn
