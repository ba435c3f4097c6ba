// One instantiation unit of the forward kernels.  The build compiles this file
// once per (element type, head dims) pair listed in MI_ATTN_FWD_INSTANCES,
// selected by -DMI_ATTN_INST_TAG / _T / _DQK / _DV, so that the instances
// compile in parallel.
#include "attn_fwd_kernels.h"

#if !defined(MI_ATTN_INST_TAG) || !defined(MI_ATTN_INST_T) || !defined(MI_ATTN_INST_DQK) || \
    !defined(MI_ATTN_INST_DV)
#error "compile with -DMI_ATTN_INST_TAG=<bf16|f16|f32> -DMI_ATTN_INST_T=<type> -DMI_ATTN_INST_DQK=<n> -DMI_ATTN_INST_DV=<n>"
#endif

#define MI_ATTN_EXPAND_NAME(tag, dqk, dv) MI_ATTN_FWD_INSTANCE_NAME(tag, dqk, dv)

namespace mi_attn {

hipError_t MI_ATTN_EXPAND_NAME(MI_ATTN_INST_TAG, MI_ATTN_INST_DQK, MI_ATTN_INST_DV)(
    const KernelArgs& a, bool bias, bool out_f32, dim3 grid, hipStream_t s) {
  return launch_dims<MI_ATTN_INST_T, MI_ATTN_INST_DQK, MI_ATTN_INST_DV>(a, bias, out_f32, grid, s);
}

}  // namespace mi_attn
