// Host-side dispatch of the forward kernels: tile shapes and the choice of
// the compiled instance for (element type, head dims).  The kernels
// themselves are in attn_fwd_kernels.h, instantiated by attn_fwd_inst.hip.
#include "attn_fwd_kernels.h"

namespace mi_attn {

int tile_bn(int in_dtype, int dqk, int dv) {
  if (in_dtype == kF32) return Geo<float, 64, 64>::BN;
  if (dqk == 64 && dv == 64) return WaveBlocks<64, 64>::kReportBN;
  if (dqk == 128 && dv == 128) return WaveBlocks<128, 128>::kReportBN;
  if (dqk == 256 && dv == 256) return WaveBlocks<256, 256>::kReportBN;
  if (dqk == 96 && dv == 96) return WaveBlocks<96, 96>::kReportBN;
  return WaveBlocks<192, 128>::kReportBN;
}

int tile_bm(int in_dtype, int dqk, int dv) {
  if (in_dtype == kF32) return kBM;
  if (dqk == 64 && dv == 64) return 4 * 32 * WaveBlocks<64, 64>::NB;
  if (dqk == 128 && dv == 128) return 4 * 32 * WaveBlocks<128, 128>::NB;
  if (dqk == 256 && dv == 256) return 4 * 32 * WaveBlocks<256, 256>::NB;
  if (dqk == 96 && dv == 96) return 4 * 32 * WaveBlocks<96, 96>::NB;
  return 4 * 32 * WaveBlocks<192, 128>::NB;
}

hipError_t launch_attn_fwd(const KernelArgs& a, int in_dtype, int out_dtype, int dqk, int dv,
                           bool bias, dim3 grid, hipStream_t stream) {
  (void)hipGetLastError();  // clear a stale error so the check below is about this launch
  const bool out_f32 = out_dtype == kF32;
  constexpr int kTag_bf16 = kBF16, kTag_f16 = kF16, kTag_f32 = kF32;
#define MI_ATTN_FWD_DISPATCH(t, T, DQK, DV)                                                  \
  if (in_dtype == kTag_##t && dqk == DQK && dv == DV)                                        \
    return MI_ATTN_FWD_INSTANCE_NAME(t, DQK, DV)(a, bias, out_f32 || in_dtype == kF32, grid, stream);
  MI_ATTN_FWD_INSTANCES(MI_ATTN_FWD_DISPATCH)
#undef MI_ATTN_FWD_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace mi_attn
