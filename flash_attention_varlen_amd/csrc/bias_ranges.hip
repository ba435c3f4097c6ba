// Key ranges of additive-bias rows: for every query row and bias head, the
// first and one-past-last key of its sequence whose bias is not -inf.  Keys
// whose bias is -inf contribute exactly nothing to the softmax (mtlattn 0.3.0
// project page, section "Use": the bias composes with the masks; the
// triton-msl part-2 post, section "FlashAttention: faster than PyTorch,
// competitive with MLX": skipping fully masked tiles is exact), so the
// forward kernels skip the key tiles outside a workgroup's hull of these
// ranges.  One wave per row; the row is read once with 16-byte loads, so the
// pass is bound by HBM bandwidth (4 bytes per bias element).  Optionally it
// also marks the rows that are plain key intervals: bias exactly 0 on every
// key of [lo, hi) (and -inf on the others, by the definition of the range),
// i.e. the number of zero values equals hi - lo.  The forward kernels mask
// such rows to their interval instead of reading their bias.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bias_ranges.h"

namespace mi_attn {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__global__ __launch_bounds__(256) void bias_key_ranges_kernel(const BiasRangeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seq = blockIdx.y;
  const int hb = blockIdx.z;
  const int r = blockIdx.x * 4 + wave;  // local row of the sequence
  const int cq0 = a.cu_q[seq];
  const int lq = a.cu_q[seq + 1] - cq0;
  if (r >= lq) return;
  const int lk = min(a.cu_kv[seq + 1] - a.cu_kv[seq], a.bias_cols);
  const float* row = a.bias + (int64_t)(cq0 + r) * a.b_st + (int64_t)hb * a.b_sh;
  int lo = 0x7fffffff, hi = 0, zeros = 0;
  // full 16-byte chunks: 64 lanes x 4 keys per pass, four passes in flight
  const int full = lk & ~3;
  for (int j0 = 4 * lane; j0 < full; j0 += 4 * 64 * 4) {
    f32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * 256;
      v[u] = j < full ? *reinterpret_cast<const f32x4_t*>(row + j)
                      : (f32x4_t){-__builtin_inff(), -__builtin_inff(), -__builtin_inff(),
                                  -__builtin_inff()};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (v[u][e] != -__builtin_inff()) {
          const int j = j0 + u * 256 + e;
          lo = min(lo, j);
          hi = max(hi, j + 1);
        }
        zeros += v[u][e] == 0.0f;
      }
  }
  // the last lk % 4 keys
  if (lane < lk - full) {
    const float x = row[full + lane];
    if (x != -__builtin_inff()) {
      lo = min(lo, full + lane);
      hi = max(hi, full + lane + 1);
    }
    zeros += x == 0.0f;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
    zeros += __shfl_xor(zeros, o);
  }
  if (lane == 0) {
    const int64_t i = (int64_t)hb * a.total_q + cq0 + r;
    a.ranges[2 * i] = hi > 0 ? lo : 0;
    a.ranges[2 * i + 1] = hi;
    if (a.pure != nullptr) a.pure[i] = zeros == (hi > 0 ? hi - lo : 0) ? 1 : 0;
  }
}

// The same for a byte mask: the first and one-past-last key whose mask
// byte is nonzero; 4 keys per lane and 32-bit load.
__global__ __launch_bounds__(256) void mask_key_ranges_kernel(const BiasRangeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seq = blockIdx.y;
  const int hb = blockIdx.z;
  const int r = blockIdx.x * 4 + wave;
  const int cq0 = a.cu_q[seq];
  const int lq = a.cu_q[seq + 1] - cq0;
  if (r >= lq) return;
  const int lk = min(a.cu_kv[seq + 1] - a.cu_kv[seq], a.bias_cols);
  const uint8_t* row = a.mask + (int64_t)(cq0 + r) * a.b_st + (int64_t)hb * a.b_sh;
  int lo = 0x7fffffff, hi = 0, vis = 0;  // vis: visible keys (the zeros of the bias)
  const int full = lk & ~3;
  for (int j0 = 4 * lane; j0 < full; j0 += 4 * 64) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(row + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((w >> (8 * e)) & 0xffu) {
        lo = min(lo, j0 + e);
        hi = max(hi, j0 + e + 1);
        ++vis;
      }
  }
  if (lane < lk - full && row[full + lane] != 0) {
    lo = min(lo, full + lane);
    hi = max(hi, full + lane + 1);
    ++vis;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
    vis += __shfl_xor(vis, o);
  }
  if (lane == 0) {
    const int64_t i = (int64_t)hb * a.total_q + cq0 + r;
    a.ranges[2 * i] = hi > 0 ? lo : 0;
    a.ranges[2 * i + 1] = hi;
    if (a.pure != nullptr) a.pure[i] = vis == (hi > 0 ? hi - lo : 0) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_bias_key_ranges(const BiasRangeArgs& a, int max_seqlen_q, int num_seqs,
                                  int bias_heads, hipStream_t stream) {
  (void)hipGetLastError();
  const dim3 grid((unsigned)((max_seqlen_q + 3) / 4), (unsigned)num_seqs, (unsigned)bias_heads);
  if (a.mask != nullptr)
    hipLaunchKernelGGL(mask_key_ranges_kernel, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bias_key_ranges_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mi_attn
