// Key-padding front end: a padded batch [batch, seqlen] with a mask of its
// valid tokens becomes the packed varlen layout the forward takes, and back.
// The mtlattn 0.3.0 project page (section "Drop-in for
// scaled_dot_product_attention") converts a self-attention key-padding mask
// to varlen this way: the valid tokens are packed and the padding is never
// computed.  Packing keeps the order of a row's valid tokens, so causal
// visibility between valid tokens is the same in both layouts.
//
// Three kernels, all bound by HBM bandwidth: ranks (one workgroup per batch
// row: ballot prefix counts over 256-token chunks), a one-workgroup scan of
// the row counts into cu_seqlens, and a 16-byte-per-lane gather / scatter.
// A right-padded batch (every row's valid tokens first) needs no packing at
// all: two more kernels find each row's count and whether the batch is
// right-padded, for the forward's seqused form.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "padding.h"

namespace mi_attn {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// Rank of every token among its row's valid tokens (-1 for padding); the
// row's count goes to cu[b + 1] for the scan below.
__global__ __launch_bounds__(256) void padding_ranks_kernel(const PadRankArgs a) {
  __shared__ int wave_count[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;
  const uint8_t* m = a.mask + (int64_t)b * a.mask_st;
  int32_t* rk = a.ranks + (int64_t)b * a.seqlen;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes < this one
  int run = 0;
  for (int n0 = 0; n0 < a.seqlen; n0 += 256) {
    const int n = n0 + tid;
    const bool valid = n < a.seqlen && m[n] != 0;
    const uint64_t bal = __ballot(valid);
    if (lane == 0) wave_count[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += w < wave ? wave_count[w] : 0;
      total += wave_count[w];
    }
    if (n < a.seqlen) rk[n] = valid ? run + before + __popcll(bal & below) : -1;
    run += total;
    __syncthreads();  // wave_count is rewritten by the next chunk
  }
  if (tid == 0) a.cu[b + 1] = run;
}

// cu[0] = 0 and the inclusive scan of the counts in cu[1..batch], in place;
// stats = (total, longest row).  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void padding_scan_kernel(const PadRankArgs a) {
  __shared__ int wave_sum[16];
  __shared__ int wave_max[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0, longest = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 1024) {
    const int b = b0 + tid;
    const int c = b < a.batch ? a.cu[b + 1] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int mx = c;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
    if (lane == 63) wave_sum[wave] = incl;
    if (lane == 0) wave_max[wave] = mx;
    __syncthreads();
    int before = 0, total = 0, cmax = 0;
    for (int w = 0; w < 16; ++w) {
      before += w < wave ? wave_sum[w] : 0;
      total += wave_sum[w];
      cmax = max(cmax, wave_max[w]);
    }
    if (b < a.batch) a.cu[b + 1] = carry + before + incl;
    carry += total;
    longest = max(longest, cmax);
    __syncthreads();
  }
  if (tid == 0) {
    a.cu[0] = 0;
    if (a.stats) {
      a.stats[0] = carry;
      a.stats[1] = longest;
    }
  }
}

// Row b's valid-token count and whether its valid tokens are its first ones
// (the last valid position + 1 equals the count); the flag goes to
// spans[b + 1] until padding_lengths_stats_kernel overwrites it.
__global__ __launch_bounds__(256) void padding_lengths_kernel(const PadLengthArgs a) {
  __shared__ int wave_count[4];
  __shared__ int wave_end[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;
  const uint8_t* m = a.mask + (int64_t)b * a.mask_st;
  int count = 0, end = 0;  // this thread's share: valid tokens, last valid position + 1
  for (int n = tid; n < a.seqlen; n += 256)
    if (m[n] != 0) {
      ++count;
      end = n + 1;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    count += __shfl_xor(count, o);
    end = max(end, __shfl_xor(end, o));
  }
  if (lane == 0) {
    wave_count[wave] = count;
    wave_end[wave] = end;
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0, e = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      c += wave_count[w];
      e = max(e, wave_end[w]);
    }
    a.lengths[b] = c;
    a.spans[b + 1] = e == c ? 1 : 0;
  }
}

// stats = (every row right-padded, longest row); spans[b] = b * seqlen.  One
// workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void padding_lengths_stats_kernel(const PadLengthArgs a) {
  __shared__ int wave_all[16];
  __shared__ int wave_max[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int all = 1, longest = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 1024) {
    const int b = b0 + tid;
    int ok = 1, len = 0;
    if (b < a.batch) {
      ok = a.spans[b + 1];
      len = a.lengths[b];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      ok = min(ok, __shfl_xor(ok, o));
      len = max(len, __shfl_xor(len, o));
    }
    if (lane == 0) {
      wave_all[wave] = ok;
      wave_max[wave] = len;
    }
    __syncthreads();
    for (int w = 0; w < 16; ++w) {
      all = min(all, wave_all[w]);
      longest = max(longest, wave_max[w]);
    }
    __syncthreads();  // the flags are read before they are overwritten, and the
                      // shared slots before the next round rewrites them
    if (b < a.batch) a.spans[b + 1] = (b + 1) * a.seqlen;
  }
  if (tid == 0) {
    a.spans[0] = 0;
    if (a.stats) {
      a.stats[0] = all;
      a.stats[1] = longest;
    }
  }
}

// One 16-byte chunk per lane: a workgroup takes tok_per_wg tokens (or one
// token whose chunks it loops over).
__global__ __launch_bounds__(256) void pack_tokens_kernel(const PackArgs a) {
  const int tid = threadIdx.x;
  const int lt = tid / a.chunks;  // token of this lane within the workgroup
  if (lt >= a.tok_per_wg) return;
  const int tok = blockIdx.x * a.tok_per_wg + lt;
  if (tok >= a.tokens) return;
  const int b = tok / a.seqlen;
  const int n = tok - b * a.seqlen;
  const int rank = a.ranks ? a.ranks[tok] : n;
  const int row = rank < 0 ? -1 : (a.ranks ? a.cu[b] + rank : tok);
  const int step = a.tok_per_wg > 1 ? a.chunks : 256;  // one token per workgroup: loop
  for (int c = tid - lt * a.chunks; c < a.chunks; c += step) {
    const int h = c / a.row_chunks;
    const int w = c - h * a.row_chunks;
    u32x4_t* pd = reinterpret_cast<u32x4_t*>(a.padded + b * a.pd_sb + n * a.pd_st + h * a.pd_sh +
                                             w * 16);
    if (row < 0) {
      if (a.unpack) *pd = (u32x4_t){0u, 0u, 0u, 0u};
      continue;
    }
    u32x4_t* pk = reinterpret_cast<u32x4_t*>(a.packed + row * a.pk_st + h * a.pk_sh + w * 16);
    if (a.unpack)
      *pd = *pk;
    else
      *pk = *pd;
  }
}

}  // namespace

hipError_t launch_padding_ranks(const PadRankArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.batch > 0) hipLaunchKernelGGL(padding_ranks_kernel, dim3((unsigned)a.batch), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(padding_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_padding_lengths(const PadLengthArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.batch > 0)
    hipLaunchKernelGGL(padding_lengths_kernel, dim3((unsigned)a.batch), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(padding_lengths_stats_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_pack_tokens(const PackArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  const unsigned wgs = (unsigned)((a.tokens + a.tok_per_wg - 1) / a.tok_per_wg);
  if (wgs > 0) hipLaunchKernelGGL(pack_tokens_kernel, dim3(wgs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mi_attn
