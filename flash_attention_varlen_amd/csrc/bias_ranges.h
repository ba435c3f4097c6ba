// Internal interface of the bias key-range pass (bias_ranges.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

struct BiasRangeArgs {
  const float* bias;     // fp32 bias, or
  const uint8_t* mask;   // a byte mask (nonzero = visible), b_st / b_sh in bytes
  const int32_t* cu_q;
  const int32_t* cu_kv;
  int32_t* ranges;  // [bias_heads, total_q, 2]
  uint8_t* pure;    // optional [bias_heads, total_q]: 1 when the row is a key interval
  int64_t b_st, b_sh;
  int64_t total_q;
  int32_t bias_cols;
};

// grid (ceil(max_seqlen_q / 4), num_seqs, bias_heads), one wave per row
hipError_t launch_bias_key_ranges(const BiasRangeArgs& a, int max_seqlen_q, int num_seqs,
                                  int bias_heads, hipStream_t stream);

}  // namespace mi_attn
