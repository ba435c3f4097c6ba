// Internal interface of the key-padding front end (padding.hip): ranks of
// the valid tokens of a padded batch, their cumulative counts, and the
// gather / scatter between the padded and the packed token layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

struct PadRankArgs {
  const uint8_t* mask;  // [batch, seqlen] bytes, nonzero = valid token
  int64_t mask_st;      // bytes between batch rows
  int32_t* ranks;       // [batch * seqlen]: rank among the row's valid tokens, -1 = padding
  int32_t* cu;          // [batch + 1] cumulative counts
  int32_t* stats;       // optional [2]: total valid tokens, longest row
  int32_t batch;
  int32_t seqlen;
};

struct PackArgs {
  char* padded;          // [batch, seqlen, heads, row bytes]
  char* packed;          // [total, heads, row bytes]
  const int32_t* ranks;  // NULL: every token valid, packed row = token index
  const int32_t* cu;
  int64_t pd_sb, pd_st, pd_sh;  // padded strides, bytes
  int64_t pk_st, pk_sh;         // packed strides, bytes
  int32_t seqlen;
  int32_t tokens;     // batch * seqlen
  int32_t chunks;     // 16-byte chunks per token (heads * row bytes / 16)
  int32_t row_chunks; // 16-byte chunks per head row
  int32_t tok_per_wg; // tokens one workgroup copies (256 / chunks, at least 1)
  int32_t unpack;     // 0: padded -> packed; 1: packed -> padded, zeros at padding
};

// Right-padding check: every row's valid-token count, whether each row's
// valid tokens are its first ones, and the spans of the padded rows.
struct PadLengthArgs {
  const uint8_t* mask;  // [batch, seqlen] bytes, nonzero = valid token
  int64_t mask_st;      // bytes between batch rows
  int32_t* lengths;     // [batch]: valid tokens of each row
  int32_t* spans;       // [batch + 1]: b * seqlen (first a per-row flag, see the kernels)
  int32_t* stats;       // optional [2]: all rows right-padded (1 / 0), longest row
  int32_t batch;
  int32_t seqlen;
};

hipError_t launch_padding_ranks(const PadRankArgs& a, hipStream_t stream);
hipError_t launch_padding_lengths(const PadLengthArgs& a, hipStream_t stream);
hipError_t launch_pack_tokens(const PackArgs& a, hipStream_t stream);

}  // namespace mi_attn
