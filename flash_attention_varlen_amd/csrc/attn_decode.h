// Internal interface between the C-ABI front end (mi_attn.cpp) and the
// split-KV decode kernels (attn_decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* seqused_kv;  // optional [num_seqs]: keys used of each sequence's span
  float* ws_o;   // [n_chunks, total_q, hq, d_v] unnormalised partial outputs
  float* ws_ml;  // [n_chunks, total_q, hq, 2] running max (log2 units) and sum
  void* out;
  float* lse;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  int64_t total_q;
  int32_t num_seqs, hq, hkv, group;
  int32_t causal, window;
  int32_t chunk_tiles;  // 32-key tiles per chunk
  int32_t n_chunks;
  float scale_log2;
  float split_l;  // low half of P multiplied in while a row's sum is below this (times its largest p)
};

// Partial kernel (grid (num_seqs * hkv, n_chunks), one wave per workgroup,
// nb = 32-row blocks of packed rows) then the merge, on `stream`.
hipError_t launch_attn_decode(const DecodeArgs& a, int in_dtype, bool out_f32, int d, int nb,
                              hipStream_t stream);

}  // namespace mi_attn
