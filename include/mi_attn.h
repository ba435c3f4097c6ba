/*
 * mi_attn — fused variable-length attention for AMD MI355X (gfx950): the
 * forward, a split-KV decode form of it, its backward, the bias key-range
 * pass (tile skipping and interval rows) and the key-padding front end
 * (padded batch <-> packed varlen).
 *
 * C ABI.  No HIP or PyTorch types appear in the signatures: device buffers
 * are plain pointers, sizes and strides are integers, the stream is an
 * opaque pointer (a hipStream_t, NULL for the default stream).
 *
 * The operation (mtlattn 0.3.0 project page, section "Use"):
 *   packed ragged q [total_q, hq, d_qk], k [total_kv, hkv, d_qk],
 *   v [total_kv, hkv, d_v]; sequence s owns q rows cu_seqlens_q[s] ..
 *   cu_seqlens_q[s+1]-1 and kv rows cu_seqlens_kv[s] .. cu_seqlens_kv[s+1]-1;
 *   query head h reads kv head h / (hq / hkv) (GQA / MQA);
 *   logit(i, j) = scale * (q_i . k_j) + bias[global row of i][h or 0][j];
 *   causal: local query i sees local key j iff j <= i + (Lk - Lq)
 *   (end-aligned, so self-attention and cached decode both hold);
 *   window W > 0 (with causal): additionally j > i + (Lk - Lq) - W, i.e. the
 *   last W keys up to that diagonal;
 *   out_i = sum_j softmax_j(logit(i, .)) v_j over the visible keys whose
 *   logit is not -inf, and lse_i = ln sum_j exp(logit(i, j)) (natural log).
 *   A row with no such key gets out = 0 and lse = -inf.
 * The softmax is streamed over key tiles with fp32 running max and sum
 * (triton-msl part-1 post, section "What works, and where the edges are";
 * mtlattn page, section "Notes": fp32 accumulation for every input dtype);
 * no Lq x Lk matrix is ever stored.
 *
 * Supported set (anything else is refused, nothing is launched):
 *   (d_qk, d_v) in {(64,64), (96,96), (128,128), (192,128), (256,256)};
 *   bf16 / fp16 inputs for all five (the mtlattn page, section "Drop-in for
 *   scaled_dot_product_attention", lists head dims 64, 96, 128 and 256 for
 *   its fast path), fp32 inputs for (64,64) and (128,128);
 *   out dtype = input dtype or fp32; hq % hkv == 0; window > 0 needs causal.
 * The refusal follows the correct-or-refuse contract on the triton-msl
 * part-1 post (section "Correct-or-refuse"): an unsupported request returns
 * an error code and a reason, never a plausible wrong answer.
 */
#ifndef MI_ATTN_H
#define MI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_ATTN_VERSION 170 /* 1.7.0 */

/* Return codes.  On any error nothing is launched and out / lse are untouched. */
enum {
  MI_ATTN_OK = 0,
  MI_ATTN_ERR_INVALID_ARG = -1, /* malformed arguments (null pointer, bad size, misalignment) */
  MI_ATTN_ERR_UNSUPPORTED = -2, /* well-formed but outside the supported set */
  MI_ATTN_ERR_LAUNCH = -3,      /* the HIP runtime rejected the launch */
  MI_ATTN_ERR_VALIDATION = -4   /* MI_ATTN_VALIDATE=1 found a bad cu_seqlens / size contract */
};

/* Element types. */
enum { MI_ATTN_F32 = 0, MI_ATTN_F16 = 1, MI_ATTN_BF16 = 2 };

/*
 * Arguments of one forward call.  Set struct_size = sizeof(mi_attn_fwd_params)
 * so the struct can grow without breaking callers.
 *
 * Pointers (all device memory, owned by the caller; the library keeps none
 * of them after the call returns and allocates nothing):
 *   q, k, v      input tensors, element type in_dtype, last dim contiguous,
 *                16-byte aligned.
 *   out          [total_q, hq, d_v] output, element type out_dtype, last dim
 *                contiguous, 16-byte aligned.  Written for every row of every
 *                sequence.
 *   lse          [hq, total_q] fp32, row h contiguous (element h*total_q + t);
 *                may be NULL.
 *   cu_seqlens_q, cu_seqlens_kv   int32 [num_seqs + 1], cumulative lengths.
 *   bias         optional fp32 additive bias [total_q, bias_heads, bias_cols]
 *                addressed as bias[t*bias_stride_tok + hb*bias_stride_head + j]
 *                with t the global query row, hb = 0 if bias_heads == 1 else
 *                the query head, j the key position inside its sequence;
 *                16-byte aligned, strides multiples of 4.  Values must be
 *                finite or -inf.
 *   tile_counts  optional int32 [hq * num_seqs * n_qtiles] (debug): for every
 *                workgroup, the number of BN-key tiles spanned by the keys
 *                its loop visited, at index (qtile * num_seqs + seq) * hq +
 *                head, where n_qtiles = ceil(max_seqlen_q / BM) and BM, BN
 *                come from mi_attn_tile_shape.  NULL in normal use.
 *
 * Sizes: num_seqs >= 0, max_seqlen_q >= every sequence's query length,
 * total_q / total_kv = cu_seqlens_q[num_seqs] / cu_seqlens_kv[num_seqs],
 * bias_cols >= every sequence's key length (the kernels never read a bias
 * column at or past bias_cols: a key there would get a bias of 0).
 * Strides are in elements (not bytes); *_stride_tok between consecutive
 * tokens, *_stride_head between consecutive heads; each must be a multiple
 * of 8 elements for 16-bit types and of 4 for fp32.  q/k token strides must
 * be >= d_qk (>= 128 with q_rope / k_rope) and v's and out's >= d_v; for 16-bit types 64 q/k/v token
 * strides and 32 out token strides must fit in 2^31 bytes; the out strides
 * must keep the [total_q, hq, d_v] rows disjoint.  Anything else is refused
 * with MI_ATTN_ERR_UNSUPPORTED.
 *
 * The device-side contracts (cu_seqlens non-decreasing from 0 to total,
 * lengths within max_seqlen_q / bias_cols) are the caller's; with the
 * environment variable MI_ATTN_VALIDATE=1 the library copies both
 * cu_seqlens arrays to the host (synchronously) and refuses violations.
 */
typedef struct mi_attn_fwd_params {
  size_t struct_size;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_kv;
  const float* bias;
  int32_t* tile_counts;
  int64_t num_seqs;
  int64_t max_seqlen_q;
  int64_t total_q;
  int64_t total_kv;
  int32_t hq, hkv, d_qk, d_v;
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t out_stride_tok, out_stride_head;
  int32_t bias_heads; /* 1 or hq; ignored when bias is NULL */
  int64_t bias_cols;
  int64_t bias_stride_tok, bias_stride_head;
  int32_t in_dtype;  /* MI_ATTN_F32 / F16 / BF16 */
  int32_t out_dtype; /* in_dtype or MI_ATTN_F32 */
  float scale;       /* softmax scale, e.g. 1/sqrt(d_qk) */
  int32_t causal;    /* 0 or 1 */
  int32_t window;    /* 0 = none, else W >= 1 (requires causal) */
  /* Added in version 1.1 (callers built against 1.0 pass a smaller
   * struct_size and get NULL here):
   * optional int32 [bias_heads, total_q, 2] key ranges of the bias rows, as
   * mi_attn_bias_key_ranges writes them for this bias.  With them the kernels
   * skip, exactly, the key tiles in which every bias value of a workgroup's
   * (or a wave's) rows is -inf.  NULL: no skipping.  Ignored without a bias. */
  const int32_t* bias_ranges;
  /* Added in version 1.5 (NULL for older callers):
   * split operands of the latent-attention head (d_qk = 192, d_v = 128,
   * 16-bit inputs).  The triton-msl part-2 post (section "Latent attention,
   * the 2026 frontier") describes that head's score as the sum of two
   * query-key products: a 128-wide part without position encoding ("nope")
   * and a 64-wide rotary part ("rope").  With q_rope and k_rope
   * set, q and k hold only the nope part (their first 128 dims are read)
   * and q_rope / k_rope the rope part, [total_q, hq, 64] and
   * [total_kv, hkv, 64] addressed with the strides below (elements,
   * multiples of 8, token strides >= 64 and within 32 MiB); the result is
   * that of one call on the concatenation [nope | rope] of each.  Both set
   * or both NULL; 16-byte aligned.  Only mi_attn_varlen_fwd reads them
   * (the decode and backward entry points refuse them). */
  const void* q_rope;
  const void* k_rope;
  int64_t q_rope_stride_tok, q_rope_stride_head;
  int64_t k_rope_stride_tok, k_rope_stride_head;
  /* Added in version 1.5 (NULL for older callers): ALiBi computed in the
   * kernels instead of read from a bias tensor.  The mtlattn 0.3.0 page
   * (section "Use") lists ALiBi among the patterns its additive bias
   * expresses; the pages give no formula, and the one used here is the
   * usual linear distance penalty: the logit of query row i and key j of a
   * sequence gains -slope * |i + (Lk - Lq) - j| (distance from the query's
   * end-aligned position), slope = alibi_slopes[s * alibi_stride_seq + h]
   * for sequence s and query head h (alibi_stride_seq = 0: one slope per
   * head for every sequence).  fp32 device array, 4-byte aligned, finite
   * values.  Composes with causal / window / GQA; refused together with a
   * bias tensor. */
  const float* alibi_slopes;
  int64_t alibi_stride_seq;
  /* Added in version 1.5 (NULL for older callers): a boolean mask read by
   * the kernels in place of the fp32 bias, one byte per element (the
   * mtlattn 0.3.0 page, section "Use", turns a bool mask into the 0 / -inf
   * additive bias; reading the bytes moves a quarter of the fp32 bias's
   * bytes).  uint8 [total_q, bias_heads, bias_cols], nonzero = visible
   * (bias 0), 0 = masked (bias -inf), addressed with bias_heads, bias_cols,
   * bias_stride_tok and bias_stride_head exactly as the bias (strides in
   * bytes here, multiples of 4; 4-byte aligned).  Columns at or past
   * bias_cols count as visible, as a bias of 0 does.  bias_ranges (from
   * mi_attn_bias_key_ranges with this mask) apply as for a bias.  Not
   * together with bias or alibi_slopes; the decode entry points refuse it. */
  const uint8_t* mask;
  /* Added in version 1.6 (NULL for older callers): per bias head and query
   * row, one byte [bias_heads, total_q] (uint8, device, caller-owned):
   * nonzero when the row's bias (or mask) is exactly 0 (visible) on every
   * key of its range [lo, hi) from bias_ranges and -inf (masked) on every
   * other key, i.e. the row is a plain key interval.  Written by
   * mi_attn_bias_key_ranges when non-NULL; read by mi_attn_varlen_fwd, which
   * then needs bias_ranges from the same call: a wave of rows that are all
   * such intervals reads no bias and masks each row to its interval
   * instead, with results equal to those of the bias.  Like bias_ranges it
   * assumes bias_cols >= every sequence's key length. */
  const uint8_t* bias_pure;
  /* Added in version 1.7 (NULL for older callers): optional int32
   * [num_seqs] device arrays.  Sequence s then uses only the first
   * seqused_q[s] query rows of its span cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1
   * and the first seqused_kv[s] keys of its key span (values clamped to
   * [0, span]): Lq and Lk above are these counts, the causal diagonal is
   * end-aligned on them, and keys past seqused_kv are never read.  Unused
   * query rows of a span get out = 0 and lse = -inf, as rows that see no
   * key do (mi_attn_varlen_fwd).  This lets
   * a right-padded batch (spans of one padded length, the valid tokens
   * first) run without packing, and a decode call read a key cache that is
   * allocated longer than it is filled.  mi_attn_varlen_decode reads
   * seqused_kv and refuses seqused_q.  4-byte aligned. */
  const int32_t* seqused_q;
  const int32_t* seqused_kv;
} mi_attn_fwd_params;

/*
 * Enqueue the forward pass on `stream` (a hipStream_t; NULL = default
 * stream) and return without waiting: results are visible in stream order,
 * as the mtlattn page's section "Notes" describes for its own stream.
 * Returns MI_ATTN_OK or a negative code; mi_attn_last_error() then says why.
 * Re-entrant and thread-safe; the run is bitwise deterministic (fixed
 * reduction order, no atomics).
 */
int mi_attn_varlen_fwd(const mi_attn_fwd_params* p, void* stream);

/*
 * Key ranges of the bias (or mask) rows: for every bias head hb and query row t (global)
 * of sequence s, ranges[(hb * total_q + t) * 2 + 0 .. 1] = [lo, hi), the
 * first and one-past-last key j < min(Lk(s), bias_cols) whose bias value
 * p->bias[t][hb][j] is not -inf, or with p->mask set (and no bias) whose
 * mask byte is nonzero ([0, 0) when there is none).  Reads the
 * bias, cu_seqlens, sizes and strides of *p (the same struct a forward call
 * takes; q/k/v/out are not used) and writes ranges, an int32 device buffer
 * of 2 * bias_heads * total_q elements, 8-byte aligned, owned by the caller.
 * Keys with a -inf bias contribute nothing to the softmax, so skipping the
 * tiles outside these ranges is exact (mtlattn 0.3.0 project page, section
 * "Use", for the bias; triton-msl part-2 post, section "FlashAttention:
 * faster than PyTorch, competitive with MLX", for skipping masked tiles).
 * The ranges stay valid for as long as the bias and cu_seqlens do: compute
 * them once per bias, pass them in mi_attn_fwd_params.bias_ranges.  With
 * p->bias_pure non-NULL it also writes, per row, whether the row is a plain
 * key interval (bias exactly 0 on [lo, hi), -inf elsewhere; mask bytes
 * nonzero on [lo, hi), 0 elsewhere), for mi_attn_fwd_params.bias_pure.
 * Asynchronous on `stream`; one read of the bias.  Returns MI_ATTN_OK or a
 * negative code (nothing launched).
 */
int mi_attn_bias_key_ranges(const mi_attn_fwd_params* p, int32_t* ranges, void* stream);

/*
 * Key-padding front end (added in version 1.5).  The mtlattn 0.3.0 page
 * (section "Drop-in for scaled_dot_product_attention") turns a
 * self-attention key-padding mask into varlen form: the valid tokens are
 * packed and the padding is never computed.  Packing keeps the order of a
 * row's valid tokens, so causal visibility between valid tokens is the same
 * before and after.
 *
 * mi_attn_padding_to_varlen: mask is uint8 [batch, seqlen] (nonzero = valid
 * token; row b at mask + b * mask_stride_batch bytes, tokens contiguous).
 * Writes ranks, int32 [batch * seqlen]: the rank of token (b, n) among row
 * b's valid tokens, -1 for padding; cu_seqlens, int32 [batch + 1], the
 * cumulative valid counts (cu_seqlens[0] = 0); and, if stats is not NULL,
 * stats[0] = total valid tokens, stats[1] = the longest row (what a forward
 * call needs as total_q and max_seqlen_q; reading them on the host means a
 * synchronisation the caller chooses).  batch * seqlen must fit in int32.
 * All buffers are device memory owned by the caller; int32 outputs 4-byte
 * aligned.  Asynchronous on `stream`.
 */
int mi_attn_padding_to_varlen(const uint8_t* mask, int64_t batch, int64_t seqlen,
                              int64_t mask_stride_batch, int32_t* ranks, int32_t* cu_seqlens,
                              int32_t* stats, void* stream);

/*
 * Right-padding check (added in version 1.7): for the same mask, lengths
 * (int32 [batch]) gets each row's valid-token count, spans (int32
 * [batch + 1]) gets b * seqlen, and, if stats is not NULL, stats[0] = 1 when
 * every row's valid tokens are its first lengths[b] tokens (a right-padded
 * batch) and 0 otherwise, stats[1] = the longest row.  For a right-padded
 * batch a forward call can take the padded tensors as they are, with
 * cu_seqlens = spans and seqused_q / seqused_kv = lengths (mi_attn_fwd_params),
 * instead of packing them.  Same buffer and size rules as
 * mi_attn_padding_to_varlen; asynchronous on `stream`.
 */
int mi_attn_padding_lengths(const uint8_t* mask, int64_t batch, int64_t seqlen,
                            int64_t mask_stride_batch, int32_t* lengths, int32_t* spans,
                            int32_t* stats, void* stream);

/*
 * Gather (mi_attn_pack_tokens) the valid tokens of a padded view
 * [batch, seqlen, heads, dim] into packed rows [total, heads, dim], or
 * scatter (mi_attn_unpack_tokens) packed rows back into the padded view,
 * writing zeros at padding.  Valid token (b, n) is packed row
 * cu_seqlens[b] + ranks[b * seqlen + n] (arrays from
 * mi_attn_padding_to_varlen); with ranks = NULL every token is valid and
 * its packed row is b * seqlen + n.  Pure data movement: bit-exact copies of
 * elem_bytes-wide elements (2 or 4), dim * elem_bytes a multiple of 16,
 * pointers 16-byte aligned, strides in elements and multiples of
 * 16 / elem_bytes, last dim contiguous; the written side's rows must not
 * overlap.  Set struct_size = sizeof(mi_attn_pack_params).
 */
typedef struct mi_attn_pack_params {
  size_t struct_size;
  void* padded;             /* read by pack, written by unpack */
  void* packed;             /* written by pack, read by unpack */
  const int32_t* ranks;     /* [batch * seqlen] or NULL (all valid) */
  const int32_t* cu_seqlens; /* [batch + 1]; required with ranks */
  int64_t batch, seqlen;
  int32_t heads, dim;
  int32_t elem_bytes;
  int64_t padded_stride_batch, padded_stride_tok, padded_stride_head;
  int64_t packed_stride_tok, packed_stride_head;
} mi_attn_pack_params;

int mi_attn_pack_tokens(const mi_attn_pack_params* p, void* stream);
int mi_attn_unpack_tokens(const mi_attn_pack_params* p, void* stream);

/*
 * Backward of the forward above: the gradients dq, dk, dv of a loss with
 * respect to q, k, v, given its gradient dout with respect to out (the LSE
 * output is not differentiated).  From the forward's definition, with p the
 * forward's probabilities of each (query row, visible key):
 *   dv_j = sum_i p_ij dout_i,  D_i = dout_i . out_i,
 *   ds_ij = p_ij (dout_i . v_j - D_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 * dk and dv summed over the query heads that share a kv head.  This is the
 * tiled FlashAttention-2 backward the triton-msl part-2 post describes
 * (section "Beyond softmax: linear attention and a trainable backward"); the
 * mtlattn 0.3.0 page (section "Drop-in for scaled_dot_product_attention")
 * composes it with causal, GQA/MQA and the sliding window, as here, and
 * with a constant additive bias.  p is recomputed from the forward's lse,
 * tile by tile.
 *
 * Supported: in_dtype BF16 or F16 (q, k, v, out, dout), dq / dk / dv in
 * in_dtype or fp32, (d_qk, d_v) in {(64,64), (96,96), (128,128)}, hq % hkv == 0,
 * window > 0 only with causal.  Anything else is refused
 * (MI_ATTN_ERR_UNSUPPORTED).
 */
typedef struct mi_attn_bwd_params {
  size_t struct_size; /* sizeof(mi_attn_bwd_params) */
  const void* q;      /* the forward's inputs, layouts as in mi_attn_fwd_params */
  const void* k;
  const void* v;
  const void* out;    /* the forward's output [total_q, hq, d_v] (in_dtype) */
  const float* lse;   /* the forward's LSE [hq, total_q] */
  const void* dout;   /* gradient of the loss w.r.t. out, [total_q, hq, d_v] (in_dtype) */
  void* dq;           /* outputs, [total_q, hq, d_qk], [total_kv, hkv, d_qk], */
  void* dk;           /* [total_kv, hkv, d_v] in grad_dtype, every element */
  void* dv;           /* written; their rows must not overlap */
  float* delta;       /* workspace: fp32 [hq, total_q], caller-owned, overwritten */
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_kv;
  int64_t num_seqs;
  int64_t max_seqlen_q;  /* >= every sequence's query length */
  int64_t max_seqlen_kv; /* >= every sequence's key length */
  int64_t total_q;
  int64_t total_kv;
  int32_t hq, hkv, d_qk, d_v;
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t out_stride_tok, out_stride_head;
  int64_t dout_stride_tok, dout_stride_head;
  int64_t dq_stride_tok, dq_stride_head;
  int64_t dk_stride_tok, dk_stride_head;
  int64_t dv_stride_tok, dv_stride_head;
  int32_t in_dtype;   /* MI_ATTN_BF16 or MI_ATTN_F16 */
  int32_t grad_dtype; /* in_dtype or MI_ATTN_F32 (dq, dk, dv) */
  float scale;        /* the forward's softmax scale */
  int32_t causal;   /* the forward's flags */
  int32_t window;
  /* Added in version 1.4 (a smaller struct_size reads these as NULL / 0): the
   * forward's additive bias, same layout and rules as in mi_attn_fwd_params,
   * treated as a constant (its gradient is not computed; the mtlattn page,
   * section "Use", applies the bias in forward and backward this way).
   * NULL: no bias. */
  const float* bias;
  int32_t bias_heads;
  int64_t bias_cols;
  int64_t bias_stride_tok, bias_stride_head;
  /* Added in version 1.5: the forward's ALiBi slopes, same layout and rule
   * as in mi_attn_fwd_params (not with a bias).  NULL: none. */
  const float* alibi_slopes;
  int64_t alibi_stride_seq;
} mi_attn_bwd_params;

/*
 * Enqueue the backward on `stream` (three kernels: delta, dk/dv, dq) and
 * return without waiting.  Pointers are device memory owned by the caller;
 * the library allocates nothing.  Strides follow the forward's rules
 * (multiples of 8 elements, 16-byte aligned pointers).  No atomics: the run
 * is bitwise deterministic.  Returns MI_ATTN_OK or a negative code (nothing
 * launched); MI_ATTN_VALIDATE=1 checks the cu_seqlens contracts as for the
 * forward.
 */
int mi_attn_varlen_bwd(const mi_attn_bwd_params* p, void* stream);

/*
 * Split-KV decode: the forward above for calls with few query rows per
 * sequence and long key/value caches (cached decode, end-aligned causal
 * rule: the mtlattn 0.3.0 project page, section "Use", notes that this
 * convention makes self-attention and cached decode both hold).  The visible
 * key range of every (sequence, kv head) is cut into chunks computed by
 * separate workgroups; all query heads of a kv head's group and all query
 * rows of a sequence share each K/V read.  The chunks' unnormalised outputs
 * and running max / sum go to `workspace`, and a second kernel merges them
 * with the log-sum-exp rule: M = max m_c, L = sum l_c 2^(m_c - M),
 * out = sum O_c 2^(m_c - M) / L, lse = (M + log2 L) ln 2.
 *
 * Takes the forward's params (same meaning, same results to rounding), plus
 * max_seqlen_kv >= every sequence's key length and num_splits (chunks per
 * (sequence, kv head); 0 = enough to fill the GPU).  Supported: bf16 / fp16,
 * (d_qk, d_v) in {(64,64), (128,128)}, no bias, (hq / hkv) * max_seqlen_q
 * <= 64; anything else is refused (use mi_attn_varlen_fwd).
 * workspace: caller-owned device memory of at least
 * mi_attn_decode_workspace_size(p, max_seqlen_kv, num_splits) bytes, 16-byte
 * aligned; overwritten.  Asynchronous on `stream`, deterministic.
 */
size_t mi_attn_decode_workspace_size(const mi_attn_fwd_params* p, int64_t max_seqlen_kv,
                                     int32_t num_splits);
int mi_attn_varlen_decode(const mi_attn_fwd_params* p, int64_t max_seqlen_kv, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mi_attn_varlen_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the partial results go to a fixed device
 * array of 16 MiB that the library holds on every GPU it runs on until the
 * process ends (no hipMalloc, hipFree or allocating call, ever).  When the
 * requested (or automatic) number of chunks would not fit, fewer and longer
 * chunks are used; when even one chunk per (sequence, kv head) needs more
 * than 16 MiB (total_q * hq * (d_v + 2) * 4 bytes), the call is refused with
 * MI_ATTN_ERR_UNSUPPORTED.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * ordered by the caller.  Nothing in the array needs clearing between calls.
 * Same arguments, checks and results as mi_attn_varlen_decode.
 */
int mi_attn_varlen_decode_noalloc(const mi_attn_fwd_params* p, int64_t max_seqlen_kv,
                                  int32_t num_splits, void* stream);

/* Reason for the last non-OK return on the calling thread ("" if none). */
const char* mi_attn_last_error(void);

/* MI_ATTN_VERSION of the built library. */
int mi_attn_version(void);

/*
 * Tile shape the kernel uses for (in_dtype, d_qk, d_v) without a bias:
 * *bm query rows per workgroup and *bn keys per key tile (with a bias the
 * 16-bit kernel for d_qk = 128 steps through 32-key halves of these tiles;
 * tile_counts are still given in *bn units).  Returns MI_ATTN_OK, or
 * MI_ATTN_ERR_UNSUPPORTED for a combination outside the supported set.
 */
int mi_attn_tile_shape(int32_t in_dtype, int32_t d_qk, int32_t d_v, int32_t* bm, int32_t* bn);

#ifdef __cplusplus
}
#endif

#endif /* MI_ATTN_H */
