// C-ABI front end of the varlen attention forward: argument validation
// (correct-or-refuse, as the triton-msl part-1 post describes in its section
// "Correct-or-refuse"), grid construction and the launch on the caller's
// stream.  No device memory is allocated here and no host synchronisation
// happens unless MI_ATTN_VALIDATE=1 asks for the cu_seqlens check.
#include "mi_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "attn_bwd.h"
#include "attn_decode.h"
#include "attn_fwd.h"
#include "bias_ranges.h"
#include "padding.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int32_t dt) { return dt == MI_ATTN_F32 ? 4 : 2; }

bool dims_supported(int32_t dt, int32_t dqk, int32_t dv) {
  if (dqk == 64 && dv == 64) return true;
  if (dqk == 128 && dv == 128) return true;
  if (dqk == 192 && dv == 128) return dt != MI_ATTN_F32;
  if (dqk == 256 && dv == 256) return dt != MI_ATTN_F32;
  if (dqk == 96 && dv == 96) return dt != MI_ATTN_F32;
  return false;
}

// The params of a 1.0 caller end before bias_ranges; later fields read as 0.
constexpr size_t kParamsSizeV1 = offsetof(mi_attn_fwd_params, bias_ranges);

int copy_params(const mi_attn_fwd_params* p, mi_attn_fwd_params* out) {
  if (p == nullptr) return fail(MI_ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->struct_size < kParamsSizeV1)
    return fail(MI_ATTN_ERR_INVALID_ARG, "struct_size %zu < %zu (not an mi_attn_fwd_params)",
                p->struct_size, kParamsSizeV1);
  std::memset(out, 0, sizeof(*out));
  std::memcpy(out, p, p->struct_size < sizeof(*out) ? p->struct_size : sizeof(*out));
  return MI_ATTN_OK;
}

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

// While a row's softmax sum l (in units of its largest p) is below this
// after a tile, the tile's P is carried to 16 bits (hi + lo halves) in the
// PV product.  bf16 keeps 8 significant bits: P rounded once errs by up to
// 2^-9 of each p, and with only a few keys carrying the row that reaches
// ~2e-3 of |v| in the output.  fp16 keeps 11 bits, 8x less.
constexpr float kSplitLBf16 = 12.0f;
constexpr float kSplitLF16 = 3.0f;

// The n_tok x n_head x width elements at t * st + h * sh + d (d < width)
// are pairwise distinct: the smaller stride spans a full row and the larger
// one spans the whole extent of the smaller dimension (a dimension of size 1
// places no constraint).  Exotic interleavings that are disjoint but fail
// this test are refused, not miscomputed.
bool layout_disjoint(int64_t st, int64_t n_tok, int64_t sh, int64_t n_head, int64_t width) {
  if (n_tok <= 1 && n_head <= 1) return true;
  if (n_tok <= 1) return sh >= width;
  if (n_head <= 1) return st >= width;
  const bool tok_inner = st <= sh;
  const int64_t s_in = tok_inner ? st : sh, n_in = tok_inner ? n_tok : n_head;
  const int64_t s_out = tok_inner ? sh : st;
  return s_in >= width && s_out >= s_in * (n_in - 1) + width;
}

// Rows of `width` bytes at sum_i idx_i * st[i] (0 <= idx_i < n[i]) never
// overlap: taken by increasing stride, each stride clears the extent of the
// levels inside it (sufficient, the usual nesting of a strided view).
bool nested_disjoint(std::vector<std::pair<int64_t, int64_t>> lv, int64_t width) {
  std::sort(lv.begin(), lv.end());
  int64_t extent = width;
  for (const auto& l : lv) {
    if (l.second <= 1) continue;
    if (l.first < extent) return false;
    extent = l.first * (l.second - 1) + extent;
  }
  return true;
}

int validate_cu(const int32_t* cu_dev, int64_t n, int64_t total, int64_t max_len,
                const char* what) {
  std::vector<int32_t> cu(static_cast<size_t>(n + 1));
  hipError_t e = hipMemcpy(cu.data(), cu_dev, sizeof(int32_t) * (n + 1), hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return fail(MI_ATTN_ERR_VALIDATION, "%s: copying cu_seqlens failed: %s", what,
                hipGetErrorString(e));
  if (cu[0] != 0) return fail(MI_ATTN_ERR_VALIDATION, "%s[0] = %d, expected 0", what, cu[0]);
  for (int64_t s = 0; s < n; ++s) {
    const int64_t len = (int64_t)cu[s + 1] - cu[s];
    if (len < 0)
      return fail(MI_ATTN_ERR_VALIDATION, "%s decreases at sequence %lld", what, (long long)s);
    if (max_len >= 0 && len > max_len)
      return fail(MI_ATTN_ERR_VALIDATION, "%s: sequence %lld has length %lld > bound %lld", what,
                  (long long)s, (long long)len, (long long)max_len);
  }
  if (cu[n] != total)
    return fail(MI_ATTN_ERR_VALIDATION, "%s[%lld] = %d, expected total %lld", what, (long long)n,
                cu[n], (long long)total);
  return MI_ATTN_OK;
}

// Checks of a forward call shared by the forward and the decode entry points
// (correct-or-refuse); *empty is set when there is nothing to compute.
int check_fwd_params(const mi_attn_fwd_params* p, bool* empty) {
  *empty = false;
  const int32_t dt = p->in_dtype;
  if (dt != MI_ATTN_F32 && dt != MI_ATTN_F16 && dt != MI_ATTN_BF16)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "unknown in_dtype %d", dt);
  if (p->out_dtype != dt && p->out_dtype != MI_ATTN_F32)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "out_dtype must equal in_dtype or be F32 (got %d)",
                p->out_dtype);
  if (!dims_supported(dt, p->d_qk, p->d_v))
    return fail(MI_ATTN_ERR_UNSUPPORTED,
                "head dims (d_qk=%d, d_v=%d) unsupported for this dtype; supported: (64,64), "
                "(128,128), and (96,96), (192,128) and (256,256) for 16-bit inputs",
                p->d_qk, p->d_v);
  if (p->hq <= 0 || p->hkv <= 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "head counts must be positive (hq=%d, hkv=%d)", p->hq,
                p->hkv);
  if (p->hq % p->hkv != 0)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "hq (%d) must be a multiple of hkv (%d)", p->hq, p->hkv);
  if (p->num_seqs < 0 || p->max_seqlen_q < 0 || p->total_q < 0 || p->total_kv < 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "negative size");
  if (p->window < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "window must be >= 0");
  if (p->causal != 0 && p->causal != 1) return fail(MI_ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->window > 0 && !p->causal)
    return fail(MI_ATTN_ERR_UNSUPPORTED,
                "a sliding window is defined relative to the causal diagonal; set causal=1");
  const bool rope = p->q_rope != nullptr || p->k_rope != nullptr;
  if (rope) {
    if (p->q_rope == nullptr || p->k_rope == nullptr)
      return fail(MI_ATTN_ERR_INVALID_ARG, "q_rope and k_rope must be given together");
    if (dt == MI_ATTN_F32 || p->d_qk != 192 || p->d_v != 128)
      return fail(MI_ATTN_ERR_UNSUPPORTED,
                  "split nope / rope operands need 16-bit inputs with d_qk = 192, d_v = 128");
  }
  if (!std::isfinite(p->scale)) return fail(MI_ATTN_ERR_INVALID_ARG, "scale is not finite");
  if (!(p->scale > 0.0f))
    return fail(MI_ATTN_ERR_UNSUPPORTED, "scale must be > 0 (got %g)", (double)p->scale);
  if (p->total_q > INT32_MAX || p->total_kv > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "total token counts must fit in int32 (cu_seqlens)");

  if (p->num_seqs == 0 || p->max_seqlen_q == 0 || p->total_q == 0) {
    *empty = true;
    return MI_ATTN_OK;
  }

  if (!p->q || !p->k || !p->v || !p->out || !p->cu_seqlens_q || !p->cu_seqlens_kv)
    return fail(MI_ATTN_ERR_INVALID_ARG, "q, k, v, out, cu_seqlens_q and cu_seqlens_kv are required");
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->out))
    return fail(MI_ATTN_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  const int64_t in_mult = 16 / elem_size(dt);
  const int64_t out_mult = 16 / elem_size(p->out_dtype);
  const int64_t in_strides[6] = {p->q_stride_tok, p->q_stride_head, p->k_stride_tok,
                                 p->k_stride_head, p->v_stride_tok, p->v_stride_head};
  for (int64_t s : in_strides)
    if (s < 0 || s % in_mult != 0)
      return fail(MI_ATTN_ERR_INVALID_ARG,
                  "q/k/v strides must be non-negative multiples of %lld elements (got %lld)",
                  (long long)in_mult, (long long)s);
  const int64_t dqk_main = rope ? p->d_qk - 64 : p->d_qk;  // width q and k hold
  if (p->q_stride_tok < dqk_main || p->k_stride_tok < dqk_main || p->v_stride_tok < p->d_v)
    return fail(MI_ATTN_ERR_UNSUPPORTED,
                "q/k/v token strides must cover a full head row (q_stride_tok, k_stride_tok >= d_qk, "
                "or 128 with q_rope / k_rope; v_stride_tok >= d_v)");
  if (rope) {
    if (!aligned16(p->q_rope) || !aligned16(p->k_rope))
      return fail(MI_ATTN_ERR_INVALID_ARG, "q_rope and k_rope must be 16-byte aligned");
    const int64_t rs[4] = {p->q_rope_stride_tok, p->q_rope_stride_head, p->k_rope_stride_tok,
                           p->k_rope_stride_head};
    for (int64_t s : rs)
      if (s < 0 || s % 8 != 0)
        return fail(MI_ATTN_ERR_INVALID_ARG,
                    "q_rope/k_rope strides must be non-negative multiples of 8 elements (got %lld)",
                    (long long)s);
    if (p->q_rope_stride_tok < 64 || p->k_rope_stride_tok < 64)
      return fail(MI_ATTN_ERR_UNSUPPORTED, "q_rope/k_rope token strides must be >= 64");
    if (p->q_rope_stride_tok * 2 * 64 > INT32_MAX || p->k_rope_stride_tok * 2 * 64 > INT32_MAX)
      return fail(MI_ATTN_ERR_UNSUPPORTED,
                  "q_rope/k_rope token strides too large (more than 32 MiB per token)");
  }
  // 16-bit Q rows and K/V tiles are fetched through 32-bit buffer offsets
  // spanning at most 64 tokens.
  if (dt != MI_ATTN_F32 &&
      (p->q_stride_tok * elem_size(dt) * 64 > INT32_MAX || p->k_stride_tok * elem_size(dt) * 64 > INT32_MAX ||
       p->v_stride_tok * elem_size(dt) * 64 > INT32_MAX))
    return fail(MI_ATTN_ERR_UNSUPPORTED, "q/k/v token strides too large (more than 32 MiB per token)");
  if (p->out_stride_tok < 0 || p->out_stride_head < 0 || p->out_stride_tok % out_mult != 0 ||
      p->out_stride_head % out_mult != 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "out strides must be non-negative multiples of %lld",
                (long long)out_mult);
  // Output rows must not overlap (different workgroups would write the same
  // addresses); the 16-bit kernels store 32-row blocks through 32-bit buffer
  // offsets.
  if (p->out_stride_tok < p->d_v)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "out token stride must be >= d_v");
  if (!layout_disjoint(p->out_stride_tok, p->total_q, p->out_stride_head, p->hq, p->d_v))
    return fail(MI_ATTN_ERR_UNSUPPORTED,
                "out strides (token %lld, head %lld) make the [%lld, %d, %d] rows overlap",
                (long long)p->out_stride_tok, (long long)p->out_stride_head, (long long)p->total_q,
                p->hq, p->d_v);
  if (dt != MI_ATTN_F32 && p->out_stride_tok * elem_size(p->out_dtype) * 32 > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "out token stride too large (more than 64 MiB per token)");
  if (p->mask != nullptr && p->bias != nullptr)
    return fail(MI_ATTN_ERR_INVALID_ARG, "give a bias or a mask, not both");
  const bool has_mask = p->mask != nullptr;
  const bool has_bias = p->bias != nullptr || has_mask;
  if (p->alibi_slopes != nullptr) {
    if (has_bias)
      return fail(MI_ATTN_ERR_UNSUPPORTED,
                  "ALiBi slopes together with a bias tensor or a mask are not supported");
    if ((reinterpret_cast<uintptr_t>(p->alibi_slopes) & 3u) != 0 || p->alibi_stride_seq < 0)
      return fail(MI_ATTN_ERR_INVALID_ARG,
                  "alibi_slopes must be 4-byte aligned with a non-negative sequence stride");
  }
  if (has_bias) {
    if (p->bias_heads != 1 && p->bias_heads != p->hq)
      return fail(MI_ATTN_ERR_UNSUPPORTED, "bias_heads must be 1 or hq (got %d)", p->bias_heads);
    if (has_mask) {
      if ((reinterpret_cast<uintptr_t>(p->mask) & 3u) != 0 || p->bias_stride_tok < 0 ||
          p->bias_stride_head < 0 || p->bias_stride_tok % 4 != 0 || p->bias_stride_head % 4 != 0)
        return fail(MI_ATTN_ERR_INVALID_ARG,
                    "mask must be 4-byte aligned with strides that are multiples of 4 bytes");
    } else if (!aligned16(p->bias) || p->bias_stride_tok < 0 || p->bias_stride_head < 0 ||
               p->bias_stride_tok % 4 != 0 || p->bias_stride_head % 4 != 0) {
      return fail(MI_ATTN_ERR_INVALID_ARG,
                  "bias must be 16-byte aligned with strides that are multiples of 4");
    }
    if (p->bias_cols <= 0) return fail(MI_ATTN_ERR_INVALID_ARG, "bias_cols must be > 0");
    if (p->bias_ranges != nullptr && (reinterpret_cast<uintptr_t>(p->bias_ranges) & 7u) != 0)
      return fail(MI_ATTN_ERR_INVALID_ARG, "bias_ranges must be 8-byte aligned");
  }
  if (p->bias_pure != nullptr && !has_bias)
    return fail(MI_ATTN_ERR_INVALID_ARG, "bias_pure is given without a bias or a mask");
  if ((reinterpret_cast<uintptr_t>(p->seqused_q) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(p->seqused_kv) & 3u) != 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "seqused_q / seqused_kv must be 4-byte aligned");

  return MI_ATTN_OK;
}

// Chunking of a split-KV decode call.
struct DecodePlan {
  int nb;           // 32-row blocks of packed rows (group * max_seqlen_q <= 32 nb)
  int chunk_tiles;  // 32-key tiles per chunk
  int n_chunks;
  size_t ws_o_bytes, ws_bytes;
};

constexpr int kDecodeTileKeys = 32;
// One one-wave workgroup per SIMD (256 CUs x 4): every chunk runs in the
// first and only round of workgroups.  Measured on the 8 x (10K-51K key)
// decode workload: 256 / 512 / 1024 / 2048 / 4096 / 8192 / 16384 target
// waves gave 1.94 / 3.58 / 4.49 / 4.28 / 4.15 / 3.86 / 3.66 TB/s.
constexpr int64_t kDecodeTargetWaves = 1024;

// Checks a decode call and plans its chunks: num_splits chunks per (sequence,
// kv head) if > 0, else enough for kDecodeTargetWaves workgroups; at most
// max_ws bytes of workspace (fewer, longer chunks when it would not fit).
int plan_decode(const mi_attn_fwd_params* p, int64_t max_seqlen_kv, int32_t num_splits,
                size_t max_ws, DecodePlan* plan, bool* empty) {
  const int rc = check_fwd_params(p, empty);
  if (rc != MI_ATTN_OK) return rc;
  if (p->in_dtype == MI_ATTN_F32)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "split-KV decode takes bf16 or fp16 inputs");
  if (!((p->d_qk == 64 && p->d_v == 64) || (p->d_qk == 128 && p->d_v == 128)))
    return fail(MI_ATTN_ERR_UNSUPPORTED, "split-KV decode head dims: (64,64) or (128,128)");
  if (p->bias != nullptr) return fail(MI_ATTN_ERR_UNSUPPORTED, "split-KV decode takes no bias");
  if (p->q_rope != nullptr || p->k_rope != nullptr)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "split-KV decode takes no q_rope / k_rope");
  if (p->alibi_slopes != nullptr)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "split-KV decode takes no ALiBi slopes");
  if (p->mask != nullptr) return fail(MI_ATTN_ERR_UNSUPPORTED, "split-KV decode takes no mask");
  if (p->seqused_q != nullptr)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "split-KV decode uses every query row (no seqused_q)");
  if (num_splits < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "num_splits must be >= 0 (0 = auto)");
  if (max_seqlen_kv < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "max_seqlen_kv must be >= 0");
  const int64_t group = p->hq / p->hkv;
  if (group * p->max_seqlen_q > 64)
    return fail(MI_ATTN_ERR_UNSUPPORTED,
                "split-KV decode packs (hq / hkv) * max_seqlen_q <= 64 rows per kv head (got %lld); "
                "use mi_attn_varlen_fwd",
                (long long)(group * p->max_seqlen_q));
  if (*empty) return MI_ATTN_OK;
  int64_t vis = max_seqlen_kv;
  if (p->window > 0 && vis > (int64_t)p->window + p->max_seqlen_q - 1)
    vis = (int64_t)p->window + p->max_seqlen_q - 1;
  const int64_t tiles = (vis + kDecodeTileKeys - 1) / kDecodeTileKeys + 1;  // +1: unaligned start
  const int64_t units = (int64_t)p->num_seqs * p->hkv;
  if (units > INT32_MAX) return fail(MI_ATTN_ERR_UNSUPPORTED, "too many (sequence, kv head) units");
  // the merge runs one 256-thread workgroup per (row, head)
  if ((int64_t)p->total_q * p->hq > (int64_t)1 << 24)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "too many (row, head) pairs for the merge (at most 2^24)");
  int64_t splits = num_splits > 0 ? num_splits : (kDecodeTargetWaves + units - 1) / units;
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, tiles));
  const size_t row_bytes = (size_t)p->total_q * (size_t)p->hq * (size_t)(p->d_v + 2) * 4;
  if (row_bytes > max_ws) return fail(MI_ATTN_ERR_UNSUPPORTED, "decode workspace limit too small");
  const int64_t fit = (int64_t)(max_ws / row_bytes);
  if (splits > fit) splits = fit;
  plan->chunk_tiles = (int)((tiles + splits - 1) / splits);
  plan->n_chunks = (int)((tiles + plan->chunk_tiles - 1) / plan->chunk_tiles);
  if (plan->n_chunks > 65535) return fail(MI_ATTN_ERR_UNSUPPORTED, "too many chunks");
  plan->nb = group * p->max_seqlen_q <= 32 ? 1 : 2;
  plan->ws_o_bytes = (size_t)plan->n_chunks * p->total_q * p->hq * p->d_v * 4;
  plan->ws_bytes = plan->ws_o_bytes + (size_t)plan->n_chunks * p->total_q * p->hq * 2 * 4;
  return MI_ATTN_OK;
}

int launch_decode(const mi_attn_fwd_params* p, const DecodePlan& plan, void* ws, void* stream) {
  mi_attn::DecodeArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v;
  a.cu_q = p->cu_seqlens_q; a.cu_kv = p->cu_seqlens_kv;
  a.seqused_kv = p->seqused_kv;
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + plan.ws_o_bytes);
  a.out = p->out; a.lse = p->lse;
  a.q_st = p->q_stride_tok; a.q_sh = p->q_stride_head;
  a.k_st = p->k_stride_tok; a.k_sh = p->k_stride_head;
  a.v_st = p->v_stride_tok; a.v_sh = p->v_stride_head;
  a.o_st = p->out_stride_tok; a.o_sh = p->out_stride_head;
  a.total_q = p->total_q;
  a.num_seqs = (int32_t)p->num_seqs;
  a.hq = p->hq; a.hkv = p->hkv; a.group = p->hq / p->hkv;
  a.causal = p->causal; a.window = p->window;
  a.chunk_tiles = plan.chunk_tiles;
  a.n_chunks = plan.n_chunks;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  a.split_l = p->in_dtype == MI_ATTN_BF16 ? kSplitLBf16 : kSplitLF16;
  if (env_flag("MI_ATTN_VALIDATE")) {
    int rc = validate_cu(p->cu_seqlens_q, p->num_seqs, p->total_q, p->max_seqlen_q, "cu_seqlens_q");
    if (rc != MI_ATTN_OK) return rc;
    rc = validate_cu(p->cu_seqlens_kv, p->num_seqs, p->total_kv, -1, "cu_seqlens_kv");
    if (rc != MI_ATTN_OK) return rc;
  }
  hipError_t e = mi_attn::launch_attn_decode(a, p->in_dtype, p->out_dtype == MI_ATTN_F32, p->d_qk,
                                             plan.nb, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return MI_ATTN_OK;
}

// Device scratch of the non-allocating decode entry point: one array per
// GPU, alive until the process ends.  Host code never passes its name to a
// kernel (on the host the name is not a device address): the address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kDecodeScratchBytes = 16u << 20;  // 16 MiB
__device__ __attribute__((aligned(256))) char scratch[kDecodeScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device id, filled on first use

int scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_ptr[(size_t)dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MI_ATTN_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[(size_t)dev] = p;
  }
  *ptr = g_scratch_ptr[(size_t)dev];
  return MI_ATTN_OK;
}

}  // namespace

extern "C" {

const char* mi_attn_last_error(void) { return g_last_error.c_str(); }

int mi_attn_version(void) { return MI_ATTN_VERSION; }

int mi_attn_tile_shape(int32_t in_dtype, int32_t d_qk, int32_t d_v, int32_t* bm, int32_t* bn) {
  if (in_dtype != MI_ATTN_F32 && in_dtype != MI_ATTN_F16 && in_dtype != MI_ATTN_BF16)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "unknown dtype %d", in_dtype);
  if (!dims_supported(in_dtype, d_qk, d_v))
    return fail(MI_ATTN_ERR_UNSUPPORTED, "head dims (%d, %d) unsupported for dtype %d", d_qk, d_v,
                in_dtype);
  if (bm) *bm = mi_attn::tile_bm(in_dtype, d_qk, d_v);
  if (bn) *bn = mi_attn::tile_bn(in_dtype, d_qk, d_v);
  return MI_ATTN_OK;
}

int mi_attn_varlen_fwd(const mi_attn_fwd_params* p_in, void* stream) {
  g_last_error.clear();
  mi_attn_fwd_params local;
  const int rc_copy = copy_params(p_in, &local);
  if (rc_copy != MI_ATTN_OK) return rc_copy;
  const mi_attn_fwd_params* p = &local;
  const int32_t dt = p->in_dtype;
  bool empty = false;
  const int rc_check = check_fwd_params(p, &empty);
  if (rc_check != MI_ATTN_OK || empty) return rc_check;
  const bool has_bias = p->bias != nullptr || p->mask != nullptr;  // a tensor bias or a byte mask
  if (p->bias_pure != nullptr && p->bias_ranges == nullptr)
    return fail(MI_ATTN_ERR_INVALID_ARG, "bias_pure needs the bias_ranges it was computed with");

  int32_t bm = 0, bn = 0;
  if (mi_attn_tile_shape(dt, p->d_qk, p->d_v, &bm, &bn) != MI_ATTN_OK) return MI_ATTN_ERR_UNSUPPORTED;
  const int64_t n_qtiles = (p->max_seqlen_q + bm - 1) / bm;
  const int64_t grid_x = (int64_t)p->hq * p->num_seqs;
  if (grid_x > INT32_MAX || n_qtiles > 65535)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "problem too large for one launch (hq*num_seqs=%lld, "
                "q tiles=%lld)", (long long)grid_x, (long long)n_qtiles);

  if (env_flag("MI_ATTN_VALIDATE")) {
    int rc = validate_cu(p->cu_seqlens_q, p->num_seqs, p->total_q, p->max_seqlen_q, "cu_seqlens_q");
    if (rc != MI_ATTN_OK) return rc;
    rc = validate_cu(p->cu_seqlens_kv, p->num_seqs, p->total_kv, has_bias ? p->bias_cols : -1,
                     "cu_seqlens_kv");
    if (rc != MI_ATTN_OK) return rc;
  }

  mi_attn::KernelArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.out = p->out;
  a.lse = p->lse;
  a.cu_q = p->cu_seqlens_q;
  a.cu_kv = p->cu_seqlens_kv;
  a.bias = p->bias;
  a.mask = p->mask;
  a.bias_ranges = has_bias ? p->bias_ranges : nullptr;
  a.bias_pure = has_bias ? p->bias_pure : nullptr;
  a.seqused_q = p->seqused_q;
  a.seqused_kv = p->seqused_kv;
  a.q_rope = p->q_rope;
  a.k_rope = p->k_rope;
  a.qr_st = p->q_rope_stride_tok;
  a.qr_sh = p->q_rope_stride_head;
  a.kr_st = p->k_rope_stride_tok;
  a.kr_sh = p->k_rope_stride_head;
  a.alibi = p->alibi_slopes;
  a.alibi_ss = p->alibi_stride_seq;
  a.tile_counts = p->tile_counts;
  a.q_st = p->q_stride_tok;
  a.q_sh = p->q_stride_head;
  a.k_st = p->k_stride_tok;
  a.k_sh = p->k_stride_head;
  a.v_st = p->v_stride_tok;
  a.v_sh = p->v_stride_head;
  a.o_st = p->out_stride_tok;
  a.o_sh = p->out_stride_head;
  a.b_st = has_bias ? p->bias_stride_tok : 0;
  a.bias_cols = has_bias ? (int32_t)(p->bias_cols < INT32_MAX ? p->bias_cols : INT32_MAX) : 0;
  a.b_sh = has_bias ? p->bias_stride_head : 0;
  a.total_q = p->total_q;
  a.num_seqs = (int32_t)p->num_seqs;
  a.hq = p->hq;
  a.group = p->hq / p->hkv;
  a.bias_heads = has_bias ? p->bias_heads : 1;
  a.causal = p->causal;
  a.window = p->window;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  a.split_l = dt == MI_ATTN_BF16 ? kSplitLBf16 : (dt == MI_ATTN_F16 ? kSplitLF16 : 0.0f);

  a.n_qtiles = (int32_t)n_qtiles;
  // A bias shared by all query heads (16-bit kernels): every head of one
  // (sequence, query tile) runs on one XCD so that its bias rows are read
  // from HBM once, not once per head.  One-dimensional grid, kept well
  // below 2^32 work-items.
  const int64_t groups8 = ((int64_t)p->num_seqs * n_qtiles + 7) / 8 * 8;
  const int64_t hm_wgs = (int64_t)p->hq * groups8;
  a.head_major = (dt != MI_ATTN_F32 && has_bias && p->bias_heads == 1 && p->hq > 1 &&
                  hm_wgs <= (int64_t)INT32_MAX / 256) ? 1 : 0;
  // Many heads without kv sharing (16-bit kernels): more items per row and
  // XCD (hq * num_seqs / 8) than the 64 an XCD holds at once means that the
  // items running together would each stream different K/V; run up to
  // kKvRows rows of one head together instead so that they share it through
  // L2 (never more rows than there are, which would only add empty items).
  constexpr int64_t kKvRows = 8;
  const int64_t kv_r = n_qtiles < kKvRows ? n_qtiles : kKvRows;
  const int64_t kv_rows_wgs = kv_r > 0 ? grid_x * ((n_qtiles + kv_r - 1) / kv_r * kv_r) : 0;
  a.kv_rows = (!a.head_major && dt != MI_ATTN_F32 && p->hq == p->hkv && grid_x % 8 == 0 &&
               grid_x / 8 >= 64 && kv_r >= 2 && kv_rows_wgs <= (int64_t)INT32_MAX / 256)
                  ? (int32_t)kv_r : 0;
  const dim3 grid = a.head_major ? dim3((unsigned)hm_wgs, 1u)
                    : a.kv_rows   ? dim3((unsigned)kv_rows_wgs, 1u)
                                  : dim3((unsigned)grid_x, (unsigned)n_qtiles);
  hipError_t e = mi_attn::launch_attn_fwd(a, dt, p->out_dtype, p->d_qk, p->d_v, has_bias, grid,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return MI_ATTN_OK;
}

int mi_attn_varlen_bwd(const mi_attn_bwd_params* p_in, void* stream) {
  g_last_error.clear();
  if (p_in == nullptr) return fail(MI_ATTN_ERR_INVALID_ARG, "params is NULL");
  // the params of a 1.2 / 1.3 caller end before bias; later fields read as 0
  constexpr size_t kBwdSizeV1 = offsetof(mi_attn_bwd_params, bias);
  if (p_in->struct_size < kBwdSizeV1)
    return fail(MI_ATTN_ERR_INVALID_ARG, "struct_size %zu < %zu", p_in->struct_size, kBwdSizeV1);
  mi_attn_bwd_params local;
  std::memset(&local, 0, sizeof(local));
  std::memcpy(&local, p_in, p_in->struct_size < sizeof(local) ? p_in->struct_size : sizeof(local));
  const mi_attn_bwd_params* p = &local;
  const int32_t dt = p->in_dtype;
  if (dt != MI_ATTN_F16 && dt != MI_ATTN_BF16)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "the backward takes bf16 or fp16 inputs (got dtype %d)", dt);
  if (!((p->d_qk == 64 && p->d_v == 64) || (p->d_qk == 96 && p->d_v == 96) ||
        (p->d_qk == 128 && p->d_v == 128)))
    return fail(MI_ATTN_ERR_UNSUPPORTED,
                "backward head dims (d_qk=%d, d_v=%d) unsupported; supported: (64,64), (96,96), "
                "(128,128)",
                p->d_qk, p->d_v);
  if (p->hq <= 0 || p->hkv <= 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "head counts must be positive (hq=%d, hkv=%d)", p->hq, p->hkv);
  if (p->hq % p->hkv != 0)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "hq (%d) must be a multiple of hkv (%d)", p->hq, p->hkv);
  if (p->num_seqs < 0 || p->max_seqlen_q < 0 || p->max_seqlen_kv < 0 || p->total_q < 0 ||
      p->total_kv < 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "negative size");
  if (p->window < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "window must be >= 0");
  if (p->causal != 0 && p->causal != 1) return fail(MI_ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->window > 0 && !p->causal)
    return fail(MI_ATTN_ERR_UNSUPPORTED,
                "a sliding window is defined relative to the causal diagonal; set causal=1");
  if (!std::isfinite(p->scale) || !(p->scale > 0.0f))
    return fail(MI_ATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (p->total_q > INT32_MAX || p->total_kv > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "total token counts must fit in int32 (cu_seqlens)");
  if (p->num_seqs == 0 || (p->total_q == 0 && p->total_kv == 0)) return MI_ATTN_OK;
  if (!p->q || !p->k || !p->v || !p->out || !p->lse || !p->dout || !p->dq || !p->dk || !p->dv ||
      !p->delta || !p->cu_seqlens_q || !p->cu_seqlens_kv)
    return fail(MI_ATTN_ERR_INVALID_ARG, "every pointer of the backward params is required");
  if (p->grad_dtype != dt && p->grad_dtype != MI_ATTN_F32)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "grad_dtype must equal in_dtype or be F32 (got %d)",
                p->grad_dtype);
  const void* ptrs16[] = {p->q, p->k, p->v, p->out, p->dout, p->dq, p->dk, p->dv};
  for (const void* q : ptrs16)
    if (!aligned16(q)) return fail(MI_ATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const int64_t strides[] = {p->q_stride_tok, p->q_stride_head, p->k_stride_tok, p->k_stride_head,
                             p->v_stride_tok, p->v_stride_head, p->out_stride_tok, p->out_stride_head,
                             p->dout_stride_tok, p->dout_stride_head, p->dq_stride_tok,
                             p->dq_stride_head, p->dk_stride_tok, p->dk_stride_head,
                             p->dv_stride_tok, p->dv_stride_head};
  for (int i = 0; i < 16; ++i) {
    const int64_t mult = (i >= 10 && p->grad_dtype == MI_ATTN_F32) ? 4 : 8;  // 16 bytes
    if (strides[i] < 0 || strides[i] % mult != 0)
      return fail(MI_ATTN_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  }
  const int64_t d = p->d_qk;
  const int64_t tok_strides[] = {p->q_stride_tok, p->k_stride_tok, p->v_stride_tok, p->out_stride_tok,
                                 p->dout_stride_tok, p->dq_stride_tok, p->dk_stride_tok,
                                 p->dv_stride_tok};
  for (int64_t st : tok_strides) {
    if (st < d) return fail(MI_ATTN_ERR_UNSUPPORTED, "token strides must cover a full head row");
    if (st * 4 * 64 > INT32_MAX)
      return fail(MI_ATTN_ERR_UNSUPPORTED, "token strides too large (more than 32 MiB per token)");
  }
  if (!layout_disjoint(p->dq_stride_tok, p->total_q, p->dq_stride_head, p->hq, d) ||
      !layout_disjoint(p->dk_stride_tok, p->total_kv, p->dk_stride_head, p->hkv, d) ||
      !layout_disjoint(p->dv_stride_tok, p->total_kv, p->dv_stride_head, p->hkv, d))
    return fail(MI_ATTN_ERR_UNSUPPORTED, "dq / dk / dv strides make their rows overlap");
  const bool has_bias = p->bias != nullptr;
  if (has_bias) {
    if (p->bias_heads != 1 && p->bias_heads != p->hq)
      return fail(MI_ATTN_ERR_UNSUPPORTED, "bias_heads must be 1 or hq (got %d)", p->bias_heads);
    if (!aligned16(p->bias) || p->bias_stride_tok < 0 || p->bias_stride_head < 0 ||
        p->bias_stride_tok % 4 != 0 || p->bias_stride_head % 4 != 0)
      return fail(MI_ATTN_ERR_INVALID_ARG,
                  "bias must be 16-byte aligned with strides that are multiples of 4");
    if (p->bias_cols <= 0) return fail(MI_ATTN_ERR_INVALID_ARG, "bias_cols must be > 0");
  }
  if (p->alibi_slopes != nullptr) {
    if (has_bias)
      return fail(MI_ATTN_ERR_UNSUPPORTED, "ALiBi slopes and a bias tensor together are not supported");
    if ((reinterpret_cast<uintptr_t>(p->alibi_slopes) & 3u) != 0 || p->alibi_stride_seq < 0)
      return fail(MI_ATTN_ERR_INVALID_ARG,
                  "alibi_slopes must be 4-byte aligned with a non-negative sequence stride");
  }
  const int64_t n_kt = (p->max_seqlen_kv + 127) / 128, n_qt = (p->max_seqlen_q + 127) / 128;
  if ((int64_t)p->hq * p->num_seqs > INT32_MAX || n_kt > 65535 || n_qt > 65535 ||
      (int64_t)p->total_q * p->hq * (d / 8) > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  if (env_flag("MI_ATTN_VALIDATE")) {
    int rc = validate_cu(p->cu_seqlens_q, p->num_seqs, p->total_q, p->max_seqlen_q, "cu_seqlens_q");
    if (rc != MI_ATTN_OK) return rc;
    rc = validate_cu(p->cu_seqlens_kv, p->num_seqs, p->total_kv, p->max_seqlen_kv, "cu_seqlens_kv");
    if (rc != MI_ATTN_OK) return rc;
  }
  mi_attn::BwdArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.out = p->out; a.dout = p->dout; a.lse = p->lse;
  a.dq = p->dq; a.dk = p->dk; a.dv = p->dv; a.delta = p->delta;
  a.cu_q = p->cu_seqlens_q; a.cu_kv = p->cu_seqlens_kv;
  a.q_st = p->q_stride_tok; a.q_sh = p->q_stride_head;
  a.k_st = p->k_stride_tok; a.k_sh = p->k_stride_head;
  a.v_st = p->v_stride_tok; a.v_sh = p->v_stride_head;
  a.o_st = p->out_stride_tok; a.o_sh = p->out_stride_head;
  a.do_st = p->dout_stride_tok; a.do_sh = p->dout_stride_head;
  a.dq_st = p->dq_stride_tok; a.dq_sh = p->dq_stride_head;
  a.dk_st = p->dk_stride_tok; a.dk_sh = p->dk_stride_head;
  a.dv_st = p->dv_stride_tok; a.dv_sh = p->dv_stride_head;
  a.total_q = p->total_q;
  a.num_seqs = (int32_t)p->num_seqs;
  a.hq = p->hq; a.hkv = p->hkv; a.group = p->hq / p->hkv;
  a.causal = p->causal; a.window = p->window;
  a.scale = p->scale;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  if (has_bias) {
    a.bias = p->bias;
    a.b_st = p->bias_stride_tok;
    a.b_sh = p->bias_stride_head;
    a.bias_heads = p->bias_heads;
    a.bias_cols = (int32_t)(p->bias_cols < INT32_MAX ? p->bias_cols : INT32_MAX);
  }
  a.alibi = p->alibi_slopes;
  a.alibi_ss = p->alibi_stride_seq;
  hipError_t e = mi_attn::launch_attn_bwd(a, dt, p->grad_dtype == MI_ATTN_F32, has_bias, (int)d,
                                          (int)p->max_seqlen_q, (int)p->max_seqlen_kv,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return MI_ATTN_OK;
}

size_t mi_attn_decode_workspace_size(const mi_attn_fwd_params* p_in, int64_t max_seqlen_kv,
                                     int32_t num_splits) {
  g_last_error.clear();
  mi_attn_fwd_params local;
  if (copy_params(p_in, &local) != MI_ATTN_OK) return 0;
  DecodePlan plan{};
  bool empty = false;
  if (plan_decode(&local, max_seqlen_kv, num_splits, SIZE_MAX, &plan, &empty) != MI_ATTN_OK) return 0;
  return empty ? 0 : plan.ws_bytes;
}

int mi_attn_varlen_decode(const mi_attn_fwd_params* p_in, int64_t max_seqlen_kv, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mi_attn_fwd_params local;
  const int rc_copy = copy_params(p_in, &local);
  if (rc_copy != MI_ATTN_OK) return rc_copy;
  DecodePlan plan{};
  bool empty = false;
  int rc = plan_decode(&local, max_seqlen_kv, num_splits, SIZE_MAX, &plan, &empty);
  if (rc != MI_ATTN_OK || empty) return rc;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "workspace must be a 16-byte aligned device pointer");
  if (workspace_bytes < plan.ws_bytes)
    return fail(MI_ATTN_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes,
                plan.ws_bytes);
  return launch_decode(&local, plan, workspace, stream);
}

int mi_attn_varlen_decode_noalloc(const mi_attn_fwd_params* p_in, int64_t max_seqlen_kv,
                                  int32_t num_splits, void* stream) {
  g_last_error.clear();
  mi_attn_fwd_params local;
  const int rc_copy = copy_params(p_in, &local);
  if (rc_copy != MI_ATTN_OK) return rc_copy;
  DecodePlan plan{};
  bool empty = false;
  int rc = plan_decode(&local, max_seqlen_kv, num_splits, kDecodeScratchBytes, &plan, &empty);
  if (rc != MI_ATTN_OK || empty) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != MI_ATTN_OK) return rc;
  return launch_decode(&local, plan, ws, stream);
}

int mi_attn_padding_to_varlen(const uint8_t* mask, int64_t batch, int64_t seqlen,
                              int64_t mask_stride_batch, int32_t* ranks, int32_t* cu_seqlens,
                              int32_t* stats, void* stream) {
  g_last_error.clear();
  if (batch < 0 || seqlen < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "negative size");
  if (batch >= INT32_MAX || seqlen > INT32_MAX || batch * seqlen > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "batch * seqlen must fit in int32 (cu_seqlens)");
  if (cu_seqlens == nullptr) return fail(MI_ATTN_ERR_INVALID_ARG, "cu_seqlens is required");
  const bool any = batch * seqlen > 0;
  if (any && (mask == nullptr || ranks == nullptr))
    return fail(MI_ATTN_ERR_INVALID_ARG, "mask and ranks are required");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(ranks) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(stats) & 3u) != 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "ranks, cu_seqlens and stats must be 4-byte aligned");
  if (mask_stride_batch < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "negative mask stride");
  mi_attn::PadRankArgs a{};
  a.mask = mask;
  a.mask_st = mask_stride_batch;
  a.ranks = ranks;
  a.cu = cu_seqlens;
  a.stats = stats;
  a.batch = (int32_t)batch;
  a.seqlen = (int32_t)seqlen;
  hipError_t e = mi_attn::launch_padding_ranks(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return MI_ATTN_OK;
}

int mi_attn_padding_lengths(const uint8_t* mask, int64_t batch, int64_t seqlen,
                            int64_t mask_stride_batch, int32_t* lengths, int32_t* spans,
                            int32_t* stats, void* stream) {
  g_last_error.clear();
  if (batch < 0 || seqlen < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "negative size");
  if (batch >= INT32_MAX || seqlen > INT32_MAX || batch * seqlen > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "batch * seqlen must fit in int32 (spans)");
  if (spans == nullptr || (batch > 0 && lengths == nullptr))
    return fail(MI_ATTN_ERR_INVALID_ARG, "lengths and spans are required");
  if (batch * seqlen > 0 && mask == nullptr) return fail(MI_ATTN_ERR_INVALID_ARG, "mask is required");
  if ((reinterpret_cast<uintptr_t>(lengths) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(spans) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(stats) & 3u) != 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "lengths, spans and stats must be 4-byte aligned");
  if (mask_stride_batch < 0) return fail(MI_ATTN_ERR_INVALID_ARG, "negative mask stride");
  mi_attn::PadLengthArgs a{};
  a.mask = mask;
  a.mask_st = mask_stride_batch;
  a.lengths = lengths;
  a.spans = spans;
  a.stats = stats;
  a.batch = (int32_t)batch;
  a.seqlen = (int32_t)seqlen;
  hipError_t e = mi_attn::launch_padding_lengths(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return MI_ATTN_OK;
}

namespace {

int pack_common(const mi_attn_pack_params* p_in, int unpack, void* stream) {
  g_last_error.clear();
  if (p_in == nullptr) return fail(MI_ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p_in->struct_size < sizeof(mi_attn_pack_params))
    return fail(MI_ATTN_ERR_INVALID_ARG, "struct_size %zu < %zu (not an mi_attn_pack_params)",
                p_in->struct_size, sizeof(mi_attn_pack_params));
  const mi_attn_pack_params& p = *p_in;
  if (p.elem_bytes != 2 && p.elem_bytes != 4)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "elem_bytes must be 2 or 4 (got %d)", p.elem_bytes);
  if (p.batch < 0 || p.seqlen < 0 || p.heads <= 0 || p.dim <= 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "sizes must be >= 0 (heads, dim > 0)");
  if (p.batch * p.seqlen > INT32_MAX || p.seqlen > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "batch * seqlen must fit in int32");
  const int64_t row_bytes = (int64_t)p.dim * p.elem_bytes;
  if (row_bytes % 16 != 0)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "dim * elem_bytes must be a multiple of 16 bytes");
  const int64_t chunks = (int64_t)p.heads * (row_bytes / 16);
  if (chunks > INT32_MAX) return fail(MI_ATTN_ERR_UNSUPPORTED, "heads * dim too large");
  const int64_t tokens = p.batch * p.seqlen;
  if (tokens == 0) return MI_ATTN_OK;
  if (p.padded == nullptr || p.packed == nullptr)
    return fail(MI_ATTN_ERR_INVALID_ARG, "padded and packed are required");
  if (p.ranks != nullptr && p.cu_seqlens == nullptr)
    return fail(MI_ATTN_ERR_INVALID_ARG, "ranks need the cu_seqlens they were computed with");
  if (!aligned16(p.padded) || !aligned16(p.packed))
    return fail(MI_ATTN_ERR_INVALID_ARG, "padded and packed must be 16-byte aligned");
  const int64_t mult = 16 / p.elem_bytes;
  const int64_t strides[5] = {p.padded_stride_batch, p.padded_stride_tok, p.padded_stride_head,
                              p.packed_stride_tok, p.packed_stride_head};
  for (int64_t st : strides)
    if (st < 0 || st % mult != 0)
      return fail(MI_ATTN_ERR_INVALID_ARG,
                  "strides must be non-negative multiples of %lld elements", (long long)mult);
  const int64_t eb = p.elem_bytes;
  // the side that is written must not overlap itself
  const bool ok = unpack
      ? nested_disjoint({{p.padded_stride_batch * eb, p.batch}, {p.padded_stride_tok * eb, p.seqlen},
                         {p.padded_stride_head * eb, p.heads}}, row_bytes)
      : nested_disjoint({{p.packed_stride_tok * eb, tokens}, {p.packed_stride_head * eb, p.heads}},
                        row_bytes);
  if (!ok)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "the %s strides make its rows overlap",
                unpack ? "padded" : "packed");
  mi_attn::PackArgs a{};
  a.padded = reinterpret_cast<char*>(p.padded);
  a.packed = reinterpret_cast<char*>(p.packed);
  a.ranks = p.ranks;
  a.cu = p.cu_seqlens;
  a.pd_sb = p.padded_stride_batch * eb;
  a.pd_st = p.padded_stride_tok * eb;
  a.pd_sh = p.padded_stride_head * eb;
  a.pk_st = p.packed_stride_tok * eb;
  a.pk_sh = p.packed_stride_head * eb;
  a.seqlen = (int32_t)p.seqlen;
  a.tokens = (int32_t)tokens;
  a.chunks = (int32_t)chunks;
  a.row_chunks = (int32_t)(row_bytes / 16);
  a.tok_per_wg = chunks >= 256 ? 1 : (int32_t)(256 / chunks);
  a.unpack = unpack;
  hipError_t e = mi_attn::launch_pack_tokens(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return MI_ATTN_OK;
}

}  // namespace

int mi_attn_pack_tokens(const mi_attn_pack_params* p, void* stream) { return pack_common(p, 0, stream); }

int mi_attn_unpack_tokens(const mi_attn_pack_params* p, void* stream) {
  return pack_common(p, 1, stream);
}

int mi_attn_bias_key_ranges(const mi_attn_fwd_params* p_in, int32_t* ranges, void* stream) {
  g_last_error.clear();
  mi_attn_fwd_params local;
  const int rc_copy = copy_params(p_in, &local);
  if (rc_copy != MI_ATTN_OK) return rc_copy;
  const mi_attn_fwd_params* p = &local;
  const bool has_mask = p->mask != nullptr;
  if ((p->bias == nullptr) == !has_mask || ranges == nullptr || p->cu_seqlens_q == nullptr ||
      p->cu_seqlens_kv == nullptr)
    return fail(MI_ATTN_ERR_INVALID_ARG,
                "a bias or a mask (one of them), ranges and both cu_seqlens are required");
  if (p->hq <= 0 || (p->bias_heads != 1 && p->bias_heads != p->hq))
    return fail(MI_ATTN_ERR_UNSUPPORTED, "bias_heads must be 1 or hq (got %d, hq %d)",
                p->bias_heads, p->hq);
  if (has_mask ? ((reinterpret_cast<uintptr_t>(p->mask) & 3u) != 0)
               : !aligned16(p->bias))
    return fail(MI_ATTN_ERR_INVALID_ARG, "bias must be 16-byte aligned, a mask 4-byte aligned");
  if (p->bias_stride_tok < 0 || p->bias_stride_head < 0 || p->bias_stride_tok % 4 != 0 ||
      p->bias_stride_head % 4 != 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "bias / mask strides must be multiples of 4");
  if ((reinterpret_cast<uintptr_t>(ranges) & 7u) != 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "ranges must be 8-byte aligned");
  if (p->bias_cols <= 0) return fail(MI_ATTN_ERR_INVALID_ARG, "bias_cols must be > 0");
  if (p->num_seqs < 0 || p->max_seqlen_q < 0 || p->total_q < 0)
    return fail(MI_ATTN_ERR_INVALID_ARG, "negative size");
  if (p->num_seqs == 0 || p->max_seqlen_q == 0 || p->total_q == 0) return MI_ATTN_OK;
  if (p->num_seqs > 65535 || (p->max_seqlen_q + 3) / 4 > INT32_MAX || p->total_q > INT32_MAX)
    return fail(MI_ATTN_ERR_UNSUPPORTED, "too many sequences (at most 65535) or rows");
  if (env_flag("MI_ATTN_VALIDATE")) {
    int rc = validate_cu(p->cu_seqlens_q, p->num_seqs, p->total_q, p->max_seqlen_q, "cu_seqlens_q");
    if (rc != MI_ATTN_OK) return rc;
  }
  mi_attn::BiasRangeArgs a{};
  a.bias = p->bias;
  a.mask = p->mask;
  a.cu_q = p->cu_seqlens_q;
  a.cu_kv = p->cu_seqlens_kv;
  a.ranges = ranges;
  a.pure = const_cast<uint8_t*>(p->bias_pure);  // an output here
  a.b_st = p->bias_stride_tok;
  a.b_sh = p->bias_stride_head;
  a.total_q = p->total_q;
  a.bias_cols = (int32_t)(p->bias_cols < INT32_MAX ? p->bias_cols : INT32_MAX);
  hipError_t e = mi_attn::launch_bias_key_ranges(a, (int)p->max_seqlen_q, (int)p->num_seqs,
                                                  p->bias_heads, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MI_ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return MI_ATTN_OK;
}

}  // extern "C"
