"""Fused variable-length attention forward for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/mi_attn.h``
(``libmi_attn.so``, built in-tree by ``flash_attention_varlen_amd.build``).
PyTorch supplies device memory and the stream; every step of the attention
runs in the library's HIP kernels.  There is no fallback: if the library is
missing or refuses a call, an exception is raised.

``varlen_attention`` mirrors the call on the mtlattn 0.3.0 project page
(section "Use"): q, k, v packed ``[total_tokens, heads, head_dim]``,
``cu_seqlens_*`` int32 ``[num_seqs + 1]``, ``max_seqlen_q``, ``scale``
(default ``1/sqrt(head_dim)``), ``causal`` (end-aligned), ``window``
(last W keys up to the causal diagonal), ``attn_bias`` (additive fp32
``[total_q, H or 1, max_kv]``, a bool mask becomes 0 / -inf).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["mi_attn_varlen_fwd", "mi_attn_varlen_bwd", "mi_attn_last_error", "mi_attn_version",
           "mi_attn_tile_shape", "mi_attn_bias_key_ranges", "bias_key_ranges", "varlen_attention",
           "varlen_attention_backward", "varlen_decode", "mi_attn_varlen_decode",
           "mi_attn_decode_workspace_size", "MiAttnBwdParams", "flash_attn_varlen_qkvpacked_func",
           "flash_attn_varlen_kvpacked_func", "varlen_decode_noalloc",
           "mi_attn_varlen_decode_noalloc", "MiAttnFwdParams", "MiAttnError", "load_library", "LIB_PATH",
           "F32", "F16", "BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi_attn.so")

# dtype codes and return codes of include/mi_attn.h
F32, F16, BF16 = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_VALIDATION = 0, -1, -2, -3, -4


class MiAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"mi_attn error {code}: {message}")
        self.code = code


class MiAttnFwdParams(ctypes.Structure):
    """Field-for-field mirror of ``mi_attn_fwd_params``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_kv", ctypes.c_void_p),
        ("bias", ctypes.c_void_p), ("tile_counts", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int64), ("max_seqlen_q", ctypes.c_int64),
        ("total_q", ctypes.c_int64), ("total_kv", ctypes.c_int64),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_tok", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("out_stride_tok", ctypes.c_int64), ("out_stride_head", ctypes.c_int64),
        ("bias_heads", ctypes.c_int32), ("bias_cols", ctypes.c_int64),
        ("bias_stride_tok", ctypes.c_int64), ("bias_stride_head", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("bias_ranges", ctypes.c_void_p),
        ("q_rope", ctypes.c_void_p), ("k_rope", ctypes.c_void_p),
        ("q_rope_stride_tok", ctypes.c_int64), ("q_rope_stride_head", ctypes.c_int64),
        ("k_rope_stride_tok", ctypes.c_int64), ("k_rope_stride_head", ctypes.c_int64),
        ("alibi_slopes", ctypes.c_void_p), ("alibi_stride_seq", ctypes.c_int64),
        ("mask", ctypes.c_void_p),
        ("bias_pure", ctypes.c_void_p),
        ("seqused_q", ctypes.c_void_p), ("seqused_kv", ctypes.c_void_p),
    ]


class MiAttnBwdParams(ctypes.Structure):
    """Field-for-field mirror of ``mi_attn_bwd_params``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("dout", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("delta", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_kv", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int64), ("max_seqlen_q", ctypes.c_int64),
        ("max_seqlen_kv", ctypes.c_int64), ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_tok", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("out_stride_tok", ctypes.c_int64), ("out_stride_head", ctypes.c_int64),
        ("dout_stride_tok", ctypes.c_int64), ("dout_stride_head", ctypes.c_int64),
        ("dq_stride_tok", ctypes.c_int64), ("dq_stride_head", ctypes.c_int64),
        ("dk_stride_tok", ctypes.c_int64), ("dk_stride_head", ctypes.c_int64),
        ("dv_stride_tok", ctypes.c_int64), ("dv_stride_head", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("bias", ctypes.c_void_p), ("bias_heads", ctypes.c_int32), ("bias_cols", ctypes.c_int64),
        ("bias_stride_tok", ctypes.c_int64), ("bias_stride_head", ctypes.c_int64),
        ("alibi_slopes", ctypes.c_void_p), ("alibi_stride_seq", ctypes.c_int64),
    ]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmi_attn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing; build it with `python -m flash_attention_varlen_amd.build`")
    lib = ctypes.CDLL(p)
    lib.mi_attn_varlen_fwd.argtypes = [ctypes.POINTER(MiAttnFwdParams), ctypes.c_void_p]
    lib.mi_attn_varlen_fwd.restype = ctypes.c_int
    lib.mi_attn_last_error.argtypes = []
    lib.mi_attn_last_error.restype = ctypes.c_char_p
    lib.mi_attn_version.argtypes = []
    lib.mi_attn_version.restype = ctypes.c_int
    lib.mi_attn_tile_shape.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.mi_attn_tile_shape.restype = ctypes.c_int
    lib.mi_attn_bias_key_ranges.argtypes = [ctypes.POINTER(MiAttnFwdParams), ctypes.c_void_p,
                                            ctypes.c_void_p]
    lib.mi_attn_bias_key_ranges.restype = ctypes.c_int
    lib.mi_attn_varlen_bwd.argtypes = [ctypes.POINTER(MiAttnBwdParams), ctypes.c_void_p]
    lib.mi_attn_varlen_bwd.restype = ctypes.c_int
    lib.mi_attn_decode_workspace_size.argtypes = [ctypes.POINTER(MiAttnFwdParams), ctypes.c_int64,
                                                  ctypes.c_int32]
    lib.mi_attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.mi_attn_varlen_decode.argtypes = [ctypes.POINTER(MiAttnFwdParams), ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]
    lib.mi_attn_varlen_decode.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def variant_library(name: str) -> ctypes.CDLL:
    """A schedule variant of the library (``slots2``, ``synccopies``, ``shallow``), built
    beside it for the LDS race check; its results must equal the shipping
    library's bit for bit."""
    from .build import variant_path
    return load_library(variant_path(name))


def mi_attn_last_error() -> str:
    return load_library().mi_attn_last_error().decode()


def mi_attn_version() -> int:
    return int(load_library().mi_attn_version())


def mi_attn_tile_shape(in_dtype: int, d_qk: int, d_v: int):
    """(BM, BN) of the kernel for this dtype and head dims."""
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    rc = load_library().mi_attn_tile_shape(in_dtype, d_qk, d_v, ctypes.byref(bm), ctypes.byref(bn))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())
    return bm.value, bn.value


def mi_attn_varlen_fwd(params: MiAttnFwdParams, stream: int = 0) -> None:
    """Call the C entry point; raise MiAttnError on a non-OK return."""
    params.struct_size = ctypes.sizeof(MiAttnFwdParams)
    rc = load_library().mi_attn_varlen_fwd(ctypes.byref(params), ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


def mi_attn_varlen_bwd(params: MiAttnBwdParams, stream: int = 0) -> None:
    """Call the C entry point; raise MiAttnError on a non-OK return."""
    params.struct_size = ctypes.sizeof(MiAttnBwdParams)
    rc = load_library().mi_attn_varlen_bwd(ctypes.byref(params), ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


def mi_attn_decode_workspace_size(params: MiAttnFwdParams, max_seqlen_kv: int, num_splits: int = 0) -> int:
    """Workspace bytes mi_attn_varlen_decode needs (0: nothing to compute, or refused)."""
    params.struct_size = ctypes.sizeof(MiAttnFwdParams)
    return int(load_library().mi_attn_decode_workspace_size(ctypes.byref(params), max_seqlen_kv,
                                                            num_splits))


def mi_attn_varlen_decode(params: MiAttnFwdParams, max_seqlen_kv: int, num_splits: int,
                          workspace_ptr: int, workspace_bytes: int, stream: int = 0) -> None:
    """Call the C entry point; raise MiAttnError on a non-OK return."""
    params.struct_size = ctypes.sizeof(MiAttnFwdParams)
    rc = load_library().mi_attn_varlen_decode(ctypes.byref(params), max_seqlen_kv, num_splits,
                                              ctypes.c_void_p(workspace_ptr), workspace_bytes,
                                              ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


def mi_attn_bias_key_ranges(params: MiAttnFwdParams, ranges_ptr: int, stream: int = 0) -> None:
    """Call the C entry point; raise MiAttnError on a non-OK return."""
    params.struct_size = ctypes.sizeof(MiAttnFwdParams)
    rc = load_library().mi_attn_bias_key_ranges(ctypes.byref(params), ctypes.c_void_p(ranges_ptr),
                                                ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


# ---------------------------------------------------------------- torch front end
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t not in codes:
        raise MiAttnError(ERR_UNSUPPORTED, f"dtype {t} is not supported (fp32, fp16, bf16)")
    return codes[t]


def varlen_attention(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int,
                     scale: Optional[float] = None, causal: bool = False, window: int = 0,
                     attn_bias=None, out_dtype=None, return_lse: bool = False, out=None,
                     lse=None, tile_counts=None, stream=None, bias_ranges=None,
                     max_seqlen_kv=None, q_rope=None, k_rope=None, alibi_slopes=None,
                     bias_pure=None, seqused_q=None, seqused_kv=None):
    """Fused varlen attention forward.  Returns ``out`` or ``(out, lse)``.

    q ``[Tq, Hq, Dqk]``, k ``[Tk, Hkv, Dqk]``, v ``[Tk, Hkv, Dv]`` (device,
    last dim contiguous, any token / head strides the C ABI accepts);
    ``out`` is ``[Tq, Hq, Dv]`` in ``out_dtype`` (default: q's dtype;
    ``torch.float32`` is also accepted); ``lse`` is ``[Hq, Tq]`` fp32
    (natural log).  If q, k or v require grad (and grad mode is on), the call
    is differentiable: ``out``'s gradient flows back through
    ``mi_attn_varlen_bwd`` (bf16 / fp16, head dims 64 / 96 / 128;
    ``max_seqlen_kv`` is read from ``cu_seqlens_kv`` when not given; a bias
    enters as a constant, and one that requires grad is refused).

    ``stream`` (a ``torch.cuda.Stream``, a raw ``hipStream_t`` handle, or
    None for the current stream) is where the kernel runs; outputs and the
    converted bias are allocated on it too.  The caller orders the inputs'
    producers before it.  A bool ``attn_bias`` (True = visible) becomes a
    byte mask that the kernels read directly (copied, last dim padded to a
    multiple of 4, only when its strides are not multiples of 4); an fp32
    bias whose strides are not multiples of 4 elements is copied into such a
    layout.  (The differentiable path turns a bool mask into the fp32 0 /
    -inf bias the backward reads.)  ``bias_ranges`` (from ``bias_key_ranges`` on the same
    bias) lets the kernels skip key tiles that are -inf for all their rows;
    ``bias_pure`` (from ``bias_key_ranges(..., return_pure=True)``, with those
    ranges) lets them mask rows that are plain key intervals instead of
    reading their bias.

    Latent-attention head: with ``q_rope`` ``[Tq, Hq, 64]`` and ``k_rope``
    ``[Tk, Hkv, 64]`` (bf16 / fp16, ``v`` 128 wide), q and k are the 128-wide
    nope parts and the scores are ``q.k + q_rope.k_rope``, as for one call on
    the concatenations, without forming them (forward only).

    ``alibi_slopes`` (fp32 ``[Hq]`` or ``[num_seqs, Hq]``, device): the
    kernels add ``-slope * |i + (Lk - Lq) - j|`` to the logit of query row i
    and key j (no bias tensor with it); differentiable like a bias.

    ``seqused_q`` / ``seqused_kv`` (int32 ``[num_seqs]``, device): sequence s
    uses only the first ``seqused[s]`` rows of its span (a right-padded batch
    with spans of the padded length); rows of ``out`` past ``seqused_q`` are
    0 and their ``lse`` -inf (forward only).
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise MiAttnError(ERR_INVALID_ARG, f"{name} must be a device tensor")
        if t.dim() != 3 or t.stride(-1) != 1:
            raise MiAttnError(ERR_INVALID_ARG, f"{name} must be [tokens, heads, dim], last dim contiguous")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise MiAttnError(ERR_INVALID_ARG, "q, k and v must share one dtype")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if t.dtype != torch.int32 or not t.is_cuda or t.dim() != 1 or not t.is_contiguous():
            raise MiAttnError(ERR_INVALID_ARG, f"{name} must be a contiguous int32 device vector")
    if cu_seqlens_q.numel() != cu_seqlens_kv.numel():
        raise MiAttnError(ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_kv differ in length")
    tq, hq, dqk = q.shape
    tk, hkv, _ = k.shape
    dv = v.shape[2]
    if k.shape[2] != dqk or v.shape[0] != tk or v.shape[1] != hkv:
        raise MiAttnError(ERR_INVALID_ARG, "k/v shapes do not match q")
    if (q_rope is None) != (k_rope is None):
        raise MiAttnError(ERR_INVALID_ARG, "q_rope and k_rope go together")
    if q_rope is not None:
        for name, t, rows, heads in (("q_rope", q_rope, tq, hq), ("k_rope", k_rope, tk, hkv)):
            if (not t.is_cuda or t.dtype != q.dtype or t.dim() != 3 or t.stride(-1) != 1
                    or tuple(t.shape) != (rows, heads, 64)):
                raise MiAttnError(ERR_INVALID_ARG, f"{name} must be [{rows}, {heads}, 64] "
                                                   f"{q.dtype}, last dim contiguous")
        if torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v, q_rope, k_rope)):
            raise MiAttnError(ERR_UNSUPPORTED, "split q_rope / k_rope operands are forward only")
        dqk = dqk + 64  # the contraction width
    if alibi_slopes is not None:
        nseq = cu_seqlens_q.numel() - 1
        if (alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_cuda
                or alibi_slopes.stride(-1) != 1
                or tuple(alibi_slopes.shape) not in ((hq,), (nseq, hq))):
            raise MiAttnError(ERR_INVALID_ARG, "alibi_slopes must be fp32 [Hq] or [num_seqs, Hq] "
                                               "on the device, last dim contiguous")
        if attn_bias is not None:
            raise MiAttnError(ERR_UNSUPPORTED, "alibi_slopes and attn_bias together")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if torch.is_grad_enabled() and (q.requires_grad or k.requires_grad or v.requires_grad):
        # differentiable path (mtlattn page, "Drop-in for scaled_dot_product_attention":
        # inputs that require grad route through the backward kernel)
        if attn_bias is not None and attn_bias.requires_grad:
            raise MiAttnError(ERR_UNSUPPORTED, "the bias is a constant: a bias that requires grad "
                                               "is refused")
        if seqused_q is not None or seqused_kv is not None:
            raise MiAttnError(ERR_UNSUPPORTED, "seqused_q / seqused_kv are forward only")
        if out_dtype != q.dtype or q.dtype == torch.float32 or out is not None or \
                lse is not None or tile_counts is not None:
            raise MiAttnError(ERR_UNSUPPORTED,
                              "the differentiable path takes bf16/fp16 inputs, the default output "
                              "dtype and no preallocated outputs")
        s_obj = _stream_of(stream, q.device)
        with torch.cuda.stream(s_obj):
            o, l = _differentiable_attention(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
                                             max_seqlen_kv, scale, causal, window, attn_bias,
                                             alibi_slopes)
        return (o, l) if return_lse else o
    s_obj = _stream_of(stream, q.device)
    for name, t in (("seqused_q", seqused_q), ("seqused_kv", seqused_kv)):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()
                              or tuple(t.shape) != (cu_seqlens_q.numel() - 1,)):
            raise MiAttnError(ERR_INVALID_ARG, f"{name} must be a contiguous int32 [num_seqs] "
                                               "device tensor")
    if bias_ranges is not None:
        if attn_bias is None:
            raise MiAttnError(ERR_INVALID_ARG, "bias_ranges needs the attn_bias it was computed from")
        if (bias_ranges.dtype != torch.int32 or not bias_ranges.is_contiguous()
                or bias_ranges.shape != (attn_bias.shape[1], tq, 2)):
            raise MiAttnError(ERR_INVALID_ARG, "bias_ranges must be contiguous int32 [H_b, Tq, 2]")
    if bias_pure is not None:
        if bias_ranges is None:
            raise MiAttnError(ERR_INVALID_ARG, "bias_pure needs the bias_ranges it was computed with")
        if (bias_pure.dtype != torch.uint8 or not bias_pure.is_contiguous()
                or bias_pure.shape != (attn_bias.shape[1], tq)):
            raise MiAttnError(ERR_INVALID_ARG, "bias_pure must be contiguous uint8 [H_b, Tq]")
    with torch.cuda.stream(s_obj):
        return _varlen_attention_on_stream(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
                                           scale, causal, window, attn_bias, out_dtype,
                                           return_lse, out, lse, tile_counts, s_obj, tq, hq, dqk,
                                           tk, hkv, dv, bias_ranges, q_rope, k_rope,
                                           alibi_slopes, bias_pure, seqused_q, seqused_kv)


def _stream_of(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def bias_key_ranges(attn_bias, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int, stream=None,
                    return_pure: bool = False):
    """int32 ``[H_b, Tq, 2]``: for each bias row, the first and one-past-last
    key of its sequence whose bias is not -inf (``[0, 0)`` if none).  Pass the
    result as ``bias_ranges`` to ``varlen_attention`` with the same bias: the
    kernels then skip, exactly, key tiles whose bias is -inf for all their
    rows.  Valid for as long as the bias and cu_seqlens are.

    With ``return_pure`` also uint8 ``[H_b, Tq]``, 1 for the rows that are
    plain key intervals (bias exactly 0 on the range, -inf elsewhere; for a
    bool mask, True exactly on the range): returns ``(ranges, pure)``, to be
    passed as ``bias_ranges`` and ``bias_pure``."""
    import torch
    if attn_bias.dim() != 3 or not attn_bias.is_cuda or attn_bias.stride(-1) != 1:
        raise MiAttnError(ERR_INVALID_ARG, "attn_bias must be [Tq, H or 1, max_kv] on device")
    s_obj = _stream_of(stream, attn_bias.device)
    with torch.cuda.stream(s_obj):
        if attn_bias.dtype == torch.bool:
            bias = _aligned_mask(attn_bias)
        elif attn_bias.dtype == torch.float32:
            bias = _aligned_bias(attn_bias)
        else:
            raise MiAttnError(ERR_INVALID_ARG, "attn_bias must be fp32 or bool")
        tq, hb, cols = bias.shape
        ranges = torch.empty(hb, tq, 2, dtype=torch.int32, device=bias.device)
        pure = torch.empty(hb, tq, dtype=torch.uint8, device=bias.device) if return_pure else None
        p = MiAttnFwdParams()
        p.bias_pure = pure.data_ptr() if pure is not None else None
        if bias.dtype == torch.uint8:
            p.mask = bias.data_ptr()
        else:
            p.bias = bias.data_ptr()
        p.cu_seqlens_q, p.cu_seqlens_kv = cu_seqlens_q.data_ptr(), cu_seqlens_kv.data_ptr()
        p.num_seqs = cu_seqlens_q.numel() - 1
        p.max_seqlen_q = int(max_seqlen_q)
        p.total_q = tq
        p.hq = hb
        p.bias_heads = hb
        p.bias_cols = cols
        p.bias_stride_tok, p.bias_stride_head = bias.stride(0), bias.stride(1)
        mi_attn_bias_key_ranges(p, ranges.data_ptr(), int(s_obj.cuda_stream))
    return (ranges, pure) if return_pure else ranges


def _aligned_mask(mask):
    """uint8 view [Tq, H, C] of a bool mask (True = visible) whose strides are
    multiples of 4 bytes and whose data is 4-byte aligned; copied into such a
    layout (last dim padded to a multiple of 4) when it is not one."""
    import torch
    m = mask.view(torch.uint8)
    if m.stride(-1) == 1 and m.stride(0) % 4 == 0 and m.stride(1) % 4 == 0 and \
            m.data_ptr() % 4 == 0:
        return m
    cols = m.shape[2]
    buf = torch.zeros(m.shape[0], m.shape[1], (cols + 3) // 4 * 4, dtype=torch.uint8,
                      device=m.device)
    view = buf[:, :, :cols]
    view.copy_(m)
    return view


def _aligned_bias(bias):
    """fp32 [Tq, H, C] with strides that are multiples of 4 elements, from a
    bool mask (True = visible -> 0, False -> -inf) or an fp32 bias."""
    import torch
    cols = bias.shape[2]
    if bias.dtype == torch.bool:
        buf = torch.empty(bias.shape[0], bias.shape[1], (cols + 3) // 4 * 4, dtype=torch.float32,
                          device=bias.device)
        view = buf[:, :, :cols]
        view.zero_().masked_fill_(~bias, float("-inf"))
        return view
    if bias.stride(0) % 4 == 0 and bias.stride(1) % 4 == 0 and bias.data_ptr() % 16 == 0:
        return bias
    buf = torch.empty(bias.shape[0], bias.shape[1], (cols + 3) // 4 * 4, dtype=torch.float32,
                      device=bias.device)
    view = buf[:, :, :cols]
    view.copy_(bias)
    return view


def _varlen_attention_on_stream(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, scale, causal,
                                window, attn_bias, out_dtype, return_lse, out, lse, tile_counts,
                                s_obj, tq, hq, dqk, tk, hkv, dv, bias_ranges=None, q_rope=None,
                                k_rope=None, alibi_slopes=None, bias_pure=None, seqused_q=None,
                                seqused_kv=None):
    import torch
    bias = attn_bias
    if bias is not None:
        if (bias.dtype not in (torch.float32, torch.bool) or bias.dim() != 3
                or bias.stride(-1) != 1 or not bias.is_cuda):
            raise MiAttnError(ERR_INVALID_ARG,
                              "attn_bias must be fp32 or bool [Tq, H or 1, max_kv] on device")
        if bias.shape[0] != tq or bias.shape[1] not in (1, hq):
            raise MiAttnError(ERR_INVALID_ARG, "attn_bias must be [Tq, H or 1, max_kv]")
        # a bool mask goes to the kernels as bytes; an fp32 bias as it is
        bias = _aligned_mask(bias) if bias.dtype == torch.bool else _aligned_bias(bias)
    if out is None:
        out = torch.empty(tq, hq, dv, dtype=out_dtype, device=q.device)
    elif out.shape != (tq, hq, dv) or out.dtype != out_dtype or out.stride(-1) != 1:
        raise MiAttnError(ERR_INVALID_ARG, "out has the wrong shape, dtype or layout")
    if return_lse and lse is None:
        lse = torch.empty(hq, tq, dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (hq, tq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise MiAttnError(ERR_INVALID_ARG, "lse must be a contiguous fp32 [Hq, Tq] tensor")

    p = MiAttnFwdParams()
    p.q, p.k, p.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    p.out = out.data_ptr()
    p.lse = lse.data_ptr() if lse is not None else None
    p.cu_seqlens_q, p.cu_seqlens_kv = cu_seqlens_q.data_ptr(), cu_seqlens_kv.data_ptr()
    if bias is not None and bias.dtype == torch.uint8:
        p.mask = bias.data_ptr()
    else:
        p.bias = bias.data_ptr() if bias is not None else None
    p.bias_ranges = bias_ranges.data_ptr() if bias_ranges is not None else None
    p.bias_pure = bias_pure.data_ptr() if bias_pure is not None else None
    p.seqused_q = seqused_q.data_ptr() if seqused_q is not None else None
    p.seqused_kv = seqused_kv.data_ptr() if seqused_kv is not None else None
    if q_rope is not None:
        p.q_rope, p.k_rope = q_rope.data_ptr(), k_rope.data_ptr()
        p.q_rope_stride_tok, p.q_rope_stride_head = q_rope.stride(0), q_rope.stride(1)
        p.k_rope_stride_tok, p.k_rope_stride_head = k_rope.stride(0), k_rope.stride(1)
    if alibi_slopes is not None:
        p.alibi_slopes = alibi_slopes.data_ptr()
        p.alibi_stride_seq = alibi_slopes.stride(0) if alibi_slopes.dim() == 2 else 0
    p.tile_counts = tile_counts.data_ptr() if tile_counts is not None else None
    p.num_seqs = cu_seqlens_q.numel() - 1
    p.max_seqlen_q = int(max_seqlen_q)
    p.total_q, p.total_kv = tq, tk
    p.hq, p.hkv, p.d_qk, p.d_v = hq, hkv, dqk, dv
    p.q_stride_tok, p.q_stride_head = q.stride(0), q.stride(1)
    p.k_stride_tok, p.k_stride_head = k.stride(0), k.stride(1)
    p.v_stride_tok, p.v_stride_head = v.stride(0), v.stride(1)
    p.out_stride_tok, p.out_stride_head = out.stride(0), out.stride(1)
    if bias is not None:
        p.bias_heads = bias.shape[1]
        p.bias_cols = bias.shape[2]
        p.bias_stride_tok, p.bias_stride_head = bias.stride(0), bias.stride(1)
    p.in_dtype = _dtype_code(q.dtype)
    p.out_dtype = _dtype_code(out_dtype)
    p.scale = float(scale)
    p.causal = 1 if causal else 0
    p.window = int(window)
    mi_attn_varlen_fwd(p, int(s_obj.cuda_stream))
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------- backward
def varlen_attention_backward(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_kv,
                              max_seqlen_q: int, max_seqlen_kv: int, scale: Optional[float] = None,
                              causal: bool = False, window: int = 0, dq=None, dk=None, dv=None,
                              grad_dtype=None, attn_bias=None, stream=None, alibi_slopes=None):
    """Gradients ``(dq, dk, dv)`` of the forward from its inputs, its output
    ``out`` and ``lse`` and the output gradient ``dout`` (bf16 / fp16,
    head dims 64, 96 or 128; ``attn_bias``, the forward's additive bias, enters as
    a constant).  Outputs (and the fp32 [Hq, Tq] delta workspace) are
    allocated on ``stream`` unless given."""
    import torch
    tq, hq, dqk = q.shape
    tk, hkv, _ = k.shape
    dvd = v.shape[2]
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != (tq, hq, dvd) or t.dtype != q.dtype or t.stride(-1) != 1:
            raise MiAttnError(ERR_INVALID_ARG, f"{name} must be [Tq, Hq, Dv] in q's dtype")
    if lse.shape != (hq, tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise MiAttnError(ERR_INVALID_ARG, "lse must be a contiguous fp32 [Hq, Tq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    s_obj = _stream_of(stream, q.device)
    with torch.cuda.stream(s_obj):
        gdt = q.dtype if grad_dtype is None else grad_dtype
        dq = torch.empty(q.shape, dtype=gdt, device=q.device) if dq is None else dq
        dk = torch.empty(k.shape, dtype=gdt, device=q.device) if dk is None else dk
        dv = torch.empty(v.shape, dtype=gdt, device=q.device) if dv is None else dv
        for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            if t.shape != ref.shape or t.dtype != gdt or t.stride(-1) != 1:
                raise MiAttnError(ERR_INVALID_ARG, f"{name} has the wrong shape, dtype or layout")
        delta = torch.empty(hq, tq, dtype=torch.float32, device=q.device)
        p = MiAttnBwdParams()
        p.q, p.k, p.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
        p.out, p.lse, p.dout = out.data_ptr(), lse.data_ptr(), dout.data_ptr()
        p.dq, p.dk, p.dv, p.delta = dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr()
        p.cu_seqlens_q, p.cu_seqlens_kv = cu_seqlens_q.data_ptr(), cu_seqlens_kv.data_ptr()
        p.num_seqs = cu_seqlens_q.numel() - 1
        p.max_seqlen_q, p.max_seqlen_kv = int(max_seqlen_q), int(max_seqlen_kv)
        p.total_q, p.total_kv = tq, tk
        p.hq, p.hkv, p.d_qk, p.d_v = hq, hkv, dqk, dvd
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq),
                        ("dk", dk), ("dv", dv)):
            setattr(p, f"{name}_stride_tok", t.stride(0))
            setattr(p, f"{name}_stride_head", t.stride(1))
        if attn_bias is not None:
            bias = _aligned_bias(attn_bias)
            p.bias = bias.data_ptr()
            p.bias_heads, p.bias_cols = bias.shape[1], bias.shape[2]
            p.bias_stride_tok, p.bias_stride_head = bias.stride(0), bias.stride(1)
        if alibi_slopes is not None:
            p.alibi_slopes = alibi_slopes.data_ptr()
            p.alibi_stride_seq = alibi_slopes.stride(0) if alibi_slopes.dim() == 2 else 0
        p.in_dtype = _dtype_code(q.dtype)
        p.grad_dtype = _dtype_code(gdt)
        p.scale = float(scale)
        p.causal = 1 if causal else 0
        p.window = int(window)
        mi_attn_varlen_bwd(p, int(s_obj.cuda_stream))
    return dq, dk, dv


def _autograd_fn():
    import torch

    class VarlenAttentionFn(torch.autograd.Function):
        """Forward through mi_attn_varlen_fwd, backward through
        mi_attn_varlen_bwd (the lse output is not differentiated)."""

        @staticmethod
        def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, scale,
                    causal, window, bias, alibi):
            with torch.no_grad():
                if bias is not None:
                    bias = _aligned_bias(bias)  # one fp32 layout for both passes
                out, lse = varlen_attention(q.detach(), k.detach(), v.detach(), cu_seqlens_q,
                                            cu_seqlens_kv, max_seqlen_q, scale=scale, causal=causal,
                                            window=window, attn_bias=bias, return_lse=True,
                                            alibi_slopes=alibi)
            ctx.bias = bias
            ctx.alibi = alibi
            ctx.save_for_backward(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_kv)
            ctx.args = (max_seqlen_q, max_seqlen_kv, scale, causal, window)
            ctx.mark_non_differentiable(lse)
            return out, lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            q, k, v, out, lse, cq, ck = ctx.saved_tensors
            max_seqlen_q, max_seqlen_kv, scale, causal, window = ctx.args
            dq, dk, dv = varlen_attention_backward(q, k, v, out, lse, dout.contiguous(), cq, ck,
                                                   max_seqlen_q, max_seqlen_kv, scale, causal,
                                                   window, attn_bias=ctx.bias,
                                                   alibi_slopes=ctx.alibi)
            return dq, dk, dv, None, None, None, None, None, None, None, None, None

    return VarlenAttentionFn


_FN = None


def _differentiable_attention(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                              scale, causal, window, bias=None, alibi=None):
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    if max_seqlen_kv is None:
        max_seqlen_kv = int((cu_seqlens_kv[1:] - cu_seqlens_kv[:-1]).max().item()) \
            if cu_seqlens_kv.numel() > 1 else 0
    return _FN.apply(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, scale,
                     causal, window, bias, alibi)


# ---------------------------------------------------------------- split-KV decode
def _fwd_params(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, scale, causal, window, out,
                lse, out_dtype):
    p = MiAttnFwdParams()
    tq, hq, dqk = q.shape
    tk, hkv, _ = k.shape
    p.q, p.k, p.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    p.out = out.data_ptr()
    p.lse = lse.data_ptr() if lse is not None else None
    p.cu_seqlens_q, p.cu_seqlens_kv = cu_seqlens_q.data_ptr(), cu_seqlens_kv.data_ptr()
    p.num_seqs = cu_seqlens_q.numel() - 1
    p.max_seqlen_q = int(max_seqlen_q)
    p.total_q, p.total_kv = tq, tk
    p.hq, p.hkv, p.d_qk, p.d_v = hq, hkv, dqk, v.shape[2]
    p.q_stride_tok, p.q_stride_head = q.stride(0), q.stride(1)
    p.k_stride_tok, p.k_stride_head = k.stride(0), k.stride(1)
    p.v_stride_tok, p.v_stride_head = v.stride(0), v.stride(1)
    p.out_stride_tok, p.out_stride_head = out.stride(0), out.stride(1)
    p.in_dtype = _dtype_code(q.dtype)
    p.out_dtype = _dtype_code(out_dtype)
    p.scale = float(scale)
    p.causal = 1 if causal else 0
    p.window = int(window)
    return p


def varlen_decode(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int, max_seqlen_kv: int,
                  scale: Optional[float] = None, causal: bool = False, window: int = 0,
                  num_splits: int = 0, out_dtype=None, return_lse: bool = False, out=None,
                  lse=None, workspace=None, stream=None, seqused_kv=None):
    """Split-KV decode (``mi_attn_varlen_decode``): the forward for few query
    rows per sequence against long key/value caches.  Same arguments and
    results as ``varlen_attention`` (bf16 / fp16, head dims 64 / 128, no
    bias), plus ``max_seqlen_kv``, ``num_splits`` (0 = auto), an optional
    preallocated uint8 ``workspace`` (else allocated on the stream) and
    ``seqused_kv`` (int32 ``[num_seqs]``: the keys in use of each sequence's
    cache span)."""
    import torch
    tq, hq, dqk = q.shape
    dv = v.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    s_obj = _stream_of(stream, q.device)
    with torch.cuda.stream(s_obj):
        if out is None:
            out = torch.empty(tq, hq, dv, dtype=out_dtype, device=q.device)
        if return_lse and lse is None:
            lse = torch.empty(hq, tq, dtype=torch.float32, device=q.device)
        p = _fwd_params(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, scale, causal, window,
                        out, lse, out_dtype)
        if seqused_kv is not None:
            if (seqused_kv.dtype != torch.int32 or not seqused_kv.is_contiguous()
                    or tuple(seqused_kv.shape) != (cu_seqlens_q.numel() - 1,)):
                raise MiAttnError(ERR_INVALID_ARG, "seqused_kv must be a contiguous int32 "
                                                   "[num_seqs] device tensor")
            p.seqused_kv = seqused_kv.data_ptr()
        need = mi_attn_decode_workspace_size(p, int(max_seqlen_kv), int(num_splits))
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        mi_attn_varlen_decode(p, int(max_seqlen_kv), int(num_splits), workspace.data_ptr(),
                              workspace.numel(), int(s_obj.cuda_stream))
    return (out, lse) if return_lse else out


def mi_attn_varlen_decode_noalloc(params: MiAttnFwdParams, max_seqlen_kv: int, num_splits: int,
                                  stream: int = 0) -> None:
    """Call the non-allocating decode entry point; raise MiAttnError on a non-OK return."""
    lib = load_library()
    fn = lib.mi_attn_varlen_decode_noalloc
    fn.argtypes = [ctypes.POINTER(MiAttnFwdParams), ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    params.struct_size = ctypes.sizeof(MiAttnFwdParams)
    rc = fn(ctypes.byref(params), max_seqlen_kv, num_splits, ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


def varlen_decode_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int,
                          max_seqlen_kv: int, out, lse=None, scale: Optional[float] = None,
                          causal: bool = False, window: int = 0, num_splits: int = 0,
                          stream=None):
    """``varlen_decode`` through ``mi_attn_varlen_decode_noalloc``: the caller
    passes ``out`` (and ``lse``); the library allocates nothing (its workspace
    is a fixed device array, so calls that overlap on one GPU race)."""
    import torch
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    s_obj = _stream_of(stream, q.device)
    p = _fwd_params(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, scale, causal, window, out,
                    lse, out.dtype)
    mi_attn_varlen_decode_noalloc(p, int(max_seqlen_kv), int(num_splits), int(s_obj.cuda_stream))
    return out


# ---------------------------------------------------------------- packed layouts
def flash_attn_varlen_qkvpacked_func(qkv, cu_seqlens, max_seqlen: int, scale: Optional[float] = None,
                                     causal: bool = False, window: int = 0, attn_bias=None,
                                     return_lse: bool = False, out_dtype=None, stream=None):
    """Self-attention on a packed ``[T, 3, H, D]`` tensor (q, k, v along dim 1),
    the wrapper the mtlattn 0.3.0 page lists in section "Use".  The three
    views go to the C ABI as they are (token stride 3 H D, no copy);
    differentiable like ``varlen_attention`` (the gradient lands in ``qkv``)."""
    if qkv.dim() != 4 or qkv.shape[1] != 3:
        raise MiAttnError(ERR_INVALID_ARG, "qkv must be [T, 3, H, D]")
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    return varlen_attention(q, k, v, cu_seqlens, cu_seqlens, max_seqlen, scale=scale,
                            causal=causal, window=window, attn_bias=attn_bias,
                            return_lse=return_lse, out_dtype=out_dtype, stream=stream,
                            max_seqlen_kv=max_seqlen)


def flash_attn_varlen_kvpacked_func(q, kv, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int,
                                    max_seqlen_kv: int, scale: Optional[float] = None,
                                    causal: bool = False, window: int = 0, attn_bias=None,
                                    return_lse: bool = False, out_dtype=None, stream=None):
    """Attention with k and v packed as ``[Tk, 2, Hkv, D]`` (mtlattn 0.3.0
    page, section "Use"); views, no copy; differentiable."""
    if kv.dim() != 4 or kv.shape[1] != 2:
        raise MiAttnError(ERR_INVALID_ARG, "kv must be [Tk, 2, Hkv, D]")
    return varlen_attention(q, kv[:, 0], kv[:, 1], cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
                            scale=scale, causal=causal, window=window, attn_bias=attn_bias,
                            return_lse=return_lse, out_dtype=out_dtype, stream=stream,
                            max_seqlen_kv=max_seqlen_kv)


# ---------------------------------------------------------------- key-padding front end
class MiAttnPackParams(ctypes.Structure):
    """Field-for-field mirror of ``mi_attn_pack_params``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("padded", ctypes.c_void_p), ("packed", ctypes.c_void_p),
        ("ranks", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
        ("padded_stride_batch", ctypes.c_int64), ("padded_stride_tok", ctypes.c_int64),
        ("padded_stride_head", ctypes.c_int64),
        ("packed_stride_tok", ctypes.c_int64), ("packed_stride_head", ctypes.c_int64),
    ]


def mi_attn_padding_to_varlen(mask_ptr: int, batch: int, seqlen: int, mask_stride_batch: int,
                              ranks_ptr: int, cu_ptr: int, stats_ptr: int, stream: int = 0) -> None:
    """Call the C entry point; raise MiAttnError on a non-OK return."""
    lib = load_library()
    f = lib.mi_attn_padding_to_varlen
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    rc = f(mask_ptr, batch, seqlen, mask_stride_batch, ranks_ptr, cu_ptr, stats_ptr,
           ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


def _pack_call(name: str, params: MiAttnPackParams, stream: int) -> None:
    f = getattr(load_library(), name)
    f.argtypes = [ctypes.POINTER(MiAttnPackParams), ctypes.c_void_p]
    f.restype = ctypes.c_int
    params.struct_size = ctypes.sizeof(MiAttnPackParams)
    rc = f(ctypes.byref(params), ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


def mi_attn_pack_tokens(params: MiAttnPackParams, stream: int = 0) -> None:
    _pack_call("mi_attn_pack_tokens", params, stream)


def mi_attn_unpack_tokens(params: MiAttnPackParams, stream: int = 0) -> None:
    _pack_call("mi_attn_unpack_tokens", params, stream)


def padding_to_varlen(mask, stream=None, sync: bool = True):
    """Key-padding mask -> varlen form.  ``mask`` bool (or uint8) ``[B, N]``
    on the device, True = valid token (the last dim may be a view with a
    batch stride).  Returns ``(ranks, cu_seqlens, total, longest)``: int32
    ``[B, N]`` ranks (-1 at padding), int32 ``[B + 1]`` cumulative counts,
    and, with ``sync`` (one device-to-host read), the total valid tokens and
    the longest row as ints (else the int32 ``[2]`` device tensor)."""
    import torch
    if mask.dim() != 2 or not mask.is_cuda or mask.dtype not in (torch.bool, torch.uint8):
        raise MiAttnError(ERR_INVALID_ARG, "mask must be a bool / uint8 [B, N] device tensor")
    if mask.shape[1] > 1 and mask.stride(1) != 1:
        mask = mask.contiguous()
    bsz, n = mask.shape
    s_obj = _stream_of(stream, mask.device)
    with torch.cuda.stream(s_obj):
        ranks = torch.empty(bsz, n, dtype=torch.int32, device=mask.device)
        cu = torch.empty(bsz + 1, dtype=torch.int32, device=mask.device)
        stats = torch.empty(2, dtype=torch.int32, device=mask.device)
        mi_attn_padding_to_varlen(mask.data_ptr(), bsz, n, mask.stride(0) if bsz > 1 else n,
                                  ranks.data_ptr(), cu.data_ptr(), stats.data_ptr(),
                                  int(s_obj.cuda_stream))
    if not sync:
        return ranks, cu, stats
    total, longest = (int(x) for x in stats.tolist())
    return ranks, cu, total, longest


def mi_attn_padding_lengths(mask_ptr: int, batch: int, seqlen: int, mask_stride_batch: int,
                            lengths_ptr: int, spans_ptr: int, stats_ptr: int,
                            stream: int = 0) -> None:
    """Call the C entry point; raise MiAttnError on a non-OK return."""
    lib = load_library()
    f = lib.mi_attn_padding_lengths
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    rc = f(mask_ptr, batch, seqlen, mask_stride_batch, lengths_ptr, spans_ptr, stats_ptr,
           ctypes.c_void_p(stream))
    if rc != OK:
        raise MiAttnError(rc, mi_attn_last_error())


def padding_lengths(mask, stream=None, sync: bool = True):
    """Right-padding check of a key-padding mask (bool or uint8 ``[B, N]`` on
    the device, True = valid token).  Returns ``(lengths, spans, right_padded,
    longest)``: int32 ``[B]`` valid counts, int32 ``[B + 1]`` spans ``b * N``
    and, with ``sync`` (one device-to-host read), whether every row's valid
    tokens are its first ones and the longest row (else the int32 ``[2]``
    device tensor).  For a right-padded batch the forward takes the padded
    tensors as they are: ``cu_seqlens = spans``, ``seqused_q = seqused_kv =
    lengths``."""
    import torch
    if mask.dim() != 2 or not mask.is_cuda or mask.dtype not in (torch.bool, torch.uint8):
        raise MiAttnError(ERR_INVALID_ARG, "mask must be a bool / uint8 [B, N] device tensor")
    if mask.shape[1] > 1 and mask.stride(1) != 1:
        mask = mask.contiguous()
    bsz, n = mask.shape
    s_obj = _stream_of(stream, mask.device)
    with torch.cuda.stream(s_obj):
        lengths = torch.empty(bsz, dtype=torch.int32, device=mask.device)
        spans = torch.empty(bsz + 1, dtype=torch.int32, device=mask.device)
        stats = torch.empty(2, dtype=torch.int32, device=mask.device)
        mi_attn_padding_lengths(mask.data_ptr(), bsz, n, mask.stride(0) if bsz > 1 else n,
                                lengths.data_ptr(), spans.data_ptr(), stats.data_ptr(),
                                int(s_obj.cuda_stream))
    if not sync:
        return lengths, spans, stats
    right, longest = (int(x) for x in stats.tolist())
    return lengths, spans, bool(right), longest


def _pack_params(padded, packed, ranks, cu, bsz, n):
    p = MiAttnPackParams()
    p.padded, p.packed = padded.data_ptr(), packed.data_ptr()
    p.ranks = ranks.data_ptr() if ranks is not None else None
    p.cu_seqlens = cu.data_ptr() if cu is not None else None
    p.batch, p.seqlen = bsz, n
    p.heads, p.dim = padded.shape[2], padded.shape[3]
    p.elem_bytes = padded.element_size()
    p.padded_stride_batch, p.padded_stride_tok, p.padded_stride_head = (
        padded.stride(0), padded.stride(1), padded.stride(2))
    p.packed_stride_tok, p.packed_stride_head = packed.stride(0), packed.stride(1)
    return p


def pack_tokens(padded, ranks=None, cu_seqlens=None, total=None, out=None, stream=None):
    """Gather ``padded`` ``[B, N, H, D]`` (any strides, last dim contiguous)
    into packed ``[total, H, D]``; ``ranks=None`` packs every token."""
    import torch
    bsz, n, h, d = padded.shape
    if padded.stride(-1) != 1:
        raise MiAttnError(ERR_INVALID_ARG, "padded must have a contiguous last dim")
    if total is None:
        total = bsz * n
    if ranks is not None and tuple(ranks.shape) != (bsz, n):
        raise MiAttnError(ERR_INVALID_ARG, "ranks must be [B, N]")
    s_obj = _stream_of(stream, padded.device)
    with torch.cuda.stream(s_obj):
        if out is None:
            out = torch.empty(total, h, d, dtype=padded.dtype, device=padded.device)
        elif tuple(out.shape) != (total, h, d) or out.dtype != padded.dtype:
            raise MiAttnError(ERR_INVALID_ARG, "out has the wrong shape or dtype")
        mi_attn_pack_tokens(_pack_params(padded, out, ranks, cu_seqlens, bsz, n),
                            int(s_obj.cuda_stream))
    return out


def unpack_tokens(packed, out, ranks=None, cu_seqlens=None, stream=None):
    """Scatter packed ``[total, H, D]`` into ``out`` ``[B, N, H, D]`` (any
    strides, last dim contiguous), zeros at padding; returns ``out``."""
    import torch
    bsz, n, h, d = out.shape
    if out.stride(-1) != 1 or packed.dtype != out.dtype or tuple(packed.shape[1:]) != (h, d):
        raise MiAttnError(ERR_INVALID_ARG, "out / packed shapes, dtypes or layout do not match")
    if ranks is not None and tuple(ranks.shape) != (bsz, n):
        raise MiAttnError(ERR_INVALID_ARG, "ranks must be [B, N]")
    s_obj = _stream_of(stream, out.device)
    with torch.cuda.stream(s_obj):
        mi_attn_unpack_tokens(_pack_params(out, packed, ranks, cu_seqlens, bsz, n),
                              int(s_obj.cuda_stream))
    return out


def _key_padding_of(attn_mask, bsz, nkv):
    """The [B, Nkv] key mask if ``attn_mask`` is a bool key-padding mask
    ``[B, 1, 1, Nkv]``, else None."""
    import torch
    if attn_mask is None or attn_mask.dtype != torch.bool or attn_mask.dim() != 4:
        return None
    if tuple(attn_mask.shape) == (bsz, 1, 1, nkv):
        return attn_mask[:, 0, 0, :]
    return None


def sdpa(query, key, value, attn_mask=None, dropout_p: float = 0.0, is_causal: bool = False,
         scale: Optional[float] = None, enable_gqa: bool = False, stream=None, out_dtype=None):
    """``scaled_dot_product_attention`` on dense ``[B, H, N, D]`` tensors
    through the varlen kernels (the adapter of the mtlattn 0.3.0 page,
    section "Drop-in for scaled_dot_product_attention"), forward only.

    * A boolean key-padding mask (``[B, 1, 1, Nkv]`` or ``[B, Nkv]``, True =
      valid) is turned into varlen form: the valid keys (and, for
      self-attention, the valid queries) are packed and padding is never
      computed.  Output rows of padded queries are 0.  A right-padded
      self-attention batch whose tensors are views of token-major
      ``[B, N, H, D]`` storage needs no packing: it runs in place, and the
      output is then returned as such a view too.
    * Any other mask (bool or float, broadcastable to ``[B, H, Nq, Nkv]``)
      becomes the kernel's additive bias (bool: True -> 0, False -> -inf).
    * ``is_causal`` follows SDPA's top-left diagonal, which equals the
      kernel's end-aligned one only when Nq == Nkv; other shapes are refused.
    Rows that see no key are 0 (SDPA gives NaN there).  ``out_dtype``
    (default: the input dtype) may be ``torch.float32``.
    """
    import torch
    if dropout_p != 0.0:
        raise MiAttnError(ERR_UNSUPPORTED, "dropout is not supported")
    for name, t in (("query", query), ("key", key), ("value", value)):
        if t.dim() != 4 or not t.is_cuda:
            raise MiAttnError(ERR_INVALID_ARG, f"{name} must be a [B, H, N, D] device tensor")
    bsz, hq, nq, d = query.shape
    _, hkv, nkv, _ = key.shape
    dv = value.shape[3]
    if key.shape[0] != bsz or tuple(value.shape[:3]) != (bsz, hkv, nkv):
        raise MiAttnError(ERR_INVALID_ARG, "query / key / value shapes do not match")
    if hq != hkv and not enable_gqa:
        raise MiAttnError(ERR_INVALID_ARG, "key / value have fewer heads: pass enable_gqa=True")
    if is_causal and nq != nkv:
        raise MiAttnError(ERR_UNSUPPORTED, "is_causal with Nq != Nkv (top-left diagonal) is not "
                                           "the kernel's end-aligned rule")
    if is_causal and attn_mask is not None and _key_padding_of(attn_mask, bsz, nkv) is None:
        raise MiAttnError(ERR_INVALID_ARG, "is_causal together with a general attn_mask")
    if torch.is_grad_enabled() and any(t.requires_grad for t in (query, key, value)):
        raise MiAttnError(ERR_UNSUPPORTED, "sdpa is forward only; use varlen_attention for "
                                           "gradients")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_obj = _stream_of(stream, query.device)
    dev = query.device
    with torch.cuda.stream(s_obj):
        # token-major views [B, N, H, D] of the head-major inputs: no copy
        qv, kv_, vv = query.transpose(1, 2), key.transpose(1, 2), value.transpose(1, 2)
        out_dtype = query.dtype if out_dtype is None else out_dtype
        keymask = _key_padding_of(attn_mask, bsz, nkv)
        if keymask is not None and nq == nkv and all(
                t.stride(0) == nq * t.stride(1) for t in (qv, kv_, vv)):
            # self-attention on token-major storage: a right-padded batch runs
            # in place (spans of N tokens, the first lengths[b] used), no packing
            lengths, spans, right, _ = padding_lengths(keymask, stream=s_obj)
            if right:
                flat = [t.as_strided((bsz * nq, t.shape[2], t.shape[3]),
                                     (t.stride(1), t.stride(2), t.stride(3)))
                        for t in (qv, kv_, vv)]
                out_tm = torch.empty(bsz, nq, hq, dv, dtype=out_dtype, device=dev)
                varlen_attention(flat[0], flat[1], flat[2], spans, spans, nq, scale=scale,
                                 causal=is_causal, out_dtype=out_dtype, stream=s_obj,
                                 out=out_tm.view(bsz * nq, hq, dv), seqused_q=lengths,
                                 seqused_kv=lengths)
                return out_tm.transpose(1, 2)
        out = torch.empty(bsz, hq, nq, dv, dtype=out_dtype, device=dev)
        ov = out.transpose(1, 2)
        if keymask is not None:
            rk, cu_k, tot_k, max_k = padding_to_varlen(keymask, stream=s_obj)
            if nq == nkv:
                rq, cu_q, tot_q, max_q = rk, cu_k, tot_k, max_k
            else:
                rq, cu_q, tot_q, max_q = None, None, bsz * nq, nq
            bias = None
        else:
            rk = rq = None
            cu_k = torch.arange(0, bsz + 1, dtype=torch.int32, device=dev) * nkv
            cu_q = torch.arange(0, bsz + 1, dtype=torch.int32, device=dev) * nq
            tot_k, tot_q, max_q = bsz * nkv, bsz * nq, nq
            bias = None
            if attn_mask is not None:
                m = attn_mask
                while m.dim() < 4:
                    m = m.unsqueeze(0)
                if m.dim() != 4 or m.shape[1] not in (1, hq):
                    raise MiAttnError(ERR_INVALID_ARG, "attn_mask must broadcast to [B, H or 1, "
                                                       "Nq, Nkv]")
                m = m.expand(bsz, m.shape[1], nq, nkv)
                if m.dtype == torch.bool:
                    bias = torch.zeros(m.shape, dtype=torch.float32, device=dev).masked_fill_(
                        ~m, float("-inf"))
                else:
                    bias = m.to(torch.float32)
                # [B, Hb, Nq, Nkv] -> rows of global query tokens [B * Nq, Hb, Nkv]
                bias = bias.permute(0, 2, 1, 3).reshape(bsz * nq, m.shape[1], nkv)
        pq = pack_tokens(qv, rq, cu_q, tot_q, stream=s_obj)
        pk = pack_tokens(kv_, rk, cu_k, tot_k, stream=s_obj)
        pv = pack_tokens(vv, rk, cu_k, tot_k, stream=s_obj)
        if cu_q is None:
            cu_q = torch.arange(0, bsz + 1, dtype=torch.int32, device=dev) * nq
        po = varlen_attention(pq, pk, pv, cu_q, cu_k, max_q, scale=scale, causal=is_causal,
                              attn_bias=bias, out_dtype=out_dtype, stream=s_obj)
        unpack_tokens(po, ov, rq, cu_q, stream=s_obj)
    return out
