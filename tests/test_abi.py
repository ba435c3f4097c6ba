"""The C-ABI library loads, exports every symbol include/mi_attn.h declares,
its params struct matches the ctypes mirror, and host-side validation refuses
malformed or unsupported calls before touching the GPU (CPU only)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import flash_attention_varlen_amd as fav

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mi_attn_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names == ["mi_attn_bias_key_ranges", "mi_attn_decode_workspace_size", "mi_attn_last_error",
                     "mi_attn_pack_tokens", "mi_attn_padding_lengths", "mi_attn_padding_to_varlen",
                     "mi_attn_tile_shape",
                     "mi_attn_unpack_tokens", "mi_attn_varlen_bwd", "mi_attn_varlen_decode",
                     "mi_attn_varlen_decode_noalloc", "mi_attn_varlen_fwd", "mi_attn_version"]
    lib = fav.load_library()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fav.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (mi_attn_\w+)", out))
    assert set(names) <= exported


def test_version_and_tile_shape():
    assert fav.mi_attn_version() == 170
    for dt in (fav.BF16, fav.F16):
        for dqk, dv in ((64, 64), (96, 96), (128, 128), (192, 128), (256, 256)):
            bm, bn = fav.mi_attn_tile_shape(dt, dqk, dv)
            assert bm % 128 == 0 and bn % 32 == 0 and bm > 0 and bn > 0
    assert fav.mi_attn_tile_shape(fav.F32, 64, 64) == (128, 32)
    with pytest.raises(fav.MiAttnError):
        fav.mi_attn_tile_shape(fav.F32, 192, 128)
    with pytest.raises(fav.MiAttnError):
        fav.mi_attn_tile_shape(fav.BF16, 80, 80)
    for dqk, dv in ((96, 96), (256, 256)):  # 16-bit only
        with pytest.raises(fav.MiAttnError):
            fav.mi_attn_tile_shape(fav.F32, dqk, dv)


@pytest.mark.parametrize("cls,cname", [(fav.MiAttnFwdParams, "mi_attn_fwd_params"),
                                       (fav.MiAttnBwdParams, "mi_attn_bwd_params"),
                                       (fav.MiAttnPackParams, "mi_attn_pack_params")])
def test_struct_layout_matches_header(cls, cname):
    fields = [f[0] for f in cls._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"mi_attn.h\"\nint main(void){\n"
    src += f'printf("%zu\\n", sizeof({cname}));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof({cname}, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(cls)
    for f, off in zip(fields, vals[1:]):
        assert getattr(cls, f).offset == off, f


def _valid_params():
    p = fav.MiAttnFwdParams()
    fake = 1 << 20  # aligned non-null addresses; never dereferenced by refused calls
    p.q = p.k = p.v = p.out = fake
    p.cu_seqlens_q = p.cu_seqlens_kv = fake
    p.num_seqs, p.max_seqlen_q, p.total_q, p.total_kv = 2, 64, 100, 100
    p.hq, p.hkv, p.d_qk, p.d_v = 8, 2, 128, 128
    p.q_stride_tok, p.q_stride_head = 8 * 128, 128
    p.k_stride_tok, p.k_stride_head = 2 * 128, 128
    p.v_stride_tok, p.v_stride_head = 2 * 128, 128
    p.out_stride_tok, p.out_stride_head = 8 * 128, 128
    p.in_dtype = p.out_dtype = fav.BF16
    p.scale = 0.088
    return p


REFUSALS = {
    "bad_dtype": (dict(in_dtype=7), fav.ERR_UNSUPPORTED),
    "bad_out_dtype": (dict(out_dtype=fav.F16), fav.ERR_UNSUPPORTED),
    "head_dims": (dict(d_qk=80, d_v=80), fav.ERR_UNSUPPORTED),
    "head_dims_mixed": (dict(d_qk=256, d_v=128), fav.ERR_UNSUPPORTED),
    "f32_d96": (dict(in_dtype=fav.F32, out_dtype=fav.F32, d_qk=96, d_v=96), fav.ERR_UNSUPPORTED),
    "f32_d256": (dict(in_dtype=fav.F32, out_dtype=fav.F32, d_qk=256, d_v=256), fav.ERR_UNSUPPORTED),
    "f32_latent": (dict(in_dtype=fav.F32, out_dtype=fav.F32, d_qk=192, d_v=128), fav.ERR_UNSUPPORTED),
    "gqa_ratio": (dict(hq=6, hkv=4), fav.ERR_UNSUPPORTED),
    "zero_heads": (dict(hkv=0), fav.ERR_INVALID_ARG),
    "window_without_causal": (dict(window=16), fav.ERR_UNSUPPORTED),
    "negative_window": (dict(window=-1, causal=1), fav.ERR_INVALID_ARG),
    "bad_causal": (dict(causal=2), fav.ERR_INVALID_ARG),
    "negative_size": (dict(total_q=-1), fav.ERR_INVALID_ARG),
    "null_q": (dict(q=None), fav.ERR_INVALID_ARG),
    "null_cu": (dict(cu_seqlens_kv=None), fav.ERR_INVALID_ARG),
    "misaligned_q": (dict(q=(1 << 20) + 8), fav.ERR_INVALID_ARG),
    "odd_stride": (dict(k_stride_tok=2 * 128 + 4), fav.ERR_INVALID_ARG),
    "nan_scale": (dict(scale=float("nan")), fav.ERR_INVALID_ARG),
    "zero_scale": (dict(scale=0.0), fav.ERR_UNSUPPORTED),
    "bias_heads": (dict(bias=1 << 20, bias_heads=3, bias_cols=64, bias_stride_tok=8 * 64,
                        bias_stride_head=64), fav.ERR_UNSUPPORTED),
    "bias_stride": (dict(bias=1 << 20, bias_heads=1, bias_cols=64, bias_stride_tok=66,
                         bias_stride_head=0), fav.ERR_INVALID_ARG),
    "too_many_q_tiles": (dict(max_seqlen_q=128 * 65536), fav.ERR_UNSUPPORTED),
    "overlapping_out_rows": (dict(out_stride_tok=64, out_stride_head=8), fav.ERR_UNSUPPORTED),
    "huge_out_stride": (dict(out_stride_tok=1 << 26), fav.ERR_UNSUPPORTED),
    # head slices of one token overlap (head stride below d_v)
    "overlapping_out_heads": (dict(out_stride_tok=8 * 128 * 8, out_stride_head=64),
                              fav.ERR_UNSUPPORTED),
    # token rows overlap the next token's heads (token stride below hq * d_v)
    "overlapping_out_tokens": (dict(out_stride_tok=512, out_stride_head=128), fav.ERR_UNSUPPORTED),
    # split nope / rope operands: both pointers, the latent head, 16-bit, aligned strides
    "rope_without_k_rope": (dict(d_qk=192, q_rope=1 << 20, q_rope_stride_tok=8 * 64,
                                 q_rope_stride_head=64), fav.ERR_INVALID_ARG),
    "rope_square_head": (dict(q_rope=1 << 20, k_rope=1 << 20, q_rope_stride_tok=8 * 64,
                              q_rope_stride_head=64, k_rope_stride_tok=2 * 64,
                              k_rope_stride_head=64), fav.ERR_UNSUPPORTED),
    "rope_f32": (dict(in_dtype=fav.F32, out_dtype=fav.F32, d_qk=192, q_rope=1 << 20,
                      k_rope=1 << 20, q_rope_stride_tok=8 * 64, q_rope_stride_head=64,
                      k_rope_stride_tok=2 * 64, k_rope_stride_head=64), fav.ERR_UNSUPPORTED),
    "rope_misaligned": (dict(d_qk=192, q_rope=1 << 20, k_rope=(1 << 20) + 8,
                             q_rope_stride_tok=8 * 64, q_rope_stride_head=64,
                             k_rope_stride_tok=2 * 64, k_rope_stride_head=64), fav.ERR_INVALID_ARG),
    "rope_odd_stride": (dict(d_qk=192, q_rope=1 << 20, k_rope=1 << 20, q_rope_stride_tok=8 * 64 + 4,
                             q_rope_stride_head=64, k_rope_stride_tok=2 * 64,
                             k_rope_stride_head=64), fav.ERR_INVALID_ARG),
    "rope_short_row": (dict(d_qk=192, q_rope=1 << 20, k_rope=1 << 20, q_rope_stride_tok=8 * 64,
                            q_rope_stride_head=64, k_rope_stride_tok=56,
                            k_rope_stride_head=0), fav.ERR_UNSUPPORTED),
    "alibi_with_bias": (dict(alibi_slopes=1 << 20, bias=1 << 20, bias_heads=1, bias_cols=64,
                             bias_stride_tok=64, bias_stride_head=0), fav.ERR_UNSUPPORTED),
    "alibi_misaligned": (dict(alibi_slopes=(1 << 20) + 2), fav.ERR_INVALID_ARG),
    "alibi_negative_stride": (dict(alibi_slopes=1 << 20, alibi_stride_seq=-8), fav.ERR_INVALID_ARG),
    # byte mask: not with a bias or ALiBi; 4-byte aligned, strides multiples of 4 bytes
    "mask_and_bias": (dict(mask=1 << 20, bias=1 << 20, bias_heads=1, bias_cols=64,
                           bias_stride_tok=64, bias_stride_head=0), fav.ERR_INVALID_ARG),
    "mask_and_alibi": (dict(mask=1 << 20, alibi_slopes=1 << 20, bias_heads=1, bias_cols=64,
                            bias_stride_tok=64, bias_stride_head=0), fav.ERR_UNSUPPORTED),
    "mask_misaligned": (dict(mask=(1 << 20) + 2, bias_heads=1, bias_cols=64, bias_stride_tok=64,
                             bias_stride_head=0), fav.ERR_INVALID_ARG),
    "mask_odd_stride": (dict(mask=1 << 20, bias_heads=1, bias_cols=63, bias_stride_tok=63,
                             bias_stride_head=0), fav.ERR_INVALID_ARG),
    "mask_heads": (dict(mask=1 << 20, bias_heads=3, bias_cols=64, bias_stride_tok=64,
                        bias_stride_head=64), fav.ERR_UNSUPPORTED),
    # interval flags of the bias rows: only with a bias or a mask, and with their ranges
    "pure_without_bias": (dict(bias_pure=1 << 20), fav.ERR_INVALID_ARG),
    "pure_without_ranges": (dict(bias_pure=1 << 20, bias=1 << 20, bias_heads=1, bias_cols=64,
                                 bias_stride_tok=64, bias_stride_head=0), fav.ERR_INVALID_ARG),
    "seqused_q_misaligned": (dict(seqused_q=(1 << 20) + 2), fav.ERR_INVALID_ARG),
    "seqused_kv_misaligned": (dict(seqused_kv=(1 << 20) + 1), fav.ERR_INVALID_ARG),
    # with split operands q / k hold 128 dims; without them a 128-wide stride is short of 192
    "latent_short_q_stride": (dict(d_qk=192, q_stride_tok=128, q_stride_head=0, hq=2, hkv=2,
                                   out_stride_tok=2 * 128), fav.ERR_UNSUPPORTED),
}


@pytest.mark.parametrize("name", sorted(REFUSALS))
def test_host_validation_refuses(name):
    changes, code = REFUSALS[name]
    p = _valid_params()
    for k, v in changes.items():
        setattr(p, k, v)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.mi_attn_varlen_fwd(p, 0)
    assert ei.value.code == code, fav.mi_attn_last_error()
    assert fav.mi_attn_last_error() != ""


def test_short_struct_is_refused():
    p = _valid_params()
    lib = fav.load_library()
    p.struct_size = 8
    assert lib.mi_attn_varlen_fwd(ctypes.byref(p), None) == fav.ERR_INVALID_ARG


def test_version_1_0_struct_is_accepted():
    """A caller built against 1.0 passes the struct without bias_ranges: the
    library reads the fields it has and takes bias_ranges as NULL (the call
    below is a refusal found after the copy: an unsupported head size)."""
    p = _valid_params()
    lib = fav.load_library()
    p.struct_size = fav.MiAttnFwdParams.bias_ranges.offset
    p.bias_ranges = 1 << 20  # beyond the 1.0 struct: must not be read
    p.d_qk = p.d_v = 80
    assert lib.mi_attn_varlen_fwd(ctypes.byref(p), None) == fav.ERR_UNSUPPORTED
    assert "head dims" in fav.mi_attn_last_error()


RANGE_REFUSALS = {
    "no_bias": (dict(bias=None), fav.ERR_INVALID_ARG),
    "bias_and_mask": (dict(mask=1 << 20), fav.ERR_INVALID_ARG),
    "misaligned_mask": (dict(bias=None, mask=(1 << 20) + 1), fav.ERR_INVALID_ARG),
    "bias_heads": (dict(bias_heads=3), fav.ERR_UNSUPPORTED),
    "odd_bias_stride": (dict(bias_stride_tok=66), fav.ERR_INVALID_ARG),
    "zero_cols": (dict(bias_cols=0), fav.ERR_INVALID_ARG),
}


@pytest.mark.parametrize("name", sorted(RANGE_REFUSALS))
def test_bias_key_ranges_refuses(name):
    changes, code = RANGE_REFUSALS[name]
    p = _valid_params()
    p.bias, p.bias_heads, p.bias_cols = 1 << 20, 1, 64
    p.bias_stride_tok, p.bias_stride_head = 64, 64
    for k, v in changes.items():
        setattr(p, k, v)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.mi_attn_bias_key_ranges(p, 1 << 21, 0)
    assert ei.value.code == code, fav.mi_attn_last_error()


def test_empty_problem_is_a_no_op():
    p = _valid_params()
    p.num_seqs = 0
    fav.mi_attn_varlen_fwd(p, 0)
    p = _valid_params()
    p.total_q = 0
    fav.mi_attn_varlen_fwd(p, 0)


def _valid_bwd_params():
    p = fav.MiAttnBwdParams()
    fake = 1 << 20
    for name in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "delta", "cu_seqlens_q",
                 "cu_seqlens_kv"):
        setattr(p, name, fake)
    p.num_seqs, p.max_seqlen_q, p.max_seqlen_kv, p.total_q, p.total_kv = 2, 64, 64, 100, 100
    p.hq, p.hkv, p.d_qk, p.d_v = 8, 2, 128, 128
    for name, hd in (("q", 8), ("k", 2), ("v", 2), ("out", 8), ("dout", 8), ("dq", 8), ("dk", 2),
                     ("dv", 2)):
        setattr(p, f"{name}_stride_tok", hd * 128)
        setattr(p, f"{name}_stride_head", 128)
    p.in_dtype = p.grad_dtype = fav.BF16
    p.scale = 0.088
    return p


BWD_REFUSALS = {
    "fp32_inputs": (dict(in_dtype=fav.F32, grad_dtype=fav.F32), fav.ERR_UNSUPPORTED),
    "latent_dims": (dict(d_qk=192, d_v=128), fav.ERR_UNSUPPORTED),
    "dims_256": (dict(d_qk=256, d_v=256), fav.ERR_UNSUPPORTED),
    "dims_80": (dict(d_qk=80, d_v=80), fav.ERR_UNSUPPORTED),
    "grad_dtype": (dict(grad_dtype=fav.F16), fav.ERR_UNSUPPORTED),
    "alibi_with_bias": (dict(alibi_slopes=1 << 20, bias=1 << 20, bias_heads=1, bias_cols=64,
                             bias_stride_tok=64, bias_stride_head=0), fav.ERR_UNSUPPORTED),
    "alibi_misaligned": (dict(alibi_slopes=(1 << 20) + 1), fav.ERR_INVALID_ARG),
    "gqa_ratio": (dict(hq=6, hkv=4), fav.ERR_UNSUPPORTED),
    "window_without_causal": (dict(window=8), fav.ERR_UNSUPPORTED),
    "null_delta": (dict(delta=None), fav.ERR_INVALID_ARG),
    "misaligned_dk": (dict(dk=(1 << 20) + 8), fav.ERR_INVALID_ARG),
    "odd_stride": (dict(dout_stride_tok=8 * 128 + 4), fav.ERR_INVALID_ARG),
    "overlapping_dq": (dict(dq_stride_tok=128, dq_stride_head=128), fav.ERR_UNSUPPORTED),
    "too_many_key_tiles": (dict(max_seqlen_kv=128 * 65536), fav.ERR_UNSUPPORTED),
}


@pytest.mark.parametrize("name", sorted(BWD_REFUSALS))
def test_backward_host_validation_refuses(name):
    changes, code = BWD_REFUSALS[name]
    p = _valid_bwd_params()
    for k, v in changes.items():
        setattr(p, k, v)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.mi_attn_varlen_bwd(p, 0)
    assert ei.value.code == code, fav.mi_attn_last_error()


DECODE_REFUSALS = {
    "fp32": (dict(in_dtype=fav.F32, out_dtype=fav.F32), 1 << 20, fav.ERR_UNSUPPORTED),
    "latent_dims": (dict(d_qk=192, d_v=128), 1 << 20, fav.ERR_UNSUPPORTED),
    "alibi": (dict(alibi_slopes=1 << 20), 1 << 20, fav.ERR_UNSUPPORTED),
    "mask": (dict(mask=1 << 20, bias_heads=1, bias_cols=64, bias_stride_tok=64,
                  bias_stride_head=0), 1 << 20, fav.ERR_UNSUPPORTED),
    "rope": (dict(q_rope=1 << 20, k_rope=1 << 20, q_rope_stride_tok=8 * 64, q_rope_stride_head=64,
                  k_rope_stride_tok=2 * 64, k_rope_stride_head=64), 1 << 20, fav.ERR_UNSUPPORTED),
    "bias": (dict(bias=1 << 20, bias_heads=1, bias_cols=64, bias_stride_tok=64, bias_stride_head=64),
             1 << 20, fav.ERR_UNSUPPORTED),
    "too_many_rows": (dict(max_seqlen_q=17), 1 << 20, fav.ERR_UNSUPPORTED),  # 4 heads x 17 > 64
    "seqused_q": (dict(seqused_q=1 << 20), 1 << 20, fav.ERR_UNSUPPORTED),
    "misaligned_workspace": (dict(max_seqlen_q=1), (1 << 20) + 8, fav.ERR_INVALID_ARG),
    "null_workspace": (dict(max_seqlen_q=1), 0, fav.ERR_INVALID_ARG),
}


@pytest.mark.parametrize("name", sorted(DECODE_REFUSALS))
def test_decode_host_validation_refuses(name):
    changes, ws, code = DECODE_REFUSALS[name]
    p = _valid_params()
    for k, v in changes.items():
        setattr(p, k, v)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.mi_attn_varlen_decode(p, 4096, 0, ws, 1 << 30, 0)
    assert ei.value.code == code, fav.mi_attn_last_error()


def test_decode_workspace_size_and_short_workspace():
    """The size query matches the plan (chunks x rows x heads x (d_v + 2)
    floats) and a workspace one byte short is refused."""
    p = _valid_params()
    p.max_seqlen_q, p.total_q = 1, 2
    n = fav.mi_attn_decode_workspace_size(p, 4096, 8)
    chunks = -(-(4096 // 32 + 1) // -(-(4096 // 32 + 1) // 8))
    assert n == chunks * 2 * 8 * (128 + 2) * 4
    with pytest.raises(fav.MiAttnError) as ei:
        fav.mi_attn_varlen_decode(p, 4096, 8, 1 << 20, n - 1, 0)
    assert ei.value.code == fav.ERR_INVALID_ARG and "workspace" in fav.mi_attn_last_error()


# ---------------------------------------------------------------- key-padding front end
def _valid_pack():
    p = fav.MiAttnPackParams()
    fake = 1 << 20
    p.padded = p.packed = p.ranks = p.cu_seqlens = fake
    p.batch, p.seqlen, p.heads, p.dim, p.elem_bytes = 2, 10, 4, 64, 2
    p.padded_stride_batch, p.padded_stride_tok, p.padded_stride_head = 4 * 10 * 64, 64, 10 * 64
    p.packed_stride_tok, p.packed_stride_head = 4 * 64, 64
    return p


PACK_REFUSALS = {
    "elem_bytes": (dict(elem_bytes=1), fav.ERR_UNSUPPORTED, "both"),
    "row_not_16_bytes": (dict(dim=12), fav.ERR_UNSUPPORTED, "both"),
    "zero_heads": (dict(heads=0), fav.ERR_INVALID_ARG, "both"),
    "negative_batch": (dict(batch=-1), fav.ERR_INVALID_ARG, "both"),
    "huge": (dict(batch=1 << 20, seqlen=1 << 12), fav.ERR_UNSUPPORTED, "both"),
    "null_packed": (dict(packed=None), fav.ERR_INVALID_ARG, "both"),
    "ranks_without_cu": (dict(cu_seqlens=None), fav.ERR_INVALID_ARG, "both"),
    "misaligned": (dict(padded=(1 << 20) + 8), fav.ERR_INVALID_ARG, "both"),
    "odd_stride": (dict(packed_stride_tok=4 * 64 + 4), fav.ERR_INVALID_ARG, "both"),
    # the written side must not overlap itself
    "packed_rows_overlap": (dict(packed_stride_tok=64), fav.ERR_UNSUPPORTED, "pack"),
    "padded_rows_overlap": (dict(padded_stride_batch=64), fav.ERR_UNSUPPORTED, "unpack"),
}


@pytest.mark.parametrize("direction", ["pack", "unpack"])
@pytest.mark.parametrize("name", sorted(PACK_REFUSALS))
def test_pack_host_validation_refuses(name, direction):
    changes, code, which = PACK_REFUSALS[name]
    if which not in ("both", direction):
        pytest.skip("checked for the other direction")
    p = _valid_pack()
    for k, v in changes.items():
        setattr(p, k, v)
    fn = fav.mi_attn_pack_tokens if direction == "pack" else fav.mi_attn_unpack_tokens
    with pytest.raises(fav.MiAttnError) as ei:
        fn(p, 0)
    assert ei.value.code == code, fav.mi_attn_last_error()


def test_empty_pack_is_a_no_op():
    """No tokens: OK before any pointer is used."""
    p = _valid_pack()
    p.batch = 0
    p.padded = p.packed = None
    fav.mi_attn_pack_tokens(p, 0)
    fav.mi_attn_unpack_tokens(p, 0)


def test_short_pack_struct_is_refused():
    p = _valid_pack()
    p.struct_size = 8
    lib = fav.load_library()
    f = lib.mi_attn_pack_tokens
    f.argtypes = [ctypes.POINTER(fav.MiAttnPackParams), ctypes.c_void_p]
    assert f(ctypes.byref(p), None) == fav.ERR_INVALID_ARG


PADDING_REFUSALS = {
    "negative": (dict(batch=-1), fav.ERR_INVALID_ARG),
    "too_many_tokens": (dict(batch=1 << 16, seqlen=1 << 16), fav.ERR_UNSUPPORTED),
    "null_cu": (dict(cu=0), fav.ERR_INVALID_ARG),
    "null_mask": (dict(mask=0), fav.ERR_INVALID_ARG),
    "null_ranks": (dict(ranks=0), fav.ERR_INVALID_ARG),
    "misaligned_ranks": (dict(ranks=(1 << 20) + 2), fav.ERR_INVALID_ARG),
    "negative_stride": (dict(stride=-1), fav.ERR_INVALID_ARG),
}


@pytest.mark.parametrize("name", sorted(PADDING_REFUSALS))
def test_padding_to_varlen_refuses(name):
    args = dict(mask=1 << 20, batch=2, seqlen=10, stride=10, ranks=1 << 20, cu=1 << 20,
                stats=0)
    changes, code = PADDING_REFUSALS[name]
    args.update(changes)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.mi_attn_padding_to_varlen(args["mask"], args["batch"], args["seqlen"], args["stride"],
                                      args["ranks"], args["cu"], args["stats"], 0)
    assert ei.value.code == code, fav.mi_attn_last_error()


LENGTH_REFUSALS = {
    "negative": (dict(batch=-1), fav.ERR_INVALID_ARG),
    "too_many_tokens": (dict(batch=1 << 16, seqlen=1 << 16), fav.ERR_UNSUPPORTED),
    "null_spans": (dict(spans=0), fav.ERR_INVALID_ARG),
    "null_lengths": (dict(lengths=0), fav.ERR_INVALID_ARG),
    "null_mask": (dict(mask=0), fav.ERR_INVALID_ARG),
    "misaligned_lengths": (dict(lengths=(1 << 20) + 2), fav.ERR_INVALID_ARG),
    "misaligned_stats": (dict(stats=(1 << 20) + 1), fav.ERR_INVALID_ARG),
    "negative_stride": (dict(stride=-1), fav.ERR_INVALID_ARG),
}


@pytest.mark.parametrize("name", sorted(LENGTH_REFUSALS))
def test_padding_lengths_refuses(name):
    args = dict(mask=1 << 20, batch=2, seqlen=10, stride=10, lengths=1 << 20, spans=1 << 20,
                stats=0)
    changes, code = LENGTH_REFUSALS[name]
    args.update(changes)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.mi_attn_padding_lengths(args["mask"], args["batch"], args["seqlen"], args["stride"],
                                    args["lengths"], args["spans"], args["stats"], 0)
    assert ei.value.code == code, fav.mi_attn_last_error()
