"""Layout variants of the forward at the C ABI: split nope / rope operands of
the latent-attention head (q, k 128 wide plus q_rope, k_rope 64 wide; the
triton-msl part-2 post, section "Latent attention, the 2026 frontier")
against the fp64 oracle on the concatenated operands, and bitwise against
one call on the concatenation (same products, same accumulation order)."""
import pytest
import torch

import flash_attention_varlen_amd as fav
import workloads
from gpu_helpers import check, check_sampled, run_oracle, say, to_device

pytestmark = pytest.mark.gpu

W = workloads.Workload

CASES = {
    "bf16_causal_gqa": W(name="rope_bf16_causal_gqa", seqlens_q=(300, 129, 1),
                         seqlens_kv=(300, 129, 1), hq=4, hkv=2, d_qk=192, d_v=128, dtype="bf16",
                         causal=True, nope_rope=(128, 64), seed=70),
    "f16_full": W(name="rope_f16_full", seqlens_q=(150, 65), seqlens_kv=(150, 65), hq=2, hkv=1,
                  d_qk=192, d_v=128, dtype="f16", causal=False, nope_rope=(128, 64), seed=71),
    "bf16_prefix_bias": W(name="rope_bf16_prefix_bias", seqlens_q=(200, 97), seqlens_kv=(200, 97),
                          hq=2, hkv=2, d_qk=192, d_v=128, dtype="bf16", causal=False,
                          bias="prefix_lm", prefix=50, nope_rope=(128, 64), seed=72),
    "bf16_window_cross": W(name="rope_bf16_window_cross", seqlens_q=(90, 40),
                           seqlens_kv=(260, 41), hq=2, hkv=1, d_qk=192, d_v=128, dtype="bf16",
                           causal=True, window=70, nope_rope=(128, 64), seed=73),
}


def _split(q, k, how):
    if how == "views":  # slices of the concatenated tensors: strides 192 per head
        return q[..., :128], q[..., 128:], k[..., :128], k[..., 128:]
    return (q[..., :128].contiguous(), q[..., 128:].contiguous(), k[..., :128].contiguous(),
            k[..., 128:].contiguous())


def _pair(w, q, k, v, cq, ck, b, how, out_dtype):
    qn, qr, kn, kr = _split(q, k, how)
    kw = dict(scale=w.softmax_scale, causal=w.causal, window=w.window, attn_bias=b,
              out_dtype=out_dtype, return_lse=True)
    out, lse = fav.varlen_attention(qn, kn, v, cq, ck, w.max_seqlen_q, q_rope=qr, k_rope=kr, **kw)
    ref_out, ref_lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, **kw)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


@pytest.mark.parametrize("how", ["views", "separate"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_split_nope_rope_matches_oracle_and_concatenation(name, how):
    w = CASES[name]
    say(f"[rope] {name} {how}")
    inp = workloads.make_inputs(w)
    q, k, v, cq, ck, b = to_device(inp)
    out, lse, cat_out, cat_lse = _pair(w, q, k, v, cq, ck, b, how, torch.float32)
    assert torch.equal(out, cat_out) and torch.equal(lse, cat_lse)
    ref_out, ref_lse = run_oracle(inp)
    check(name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


def test_split_nope_rope_16bit_output():
    w = CASES["bf16_causal_gqa"]
    inp = workloads.make_inputs(w)
    q, k, v, cq, ck, b = to_device(inp)
    out, lse, cat_out, cat_lse = _pair(w, q, k, v, cq, ck, b, "separate", torch.bfloat16)
    assert out.dtype == torch.bfloat16
    assert torch.equal(out, cat_out) and torch.equal(lse, cat_lse)


def test_split_nope_rope_full_latent_shape():
    """The latent-attention workload at full size (4 x 4096 tokens, 128
    heads, causal): bitwise equal to the concatenated call, sampled rows
    against the oracle."""
    w = workloads.ALL["mla_bf16"]
    say(f"[rope] full {w.name}")
    inp = workloads.make_inputs(w)
    q, k, v, cq, ck, b = to_device(inp)
    # fp32 output: the tolerance covers the kernel's arithmetic, not a final bf16 rounding
    out, lse, cat_out, cat_lse = _pair(w, q, k, v, cq, ck, b, "separate", torch.float32)
    assert torch.equal(out, cat_out) and torch.equal(lse, cat_lse)
    del cat_out, cat_lse, q, k, v
    check_sampled(inp, out, lse, heads=[0, 63, 127], rows_per_seq=8, seed=3)


def test_split_operands_refused_for_grad_and_mismatched_shapes():
    w = CASES["f16_full"]
    inp = workloads.make_inputs(w)
    q, k, v, cq, ck, _ = to_device(inp)
    qn, qr, kn, kr = _split(q, k, "separate")
    with pytest.raises(fav.MiAttnError):
        fav.varlen_attention(qn, kn, v, cq, ck, w.max_seqlen_q, q_rope=qr)
    with pytest.raises(fav.MiAttnError):
        fav.varlen_attention(qn, kn, v, cq, ck, w.max_seqlen_q, q_rope=qr[..., :32],
                             k_rope=kr[..., :32])
    with pytest.raises(fav.MiAttnError):
        fav.varlen_attention(qn.requires_grad_(), kn, v, cq, ck, w.max_seqlen_q, q_rope=qr,
                             k_rope=kr)
