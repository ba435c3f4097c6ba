"""Key-padding front end at the C ABI (mtlattn 0.3.0 page, section "Drop-in
for scaled_dot_product_attention"): ranks / cu_seqlens and the gather /
scatter bit-exact against the oracle, and the dense ``sdpa`` adapter (key
padding packed to varlen, other masks as an additive bias) against the fp64
oracle's dense definition."""
import math

import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
from gpu_helpers import LSE_TOL, OUT_TOL, max_abs, say

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _mask(bsz, n, seed, p=0.7):
    g = torch.Generator().manual_seed(seed)
    m = torch.rand(bsz, n, generator=g) < p
    if bsz > 2:
        m[0] = True        # full row
        m[1] = False       # all padding
        m[2, : n // 2] = False  # left padding
    return m


@pytest.mark.parametrize("bsz,n", [(3, 5), (7, 300), (1500, 33), (2, 1000), (4, 0), (0, 8)])
def test_padding_to_varlen_matches_oracle(bsz, n):
    say(f"[padding] ranks B={bsz} N={n}")
    m = _mask(bsz, n, seed=bsz * 7 + n)
    ranks, cu, total, longest = fav.padding_to_varlen(m.cuda())
    r_ref, cu_ref, (t_ref, l_ref) = oracle.padding_to_varlen(m.numpy())
    assert np.array_equal(ranks.cpu().numpy(), r_ref)
    assert np.array_equal(cu.cpu().numpy(), cu_ref)
    assert (total, longest) == (t_ref, l_ref)


def test_padding_mask_row_stride_view():
    """A [B, 1, 1, N] bool key-padding mask viewed as [B, N] (batch stride N)
    and a sliced mask with a batch stride larger than N."""
    m = _mask(6, 40, seed=5)
    wide = torch.zeros(6, 64, dtype=torch.bool)
    wide[:, :40] = m
    for view in (m.cuda()[:, None, None, :][:, 0, 0, :], wide.cuda()[:, :40]):
        ranks, cu, total, longest = fav.padding_to_varlen(view)
        r_ref, cu_ref, stats = oracle.padding_to_varlen(m.numpy())
        assert np.array_equal(ranks.cpu().numpy(), r_ref) and (total, longest) == stats


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_pack_unpack_bit_exact(dtype, layout):
    bsz, n, h, d = 5, 77, 3, 64
    say(f"[padding] pack {dtype} {layout}")
    m = _mask(bsz, n, seed=11)
    g = torch.Generator().manual_seed(12)
    x = torch.randn(bsz, n, h, d, generator=g).to(DT[dtype])
    xd = x.cuda() if layout == "token_major" else x.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    ranks, cu, total, _ = fav.padding_to_varlen(m.cuda())
    packed = fav.pack_tokens(xd, ranks, cu, total)
    ref = oracle.pack_tokens(x.float().numpy(), m.numpy())
    assert packed.shape == (total, h, d)
    assert np.array_equal(packed.float().cpu().numpy(), ref)
    out = torch.full((bsz, h, n, d), 7.0, dtype=DT[dtype], device="cuda").transpose(1, 2)
    fav.unpack_tokens(packed, out, ranks, cu)
    back = oracle.unpack_tokens(ref, m.numpy())
    assert np.array_equal(out.float().cpu().numpy(), back)
    # all valid (ranks None): packed row = b * n + token
    allp = fav.pack_tokens(xd)
    assert torch.equal(allp.cpu(), x.reshape(bsz * n, h, d))


def _sdpa_inputs(bsz, hq, hkv, nq, nkv, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(bsz, hq, nq, d, generator=g).to(DT[dtype])
    k = torch.randn(bsz, hkv, nkv, d, generator=g).to(DT[dtype])
    v = torch.randn(bsz, hkv, nkv, d, generator=g).to(DT[dtype])
    return q, k, v


def _check(name, got, ref, dtype, rows=None):
    got = got.float().cpu().numpy()
    if rows is not None:
        got, ref = got[rows], ref[rows]
    e = max_abs(got, ref)
    say(f"  {name}: max|out-ref|={e:.3e} (tol {OUT_TOL[dtype]:.0e})")
    assert e <= OUT_TOL[dtype], e


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 8, 2), ("f16", 64, 4, 4)])
def test_sdpa_key_padding_self_attention(causal, dtype, d, hq, hkv):
    bsz, n = 4, 333
    say(f"[padding] sdpa key padding causal={causal} {dtype} d={d}")
    q, k, v = _sdpa_inputs(bsz, hq, hkv, n, n, d, dtype, seed=40 + d)
    m = _mask(bsz, n, seed=41)
    am = m[:, None, None, :].cuda()
    out = fav.sdpa(q.cuda(), k.cuda(), v.cuda(), attn_mask=am, is_causal=causal,
                   enable_gqa=hq != hkv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.masked_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  m.numpy(), 1.0 / math.sqrt(d), causal)
    _check("sdpa_key_padding", out, ref, dtype)
    # the input-dtype output is the fp32 result rounded once
    out16 = fav.sdpa(q.cuda(), k.cuda(), v.cuda(), attn_mask=am, is_causal=causal,
                     enable_gqa=hq != hkv)
    assert out16.dtype == DT[dtype] and torch.equal(out16, out.to(DT[dtype]))


def test_sdpa_key_padding_cross_attention():
    """Nq != Nkv: the keys are packed, every query row is computed."""
    bsz, nq, nkv, d = 3, 50, 200, 64
    q, k, v = _sdpa_inputs(bsz, 2, 2, nq, nkv, d, "bf16", seed=50)
    m = _mask(bsz, nkv, seed=51)
    out = fav.sdpa(q.cuda(), k.cuda(), v.cuda(), attn_mask=m[:, None, None, :].cuda(),
                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = np.zeros(out.shape)
    for b in range(bsz):
        for h in range(2):
            z = (qd[b, h] @ kd[b, h].T) / math.sqrt(d)
            z = np.where(m[b].numpy()[None, :], z, -np.inf)
            if not m[b].any():
                continue
            p = np.exp(z - z.max(axis=1, keepdims=True))
            ref[b, h] = (p / p.sum(axis=1, keepdims=True)) @ vd[b, h]
    _check("sdpa_cross_key_padding", out, ref, "bf16")


@pytest.mark.parametrize("kind", ["bool_2d", "float_4d_heads", "bool_broadcast_batch"])
def test_sdpa_general_mask_as_bias(kind):
    bsz, h, nq, nkv, d = 2, 4, 130, 97, 64
    q, k, v = _sdpa_inputs(bsz, h, h, nq, nkv, d, "bf16", seed=60)
    g = torch.Generator().manual_seed(61)
    if kind == "bool_2d":
        mask = torch.rand(nq, nkv, generator=g) < 0.5
        mask[:, 0] = True
        dense = torch.zeros(nq, nkv, dtype=torch.float64).masked_fill(~mask, -math.inf)
        dense = dense.expand(bsz, 1, nq, nkv)
    elif kind == "float_4d_heads":
        mask = torch.randn(bsz, h, nq, nkv, generator=g)
        dense = mask.double()
    else:
        mask = torch.rand(1, 1, nq, nkv, generator=g) < 0.8
        mask[..., 0] = True
        dense = torch.zeros(1, 1, nq, nkv, dtype=torch.float64).masked_fill(~mask, -math.inf)
        dense = dense.expand(bsz, 1, nq, nkv)
    out = fav.sdpa(q.cuda(), k.cuda(), v.cuda(), attn_mask=mask.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    # oracle: varlen attention of the batch as sequences, the mask as its bias rows
    cu_q = np.arange(bsz + 1, dtype=np.int64) * nq
    cu_k = np.arange(bsz + 1, dtype=np.int64) * nkv
    qd = q.double().permute(0, 2, 1, 3).reshape(bsz * nq, h, d).numpy()
    kd = k.double().permute(0, 2, 1, 3).reshape(bsz * nkv, h, d).numpy()
    vd = v.double().permute(0, 2, 1, 3).reshape(bsz * nkv, h, d).numpy()
    bias = dense.permute(0, 2, 1, 3).reshape(bsz * nq, dense.shape[1], nkv).numpy()
    ref, _ = oracle.varlen_attention(qd, kd, vd, cu_q, cu_k, 1.0 / math.sqrt(d), False, 0, bias)
    ref = ref.reshape(bsz, nq, h, d).transpose(0, 2, 1, 3)
    _check(f"sdpa_{kind}", out, ref, "bf16")


def test_sdpa_refusals():
    q, k, v = _sdpa_inputs(1, 2, 2, 10, 12, 64, "bf16", seed=70)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    with pytest.raises(fav.MiAttnError):
        fav.sdpa(q, k, v, is_causal=True)  # Nq != Nkv: top-left diagonal
    with pytest.raises(fav.MiAttnError):
        fav.sdpa(q, k, v, dropout_p=0.1)
    with pytest.raises(fav.MiAttnError):
        fav.sdpa(q, k[:, :1], v[:, :1])  # fewer kv heads without enable_gqa
