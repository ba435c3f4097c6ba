"""Mask front-ends through the C ABI: the bias key-range pass against the
oracle (integer-exact), and the forward with those ranges skipping -inf
tiles: bitwise equal to the forward without them, fewer tiles visited,
and within tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import check, run_oracle, say

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _banded_bias(seqlens, heads, cols, seed):
    """Random fp32 bias whose rows are -inf outside a random band, with some
    rows -inf everywhere and scattered -inf inside the band."""
    g = torch.Generator().manual_seed(seed)
    tq = int(sum(seqlens))
    b = torch.randn(tq, heads, cols, generator=g)
    lo = torch.randint(0, cols, (tq, heads, 1), generator=g)
    width = torch.randint(0, cols, (tq, heads, 1), generator=g)
    j = torch.arange(cols).view(1, 1, cols)
    b.masked_fill_((j < lo) | (j >= lo + width), float("-inf"))
    b.masked_fill_(torch.rand(tq, heads, cols, generator=g) < 0.1, float("-inf"))
    b[::17] = float("-inf")
    return b


@pytest.mark.parametrize("kind", ["prefix_lm", "banded_per_head", "banded_shared"])
def test_bias_key_ranges_match_oracle(kind):
    lens_q, lens_k = (300, 1, 129, 64), (300, 7, 129, 90)
    if kind == "prefix_lm":
        bias = workloads.prefix_lm_bias(lens_q, 100, 300)
        lens_k = lens_q
    else:
        bias = _banded_bias(lens_q, 3 if kind == "banded_per_head" else 1, 301, seed=70)
    cq, ck = workloads.cu_seqlens(lens_q), workloads.cu_seqlens(lens_k)
    say(f"[ranges] {kind} bias {tuple(bias.shape)}")
    got = fav.bias_key_ranges(bias.cuda(), cq.cuda(), ck.cuda(), max(lens_q))
    torch.cuda.synchronize()
    ref = oracle.bias_key_ranges(bias.numpy(), cq.numpy(), ck.numpy())
    assert np.array_equal(got.cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("case", ["prefix_f16_d128", "prefix_bf16_d64", "banded_bf16_d128",
                                  "banded_f16_d192", "banded_f32_d64"])
def test_forward_with_ranges_is_exact(case):
    """Skipping the tiles outside the rows' key ranges changes nothing: the
    output and LSE are bitwise equal to the run that visits every tile, and
    both match the oracle."""
    kind, dt, d = case.split("_")
    d = int(d[1:])
    dqk, dv = (192, 128) if d == 192 else (d, d)
    lens = (700, 257, 1) if kind == "prefix" else (500, 130)
    hq = 4
    w = W(name=f"ranges_{case}", seqlens_q=lens, seqlens_kv=lens, hq=hq, hkv=2, d_qk=dqk, d_v=dv,
          dtype=dt, causal=False, seed=71)
    inp = workloads.make_inputs(w)
    if kind == "prefix":
        inp.bias = workloads.prefix_lm_bias(lens, 100, max(lens))
    else:
        inp.bias = _banded_bias(lens, hq, max(lens), seed=72)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    b = inp.bias.to(dev)
    bm, bn = fav.mi_attn_tile_shape({"bf16": fav.BF16, "f16": fav.F16, "f32": fav.F32}[dt], dqk, dv)
    n_qt = (w.max_seqlen_q + bm - 1) // bm
    tc0 = torch.zeros(n_qt * w.num_seqs * hq, dtype=torch.int32, device=dev)
    tc1 = torch.zeros_like(tc0)
    say(f"[ranges fwd] {case}")
    out0, lse0 = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=b,
                                      out_dtype=torch.float32, return_lse=True, tile_counts=tc0)
    rg = fav.bias_key_ranges(b, cq, ck, w.max_seqlen_q)
    out1, lse1 = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=b,
                                      out_dtype=torch.float32, return_lse=True, tile_counts=tc1,
                                      bias_ranges=rg)
    torch.cuda.synchronize()
    say(f"  tiles visited: {int(tc0.sum())} -> {int(tc1.sum())}")
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1), "skipping changed the result"
    assert int(tc1.sum()) < int(tc0.sum())
    ref_out, ref_lse = run_oracle(inp)
    check(case, out1.cpu().numpy(), lse1.cpu().numpy(), ref_out, ref_lse, w.dtype)


# ---------------------------------------------------------------- byte masks
def _bool_mask(seqlens, heads, cols, seed):
    """True = visible: the finite entries of the banded bias."""
    return torch.isfinite(_banded_bias(seqlens, heads, cols, seed))


@pytest.mark.parametrize("case", ["bf16_d128_h1", "f16_d64_hq", "bf16_d192_hq", "f32_d64_h1",
                                  "bf16_d256_h1", "f16_d96_hq"])
@pytest.mark.parametrize("flags", ["full", "causal_window"])
def test_byte_mask_equals_fp32_bias(case, flags):
    """A bool mask read by the kernels as bytes gives bit for bit the result
    of the same mask as an fp32 0 / -inf bias (same logits, same sums); odd
    column counts go through the padded copy; the key ranges of the mask
    equal those of the bias and skipping with them changes nothing."""
    dt, d, h = case.split("_")
    d = int(d[1:])
    dqk, dv = (192, 128) if d == 192 else (d, d)
    lens = (300, 1, 77)
    hq = 4
    causal = flags != "full"
    w = W(name=f"bytemask_{case}", seqlens_q=lens, seqlens_kv=lens, hq=hq, hkv=2, d_qk=dqk, d_v=dv,
          dtype=dt, causal=causal, window=90 if causal else 0, seed=73)
    inp = workloads.make_inputs(w)
    mask = _bool_mask(lens, 1 if h == "h1" else hq, 301, seed=74)
    fbias = torch.zeros(mask.shape).masked_fill_(~mask, float("-inf"))
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    say(f"[byte mask] {case} {flags}")
    kw = dict(causal=causal, window=w.window, out_dtype=torch.float32, return_lse=True)
    out_m, lse_m = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=mask.to(dev), **kw)
    out_b, lse_b = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=fbias.to(dev), **kw)
    rg_m = fav.bias_key_ranges(mask.to(dev), cq, ck, w.max_seqlen_q)
    rg_b = fav.bias_key_ranges(fbias.to(dev), cq, ck, w.max_seqlen_q)
    out_r, lse_r = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=mask.to(dev),
                                        bias_ranges=rg_m, **kw)
    torch.cuda.synchronize()
    assert torch.equal(rg_m, rg_b)
    assert torch.equal(out_m, out_b) and torch.equal(lse_m, lse_b)
    assert torch.equal(out_r, out_m) and torch.equal(lse_r, lse_m)
    inp.bias = fbias
    ref_out, ref_lse = run_oracle(inp)
    check(f"bytemask_{case}", out_m.cpu().numpy(), lse_m.cpu().numpy(), ref_out, ref_lse, w.dtype)
