"""Interval rows through the C ABI: the key-range pass's per-row flag (the
row's bias is exactly 0 on its key range and -inf elsewhere) against the
oracle, integer-exact; and the forward that masks such rows to their range
instead of reading their bias: equal to the forward that reads the bias,
bit for bit, and within tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import check, run_oracle, say

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _interval_bias(seqlens, heads, cols, seed, impure_every=0, seqlens_kv=None):
    """fp32 bias whose rows are 0 on a random key interval (causal-like,
    window-like or arbitrary) and -inf elsewhere; with impure_every > 0,
    every impure_every-th row is spoiled in one of four ways (a -inf hole, a
    nonzero value, a NaN-free negative value, or -0.0, which stays pure).
    Key intervals lie within each sequence's key length (seqlens_kv, by
    default the query lengths)."""
    g = torch.Generator().manual_seed(seed)
    tq = int(sum(seqlens))
    b = torch.full((tq, heads, cols), float("-inf"))
    t0 = 0
    for nq, n in zip(seqlens, seqlens_kv or seqlens):
        for r in range(nq):
            i = min(r, n - 1)  # the row's position among the keys (clamped)
            for h in range(heads):
                kind = int(torch.randint(0, 3, (1,), generator=g))
                if kind == 0:      # causal with a prefix
                    lo, hi = 0, max(min(n, 17), i + 1)
                elif kind == 1:    # a window ending at the diagonal
                    hi = i + 1
                    lo = max(0, hi - int(torch.randint(1, 64, (1,), generator=g)))
                else:              # anywhere
                    lo = int(torch.randint(0, n, (1,), generator=g))
                    hi = int(torch.randint(lo + 1, n + 1, (1,), generator=g))
                b[t0 + r, h, lo:hi] = 0.0
                if impure_every and (t0 + r) % impure_every == 0 and hi - lo >= 3:
                    how = (t0 + r) // impure_every % 4
                    mid = (lo + hi) // 2
                    b[t0 + r, h, mid] = [float("-inf"), 0.75, -2.0, -0.0][how]
        t0 += nq
    return b


@pytest.mark.parametrize("kind", ["prefix_lm", "intervals", "mixed", "banded", "mask_mixed"])
def test_interval_flags_match_oracle(kind):
    lens_q, lens_k = (300, 1, 129, 64), (300, 7, 129, 90)
    if kind == "prefix_lm":
        bias = workloads.prefix_lm_bias(lens_q, 100, 300)
        lens_k = lens_q
    elif kind == "banded":
        g = torch.Generator().manual_seed(80)
        bias = torch.randn(sum(lens_q), 2, 301, generator=g)
        bias.masked_fill_(torch.rand(bias.shape, generator=g) < 0.3, float("-inf"))
    else:
        lens_k = lens_q
        bias = _interval_bias(lens_q, 3, 301, seed=81, impure_every=0 if kind == "intervals" else 5)
    cq, ck = workloads.cu_seqlens(lens_q), workloads.cu_seqlens(lens_k)
    dev_bias = bias.cuda()
    if kind == "mask_mixed":
        # the same rows as a bool mask: True where the bias is finite (a
        # nonzero finite value is visible, so only holes spoil a mask row)
        dev_bias = torch.isfinite(dev_bias)
        bias = torch.zeros(bias.shape).masked_fill_(~torch.isfinite(bias), float("-inf"))
    say(f"[interval flags] {kind} bias {tuple(bias.shape)}")
    rg, pure = fav.bias_key_ranges(dev_bias, cq.cuda(), ck.cuda(), max(lens_q), return_pure=True)
    torch.cuda.synchronize()
    ref_rg = oracle.bias_key_ranges(bias.numpy(), cq.numpy(), ck.numpy())
    ref_pure = oracle.bias_rows_are_intervals(bias.numpy(), cq.numpy(), ck.numpy())
    assert np.array_equal(rg.cpu().numpy().astype(np.int64), ref_rg)
    assert np.array_equal(pure.cpu().numpy(), ref_pure)
    n_pure = int(ref_pure.sum())
    say(f"  interval rows: {n_pure} of {ref_pure.size}")
    if kind in ("prefix_lm", "intervals"):
        assert n_pure == ref_pure.size
    elif kind == "banded":
        assert n_pure < ref_pure.size
    else:
        assert 0 < n_pure < ref_pure.size


@pytest.mark.parametrize("case", ["prefix_f16_d128", "prefix_bf16_d64", "intervals_bf16_d128",
                                  "mixed_f16_d128", "mixed_bf16_d64", "intervals_bf16_d192",
                                  "intervals_f16_d256", "intervals_bf16_d96", "mask_f16_d128",
                                  "intervals_f32_d64", "causal_bf16_d128", "window_f16_d64",
                                  "cross_bf16_d128"])
def test_forward_with_interval_rows_is_exact(case):
    """A wave whose rows are all intervals reads no bias and masks each row
    to its range: output and LSE equal, bit for bit, those of the forward
    that reads the bias (with and without the key ranges), the same tiles
    are visited as with the ranges alone, and all match the oracle."""
    kind, dt, d = case.split("_")
    d = int(d[1:])
    dqk, dv = (192, 128) if d == 192 else (d, d)
    lens = (700, 257, 1) if kind == "prefix" else (500, 130, 33)
    # cross attention: more keys than queries in one sequence, fewer in another
    lens_kv = (620, 90, 33) if kind == "cross" else lens
    hq = 4
    # the masks compose with the interval rows (causal / window flags too)
    causal = kind in ("causal", "window", "cross")
    w = W(name=f"interval_{case}", seqlens_q=lens, seqlens_kv=lens_kv, hq=hq, hkv=2, d_qk=dqk,
          d_v=dv, dtype=dt, causal=causal, window=100 if kind == "window" else 0, seed=82)
    inp = workloads.make_inputs(w)
    if kind == "prefix":
        inp.bias = workloads.prefix_lm_bias(lens, 100, max(lens))
    else:
        inp.bias = _interval_bias(lens, hq if kind != "mask" else 1, max(lens_kv), seed=83,
                                  impure_every=37 if kind == "mixed" else 0, seqlens_kv=lens_kv)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    b = inp.bias.to(dev)
    if kind == "mask":
        b = torch.isfinite(b)
    bm, _ = fav.mi_attn_tile_shape({"bf16": fav.BF16, "f16": fav.F16, "f32": fav.F32}[dt], dqk, dv)
    n_qt = (w.max_seqlen_q + bm - 1) // bm
    tc1 = torch.zeros(n_qt * w.num_seqs * hq, dtype=torch.int32, device=dev)
    tc2 = torch.zeros_like(tc1)
    say(f"[interval fwd] {case}")
    flags = dict(causal=w.causal, window=w.window)
    kw = dict(attn_bias=b, out_dtype=torch.float32, return_lse=True, **flags)
    out0, lse0 = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, **kw)
    rg, pure = fav.bias_key_ranges(b, cq, ck, w.max_seqlen_q, return_pure=True)
    out1, lse1 = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, bias_ranges=rg,
                                      tile_counts=tc1, **kw)
    out2, lse2 = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, bias_ranges=rg,
                                      bias_pure=pure, tile_counts=tc2, **kw)
    # the input-type output too (the timed configuration)
    o16 = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=b, bias_ranges=rg,
                               **flags)
    o16p = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=b, bias_ranges=rg,
                                bias_pure=pure, **flags)
    torch.cuda.synchronize()
    say(f"  interval rows {int(pure.sum())} of {pure.numel()}")
    assert torch.equal(out2, out1) and torch.equal(lse2, lse1), "interval masking changed the result"
    assert torch.equal(out1, out0) and torch.equal(lse1, lse0)
    assert torch.equal(o16p, o16)
    assert torch.equal(tc2, tc1)
    if kind == "mask":
        inp.bias = torch.zeros(inp.bias.shape).masked_fill_(~torch.isfinite(inp.bias), float("-inf"))
    ref_out, ref_lse = run_oracle(inp)
    check(case, out2.cpu().numpy(), lse2.cpu().numpy(), ref_out, ref_lse, w.dtype)


def test_interval_rows_refusals():
    """bias_pure needs the ranges it came with, of the right shape."""
    lens = (64, 10)
    w = W(name="interval_refusal", seqlens_q=lens, seqlens_kv=lens, hq=2, hkv=2, d_qk=64, d_v=64,
          dtype="bf16", causal=False, seed=84)
    inp = workloads.make_inputs(w)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    b = workloads.prefix_lm_bias(lens, 8).to(dev)
    rg, pure = fav.bias_key_ranges(b, cq, ck, w.max_seqlen_q, return_pure=True)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=b, bias_pure=pure)
    assert ei.value.code == fav.ERR_INVALID_ARG
    with pytest.raises(fav.MiAttnError) as ei:
        fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, attn_bias=b, bias_ranges=rg,
                             bias_pure=pure[:, :-1].contiguous())
    assert ei.value.code == fav.ERR_INVALID_ARG
