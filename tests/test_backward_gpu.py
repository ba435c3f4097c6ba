"""Backward (mi_attn_varlen_bwd) against the fp64 oracle, through the C ABI.

The kernels round P and dS to the input type for the MFMAs (relative error
up to 2^-9 for bf16, 2^-12 for fp16, per term) and take D = rowsum(dout *
out) from the stored 16-bit output; a CPU emulation of that arithmetic on
N(0,1) inputs of these shapes errs by up to 2.8e-3 (bf16) and 5.6e-4 (fp16)
of the largest gradient magnitude.  The tolerances below are about twice
that, relative to each tensor's largest reference magnitude, on fp32
gradients; the 16-bit gradients must be the RNE rounding of the fp32 ones,
bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import say

pytestmark = pytest.mark.gpu

W = workloads.Workload
GRAD_TOL = {"bf16": 6e-3, "f16": 1.5e-3}


def _inputs(w, seed):
    inp = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn(w.total_q, w.hq, w.d_v, generator=g).to(inp.q.dtype)
    return inp, dout


def _run(inp, dout, grad_dtype=torch.float32, dev=None):
    w = inp.workload
    d = "cuda"
    q, k, v = inp.q.to(d), inp.k.to(d), inp.v.to(d)
    cq, ck = inp.cu_seqlens_q.to(d), inp.cu_seqlens_kv.to(d)
    out, lse = fav.varlen_attention(q, k, v, cq, ck, max(w.max_seqlen_q, 1), scale=w.softmax_scale,
                                    causal=w.causal, window=w.window, return_lse=True)
    grads = fav.varlen_attention_backward(q, k, v, out, lse, dout.to(d), cq, ck,
                                          max(w.max_seqlen_q, 1), max(w.max_seqlen_kv, 1),
                                          scale=w.softmax_scale, causal=w.causal, window=w.window,
                                          grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return grads


def _check(name, got, ref, dtype):
    for gname, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.float().cpu().numpy().astype(np.float64)
        scale = max(float(np.abs(r).max(initial=0.0)), 1e-3)
        err = float(np.abs(g - r).max(initial=0.0))
        say(f"  {name} {gname}: max err {err:.3e} = {err / scale:.2e} of max|ref| {scale:.3g}")
        assert np.isfinite(g).all()
        assert err <= GRAD_TOL[dtype] * scale, f"{name} {gname}: {err / scale:.3e} of max|ref|"


def _oracle(inp, dout, **kw):
    w = inp.workload
    return oracle.varlen_attention_backward(inp.q.double().numpy(), inp.k.double().numpy(),
                                            inp.v.double().numpy(), dout.double().numpy(),
                                            inp.cu_seqlens_q.numpy(), inp.cu_seqlens_kv.numpy(),
                                            w.softmax_scale, w.causal, w.window, None, **kw)


def _cases():
    c = {}
    for dt in ("bf16", "f16"):
        for d in (64, 128):
            c[f"gqa_causal_{dt}_d{d}"] = W(name="b", seqlens_q=(300, 1, 129, 64),
                                           seqlens_kv=(300, 1, 129, 64), hq=8, hkv=2, d_qk=d,
                                           d_v=d, dtype=dt, causal=True, seed=80 + d)
            c[f"full_{dt}_d{d}"] = W(name="b", seqlens_q=(200, 77), seqlens_kv=(200, 77), hq=3,
                                     hkv=3, d_qk=d, d_v=d, dtype=dt, causal=False, seed=81 + d)
    c["gqa_causal_bf16_d96"] = W(name="b", seqlens_q=(300, 1, 129, 64), seqlens_kv=(300, 1, 129, 64),
                                 hq=8, hkv=2, d_qk=96, d_v=96, dtype="bf16", causal=True, seed=83)
    c["full_f16_d96"] = W(name="b", seqlens_q=(200, 77), seqlens_kv=(200, 77), hq=3, hkv=3, d_qk=96,
                          d_v=96, dtype="f16", causal=False, seed=84)
    c["window_bf16_d128"] = W(name="b", seqlens_q=(500, 90), seqlens_kv=(500, 90), hq=4, hkv=1,
                              d_qk=128, d_v=128, dtype="bf16", causal=True, window=70, seed=82)
    c["cross_kv_longer_f16_d64"] = W(name="b", seqlens_q=(5, 130, 1), seqlens_kv=(700, 260, 90),
                                     hq=4, hkv=2, d_qk=64, d_v=64, dtype="f16", causal=True,
                                     seed=83)
    c["cross_kv_shorter_bf16_d64"] = W(name="b", seqlens_q=(200, 64), seqlens_kv=(70, 3), hq=2,
                                       hkv=1, d_qk=64, d_v=64, dtype="bf16", causal=True, seed=84)
    c["cross_window_bf16_d128"] = W(name="b", seqlens_q=(150, 40), seqlens_kv=(400, 41), hq=4,
                                    hkv=2, d_qk=128, d_v=128, dtype="bf16", causal=True, window=77,
                                    seed=85)
    c["empty_sequences_f16_d128"] = W(name="b", seqlens_q=(0, 50, 0, 3, 9),
                                      seqlens_kv=(0, 50, 7, 0, 9), hq=2, hkv=2, d_qk=128, d_v=128,
                                      dtype="f16", causal=False, seed=86)
    c["mqa_bf16_d64"] = W(name="b", seqlens_q=(257, 190), seqlens_kv=(257, 190), hq=8, hkv=1,
                          d_qk=64, d_v=64, dtype="bf16", causal=True, seed=87)
    return c


CASES = _cases()


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_oracle(name):
    w = CASES[name].with_(name=name)
    say(f"[bwd] {name}: q {w.seqlens_q} kv {w.seqlens_kv} hq={w.hq} hkv={w.hkv} d={w.d_qk} "
        f"causal={w.causal} window={w.window}")
    inp, dout = _inputs(w, seed=90)
    g32 = _run(inp, dout, torch.float32)
    _check(name, g32, _oracle(inp, dout), w.dtype)
    g16 = _run(inp, dout, inp.q.dtype)
    for a, b in zip(g16, g32):
        assert torch.equal(a, b.to(inp.q.dtype)), "16-bit gradients are not RNE(fp32 gradients)"


def test_backward_is_deterministic():
    w = CASES["gqa_causal_bf16_d128"]
    inp, dout = _inputs(w, seed=91)
    a = _run(inp, dout, torch.float32)
    b = _run(inp, dout, torch.float32)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_autograd_through_varlen_attention(dtype):
    """varlen_attention with inputs that require grad is differentiable; its
    gradients equal the direct backward call's bit for bit."""
    w = W(name="ag", seqlens_q=(130, 61), seqlens_kv=(130, 61), hq=4, hkv=2, d_qk=64, d_v=64,
          dtype=dtype, causal=True, seed=92)
    inp, dout = _inputs(w, seed=93)
    d = "cuda"
    q, k, v = (t.to(d).requires_grad_() for t in (inp.q, inp.k, inp.v))
    cq, ck = inp.cu_seqlens_q.to(d), inp.cu_seqlens_kv.to(d)
    out = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, causal=True)
    gq, gk, gv = torch.autograd.grad(out, (q, k, v), dout.to(d))
    ref = _run(inp, dout, inp.q.dtype)
    for a, b in zip((gq, gk, gv), ref):
        assert torch.equal(a, b)


def test_full_size_backward_sampled():
    """The bench workload (bf16 causal GQA, 8 sequences, T = 20205, Hq = 32,
    Hkv = 8, D = 128): dq / dk / dv of one kv head (its four query heads) in
    the shortest and longest sequences against the oracle."""
    w = workloads.ALL["gqa_causal_bf16"]
    inp, dout = _inputs(w, seed=94)
    say("[bwd full] gqa_causal_bf16")
    g32 = _run(inp, dout, torch.float32)
    seqs, kvh = [4, 5], [3]
    ref = _oracle(inp, dout, seqs=seqs, kv_heads=kvh)
    cq, ck = inp.cu_seqlens_q.numpy(), inp.cu_seqlens_kv.numpy()
    rows = np.concatenate([np.arange(cq[s], cq[s + 1]) for s in seqs])
    keys = np.concatenate([np.arange(ck[s], ck[s + 1]) for s in seqs])
    heads = [h for h in range(w.hq) if h // (w.hq // w.hkv) in kvh]
    got = (g32[0].cpu()[rows][:, heads], g32[1].cpu()[keys][:, kvh], g32[2].cpu()[keys][:, kvh])
    want = (ref[0][rows][:, heads], ref[1][keys][:, kvh], ref[2][keys][:, kvh])
    _check("gqa_causal_bf16", got, want, "bf16")


@pytest.mark.parametrize("bias_heads", [1, "hq"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_backward_with_constant_bias(dtype, d, bias_heads):
    """A constant additive bias with -inf entries (and a row that sees
    nothing), shared by all heads or one per query head."""
    w = W(name=f"bwd_bias_{dtype}_{d}_{bias_heads}", seqlens_q=(190, 75), seqlens_kv=(260, 75),
          hq=4, hkv=2, d_qk=d, d_v=d, dtype=dtype, causal=True, seed=95)
    inp, dout = _inputs(w, seed=96)
    nb = w.hq if bias_heads == "hq" else 1
    bias = workloads.random_bias(w.seqlens_q, nb, 272, seed=97, neg_inf_frac=0.2)
    bias[7] = float("-inf")
    say(f"[bwd bias] {w.name}")
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    b = bias.to(dev)
    out, lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, causal=True, attn_bias=b,
                                    return_lse=True)
    g32 = fav.varlen_attention_backward(q, k, v, out, lse, dout.to(dev), cq, ck, w.max_seqlen_q,
                                        w.max_seqlen_kv, causal=True, attn_bias=b,
                                        grad_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.varlen_attention_backward(inp.q.double().numpy(), inp.k.double().numpy(),
                                           inp.v.double().numpy(), dout.double().numpy(),
                                           inp.cu_seqlens_q.numpy(), inp.cu_seqlens_kv.numpy(),
                                           w.softmax_scale, True, 0, bias.double().numpy())
    _check(w.name, g32, ref, dtype)
    # the same through autograd, with the bias as a bool mask where it is 0 / -inf
    qg, kg, vg = (t.clone().requires_grad_() for t in (q, k, v))
    o = fav.varlen_attention(qg, kg, vg, cq, ck, w.max_seqlen_q, causal=True, attn_bias=b)
    gq, gk, gv = torch.autograd.grad(o, (qg, kg, vg), dout.to(dev))
    g16 = fav.varlen_attention_backward(q, k, v, out, lse, dout.to(dev), cq, ck, w.max_seqlen_q,
                                        w.max_seqlen_kv, causal=True, attn_bias=b)
    for x, y in zip((gq, gk, gv), g16):
        assert torch.equal(x, y)


def test_bias_that_requires_grad_is_refused():
    w = W(name="bwd_bias_grad", seqlens_q=(20,), seqlens_kv=(20,), hq=2, hkv=2, d_qk=64, d_v=64,
          dtype="bf16", causal=False, seed=98)
    inp = workloads.make_inputs(w)
    dev = "cuda"
    q = inp.q.to(dev).requires_grad_()
    b = torch.zeros(20, 1, 20, device=dev, requires_grad=True)
    with pytest.raises(fav.MiAttnError):
        fav.varlen_attention(q, inp.k.to(dev), inp.v.to(dev), inp.cu_seqlens_q.to(dev),
                             inp.cu_seqlens_kv.to(dev), 20, attn_bias=b)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_packed_wrappers_forward_and_backward(dtype):
    """flash_attn_varlen_qkvpacked_func / _kvpacked_func: views of one packed
    tensor go to the C ABI as they are; the outputs equal the unpacked call
    and the gradients land in the packed tensors."""
    lens = (130, 1, 67)
    w = W(name="packed_bwd", seqlens_q=lens, seqlens_kv=lens, hq=4, hkv=4, d_qk=64, d_v=64,
          dtype=dtype, causal=True, seed=99)
    inp, dout = _inputs(w, seed=100)
    dev = "cuda"
    cu = inp.cu_seqlens_q.to(dev)
    qkv = torch.stack([inp.q, inp.k, inp.v], dim=1).to(dev).requires_grad_()
    out = fav.flash_attn_varlen_qkvpacked_func(qkv, cu, w.max_seqlen_q, causal=True)
    (g_qkv,) = torch.autograd.grad(out, (qkv,), dout.to(dev))
    ref = _run(inp, dout, inp.q.dtype)
    assert torch.equal(g_qkv[:, 0], ref[0]) and torch.equal(g_qkv[:, 1], ref[1])
    assert torch.equal(g_qkv[:, 2], ref[2])
    q = inp.q.to(dev).requires_grad_()
    kv = torch.stack([inp.k, inp.v], dim=1).to(dev).requires_grad_()
    out2 = fav.flash_attn_varlen_kvpacked_func(q, kv, cu, cu, w.max_seqlen_q, w.max_seqlen_kv,
                                               causal=True)
    assert torch.equal(out2, out)
    gq, gkv = torch.autograd.grad(out2, (q, kv), dout.to(dev))
    assert torch.equal(gq, ref[0]) and torch.equal(gkv[:, 0], ref[1]) and torch.equal(gkv[:, 1], ref[2])
