"""In-kernel ALiBi (mi_attn_fwd_params.alibi_slopes / mi_attn_bwd_params
.alibi_slopes) through the C ABI: forward against the fp64 oracle with the
ALiBi bias written out densely (oracle.alibi_bias), bitwise against the
tensor-bias path fed the same bias rounded to fp32 (the kernels' slope times
an exact integer distance is that same fp32 value), and the backward against
the fp64 backward oracle."""
import math

import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import LSE_TOL, OUT_TOL, max_abs, say, to_device

pytestmark = pytest.mark.gpu

W = workloads.Workload

CASES = {
    "bf16_causal_gqa": W(name="alibi_bf16_causal_gqa", seqlens_q=(300, 129, 1),
                         seqlens_kv=(300, 129, 1), hq=8, hkv=2, d_qk=128, d_v=128, dtype="bf16",
                         causal=True, seed=80),
    "f16_full_cross": W(name="alibi_f16_full_cross", seqlens_q=(70, 200), seqlens_kv=(260, 90),
                        hq=4, hkv=4, d_qk=64, d_v=64, dtype="f16", causal=False, seed=81),
    "bf16_window": W(name="alibi_bf16_window", seqlens_q=(400, 77), seqlens_kv=(400, 77), hq=4,
                     hkv=1, d_qk=64, d_v=64, dtype="bf16", causal=True, window=90, seed=82),
    "bf16_latent": W(name="alibi_bf16_latent", seqlens_q=(150, 65), seqlens_kv=(150, 65), hq=2,
                     hkv=2, d_qk=192, d_v=128, dtype="bf16", causal=True, seed=83),
    "f32_causal": W(name="alibi_f32_causal", seqlens_q=(130, 40), seqlens_kv=(130, 40), hq=2,
                    hkv=1, d_qk=64, d_v=64, dtype="f32", causal=True, seed=84),
}


def _slopes(hq, nseq=None):
    # the geometric sequence 2^(-8 h / hq), one slope per head (and per
    # sequence when nseq is given: scaled by the sequence index + 1)
    base = np.array([2.0 ** (-8.0 * (h + 1) / hq) for h in range(hq)], dtype=np.float32)
    if nseq is None:
        return base
    return np.stack([base * (s + 1) for s in range(nseq)]).astype(np.float32)


def _dense_bias(w, inp, slopes):
    return oracle.alibi_bias(slopes.astype(np.float64), inp.cu_seqlens_q.numpy(),
                             inp.cu_seqlens_kv.numpy(), w.hq, w.max_seqlen_kv)


@pytest.mark.parametrize("per_seq", [False, True])
@pytest.mark.parametrize("name", sorted(CASES))
def test_alibi_forward(name, per_seq):
    w = CASES[name]
    say(f"[alibi] fwd {name} per_seq={per_seq}")
    inp = workloads.make_inputs(w)
    q, k, v, cq, ck, _ = to_device(inp)
    sl = _slopes(w.hq, w.num_seqs if per_seq else None)
    sl_d = torch.from_numpy(sl).cuda()
    out, lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale,
                                    causal=w.causal, window=w.window, alibi_slopes=sl_d,
                                    out_dtype=torch.float32, return_lse=True)
    dense = _dense_bias(w, inp, sl)
    # the same bias as a tensor, rounded to fp32 (exact: the kernels' value)
    bt = torch.from_numpy(dense.astype(np.float32)).cuda()
    out_b, lse_b = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale,
                                        causal=w.causal, window=w.window, attn_bias=bt,
                                        out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_b) and torch.equal(lse, lse_b)
    ref_o, ref_l = oracle.varlen_attention(
        inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy(),
        inp.cu_seqlens_q.numpy(), inp.cu_seqlens_kv.numpy(), w.softmax_scale, w.causal, w.window,
        dense)
    eo = max_abs(out.cpu().numpy(), ref_o)
    el = max_abs(lse.cpu().numpy(), ref_l)
    say(f"  max|out-ref|={eo:.3e} max|lse-ref|={el:.3e}")
    assert eo <= OUT_TOL[w.dtype] and el <= LSE_TOL


@pytest.mark.parametrize("name", ["bf16_causal_gqa", "f16_full_cross", "bf16_window"])
def test_alibi_backward(name):
    w = CASES[name]
    say(f"[alibi] bwd {name}")
    inp = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 500)
    dout = torch.randn(w.total_q, w.hq, w.d_v, generator=g).to(inp.q.dtype)
    q, k, v, cq, ck, _ = to_device(inp)
    sl = _slopes(w.hq)
    sl_d = torch.from_numpy(sl).cuda()
    kw = dict(scale=w.softmax_scale, causal=w.causal, window=w.window)
    out, lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, alibi_slopes=sl_d,
                                    return_lse=True, **kw)
    grads = fav.varlen_attention_backward(q, k, v, out, lse, dout.cuda(), cq, ck, w.max_seqlen_q,
                                          w.max_seqlen_kv, grad_dtype=torch.float32,
                                          alibi_slopes=sl_d, **kw)
    dense = _dense_bias(w, inp, sl)
    bt = torch.from_numpy(dense.astype(np.float32)).cuda()
    grads_b = fav.varlen_attention_backward(q, k, v, out, lse, dout.cuda(), cq, ck,
                                            w.max_seqlen_q, w.max_seqlen_kv,
                                            grad_dtype=torch.float32, attn_bias=bt, **kw)
    torch.cuda.synchronize()
    for a, b in zip(grads, grads_b):
        assert torch.equal(a, b)
    ref = oracle.varlen_attention_backward(
        inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy(),
        dout.double().numpy(), inp.cu_seqlens_q.numpy(), inp.cu_seqlens_kv.numpy(),
        w.softmax_scale, w.causal, w.window, dense)
    tol = {"bf16": 6e-3, "f16": 1.5e-3}[w.dtype]
    for gname, gg, r in zip(("dq", "dk", "dv"), grads, ref):
        gg = gg.cpu().numpy().astype(np.float64)
        scale = max(float(np.abs(r).max(initial=0.0)), 1e-3)
        err = float(np.abs(gg - r).max(initial=0.0))
        say(f"  {gname}: {err / scale:.2e} of max|ref|")
        assert err <= tol * scale


def test_alibi_autograd_matches_explicit_backward():
    w = CASES["bf16_causal_gqa"]
    inp = workloads.make_inputs(w)
    q, k, v, cq, ck, _ = to_device(inp)
    sl_d = torch.from_numpy(_slopes(w.hq)).cuda()
    qg, kg, vg = (t.clone().requires_grad_() for t in (q, k, v))
    out = fav.varlen_attention(qg, kg, vg, cq, ck, w.max_seqlen_q, causal=True, alibi_slopes=sl_d,
                               max_seqlen_kv=w.max_seqlen_kv)
    g = torch.Generator().manual_seed(7)
    dout = torch.randn(out.shape, generator=g).to(out.dtype).cuda()
    out.backward(dout)
    o2, l2 = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, causal=True, alibi_slopes=sl_d,
                                  return_lse=True)
    dq, dk, dv = fav.varlen_attention_backward(q, k, v, o2, l2, dout, cq, ck, w.max_seqlen_q,
                                               w.max_seqlen_kv, causal=True, alibi_slopes=sl_d)
    torch.cuda.synchronize()
    assert torch.equal(qg.grad, dq) and torch.equal(kg.grad, dk) and torch.equal(vg.grad, dv)
