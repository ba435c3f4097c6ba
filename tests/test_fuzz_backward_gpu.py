"""A seeded fuzzer for the backward (mi_attn_varlen_bwd) through the C ABI,
against the fp64 oracle: bf16 / fp16, head dims 64, 96 and 128, GQA ratios,
self- and cross-attention with empty and ragged sequences, causal and
window flags, and no bias, an fp32 bias (1 or Hq heads, with -inf entries)
or ALiBi slopes.  The tolerances are those of the backward parity tests
(relative to each gradient's largest reference magnitude)."""
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


def _case(i):
    rng = np.random.default_rng(11000 + i)
    dtype = ["bf16", "f16"][rng.integers(2)]
    d = int(rng.choice([64, 96, 128]))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    ns = int(rng.integers(1, 4))
    sq = [int(x) for x in rng.integers(0, 200, ns)]
    self_attn = rng.random() < 0.7
    sk = sq if self_attn else [int(x) for x in rng.integers(0, 260, ns)]
    causal = bool(rng.random() < 0.6)
    window = int(rng.integers(1, 120)) if causal and rng.random() < 0.3 else 0
    extra = ["none", "bias", "alibi"][i % 3]
    w = W(name=f"fuzzb{i}", seqlens_q=tuple(sq), seqlens_kv=tuple(sk), hq=hq, hkv=hkv, d_qk=d,
          d_v=d, dtype=dtype, causal=causal, window=window, seed=12000 + i)
    return w, extra, rng


@pytest.mark.parametrize("i", range(45))
def test_fuzz_backward_against_oracle(i):
    w, extra, rng = _case(i)
    say(f"[fuzz bwd {i}] {extra} {w.dtype} d={w.d_qk} hq={w.hq} hkv={w.hkv} q={w.seqlens_q} "
        f"kv={w.seqlens_kv} causal={w.causal} window={w.window}")
    inp = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(13000 + i)
    dout = torch.randn(w.total_q, w.hq, w.d_v, generator=g).to(inp.q.dtype)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    mq, mk = max(w.max_seqlen_q, 1), max(w.max_seqlen_kv, 1)
    cols = mk
    kw = dict(scale=w.softmax_scale, causal=w.causal, window=w.window)
    ref_bias = None
    if extra == "bias":
        bias = workloads.random_bias(w.seqlens_q, [1, w.hq][rng.integers(2)], cols,
                                     seed=14000 + i, neg_inf_frac=0.2)
        kw["attn_bias"] = bias.to(dev)
        ref_bias = bias.double().numpy()
    elif extra == "alibi":
        slopes = (2.0 ** (-8.0 * (np.arange(w.hq) + 1) / w.hq)).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).to(dev)
        ref_bias = oracle.alibi_bias(slopes.astype(np.float64), inp.cu_seqlens_q.numpy(),
                                     inp.cu_seqlens_kv.numpy(), w.hq, cols)
    out, lse = fav.varlen_attention(q, k, v, cq, ck, mq, return_lse=True, **kw)
    grads = fav.varlen_attention_backward(q, k, v, out, lse, dout.to(dev), cq, ck, mq, mk,
                                          grad_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    ref = oracle.varlen_attention_backward(inp.q.double().numpy(), inp.k.double().numpy(),
                                           inp.v.double().numpy(), dout.double().numpy(),
                                           inp.cu_seqlens_q.numpy(), inp.cu_seqlens_kv.numpy(),
                                           w.softmax_scale, w.causal, w.window, ref_bias)
    for gname, gt, r in zip(("dq", "dk", "dv"), grads, ref):
        gt = gt.float().cpu().numpy().astype(np.float64)
        scale = max(float(np.abs(r).max(initial=0.0)), 1e-3)
        err = float(np.abs(gt - r).max(initial=0.0))
        say(f"  {gname}: max err {err:.3e} = {err / scale:.2e} of max|ref| {scale:.3g}")
        assert np.isfinite(gt).all(), f"{gname}: non-finite values"
        assert err <= GRAD_TOL[w.dtype] * scale, f"{gname}: {err / scale:.3e} of max|ref|"
