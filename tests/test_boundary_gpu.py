"""The boundary as specified: MI_ATTN_VALIDATE refusals that leave out / lse
untouched, bool-mask bias, strided (packed) views, the bias column bound,
and a seeded fuzzer over flags, dtypes, head dims and lengths, all through
the C ABI against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import OUT_TOL, LSE_TOL, check, max_abs, run_oracle, say

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _small_inputs(dtype="bf16", lens=(50, 50), hq=2, hkv=2, d=64, seed=60):
    w = W(name="boundary", seqlens_q=lens, seqlens_kv=lens, hq=hq, hkv=hkv, d_qk=d, d_v=d,
          dtype=dtype, causal=True, seed=seed)
    return w, workloads.make_inputs(w)


VALIDATE_CASES = {
    "q_not_from_zero": dict(cu_q=[2, 52, 100]),
    "q_decreasing": dict(cu_q=[0, 60, 50]),
    "q_wrong_total": dict(cu_q=[0, 50, 90]),
    "q_longer_than_max": dict(max_seqlen_q=40),
    "kv_wrong_total": dict(cu_kv=[0, 50, 120]),
    "kv_past_bias_cols": dict(bias_cols=32),
}


@pytest.mark.parametrize("case", sorted(VALIDATE_CASES))
def test_validate_refuses_and_leaves_outputs(case, monkeypatch):
    """MI_ATTN_VALIDATE=1: a cu_seqlens / size contract violation returns
    MI_ATTN_ERR_VALIDATION and launches nothing (NaN-poisoned out and lse
    stay NaN)."""
    monkeypatch.setenv("MI_ATTN_VALIDATE", "1")
    say(f"[validate] {case}")
    w, inp = _small_inputs()
    c = VALIDATE_CASES[case]
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq = torch.tensor(c.get("cu_q", [0, 50, 100]), dtype=torch.int32, device=dev)
    ck = torch.tensor(c.get("cu_kv", [0, 50, 100]), dtype=torch.int32, device=dev)
    bias = None
    if "bias_cols" in c:
        bias = torch.zeros(100, 1, c["bias_cols"], dtype=torch.float32, device=dev)
    out = torch.full((100, 2, 64), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((2, 100), float("nan"), dtype=torch.float32, device=dev)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.varlen_attention(q, k, v, cq, ck, c.get("max_seqlen_q", 50), causal=True,
                             attn_bias=bias, out=out, lse=lse, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert ei.value.code == fav.ERR_VALIDATION, str(ei.value)
    say(f"  refused: {ei.value}")
    assert torch.isnan(out).all() and torch.isnan(lse).all()


def test_validate_accepts_a_valid_call(monkeypatch):
    monkeypatch.setenv("MI_ATTN_VALIDATE", "1")
    w, inp = _small_inputs(lens=(50, 1, 77))
    dev = "cuda"
    out, lse = fav.varlen_attention(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                                    inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev),
                                    w.max_seqlen_q, causal=True, out_dtype=torch.float32,
                                    return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(inp)
    check("validate_ok", out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("heads", [1, "hq"])
def test_bool_mask_bias(heads):
    """A bool attn_bias (True = visible) with an odd number of columns; some
    rows see nothing (out 0, lse -inf)."""
    w, inp = _small_inputs(lens=(130, 77), hq=4, hkv=2, d=128, seed=61)
    w = w.with_(causal=False)
    inp.workload = w
    g = torch.Generator().manual_seed(62)
    nb = w.hq if heads == "hq" else 1
    mask = torch.rand(w.total_q, nb, 131, generator=g) > 0.3
    mask[5] = False  # a row with no visible key
    say(f"[bool mask] heads={nb}")
    dev = "cuda"
    out, lse = fav.varlen_attention(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                                    inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev),
                                    w.max_seqlen_q, causal=False, attn_bias=mask.to(dev),
                                    out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    inp.bias = torch.zeros(mask.shape).masked_fill_(~mask, float("-inf"))
    ref_out, ref_lse = run_oracle(inp)
    check("bool_mask", out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)
    assert bool((out[5] == 0).all()) and bool(torch.isneginf(lse[:, 5]).all())


def test_requires_grad_is_refused_by_the_forward_call():
    w, inp = _small_inputs()
    q = inp.q.to("cuda").float().requires_grad_()
    with pytest.raises(fav.MiAttnError):
        fav.varlen_attention(q, inp.k.to("cuda").float(), inp.v.to("cuda").float(),
                             inp.cu_seqlens_q.to("cuda"), inp.cu_seqlens_kv.to("cuda"), 50)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_packed_qkv_views_and_padded_out(dtype):
    """q, k, v sliced from one packed [T, 3, H, D] tensor (token stride 3*H*D),
    and an output with a padded token / head stride."""
    lens = (200, 1, 129)
    w = W(name="packed", seqlens_q=lens, seqlens_kv=lens, hq=4, hkv=4, d_qk=64, d_v=64,
          dtype=dtype, causal=True, seed=63)
    inp = workloads.make_inputs(w)
    dev = "cuda"
    qkv = torch.stack([inp.q, inp.k, inp.v], dim=1).to(dev)  # [T, 3, H, D]
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    assert q.stride(0) == 3 * 4 * 64 and not q.is_contiguous()
    out_buf = torch.full((w.total_q, 4, 64 + 16), float("nan"), dtype=torch.float32, device=dev)
    out = out_buf[:, :, :64]
    say(f"[strided] {dtype}: q stride {q.stride()}, out stride {out.stride()}")
    _, lse = fav.varlen_attention(q, k, v, inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev),
                                  w.max_seqlen_q, causal=True, out=out, out_dtype=torch.float32,
                                  return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(inp)
    check(f"packed_{dtype}", out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)
    assert torch.isnan(out_buf[:, :, 64:]).all(), "padding of the output rows was written"


def test_bias_narrower_than_keys_reads_zero():
    """bias_cols below a sequence's key length breaks the caller contract;
    the kernels still never read past bias_cols (those keys get a bias of 0),
    so nothing faults and the result equals a zero-extended bias."""
    w, inp = _small_inputs(lens=(100, 40), hq=2, hkv=2, d=128, seed=64)
    g = torch.Generator().manual_seed(65)
    narrow = torch.randn(w.total_q, 1, 64, generator=g)
    dev = "cuda"
    out, lse = fav.varlen_attention(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                                    inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev),
                                    w.max_seqlen_q, causal=True, attn_bias=narrow.to(dev),
                                    out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    inp.bias = torch.cat([narrow, torch.zeros(w.total_q, 1, 36)], dim=2)
    ref_out, ref_lse = run_oracle(inp)
    check("narrow_bias", out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


def _fuzz_case(i):
    rng = np.random.default_rng(1000 + i)
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    dims = [(64, 64), (128, 128), (192, 128)]
    if dtype == "f32":
        dims = dims[:2]
    dqk, dv = dims[rng.integers(len(dims))]
    hkv = int(rng.choice([1, 2, 3]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    ns = int(rng.integers(1, 5))
    lq = [int(x) for x in rng.integers(0, 300, ns)]
    self_attn = rng.random() < 0.6
    lk = lq if self_attn else [int(x) for x in rng.integers(0, 400, ns)]
    causal = bool(rng.random() < 0.6)
    window = int(rng.integers(1, 200)) if causal and rng.random() < 0.4 else 0
    bias = [None, 1, hq][rng.integers(3)]
    return W(name=f"fuzz{i}", seqlens_q=tuple(lq), seqlens_kv=tuple(lk), hq=hq, hkv=hkv,
             d_qk=dqk, d_v=dv, dtype=dtype, causal=causal, window=window, seed=2000 + i), bias


@pytest.mark.parametrize("i", range(40))
def test_fuzz_against_oracle(i):
    w, bias_heads = _fuzz_case(i)
    say(f"[fuzz {i}] {w.dtype} d=({w.d_qk},{w.d_v}) hq={w.hq} hkv={w.hkv} q={w.seqlens_q} "
        f"kv={w.seqlens_kv} causal={w.causal} window={w.window} bias={bias_heads}")
    inp = workloads.make_inputs(w)
    if bias_heads is not None:
        cols = max(max(w.seqlens_kv), 1)
        inp.bias = workloads.random_bias(w.seqlens_q, bias_heads, cols, seed=3000 + i,
                                         neg_inf_frac=0.15)
    dev = "cuda"
    out, lse = fav.varlen_attention(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                                    inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev),
                                    max(w.max_seqlen_q, 1), scale=w.softmax_scale,
                                    causal=w.causal, window=w.window,
                                    attn_bias=inp.bias.to(dev) if inp.bias is not None else None,
                                    out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)
