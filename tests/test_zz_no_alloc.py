"""The non-allocating decode entry point (mi_attn_varlen_decode_noalloc),
called through the C ABI: two calls in a row, the second with a smaller
input, each checked against the workspace entry point (mi_attn_varlen_decode)
and the fp64 oracle."""
import pytest
import torch

import flash_attention_varlen_amd as fav
import workloads
from gpu_helpers import check, run_oracle, say

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _inputs(lq, lk, seed):
    w = W(name="noalloc", seqlens_q=lq, seqlens_kv=lk, hq=16, hkv=4, d_qk=128, d_v=128,
          dtype="bf16", causal=True, seed=seed)
    return w, workloads.make_inputs(w)


def _both(w, inp, splits):
    d = "cuda"
    q, k, v = inp.q.to(d), inp.k.to(d), inp.v.to(d)
    cq, ck = inp.cu_seqlens_q.to(d), inp.cu_seqlens_kv.to(d)
    out_n = torch.full((w.total_q, w.hq, w.d_v), float("nan"), dtype=torch.float32, device=d)
    lse_n = torch.full((w.hq, w.total_q), float("nan"), dtype=torch.float32, device=d)
    fav.varlen_decode_noalloc(q, k, v, cq, ck, w.max_seqlen_q, w.max_seqlen_kv, out_n, lse_n,
                              causal=True, num_splits=splits)
    out_w, lse_w = fav.varlen_decode(q, k, v, cq, ck, w.max_seqlen_q, w.max_seqlen_kv,
                                     causal=True, num_splits=splits, out_dtype=torch.float32,
                                     return_lse=True)
    torch.cuda.synchronize()
    return out_n, lse_n, out_w, lse_w


@pytest.mark.parametrize("splits", [6, 0])
def test_noalloc_decode_two_calls(splits):
    """First a larger call, then a smaller one (the scratch keeps the first
    call's contents).  With an explicit split count both entry points run the
    same chunks: bitwise equal; with the automatic count both match the
    oracle."""
    for lq, lk, seed in (((4, 1, 2), (9000, 300, 4000), 110), ((1, 2), (500, 70), 111)):
        w, inp = _inputs(lq, lk, seed)
        say(f"[noalloc] splits={splits} q {lq} kv {lk}")
        out_n, lse_n, out_w, lse_w = _both(w, inp, splits)
        ref_out, ref_lse = run_oracle(inp)
        check("noalloc", out_n.cpu().numpy(), lse_n.cpu().numpy(), ref_out, ref_lse, "bf16")
        if splits:
            assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)
        else:
            assert float((out_n - out_w).abs().max()) <= 2e-3


def test_noalloc_refuses_what_does_not_fit():
    """Rows x heads x (d_v + 2) floats of one chunk above the 16 MiB scratch:
    refused with a clear error, nothing launched."""
    tq, hq = 8200, 4  # 8200 * 4 * 130 * 4 bytes > 16 MiB even with one chunk
    d = "cuda"
    q = torch.zeros(tq, hq, 128, dtype=torch.bfloat16, device=d)
    k = torch.zeros(64, 1, 128, dtype=torch.bfloat16, device=d)
    cq = torch.tensor([0, tq // 2, tq], dtype=torch.int32, device=d)
    ck = torch.tensor([0, 32, 64], dtype=torch.int32, device=d)
    out = torch.full((tq, hq, 128), float("nan"), dtype=torch.float32, device=d)
    with pytest.raises(fav.MiAttnError) as ei:
        fav.varlen_decode_noalloc(q, k, k, cq, ck, 16, 32, out, num_splits=0)
    torch.cuda.synchronize()
    assert ei.value.code == fav.ERR_UNSUPPORTED and "workspace" in str(ei.value)
    assert torch.isnan(out).all()
