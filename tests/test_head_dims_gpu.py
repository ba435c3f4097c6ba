"""The 96- and 256-wide heads (bf16 / fp16; the mtlattn 0.3.0 page, section
"Drop-in for scaled_dot_product_attention", lists head dims 64, 96, 128 and
256) against the fp64 oracle through the C ABI: causal, full, sliding
window and cross lengths, GQA, a bias and ALiBi, ragged lengths that span
several tiles, and the 16-bit output as the RNE rounding of the fp32 one."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import check, run_gpu, run_oracle, say, to_device

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _cases():
    c = {}
    for d in (96, 256):
        c[f"bf16_d{d}_causal_gqa"] = W(name=f"hd_bf16_d{d}_causal_gqa", seqlens_q=(300, 129, 1),
                                      seqlens_kv=(300, 129, 1), hq=4, hkv=2, d_qk=d, d_v=d,
                                      dtype="bf16", causal=True, seed=100 + d)
        c[f"f16_d{d}_full"] = W(name=f"hd_f16_d{d}_full", seqlens_q=(200, 65), seqlens_kv=(200, 65),
                               hq=2, hkv=1, d_qk=d, d_v=d, dtype="f16", causal=False, seed=101 + d)
        c[f"bf16_d{d}_window_cross"] = W(name=f"hd_bf16_d{d}_window_cross", seqlens_q=(90, 40),
                                        seqlens_kv=(260, 41), hq=2, hkv=2, d_qk=d, d_v=d,
                                        dtype="bf16", causal=True, window=70, seed=102 + d)
        c[f"f16_d{d}_prefix_bias"] = W(name=f"hd_f16_d{d}_prefix_bias", seqlens_q=(180, 70),
                                      seqlens_kv=(180, 70), hq=2, hkv=2, d_qk=d, d_v=d,
                                      dtype="f16", causal=False, bias="prefix_lm", prefix=60,
                                      seed=103 + d)
    return c


CASES = _cases()


@pytest.mark.parametrize("name", sorted(CASES))
def test_head_dim_against_oracle(name):
    w = CASES[name]
    say(f"[head dims] {name}")
    inp = workloads.make_inputs(w)
    dev = to_device(inp)
    out, lse = run_gpu(inp, dev=dev)
    ref_out, ref_lse = run_oracle(inp)
    check(name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)
    out16, lse16 = run_gpu(inp, out_dtype=inp.q.dtype, dev=dev)
    assert torch.equal(out16, out.to(inp.q.dtype)) and torch.equal(lse16, lse)


@pytest.mark.parametrize("d", [96, 256])
def test_head_dim_alibi(d):
    w = W(name=f"hd_alibi_d{d}", seqlens_q=(150, 33), seqlens_kv=(150, 33), hq=4, hkv=2, d_qk=d,
          d_v=d, dtype="bf16", causal=True, seed=110 + d)
    inp = workloads.make_inputs(w)
    q, k, v, cq, ck, _ = to_device(inp)
    sl = np.array([2.0 ** (-(h + 1)) for h in range(w.hq)], dtype=np.float32)
    out, lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale,
                                    causal=True, alibi_slopes=torch.from_numpy(sl).cuda(),
                                    out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    dense = oracle.alibi_bias(sl.astype(np.float64), inp.cu_seqlens_q.numpy(),
                              inp.cu_seqlens_kv.numpy(), w.hq, w.max_seqlen_kv)
    ref_out, ref_lse = oracle.varlen_attention(
        inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy(),
        inp.cu_seqlens_q.numpy(), inp.cu_seqlens_kv.numpy(), w.softmax_scale, True, 0, dense)
    check(f"alibi_d{d}", out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("d", [96, 256])
def test_head_dim_strided_views(d):
    """q, k, v sliced out of one packed [T, 3, H, d] tensor, out with a padded
    token stride: the kernels read and write through the strides."""
    w = W(name=f"hd_views_d{d}", seqlens_q=(200, 77), seqlens_kv=(200, 77), hq=2, hkv=2, d_qk=d,
          d_v=d, dtype="bf16", causal=True, seed=120 + d)
    inp = workloads.make_inputs(w)
    qkv = torch.stack([inp.q, inp.k, inp.v], dim=1).cuda()
    cu = inp.cu_seqlens_q.cuda()
    out_buf = torch.full((w.total_q, w.hq, d + 32), float("nan"), dtype=torch.float32, device="cuda")
    out = out_buf[:, :, :d]
    fav.varlen_attention(qkv[:, 0], qkv[:, 1], qkv[:, 2], cu, cu, w.max_seqlen_q, causal=True,
                         out=out, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_out, _ = run_oracle(inp)
    err = float(np.abs(out.cpu().numpy() - ref_out).max())
    say(f"  views d{d}: max|out-ref|={err:.3e}")
    assert err <= 2e-3
    assert torch.isnan(out_buf[:, :, d:]).all()
