"""Split-KV decode (mi_attn_varlen_decode) against the fp64 oracle, through
the C ABI: one to sixteen query rows per sequence against key caches of up
to 64K keys, GQA / MQA / MHA, causal (end-aligned), full and windowed, forced
and automatic split counts."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import workloads
from gpu_helpers import check, check_sampled, run_oracle, say

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _decode(inp, num_splits=0, out_dtype=torch.float32):
    w = inp.workload
    d = "cuda"
    out, lse = fav.varlen_decode(inp.q.to(d), inp.k.to(d), inp.v.to(d), inp.cu_seqlens_q.to(d),
                                 inp.cu_seqlens_kv.to(d), w.max_seqlen_q, w.max_seqlen_kv,
                                 scale=w.softmax_scale, causal=w.causal, window=w.window,
                                 num_splits=num_splits, out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


CASES = {
    # name: (q lens, kv lens, hq, hkv, d, dtype, causal, window, splits)
    "q1_gqa_bf16": ((1, 1, 1), (5000, 17, 777), 32, 8, 128, "bf16", True, 0, 0),
    "q4_gqa_f16": ((4, 4, 2), (3000, 129, 1000), 16, 4, 64, "f16", True, 0, 0),
    "q16_gqa4_bf16": ((16, 3), (2100, 100), 8, 2, 128, "bf16", True, 0, 0),
    "q8_mha_f16_full": ((8, 1), (900, 1200), 4, 4, 128, "f16", False, 0, 0),
    "q1_mqa_bf16": ((1, 1), (4000, 1), 16, 1, 64, "bf16", True, 0, 0),
    "q4_window_bf16": ((4, 1), (3000, 700), 8, 2, 128, "bf16", True, 500, 0),
    "q2_one_split_bf16": ((2, 2), (1500, 40), 8, 4, 128, "bf16", True, 0, 1),
    "q2_many_splits_f16": ((2, 2), (1500, 40), 8, 4, 64, "f16", True, 0, 37),
    "empty_and_short": ((1, 0, 3, 1), (0, 10, 2, 64), 4, 2, 64, "bf16", True, 0, 0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_matches_oracle(name):
    lq, lk, hq, hkv, d, dt, causal, window, splits = CASES[name]
    w = W(name=name, seqlens_q=lq, seqlens_kv=lk, hq=hq, hkv=hkv, d_qk=d, d_v=d, dtype=dt,
          causal=causal, window=window, seed=100)
    say(f"[decode] {name}: q {lq} kv {lk} hq={hq} hkv={hkv} d={d} causal={causal} W={window} "
        f"splits={splits}")
    inp = workloads.make_inputs(w)
    out, lse = _decode(inp, splits)
    ref_out, ref_lse = run_oracle(inp)
    check(name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, dt)
    if splits == 0:
        out16, lse16 = _decode(inp, 0, inp.q.dtype)
        assert torch.equal(out16, out.to(inp.q.dtype)) and torch.equal(lse16, lse)


def test_decode_long_cache_64k():
    """Key caches of 64K and 40K keys, one query row each, Hq = 32, Hkv = 8."""
    w = W(name="decode_64k", seqlens_q=(1, 1), seqlens_kv=(65536, 40000), hq=32, hkv=8,
          d_qk=128, d_v=128, dtype="bf16", causal=True, seed=101)
    inp = workloads.make_inputs(w)
    say("[decode] 64K keys")
    out, lse = _decode(inp)
    check_sampled(inp, out, lse, list(range(w.hq)), rows_per_seq=1)


def test_decode_equals_forward_to_rounding():
    """The decode path and the one-pass forward compute the same function:
    both within the tolerance of the oracle, and close to each other."""
    w = W(name="dec_vs_fwd", seqlens_q=(4, 1, 16), seqlens_kv=(2000, 333, 4096), hq=8, hkv=2,
          d_qk=128, d_v=128, dtype="bf16", causal=True, seed=102)
    inp = workloads.make_inputs(w)
    out_d, lse_d = _decode(inp, 5)
    dev = "cuda"
    out_f, lse_f = fav.varlen_attention(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                                        inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev),
                                        w.max_seqlen_q, causal=True, out_dtype=torch.float32,
                                        return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(inp)
    check("decode", out_d.cpu().numpy(), lse_d.cpu().numpy(), ref_out, ref_lse, "bf16")
    check("forward", out_f.cpu().numpy(), lse_f.cpu().numpy(), ref_out, ref_lse, "bf16")
    assert float((out_d - out_f).abs().max()) <= 2e-3


def test_decode_is_deterministic():
    w = W(name="dec_det", seqlens_q=(2, 3), seqlens_kv=(3000, 1000), hq=8, hkv=2, d_qk=64,
          d_v=64, dtype="f16", causal=True, seed=103)
    inp = workloads.make_inputs(w)
    a = _decode(inp)
    b = _decode(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_full_size_workload():
    """The benchmark's decode workload (eight one-row sequences against 10K
    to 51K cached keys, Hq = 32, Hkv = 8, D = 128) in its launch (automatic
    split count): every row of every head against the oracle, and the bf16
    output equal to the RNE rounding of the fp32 one."""
    w = workloads.ALL["decode_bf16"]
    inp = workloads.make_inputs(w)
    say(f"[decode] full size {w.name}: kv {w.seqlens_kv}")
    out, lse = _decode(inp)
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)
    out16, lse16 = _decode(inp, 0, inp.q.dtype)
    assert torch.equal(out16, out.to(inp.q.dtype)) and torch.equal(lse16, lse)
