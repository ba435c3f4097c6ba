"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the fp64 oracle on the same seeded inputs, compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads

# Max-abs tolerances on the fp32 output, by input dtype, and on the LSE.
OUT_TOL = {"bf16": 2e-3, "f16": 1e-3, "f32": 1e-5}
LSE_TOL = 1e-4


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: workloads.Inputs, device="cuda"):
    q = inp.q.to(device)
    k = inp.k.to(device)
    v = inp.v.to(device)
    cq = inp.cu_seqlens_q.to(device)
    ck = inp.cu_seqlens_kv.to(device)
    b = inp.bias.to(device) if inp.bias is not None else None
    return q, k, v, cq, ck, b


def run_gpu(inp: workloads.Inputs, out_dtype=torch.float32, dev=None, tile_counts=None, **kw):
    w = inp.workload
    q, k, v, cq, ck, b = dev if dev is not None else to_device(inp)
    say(f"  gpu launch: {w.name} dtype={w.dtype} out={out_dtype} T={w.total_q} hq={w.hq} "
        f"hkv={w.hkv} d=({w.d_qk},{w.d_v}) causal={w.causal} window={w.window} "
        f"bias={b is not None}")
    out, lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale,
                                    causal=w.causal, window=w.window, attn_bias=b,
                                    out_dtype=out_dtype, return_lse=True,
                                    tile_counts=tile_counts, **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_inputs(inp: workloads.Inputs):
    q = inp.q.double().numpy()
    k = inp.k.double().numpy()
    v = inp.v.double().numpy()
    b = inp.bias.double().numpy() if inp.bias is not None else None
    return q, k, v, inp.cu_seqlens_q.numpy().astype(np.int64), inp.cu_seqlens_kv.numpy().astype(
        np.int64), b


def run_oracle(inp: workloads.Inputs):
    w = inp.workload
    q, k, v, cq, ck, b = oracle_inputs(inp)
    return oracle.varlen_attention(q, k, v, cq, ck, w.softmax_scale, w.causal, w.window, b)


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_neg_inf = (a == -np.inf) & (b == -np.inf)
    fin = np.isfinite(a) & np.isfinite(b)
    bad = ~(fin | both_neg_inf)
    if bad.any():
        return math.inf
    d = np.abs(np.subtract(a, b, out=np.zeros_like(a), where=fin))
    return float(d.max(initial=0.0))


def check(name, out_gpu, lse_gpu, out_ref, lse_ref, dtype: str):
    eo = max_abs(out_gpu, out_ref)
    el = max_abs(lse_gpu, lse_ref)
    say(f"  {name}: max|out-ref|={eo:.3e} (tol {OUT_TOL[dtype]:.0e})  max|lse-ref|={el:.3e} "
        f"(tol {LSE_TOL:.0e})")
    assert eo <= OUT_TOL[dtype], f"{name}: out error {eo} > {OUT_TOL[dtype]}"
    assert el <= LSE_TOL, f"{name}: lse error {el} > {LSE_TOL}"


def sample_rows(inp: workloads.Inputs, heads, rows_per_seq: int, seed: int):
    """(seq, head, local rows) samples: tile edges, both ends and random rows."""
    rng = np.random.default_rng(seed)
    out = []
    for s, lq in enumerate(inp.workload.seqlens_q):
        if lq == 0:
            continue
        fixed = {0, 1, 31, 32, 63, 64, 127, 128, lq // 2, lq - 2, lq - 1}
        rnd = set(rng.choice(lq, size=min(lq, rows_per_seq), replace=False).tolist())
        rows = sorted(r for r in fixed | rnd if 0 <= r < lq)
        for h in heads:
            out.append((s, h, np.array(rows, dtype=np.int64)))
    return out


def check_sampled(inp: workloads.Inputs, out_gpu, lse_gpu, heads, rows_per_seq=24, seed=0):
    """Oracle rows computed one (sequence, head) at a time vs the GPU output."""
    w = inp.workload
    q, k, v, cq, ck, b = oracle_inputs(inp)
    og = out_gpu.float().cpu().numpy()
    lg = lse_gpu.cpu().numpy()
    worst_o = worst_l = 0.0
    for s, h, rows in sample_rows(inp, heads, rows_per_seq, seed):
        o, l = oracle.attention_rows(q, k, v, cq, ck, s, h, rows, w.softmax_scale, w.causal,
                                     w.window, b)
        worst_o = max(worst_o, max_abs(og[cq[s] + rows, h], o))
        worst_l = max(worst_l, max_abs(lg[h, cq[s] + rows], l))
    say(f"  {w.name} sampled: max|out-ref|={worst_o:.3e} max|lse-ref|={worst_l:.3e}")
    assert worst_o <= OUT_TOL[w.dtype], worst_o
    assert worst_l <= LSE_TOL, worst_l


def rne_to(x: torch.Tensor, dtype) -> torch.Tensor:
    """fp32 -> bf16/fp16 with round-to-nearest-even (torch's cast)."""
    return x.to(dtype)
