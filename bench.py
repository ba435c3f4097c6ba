#!/usr/bin/env python3
"""Benchmark of the fused varlen attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 15] [--workload gqa_causal_bf16]

One step is one call of the whole hot path (one kernel launch computing
out and lse) over the workload's packed batch, with q/k/v/cu_seqlens
already resident in HBM.  The default workload is the bf16 causal GQA
varlen prefill: 8 sequences (lengths 1677, 2626, 1676, 2065, 630, 4080,
4078, 3373 drawn from seed 1), Hq=32, Hkv=8, D=128, scale 1/sqrt(128).

Reported value: useful TFLOP/s, i.e. (2*Dqk + 2*Dv) FLOPs per unmasked
(query, key, head) triple divided by the time of one launch.  The JSON line
also carries the MFMA roofline of the kernel and the fp64 CPU oracle timed
on a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "attn fwd useful TFLOP/s + % of MI355X bf16 MFMA peak (causal GQA D=128)"
# MI355X dense MFMA peaks (TFLOP/s): 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU for
# bf16/fp16; fp32 matrix 157.3.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_GBPS = 8000.0
CPU_SHARE = 16  # host cores a one-GPU machine is given
CSRC = os.path.join(ROOT, "flash_attention_varlen_amd", "csrc")
# the sources of each pass's kernels (a stored counter reading is valid while they are unchanged)
KERNEL_SOURCES = {"fwd": ("attn_fwd_kernels.h", "attn_fwd.h"), "bwd": ("attn_bwd_kernels.h", "attn_bwd.h"),
                  "decode": ("attn_decode.hip", "attn_decode.h")}
PROFILES = os.path.join(ROOT, "profiles")


# ----------------------------------------------------------------- accounting
def visible_pairs_per_row(lq: int, lk: int, causal: bool, window: int) -> np.ndarray:
    """Closed-form number of visible keys of each query row (end-aligned)."""
    i = np.arange(lq, dtype=np.int64)
    off = lk - lq
    hi = np.clip(i + off + 1, 0, lk) if causal else np.full(lq, lk, dtype=np.int64)
    lo = np.clip(i + off - window + 1, 0, lk) if window else np.zeros(lq, dtype=np.int64)
    return np.maximum(hi - lo, 0)


def useful_pairs(w: workloads.Workload, bias=None) -> int:
    """Unmasked (query, key) pairs summed over sequences and query heads.

    With a bias, keys whose bias is -inf are masked too; the count then
    comes from the bias tensor itself (per head if it has one per head).
    """
    total = 0
    q0 = 0
    for lq, lk in zip(w.seqlens_q, w.seqlens_kv):
        if bias is None:
            total += int(visible_pairs_per_row(lq, lk, w.causal, w.window).sum()) * w.hq
        else:
            import torch
            b = bias[q0:q0 + lq, :, :lk]
            finite = torch.isfinite(b)
            i = torch.arange(lq).view(lq, 1, 1)
            j = torch.arange(lk).view(1, 1, lk)
            off = lk - lq
            vis = torch.ones(lq, 1, lk, dtype=torch.bool)
            if w.causal:
                vis &= j <= i + off
            if w.window:
                vis &= j > i + off - w.window
            per_head = (finite & vis).sum(dim=(0, 2))
            total += int(per_head.sum()) * (w.hq if b.shape[1] == 1 else 1)
        q0 += lq
    return total


def useful_flops(w: workloads.Workload, bias=None) -> float:
    return float(useful_pairs(w, bias)) * (2 * w.d_qk + 2 * w.d_v)


def algorithmic_bytes(w: workloads.Workload, out_bytes: int) -> float:
    """q, k, v, out and lse each moved once (the bias once if present)."""
    e = 4 if w.dtype == "f32" else 2
    b = w.total_q * w.hq * w.d_qk * e + w.total_kv * w.hkv * (w.d_qk + w.d_v) * e
    b += w.total_q * w.hq * w.d_v * out_bytes + w.total_q * w.hq * 4
    if w.bias is not None:
        b += w.total_q * w.max_seqlen_kv * 4
    return float(b)


def kernel_source_hash(mode: str = "fwd") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[mode]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_key: str, launches: int = 1, mode: str = "fwd"):
    """HBM bytes per step from the committed PMC summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_attn_{mode}_{workload_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash(mode):
        return None
    return float(t["hbm_bytes_per_launch"]) * launches


# ----------------------------------------------------------------- CPU oracle baseline
def _oracle_unit(args):
    """One (sequence, head) of the oracle, single-threaded BLAS."""
    s, h, scale, causal, window = args
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(1):
        lq = int(_G["cq"][s + 1] - _G["cq"][s])
        for r0 in range(0, lq, 256):
            rows = np.arange(r0, min(lq, r0 + 256))
            oracle.attention_rows(_G["q"], _G["k"], _G["v"], _G["cq"], _G["ck"], s, h, rows,
                                  scale, causal, window, _G["b"])
    return s, h


_G = {}


def _pool_init(q, k, v, cq, ck, b):
    _G.update(q=q, k=k, v=v, cq=cq, ck=ck, b=b)


def cpu_baseline(inp: workloads.Inputs, heads, cores: int):
    """Time the fp64 oracle (as it is) over the sampled heads of every
    sequence on `cores` worker processes; returns the baseline object."""
    import multiprocessing as mp
    w = inp.workload
    q = inp.q.double().numpy()
    k = inp.k.double().numpy()
    v = inp.v.double().numpy()
    b = inp.bias.double().numpy() if inp.bias is not None else None
    cq = inp.cu_seqlens_q.numpy().astype(np.int64)
    ck = inp.cu_seqlens_kv.numpy().astype(np.int64)
    units = [(s, h, w.softmax_scale, w.causal, w.window) for s in range(w.num_seqs)
             for h in heads]
    # biggest units first so the pool drains evenly
    units.sort(key=lambda u: -(w.seqlens_q[u[0]] * w.seqlens_kv[u[0]]))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores, initializer=_pool_init, initargs=(q, k, v, cq, ck, b)) as pool:
        for _ in pool.imap_unordered(_oracle_unit, units):
            pass
    dt = time.perf_counter() - t0
    pairs_per_head = useful_pairs(w.with_(hq=1, hkv=1), None) if b is None else None
    if pairs_per_head is None:
        pairs = useful_pairs(w, inp.bias) * len(heads) / w.hq
    else:
        pairs = pairs_per_head * len(heads)
    flops = pairs * (2 * w.d_qk + 2 * w.d_v)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 NumPy oracle on query heads {list(heads)} of all {w.num_seqs} "
                      f"sequences ({len(units)} (sequence, head) units, "
                      f"{pairs:.3e} useful pairs), {dt:.1f} s wall on {cores} processes with "
                      f"1 BLAS thread each",
            "seconds": round(dt, 2), "seconds_exact": dt}


# ----------------------------------------------------------------- GPU timing
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--prewarm-ms", type=float, default=1000.0,
                    help="before the warmup steps, run the step back to back for this long so the "
                         "GPU reaches its steady clock (0 = off)")
    ap.add_argument("--workload", default="gqa_causal_bf16", choices=sorted(workloads.ALL))
    ap.add_argument("--out-dtype", default="input", choices=["input", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="query heads per sequence the CPU oracle baseline covers")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC calibration)")
    ap.add_argument("--cold-steps", type=int, default=0,
                    help="after the timed region, time this many launches each preceded by a "
                         "write of --flush-mib MiB (evicts L2 and the MALL); reported under 'cold'")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (delta, dk/dv, dq kernels) instead of the forward; "
                         "useful FLOPs are 2.5x the forward's (five products of the same size)")
    ap.add_argument("--no-bias-ranges", action="store_true",
                    help="with a bias, do not compute the bias key ranges (visit every tile)")
    ap.add_argument("--window", type=int, default=None,
                    help="override the window width of a sliding-window workload (cost vs W)")
    ap.add_argument("--sdpa-keypad", action="store_true",
                    help="time the key-padding front end: the workload's sequences as a padded "
                         "[B, H, N, D] batch with a bool key-padding mask through sdpa() (the "
                         "right-padding check, then the forward in place on the padded "
                         "storage), self-attention without a bias")
    ap.add_argument("--no-interval-rows", action="store_true",
                    help="with a bias: compute its key ranges only, so that the forward reads "
                         "the bias of every row (no interval flags)")
    ap.add_argument("--split-rope", action="store_true",
                    help="latent workload: pass q, k as 128-wide nope tensors plus 64-wide "
                         "q_rope / k_rope tensors instead of the concatenation")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build runs the forward on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); multi-GPU runs are not "
              f"part of it.", file=sys.stderr)
        sys.exit(2)

    w = workloads.ALL[args.workload]
    if args.window is not None:
        if not w.window or args.window < 1:
            print("--window applies to a sliding-window workload, with W >= 1", file=sys.stderr)
            sys.exit(2)
        base = w.name[:w.name.rfind("_w")] if "_w" in w.name else w.name
        w = w.with_(name=f"{base}_w{args.window}", window=args.window,
                    description=f"{w.description}, window overridden to {args.window}")
    print(f"# workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w)

    # The CPU oracle runs first, in forked worker processes, before anything
    # in this process touches the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        # One process per host core this process may use, at most 16: a
        # one-GPU machine is given a 16-core share of its host, whatever the
        # affinity mask shows.
        visible = len(os.sched_getaffinity(0))
        cores = min(visible, CPU_SHARE)
        heads = list(range(0, w.hq, max(1, w.hq // args.cpu_heads)))[:args.cpu_heads]
        print(f"# CPU oracle baseline on {cores} processes, heads {heads} ...", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(inp, heads, cores)
        if w.name.startswith("decode"):
            frac = len(heads) / w.hq
            cpu["value"] = algorithmic_bytes(w, 2) * frac / cpu["seconds_exact"] / 1e9
            cpu["unit"] = "GB/s"
        cpu["host_cores_visible"] = visible
        cpu["cores_note"] = (f"{cores} worker processes: all {visible} cores this process may use"
                             if cores == visible else
                             f"{cores} worker processes: the {CPU_SHARE}-core share of the host a "
                             f"one-GPU box is given ({visible} cores visible)")
        print(f"# CPU oracle: {cpu['value']:.4g} TFLOP/s in {cpu['seconds']} s", file=sys.stderr,
              flush=True)

    import torch
    import flash_attention_varlen_amd as fav

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fav.load_library()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    bias = inp.bias.to(dev) if inp.bias is not None else None
    rope_kw = {}
    if args.split_rope:
        if w.nope_rope is None:
            print("--split-rope applies to the latent-attention workload", file=sys.stderr)
            sys.exit(2)
        dn = w.nope_rope[0]
        rope_kw = dict(q_rope=q[..., dn:].contiguous(), k_rope=k[..., dn:].contiguous())
        q, k = q[..., :dn].contiguous(), k[..., :dn].contiguous()
    out_dtype = q.dtype if args.out_dtype == "input" else torch.float32
    out = torch.empty(w.total_q, w.hq, w.d_v, dtype=out_dtype, device=dev)
    lse = torch.empty(w.hq, w.total_q, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # With a bias, each step first computes the bias rows' key ranges and
    # interval flags (one read of the bias), then the forward skips the -inf
    # tiles outside the ranges and masks interval rows without reading their
    # bias.
    use_ranges = bias is not None and not args.no_bias_ranges
    use_pure = use_ranges and not args.no_interval_rows

    is_decode = w.name.startswith("decode")
    if is_decode:
        ws = torch.empty(16 << 20, dtype=torch.uint8, device=dev)  # grown below if too small
        p_probe = fav._fwd_params(q, k, v, cq, ck, w.max_seqlen_q, w.softmax_scale, w.causal,
                                  w.window, out, lse, out_dtype)
        need = fav.mi_attn_decode_workspace_size(p_probe, w.max_seqlen_kv, 0)
        if need > ws.numel():
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if args.backward:
        if bias is not None or w.dtype == "f32" or w.d_qk != w.d_v or w.d_qk not in (64, 96, 128):
            print("the backward takes bf16/fp16, head dims 64, 96 or 128, no bias", file=sys.stderr)
            sys.exit(2)
        out_f, lse_f = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale,
                                            causal=w.causal, window=w.window, return_lse=True)
        g_do = torch.Generator().manual_seed(w.seed + 1000)
        dout = torch.randn(w.total_q, w.hq, w.d_v, generator=g_do).to(q.dtype).to(dev)
        dq_b, dk_b, dv_b = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        torch.cuda.synchronize()

    if args.sdpa_keypad:
        if (bias is not None or w.window or list(w.seqlens_q) != list(w.seqlens_kv)
                or is_decode or args.backward or rope_kw):
            print("--sdpa-keypad takes a self-attention forward workload without a bias or window",
                  file=sys.stderr)
            sys.exit(2)
        # the sequences right-padded into [B, N, H, D] buffers, seen as SDPA's [B, H, N, D]
        nmax = max(w.seqlens_q)
        pads = []
        for t in (q, k, v):
            buf = torch.zeros(w.num_seqs, nmax, t.shape[1], t.shape[2], dtype=t.dtype, device=dev)
            for i, n in enumerate(w.seqlens_q):
                c0 = int(inp.cu_seqlens_q[i])
                buf[i, :n] = t[c0:c0 + n]
            pads.append(buf.transpose(1, 2))
        keymask = torch.zeros(w.num_seqs, nmax, dtype=torch.bool, device=dev)
        for i, n in enumerate(w.seqlens_q):
            keymask[i, :n] = True
        keymask4 = keymask[:, None, None, :]

    def step(mid_event=None):
        if args.sdpa_keypad:
            if mid_event is not None:
                mid_event.record(stream)
            fav.sdpa(pads[0], pads[1], pads[2], attn_mask=keymask4, is_causal=w.causal,
                     scale=w.softmax_scale, enable_gqa=True, stream=stream)
            return
        if is_decode:
            if mid_event is not None:
                mid_event.record(stream)
            fav.varlen_decode(q, k, v, cq, ck, w.max_seqlen_q, w.max_seqlen_kv,
                              scale=w.softmax_scale, causal=w.causal, window=w.window, out=out,
                              lse=lse, out_dtype=out_dtype, workspace=ws, stream=stream)
            return
        if args.backward:
            if mid_event is not None:
                mid_event.record(stream)
            fav.varlen_attention_backward(q, k, v, out_f, lse_f, dout, cq, ck, w.max_seqlen_q,
                                          w.max_seqlen_kv, scale=w.softmax_scale, causal=w.causal,
                                          window=w.window, dq=dq_b, dk=dk_b, dv=dv_b, stream=stream)
            return
        rg = pure = None
        if use_pure:
            rg, pure = fav.bias_key_ranges(bias, cq, ck, w.max_seqlen_q, stream=stream,
                                           return_pure=True)
        elif use_ranges:
            rg = fav.bias_key_ranges(bias, cq, ck, w.max_seqlen_q, stream=stream)
        if mid_event is not None:
            mid_event.record(stream)
        fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale,
                             causal=w.causal, window=w.window, attn_bias=bias, out=out, lse=lse,
                             out_dtype=out_dtype, stream=stream, bias_ranges=rg, bias_pure=pure,
                             **rope_kw)

    # GPU clocks depend on the load state: a cold GPU reads well below its
    # warmed rate (the mtlattn 0.3.0 page, section "Performance", gives the
    # same caveat for Apple GPUs).  Run the step back to back until the clock
    # settles, then the W warmup steps, then exactly K timed steps.
    prewarm_launches = 0
    if args.prewarm_ms > 0:
        t_pw = time.perf_counter()
        while (time.perf_counter() - t_pw) * 1e3 < args.prewarm_ms:
            for _ in range(20):
                step()
            prewarm_launches += 20
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-launch events on the launch stream (for the median) and one pair
    # around the whole timed region
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    start_all = torch.cuda.Event(enable_timing=True)
    end_all = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start_all.record(stream)
    for (s, e), m in zip(evs, mids):
        s.record(stream)
        step(m)
        e.record(stream)
    end_all.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start_all.elapsed_time(end_all)
    # the attention kernel alone: from the event after the range pass (if
    # any) to the end of the step
    per = sorted(m.elapsed_time(e) for (s, e), m in zip(evs, mids))
    pre_ms = [s.elapsed_time(m) for (s, e), m in zip(evs, mids)]
    ms_per_step = total_ms / args.steps
    kernel_ms = sum(per) / len(per)

    flops = useful_flops(w, inp.bias) * (2.5 if args.backward else 1.0)
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    if is_decode:
        # decode is bound by HBM: every K/V byte of the visible ranges read once
        alg_bytes = algorithmic_bytes(w, out.element_size())
        value = alg_bytes / (ms_per_step * 1e-3) / 1e9
        peak = HBM_GBPS
        achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    out_bytes = out.element_size()
    # stored counter readings belong to the workload as defined (not to an overridden window)
    mode = "decode" if is_decode else "bwd" if args.backward else "fwd"
    traffic = stored_traffic(args.workload, mode=mode) if args.window is None else None

    cold = None
    if args.cold_steps > 0:
        # Cold-cache launches: a large write between launches evicts L2 and the
        # MALL (256 MB), so inputs come from HBM again.  Each launch is timed
        # on its own; the flush is outside its events.
        flush = torch.empty(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_steps)]
        for s_, e_ in cev:
            flush.fill_(1.0)
            s_.record(stream)
            step()
            e_.record(stream)
        torch.cuda.synchronize()
        cms = sorted(s_.elapsed_time(e_) for s_, e_ in cev)
        cmean = sum(cms) / len(cms)
        cold = {"launches": args.cold_steps, "flush_mib": args.flush_mib,
                "kernel_ms": round(cmean, 4), "median_ms": round(cms[len(cms) // 2], 4),
                "tflops": round(flops / (cmean * 1e-3) / 1e12, 2),
                "algorithmic_gbps": round(algorithmic_bytes(w, out.element_size()) / (cmean * 1e-3) / 1e9, 1)}
        del flush

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy calibration: {n * 4} bytes read, {n * 4} bytes written per copy, 3 copies",
              file=sys.stderr, flush=True)

    result = {
        "metric": ("attn split-KV decode GB/s (q, k, v, out, lse moved once) + % of MI355X HBM peak"
                   if is_decode else METRIC if not args.backward else
                   "attn bwd useful TFLOP/s (2.5x the forward's useful FLOPs) + % of MI355X bf16 "
                   "MFMA peak"),
        "value": round(value, 2),
        "unit": "GB/s" if is_decode else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, RNE cast; no dataset or weights)",
        "config": {
            "workload": w.name,
            "seqlens_q": list(w.seqlens_q),
            "total_tokens": w.total_q,
            "hq": w.hq, "hkv": w.hkv, "d_qk": w.d_qk, "d_v": w.d_v,
            "causal": w.causal, "window": w.window,
            "bias": w.bias, "out_dtype": str(out_dtype).replace("torch.", ""),
            "operands": "split nope / rope" if args.split_rope else "concatenated",
            "useful_flops_per_step": flops,
            "pct_of_peak": round(100.0 * value / peak, 2),
            "median_launch_ms": round(per[len(per) // 2], 4),
            "host_wall_s": round(wall, 3),
            "prewarm": {"ms": args.prewarm_ms, "launches": prewarm_launches},
            "bias_ranges_pass_ms": round(sum(pre_ms) / len(pre_ms), 4) if use_ranges else None,
            "interval_rows": use_pure if bias is not None else None,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm" if is_decode else "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "GB/s" if is_decode else "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "algorithmic_bytes": algorithmic_bytes(w, out_bytes),
            "kernel": ("decode_kernel + decode_merge_kernel" if is_decode else
                       "delta_kernel + dkdv_kernel + dq_kernel" if args.backward else
                       "sdpa key-padding front end (whole step: padding_lengths kernels, "
                       "attn_fwd16p_kernel in place)" if args.sdpa_keypad else
                       "attn_fwd_kernel" if w.dtype == "f32" else "attn_fwd16p_kernel"),
            "kernel_ms": round(kernel_ms, 4),
        },
        "cpu_baseline": cpu,
    }
    if cold is not None:
        result["cold"] = cold
    if args.backward:
        result["config"]["pass"] = "backward"
        result["cpu_baseline"] = None  # the oracle baseline is timed for the forward only
    if args.sdpa_keypad:
        result["config"]["front_end"] = (f"sdpa: [B={w.num_seqs}, H, N={max(w.seqlens_q)}, D] "
                                         f"right-padded batch, bool key-padding mask")
        result["roofline"]["traffic"] = None
    unit = "GB/s" if is_decode else "useful TFLOP/s"
    print(f"# GPU: {ms_per_step:.4f} ms/step, {value:.1f} {unit} "
          f"({100 * value / peak:.1f}% of {peak})", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
