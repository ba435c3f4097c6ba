"""HIP path vs the fp64 oracle, element by element, on seeded inputs.

Small cases (the oracle finishes in seconds) span several query and key
tiles with ragged tails; the five full-size workloads run in the same launch
configuration as the benchmark and are checked on sampled rows the oracle
computes one by one.  Tolerances on the fp32 output: 2e-3 (bf16), 1e-3
(fp16), 1e-5 (fp32); LSE within 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import workloads
from gpu_helpers import (check, check_sampled, run_gpu, run_oracle, say, to_device)

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _small_cases():
    c = {}
    c["tiny_f32_full"] = workloads.TINY_F32
    c["tiny_f32_causal"] = workloads.TINY_F32.with_(name="tiny_f32_causal", causal=True)
    c["f32_d128_gqa_causal"] = W(name="f32_d128_gqa_causal", seqlens_q=(200, 77), seqlens_kv=(200, 77),
                                 hq=4, hkv=2, d_qk=128, d_v=128, dtype="f32", causal=True, seed=11)
    c["gqa_bf16_small"] = W(name="gqa_bf16_small", seqlens_q=(300, 1, 517, 64),
                            seqlens_kv=(300, 1, 517, 64), hq=8, hkv=2, d_qk=128, d_v=128,
                            dtype="bf16", causal=True, seed=12)
    c["gqa_bf16_small_full"] = c["gqa_bf16_small"].with_(name="gqa_bf16_small_full", causal=False)
    for d in (64, 128):
        for causal in (False, True):
            n = f"f16_d{d}_{'causal' if causal else 'full'}_small"
            c[n] = W(name=n, seqlens_q=(333, 130), seqlens_kv=(333, 130), hq=3, hkv=3, d_qk=d,
                     d_v=d, dtype="f16", causal=causal, seed=13 + d)
        n = f"f16_d{d}_prefix_lm_small"
        c[n] = W(name=n, seqlens_q=(700, 257), seqlens_kv=(700, 257), hq=2, hkv=2, d_qk=d, d_v=d,
                 dtype="f16", causal=False, bias="prefix_lm", prefix=100, seed=17)
    c["swa_bf16_small"] = W(name="swa_bf16_small", seqlens_q=(1000, 333), seqlens_kv=(1000, 333),
                            hq=4, hkv=1, d_qk=128, d_v=128, dtype="bf16", causal=True, window=200,
                            seed=18)
    c["swa_bf16_tiny_window"] = W(name="swa_bf16_tiny_window", seqlens_q=(300,), seqlens_kv=(300,),
                                  hq=2, hkv=2, d_qk=64, d_v=64, dtype="bf16", causal=True,
                                  window=3, seed=19)
    c["mla_bf16_small"] = W(name="mla_bf16_small", seqlens_q=(300, 129), seqlens_kv=(300, 129),
                            hq=4, hkv=4, d_qk=192, d_v=128, dtype="bf16", causal=True,
                            nope_rope=(128, 64), seed=20)
    c["mla_f16_small_full"] = W(name="mla_f16_small_full", seqlens_q=(150,), seqlens_kv=(150,),
                                hq=2, hkv=1, d_qk=192, d_v=128, dtype="f16", causal=False, seed=21)
    # cross attention: kv longer than q (cached decode style) and shorter (empty rows)
    c["cross_bf16_kv_longer"] = W(name="cross_bf16_kv_longer", seqlens_q=(5, 130, 1),
                                  seqlens_kv=(700, 260, 90), hq=8, hkv=8, d_qk=128, d_v=128,
                                  dtype="bf16", causal=True, seed=22)
    c["cross_f16_kv_shorter"] = W(name="cross_f16_kv_shorter", seqlens_q=(200, 64),
                                  seqlens_kv=(70, 3), hq=2, hkv=1, d_qk=64, d_v=64, dtype="f16",
                                  causal=True, seed=23)
    c["cross_bf16_window"] = W(name="cross_bf16_window", seqlens_q=(150, 40),
                               seqlens_kv=(400, 41), hq=4, hkv=2, d_qk=128, d_v=128,
                               dtype="bf16", causal=True, window=77, seed=24)
    c["zero_length_sequences"] = W(name="zero_length_sequences", seqlens_q=(0, 50, 0, 3, 0),
                                   seqlens_kv=(0, 50, 7, 0, 0), hq=2, hkv=2, d_qk=64, d_v=64,
                                   dtype="bf16", causal=False, seed=25)
    lens = tuple(workloads.random_lengths(200, 1, 16, seed=26))
    c["many_tiny_windows"] = W(name="many_tiny_windows", seqlens_q=lens, seqlens_kv=lens, hq=2,
                               hkv=1, d_qk=64, d_v=64, dtype="f16", causal=True, window=4, seed=27)
    c["mqa_bf16"] = W(name="mqa_bf16", seqlens_q=(257, 190), seqlens_kv=(257, 190), hq=8, hkv=1,
                      d_qk=64, d_v=64, dtype="bf16", causal=True, seed=28)
    return c


SMALL = _small_cases()


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_case_matches_oracle(name):
    w = SMALL[name]
    say(f"[small] {name}")
    inp = workloads.make_inputs(w)
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    check(name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("bias_heads", [1, "hq"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_random_bias_matches_oracle(dtype, bias_heads):
    w = W(name=f"random_bias_{dtype}", seqlens_q=(190, 75), seqlens_kv=(260, 75), hq=4, hkv=2,
          d_qk=128, d_v=128, dtype=dtype, causal=True, seed=30)
    say(f"[bias] {w.name} heads={bias_heads}")
    inp = workloads.make_inputs(w)
    nb = w.hq if bias_heads == "hq" else 1
    inp.bias = workloads.random_bias(w.seqlens_q, nb, 272, seed=31, neg_inf_frac=0.2)
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("dims", [(64, 64), (192, 128)])
def test_broadcast_bias_mixed_lengths(dims):
    """A bias shared by all query heads is scheduled head-major (all heads of
    a (sequence, tile) back to back); odd head and sequence counts leave a
    partial last round of groups and sequences with fewer tiles than the
    longest."""
    dqk, dv = dims
    w = W(name=f"bcast_bias_d{dqk}", seqlens_q=(400, 1, 257), seqlens_kv=(420, 9, 257), hq=6,
          hkv=3, d_qk=dqk, d_v=dv, dtype="bf16", causal=True, seed=34)
    say(f"[bias] {w.name} broadcast")
    inp = workloads.make_inputs(w)
    inp.bias = workloads.random_bias(w.seqlens_q, 1, 432, seed=35, neg_inf_frac=0.1)
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("lens", [(300, 1, 129, 700, 64, 5, 257, 513),  # 6 q-tiles: groups of 6
                                  (200, 1, 129, 256, 64, 5, 17, 3),     # 2 q-tiles: groups of 2
                                  (100, 1, 128, 64, 64, 5, 17, 3)])     # 1 q-tile: plain order
def test_many_heads_without_kv_sharing(lens):
    """hq = hkv with hq * num_seqs >= 512 takes the schedule that runs several
    query tiles of one head together (as many as the longest sequence has,
    up to 8); varlen lengths leave empty items."""
    w = W(name="mha_many_heads", seqlens_q=lens, seqlens_kv=lens, hq=64, hkv=64, d_qk=64, d_v=64,
          dtype="bf16", causal=True, seed=36)
    say(f"[small] {w.name}")
    inp = workloads.make_inputs(w)
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_late_dominant_key(dtype, d):
    """One key in a later tile dominates most rows (weight up to ~1) and its
    value is large.  Its p must come out exactly 1 (running max up to date):
    a stale running max leaves it at 2^f, f fractional, and its 16-bit
    rounding then shows up at ~0.4% of |v| (bf16), above the tolerance."""
    lens = (300, 190)
    w = W(name=f"late_dominant_{dtype}_d{d}", seqlens_q=lens, seqlens_kv=lens, hq=2, hkv=2,
          d_qk=d, d_v=d, dtype=dtype, causal=False, seed=37)
    say(f"[small] {w.name}")
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(38)
    u = np.ones(d) / math.sqrt(d)
    q = inp.q.double().numpy() + 3.0 * u
    k = inp.k.double().numpy()
    v = inp.v.double().numpy()
    for s0, key in ((0, 200), (300, 150)):  # a key in the fourth / third 64-key tile
        k[s0 + key] = 2.2 * math.sqrt(d) * u + 0.3 * rng.standard_normal((w.hkv, d))
        v[s0 + key] = 3.0
    dt = inp.q.dtype
    inp.q, inp.k, inp.v = (torch.from_numpy(x).to(dt) for x in (q, k, v))
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("bias_heads", [1, "hq"])
def test_many_heads_bias_window(bias_heads):
    """Every schedule feature at once: 64 unshared heads over 8 varlen
    sequences (row-grouped order, or head-major with a shared bias), a
    sliding window, a bias with -inf entries, and the 128-wide head's
    32-key four-slot tiles."""
    lens = (300, 1, 129, 700, 64, 5, 257, 513)
    w = W(name=f"mha_bias_window_{bias_heads}", seqlens_q=lens, seqlens_kv=lens, hq=64, hkv=64,
          d_qk=128, d_v=128, dtype="bf16", causal=True, window=150, seed=39)
    say(f"[bias] {w.name}")
    inp = workloads.make_inputs(w)
    nb = w.hq if bias_heads == "hq" else 1
    inp.bias = workloads.random_bias(w.seqlens_q, nb, 704, seed=40, neg_inf_frac=0.05)
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("n_dom", [2, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_near_tied_dominant_keys(d, dtype, n_dom):
    """Rows that see 300-700 keys, where two or three keys in later tiles
    carry almost all of the weight with logits a fraction of a unit apart
    (p of the second and third near 0.5-1, not exactly representable) and
    their values are large.  16-bit rounding of those p lands directly on
    the output; the kernel must still meet the tolerance."""
    lens = (700, 410)
    w = W(name=f"near_tied_{n_dom}_{dtype}_d{d}", seqlens_q=lens, seqlens_kv=lens, hq=4, hkv=2,
          d_qk=d, d_v=d, dtype=dtype, causal=True, seed=41 + d + n_dom)
    say(f"[small] {w.name}")
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(42 + d + n_dom)
    u = np.ones(d) / math.sqrt(d)
    q = inp.q.double().numpy() + 3.0 * u
    k = inp.k.double().numpy()
    v = inp.v.double().numpy()
    # dominant keys: one at the start of a tile, one mid-tile, one in the last tile
    for s0, lk, keys in ((0, 700, (300, 301, 650)), (700, 410, (260, 333, 400))):
        for i, key in enumerate(keys[:n_dom]):
            k[s0 + key] = (2.2 - 0.04 * i) * math.sqrt(d) * u + 0.3 * rng.standard_normal((w.hkv, d))
            v[s0 + key] = 2.5 * np.sign(rng.standard_normal((w.hkv, d)))
    dt = inp.q.dtype
    inp.q, inp.k, inp.v = (torch.from_numpy(x).to(dt) for x in (q, k, v))
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)


@pytest.mark.parametrize("d", [64, 128])
def test_outlier_channels_bf16(d):
    """bf16 with outlier channels (values 1e2..1e3 in four channels of q, k
    and v, as transformer activations spike).  fp32 accumulation keeps the
    result finite; channels without outliers meet the absolute bf16
    tolerance, the outlier channels (magnitude ~1e3, where one fp32 ulp is
    already 6e-5) the same tolerance relative to their magnitude."""
    w = W(name=f"outlier_bf16_d{d}", seqlens_q=(333, 200), seqlens_kv=(333, 200), hq=2, hkv=2,
          d_qk=d, d_v=d, dtype="bf16", causal=True, seed=43 + d)
    inp = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(44 + d)
    chans = {}
    for name in ("q", "k", "v"):
        t = getattr(inp, name)
        ch = torch.randperm(d, generator=g)[:4]
        t[:, :, ch] = (torch.rand(t.shape[0], t.shape[1], 4, generator=g) * 900 + 100).to(t.dtype)
        chans[name] = ch
    say(f"[outlier] {w.name}")
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    vch = chans["v"].numpy()
    plain = np.setdiff1d(np.arange(d), vch)
    e_plain = float(np.abs(out[:, :, plain] - ref_out[:, :, plain]).max())
    scale = float(np.abs(ref_out[:, :, vch]).max())
    e_out = float(np.abs(out[:, :, vch] - ref_out[:, :, vch]).max()) / scale
    e_lse = float(np.abs(lse.cpu().numpy() - ref_lse).max())
    say(f"  plain channels {e_plain:.3e}, outlier channels {e_out:.3e} of {scale:.0f}, "
        f"lse {e_lse:.3e} (|lse| up to {np.abs(ref_lse).max():.3g})")
    assert e_plain <= 2e-3
    assert e_out <= 2e-3
    assert e_lse <= 1e-4 * max(1.0, float(np.abs(ref_lse).max()))


def test_outlier_channels_fp32_accumulation():
    """A few channels of magnitude 1e2..1e3: 16-bit accumulation would
    overflow; fp32 accumulation must keep the result finite and correct."""
    w = W(name="outlier_f16", seqlens_q=(200,), seqlens_kv=(200,), hq=2, hkv=2, d_qk=128,
          d_v=128, dtype="f16", causal=True, scale=1.0 / math.sqrt(128), seed=32)
    inp = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(33)
    for t in (inp.q, inp.k, inp.v):
        ch = torch.randint(0, 128, (4,), generator=g)
        t[:, :, ch] = (torch.rand(t.shape[0], t.shape[1], 4, generator=g) * 900 + 100).to(t.dtype)
    say("[outlier] fp16 with outlier channels")
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    ref_out, ref_lse = run_oracle(inp)
    assert torch.isfinite(out).all()
    # the outputs here are O(1e3): compare relative to the value scale
    scale = max(1.0, float(np.abs(ref_out).max()))
    err = float(np.abs(out.cpu().numpy() - ref_out).max()) / scale
    say(f"  outlier relative error {err:.3e}")
    assert err <= 1e-3
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= 1e-3 * max(1.0, np.abs(ref_lse).max())


FULL = ["tiny_f32", "gqa_causal_bf16", "dense_f16_d128_full", "dense_f16_d128_causal",
        "dense_f16_d128_prefix_lm", "dense_f16_d64_full", "dense_f16_d64_causal",
        "dense_f16_d64_prefix_lm", "swa_bf16", "mla_bf16", "dense_bf16_d96_causal",
        "dense_bf16_d256_causal"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_sampled(name):
    """Full-size workloads, same launch as the benchmark (output in the input
    dtype) plus an fp32-output launch; sampled rows vs the oracle, and the
    16-bit output must be the RNE rounding of the fp32 one, bit for bit."""
    w = workloads.ALL[name]
    say(f"[full] {name}")
    inp = workloads.make_inputs(w)
    dev = to_device(inp)
    kw = {}
    if inp.bias is not None:
        # the benchmark's launch: the bias rows' key ranges and interval flags
        q, k, v, cq, ck, b = dev
        rg, pure = fav.bias_key_ranges(b, cq, ck, w.max_seqlen_q, return_pure=True)
        kw = dict(bias_ranges=rg, bias_pure=pure)
    out32, lse32 = run_gpu(inp, out_dtype=torch.float32, dev=dev, **kw)
    # every query head, on sampled rows of every sequence (tile edges, both
    # ends and random rows)
    check_sampled(inp, out32, lse32, list(range(w.hq)), rows_per_seq=12 if w.total_q > 50000 else 24)
    if w.dtype != "f32":
        outn, lsen = run_gpu(inp, out_dtype=inp.q.dtype, dev=dev, **kw)
        assert torch.equal(outn, out32.to(inp.q.dtype)), "16-bit output is not RNE(fp32 output)"
        assert torch.equal(lsen, lse32)
    if kw:
        # the same as reading the whole bias, bit for bit
        out_b, lse_b = run_gpu(inp, out_dtype=torch.float32, dev=dev)
        assert torch.equal(out_b, out32) and torch.equal(lse_b, lse32)
    assert torch.isfinite(out32).all()
