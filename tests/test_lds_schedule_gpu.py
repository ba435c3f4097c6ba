"""LDS race check of the forward's copy schedule: the shipping library
against three schedule variants built from the same source (all 16-bit
kernels on two K/V slots; every step waiting for its own tile copies behind
a barrier before any read; the four-slot kernels with their copies one step
less ahead).  A slot refilled while still being read, or a tile read before
its copy landed, would make the results depend on timing; the variants
change that timing, so their outputs must equal the shipping kernels' bit
for bit on the four-slot instances (latent head, biased heads read as a
bias or as interval rows, the 256-wide head) and the two-slot ones (the GQA
causal prefill, the 96- and 64-wide heads)."""
import contextlib

import pytest
import torch

import flash_attention_varlen_amd as fav
import workloads
from gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu

W = workloads.Workload

CASES = {
    "latent_bf16": W(name="lds_latent_bf16", seqlens_q=(700, 129, 1), seqlens_kv=(700, 129, 1),
                     hq=4, hkv=4, d_qk=192, d_v=128, dtype="bf16", causal=True, seed=90),
    "bias_bf16_d128": W(name="lds_bias_bf16_d128", seqlens_q=(600, 77), seqlens_kv=(600, 77),
                        hq=4, hkv=2, d_qk=128, d_v=128, dtype="bf16", causal=False,
                        bias="prefix_lm", prefix=150, seed=91),
    "bias_f16_d64": W(name="lds_bias_f16_d64", seqlens_q=(900, 33), seqlens_kv=(900, 33), hq=2,
                      hkv=1, d_qk=64, d_v=64, dtype="f16", causal=False, bias="prefix_lm",
                      prefix=300, seed=92),
    # the same biases as interval rows (key ranges and interval flags given)
    "interval_bf16_d128": W(name="lds_interval_bf16_d128", seqlens_q=(600, 77),
                            seqlens_kv=(600, 77), hq=4, hkv=2, d_qk=128, d_v=128, dtype="bf16",
                            causal=False, bias="prefix_lm", prefix=150, seed=97),
    "interval_f16_d64": W(name="lds_interval_f16_d64", seqlens_q=(900, 33), seqlens_kv=(900, 33),
                          hq=2, hkv=1, d_qk=64, d_v=64, dtype="f16", causal=False,
                          bias="prefix_lm", prefix=300, seed=98),
    "gqa_causal_bf16": W(name="lds_gqa_causal_bf16", seqlens_q=(1000, 333, 64),
                         seqlens_kv=(1000, 333, 64), hq=8, hkv=2, d_qk=128, d_v=128,
                         dtype="bf16", causal=True, seed=93),
    "window_f16_d64": W(name="lds_window_f16_d64", seqlens_q=(1200,), seqlens_kv=(1200,), hq=4,
                        hkv=4, d_qk=64, d_v=64, dtype="f16", causal=True, window=300, seed=94),
    # the 256-wide head runs four slots (one workgroup per CU), the 96-wide two
    "causal_bf16_d256": W(name="lds_causal_bf16_d256", seqlens_q=(500, 77), seqlens_kv=(500, 77),
                          hq=2, hkv=1, d_qk=256, d_v=256, dtype="bf16", causal=True, seed=95),
    "full_f16_d96": W(name="lds_full_f16_d96", seqlens_q=(600, 31), seqlens_kv=(600, 31), hq=2,
                      hkv=2, d_qk=96, d_v=96, dtype="f16", causal=False, seed=96),
}


@contextlib.contextmanager
def _library(lib):
    saved = fav._lib
    fav._lib = lib
    try:
        yield
    finally:
        fav._lib = saved


def _run(w, dev):
    q, k, v, cq, ck, b = dev
    rg = pure = None
    if w.name.startswith("lds_interval"):
        rg, pure = fav.bias_key_ranges(b, cq, ck, w.max_seqlen_q, return_pure=True)
        assert bool(pure.all())
    out, lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale,
                                    causal=w.causal, window=w.window, attn_bias=b,
                                    out_dtype=torch.float32, return_lse=True, bias_ranges=rg,
                                    bias_pure=pure)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("variant", ["slots2", "synccopies", "shallow"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_schedule_variant_is_bitwise_equal(name, variant):
    w = CASES[name]
    say(f"[lds] {name} vs {variant}")
    inp = workloads.make_inputs(w)
    dev = to_device(inp)
    fav.load_library()
    ref_out, ref_lse = _run(w, dev)
    with _library(fav.variant_library(variant)):
        out, lse = _run(w, dev)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
