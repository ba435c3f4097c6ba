"""Seeded input generators (CPU only)."""
import torch

import workloads


def test_gqa_lengths_drawn_from_seed_one():
    assert workloads.cfg2_lengths() == [1677, 2626, 1676, 2065, 630, 4080, 4078, 3373]
    assert list(workloads.GQA_CAUSAL_BF16.seqlens_q) == workloads.cfg2_lengths()
    assert workloads.GQA_CAUSAL_BF16.total_q == 20205


def test_tiny_inputs_shapes_and_determinism():
    w = workloads.TINY_F32
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    assert a.q.shape == (210, 2, 64) and a.q.dtype == torch.float32
    assert a.cu_seqlens_q.tolist() == [0, 17, 81, 210]
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)


def test_latent_attention_concatenates_nope_and_rope():
    w = workloads.MLA_BF16.with_(seqlens_q=(5, 3), seqlens_kv=(5, 3), hq=2, hkv=2)
    x = workloads.make_inputs(w)
    assert x.q.shape == (8, 2, 192) and x.k.shape == (8, 2, 192) and x.v.shape == (8, 2, 128)
    g = torch.Generator().manual_seed(w.seed)
    qn = torch.randn(8, 2, 128, generator=g)
    qr = torch.randn(8, 2, 64, generator=g)
    assert torch.equal(x.q, torch.cat([qn, qr], -1).to(torch.bfloat16))


def test_bf16_cast_is_round_to_nearest_even():
    w = workloads.GQA_CAUSAL_BF16.with_(seqlens_q=(3,), seqlens_kv=(3,))
    x = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(w.seed)
    qf = torch.randn(3, 32, 128, generator=g)
    # RNE reference: add the rounding bias to the raw fp32 bits and truncate
    bits = qf.view(torch.int32).to(torch.int64)
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = x.q.view(torch.int16).to(torch.int64) & 0xFFFF
    assert torch.equal(got, rne)


def test_decode_lengths_are_the_seeded_draw():
    assert list(workloads.DECODE_BF16.seqlens_kv) == workloads.decode_lengths()
