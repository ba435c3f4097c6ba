"""Used prefixes of padded spans through the C ABI (seqused_q / seqused_kv):
the right-padding check against the oracle, integer-exact; the forward on
spans with used prefixes equal, bit for bit, to the forward on the same
sequences packed, with the unused rows of every span at 0 / -inf and the
oracle's values on the used ones; the split-KV decode on a cache longer than
it is filled; and the SDPA adapter's in-place path for right-padded batches."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import check, run_oracle, say

pytestmark = pytest.mark.gpu

W = workloads.Workload


@pytest.mark.parametrize("kind", ["right", "left", "holes", "empty_and_full"])
def test_padding_lengths_match_oracle(kind):
    g = torch.Generator().manual_seed(110)
    bsz, n = 7, 300
    lens = torch.randint(0, n + 1, (bsz,), generator=g)
    pos = torch.arange(n)[None, :]
    if kind == "right":
        mask = pos < lens[:, None]
    elif kind == "left":
        mask = pos >= (n - lens)[:, None]
    elif kind == "holes":
        mask = (pos < lens[:, None]) & (torch.rand(bsz, n, generator=g) > 0.05)
    else:
        mask = pos < torch.tensor([0, n, 1, n - 1, 0, n, 5])[:, None]
    say(f"[lengths] {kind}")
    got_len, got_spans, got_right, got_longest = fav.padding_lengths(mask.cuda())
    c, spans, right, longest = oracle.padding_lengths(mask.numpy())
    assert np.array_equal(got_len.cpu().numpy().astype(np.int64), c)
    assert np.array_equal(got_spans.cpu().numpy().astype(np.int64), spans)
    assert got_right == right and got_longest == longest
    if kind in ("right", "empty_and_full"):
        assert got_right


CASES = {
    # name: (spans q, used q, spans kv, used kv, hq, hkv, d_qk, d_v, dtype, causal, window)
    "gqa_causal_bf16_d128": ((300, 300, 300), (300, 17, 0), (300, 300, 300), (300, 17, 0),
                             8, 2, 128, 128, "bf16", True, 0),
    "full_f16_d64": ((257, 257), (100, 257), (257, 257), (100, 257), 4, 4, 64, 64, "f16",
                     False, 0),
    "cross_bf16_d128": ((64, 200), (1, 150), (512, 512), (333, 512), 4, 1, 128, 128, "bf16",
                        True, 0),
    "window_f16_d128": ((400, 400), (390, 129), (400, 400), (390, 129), 4, 2, 128, 128, "f16",
                        True, 70),
    "latent_bf16_d192": ((200, 200), (200, 31), (200, 200), (200, 31), 2, 2, 192, 128, "bf16",
                         True, 0),
    "f32_d64": ((130, 130), (77, 1), (130, 130), (77, 1), 2, 2, 64, 64, "f32", False, 0),
}


def _spans_case(name):
    sq, uq, sk, uk, hq, hkv, dqk, dv, dt, causal, window = CASES[name]
    w = W(name=f"seqused_{name}", seqlens_q=sq, seqlens_kv=sk, hq=hq, hkv=hkv, d_qk=dqk, d_v=dv,
          dtype=dt, causal=causal, window=window, seed=111)
    return w, uq, uk


@pytest.mark.parametrize("name", sorted(CASES))
def test_forward_on_used_prefixes(name):
    w, uq, uk = _spans_case(name)
    inp = workloads.make_inputs(w)
    say(f"[seqused] {name}: spans q {w.seqlens_q} used {uq}, spans kv {w.seqlens_kv} used {uk}")
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    used_q = torch.tensor(uq, dtype=torch.int32, device=dev)
    used_k = torch.tensor(uk, dtype=torch.int32, device=dev)
    # poisoned outputs: every row of every span must be written
    out = torch.full((w.total_q, w.hq, w.d_v), float("nan"), device=dev)
    lse = torch.full((w.hq, w.total_q), float("nan"), device=dev)
    fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, scale=w.softmax_scale, causal=w.causal,
                         window=w.window, out=out, lse=lse, out_dtype=torch.float32,
                         seqused_q=used_q, seqused_kv=used_k)
    # the same sequences packed
    pq, cu_pq = oracle.used_prefixes(inp.q.numpy() if w.dtype == "f32" else inp.q.float().numpy(),
                                     inp.cu_seqlens_q.numpy(), uq)
    pk, cu_pk = oracle.used_prefixes(inp.k.float().numpy(), inp.cu_seqlens_kv.numpy(), uk)
    pv, _ = oracle.used_prefixes(inp.v.float().numpy(), inp.cu_seqlens_kv.numpy(), uk)
    tdt = inp.q.dtype
    pq_t, pk_t, pv_t = (torch.from_numpy(x).to(tdt).to(dev) for x in (pq, pk, pv))
    cpq = torch.from_numpy(cu_pq).to(torch.int32).to(dev)
    cpk = torch.from_numpy(cu_pk).to(torch.int32).to(dev)
    out_p, lse_p = fav.varlen_attention(pq_t, pk_t, pv_t, cpq, cpk, max(max(uq), 1),
                                        scale=w.softmax_scale, causal=w.causal, window=w.window,
                                        out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    cu = inp.cu_seqlens_q.tolist()
    for s, u in enumerate(uq):
        a0, p0 = cu[s], int(cu_pq[s])
        assert torch.equal(out[a0:a0 + u], out_p[p0:p0 + u]), f"sequence {s}: used rows differ"
        assert torch.equal(lse[:, a0:a0 + u], lse_p[:, p0:p0 + u])
        rest = out[a0 + u:cu[s + 1]]
        assert torch.equal(rest, torch.zeros_like(rest)), f"sequence {s}: unused rows not 0"
        assert bool((lse[:, a0 + u:cu[s + 1]] == float("-inf")).all())
    # and the packed problem against the oracle
    pinp = workloads.Inputs(workload=w.with_(name=w.name + "_packed",
                                             seqlens_q=tuple(int(x) for x in np.diff(cu_pq)),
                                             seqlens_kv=tuple(int(x) for x in np.diff(cu_pk))),
                            q=pq_t.cpu(), k=pk_t.cpu(), v=pv_t.cpu(),
                            cu_seqlens_q=cpq.cpu(), cu_seqlens_kv=cpk.cpu(), bias=None)
    ref_out, ref_lse = run_oracle(pinp)
    check(name, out_p.cpu().numpy(), lse_p.cpu().numpy(), ref_out, ref_lse, w.dtype)


def test_decode_on_a_longer_cache():
    """Key caches allocated longer than they are filled: the decode over the
    used keys equals, bit for bit, the decode over the same caches packed."""
    sk, uk = (6000, 3000, 4096), (5000, 17, 4096)
    w = W(name="seqused_decode", seqlens_q=(1, 1, 1), seqlens_kv=sk, hq=16, hkv=4, d_qk=128,
          d_v=128, dtype="bf16", causal=True, seed=112)
    inp = workloads.make_inputs(w)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    say("[seqused] decode")
    out_u, lse_u = fav.varlen_decode(q, k, v, cq, ck, 1, max(sk), scale=w.softmax_scale,
                                     causal=True, out_dtype=torch.float32, return_lse=True,
                                     seqused_kv=torch.tensor(uk, dtype=torch.int32, device=dev))
    pk, cu_pk = oracle.used_prefixes(inp.k.float().numpy(), inp.cu_seqlens_kv.numpy(), uk)
    pv, _ = oracle.used_prefixes(inp.v.float().numpy(), inp.cu_seqlens_kv.numpy(), uk)
    pk_t, pv_t = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (pk, pv))
    cpk = torch.from_numpy(cu_pk).to(torch.int32).to(dev)
    out_p, lse_p = fav.varlen_decode(q, pk_t, pv_t, cq, cpk, 1, max(sk), scale=w.softmax_scale,
                                     causal=True, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_u, out_p) and torch.equal(lse_u, lse_p)


@pytest.mark.parametrize("causal", [False, True])
def test_sdpa_right_padded_in_place(causal):
    """A right-padded self-attention batch on token-major storage runs in
    place (no packing); it equals, bit for bit, the packed path the same
    tensors take in head-major storage, and torch's SDPA (fp32) within the
    tolerance on the valid rows."""
    g = torch.Generator().manual_seed(113)
    bsz, n, hq, hkv, d = 4, 256, 8, 2, 128
    dev = "cuda"
    lens = torch.tensor([256, 100, 1, 177])
    mask = (torch.arange(n)[None, :] < lens[:, None]).to(dev)
    tm = [torch.randn(bsz, n, h, d, generator=g).to(torch.bfloat16).to(dev) for h in (hq, hkv, hkv)]
    q_tm, k_tm, v_tm = (t.transpose(1, 2) for t in tm)          # views of token-major storage
    q_hm, k_hm, v_hm = (t.contiguous() for t in (q_tm, k_tm, v_tm))  # head-major copies
    say(f"[seqused] sdpa causal={causal}")
    o_in = fav.sdpa(q_tm, k_tm, v_tm, attn_mask=mask[:, None, None, :], is_causal=causal,
                    enable_gqa=True, out_dtype=torch.float32)
    o_pk = fav.sdpa(q_hm, k_hm, v_hm, attn_mask=mask[:, None, None, :], is_causal=causal,
                    enable_gqa=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o_in.stride(2) != o_pk.stride(2)  # the two took different paths
    assert torch.equal(o_in, o_pk)
    rep = hq // hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        q_hm.float(), k_hm.float().repeat_interleave(rep, 1).contiguous(),
        v_hm.float().repeat_interleave(rep, 1).contiguous(),
        attn_mask=mask[:, None, None, :] & (torch.ones(n, n, dtype=torch.bool, device=dev).tril()
                                            if causal else True))
    for b in range(bsz):
        L = int(lens[b])
        err = float((o_in[b, :, :L] - ref[b, :, :L]).abs().max())
        assert err <= 2e-3, (b, err)
        assert bool((o_in[b, :, L:] == 0).all())
