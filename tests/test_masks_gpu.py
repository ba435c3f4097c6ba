"""Bit-exact probes of the masks and index maps, the tile schedule,
determinism and 64-bit addressing, through the C ABI.

With q = 0 every visible logit is 0, so p = 1 exactly and the fp32 row sum
is the exact visible-key count n; out * n and exp(lse) are then integers
that must match the oracle's mask exactly (integer comparison, no
tolerance).
"""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import check, run_gpu, run_oracle, say, to_device

pytestmark = pytest.mark.gpu

W = workloads.Workload

MASK_SHAPES = {
    "causal_self": dict(seqlens_q=(300, 1, 129), seqlens_kv=(300, 1, 129), causal=True, window=0),
    "full_self": dict(seqlens_q=(130, 64), seqlens_kv=(130, 64), causal=False, window=0),
    "causal_kv_longer": dict(seqlens_q=(70, 3), seqlens_kv=(333, 64), causal=True, window=0),
    "causal_kv_shorter": dict(seqlens_q=(260, 50), seqlens_kv=(100, 7), causal=True, window=0),
    "window_self": dict(seqlens_q=(500, 90), seqlens_kv=(500, 90), causal=True, window=37),
    "window_cross": dict(seqlens_q=(140, 33), seqlens_kv=(390, 20), causal=True, window=100),
}


def _probe_workload(shape, dtype="bf16", d=64, hq=4, hkv=2):
    return W(name="probe", hq=hq, hkv=hkv, d_qk=d, d_v=d, dtype=dtype, seed=40, **shape)


def _counts(w):
    """Oracle's visible-key count per (seq, local row) and per-residue histogram."""
    res = []
    for lq, lk in zip(w.seqlens_q, w.seqlens_kv):
        i = np.arange(lq)[:, None]
        j = np.arange(lk)[None, :]
        vis = oracle.visible(i, j, lq, lk, w.causal, w.window)
        res.append(vis)
    return res


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", sorted(MASK_SHAPES))
def test_count_and_one_hot_v_probe(shape, dtype):
    w = _probe_workload(MASK_SHAPES[shape], dtype=dtype)
    say(f"[probe] counts {shape} {dtype}")
    inp = workloads.make_inputs(w)
    inp.q.zero_()
    dv = w.d_v
    # one-hot V: v[j, g, d] = 1 iff d == j mod Dv (j local to its sequence)
    v = torch.zeros_like(inp.v)
    for s in range(w.num_seqs):
        a, b = int(inp.cu_seqlens_kv[s]), int(inp.cu_seqlens_kv[s + 1])
        j = torch.arange(b - a)
        v[a + j, :, j % dv] = 1
    inp.v = v
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    for s, vis in enumerate(_counts(w)):
        q0 = int(inp.cu_seqlens_q[s])
        n = vis.sum(axis=1)
        hist = np.zeros((vis.shape[0], dv), dtype=np.int64)
        for jj in range(vis.shape[1]):
            hist[:, jj % dv] += vis[:, jj]
        for h in range(w.hq):
            got_n = np.where(np.isneginf(lse[h, q0:q0 + len(n)]), 0,
                             np.rint(np.exp(lse[h, q0:q0 + len(n)]))).astype(np.int64)
            assert np.array_equal(got_n, n), f"seq {s} head {h}: visible counts differ"
            got_hist = np.rint(out[q0:q0 + len(n), h, :] * n[:, None]).astype(np.int64)
            assert np.array_equal(got_hist, hist), f"seq {s} head {h}: key histogram differs"
            assert np.all(out[q0:q0 + len(n), h, :][n == 0] == 0.0)


def test_gqa_head_map_probe():
    w = _probe_workload(MASK_SHAPES["causal_self"], d=64, hq=16, hkv=4)
    say("[probe] gqa map")
    inp = workloads.make_inputs(w)
    inp.q.zero_()
    v = torch.zeros_like(inp.v)
    for g in range(w.hkv):
        v[:, g, g] = 1
    inp.v = v
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    n = np.rint(np.exp(lse.cpu().numpy())).astype(np.int64)  # [hq, T]
    o = np.rint(out.cpu().numpy() * n.T[:, :, None]).astype(np.int64)
    for h in range(w.hq):
        expect = np.zeros((w.total_q, w.d_v), dtype=np.int64)
        expect[:, h // (w.hq // w.hkv)] = n[h]
        assert np.array_equal(o[:, h, :], expect), f"head {h} reads the wrong kv head"


def test_sequence_map_probe():
    shape = dict(seqlens_q=(40, 200, 1, 77), seqlens_kv=(90, 150, 5, 77), causal=False, window=0)
    w = _probe_workload(shape, d=64, hq=2, hkv=2)
    say("[probe] sequence map")
    inp = workloads.make_inputs(w)
    inp.q.zero_()
    v = torch.zeros_like(inp.v)
    for s in range(w.num_seqs):
        a, b = int(inp.cu_seqlens_kv[s]), int(inp.cu_seqlens_kv[s + 1])
        v[a:b, :, s] = 1
    inp.v = v
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    out = out.cpu().numpy()
    for s in range(w.num_seqs):
        a, b = int(inp.cu_seqlens_q[s]), int(inp.cu_seqlens_q[s + 1])
        expect = np.zeros(w.d_v)
        expect[s] = 1.0
        assert np.array_equal(np.rint(out[a:b] * 1e6) / 1e6, np.broadcast_to(expect, out[a:b].shape))


@pytest.mark.parametrize("shape", ["causal_self", "window_self", "causal_kv_longer"])
def test_masked_keys_do_not_leak(shape):
    """Overwrite K/V of keys that some rows cannot see with huge finite values:
    out and lse of exactly those rows, and of every other sequence, stay
    bitwise unchanged."""
    w = _probe_workload(MASK_SHAPES[shape], dtype="bf16", d=128, hq=4, hkv=2)
    say(f"[probe] leak {shape}")
    inp = workloads.make_inputs(w)
    base_out, base_lse = run_gpu(inp, out_dtype=torch.float32)
    s = 0
    lq, lk = w.seqlens_q[s], w.seqlens_kv[s]
    jstar = lk - lq // 2  # about half of the rows see it
    k0 = int(inp.cu_seqlens_kv[s])
    inp.k[k0 + jstar] = 300.0
    inp.v[k0 + jstar] = -5000.0
    out, lse = run_gpu(inp, out_dtype=torch.float32)
    i = np.arange(lq)
    blind = ~oracle.visible(i, np.full(lq, jstar), lq, lk, w.causal, w.window)
    assert blind.any()
    rows = int(inp.cu_seqlens_q[s]) + i[blind]
    assert torch.equal(out[rows], base_out[rows])
    assert torch.equal(lse[:, rows], base_lse[:, rows])
    other = slice(int(inp.cu_seqlens_q[1]), w.total_q)
    assert torch.equal(out[other], base_out[other])
    assert torch.equal(lse[:, other], base_lse[:, other])
    # and the rows that do see the key did change
    seen = int(inp.cu_seqlens_q[s]) + i[~blind]
    if len(seen):
        assert not torch.equal(out[seen], base_out[seen])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", sorted(MASK_SHAPES))
def test_tile_schedule_visits_exactly_the_needed_tiles(shape, dtype):
    """Debug tile counters: every workgroup visits exactly the key tiles that
    hold at least one visible key for its rows (diagonal skip, window jump)."""
    w = _probe_workload(MASK_SHAPES[shape], dtype=dtype)
    say(f"[probe] tiles {shape} {dtype}")
    code = {"bf16": fav.BF16, "f32": fav.F32}[dtype]
    bm, bn = fav.mi_attn_tile_shape(code, w.d_qk, w.d_v)
    nqt = (w.max_seqlen_q + bm - 1) // bm
    counts = torch.full((nqt * w.num_seqs * w.hq,), -1, dtype=torch.int32, device="cuda")
    inp = workloads.make_inputs(w)
    run_gpu(inp, out_dtype=torch.float32, tile_counts=counts)
    got = counts.cpu().numpy().reshape(nqt, w.num_seqs, w.hq)
    for s, vis in enumerate(_counts(w)):
        lq = w.seqlens_q[s]
        for t in range((lq + bm - 1) // bm):
            rows = vis[t * bm:(t + 1) * bm]
            keys = np.nonzero(rows.any(axis=0))[0]
            expect = len(set((keys // bn).tolist()))
            assert np.all(got[t, s, :] == expect), (s, t, got[t, s], expect)
        for t in range((lq + bm - 1) // bm, nqt):
            assert np.all(got[t, s, :] == -1)


@pytest.mark.parametrize("shape", ["causal_self", "causal_kv_longer", "window_self", "window_cross"])
def test_tile_schedule_with_bias_d128(shape):
    """With a bias the 128-wide 16-bit kernel walks 32-key half tiles; the
    debug counts are still reported in mi_attn_tile_shape's BN units and must
    equal the BN-tiles spanned by the visible keys (a zero bias shared by
    every head, so the head-major schedule is used too)."""
    w = _probe_workload(MASK_SHAPES[shape], dtype="bf16", d=128)
    say(f"[probe] tiles with bias {shape}")
    bm, bn = fav.mi_attn_tile_shape(fav.BF16, 128, 128)
    nqt = (w.max_seqlen_q + bm - 1) // bm
    counts = torch.full((nqt * w.num_seqs * w.hq,), -1, dtype=torch.int32, device="cuda")
    inp = workloads.make_inputs(w)
    cols = (max(w.seqlens_kv) + 3) // 4 * 4  # row stride: a multiple of 4 elements
    inp.bias = torch.zeros(w.total_q, 1, cols, dtype=torch.float32)
    run_gpu(inp, out_dtype=torch.float32, tile_counts=counts)
    got = counts.cpu().numpy().reshape(nqt, w.num_seqs, w.hq)
    for s, vis in enumerate(_counts(w)):
        lq = w.seqlens_q[s]
        for t in range((lq + bm - 1) // bm):
            rows = vis[t * bm:(t + 1) * bm]
            keys = np.nonzero(rows.any(axis=0))[0]
            expect = (int(keys.max()) // bn - int(keys.min()) // bn + 1) if len(keys) else 0
            assert np.all(got[t, s, :] == expect), (s, t, got[t, s], expect)
        for t in range((lq + bm - 1) // bm, nqt):
            assert np.all(got[t, s, :] == -1)


def test_window_cost_scales_with_window():
    """Visited tiles per query tile of a 16384-token sequence track W, not L."""
    totals = {}
    for win in (1024, 4096):
        w = W(name="swa_tiles", seqlens_q=(16384,), seqlens_kv=(16384,), hq=1, hkv=1, d_qk=128,
              d_v=128, dtype="bf16", causal=True, window=win, seed=41)
        bm, bn = fav.mi_attn_tile_shape(fav.BF16, 128, 128)
        nqt = (16384 + bm - 1) // bm
        counts = torch.full((nqt,), -1, dtype=torch.int32, device="cuda")
        inp = workloads.make_inputs(w)
        run_gpu(inp, out_dtype=torch.bfloat16, tile_counts=counts)
        c = counts.cpu().numpy()
        # closed form: query tile t covers keys [max(0, t*BM - W + 1), (t+1)*BM)
        expect = [((t + 1) * bm + bn - 1) // bn - max(0, t * bm - win + 1) // bn for t in range(nqt)]
        assert c.tolist() == expect
        totals[win] = int(c.sum())
    # cost follows W: at BM=128, BN=64 this is 2232 vs 7392 tiles (full causal: 16512)
    assert 3.0 < totals[4096] / totals[1024] < 3.6


def test_bitwise_deterministic():
    w = workloads.GQA_CAUSAL_BF16.with_(seqlens_q=(900, 1500), seqlens_kv=(900, 1500))
    say("[det] run twice")
    inp = workloads.make_inputs(w)
    dev = to_device(inp)
    o1, l1 = run_gpu(inp, out_dtype=torch.bfloat16, dev=dev)
    o2, l2 = run_gpu(inp, out_dtype=torch.bfloat16, dev=dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_offsets_beyond_2_pow_31_bytes():
    """A sequence whose q/k/v/out rows start more than 2^31 bytes into their
    buffers (64-bit address arithmetic)."""
    big, small, H, D, win = 1_050_000, 500, 8, 128, 64
    assert big * H * D * 2 > 2 ** 31
    w_small = W(name="far_seq", seqlens_q=(small,), seqlens_kv=(small,), hq=H, hkv=H, d_qk=D,
                d_v=D, dtype="bf16", causal=True, window=win, seed=42)
    inp_small = workloads.make_inputs(w_small)
    say("[far] allocating >2 GiB buffers")
    T = big + small
    q = torch.zeros(T, H, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    q[big:] = inp_small.q.cuda()
    k[big:] = inp_small.k.cuda()
    v[big:] = inp_small.v.cuda()
    cu = torch.tensor([0, big, T], dtype=torch.int32, device="cuda")
    out, lse = fav.varlen_attention(q, k, v, cu, cu, big, causal=True, window=win,
                                    out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert out[big:].data_ptr() - out.data_ptr() > 2 ** 31
    ref_out, ref_lse = run_oracle(inp_small)
    check("far_seq", out[big:].cpu().numpy(), lse[:, big:].cpu().numpy(), ref_out, ref_lse, "bf16")
    # the big all-zero sequence: out 0, exp(lse) = min(i + 1, W) visible keys
    assert torch.count_nonzero(out[:big]) == 0
    n = torch.exp(lse[:, :big].double()).round().long().cpu()
    expect = torch.clamp(torch.arange(big) + 1, max=win)
    assert torch.equal(n, expect.expand(H, big))
