"""Graph capture through the C ABI.  The forward and the non-allocating
decode launch no allocation, fill or host synchronisation, so a caller can
record them into a HIP graph (here torch.cuda.CUDAGraph) and replay it.  Each
test records one call, then replays the graph several times with new inputs
copied into the recorded buffers between replays (eager work and a
synchronisation between replays), and checks every replay, bit for bit,
against an eager call on the same inputs."""
import pytest
import torch

import flash_attention_varlen_amd as fav
import workloads
from gpu_helpers import say

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _refill(gen, *tensors):
    for t in tensors:
        t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype))


def _capture(fn):
    """Warm the call up on a side stream (first-call set-up stays out of the
    graph), then record it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_forward_graph_replays(dtype, d):
    w = W(name=f"graph_fwd_{dtype}", seqlens_q=(300, 77, 1, 513), seqlens_kv=(300, 77, 1, 513),
          hq=8, hkv=2, d_qk=d, d_v=d, dtype=dtype, causal=True, seed=120)
    inp = workloads.make_inputs(w)
    dev = "cuda"
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    out = torch.empty(w.total_q, w.hq, w.d_v, dtype=q.dtype, device=dev)
    lse = torch.empty(w.hq, w.total_q, dtype=torch.float32, device=dev)
    kw = dict(scale=w.softmax_scale, causal=True)
    say(f"[graph] forward {dtype} d={d}")
    g = _capture(lambda: fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, out=out, lse=lse, **kw))
    gen = torch.Generator().manual_seed(121)
    for r in range(3):
        _refill(gen, q, k, v)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = fav.varlen_attention(q, k, v, cq, ck, w.max_seqlen_q, return_lse=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: out differs from the eager call"
        assert torch.equal(lse, ref_lse), f"replay {r}: lse differs from the eager call"


def test_noalloc_decode_graph_replays():
    w = W(name="graph_decode", seqlens_q=(1, 1, 1), seqlens_kv=(5000, 17, 3000), hq=16, hkv=4,
          d_qk=128, d_v=128, dtype="bf16", causal=True, seed=122)
    inp = workloads.make_inputs(w)
    dev = "cuda"
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    out = torch.empty(w.total_q, w.hq, w.d_v, dtype=torch.float32, device=dev)
    lse = torch.empty(w.hq, w.total_q, dtype=torch.float32, device=dev)
    say("[graph] non-allocating decode")
    g = _capture(lambda: fav.varlen_decode_noalloc(q, k, v, cq, ck, w.max_seqlen_q, w.max_seqlen_kv,
                                                   out, lse, causal=True))
    gen = torch.Generator().manual_seed(123)
    for r in range(3):
        _refill(gen, q, k, v)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = fav.varlen_decode(q, k, v, cq, ck, w.max_seqlen_q, w.max_seqlen_kv,
                                             causal=True, out_dtype=torch.float32, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: out differs from the eager call"
        assert torch.equal(lse, ref_lse), f"replay {r}: lse differs from the eager call"
