"""A seeded fuzzer for the split-KV decode (mi_attn_varlen_decode) through the
C ABI, against the fp64 oracle: bf16 / fp16, head dims 64 and 128, GQA
ratios, 1-16 query rows per sequence (at most 64 rows per kv head), key
caches of 0 to 6000 keys, causal (end-aligned) or full, windows, used
prefixes of the caches (seqused_kv), and automatic or given chunk counts."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import check, say

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _case(i):
    rng = np.random.default_rng(15000 + i)
    dtype = ["bf16", "f16"][rng.integers(2)]
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * group
    ns = int(rng.integers(1, 5))
    max_rows = max(1, min(16, 64 // group))
    sq = [int(x) for x in rng.integers(1, max_rows + 1, ns)]
    sk = [int(x) for x in rng.integers(0, 6000, ns)]
    causal = bool(rng.random() < 0.7)
    window = int(rng.integers(1, 3000)) if causal and rng.random() < 0.3 else 0
    used = [int(rng.integers(-1, s + 2)) for s in sk] if rng.random() < 0.3 else None
    splits = int(rng.choice([0, 0, 1, 3, 17]))
    w = W(name=f"fuzzd{i}", seqlens_q=tuple(sq), seqlens_kv=tuple(sk), hq=hq, hkv=hkv, d_qk=d,
          d_v=d, dtype=dtype, causal=causal, window=window, seed=16000 + i)
    return w, used, splits


@pytest.mark.parametrize("i", range(40))
def test_fuzz_decode_against_oracle(i):
    w, used, splits = _case(i)
    say(f"[fuzz decode {i}] {w.dtype} d={w.d_qk} hq={w.hq} hkv={w.hkv} q={w.seqlens_q} "
        f"kv={w.seqlens_kv} causal={w.causal} window={w.window} used={used} splits={splits}")
    inp = workloads.make_inputs(w)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    extra = {}
    if used is not None:
        extra["seqused_kv"] = torch.tensor(used, dtype=torch.int32, device=dev)
    out, lse = fav.varlen_decode(q, k, v, cq, ck, w.max_seqlen_q, max(w.max_seqlen_kv, 1),
                                 scale=w.softmax_scale, causal=w.causal, window=w.window,
                                 num_splits=splits, out_dtype=torch.float32, return_lse=True,
                                 **extra)
    torch.cuda.synchronize()
    kk, vv, cu_k = inp.k.double().numpy(), inp.v.double().numpy(), inp.cu_seqlens_kv.numpy()
    if used is not None:  # the oracle on the used prefixes of the caches
        kk, cu_k = oracle.used_prefixes(kk, inp.cu_seqlens_kv.numpy(), used)
        vv, _ = oracle.used_prefixes(vv, inp.cu_seqlens_kv.numpy(), used)
    ref_o, ref_l = oracle.varlen_attention(inp.q.double().numpy(), kk, vv, inp.cu_seqlens_q.numpy(),
                                           cu_k, w.softmax_scale, w.causal, w.window, None)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, w.dtype)
