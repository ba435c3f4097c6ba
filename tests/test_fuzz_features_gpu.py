"""A seeded fuzzer over feature combinations, through the C ABI, against the
fp64 oracle: every 16-bit head shape (64, 96, 128, 192/128, 256), GQA
ratios, self- and cross-attention, empty and ragged sequences, causal and
window flags, each combined with one of: nothing, a bias with key ranges, a
bias of interval rows (key ranges and interval flags), a bool mask, ALiBi
slopes, or used prefixes of the spans (seqused).  It stops at its first
failure, and each case prints its parameters first."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
import oracle
import workloads
from gpu_helpers import check, run_oracle, say

pytestmark = pytest.mark.gpu

W = workloads.Workload
FEATURES = ["plain", "bias_ranges", "intervals", "mask", "alibi", "seqused"]


def _case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = ["bf16", "f16"][rng.integers(2)]
    dqk, dv = [(64, 64), (96, 96), (128, 128), (192, 128), (256, 256)][rng.integers(5)]
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    ns = int(rng.integers(1, 4))
    sq = [int(x) for x in rng.integers(0, 260, ns)]
    self_attn = rng.random() < 0.7
    sk = sq if self_attn else [int(x) for x in rng.integers(0, 330, ns)]
    causal = bool(rng.random() < 0.6)
    window = int(rng.integers(1, 150)) if causal and rng.random() < 0.3 else 0
    feature = FEATURES[i % len(FEATURES)]
    if feature == "intervals" and not self_attn:
        feature = "bias_ranges"
    w = W(name=f"fuzzf{i}", seqlens_q=tuple(sq), seqlens_kv=tuple(sk), hq=hq, hkv=hkv, d_qk=dqk,
          d_v=dv, dtype=dtype, causal=causal, window=window, seed=8000 + i)
    return w, feature, rng


@pytest.mark.parametrize("i", range(120))
def test_fuzz_features_against_oracle(i):
    w, feature, rng = _case(i)
    say(f"[fuzz features {i}] {feature} {w.dtype} d=({w.d_qk},{w.d_v}) hq={w.hq} hkv={w.hkv} "
        f"q={w.seqlens_q} kv={w.seqlens_kv} causal={w.causal} window={w.window}")
    inp = workloads.make_inputs(w)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cq, ck = inp.cu_seqlens_q.to(dev), inp.cu_seqlens_kv.to(dev)
    mq = max(w.max_seqlen_q, 1)
    cols = max(max(w.seqlens_kv), 1)
    kw = dict(scale=w.softmax_scale, causal=w.causal, window=w.window, out_dtype=torch.float32,
              return_lse=True)
    if feature == "plain":
        out, lse = fav.varlen_attention(q, k, v, cq, ck, mq, **kw)
    elif feature == "bias_ranges":
        heads = [1, w.hq][rng.integers(2)]
        inp.bias = workloads.random_bias(w.seqlens_q, heads, cols, seed=9000 + i, neg_inf_frac=0.3)
        b = inp.bias.to(dev)
        rg = fav.bias_key_ranges(b, cq, ck, mq)
        out, lse = fav.varlen_attention(q, k, v, cq, ck, mq, attn_bias=b, bias_ranges=rg, **kw)
    elif feature == "intervals":
        inp.bias = workloads.prefix_lm_bias(w.seqlens_q, int(rng.integers(0, 80)), cols)
        b = inp.bias.to(dev)
        rg, pure = fav.bias_key_ranges(b, cq, ck, mq, return_pure=True)
        out, lse = fav.varlen_attention(q, k, v, cq, ck, mq, attn_bias=b, bias_ranges=rg,
                                        bias_pure=pure, **kw)
    elif feature == "mask":
        rb = workloads.random_bias(w.seqlens_q, [1, w.hq][rng.integers(2)], cols, seed=9100 + i,
                                   neg_inf_frac=0.3)
        mask = torch.isfinite(rb)
        inp.bias = torch.zeros(rb.shape).masked_fill_(~mask, float("-inf"))
        out, lse = fav.varlen_attention(q, k, v, cq, ck, mq, attn_bias=mask.to(dev), **kw)
    elif feature == "alibi":
        slopes = (2.0 ** (-8.0 * (np.arange(w.hq) + 1) / w.hq)).astype(np.float32)
        inp.bias = torch.from_numpy(oracle.alibi_bias(slopes.astype(np.float64),
                                                      inp.cu_seqlens_q.numpy(),
                                                      inp.cu_seqlens_kv.numpy(), w.hq, cols))
        out, lse = fav.varlen_attention(q, k, v, cq, ck, mq,
                                        alibi_slopes=torch.from_numpy(slopes).to(dev), **kw)
    else:  # seqused
        uq = [int(rng.integers(-2, s + 3)) for s in w.seqlens_q]
        uk = [int(rng.integers(-2, s + 3)) for s in w.seqlens_kv]
        out, lse = fav.varlen_attention(
            q, k, v, cq, ck, mq, seqused_q=torch.tensor(uq, dtype=torch.int32, device=dev),
            seqused_kv=torch.tensor(uk, dtype=torch.int32, device=dev), **kw)
        torch.cuda.synchronize()
        og, lg = out.cpu().numpy(), lse.cpu().numpy()
        # the used rows against the oracle on the same sequences packed
        pq, cu_pq = oracle.used_prefixes(inp.q.float().numpy(), inp.cu_seqlens_q.numpy(), uq)
        pk, cu_pk = oracle.used_prefixes(inp.k.float().numpy(), inp.cu_seqlens_kv.numpy(), uk)
        pv, _ = oracle.used_prefixes(inp.v.float().numpy(), inp.cu_seqlens_kv.numpy(), uk)
        ref_o, ref_l = oracle.varlen_attention(pq, pk, pv, cu_pq, cu_pk, w.softmax_scale, w.causal,
                                               w.window, None)
        cu = inp.cu_seqlens_q.tolist()
        rows = np.concatenate([np.arange(cu[s], cu[s] + (cu_pq[s + 1] - cu_pq[s]))
                               for s in range(w.num_seqs)]).astype(np.int64)
        rest = np.setdiff1d(np.arange(w.total_q), rows)
        assert np.all(og[rest] == 0.0) and np.all(lg[:, rest] == -np.inf), "unused rows not 0 / -inf"
        check(w.name, og[rows], lg[:, rows], ref_o, ref_l, w.dtype)
        return
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(inp)
    check(w.name, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, w.dtype)
