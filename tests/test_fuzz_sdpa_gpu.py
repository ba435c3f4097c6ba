"""A seeded fuzzer for the SDPA adapter (sdpa with a boolean key-padding
mask): right-padded, left-padded and holed masks, causal or not, GQA,
head-major tensors or views of token-major storage (the in-place path), bf16
and fp16.  The reference is the dense masked softmax attention written out
in fp32 on the CPU: the valid query rows must match it within the forward
tolerance, and padded query rows (and rows that see no key) are 0."""
import numpy as np
import pytest
import torch

import flash_attention_varlen_amd as fav
from gpu_helpers import OUT_TOL, say

pytestmark = pytest.mark.gpu


def _case(i):
    rng = np.random.default_rng(17000 + i)
    dtype = ["bf16", "f16"][rng.integers(2)]
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    bsz = int(rng.integers(1, 5))
    n = int(rng.integers(1, 300))
    kind = ["right", "left", "holes"][i % 3]
    causal = bool(rng.random() < 0.5)
    token_major = bool(rng.random() < 0.6)
    lens = rng.integers(0, n + 1, bsz)
    pos = np.arange(n)[None, :]
    if kind == "right":
        mask = pos < lens[:, None]
    elif kind == "left":
        mask = pos >= (n - lens)[:, None]
    else:
        mask = (pos < lens[:, None]) & (rng.random((bsz, n)) > 0.2)
    return dict(dtype=dtype, d=d, hq=hq, hkv=hkv, bsz=bsz, n=n, kind=kind, causal=causal,
                token_major=token_major, mask=mask, seed=18000 + i)


def _reference(q, k, v, mask, causal, scale):
    """fp32 CPU: [B, H, N, D] masked softmax attention; rows that see no key 0."""
    rep = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(rep, 1)
    v = v.repeat_interleave(rep, 1)
    s = torch.matmul(q, k.transpose(2, 3).contiguous()) * scale
    vis = mask[:, None, None, :].expand(s.shape).clone()
    if causal:
        n = s.shape[2]
        vis &= torch.ones(n, n, dtype=torch.bool).tril()
    s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.where(vis.any(-1, keepdim=True), p, torch.zeros_like(p))
    return torch.matmul(p, v)


@pytest.mark.parametrize("i", range(30))
def test_fuzz_sdpa_against_dense_reference(i):
    c = _case(i)
    say(f"[fuzz sdpa {i}] {c['kind']} {c['dtype']} d={c['d']} hq={c['hq']} hkv={c['hkv']} "
        f"B={c['bsz']} N={c['n']} causal={c['causal']} token_major={c['token_major']}")
    g = torch.Generator().manual_seed(c["seed"])
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float16
    bsz, n, d = c["bsz"], c["n"], c["d"]
    tensors = []
    for h in (c["hq"], c["hkv"], c["hkv"]):
        t = torch.randn(bsz, n, h, d, generator=g).to(tdt)
        tensors.append(t)
    dev = "cuda"
    if c["token_major"]:
        qd, kd, vd = (t.to(dev).transpose(1, 2) for t in tensors)
    else:
        qd, kd, vd = (t.transpose(1, 2).contiguous().to(dev) for t in tensors)
    mask = torch.from_numpy(c["mask"])
    scale = 1.0 / d ** 0.5
    out = fav.sdpa(qd, kd, vd, attn_mask=mask.to(dev)[:, None, None, :], is_causal=c["causal"],
                   enable_gqa=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q32, k32, v32 = (t.float().transpose(1, 2).contiguous() for t in tensors)
    ref = _reference(q32, k32, v32, mask, c["causal"], scale)
    got = out.cpu()
    valid = mask[:, None, :, None].expand(got.shape)
    assert bool((got[~valid] == 0).all()), "padded query rows are not 0"
    err = float((got - ref).abs()[valid].max()) if bool(valid.any()) else 0.0
    say(f"  max|out-ref| on valid rows {err:.3e} (tol {OUT_TOL[c['dtype']]:.0e})")
    assert err <= OUT_TOL[c["dtype"]], f"sdpa error {err}"
