"""Seeded synthetic inputs for varlen attention.

This module only draws random tensors and builds ``cu_seqlens`` / bias
layouts.  It holds none of the attention arithmetic, so both the fp64
oracle (``oracle/``) and the HIP path (``flash_attention_varlen_amd``) can
be fed from it without sharing any code with each other.

Shapes follow the workloads the mtlattn 0.3.0 project page describes in
its "Use" section: q/k/v packed as ``[total_tokens, heads, head_dim]``,
``cu_seqlens`` int32 ``[num_seqs + 1]``, an additive fp32 bias
``[total_q, H or 1, max_kv]``.  The latent-attention head (a 128-wide
"nope" part concatenated with a 64-wide "rope" part for the query-key
contraction, 128-wide values) follows the section "Latent attention, the
2026 frontier" of the triton-msl part-2 post.

Recipe (the same for every config): a ``torch.Generator`` on the CPU seeded
with the config's seed draws, in this order, the sequence lengths (only
where they are random), q, k, v as ``torch.randn(..., dtype=float32)``;
each is then cast to the config dtype with round-to-nearest-even
(``Tensor.to``).  For the latent-attention shape the draw order is q_nope,
q_rope, k_nope, k_rope, v, and the halves are concatenated on the last dim.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens_q: tuple
    seqlens_kv: tuple
    hq: int
    hkv: int
    d_qk: int
    d_v: int
    dtype: str  # "f32" | "f16" | "bf16"
    causal: bool
    window: int = 0
    scale: Optional[float] = None  # None -> 1/sqrt(d_qk)
    bias: Optional[str] = None  # None | "prefix_lm"
    prefix: int = 0  # prefix length of the prefix-LM bias
    seed: int = 0
    nope_rope: Optional[tuple] = None  # (d_nope, d_rope) for latent attention
    description: str = ""

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens_q)

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_kv(self) -> int:
        return int(sum(self.seqlens_kv))

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.seqlens_q)) if self.seqlens_q else 0

    @property
    def max_seqlen_kv(self) -> int:
        return int(max(self.seqlens_kv)) if self.seqlens_kv else 0

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d_qk)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def cfg2_lengths() -> list:
    """Eight lengths uniform in [512, 4096], drawn first from seed 1."""
    g = torch.Generator().manual_seed(1)
    return torch.randint(512, 4097, (8,), generator=g).tolist()


# The workloads.  Names say what each is; sizes are spelled out.
TINY_F32 = Workload(
    name="tiny_f32_full_3seq_h2_d64", seqlens_q=(17, 64, 129), seqlens_kv=(17, 64, 129),
    hq=2, hkv=2, d_qk=64, d_v=64, dtype="f32", causal=False, scale=1.0 / 8.0, seed=0,
    description="fp32 varlen full attention, lengths 17/64/129, H=2, D=64")

_L2 = (1677, 2626, 1676, 2065, 630, 4080, 4078, 3373)
GQA_CAUSAL_BF16 = Workload(
    name="gqa_causal_bf16_8seq_hq32_hkv8_d128", seqlens_q=_L2, seqlens_kv=_L2,
    hq=32, hkv=8, d_qk=128, d_v=128, dtype="bf16", causal=True,
    scale=1.0 / math.sqrt(128), seed=1,
    description="bf16 causal GQA varlen prefill, 8 seqs (T=20205), Hq=32, Hkv=8, D=128")


def dense_f16(d: int, causal: bool, bias: bool = False) -> Workload:
    L = (8192,) * 4
    tag = "prefix_lm_bias" if bias else ("causal" if causal else "full")
    return Workload(
        name=f"dense_f16_b4_l8192_h16_d{d}_{tag}", seqlens_q=L, seqlens_kv=L,
        hq=16, hkv=16, d_qk=d, d_v=d, dtype="f16", causal=causal,
        scale=1.0 / math.sqrt(d), bias="prefix_lm" if bias else None, prefix=1024, seed=3,
        description=f"fp16 dense B=4 L=8192 H=16 D={d} {tag}")


def dense_bf16_head(d: int) -> Workload:
    """The head dims 96 and 256 at the dense causal shape (measurement of the
    head-dim variants)."""
    L = (8192,) * 4
    return Workload(
        name=f"dense_bf16_b4_l8192_h16_d{d}_causal", seqlens_q=L, seqlens_kv=L,
        hq=16, hkv=16, d_qk=d, d_v=d, dtype="bf16", causal=True,
        scale=1.0 / math.sqrt(d), seed=7,
        description=f"bf16 dense causal B=4 L=8192 H=16 D={d}")


SWA_BF16 = Workload(
    name="swa_causal_bf16_4x16384_hq32_hkv8_d128_w4096", seqlens_q=(16384,) * 4,
    seqlens_kv=(16384,) * 4, hq=32, hkv=8, d_qk=128, d_v=128, dtype="bf16", causal=True,
    window=4096, scale=1.0 / math.sqrt(128), seed=4,
    description="bf16 sliding-window causal, 4x16384 tokens, Hq=32, Hkv=8, D=128, W=4096")

MLA_BF16 = Workload(
    name="mla_causal_bf16_4x4096_h128_dqk192_dv128", seqlens_q=(4096,) * 4,
    seqlens_kv=(4096,) * 4, hq=128, hkv=128, d_qk=192, d_v=128, dtype="bf16", causal=True,
    scale=1.0 / math.sqrt(192), seed=5, nope_rope=(128, 64),
    description="bf16 latent-attention shape, 4x4096 tokens, H=128, Dqk=192 (128+64), Dv=128")

def decode_lengths() -> list:
    """Eight key-cache lengths uniform in [4096, 65536], drawn first from seed 6."""
    g = torch.Generator().manual_seed(6)
    return torch.randint(4096, 65537, (8,), generator=g).tolist()


DECODE_BF16 = Workload(
    name="decode_bf16_8seq_q1_hq32_hkv8_d128", seqlens_q=(1,) * 8,
    seqlens_kv=(30652, 22545, 46653, 24230, 12843, 44002, 50669, 10330), hq=32, hkv=8, d_qk=128,
    d_v=128, dtype="bf16", causal=True, scale=1.0 / math.sqrt(128), seed=6,
    description="bf16 cached decode: 8 sequences, 1 query row each, key caches of 4K-64K keys "
                "(seed 6), Hq=32, Hkv=8, D=128, causal (end-aligned)")

ALL = {
    "tiny_f32": TINY_F32,
    "gqa_causal_bf16": GQA_CAUSAL_BF16,
    "dense_f16_d128_full": dense_f16(128, False),
    "dense_f16_d128_causal": dense_f16(128, True),
    "dense_f16_d128_prefix_lm": dense_f16(128, False, bias=True),
    "dense_f16_d64_full": dense_f16(64, False),
    "dense_f16_d64_causal": dense_f16(64, True),
    "dense_f16_d64_prefix_lm": dense_f16(64, False, bias=True),
    "dense_bf16_d96_causal": dense_bf16_head(96),
    "dense_bf16_d256_causal": dense_bf16_head(256),
    "swa_bf16": SWA_BF16,
    "mla_bf16": MLA_BF16,
    "decode_bf16": DECODE_BF16,
}


def cu_seqlens(lengths: Sequence[int]) -> torch.Tensor:
    """int32 cumulative lengths, leading zero."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def prefix_lm_bias(seqlens: Sequence[int], prefix: int, cols: Optional[int] = None) -> torch.Tensor:
    """Additive fp32 bias [total_q, 1, cols]: 0 where key j < prefix or j <= i, else -inf.

    i and j are positions inside each sequence (self-attention, Lq == Lk).
    Columns at or beyond a sequence's own length are left at 0 (never read).
    """
    cols = cols if cols is not None else max(seqlens)
    rows = []
    for n in seqlens:
        i = torch.arange(n).view(n, 1)
        j = torch.arange(cols).view(1, cols)
        ok = (j < prefix) | (j <= i)
        b = torch.zeros(n, cols, dtype=torch.float32)
        b.masked_fill_(~ok, float("-inf"))
        rows.append(b)
    return torch.cat(rows, 0).view(-1, 1, cols)


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_kv: torch.Tensor
    bias: Optional[torch.Tensor]
    workload: Workload


def make_inputs(w: Workload) -> Inputs:
    """Draw q, k, v (and the bias) for a workload on the CPU, seeded."""
    g = torch.Generator().manual_seed(w.seed)
    dt = DTYPES[w.dtype]
    tq, tk = w.total_q, w.total_kv
    if w.nope_rope is not None:
        dn, dr = w.nope_rope
        assert dn + dr == w.d_qk
        qn = torch.randn(tq, w.hq, dn, generator=g, dtype=torch.float32)
        qr = torch.randn(tq, w.hq, dr, generator=g, dtype=torch.float32)
        kn = torch.randn(tk, w.hkv, dn, generator=g, dtype=torch.float32)
        kr = torch.randn(tk, w.hkv, dr, generator=g, dtype=torch.float32)
        q = torch.cat([qn, qr], -1).to(dt)
        k = torch.cat([kn, kr], -1).to(dt)
        del qn, qr, kn, kr
    else:
        q = torch.randn(tq, w.hq, w.d_qk, generator=g, dtype=torch.float32).to(dt)
        k = torch.randn(tk, w.hkv, w.d_qk, generator=g, dtype=torch.float32).to(dt)
    v = torch.randn(tk, w.hkv, w.d_v, generator=g, dtype=torch.float32).to(dt)
    bias = None
    if w.bias == "prefix_lm":
        bias = prefix_lm_bias(w.seqlens_q, w.prefix, w.max_seqlen_kv)
    elif w.bias is not None:
        raise ValueError(f"unknown bias kind {w.bias!r}")
    return Inputs(q=q, k=k, v=v, cu_seqlens_q=cu_seqlens(w.seqlens_q),
                  cu_seqlens_kv=cu_seqlens(w.seqlens_kv), bias=bias, workload=w)


def random_lengths(n: int, lo: int, hi: int, seed: int) -> list:
    """n lengths uniform in [lo, hi] from their own generator (small test cases)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


def random_bias(seqlens_q: Sequence[int], heads: int, cols: int, seed: int,
                neg_inf_frac: float = 0.1) -> torch.Tensor:
    """fp32 bias [total_q, heads, cols] with N(0,1) values and a fraction of -inf entries."""
    g = torch.Generator().manual_seed(seed)
    tq = int(sum(seqlens_q))
    b = torch.randn(tq, heads, cols, generator=g, dtype=torch.float32)
    u = torch.rand(tq, heads, cols, generator=g)
    b.masked_fill_(u < neg_inf_frac, float("-inf"))
    return b
