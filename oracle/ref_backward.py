"""fp64 CPU oracle for the gradients of varlen attention.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only the tests, the
smoke check and the benchmark's ``cpu_baseline`` leg may import it.  It
shares no code with the HIP path.

The forward is out = softmax(z) v per row, with z the scaled (and masked)
logits of the rows' visible keys (``ref_attention``).  Given the gradient
dout of a loss with respect to out, the chain rule through that definition
gives, per (sequence, query head h, kv head g = h // (Hq / Hkv)):

    dv_j  += sum_i p_ij dout_i                     (out_i = sum_j p_ij v_j)
    dp_ij  = dout_i . v_j
    D_i    = sum_j p_ij dp_ij  (= dout_i . out_i)
    dz_ij  = p_ij (dp_ij - D_i)                    (softmax Jacobian)
    dq_i   = scale sum_j dz_ij k_j                 (z_ij = scale q_i . k_j + bias)
    dk_j  += scale sum_i dz_ij q_i

summing dk and dv over the query heads that share a kv head (GQA).  Masked
keys and keys with a -inf bias have p = 0 and get nothing from that row; a
row with no visible key has out = 0 and contributes nothing.  The LSE output
is treated as not differentiated.  This is the backward that the triton-msl
part-2 post (section "Beyond softmax: linear attention and a trainable
backward") and the mtlattn 0.3.0 project page (sections "Drop-in for
scaled_dot_product_attention" and "Performance") describe for their tiled
FlashAttention-2 backward; the oracle computes it from explicit fp64
matrices, not tiles.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .ref_attention import bias_head, kv_head_of, logits, softmax_rows, visible


def varlen_attention_backward(q, k, v, dout, cu_q, cu_kv, scale: Optional[float] = None,
                              causal: bool = False, window: int = 0, bias=None,
                              seqs: Optional[Sequence[int]] = None,
                              kv_heads: Optional[Sequence[int]] = None):
    """Returns ``(dq, dk, dv)`` in fp64 with the shapes of q, k, v.

    With ``seqs`` / ``kv_heads`` only those sequences and kv heads (with all
    their query heads) are computed; the other entries stay zero."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s in (range(len(cu_q) - 1) if seqs is None else seqs):
        cq0, cq1 = int(cu_q[s]), int(cu_q[s + 1])
        ck0, ck1 = int(cu_kv[s]), int(cu_kv[s + 1])
        lq, lk = cq1 - cq0, ck1 - ck0
        if lq == 0 or lk == 0:
            continue
        i = np.arange(lq)[:, None]
        j = np.arange(lk)[None, :]
        mask = visible(i, j, lq, lk, causal, window)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            if kv_heads is not None and g not in kv_heads:
                continue
            qs, ks, vs = q[cq0:cq1, h], k[ck0:ck1, g], v[ck0:ck1, g]
            brows = None
            if bias is not None:
                brows = bias[cq0:cq1, bias_head(h, bias.shape[1]), :lk]
            z = logits(qs, ks, scale, brows)
            p, m, l = softmax_rows(z, mask)
            nonempty = l > 0
            p = np.where(nonempty[:, None], p / np.where(nonempty, l, 1.0)[:, None], 0.0)
            do = dout[cq0:cq1, h]
            dp = do @ vs.T
            delta = (p * dp).sum(axis=1)
            dz = p * (dp - delta[:, None])
            dq[cq0:cq1, h] += scale * (dz @ ks)
            dk[ck0:ck1, g] += scale * (dz.T @ qs)
            dv[ck0:ck1, g] += p.T @ do
    return dq, dk, dv
