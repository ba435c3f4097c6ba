"""fp64 CPU oracle for fused variable-length attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's ``cpu_baseline`` leg may import this module.  It is plain,
slow and explicit: it builds the full score matrix of every (sequence,
head) row chunk, applies the visibility mask, takes a softmax and a
weighted sum, all in float64 NumPy.  It shares no code with the HIP path
and imports nothing from it.

What is computed (the definition the fused kernels must reach, up to
rounding order):

* Packed ragged inputs: q ``[Tq, Hq, Dqk]``, k ``[Tk, Hkv, Dqk]``,
  v ``[Tk, Hkv, Dv]``; sequence ``s`` owns q rows ``cu_q[s]:cu_q[s+1]`` and
  kv rows ``cu_kv[s]:cu_kv[s+1]`` (mtlattn 0.3.0 project page, section "Use").
* GQA/MQA: query head ``h`` reads kv head ``h // (Hq // Hkv)`` (same section).
* Causal mask, end-aligned: local query ``i`` sees local key ``j`` iff
  ``j <= i + (Lk - Lq)`` (same section).
* Sliding window ``W``: query ``i`` sees only its last ``W`` keys counted
  back from that diagonal, i.e. ``i + off - W < j <= i + off``; a window is
  only defined together with the causal mask (same section: the
  Mistral-style window is causal with a window).  Reading: exactly W keys
  including the diagonal one.
* Additive bias: ``logit = scale * (q . k) + bias[global q row, h or 0,
  local key]`` (same section).
* Softmax over the visible keys whose logit is not ``-inf``; ``out`` is the
  probability-weighted sum of v.  Per-row log-sum-exp ``lse = m + ln l``
  (natural log) of the scaled, biased logits; a row with no visible key has
  ``out = 0`` and ``lse = -inf`` (the pages do not define the LSE; this is
  the plain reading).
* Default scale ``1/sqrt(Dqk)`` when ``scale`` is None.

The diagonal skip and the all-thread softmax on the triton-msl part-2 post
(section "FlashAttention: faster than PyTorch, competitive with MLX") are
described there as exact, so the oracle implements the definition and not
the tiled algorithm.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

ROW_CHUNK = 256


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """Query head h reads kv head h // (Hq / Hkv) (mtlattn page, "Use")."""
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    return h // (hq // hkv)


def visible(i: np.ndarray, j: np.ndarray, lq: int, lk: int, causal: bool, window: int) -> np.ndarray:
    """Boolean visibility of local key j for local query i (broadcasting).

    End-aligned causal: j <= i + (lk - lq).  Window W (causal only):
    j > i + (lk - lq) - W.  Keys outside [0, lk) are never visible.
    """
    off = lk - lq
    ok = (j >= 0) & (j < lk) & (i >= 0) & (i < lq)
    if causal:
        ok = ok & (j <= i + off)
    if window:
        if not causal:
            raise ValueError("a window is only defined together with the causal mask")
        ok = ok & (j > i + off - window)
    return ok


def logits(qrows: np.ndarray, kseq: np.ndarray, scale: float,
           bias_rows: Optional[np.ndarray]) -> np.ndarray:
    """z = scale * q k^T (+ bias), fp64.  qrows [n, D], kseq [Lk, D], bias_rows [n, Lk]."""
    z = scale * (qrows @ kseq.T)
    if bias_rows is not None:
        z = z + bias_rows
    return z


def bias_head(head: int, bias_heads: int) -> int:
    """Bias dim 1 of size 1 broadcasts over query heads, else it is indexed by
    the query head (mtlattn page, "Use")."""
    return 0 if bias_heads == 1 else head


def softmax_rows(z: np.ndarray, mask: np.ndarray):
    """Masked softmax of each row.

    Returns (p, m, l): p is zero where the key is masked or its logit is
    -inf; m is the row max over the unmasked logits (-inf for an empty row)
    and l the sum of exp(z - m) over them.
    """
    unmasked = mask & (z != -np.inf)
    zm = np.where(unmasked, z, -np.inf)
    m = zm.max(axis=1, initial=-np.inf)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(unmasked, np.exp(zm - safe_m[:, None]), 0.0)
    l = p.sum(axis=1)
    return p, m, l


def finish_rows(p: np.ndarray, m: np.ndarray, l: np.ndarray, vseq: np.ndarray):
    """out = (p / l) @ v and lse = m + ln l; an empty row (l == 0) gives
    out = 0 and lse = -inf.  Returns (out, lse, normalised p)."""
    nonempty = l > 0
    safe_l = np.where(nonempty, l, 1.0)
    pn = p / safe_l[:, None]
    if vseq.shape[0] > 0:
        out = pn @ vseq
    else:
        out = np.zeros((p.shape[0], vseq.shape[1]))
    out = np.where(nonempty[:, None], out, 0.0)
    lse = np.where(nonempty, np.where(np.isfinite(m), m, 0.0) + np.log(safe_l), -np.inf)
    return out, lse, pn


def attention_rows(q, k, v, cu_q, cu_kv, seq: int, head: int, rows: Sequence[int],
                   scale: Optional[float] = None, causal: bool = False, window: int = 0,
                   bias=None, return_p: bool = False):
    """Attention for the given local query rows of one (sequence, query head).

    q, k, v, bias: float64 arrays (bias may be None).  Returns
    ``(out [n, Dv], lse [n])`` and, if ``return_p``, the normalised
    probabilities ``[n, Lk]``.
    """
    hq, hkv = q.shape[1], k.shape[1]
    d_qk = q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    cq0, cq1 = int(cu_q[seq]), int(cu_q[seq + 1])
    ck0, ck1 = int(cu_kv[seq]), int(cu_kv[seq + 1])
    lq, lk = cq1 - cq0, ck1 - ck0
    g = kv_head_of(head, hq, hkv)
    rows = np.asarray(rows, dtype=np.int64)
    kseq = k[ck0:ck1, g, :]
    vseq = v[ck0:ck1, g, :]
    qrows = q[cq0 + rows, head, :]
    brows = None
    if bias is not None:
        brows = bias[cq0 + rows, bias_head(head, bias.shape[1]), :lk]
    z = logits(qrows, kseq, scale, brows)
    mask = visible(rows[:, None], np.arange(lk)[None, :], lq, lk, causal, window)
    p, m, l = softmax_rows(z, mask)
    out, lse, pn = finish_rows(p, m, l, vseq)
    if return_p:
        return out, lse, pn
    return out, lse


def varlen_attention(q, k, v, cu_q, cu_kv, scale: Optional[float] = None, causal: bool = False,
                     window: int = 0, bias=None, heads: Optional[Sequence[int]] = None,
                     seqs: Optional[Sequence[int]] = None):
    """Full varlen attention, fp64.

    Returns ``out [Tq, Hq, Dv]`` and ``lse [Hq, Tq]``; rows of sequences or
    heads not listed in ``seqs`` / ``heads`` are left at zero / NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    tq, hq = q.shape[0], q.shape[1]
    out = np.zeros((tq, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((hq, tq), np.nan, dtype=np.float64)
    nseq = len(cu_q) - 1
    for s in (range(nseq) if seqs is None else seqs):
        lq = int(cu_q[s + 1] - cu_q[s])
        for h in (range(hq) if heads is None else heads):
            for r0 in range(0, lq, ROW_CHUNK):
                rows = np.arange(r0, min(lq, r0 + ROW_CHUNK))
                o, ls = attention_rows(q, k, v, cu_q, cu_kv, s, h, rows, scale, causal,
                                       window, bias)
                out[cu_q[s] + rows, h, :] = o
                lse[h, cu_q[s] + rows] = ls
    return out, lse


def visible_counts(lq: int, lk: int, causal: bool, window: int) -> np.ndarray:
    """Number of visible keys per local query row, counted from the mask."""
    i = np.arange(lq)[:, None]
    counts = np.zeros(lq, dtype=np.int64)
    for j0 in range(0, lk, 4096):
        j = np.arange(j0, min(lk, j0 + 4096))[None, :]
        counts += visible(i, j, lq, lk, causal, window).sum(axis=1)
    return counts
