"""fp64 / integer CPU oracle for the mask front-ends.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only the tests, the
smoke check and the benchmark's ``cpu_baseline`` leg may import it.  It
shares no code with the HIP path.

* ``bias_key_ranges``: for each bias row, the first and one-past-last key of
  its sequence whose additive bias is not -inf.  A key with a -inf bias has
  logit -inf and contributes exactly nothing to the softmax (mtlattn 0.3.0
  project page, section "Use": the bias composes with the masks), so the
  kernels may skip every key outside these ranges; the triton-msl part-2
  post (section "FlashAttention: faster than PyTorch, competitive with MLX")
  makes the same point for tiles that are masked in full.
* ``bias_rows_are_intervals``: for each bias row, whether it is a plain key
  interval: bias exactly 0 on every key of its range and -inf on every
  other key.  Such a row's bias adds nothing inside the range and removes
  every key outside it, so attending over the range alone gives the same
  result (the same "Use" section: a bool mask is such a 0 / -inf bias).
* ``alibi_bias``: the ALiBi bias written out as a dense additive bias.  The
  mtlattn 0.3.0 page (section "Use") names ALiBi as one of the patterns the
  additive bias carries but gives no formula; the reading taken is the
  linear distance penalty, minus the head's slope times the distance
  between the query's end-aligned position and the key.
"""
from __future__ import annotations

import numpy as np


def bias_key_ranges(bias, cu_q, cu_kv):
    """int64 ``[H_b, Tq, 2]``: ``[lo, hi)`` with lo the first and hi - 1 the
    last key ``j < min(Lk, cols)`` of the row's sequence whose bias is not
    -inf; ``[0, 0)`` when every such key is -inf."""
    bias = np.asarray(bias)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    tq, hb, cols = bias.shape
    out = np.zeros((hb, tq, 2), dtype=np.int64)
    for s in range(len(cu_q) - 1):
        lk = min(int(cu_kv[s + 1] - cu_kv[s]), cols)
        for t in range(int(cu_q[s]), int(cu_q[s + 1])):
            for h in range(hb):
                keys = np.nonzero(bias[t, h, :lk] != -np.inf)[0]
                if keys.size:
                    out[h, t] = (keys[0], keys[-1] + 1)
    return out


def bias_rows_are_intervals(bias, cu_q, cu_kv):
    """uint8 ``[H_b, Tq]``: 1 when, over the keys ``j < min(Lk, cols)`` of the
    row's sequence, the bias is exactly 0 on every key of ``[lo, hi)`` (the
    row's ``bias_key_ranges``) and -inf on every other key; 0 otherwise.  A
    row that is -inf everywhere is the empty interval (1)."""
    bias = np.asarray(bias)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    tq, hb, cols = bias.shape
    rg = bias_key_ranges(bias, cu_q, cu_kv)
    out = np.zeros((hb, tq), dtype=np.uint8)
    for s in range(len(cu_q) - 1):
        lk = min(int(cu_kv[s + 1] - cu_kv[s]), cols)
        for t in range(int(cu_q[s]), int(cu_q[s + 1])):
            for h in range(hb):
                lo, hi = (int(x) for x in rg[h, t])
                row = bias[t, h, :lk]
                inside = row[lo:hi]
                outside = np.concatenate([row[:lo], row[hi:]])
                out[h, t] = bool(np.all(inside == 0.0) and np.all(outside == -np.inf))
    return out


def alibi_bias(slopes, cu_q, cu_kv, hq, cols):
    """fp64 ``[Tq, hq, cols]``: ``-slope[s, h] * |i + (Lk - Lq) - j|`` for
    query row i and key j < Lk of sequence s (0 past Lk, where no key is).
    ``slopes`` is ``[hq]`` (every sequence) or ``[num_seqs, hq]``."""
    slopes = np.asarray(slopes, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    out = np.zeros((int(cu_q[-1]), hq, cols), dtype=np.float64)
    for s in range(len(cu_q) - 1):
        lq = int(cu_q[s + 1] - cu_q[s])
        lk = int(cu_kv[s + 1] - cu_kv[s])
        sl = slopes if slopes.ndim == 1 else slopes[s]
        for i in range(lq):
            pos = i + lk - lq
            for h in range(hq):
                for j in range(min(lk, cols)):
                    out[int(cu_q[s]) + i, h, j] = -sl[h] * abs(pos - j)
    return out
