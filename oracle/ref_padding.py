"""fp64 / integer CPU oracle for the key-padding front end.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only the tests, the
smoke check and the benchmark's ``cpu_baseline`` leg may import it.  It
shares no code with the HIP path.

The mtlattn 0.3.0 project page (section "Drop-in for
scaled_dot_product_attention") serves a self-attention key-padding mask by
packing the valid tokens into varlen form, so that padding is skipped rather
than masked.  Written out:

* ``padding_to_varlen``: the rank of every token among its row's valid
  tokens (-1 at padding), the cumulative valid counts and (total, longest).
* ``pack_tokens`` / ``unpack_tokens``: the gather into packed rows and the
  scatter back, zeros at padding.
* ``padding_lengths``: each row's valid count and whether the batch is
  right-padded (every row's valid tokens come first), the case in which the
  padded tensors can be attended in place: a sequence is then its row's
  first ``count`` tokens.
* ``used_prefixes``: the packed varlen problem that spans with a used prefix
  each (``seqused``) stand for: sequence s is the first ``used[s]`` rows of
  its span.
* ``masked_attention``: the dense definition the packed path must reproduce,
  scaled dot-product attention over ``[B, H, N, D]`` in which a key takes
  part only where the mask marks it valid (and, with ``causal``, only keys at
  or before the query's position).  Padded query rows are never computed by
  the packed path; here they are defined as 0, as are rows that see no key.
"""
from __future__ import annotations

import numpy as np


def padding_to_varlen(mask):
    """``mask`` bool ``[B, N]`` -> (ranks int64 ``[B, N]``, cu int64 ``[B+1]``,
    (total, longest))."""
    mask = np.asarray(mask, dtype=bool)
    b, n = mask.shape
    ranks = np.full((b, n), -1, dtype=np.int64)
    counts = np.zeros(b, dtype=np.int64)
    for r in range(b):
        c = 0
        for t in range(n):
            if mask[r, t]:
                ranks[r, t] = c
                c += 1
        counts[r] = c
    cu = np.zeros(b + 1, dtype=np.int64)
    cu[1:] = np.cumsum(counts)
    return ranks, cu, (int(cu[-1]), int(counts.max(initial=0)))


def padding_lengths(mask):
    """``mask`` bool ``[B, N]`` -> (counts int64 ``[B]``, spans int64 ``[B+1]``
    = ``b * N``, right_padded, longest): right_padded is True when every row's
    valid tokens are exactly its first ``counts[b]`` positions."""
    mask = np.asarray(mask, dtype=bool)
    b, n = mask.shape
    counts = mask.sum(axis=1).astype(np.int64)
    right = all(bool(mask[r, :counts[r]].all()) for r in range(b))
    spans = np.arange(b + 1, dtype=np.int64) * n
    return counts, spans, right, int(counts.max(initial=0))


def used_prefixes(x, cu, used):
    """Rows ``[total, ...]`` grouped in spans ``cu`` -> (the first ``used[s]``
    rows of every span, packed, and their cumulative counts).  ``used`` is
    clamped to ``[0, span]``."""
    x = np.asarray(x)
    cu = np.asarray(cu, dtype=np.int64)
    parts, counts = [], []
    for s in range(len(cu) - 1):
        span = int(cu[s + 1] - cu[s])
        u = min(max(int(used[s]), 0), span)
        parts.append(x[int(cu[s]):int(cu[s]) + u])
        counts.append(u)
    out_cu = np.zeros(len(counts) + 1, dtype=np.int64)
    out_cu[1:] = np.cumsum(counts)
    packed = np.concatenate(parts) if parts else x[:0]
    return packed, out_cu


def pack_tokens(padded, mask):
    """``padded`` ``[B, N, H, D]`` -> packed ``[total, H, D]``: the valid
    tokens row by row, in order."""
    padded = np.asarray(padded)
    mask = np.asarray(mask, dtype=bool)
    rows = [padded[b, t] for b in range(mask.shape[0]) for t in range(mask.shape[1]) if mask[b, t]]
    if not rows:
        return np.zeros((0,) + padded.shape[2:], dtype=padded.dtype)
    return np.stack(rows)


def unpack_tokens(packed, mask):
    """packed ``[total, H, D]`` -> ``[B, N, H, D]`` with zeros at padding."""
    packed = np.asarray(packed)
    mask = np.asarray(mask, dtype=bool)
    out = np.zeros(mask.shape + packed.shape[1:], dtype=packed.dtype)
    i = 0
    for b in range(mask.shape[0]):
        for t in range(mask.shape[1]):
            if mask[b, t]:
                out[b, t] = packed[i]
                i += 1
    return out


def masked_attention(q, k, v, mask, scale, causal):
    """Dense fp64 attention, ``q`` ``[B, Hq, N, D]``, ``k``/``v``
    ``[B, Hkv, N, D*]`` (query head h reads kv head h // (Hq / Hkv)), key
    validity ``mask`` ``[B, N]``.  Returns ``[B, Hq, N, Dv]``; padded query
    rows and rows with no visible key are 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    bsz, hq, n, _ = q.shape
    hkv = k.shape[1]
    out = np.zeros((bsz, hq, n, v.shape[3]), dtype=np.float64)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    for b in range(bsz):
        for h in range(hq):
            g = h // (hq // hkv)
            z = scale * (q[b, h] @ k[b, g].T)
            vis = np.broadcast_to(mask[b][None, :], (n, n))
            if causal:
                vis = vis & (j <= i)
            z = np.where(vis, z, -np.inf)
            m = z.max(axis=1, keepdims=True)
            seen = np.isfinite(m[:, 0]) & mask[b]
            p = np.where(vis, np.exp(z - np.where(np.isfinite(m), m, 0.0)), 0.0)
            l = p.sum(axis=1, keepdims=True)
            o = (p / np.where(l > 0, l, 1.0)) @ v[b, g]
            out[b, h] = np.where(seen[:, None], o, 0.0)
    return out
