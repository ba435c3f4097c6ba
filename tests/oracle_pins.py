"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees
with an independent statement of what attention must return: a pure-Python
brute force written straight from the definitions, PyTorch's own
``scaled_dot_product_attention`` on the cases where it computes the same
thing, hand-derived closed forms, and invariants of softmax attention.
``test_oracle_pins.py`` runs them; ``test_oracle_mutations.py`` plants
plausible mistakes in the oracle and checks that some pin catches each.

Definitions follow the mtlattn 0.3.0 project page, section "Use" (packed
layout, cu_seqlens, end-aligned causal rule, last-W-keys window, GQA head
map, additive bias).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import ref_attention as ra

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


# ---------------------------------------------------------------- helpers
def _tiny_case(rng, nseq, max_len, hq, hkv, dqk, dv, cross=False, bias_heads=0, neg_inf=0.0):
    lq = rng.integers(0, max_len + 1, size=nseq)
    lk = rng.integers(0, max_len + 1, size=nseq) if cross else lq.copy()
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_kv = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = rng.standard_normal((int(cu_q[-1]), hq, dqk))
    k = rng.standard_normal((int(cu_kv[-1]), hkv, dqk))
    v = rng.standard_normal((int(cu_kv[-1]), hkv, dv))
    bias = None
    if bias_heads:
        cols = int(max(lk.max(initial=0), 1))
        bias = rng.standard_normal((int(cu_q[-1]), bias_heads, cols))
        bias[rng.random(bias.shape) < neg_inf] = -np.inf
    return q, k, v, cu_q, cu_kv, bias


def brute_force(q, k, v, cu_q, cu_kv, scale, causal, window, bias):
    """Scalar loops over (sequence, head, query, key, dim) with math.exp and
    math.fsum, written from the definitions without any oracle helper."""
    tq, hq, dqk = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    out = np.zeros((tq, hq, dv))
    lse = np.full((hq, tq), -math.inf)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[s]), int(cu_q[s + 1]), int(cu_kv[s]), int(cu_kv[s + 1])
        lq, lk = q1 - q0, k1 - k0
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(lq):
                zs = []
                for j in range(lk):
                    if causal and not (j <= i + lk - lq):
                        continue
                    if window and not (j > i + lk - lq - window):
                        continue
                    z = scale * math.fsum(float(q[q0 + i, h, d]) * float(k[k0 + j, g, d])
                                          for d in range(dqk))
                    if bias is not None:
                        z += float(bias[q0 + i, 0 if bias.shape[1] == 1 else h, j])
                    if z == -math.inf:
                        continue
                    zs.append((j, z))
                if not zs:
                    continue
                m = max(z for _, z in zs)
                w = [(j, math.exp(z - m)) for j, z in zs]
                l = math.fsum(x for _, x in w)
                for d in range(dv):
                    out[q0 + i, h, d] = math.fsum(x * float(v[k0 + j, g, d]) for j, x in w) / l
                lse[h, q0 + i] = m + math.log(l)
    return out, lse


def _close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    same_inf = (a == b)
    fin = np.isfinite(a) & np.isfinite(b)
    assert np.all(same_inf | fin), "non-finite mismatch"
    diff = np.subtract(a, b, out=np.zeros_like(a), where=fin)
    err = np.max(np.abs(diff), initial=0.0)
    assert err <= tol, f"max abs err {err} > {tol}"


# ---------------------------------------------------------------- pins
def pin_brute_force_tiny():
    """All flag combinations on tiny ragged inputs vs scalar brute force."""
    rng = np.random.default_rng(1234)
    combos = itertools.product([False, True], [0, 1, 3], [0, 1, 2], [False, True])
    for causal, window, bias_mode, cross in combos:
        if window and not causal:
            continue
        hq, hkv = (4, 2) if bias_mode != 1 else (4, 1)
        q, k, v, cu_q, cu_kv, bias = _tiny_case(
            rng, 3, 6, hq, hkv, 5, 3, cross=cross,
            bias_heads={0: 0, 1: 1, 2: hq}[bias_mode], neg_inf=0.2)
        scale = 0.37
        o1, l1 = oracle.varlen_attention(q, k, v, cu_q, cu_kv, scale, causal, window, bias)
        o2, l2 = brute_force(q, k, v, cu_q, cu_kv, scale, causal, window, bias)
        _close(o1, o2, 1e-12)
        _close(l1, l2, 1e-12)


def pin_sdpa_special_case():
    """Lq == Lk per sequence: torch's float64 CPU SDPA computes the same thing
    (its top-left causal diagonal equals the end-aligned one when Lq == Lk)."""
    import torch.nn.functional as F
    rng = np.random.default_rng(99)
    for causal, window, with_bias, (hq, hkv) in itertools.product(
            [False, True], [0, 4], [False, True], [(4, 4), (6, 2), (3, 1)]):
        if window and not causal:
            continue
        lens = [7, 1, 19, 12]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T, D = int(cu[-1]), 16
        q = rng.standard_normal((T, hq, D))
        k = rng.standard_normal((T, hkv, D))
        v = rng.standard_normal((T, hkv, 8))
        bias = rng.standard_normal((T, hq, max(lens))) if with_bias else None
        out, lse = oracle.varlen_attention(q, k, v, cu, cu, None, causal, window, bias)
        for s, L in enumerate(lens):
            sl = slice(int(cu[s]), int(cu[s + 1]))
            tq = torch.from_numpy(q[sl]).permute(1, 0, 2)[None]
            tk = torch.from_numpy(k[sl]).permute(1, 0, 2)[None]
            tv = torch.from_numpy(v[sl]).permute(1, 0, 2)[None]
            mask = None
            use_is_causal = causal and not window and not with_bias
            if causal and not use_is_causal:
                ones = torch.ones(L, L, dtype=torch.bool)
                band = torch.tril(ones)
                if window:
                    band = band & torch.triu(ones, diagonal=-(window - 1))
                mask = torch.zeros(L, L, dtype=torch.float64).masked_fill(~band, -math.inf)
            if with_bias:
                b = torch.from_numpy(bias[sl, :, :L]).permute(1, 0, 2)[None]
                mask = b if mask is None else mask + b
            ref = F.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=mask, is_causal=use_is_causal, enable_gqa=hq != hkv)
            _close(out[sl], ref[0].permute(1, 0, 2).numpy(), 1e-12)
            # lse against scipy's logsumexp over the explicit scores
            from scipy.special import logsumexp
            rep = hq // hkv
            for h in range(hq):
                z = (q[sl, h, :] @ k[sl, h // rep, :].T) / math.sqrt(D)
                if with_bias:
                    z = z + bias[sl, h, :L]
                i = np.arange(L)[:, None]
                j = np.arange(L)[None, :]
                if causal:
                    z = np.where(j <= i, z, -np.inf)
                if window:
                    z = np.where(j > i - window, z, -np.inf)
                _close(lse[h, sl], logsumexp(z, axis=1), 1e-12)


def pin_rows_sum_to_one():
    rng = np.random.default_rng(5)
    q, k, v, cu_q, cu_kv, bias = _tiny_case(rng, 4, 40, 2, 2, 8, 4, cross=True, bias_heads=2,
                                            neg_inf=0.3)
    for causal, window in [(False, 0), (True, 0), (True, 5)]:
        for s in range(4):
            lq = int(cu_q[s + 1] - cu_q[s])
            if lq == 0:
                continue
            _, lse, p = oracle.attention_rows(q, k, v, cu_q, cu_kv, s, 1, np.arange(lq), 0.3,
                                              causal, window, bias, return_p=True)
            sums = p.sum(axis=1)
            nonempty = np.isfinite(lse)
            assert np.all(np.abs(sums[nonempty] - 1.0) <= 1e-12)
            assert np.all(sums[~nonempty] == 0.0)
            assert np.all(p >= 0.0)


def pin_one_key_sequence():
    """A sequence with a single key returns that key's v exactly, lse = its logit."""
    rng = np.random.default_rng(6)
    q = rng.standard_normal((5, 2, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 3))
    cu_q, cu_kv = np.array([0, 5]), np.array([0, 1])
    out, lse = oracle.varlen_attention(q, k, v, cu_q, cu_kv, 0.25, False, 0, None)
    for h in range(2):
        assert np.array_equal(out[:, h, :], np.broadcast_to(v[0, h], (5, 3)))
        z = 0.25 * (q[:, h, :] @ k[0, h, :])
        _close(lse[h], z, 1e-14)


def pin_zero_queries_mean():
    """q = 0: every visible key has logit 0, so out is the mean of the visible
    v rows and lse = ln(count); the visible range is the closed form
    [max(0, i+off-W+1), min(i+off, Lk-1)]."""
    rng = np.random.default_rng(7)
    for causal, window, (lq, lk) in itertools.product(
            [False, True], [0, 3, 10], [(9, 9), (4, 11), (11, 4), (1, 1)]):
        if window and not causal:
            continue
        q = np.zeros((lq, 2, 4))
        k = rng.standard_normal((lk, 1, 4))
        v = rng.standard_normal((lk, 1, 5))
        out, lse = oracle.varlen_attention(q, k, v, np.array([0, lq]), np.array([0, lk]), None,
                                           causal, window, None)
        off = lk - lq
        for i in range(lq):
            hi = min(i + off, lk - 1) if causal else lk - 1
            lo = max(0, i + off - window + 1) if window else 0
            n = hi - lo + 1
            for h in range(2):
                if n <= 0:
                    assert np.all(out[i, h] == 0.0) and lse[h, i] == -np.inf
                else:
                    _close(out[i, h], v[lo:hi + 1, 0].mean(axis=0), 1e-14)
                    _close(lse[h, i], math.log(n), 1e-14)


def pin_key_permutation_invariance():
    rng = np.random.default_rng(8)
    q, k, v, cu_q, cu_kv, bias = _tiny_case(rng, 3, 30, 4, 2, 8, 6, cross=True)
    out, lse = oracle.varlen_attention(q, k, v, cu_q, cu_kv, None, False, 0, None)
    perm = np.arange(k.shape[0])
    for s in range(3):
        a, b = int(cu_kv[s]), int(cu_kv[s + 1])
        perm[a:b] = a + rng.permutation(b - a)
    out2, lse2 = oracle.varlen_attention(q, k[perm], v[perm], cu_q, cu_kv, None, False, 0, None)
    _close(out, out2, 1e-12)
    _close(lse, lse2, 1e-12)


def pin_neg_inf_key_is_removed():
    """A key whose bias is -inf gets probability exactly 0, and the result
    equals the result with that key deleted from the sequence."""
    rng = np.random.default_rng(9)
    L, D = 13, 8
    q = rng.standard_normal((L, 2, D))
    k = rng.standard_normal((L, 2, D))
    v = rng.standard_normal((L, 2, 4))
    bias = np.zeros((L, 1, L))
    j = 5
    bias[:, :, j] = -np.inf
    cu = np.array([0, L])
    out, lse, p = oracle.attention_rows(q, k, v, cu, cu, 0, 1, np.arange(L), None, False, 0, bias,
                                        return_p=True)
    assert np.all(p[:, j] == 0.0)
    keep = np.array([x for x in range(L) if x != j])
    out2, lse2 = oracle.attention_rows(q, k[keep], v[keep], cu, np.array([0, L - 1]), 0, 1,
                                       np.arange(L), None, False, 0, None)
    _close(out, out2, 1e-15)
    _close(lse, lse2, 1e-14)


def pin_mask_counts_closed_form():
    """Visible keys per row against closed forms, and the per-(sequence, head)
    totals of the long workloads."""
    for lq, lk in [(50, 50), (30, 70), (70, 30), (1, 9), (9, 1)]:
        off = lk - lq
        i = np.arange(lq)
        c = oracle.visible_counts(lq, lk, True, 0)
        assert np.array_equal(c, np.clip(i + off + 1, 0, lk))
        for W in (1, 4, 33):
            c = oracle.visible_counts(lq, lk, True, W)
            hi = np.clip(i + off + 1, 0, lk)
            lo = np.clip(i + off - W + 1, 0, lk)
            assert np.array_equal(c, np.maximum(hi - lo, 0))
        assert np.array_equal(oracle.visible_counts(lq, lk, False, 0), np.full(lq, lk))
    # causal total L(L+1)/2 and the 16384-token window-4096 total
    assert oracle.visible_counts(4080, 4080, True, 0).sum() == 4080 * 4081 // 2
    assert oracle.visible_counts(16384, 16384, True, 4096).sum() == 58_722_304
    # prefix-LM bias (keys < 1024 or j <= i) leaves max(1024, i+1) finite keys
    import workloads
    b = workloads.prefix_lm_bias([8192], 1024)[:, 0, :]
    finite = torch.isfinite(b).sum(dim=1).numpy()
    assert np.array_equal(finite, np.maximum(1024, np.arange(8192) + 1))
    assert finite.sum() == 34_082_304


def pin_golden_hand_worked():
    """Hand-derived tiny cases stored under tests/golden."""
    env = {"log": math.log, "exp": math.exp, "inf": math.inf}

    def ev(x):
        if isinstance(x, str):
            return float(eval(x.replace("-inf", "(-inf)"), {"__builtins__": {}}, env))
        return float(x)

    data = json.load(open(GOLDEN))
    for case in data["cases"]:
        arr = lambda key: np.vectorize(ev, otypes=[np.float64])(np.array(case[key], dtype=object))
        q, k, v = arr("q"), arr("k"), arr("v")
        bias = arr("bias") if "bias" in case else None
        out, lse = oracle.varlen_attention(q, k, v, np.array(case["cu_q"]), np.array(case["cu_kv"]),
                                           case["scale"], case["causal"], case["window"], bias)
        _close(out, arr("out"), 1e-14)
        _close(lse, arr("lse"), 1e-14)


def pin_row_subset_matches_full():
    """Sampled rows (used for full-size parity) equal the same rows of a full run."""
    rng = np.random.default_rng(10)
    q, k, v, cu_q, cu_kv, bias = _tiny_case(rng, 2, 300, 2, 1, 8, 4, cross=True, bias_heads=1,
                                            neg_inf=0.1)
    out, lse = oracle.varlen_attention(q, k, v, cu_q, cu_kv, None, True, 17, bias)
    for s in range(2):
        lq = int(cu_q[s + 1] - cu_q[s])
        rows = rng.choice(lq, size=min(lq, 11), replace=False) if lq else np.array([], int)
        o, l = oracle.attention_rows(q, k, v, cu_q, cu_kv, s, 1, rows, None, True, 17, bias)
        _close(o, out[cu_q[s] + rows, 1], 0.0)
        _close(l, lse[1, cu_q[s] + rows], 0.0)


def pin_bias_ranges_prefix_lm_closed_form():
    """Prefix-LM bias (0 where j < P or j <= i, else -inf; self-attention):
    row i's range is [0, min(L, max(P, i + 1))), by hand."""
    lens, prefix, cols = [7, 1, 12, 3], 4, 14
    rows = []
    for n in lens:
        i = np.arange(n)[:, None]
        j = np.arange(cols)[None, :]
        rows.append(np.where((j < prefix) | (j <= i), 0.0, -np.inf))
    bias = np.concatenate(rows)[:, None, :]
    cu = np.concatenate([[0], np.cumsum(lens)])
    got = oracle.bias_key_ranges(bias, cu, cu)
    for s, n in enumerate(lens):
        for i in range(n):
            assert tuple(got[0, cu[s] + i]) == (0, min(n, max(prefix, i + 1))), (s, i)


def pin_bias_ranges_skip_is_exact():
    """Attention with every key outside a row's range deleted from its
    sequence equals attention over all keys (the skip is exact); keys at the
    range ends are finite; empty ranges are exactly the all -inf rows."""
    rng = np.random.default_rng(12)
    q, k, v, cu_q, cu_kv, bias = _tiny_case(rng, 3, 40, 2, 1, 8, 4, cross=True, bias_heads=2,
                                            neg_inf=0.6)
    bias[3] = -np.inf  # a row that sees nothing
    rg = oracle.bias_key_ranges(bias, cu_q, cu_kv)
    out, lse = oracle.varlen_attention(q, k, v, cu_q, cu_kv, None, False, 0, bias)
    for s in range(len(cu_q) - 1):
        lk = int(cu_kv[s + 1] - cu_kv[s])
        for t in range(int(cu_q[s]), int(cu_q[s + 1])):
            for h in range(bias.shape[1]):
                lo, hi = rg[h, t]
                row = bias[t, h, :lk]
                if hi == 0:
                    assert np.all(row == -np.inf) and lo == 0
                    continue
                assert row[lo] != -np.inf and row[hi - 1] != -np.inf
                assert np.all(row[:lo] == -np.inf) and np.all(row[hi:] == -np.inf)
                # the row restricted to [lo, hi)
                sub_k = k[cu_kv[s] + lo:cu_kv[s] + hi]
                sub_v = v[cu_kv[s] + lo:cu_kv[s] + hi]
                sub_b = bias[t:t + 1, :, lo:hi]
                o, l = oracle.attention_rows(q[t:t + 1], sub_k, sub_v, np.array([0, 1]),
                                             np.array([0, hi - lo]), 0, h, [0], None, False, 0,
                                             sub_b)
                _close(o[0], out[t, h], 1e-13)
                _close(l[0], lse[h, t], 1e-13)


# ---------------------------------------------------------------- backward pins
def _loss_and_grads(q, k, v, cu_q, cu_kv, scale, causal, window, bias, G):
    out, _ = oracle.varlen_attention(q, k, v, cu_q, cu_kv, scale, causal, window, bias)
    return float((out * G).sum()), oracle.varlen_attention_backward(q, k, v, G, cu_q, cu_kv, scale,
                                                                     causal, window, bias)


def pin_interval_rows_hand_worked():
    """Interval rows by hand: 0 on a contiguous run and -inf elsewhere is an
    interval; a -inf hole inside the run, any nonzero finite value or a NaN
    is not; an all -inf row is the empty interval; -0.0 counts as 0; keys at
    or past the sequence's Lk are not looked at."""
    ninf, nan = -np.inf, np.nan
    rows = [
        ([0, 0, 0, 0, 0], 1),
        ([ninf, 0, 0, ninf, ninf], 1),
        ([0, ninf, 0, ninf, ninf], 0),      # hole
        ([ninf, 0, 0.5, 0, ninf], 0),       # a nonzero value
        ([ninf, -1.0, 0, ninf, ninf], 0),   # a negative value
        ([0, 0, 0.5, ninf, ninf], 0),       # nonzero at the range's last key
        ([ninf] * 5, 1),                    # empty
        ([-0.0, 0, ninf, ninf, ninf], 1),   # negative zero
        ([0, nan, ninf, ninf, ninf], 0),    # NaN
        ([ninf, ninf, ninf, ninf, 0], 1),
        ([0, 0, 0, ninf, 2.0], 1),          # the last key is past Lk = 4
    ]
    bias = np.array([r for r, _ in rows], dtype=np.float64)[:, None, :]
    cu_q = np.arange(len(rows) + 1)
    cu_kv = np.array([0] + [5] * (len(rows) - 1) + [4]).cumsum()
    got = oracle.bias_rows_are_intervals(bias, cu_q, cu_kv)
    assert got.shape == (1, len(rows))
    assert list(got[0]) == [want for _, want in rows], list(got[0])


def pin_interval_rows_attend_their_range():
    """On an interval row, attention with the bias equals attention with no
    bias over the row's key range alone (the bias-free definition applied to
    the sub-sequence)."""
    rng = np.random.default_rng(21)
    lens, d = [9, 14], 8
    cu = np.concatenate([[0], np.cumsum(lens)])
    tq = int(cu[-1])
    q = rng.standard_normal((tq, 1, d))
    k = rng.standard_normal((tq, 1, d))
    v = rng.standard_normal((tq, 1, d))
    bias = np.full((tq, 1, max(lens)), -np.inf)
    for s, n in enumerate(lens):
        for i in range(n):
            lo = int(rng.integers(0, n))
            hi = int(rng.integers(lo + 1, n + 1))
            bias[cu[s] + i, 0, lo:hi] = 0.0
    assert np.all(oracle.bias_rows_are_intervals(bias, cu, cu) == 1)
    rg = oracle.bias_key_ranges(bias, cu, cu)
    out, _ = oracle.varlen_attention(q, k, v, cu, cu, None, False, 0, bias)
    for s, n in enumerate(lens):
        for i in range(n):
            t = cu[s] + i
            lo, hi = rg[0, t]
            kk = k[cu[s] + lo:cu[s] + hi, 0]
            vv = v[cu[s] + lo:cu[s] + hi, 0]
            z = kk @ q[t, 0] / np.sqrt(d)
            p = np.exp(z - z.max())
            assert np.allclose(out[t, 0], p @ vv / p.sum(), rtol=0, atol=1e-12)


def pin_backward_finite_differences():
    """Central differences of L = sum(out * G) in fp64 against dq, dk, dv, over
    causal / full / window, cross-attention lengths, GQA and a bias with -inf
    entries (every element of q, k, v perturbed)."""
    rng = np.random.default_rng(20)
    cases = [(False, 0, 0), (True, 0, 0), (True, 3, 0), (True, 0, 4), (False, 0, 1)]
    for causal, window, bias_heads in cases:
        q, k, v, cu_q, cu_kv, bias = _tiny_case(rng, 2, 5, 4, 2, 3, 2, cross=True,
                                                bias_heads=bias_heads, neg_inf=0.2)
        G = rng.standard_normal((q.shape[0], q.shape[1], v.shape[2]))
        _, (dq, dk, dv) = _loss_and_grads(q, k, v, cu_q, cu_kv, 0.7, causal, window, bias, G)
        h = 1e-6
        for x, dx in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp, _ = _loss_and_grads(q, k, v, cu_q, cu_kv, 0.7, causal, window, bias, G)
                x[idx] = old - h
                lm, _ = _loss_and_grads(q, k, v, cu_q, cu_kv, 0.7, causal, window, bias, G)
                x[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            _close(dx, num, 1e-6)


def pin_backward_sdpa_special_case():
    """Self-attention (Lq = Lk), causal or full, GQA, additive mask: float64
    torch.autograd through scaled_dot_product_attention gives the same dq,
    dk, dv."""
    rng = np.random.default_rng(21)
    for causal in (False, True):
        for hq, hkv in ((2, 2), (4, 2)):
            L, d, dv_ = 9, 5, 3
            q = rng.standard_normal((L, hq, d))
            k = rng.standard_normal((L, hkv, d))
            v = rng.standard_normal((L, hkv, dv_))
            bias = rng.standard_normal((L, hq, L))
            bias[rng.random(bias.shape) < 0.2] = -np.inf
            bias[:, :, 0] = 0.0  # every row keeps a visible key
            G = rng.standard_normal((L, hq, dv_))
            cu = np.array([0, L])
            dq, dk, dv = oracle.varlen_attention_backward(q, k, v, G, cu, cu, 0.6, causal, 0, bias)
            tq, tk, tv = (torch.tensor(x.transpose(1, 0, 2)[None], requires_grad=True)
                          for x in (q, k, v))
            rep = hq // hkv
            kk = tk.repeat_interleave(rep, dim=1)
            vv = tv.repeat_interleave(rep, dim=1)
            mask = torch.tensor(bias.transpose(1, 0, 2)[None])
            if causal:
                mask = mask.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
            o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=mask,
                                                                 scale=0.6)
            (o * torch.tensor(G.transpose(1, 0, 2)[None])).sum().backward()
            _close(dq, tq.grad[0].numpy().transpose(1, 0, 2), 1e-12)
            _close(dk, tk.grad[0].numpy().transpose(1, 0, 2), 1e-12)
            _close(dv, tv.grad[0].numpy().transpose(1, 0, 2), 1e-12)


def pin_backward_closed_forms():
    """V equal for all keys: out does not depend on q or k, so dq = dk = 0 and
    dv_j = sum_i p_ij dout_i; a one-key sequence gives dv = sum of its rows'
    dout and dq = dk = 0; dout = 0 gives zero gradients; shifting every key
    by one vector leaves out unchanged, so dk sums to zero over a sequence."""
    rng = np.random.default_rng(22)
    q, k, v, cu_q, cu_kv, _ = _tiny_case(rng, 2, 6, 2, 1, 4, 3, cross=True)
    v[:] = rng.standard_normal(3)
    G = rng.standard_normal((q.shape[0], 2, 3))
    dq, dk, dv = oracle.varlen_attention_backward(q, k, v, G, cu_q, cu_kv, None, True, 0, None)
    _close(dq, np.zeros_like(dq), 1e-12)
    _close(dk, np.zeros_like(dk), 1e-12)
    # one key per sequence
    cu_k1 = np.arange(len(cu_q))
    k1 = rng.standard_normal((len(cu_q) - 1, 1, 4))
    v1 = rng.standard_normal((len(cu_q) - 1, 1, 3))
    dq, dk, dv = oracle.varlen_attention_backward(q, k1, v1, G, cu_q, cu_k1, None, False, 0, None)
    _close(dq, np.zeros_like(dq), 1e-12)
    _close(dk, np.zeros_like(dk), 1e-12)
    for s in range(len(cu_q) - 1):
        _close(dv[s, 0], G[cu_q[s]:cu_q[s + 1]].sum(axis=(0, 1)), 1e-12)
    # dout = 0
    q, k, v, cu_q, cu_kv, bias = _tiny_case(rng, 3, 7, 4, 2, 4, 3, cross=True, bias_heads=1,
                                            neg_inf=0.2)
    z = oracle.varlen_attention_backward(q, k, v, np.zeros((q.shape[0], 4, 3)), cu_q, cu_kv,
                                         None, True, 3, bias)
    for g in z:
        assert not np.any(g)
    # translation of the keys
    G = rng.standard_normal((q.shape[0], 4, 3))
    _, dk, _ = oracle.varlen_attention_backward(q, k, v, G, cu_q, cu_kv, None, True, 0, bias)
    for s in range(len(cu_kv) - 1):
        _close(dk[cu_kv[s]:cu_kv[s + 1]].sum(axis=0), np.zeros(dk.shape[1:]), 1e-12)


# ---------------------------------------------------------------- key-padding front end
PAD_MASK = np.array([[1, 1, 0, 1], [0, 0, 0, 0], [0, 1, 1, 1]], dtype=bool)


def pin_padding_hand_worked():
    """Ranks, cumulative counts and the gather / scatter on a 3 x 4 mask
    worked by hand: row 0 keeps tokens 0, 1, 3; row 1 is all padding; row 2
    keeps 1, 2, 3."""
    ranks, cu, stats = oracle.padding_to_varlen(PAD_MASK)
    assert ranks.tolist() == [[0, 1, -1, 2], [-1, -1, -1, -1], [-1, 0, 1, 2]], ranks
    assert cu.tolist() == [0, 3, 3, 6], cu
    assert stats == (6, 3), stats
    padded = (10.0 * np.arange(3)[:, None] + np.arange(4)[None, :])[:, :, None, None] + \
        np.array([0.0, 0.5])[None, None, :, None]  # [3, 4, 2 heads, 1]
    packed = oracle.pack_tokens(padded, PAD_MASK)
    assert packed[:, 0, 0].tolist() == [0.0, 1.0, 3.0, 21.0, 22.0, 23.0], packed[:, 0, 0]
    assert packed[:, 1, 0].tolist() == [0.5, 1.5, 3.5, 21.5, 22.5, 23.5]
    back = oracle.unpack_tokens(packed, PAD_MASK)
    assert np.array_equal(back, np.where(PAD_MASK[:, :, None, None], padded, 0.0))
    # all valid: ranks are the positions, cu the multiples of the row length
    r2, cu2, st2 = oracle.padding_to_varlen(np.ones((2, 5), dtype=bool))
    assert r2.tolist() == [list(range(5))] * 2 and cu2.tolist() == [0, 5, 10] and st2 == (10, 5)


def _padded_case(rng, bsz=3, n=9, hq=4, hkv=2, d=8, dv=6):
    mask = rng.random((bsz, n)) < 0.6
    mask[0] = True           # a full row
    mask[1, :] = False       # an empty row
    mask[1, [2, 7]] = True   # ... with two valid tokens far apart
    mask[2, 0] = False       # left padding
    q = rng.standard_normal((bsz, hq, n, d))
    k = rng.standard_normal((bsz, hkv, n, d))
    v = rng.standard_normal((bsz, hkv, n, dv))
    return mask, q, k, v


def pin_masked_attention_sdpa():
    """The dense key-padding definition against torch's float64 CPU SDPA with
    a boolean mask: on valid rows that see a key they agree; padded rows are
    0 by definition."""
    import torch.nn.functional as F
    rng = np.random.default_rng(123)
    for causal in (False, True):
        mask, q, k, v = _padded_case(rng)
        bsz, hq, n, d = q.shape
        out = oracle.masked_attention(q, k, v, mask, 1.0 / math.sqrt(d), causal)
        am = torch.from_numpy(mask)[:, None, None, :].expand(bsz, 1, n, n)
        if causal:
            am = am & torch.tril(torch.ones(n, n, dtype=torch.bool))
        rep = hq // k.shape[1]
        tk = torch.from_numpy(np.repeat(k, rep, axis=1))
        tv = torch.from_numpy(np.repeat(v, rep, axis=1))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), tk, tv, attn_mask=am).numpy()
        sees = am[:, 0].any(dim=-1).numpy() & mask  # [B, N]
        for b in range(bsz):
            for i in range(n):
                if sees[b, i]:
                    _close(out[b, :, i], ref[b, :, i], 1e-12)
                else:
                    assert np.all(out[b, :, i] == 0.0)


def pin_packed_matches_masked():
    """Packing, varlen attention on the packed rows and unpacking gives the
    dense key-padding result: causal visibility survives packing because the
    valid tokens keep their order."""
    rng = np.random.default_rng(321)
    for causal in (False, True):
        mask, q, k, v = _padded_case(rng)
        d = q.shape[3]
        _, cu, _ = oracle.padding_to_varlen(mask)
        pq = oracle.pack_tokens(q.transpose(0, 2, 1, 3), mask)
        pk = oracle.pack_tokens(k.transpose(0, 2, 1, 3), mask)
        pv = oracle.pack_tokens(v.transpose(0, 2, 1, 3), mask)
        out, _ = oracle.varlen_attention(pq, pk, pv, cu, cu, 1.0 / math.sqrt(d), causal, 0, None)
        dense = oracle.unpack_tokens(out, mask).transpose(0, 2, 1, 3)
        ref = oracle.masked_attention(q, k, v, mask, 1.0 / math.sqrt(d), causal)
        _close(dense, ref, 1e-12)


def pin_padding_lengths_hand_worked():
    """Counts, spans and the right-padding test by hand: a row whose valid
    tokens come first is right-padded; one with a hole or valid tokens after
    padding is not; empty and full rows are."""
    cases = [
        ([[1, 1, 1, 0, 0], [1, 1, 1, 1, 1], [0, 0, 0, 0, 0]], [3, 5, 0], True, 5),
        ([[1, 1, 0, 0, 0], [1, 0, 1, 0, 0]], [2, 2], False, 2),
        ([[0, 1, 1, 0, 0]], [2], False, 2),
        ([[1, 1, 1, 1, 0], [0, 0, 0, 0, 1]], [4, 1], False, 4),
    ]
    for mask, counts, right, longest in cases:
        m = np.array(mask, dtype=bool)
        c, spans, r, lg = oracle.padding_lengths(m)
        assert list(c) == counts and r == right and lg == longest, (mask, c, r, lg)
        assert list(spans) == [5 * b for b in range(len(mask) + 1)]


def pin_used_prefixes_match_key_padding():
    """Spans whose first used rows are the sequences (a right-padded batch
    attended in place) give the dense key-padding result: the used-prefix
    problem, packed, run through the varlen definition and put back at the
    spans' first rows (0 elsewhere) equals masked attention with the
    right-padding mask."""
    rng = np.random.default_rng(322)
    bsz, n, hq, hkv, d = 3, 9, 4, 2, 8
    used = np.array([9, 4, -2])  # a negative count means an empty sequence
    mask = np.arange(n)[None, :] < used[:, None]
    q = rng.standard_normal((bsz, hq, n, d))
    k = rng.standard_normal((bsz, hkv, n, d))
    v = rng.standard_normal((bsz, hkv, n, d))
    spans = np.arange(bsz + 1) * n
    for causal in (False, True):
        tok = [x.transpose(0, 2, 1, 3).reshape(bsz * n, x.shape[1], d) for x in (q, k, v)]
        pq, cu = oracle.used_prefixes(tok[0], spans, used)
        pk, _ = oracle.used_prefixes(tok[1], spans, used)
        pv, _ = oracle.used_prefixes(tok[2], spans, used)
        out, _ = oracle.varlen_attention(pq, pk, pv, cu, cu, 1.0 / math.sqrt(d), causal, 0, None)
        dense = np.zeros((bsz, n, hq, d))
        for b in range(bsz):
            dense[b, :cu[b + 1] - cu[b]] = out[cu[b]:cu[b + 1]]
        ref = oracle.masked_attention(q, k, v, mask, 1.0 / math.sqrt(d), causal)
        _close(dense.transpose(0, 2, 1, 3), ref, 1e-12)


# ---------------------------------------------------------------- ALiBi
def pin_alibi_hand_worked():
    """Two sequences (3 queries / 3 keys, 1 query / 4 keys) and slopes 0.5,
    0.25, worked by hand: the query's end-aligned position minus the key,
    in absolute value, times minus the slope."""
    b = oracle.alibi_bias([0.5, 0.25], [0, 3, 4], [0, 3, 7], 2, 4)
    assert b[0, 0].tolist() == [0.0, -0.5, -1.0, 0.0]       # row 0, position 0
    assert b[2, 0].tolist() == [-1.0, -0.5, 0.0, 0.0]       # row 2, position 2
    assert b[1, 1].tolist() == [-0.25, 0.0, -0.25, 0.0]     # slope 0.25, position 1
    assert b[3, 0].tolist() == [-1.5, -1.0, -0.5, 0.0]      # decode row: position 3 of 4 keys
    per_seq = oracle.alibi_bias([[0.5, 0.25], [2.0, 1.0]], [0, 3, 4], [0, 3, 7], 2, 4)
    assert per_seq[3, 1].tolist() == [-3.0, -2.0, -1.0, 0.0]


def pin_alibi_causal_is_a_linear_key_bias():
    """Under the causal mask every visible key sits at or before the query's
    position, so -slope * |pos - j| = slope * j - slope * pos: the output
    equals that of the bias slope * j alone (a per-row constant cancels in
    the softmax) and the LSE differs by exactly -slope * pos."""
    rng = np.random.default_rng(17)
    lens_q, lens_k = [5, 9, 1], [5, 12, 6]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    hq, hkv, d = 4, 2, 8
    q = rng.standard_normal((int(cu_q[-1]), hq, d))
    k = rng.standard_normal((int(cu_k[-1]), hkv, d))
    v = rng.standard_normal((int(cu_k[-1]), hkv, d))
    slopes = np.array([0.5, 0.25, 0.125, 1.0 / 3.0])
    cols = max(lens_k)
    out_a, lse_a = oracle.varlen_attention(q, k, v, cu_q, cu_k, None, True, 0,
                                           oracle.alibi_bias(slopes, cu_q, cu_k, hq, cols))
    lin = np.zeros((int(cu_q[-1]), hq, cols))
    shift = np.zeros((hq, int(cu_q[-1])))
    for s in range(len(lens_q)):
        for i in range(lens_q[s]):
            t = int(cu_q[s]) + i
            lin[t] = slopes[:, None] * np.arange(cols)[None, :]
            shift[:, t] = -slopes * (i + lens_k[s] - lens_q[s])
    out_l, lse_l = oracle.varlen_attention(q, k, v, cu_q, cu_k, None, True, 0, lin)
    _close(out_a, out_l, 1e-12)
    _close(lse_a, lse_l + shift, 1e-12)


ALL_PINS = [pin_brute_force_tiny, pin_sdpa_special_case, pin_rows_sum_to_one,
            pin_one_key_sequence, pin_zero_queries_mean, pin_key_permutation_invariance,
            pin_neg_inf_key_is_removed, pin_mask_counts_closed_form, pin_golden_hand_worked,
            pin_row_subset_matches_full, pin_bias_ranges_prefix_lm_closed_form,
            pin_bias_ranges_skip_is_exact, pin_backward_finite_differences,
            pin_backward_sdpa_special_case, pin_backward_closed_forms, pin_padding_hand_worked,
            pin_masked_attention_sdpa, pin_packed_matches_masked, pin_alibi_hand_worked,
            pin_alibi_causal_is_a_linear_key_bias, pin_interval_rows_hand_worked,
            pin_interval_rows_attend_their_range, pin_padding_lengths_hand_worked,
            pin_used_prefixes_match_key_padding]
