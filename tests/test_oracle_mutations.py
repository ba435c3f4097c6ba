"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch every one of them.

Each mutation edits one expression of the oracle's source, loads the edited
copy as a separate module and points the ``oracle`` package at it for the
duration of the test.  A mutation counts as caught when at least one pin
raises.
"""
import inspect
import types

import pytest

import oracle
from oracle import ref_attention, ref_backward, ref_masks, ref_padding
from oracle_pins import ALL_PINS

MUTATIONS = {
    "causal_off_by_one": ("ok = ok & (j <= i + off)", "ok = ok & (j < i + off)"),
    "causal_top_left": ("ok = ok & (j <= i + off)", "ok = ok & (j <= i)"),
    "diagonal_sign": ("off = lk - lq", "off = lq - lk"),
    "window_w_plus_one": ("ok = ok & (j > i + off - window)", "ok = ok & (j >= i + off - window)"),
    "gqa_modulo": ("return h // (hq // hkv)", "return h % hkv"),
    "scale_dropped": ("z = scale * (qrows @ kseq.T)", "z = (qrows @ kseq.T)"),
    "bias_sign": ("z = z + bias_rows", "z = z - bias_rows"),
    "bias_head_always_zero": ("return 0 if bias_heads == 1 else head", "return 0"),
    "mask_dropped": ("unmasked = mask & (z != -np.inf)", "unmasked = (z != -np.inf)"),
    "no_normalisation": ("pn = p / safe_l[:, None]", "pn = p"),
    "lse_log2": ("np.where(np.isfinite(m), m, 0.0) + np.log(safe_l)",
                 "np.where(np.isfinite(m), m, 0.0) + np.log2(safe_l)"),
    "lse_without_max": ("np.where(np.isfinite(m), m, 0.0) + np.log(safe_l)", "np.log(safe_l)"),
    "empty_row_lse_zero": ("np.log(safe_l), -np.inf)", "np.log(safe_l), 0.0)"),
    "k_rows_from_query_offsets": ("kseq = k[ck0:ck1, g, :]", "kseq = k[cq0:cq0 + lk, g, :]"),
    "v_from_query_head": ("vseq = v[ck0:ck1, g, :]", "vseq = v[ck0:ck1, head % v.shape[1], :]"),
    "key_range_upper_open": ("ok = (j >= 0) & (j < lk)", "ok = (j >= 0) & (j < lk - 1)"),
}

# mutations of the mask front-end oracle (oracle/ref_masks.py)
MASK_MUTATIONS = {
    "ranges_hi_closed": ("out[h, t] = (keys[0], keys[-1] + 1)", "out[h, t] = (keys[0], keys[-1])"),
    "ranges_ignore_key_length": ("lk = min(int(cu_kv[s + 1] - cu_kv[s]), cols)", "lk = cols"),
    "ranges_lo_zero": ("out[h, t] = (keys[0], keys[-1] + 1)", "out[h, t] = (0, keys[-1] + 1)"),
    "ranges_finite_test": ("keys = np.nonzero(bias[t, h, :lk] != -np.inf)[0]",
                           "keys = np.nonzero(bias[t, h, :lk] > 0)[0]"),
    "alibi_sign": ("= -sl[h] * abs(pos - j)", "= sl[h] * abs(pos - j)"),
    "alibi_start_aligned": ("pos = i + lk - lq", "pos = i"),
    "alibi_no_abs": ("= -sl[h] * abs(pos - j)", "= -sl[h] * (pos - j)"),
    "alibi_first_seq_slopes": ("sl = slopes if slopes.ndim == 1 else slopes[s]",
                               "sl = slopes if slopes.ndim == 1 else slopes[0]"),
    "alibi_head_reversed": ("= -sl[h] * abs(pos - j)", "= -sl[hq - 1 - h] * abs(pos - j)"),
    "interval_nonpositive_ok": ("np.all(inside == 0.0)", "np.all(inside <= 0.0)"),
    "interval_last_key_unchecked": ("inside = row[lo:hi]", "inside = row[lo:hi - 1]"),
    "interval_finite_ok": ("np.all(inside == 0.0)", "np.all(np.isfinite(inside))"),
    "interval_empty_not_interval": ("out[h, t] = bool(np.all(inside == 0.0)",
                                    "out[h, t] = hi > lo and bool(np.all(inside == 0.0)"),
}

# mutations of the backward oracle (oracle/ref_backward.py)
BACKWARD_MUTATIONS = {
    "bwd_no_delta": ("dz = p * (dp - delta[:, None])", "dz = p * dp"),
    "bwd_delta_unweighted": ("delta = (p * dp).sum(axis=1)", "delta = dp.sum(axis=1)"),
    "bwd_dq_no_scale": ("dq[cq0:cq1, h] += scale * (dz @ ks)", "dq[cq0:cq1, h] += dz @ ks"),
    "bwd_dk_untransposed": ("dk[ck0:ck1, g] += scale * (dz.T @ qs)",
                            "dk[ck0:ck1, g] += scale * (dz.T @ qs[::-1])"),
    "bwd_dv_unnormalised": ("p = np.where(nonempty[:, None], p / np.where(nonempty, l, 1.0)[:, None], 0.0)",
                            "p = np.where(nonempty[:, None], p, 0.0)"),
    "bwd_dv_from_dz": ("dv[ck0:ck1, g] += p.T @ do", "dv[ck0:ck1, g] += dz.T @ do"),
    "bwd_dk_overwrite_gqa": ("dk[ck0:ck1, g] += scale * (dz.T @ qs)",
                             "dk[ck0:ck1, g] = scale * (dz.T @ qs)"),
    "bwd_mask_dropped": ("p, m, l = softmax_rows(z, mask)", "p, m, l = softmax_rows(z, mask | True)"),
}

# mutations of the key-padding oracle (oracle/ref_padding.py)
PADDING_MUTATIONS = {
    "pad_rank_from_one": ("                ranks[r, t] = c\n", "                ranks[r, t] = c + 1\n"),
    "pad_cu_counts_not_summed": ("cu[1:] = np.cumsum(counts)", "cu[1:] = counts"),
    "pad_longest_is_total": ("int(counts.max(initial=0))", "int(counts.sum())"),
    "pad_pack_keeps_padding": ("if mask[b, t]]", "if mask[b, t] or t == 0]"),
    "pad_unpack_shifted": ("                out[b, t] = packed[i]\n                i += 1",
                           "                i += 1\n                out[b, t] = packed[i - 1 if t else i % len(packed)]"),
    "pad_query_mask_ignored": ("seen = np.isfinite(m[:, 0]) & mask[b]", "seen = np.isfinite(m[:, 0])"),
    "pad_key_mask_ignored": ("vis = np.broadcast_to(mask[b][None, :], (n, n))",
                             "vis = np.ones((n, n), dtype=bool)"),
    "pad_causal_flipped": ("vis = vis & (j <= i)", "vis = vis & (j >= i)"),
    "pad_kv_head_modulo": ("g = h // (hq // hkv)", "g = h % hkv"),
    "pad_right_any_valid": ("right = all(bool(mask[r, :counts[r]].all()) for r in range(b))",
                            "right = all(bool(mask[r, :counts[r]].any() or counts[r] == 0) for r in range(b))"),
    "pad_spans_unscaled": ("spans = np.arange(b + 1, dtype=np.int64) * n",
                           "spans = np.arange(b + 1, dtype=np.int64)"),
    "used_not_clamped_low": ("u = min(max(int(used[s]), 0), span)", "u = min(int(used[s]), span)"),
    "used_from_span_end": ("parts.append(x[int(cu[s]):int(cu[s]) + u])",
                           "parts.append(x[int(cu[s + 1]) - u:int(cu[s + 1])])"),
}

SOURCES = {"attention": inspect.getsource(ref_attention), "masks": inspect.getsource(ref_masks),
           "backward": inspect.getsource(ref_backward), "padding": inspect.getsource(ref_padding)}


def _mutant(module_key, old, new):
    src = SOURCES[module_key]
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = types.ModuleType("oracle.oracle_mutant")
    mutated.__package__ = "oracle"  # relative imports resolve inside the oracle package
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mutated.__dict__)
    return mutated


ALL_MUTATIONS = {**{("attention", k): v for k, v in MUTATIONS.items()},
                 **{("masks", k): v for k, v in MASK_MUTATIONS.items()},
                 **{("backward", k): v for k, v in BACKWARD_MUTATIONS.items()},
                 **{("padding", k): v for k, v in PADDING_MUTATIONS.items()}}


@pytest.mark.parametrize("key", sorted(ALL_MUTATIONS), ids=lambda k: f"{k[0]}-{k[1]}")
def test_pins_catch_mutation(key, monkeypatch):
    module_key, name = key
    old, new = ALL_MUTATIONS[key]
    mutated = _mutant(module_key, old, new)
    for attr in oracle.__all__:
        if hasattr(mutated, attr):
            monkeypatch.setattr(oracle, attr, getattr(mutated, attr))
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as e:  # an assertion or a crash both expose the mistake
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutation {name}"
