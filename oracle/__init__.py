"""fp64 CPU oracle for varlen attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg import this package.  It shares no code with the HIP
path.  Every function is pinned by tests against brute force, a library
routine on its special cases, closed forms and invariants; none is
"parity unpinned".
"""
from .ref_attention import (attention_rows, bias_head, finish_rows, kv_head_of, logits,
                            softmax_rows, varlen_attention, visible, visible_counts)
from .ref_backward import varlen_attention_backward
from .ref_masks import alibi_bias, bias_key_ranges, bias_rows_are_intervals
from .ref_padding import (masked_attention, pack_tokens, padding_lengths, padding_to_varlen,
                          unpack_tokens, used_prefixes)

__all__ = ["alibi_bias", "attention_rows", "bias_head", "bias_key_ranges", "bias_rows_are_intervals",
           "finish_rows", "kv_head_of", "logits",
           "masked_attention", "pack_tokens", "padding_lengths", "padding_to_varlen", "softmax_rows",
           "unpack_tokens", "used_prefixes", "varlen_attention", "varlen_attention_backward", "visible",
           "visible_counts"]
