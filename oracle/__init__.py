"""Float64 CPU oracle (test infrastructure only).

Imported by the tests, by the smoke check and by the benchmark's CPU-baseline
leg; never by the library. See `attention_ref` for what it computes and which
passages of the pages each function follows.
"""

from .attention_ref import (  # noqa: F401
    attention,
    attention_ragged_paged,
    cascade_attention,
    causal_visible,
    decode_paged,
    decode_paged_variant,
    default_threads,
    gather_paged_kv,
    log_sum_exp,
    merge_partials,
    online_softmax_row,
    split_kv_partials,
)
