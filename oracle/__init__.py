"""CPU oracle for the paged decode path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import
this package. It imports nothing from the HIP library and the library imports nothing from it.
"""
from .paged_attention import (  # noqa: F401
    attention_one_query,
    blocked_form_ref,
    causal_rows,
    copy_blocks_ref,
    gather_sequence_kv,
    k_offset,
    merge_partition_states_ref,
    paged_decode_ref,
    paged_prefill_ref,
    partition_states_ref,
    reshape_and_cache_ref,
    slot_of,
    storage_dtype,
    swap_blocks_ref,
    to_f64,
    token_kv,
    v_offset,
)
