"""CPU fp64 oracle for batch attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.  It shares
no code with the HIP path.  Parity status of each function is recorded in the
design notes; every function here is pinned by the CPU tests (brute force,
closed forms, a library routine, invariances and the merge identity).
"""
from .attention import (  # noqa: F401
    LN2,
    attention_state,
    batch_attention,
    batch_attention_paged,
    batch_attention_ragged,
    gather_paged_kv,
    gather_ragged_kv,
    kv_head_of,
    kv_len_of,
    kv_lengths,
    merge_states,
    token_location,
    visibility,
)
