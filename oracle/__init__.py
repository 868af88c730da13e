"""Float64 CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package; the library never does.
"""
from .swa_oracle import (  # noqa: F401
    allowed_set,
    allowed_mask,
    allowed_pair_count,
    attn_fwd,
    attn_lse,
    attn_fwd_rows,
    attn_fwd_parallel,
    decode,
    ring_slot,
    ring_append,
    chunk_prefill,
    chunk_prefill_lse,
    allowed_mask_two_sided,
    attn_fwd_two_sided,
    diff_attn_fwd,
    allowed_mask_global,
    attn_fwd_global,
)
