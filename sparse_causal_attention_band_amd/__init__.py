"""Causal sliding-window attention for MI355X (gfx950).

Python face of ``libswa_attn.so``: ``attn_fwd`` (band + optional strided
keys, whole-sequence forward), ``attn_fwd_two_sided`` (band without the
causal cut), ``diff_attn_fwd`` (differential attention over the band),
``attn_fwd_global`` (the band plus global tokens),
``decode`` (one token per sequence over a rolling window-slot KV
cache; ``decode_noalloc`` the same without a caller workspace), ``chunk_prefill`` and ``ring_append`` (prefill in chunks over that
cache).  The arithmetic runs in hand-written HIP kernels behind the C ABI
declared in ``include/swa_attn.h``.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    SIGNATURES,
    SwaError,
    attn_fwd,
    attn_fwd_global,
    attn_fwd_two_sided,
    chunk_prefill,
    decode,
    decode_noalloc,
    decode_workspace_bytes,
    diff_attn_fwd,
    global_workspace_bytes,
    lib,
    ring_append,
)
