"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  Holds no attention arithmetic: only random draws, shapes and casts.

Recipe (each configuration draws Q, K, V in that order from one CPU
generator seeded with its seed): i.i.d. N(0, 1) in float32, multiplied by
``qk_scale`` for Q and K when given (exact: a power of two), then rounded to
the storage dtype (round to nearest even for bfloat16).  The decode workload
draws q, the full K and V rings (every slot, valid or not) and then the
positions ``randint(1, max_pos + 1)`` from the same generator.  The chunk
workload draws q, k, v of the chunk and then both full rings; its cached
lengths p0 are fixed per sequence.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    window: int
    stride: int
    dtype: torch.dtype
    seed: int
    qk_scale: float = 1.0


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    window: int
    max_pos: int
    dtype: torch.dtype
    seed: int


@dataclass(frozen=True)
class ChunkConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int            # new tokens per sequence in the chunk
    d: int
    window: int       # ring size
    p0: tuple         # positions already cached, per sequence
    dtype: torch.dtype
    seed: int
    qk_scale: float = 1.0


# The workloads the pages describe: a tiny fp32 case, a Mistral-7B-shaped
# layer (GQA 32/8, d=128, W=4096), a Gemma-3-like SWA-1024 layer at long
# context, the local + strided sparse mask (W=256, stride 128), and a
# rolling-window decode step (64 sequences, W=4096 ring).
TINY = PrefillConfig("tiny_swa_fp32", 1, 1, 1, 256, 64, 32, 0, torch.float32, 0)
MISTRAL = PrefillConfig("mistral7b_swa4096_n16384", 1, 32, 8, 16384, 128, 4096, 0, torch.bfloat16, 1, 0.5)
GEMMA = PrefillConfig("gemma3_swa1024_n65536", 2, 32, 16, 65536, 128, 1024, 0, torch.bfloat16, 2)
STRIDED = PrefillConfig("local256_stride128_n8192", 1, 16, 16, 8192, 64, 256, 128, torch.bfloat16, 3)
DECODE = DecodeConfig("decode_ring4096_b64", 64, 32, 8, 128, 4096, 131072, torch.bfloat16, 4)

# Chunked prefill over the rolling cache: a serving batch of four
# Mistral-shaped sequences taking a 4096-token chunk each, one starting fresh,
# one with part of a window cached, two deep into long histories.
CHUNK = ChunkConfig("mistral7b_chunk4096_ring4096_b4", 4, 32, 8, 4096, 128, 4096, (0, 1500, 4095, 61440),
                    torch.bfloat16, 5, 0.5)

PREFILL_CONFIGS = (TINY, MISTRAL, GEMMA, STRIDED)


def prefill_inputs(cfg: PrefillConfig, N: int | None = None):
    """CPU tensors q [B,Hq,N,d], k, v [B,Hkv,N,d] in cfg.dtype."""
    n = cfg.N if N is None else N
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    q = torch.randn(cfg.B, cfg.Hq, n, cfg.d, generator=g)
    k = torch.randn(cfg.B, cfg.Hkv, n, cfg.d, generator=g)
    v = torch.randn(cfg.B, cfg.Hkv, n, cfg.d, generator=g)
    if cfg.qk_scale != 1.0:
        q.mul_(cfg.qk_scale)
        k.mul_(cfg.qk_scale)
    return q.to(cfg.dtype), k.to(cfg.dtype), v.to(cfg.dtype)


def random_qkv(B, Hq, Hkv, N, d, dtype, seed, qk_scale=1.0):
    """Same recipe for an arbitrary shape (parity sweeps)."""
    return prefill_inputs(PrefillConfig("adhoc", B, Hq, Hkv, N, d, 1, 0, dtype, seed, qk_scale))


def decode_inputs(cfg: DecodeConfig, B: int | None = None):
    """CPU tensors q [B,Hq,d], kring, vring [B,Hkv,W,d], pos int32 [B]."""
    b = cfg.B if B is None else B
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    q = torch.randn(b, cfg.Hq, cfg.d, generator=g)
    kr = torch.randn(b, cfg.Hkv, cfg.window, cfg.d, generator=g)
    vr = torch.randn(b, cfg.Hkv, cfg.window, cfg.d, generator=g)
    pos = torch.randint(1, cfg.max_pos + 1, (b,), generator=g, dtype=torch.int64).to(torch.int32)
    return q.to(cfg.dtype), kr.to(cfg.dtype), vr.to(cfg.dtype), pos


def chunk_inputs(cfg: ChunkConfig, T: int | None = None):
    """CPU tensors q [B,Hq,T,d], k, v [B,Hkv,T,d], kring, vring [B,Hkv,W,d]
    (every slot drawn) and p0 int32 [B], in that draw order; Q, K and both
    rings carry qk_scale like the prefill recipe."""
    t = cfg.T if T is None else T
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    q = torch.randn(cfg.B, cfg.Hq, t, cfg.d, generator=g)
    k = torch.randn(cfg.B, cfg.Hkv, t, cfg.d, generator=g)
    v = torch.randn(cfg.B, cfg.Hkv, t, cfg.d, generator=g)
    kr = torch.randn(cfg.B, cfg.Hkv, cfg.window, cfg.d, generator=g)
    vr = torch.randn(cfg.B, cfg.Hkv, cfg.window, cfg.d, generator=g)
    if cfg.qk_scale != 1.0:
        q.mul_(cfg.qk_scale)
        k.mul_(cfg.qk_scale)
        kr.mul_(cfg.qk_scale)
    p0 = torch.tensor(cfg.p0, dtype=torch.int32)
    return (q.to(cfg.dtype), k.to(cfg.dtype), v.to(cfg.dtype), kr.to(cfg.dtype), vr.to(cfg.dtype), p0)
