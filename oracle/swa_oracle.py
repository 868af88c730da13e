"""Float64 CPU oracle for causal sliding-window attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this folder.
The library under ``sparse_causal_attention_band_amd/`` never imports it, and
this module imports nothing from there: the two share no code.

Everything here is the plain definition, written out in float64 with numpy:

* The allowed key set of a query row follows the window definition of the page
  "SWA：滑动窗口注意力与跨层信息传递" (§3.1, the set N_W(i) and the mask
  M^SWA): row i may read key j iff max(1, i-W+1) <= j <= i in that page's
  1-based numbering, i.e. the window W counts the current position.  Here
  positions are 0-based, so the band is [max(0, i-W+1), i], which is also the
  range used by the sliding-window mask of the page
  "注意力变体——滑动窗口、稀疏、差分" (构建它, 第 2 步).
* The local + strided variant adds, to that band, every key j <= i with
  j mod stride == 0 (0-based j), as in the same page's step 3 ("局部 + 步进
  稀疏掩码"); the union is a set, a key is counted once.  stride <= 0 means no
  strided part.
* Attention is softmax(scale * Q K^T + M) V with the softmax taken row by row,
  so each query normalises over its own allowed keys only (SWA page, §3.1;
  the scale is 1/sqrt(d_k) there and is an explicit argument here).
* The rolling decode cache stores absolute position t (1-based) in slot
  (t-1) mod W (SWA page, §4.2); slot order is not time order, so the oracle
  gathers the valid slots back into time order before attending.
* Chunked prefill (SWA page, §4.3): the rows of a new chunk need different
  windows, so each row attends to the cached history in the ring plus the
  chunk's own earlier rows, under the same band; the history is read before
  the chunk is written into the ring.
* The two-sided (bidirectional) band drops the causal cut: row i reads keys
  i-left .. i+right, clipped to the sequence.  The attention-variants page
  (概念, 滑动窗口注意力) gives [i - W/2, i + W/2]; the explainer page
  "滑动窗口注意力" (§3.1 band mask and its §3.3 example) gives [i - w, i + w]
  with a radius w and builds the mask as start = max(0, i-w),
  end = min(n, i+w+1).  Separate left and right radii
  cover both; right = 0 is the causal band with W = left + 1.

* Differential attention (attention-variants page, 概念 and 第 4 步): two
  attention maps from separate Q/K pairs over one V, out = (A1 - lam * A2) V
  with a scalar lam per query head.  Here both maps use the same sliding-window
  band; with W >= N this is the page's causal version.

* Local + global tokens (attention-variants page, 稀疏 / 块注意力, Longformer /
  BigBird; the interview page "Sliding Window Attention 和 Sparse Attention
  有什么区别", 其他 Sparse Attention 模式, Global Token): a few global
  positions attend to every position and are attended to by every position,
  the rest keep the local window.  In the causal setting of this library
  "every position" means every position not after the row: row i may read
  key j iff j <= i and (i - j < W or j is global or i is global).

Readings where the pages leave a step open (each one is also listed in the
design notes of the repository):

* grouped query heads: query head h reads KV head h // (Hq // Hkv);
* decode ``pos[b]`` is the 1-based absolute position of the one query token,
  whose own K/V are already in the ring; it attends to the min(pos, W) most
  recent positions; pos <= 0 yields an all-zero output row;
* the oracle subtracts the row maximum before exponentiating (same value
  mathematically); every row has at least its own key, so no row is empty.

Query rows are processed in blocks only to bound memory: each row's softmax is
still taken over exactly its own allowed set (keys outside the union of the
block's allowed sets have weight exp(-inf) = 0 and are simply not gathered).
"""
from __future__ import annotations

import os
from typing import Iterable, Optional

import numpy as np

__all__ = [
    "allowed_set",
    "allowed_mask",
    "allowed_pair_count",
    "attn_fwd",
    "attn_fwd_rows",
    "decode",
    "ring_slot",
    "attn_fwd_parallel",
    "ring_append",
    "chunk_prefill",
    "allowed_mask_two_sided",
    "attn_fwd_two_sided",
    "diff_attn_fwd",
    "allowed_mask_global",
    "attn_fwd_global",
]


def allowed_set(i: int, window: int, stride: int = 0) -> list[int]:
    """Sorted allowed key positions of 0-based query row ``i``.

    Band: [max(0, i-W+1), i] (SWA page §3.1, 0-based).  Strided part: every
    j in 0, stride, 2*stride, ... that is <= i (attention-variants page, step 3).
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    lo = max(0, i - window + 1)
    keys = set(range(lo, i + 1))
    if stride > 0:
        keys.update(range(0, i + 1, stride))
    return sorted(keys)


def allowed_mask(n: int, window: int, stride: int = 0) -> np.ndarray:
    """Boolean n x n matrix, True where (row i, key j) is allowed.

    Built row by row from ``allowed_set``; used for small n only.
    """
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, allowed_set(i, window, stride)] = True
    return m


def allowed_pair_count(n: int, window: int, stride: int = 0) -> int:
    """Total number of allowed (query, key) pairs, summed over rows.

    Counted from the row sets themselves (no closed form here; the closed
    forms live in the tests, where they pin this function).
    """
    total = 0
    for i in range(n):
        lo = max(0, i - window + 1)
        band = i - lo + 1
        extra = 0
        if stride > 0 and lo > 0:
            # multiples of stride strictly below the band start (those inside
            # the band are already counted once)
            extra = (lo - 1) // stride + 1
        total += band + extra
    return total


def _block_keys(i0: int, i1: int, window: int, stride: int) -> np.ndarray:
    """Union of the allowed sets of rows i0..i1 (inclusive), sorted."""
    lo = max(0, i0 - window + 1)
    keys = list(range(lo, i1 + 1))
    if stride > 0:
        keys = sorted(set(keys).union(range(0, i1 + 1, stride)))
    return np.asarray(keys, dtype=np.int64)


def _row_allowed(rows: np.ndarray, keys: np.ndarray, window: int, stride: int) -> np.ndarray:
    """Boolean [len(rows), len(keys)]: the definition, evaluated elementwise."""
    i = rows[:, None]
    j = keys[None, :]
    in_band = (j <= i) & (j >= np.maximum(0, i - window + 1))
    if stride > 0:
        in_stride = (j <= i) & (j % stride == 0)
        return in_band | in_stride
    return in_band


def _masked_softmax_rows(scores: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Row-wise softmax over the allowed entries only (float64)."""
    s = np.where(allowed, scores, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(allowed, np.exp(s - m), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def _head_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
               window: int, stride: int, scale: float) -> np.ndarray:
    """Output rows ``rows`` of one (batch, head): q [N,d], k/v [N,d] float64."""
    out = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    if len(rows) == 0:
        return out
    # group consecutive rows so a block shares one gathered key list
    block = 256
    start = 0
    while start < len(rows):
        stop = start + 1
        while stop < len(rows) and stop - start < block and rows[stop] == rows[stop - 1] + 1:
            stop += 1
        r = rows[start:stop]
        keys = _block_keys(int(r[0]), int(r[-1]), window, stride)
        qr = np.asarray(q[r], dtype=np.float64)
        kk = np.asarray(k[keys], dtype=np.float64)
        vv = np.asarray(v[keys], dtype=np.float64)
        scores = scale * (qr @ kk.T)
        p = _masked_softmax_rows(scores, _row_allowed(r, keys, window, stride))
        out[start:stop] = p @ vv
        start = stop
    return out


def _check(q, k, v, window):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if Hq % k.shape[1] != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if window < 1:
        raise ValueError("window must be >= 1")


def attn_fwd_rows(q, k, v, window: int, stride: int, scale: float,
                  bh_rows: Iterable[tuple[int, int, int]]) -> np.ndarray:
    """Selected output rows: one float64 [d] vector per (b, h, i) triple.

    Inputs may be any real numpy dtype (e.g. float32 holding bf16 values);
    only the rows each triple needs are converted to float64.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    _check(q, k, v, window)
    G = q.shape[1] // k.shape[1]
    res = []
    for b, h, i in bh_rows:
        res.append(_head_rows(q[b, h], k[b, h // G], v[b, h // G],
                              np.asarray([i], dtype=np.int64), window, stride, scale)[0])
    return np.stack(res) if res else np.zeros((0, q.shape[3]))


def attn_fwd(q, k, v, window: int, stride: int = 0, scale: Optional[float] = None) -> np.ndarray:
    """Full forward: float64 [B, Hq, N, d].

    q: [B, Hq, N, d], k/v: [B, Hkv, N, d]; any real dtype, converted exactly
    to float64.  ``scale`` defaults to 1/sqrt(d) (SWA page §3.1).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check(q, k, v, window)
    B, Hq, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // k.shape[1]
    out = np.empty((B, Hq, N, v.shape[3]), dtype=np.float64)
    rows = np.arange(N, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = _head_rows(q[b, h], k[b, h // G], v[b, h // G], rows, window, stride, scale)
    return out



def _head_lse_rows(q: np.ndarray, k: np.ndarray, rows: np.ndarray, window: int, stride: int,
                   scale: float) -> np.ndarray:
    """Row log-sum-exp of one (batch, head): ln sum_{j in S_i} exp(scale * q_i . k_j)
    for each i in ``rows`` (float64), S_i the allowed set of ``_row_allowed``.

    This is the natural log of the row's softmax denominator (SWA page §3.1,
    the row-wise softmax over N_W(i)), taken with the row maximum factored
    out so that no exponential overflows: m + ln sum exp(s - m)."""
    out = np.empty(len(rows), dtype=np.float64)
    if len(rows) == 0:
        return out
    block = 256
    start = 0
    while start < len(rows):
        stop = start + 1
        while stop < len(rows) and stop - start < block and rows[stop] == rows[stop - 1] + 1:
            stop += 1
        r = rows[start:stop]
        keys = _block_keys(int(r[0]), int(r[-1]), window, stride)
        scores = scale * (np.asarray(q[r], dtype=np.float64) @ np.asarray(k[keys], dtype=np.float64).T)
        s = np.where(_row_allowed(r, keys, window, stride), scores, -np.inf)
        m = s.max(axis=1)
        out[start:stop] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        start = stop
    return out


def attn_lse(q, k, window: int, stride: int = 0, scale: Optional[float] = None) -> np.ndarray:
    """Row log-sum-exp of the band forward: float64 [B, Hq, N], entry (b, h, i)
    = ln sum over the allowed keys j of row i of exp(scale * q[b,h,i] . k[b,h//G,j]).

    Together with the output it lets two attention results over disjoint key
    sets be merged exactly (weights exp(lse_1 - lse) and exp(lse_2 - lse), lse
    the log of the summed denominators).  q: [B, Hq, N, d], k: [B, Hkv, N, d];
    ``scale`` defaults to 1/sqrt(d)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError("q must be [B, Hq, N, d] and k [B, Hkv, N, d]")
    if q.shape[1] % k.shape[1] != 0 or window < 1:
        raise ValueError("Hq must be a multiple of Hkv and window >= 1")
    B, Hq, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // k.shape[1]
    rows = np.arange(N, dtype=np.int64)
    out = np.empty((B, Hq, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = _head_lse_rows(q[b, h], k[b, h // G], rows, window, stride, scale)
    return out

_POOL_INPUT = None


def _pool_job(bh):
    from threadpoolctl import threadpool_limits

    q, k, v, rows, window, stride, scale, G = _POOL_INPUT
    b, h = bh
    with threadpool_limits(limits=1):
        return _head_rows(q[b, h], k[b, h // G], v[b, h // G], rows, window, stride, scale)


def attn_fwd_parallel(q, k, v, window: int, stride: int, scale: float,
                      rows: np.ndarray, workers: Optional[int] = None):
    """Same arithmetic as ``attn_fwd`` for the given query rows of every
    (b, h), spread over a forked process pool (one (b, h) per task, one BLAS
    thread per worker; the workers inherit the inputs instead of receiving
    copies).  Returns (float64 [B, Hq, len(rows), d], workers used)."""
    import multiprocessing as mp

    global _POOL_INPUT
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    _check(q, k, v, window)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    if workers is None:
        workers = len(os.sched_getaffinity(0))
    rows = np.asarray(rows, dtype=np.int64)
    _POOL_INPUT = (q, k, v, rows, window, stride, scale, G)
    try:
        ctx = mp.get_context("fork")
        with ctx.Pool(workers) as pool:
            parts = pool.map(_pool_job, [(b, h) for b in range(B) for h in range(Hq)], chunksize=1)
    finally:
        _POOL_INPUT = None
    out = np.stack(parts).reshape(B, Hq, len(rows), v.shape[3])
    return out, workers


def ring_slot(t: int, window: int) -> int:
    """Ring slot holding 1-based absolute position t (SWA page §4.2)."""
    return (t - 1) % window


def decode(q, kring, vring, pos, window: int, scale: Optional[float] = None) -> np.ndarray:
    """One decode step per sequence over a rolling W-slot cache, float64.

    q: [B, Hq, d]; kring, vring: [B, Hkv, W, d]; pos: [B] 1-based absolute
    positions of the query tokens.  The query attends to positions
    pos-n+1 .. pos with n = min(pos, W), read from slots (t-1) mod W and put
    back into time order; pos <= 0 gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    kring = np.asarray(kring, dtype=np.float64)
    vring = np.asarray(vring, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    B, Hq, d = q.shape
    if kring.shape[2] != window or vring.shape != kring.shape:
        raise ValueError("rings must be [B, Hkv, W, d]")
    if Hq % kring.shape[1] != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // kring.shape[1]
    out = np.zeros((B, Hq, vring.shape[3]), dtype=np.float64)
    for b in range(B):
        p = int(pos[b])
        if p <= 0:
            continue
        n = min(p, window)
        times = range(p - n + 1, p + 1)
        slots = np.asarray([ring_slot(t, window) for t in times], dtype=np.int64)
        for h in range(Hq):
            kk = kring[b, h // G][slots]
            vv = vring[b, h // G][slots]
            s = scale * (kk @ q[b, h])
            e = np.exp(s - s.max())
            out[b, h] = (e / e.sum()) @ vv
    return out


def ring_append(kring, vring, k, v, p0, window: int):
    """Write a chunk's K/V rows into the rolling cache (SWA page §4.2).

    kring, vring: [B, Hkv, W, d]; k, v: [B, Hkv, T, d]; p0: [B] number of
    positions already cached.  Chunk row r is absolute position p0 + r + 1
    and goes to slot (p0 + r) mod W; later rows overwrite earlier ones.
    Returns new float64 rings.
    """
    kr = np.array(kring, dtype=np.float64, copy=True)
    vr = np.array(vring, dtype=np.float64, copy=True)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    for b in range(kr.shape[0]):
        for r in range(k.shape[2]):
            slot = ring_slot(int(p0[b]) + r + 1, window)
            kr[b, :, slot] = k[b, :, r]
            vr[b, :, slot] = v[b, :, r]
    return kr, vr


def chunk_prefill(q, k, v, kring, vring, p0, window: int, scale: Optional[float] = None,
                  rows=None) -> np.ndarray:
    """Attention of a chunk of T new tokens over the ring history plus the
    chunk itself (SWA page §4.3), float64 [B, Hq, T, d] (or only the chunk
    rows listed in ``rows``, ascending: [B, Hq, len(rows), d]).

    q: [B, Hq, T, d]; k, v: [B, Hkv, T, d] (the chunk's own keys/values);
    kring, vring: [B, Hkv, W, d] holding positions up to p0[b] (not yet the
    chunk); p0: [B].  Chunk row r is absolute position i = p0 + r + 1 and
    reads positions max(1, i-W+1) .. i: the history part comes from the ring
    (position t in slot (t-1) mod W), the rest from the chunk.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kring = np.asarray(kring, dtype=np.float64)
    vring = np.asarray(vring, dtype=np.float64)
    B, Hq, T, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // k.shape[1]
    sel = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, Hq, len(sel), v.shape[3]), dtype=np.float64)
    for b in range(B):
        start = int(p0[b])
        n_hist = min(start, window - 1)  # older positions are outside every chunk row's window
        times = range(start - n_hist + 1, start + 1)
        slots = np.asarray([ring_slot(t, window) for t in times], dtype=np.int64)
        # the history in time order, then the chunk: one sequence whose last T
        # rows are the chunk's rows, each with its full window available
        for h in range(Hq):
            g = h // G
            kk = np.concatenate([kring[b, g][slots], k[b, g]])
            vv = np.concatenate([vring[b, g][slots], v[b, g]])
            qq = np.concatenate([np.zeros((n_hist, d)), q[b, h]])
            out[b, h] = _head_rows(qq, kk, vv, n_hist + sel, window, 0, scale)
    return out


def chunk_prefill_lse(q, k, kring, p0, window: int, scale: Optional[float] = None) -> np.ndarray:
    """Row log-sum-exp of chunked prefill (SWA page §4.3): float64 [B, Hq, T],
    over the same keys as ``chunk_prefill`` (the ring history in time order,
    then the chunk), i.e. the log of each chunk row's softmax denominator."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    kring = np.asarray(kring, dtype=np.float64)
    B, Hq, T, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // k.shape[1]
    out = np.empty((B, Hq, T), dtype=np.float64)
    for b in range(B):
        start = int(p0[b])
        n_hist = min(start, window - 1)
        slots = np.asarray([ring_slot(t, window) for t in range(start - n_hist + 1, start + 1)], dtype=np.int64)
        for h in range(Hq):
            g = h // G
            kk = np.concatenate([kring[b, g][slots], k[b, g]])
            qq = np.concatenate([np.zeros((n_hist, d)), q[b, h]])
            out[b, h] = _head_lse_rows(qq, kk, n_hist + np.arange(T, dtype=np.int64), window, 0, scale)
    return out


def allowed_mask_two_sided(n: int, left: int, right: int) -> np.ndarray:
    """Boolean n x n matrix of the two-sided band: key j is allowed for row i
    iff i - left <= j <= i + right (0-based, clipped to [0, n))."""
    if left < 0 or right < 0:
        raise ValueError("left and right must be >= 0")
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, max(0, i - left):min(n, i + right + 1)] = True
    return m


def attn_fwd_two_sided(q, k, v, left: int, right: int, scale: Optional[float] = None) -> np.ndarray:
    """softmax(scale * Q K^T + M) V with the two-sided band mask M (no causal
    cut), float64 [B, Hq, N, d].  Rows are taken in blocks; each row
    normalises over exactly its own keys i-left .. i+right."""
    if left < 0 or right < 0:
        raise ValueError("left and right must be >= 0")
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or v.shape != k.shape or Hq % k.shape[1] != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hq a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // k.shape[1]
    out = np.empty((B, Hq, N, v.shape[3]), dtype=np.float64)
    block = 256
    for b in range(B):
        for h in range(Hq):
            kk_all = np.asarray(k[b, h // G], dtype=np.float64)
            vv_all = np.asarray(v[b, h // G], dtype=np.float64)
            qq_all = np.asarray(q[b, h], dtype=np.float64)
            for i0 in range(0, N, block):
                i1 = min(N, i0 + block) - 1
                lo, hi = max(0, i0 - left), min(N - 1, i1 + right)
                rows = np.arange(i0, i1 + 1)
                keys = np.arange(lo, hi + 1)
                allowed = (keys[None, :] >= rows[:, None] - left) & (keys[None, :] <= rows[:, None] + right)
                scores = scale * (qq_all[i0:i1 + 1] @ kk_all[lo:hi + 1].T)
                out[b, h, i0:i1 + 1] = _masked_softmax_rows(scores, allowed) @ vv_all[lo:hi + 1]
    return out


def diff_attn_fwd(q1, k1, q2, k2, v, lam, window: int, scale: Optional[float] = None) -> np.ndarray:
    """Differential sliding-window attention, float64 [B, Hq, N, d]:
    (A1 - lam[h] * A2) V with A1 = softmax(scale Q1 K1^T + M), A2 the same
    for (Q2, K2), M the causal band of width W, and lam an array of Hq
    scalars (attention-variants page, 第 4 步).  The difference of the two
    probability matrices is formed first, then multiplied by V."""
    q1, k1, q2, k2, v = (np.asarray(x) for x in (q1, k1, q2, k2, v))
    lam = np.asarray(lam, dtype=np.float64).reshape(-1)
    B, Hq, N, d = q1.shape
    if q2.shape != q1.shape or k1.shape != k2.shape or v.shape[:3] != k1.shape[:3] or lam.shape != (Hq,):
        raise ValueError("q1/q2, k1/k2/v or lam shapes do not match")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // k1.shape[1]
    out = np.empty((B, Hq, N, v.shape[3]), dtype=np.float64)
    block = 256
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i0 in range(0, N, block):
                i1 = min(N, i0 + block) - 1
                rows = np.arange(i0, i1 + 1, dtype=np.int64)
                keys = _block_keys(i0, i1, window, 0)
                allowed = _row_allowed(rows, keys, window, 0)
                a1 = _masked_softmax_rows(scale * (np.asarray(q1[b, h, i0:i1 + 1], np.float64)
                                                   @ np.asarray(k1[b, g][keys], np.float64).T), allowed)
                a2 = _masked_softmax_rows(scale * (np.asarray(q2[b, h, i0:i1 + 1], np.float64)
                                                   @ np.asarray(k2[b, g][keys], np.float64).T), allowed)
                out[b, h, i0:i1 + 1] = (a1 - lam[h] * a2) @ np.asarray(v[b, g][keys], np.float64)
    return out


def allowed_mask_global(n: int, window: int, gidx) -> np.ndarray:
    """Boolean n x n matrix of the causal local + global pattern: (i, j)
    allowed iff j <= i and (i - j < W or j in gidx or i in gidx)."""
    if window < 1:
        raise ValueError("window must be >= 1")
    glob = np.zeros(n, dtype=bool)
    glob[np.asarray(list(gidx), dtype=np.int64)] = True
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & ((i - j < window) | glob[None, :] | glob[:, None])


def attn_fwd_global(q, k, v, window: int, gidx, scale: Optional[float] = None) -> np.ndarray:
    """Causal sliding window plus global positions gidx, float64
    [B, Hq, N, d]: global rows read every earlier key, every row reads the
    earlier global keys, other pairs follow the band."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or v.shape != k.shape or Hq % k.shape[1] != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hq a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    g = np.asarray(sorted(set(int(x) for x in gidx)), dtype=np.int64)
    glob = np.zeros(N, dtype=bool)
    glob[g] = True
    G = Hq // k.shape[1]
    out = np.empty((B, Hq, N, v.shape[3]), dtype=np.float64)
    block = 256
    for b in range(B):
        for h in range(Hq):
            kk = np.asarray(k[b, h // G], dtype=np.float64)
            vv = np.asarray(v[b, h // G], dtype=np.float64)
            for i0 in range(0, N, block):
                i1 = min(N, i0 + block) - 1
                rows = np.arange(i0, i1 + 1)
                keys = np.arange(0, i1 + 1)
                i = rows[:, None]
                j = keys[None, :]
                allowed = (j <= i) & ((i - j < window) | glob[None, :i1 + 1] | glob[i0:i1 + 1, None])
                scores = scale * (np.asarray(q[b, h, i0:i1 + 1], dtype=np.float64) @ kk[:i1 + 1].T)
                out[b, h, i0:i1 + 1] = _masked_softmax_rows(scores, allowed) @ vv[:i1 + 1]
    return out
