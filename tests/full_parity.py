"""Whole-output comparison of a kernel result with the float64 oracle.

The oracle is run one (batch, head) at a time on a pool of threads: numpy
releases the interpreter lock inside its array kernels, and BLAS is held to
one thread per task, so the pool spreads over the host cores without
forking the GPU-initialised test process.  Each task returns only error
statistics (max, sum, count over the bound, finiteness), never the float64
rows themselves, so memory stays at a few heads' worth.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, Iterable

import numpy as np

from tolerances import BF16_MAX, BF16_MEAN


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


@dataclass
class ErrStats:
    max_err: float = 0.0
    sum_err: float = 0.0
    count: int = 0
    over: int = 0
    nonfinite: int = 0
    worst: tuple = ()

    @property
    def mean_err(self) -> float:
        return self.sum_err / max(1, self.count)

    def add(self, other: "ErrStats"):
        if other.max_err > self.max_err:
            self.max_err, self.worst = other.max_err, other.worst
        self.sum_err += other.sum_err
        self.count += other.count
        self.over += other.over
        self.nonfinite += other.nonfinite


def head_stats(got: np.ndarray, want: np.ndarray, tol: float, key) -> ErrStats:
    """Error statistics of one head's rows: got (any real dtype) vs want (float64)."""
    g = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(g)
    err = np.abs(g - want)
    err = np.where(fin, err, np.inf)
    i = int(np.argmax(err))
    row = i // err.shape[-1] if err.ndim > 1 else i
    return ErrStats(max_err=float(err.flat[i]), sum_err=float(np.where(fin, err, 0.0).sum()),
                    count=int(err.size), over=int((err > tol).sum()), nonfinite=int((~fin).sum()),
                    worst=(*key, row))


def compare_heads(keys: Iterable, got_of: Callable, want_of: Callable, tol: float = BF16_MAX) -> ErrStats:
    """For every key (e.g. (b, h)) compare got_of(key) with the oracle's
    want_of(key) on the thread pool; returns the summed statistics."""
    from threadpoolctl import threadpool_limits

    def job(key):
        return head_stats(got_of(key), want_of(key), tol, key)

    total = ErrStats()
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers()) as ex:
        for st in ex.map(job, list(keys)):
            total.add(st)
    return total


def assert_bf16(st: ErrStats, what: str):
    assert st.nonfinite == 0, f"{what}: {st.nonfinite} non-finite outputs (unwritten rows?)"
    assert st.over == 0 and st.mean_err <= BF16_MEAN, (
        f"{what}: max {st.max_err:.3e} at (b, h, row) {st.worst}, mean {st.mean_err:.3e}, "
        f"{st.over} of {st.count} elements over {BF16_MAX}")
