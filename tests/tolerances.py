"""Tolerances of the parity tests against the float64 oracle (shared by the
GPU test modules; no GPU needed to import).

The bars are the ones the workloads are specified with: fp32 outputs
max |err| <= 1e-5; bf16 outputs max |err| <= 1.5e-2 and mean |err| <= 1e-3
(fp32 accumulation inside).

Element bound for bf16 outputs.  A bf16 output is the kernel's fp32 value
rounded once, which alone costs up to half an ulp of the result: 2^-8 below
|x| = 2, 2^-7 in [2, 4), 2^-6 = 1.56e-2 in [4, 8).  The flat 1.5e-2 therefore
holds for |want| < 4, leaving 1.5e-2 - 2^-7 (about 7.2e-3) for the kernel's
own arithmetic (the bf16-rounded probabilities and the fp32 sums) after the
largest rounding it must absorb.  From |want| = 4 on the rounding alone
exceeds the flat bound (small windows return near-copies of V rows, which
reach 4 and more), so there an element may differ by that same arithmetic
budget plus its own half ulp: 2.28e-2 in [4, 8), 3.84e-2 in [8, 16).

Mean bound for the small-window sweeps.  Where a row reads one or two keys
its output is a near-copy of V rows (|x| ~ 0.7 on average), and rounding the
exact value once to bf16 already costs ~9.5e-4 on average, nearly the whole
1e-3.  There the bound is on the kernel's error in excess of that rounding:
mean |got - want| <= 1e-3 + mean |bf16(want) - want|.  The configured
workloads (long windows, small outputs: the rounding share is ~2e-4) keep the
flat 1e-3.
"""
import numpy as np

F32_MAX = 1e-5
BF16_MAX = 1.5e-2
BF16_MEAN = 1e-3
BF16_ARITH = BF16_MAX - 2.0 ** -7


def bf16_rounding_mean(want: np.ndarray) -> float:
    """mean |bf16(want) - want|: what rounding the exact values once to bf16
    (round to nearest even, through float32) costs on average."""
    import torch

    w = np.asarray(want, dtype=np.float64)
    r = torch.from_numpy(w).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    return float(np.abs(r - w).mean())


def bf16_mean_bound(want: np.ndarray) -> float:
    """Mean |err| bound of the small-window sweeps (see the module text)."""
    return BF16_MEAN + bf16_rounding_mean(want)


def bf16_element_bound(want: np.ndarray) -> np.ndarray:
    """Per-element |got - want| bound for a bf16 output (see the module text)."""
    a = np.abs(np.asarray(want, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    half_ulp = 2.0 ** (e - 8)
    return np.where(a >= 4.0, BF16_ARITH + half_ulp, BF16_MAX)
