"""Seeded random configurations of every prefill entry point against the
float64 oracle: band, local+strided, two-sided band, global tokens,
differential attention and chunked prefill over a ring, with ragged
sequence lengths, group sizes 1..8, head dims 64 and 128, fp32 and bf16.
Each case prints its parameters before it touches the GPU.

Tolerances as in the other parity tests (tests/tolerances.py): fp32 max
|err| <= 1e-5; bf16 max |err| <= 1.5e-2 and mean |err| <= 1e-3, except that
small windows return near-copies of V rows, where rounding the exact value
to bf16 alone costs 2^-6 per element of magnitude 4 or more and ~1e-3 on
average: an element there may differ by its half ulp plus the flat bound's
arithmetic share, and the mean bound applies to the error in excess of that
rounding.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_causal_attention_band_amd as swa
from tolerances import F32_MAX, bf16_element_bound, bf16_mean_bound
from sparse_causal_attention_band_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KINDS = ("band", "strided", "two_sided", "global", "diff", "chunk")
NCASES = 48


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    swa.lib()
    yield
    torch.cuda.synchronize()


def f64(t):
    return t.detach().cpu().double().numpy()


def check(got, want, dtype, what):
    g = f64(got)
    assert np.isfinite(g).all(), what
    err = np.abs(g - want)
    if dtype == torch.float32:
        assert err.max() <= F32_MAX, f"{what}: max err {err.max():.3e}"
        return
    worst = np.max(err - bf16_element_bound(want))
    assert worst <= 0, f"{what}: max err {err.max():.3e} (over the bound by {worst:.3e})"
    assert err.mean() <= bf16_mean_bound(want), f"{what}: mean err {err.mean():.3e}"


def draw(i):
    """Parameters of case i (a pure function of i)."""
    rng = np.random.default_rng(20261203 + i)
    kind = KINDS[i % len(KINDS)]
    dt = torch.float32 if (i // len(KINDS)) % 2 else torch.bfloat16
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 8] if kind == "global" else [1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 3))
    N = int(rng.integers(1, 301))
    c = dict(kind=kind, dt=dt, d=d, Hkv=Hkv, Hq=G * Hkv, B=B, N=N, seed=1000 + i)
    if kind in ("band", "diff"):
        c["W"] = int(rng.integers(1, N + 41))
    elif kind == "strided":
        c["W"] = int(rng.integers(1, 65))
        c["stride"] = int(rng.integers(1, 101))
    elif kind == "two_sided":
        c["left"] = int(rng.integers(0, N + 1))
        c["right"] = int(rng.integers(0, N + 1))
    elif kind == "global":
        c["W"] = int(rng.integers(1, 65))
        ng = int(rng.integers(0, min(N, 6) + 1))
        c["gidx"] = sorted(rng.choice(N, size=ng, replace=False).tolist())
    else:  # chunk
        W = int(rng.integers(1, 201))
        c["W"] = W
        c["p0"] = [int(rng.choice([0, rng.integers(1, 2 * W + 1), rng.integers(2 * W, 10 ** 6)])) for _ in range(B)]
    return c


@pytest.mark.parametrize("i", range(NCASES))
def test_random_case(i):
    c = draw(i)
    shown = {k: (v if k != "dt" else str(v).split(".")[-1]) for k, v in c.items()}
    say(f"random {i}: {shown}")
    dt, d, B, Hq, Hkv, N = c["dt"], c["d"], c["B"], c["Hq"], c["Hkv"], c["N"]
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed=c["seed"])
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1 / math.sqrt(d)
    kind = c["kind"]
    if kind in ("band", "strided"):
        stride = c.get("stride", 0)
        out = swa.attn_fwd(qd, kd, vd, window=c["W"], stride=stride)
        want = oracle.attn_fwd(f64(q), f64(k), f64(v), c["W"], stride, scale)
    elif kind == "two_sided":
        out = swa.attn_fwd_two_sided(qd, kd, vd, c["left"], c["right"])
        want = oracle.attn_fwd_two_sided(f64(q), f64(k), f64(v), c["left"], c["right"], scale)
    elif kind == "global":
        gi = torch.tensor(c["gidx"], dtype=torch.int32, device=DEV)
        out = swa.attn_fwd_global(qd, kd, vd, c["W"], gi)
        want = oracle.attn_fwd_global(f64(q), f64(k), f64(v), c["W"], c["gidx"], scale)
    elif kind == "diff":
        q2, k2, _ = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed=c["seed"] + 500)
        lam = torch.from_numpy(np.random.default_rng(c["seed"]).uniform(0.0, 1.0, Hq).astype(np.float32))
        out = swa.diff_attn_fwd(qd, kd, q2.to(DEV), k2.to(DEV), vd, lam.to(DEV), window=c["W"])
        want = oracle.diff_attn_fwd(f64(q), f64(k), f64(q2), f64(k2), f64(v), lam.double().numpy(), c["W"], scale)
    else:
        W = c["W"]
        _, kr, vr = inputs.random_qkv(B, Hkv, Hkv, W, d, dt, seed=c["seed"] + 700)
        p0 = torch.tensor(c["p0"], dtype=torch.int32)
        out = swa.chunk_prefill(qd, kd, vd, kr.to(DEV), vr.to(DEV), p0.to(DEV))
        want = oracle.chunk_prefill(f64(q), f64(k), f64(v), f64(kr), f64(vr), c["p0"], W, scale)
    torch.cuda.synchronize()
    check(out, want, dt, f"random {i} ({kind})")
