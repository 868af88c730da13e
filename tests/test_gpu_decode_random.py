"""Seeded random decode steps against the float64 oracle: batch sizes 1-40
(so the split plan ranges from one split to many), 1-8 KV heads, 1, 2, 4 or
8 query heads per KV head, d 64 and 128, windows from a few slots to
thousands, positions below, at and past the window and pos <= 0, fp32 and
bf16, through the decode entry point with a workspace and, for bf16, the
allocation-free one.  Tolerances as in the other parity tests
(tests/tolerances.py).  Each case prints its parameters before it touches the
GPU."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_causal_attention_band_amd as swa
from tolerances import F32_MAX, bf16_element_bound, bf16_mean_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    swa.lib()
    yield
    torch.cuda.synchronize()


def draw(i):
    """Parameters and inputs of case i (a pure function of i)."""
    rng = np.random.default_rng(880000 + i)
    B = int(rng.integers(1, 41))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    W = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 5000))]))
    dt = torch.bfloat16 if i % 3 else torch.float32
    g = torch.Generator().manual_seed(880000 + i)
    q = torch.randn(B, G * Hkv, d, generator=g).to(dt)
    kr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
    vr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
    choices = [1, 2, max(1, W - 1), W, W + 1, int(rng.integers(1, 3 * W + 2)), 0]
    pos = torch.from_numpy(rng.choice(choices, size=B).astype(np.int32))
    return q, kr, vr, pos


def check(got, want, dt, what):
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all(), what
    err = np.abs(g - want)
    if dt == torch.float32:
        assert err.max() <= F32_MAX, f"{what}: max err {err.max():.3e}"
        return
    assert (err - bf16_element_bound(want)).max() <= 0, f"{what}: max err {err.max():.3e}"
    assert err.mean() <= bf16_mean_bound(want), f"{what}: mean err {err.mean():.3e}"


@pytest.mark.parametrize("i", [3, 17, 26, 41, 58, 77, 101, 137])
def test_random_decode_step(i):
    q, kr, vr, pos = draw(i)
    B, Hq, d = q.shape
    Hkv, W = kr.shape[1], kr.shape[2]
    print(f"[case] decode random {i}: B{B} Hq{Hq} Hkv{Hkv} d{d} W{W} {str(q.dtype)[6:]}", flush=True)
    sys.stdout.flush()
    want = oracle.decode(q.double().numpy(), kr.double().numpy(), vr.double().numpy(), pos.numpy(), W,
                         1 / math.sqrt(d))
    out = swa.decode(q.to(DEV), kr.to(DEV), vr.to(DEV), pos.to(DEV))
    torch.cuda.synchronize()
    check(out, want, q.dtype, f"decode {i}")
    if q.dtype == torch.bfloat16:
        out2 = swa.decode_noalloc(q.to(DEV), kr.to(DEV), vr.to(DEV), pos.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(out2, out), f"noalloc {i}"
