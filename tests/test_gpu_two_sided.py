"""GPU parity of the two-sided band (no causal cut) against the float64
oracle: sweeps over radii, ragged lengths and head groupings in fp32 and
bf16, exact allowed sets by one-hot key probes, and the two special cases
that reduce to other entry points (right = 0: causal band; both radii >= N:
full attention).  Tolerances as for the causal band."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_causal_attention_band_amd as swa
from sparse_causal_attention_band_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def check(got, want, dtype, what=""):
    g = f64(got)
    err = np.abs(g - want)
    assert np.isfinite(g).all(), what
    if dtype == torch.float32:
        assert err.max() <= 1e-5, f"{what}: max err {err.max():.3e}"
    else:
        assert err.max() <= 1.5e-2 and err.mean() <= 1e-3, f"{what}: max {err.max():.3e} mean {err.mean():.3e}"


@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,d,left,right", [
    ("f32", 1, 2, 1, 200, 64, 16, 16),
    ("f32", 2, 4, 2, 129, 128, 5, 40),
    ("f32", 1, 1, 1, 257, 64, 100, 0),
    ("bf16", 1, 8, 2, 1000, 128, 128, 128),   # 8-wave kernel (4 heads per KV head)
    ("bf16", 2, 4, 4, 333, 64, 63, 64),
    ("bf16", 1, 16, 4, 517, 128, 0, 90),       # right part only
    ("bf16", 1, 4, 2, 64, 128, 1000, 3),       # left beyond the sequence
])
def test_two_sided_vs_oracle(dtype, B, Hq, Hkv, N, d, left, right):
    say(f"two-sided {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} left={left} right={right}")
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed=N + left + 7 * right)
    out = swa.attn_fwd_two_sided(q.to(DEV), k.to(DEV), v.to(DEV), left, right)
    torch.cuda.synchronize()
    want = oracle.attn_fwd_two_sided(f64(q), f64(k), f64(v), left, right)
    check(out, want, dt, f"left={left} right={right}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,left,right", [(100, 7, 13), (130, 64, 1), (70, 0, 0), (96, 31, 33)])
def test_two_sided_exact_allowed_set(dtype, N, left, right):
    """One-hot key probes: with K = 0 except key j* (score +50 there), row i
    returns V[j*] exactly iff j* is allowed for i, and a mean of the other
    allowed values otherwise."""
    say(f"two-sided one-hot {dtype} N={N} left={left} right={right}")
    d, Hq = 64, 4
    allowed = oracle.allowed_mask_two_sided(N, left, right)
    v = torch.arange(N, dtype=torch.float32)[None, None, :, None].expand(1, 1, N, d).contiguous()
    q = torch.zeros(1, Hq, N, d)
    q[..., 0] = 1.0
    for jstar in sorted({0, 1, N // 2, N - 2, N - 1, min(left, N - 1), min(N - 1, right)}):
        k = torch.zeros(1, 1, N, d)
        k[0, 0, jstar, 0] = 50.0 * math.sqrt(d)
        out = swa.attn_fwd_two_sided(q.to(dtype).to(DEV), k.to(dtype).to(DEV), v.to(dtype).to(DEV), left, right)
        torch.cuda.synchronize()
        got = out[0, 0, :, 0].float().cpu().numpy()
        hit = np.abs(got - jstar) < 0.5 if dtype == torch.bfloat16 else np.abs(got - jstar) < 1e-3
        # rows that may read j* put all their weight there (e^50 dominates)
        assert np.array_equal(hit | ~allowed[:, jstar], np.ones(N, dtype=bool)), jstar
        # rows that may not read j* average their own keys: j* never shows
        for i in np.nonzero(~allowed[:, jstar])[0]:
            keys = np.nonzero(allowed[i])[0]
            assert abs(got[i] - keys.mean()) <= (1.0 if dtype == torch.bfloat16 else 1e-3), (i, jstar)


def test_two_sided_right_zero_is_the_causal_band_bitwise():
    say("two-sided right=0 vs swa_attn_fwd")
    for dt in (torch.float32, torch.bfloat16):
        q, k, v = inputs.random_qkv(1, 8, 2, 300, 128, dt, seed=5)
        a = swa.attn_fwd_two_sided(q.to(DEV), k.to(DEV), v.to(DEV), 40, 0)
        b = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=41)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_two_sided_full_width_is_full_attention():
    say("two-sided full width")
    q, k, v = inputs.random_qkv(1, 4, 4, 150, 64, torch.float32, seed=6)
    out = swa.attn_fwd_two_sided(q.to(DEV), k.to(DEV), v.to(DEV), 10 ** 6, 10 ** 6)
    torch.cuda.synchronize()
    want = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double()).numpy()
    check(out, want, torch.float32, "full width")
