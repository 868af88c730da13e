"""GPU parity of differential sliding-window attention, (A1 - lam*A2) V,
against the float64 oracle (fp32 and bf16, both band kernels), plus the
identities the entry point must keep: lam = 0 equals the single band map
bitwise, and identical Q/K pairs give (1 - lam) times it."""
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


def _inputs(B, Hq, Hkv, N, d, dt, seed):
    q1, k1, v = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed)
    q2, k2, _ = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed + 1000)
    g = torch.Generator().manual_seed(seed)
    lam = 0.5 + 0.3 * torch.rand(Hq, generator=g)  # the pages' typical range 0.5-0.8
    return q1, k1, q2, k2, v, lam


@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,d,W", [
    ("f32", 1, 2, 1, 200, 64, 33),
    ("f32", 2, 4, 2, 130, 128, 64),
    ("bf16", 1, 8, 2, 1000, 128, 256),   # 8-wave kernel
    ("bf16", 2, 4, 4, 333, 64, 100),     # 4-wave kernel
    ("bf16", 1, 4, 1, 77, 128, 4096),    # window beyond the sequence: the pages' causal form
])
def test_diff_vs_oracle(dtype, B, Hq, Hkv, N, d, W):
    say(f"diff {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} W={W}")
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q1, k1, q2, k2, v, lam = _inputs(B, Hq, Hkv, N, d, dt, seed=N + W)
    out = swa.diff_attn_fwd(*(x.to(DEV) for x in (q1, k1, q2, k2, v, lam)), window=W)
    torch.cuda.synchronize()
    want = oracle.diff_attn_fwd(f64(q1), f64(k1), f64(q2), f64(k2), f64(v), lam.double().numpy(), W)
    err = np.abs(f64(out) - want)
    assert np.isfinite(f64(out)).all()
    if dt == torch.float32:
        assert err.max() <= 1e-5, err.max()
    else:
        assert err.max() <= 1.5e-2 and err.mean() <= 1e-3, (err.max(), err.mean())


def test_diff_zero_lambda_is_the_band_map_bitwise():
    say("diff lam=0")
    for dt in (torch.float32, torch.bfloat16):
        q1, k1, q2, k2, v, _ = _inputs(1, 8, 2, 300, 128, dt, seed=3)
        lam = torch.zeros(8)
        a = swa.diff_attn_fwd(*(x.to(DEV) for x in (q1, k1, q2, k2, v, lam)), window=50)
        b = swa.attn_fwd(q1.to(DEV), k1.to(DEV), v.to(DEV), window=50)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_diff_identical_pairs_scale_by_one_minus_lambda():
    say("diff identical maps")
    q1, k1, _, _, v, lam = _inputs(1, 4, 2, 257, 64, torch.float32, seed=4)
    out = swa.diff_attn_fwd(*(x.to(DEV) for x in (q1, k1, q1, k1, v, lam)), window=40)
    one = swa.attn_fwd(q1.to(DEV), k1.to(DEV), v.to(DEV), window=40)
    torch.cuda.synchronize()
    want = (1 - lam.to(DEV))[None, :, None, None] * one
    assert (out - want).abs().max().item() <= 2e-6
