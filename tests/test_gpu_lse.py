"""GPU parity of the row log-sum-exp (the natural log of each row's softmax
denominator) returned with the band forward and with chunked prefill,
against the float64 oracle.

Tolerances.  fp32: |err| <= 2e-5 (the denominator is summed in fp32 from
exponentials taken in the log2 domain).  bf16: the denominator is the sum of
the bf16-rounded probabilities the product uses, each within a relative
2^-9 of its exact value, so the sum is too and its log moves by at most
2^-9 ~ 1.95e-3; the bound is 2.5e-3.  The output written together with the
log-sum-exp must be bitwise the output of the plain entry point.
Each case prints its parameters before it touches the GPU."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_causal_attention_band_amd as swa
from sparse_causal_attention_band_amd import inputs

import full_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.float32: 2e-5, torch.bfloat16: 2.5e-3}


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


# (B, Hq, Hkv, N, d, W, stride): 8-wave band kernel (Hq/Hkv = 2, 4, 8), 4-wave
# kernel (one head per KV head, strided), ragged ends and W >= N
SHAPES = [(1, 8, 2, 300, 128, 100, 0), (2, 8, 1, 257, 128, 64, 0), (1, 4, 4, 200, 64, 33, 0),
          (1, 4, 2, 513, 128, 200, 0), (1, 2, 2, 260, 64, 20, 16), (1, 8, 2, 100, 64, 500, 0),
          (1, 16, 2, 129, 128, 1, 0)]


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}_W{}_s{}".format(*s))
def test_band_lse_matches_oracle(shape, dt):
    B, Hq, Hkv, N, d, W, stride = shape
    say(f"band lse {shape} {dt}")
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed=N + W)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1 / math.sqrt(d)
    out, lse = swa.attn_fwd(qd, kd, vd, window=W, stride=stride, return_lse=True)
    plain = swa.attn_fwd(qd, kd, vd, window=W, stride=stride)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    want = oracle.attn_lse(f64(q), f64(k), W, stride, scale)
    got = f64(lse)
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= TOL[dt], f"max |lse err| {err:.3e}"


def test_band_lse_negative_scale_and_mistral_rows():
    """A negative scale (the sign enters through q), and every row of the
    Mistral-shaped workload in the launch configuration the bench times,
    against the oracle's log-sum-exp (one head per task on the host's cores)."""
    say("band lse negative scale")
    q, k, v = inputs.random_qkv(1, 8, 2, 300, 128, torch.bfloat16, seed=3)
    out, lse = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=77, scale=-0.09, return_lse=True)
    torch.cuda.synchronize()
    assert np.abs(f64(lse) - oracle.attn_lse(f64(q), f64(k), 77, 0, -0.09)).max() <= TOL[torch.bfloat16]
    say("band lse mistral, every row")
    cfg = inputs.MISTRAL
    q, k, v = inputs.prefill_inputs(cfg)
    out, lse = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=cfg.window, return_lse=True)
    torch.cuda.synchronize()
    lse = f64(lse)
    qf, kf = q.float().numpy(), k.float().numpy()
    G, scale = cfg.Hq // cfg.Hkv, 1 / math.sqrt(cfg.d)
    st = full_parity.compare_heads(
        [(0, h) for h in range(cfg.Hq)], lambda bh: lse[0, bh[1]],
        lambda bh: oracle.attn_lse(qf[:, bh[1]:bh[1] + 1], kf[:, bh[1] // G:bh[1] // G + 1], cfg.window, 0,
                                   scale)[0, 0], tol=TOL[torch.bfloat16])
    assert st.nonfinite == 0 and st.over == 0, (st.max_err, st.worst)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("G,d,W,T,p0", [(4, 128, 64, 100, [0, 37, 500]), (2, 64, 40, 70, [5, 90, 1000]),
                                        (8, 128, 200, 130, [199, 3, 64])])
def test_chunk_lse_matches_oracle(G, d, W, T, p0, dt):
    say(f"chunk lse G{G} d{d} W{W} T{T} p0{p0} {dt}")
    B, Hkv = len(p0), 2
    Hq = G * Hkv
    q, k, v = inputs.random_qkv(B, Hq, Hkv, T, d, dt, seed=T + W)
    _, kr, vr = inputs.random_qkv(B, Hkv, Hkv, W, d, dt, seed=T + W + 1)
    pos = torch.tensor(p0, dtype=torch.int32)
    out, lse = swa.chunk_prefill(q.to(DEV), k.to(DEV), v.to(DEV), kr.to(DEV), vr.to(DEV), pos.to(DEV),
                                 return_lse=True)
    plain = swa.chunk_prefill(q.to(DEV), k.to(DEV), v.to(DEV), kr.to(DEV), vr.to(DEV), pos.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    want = oracle.chunk_prefill_lse(f64(q), f64(k), f64(kr), p0, W, 1 / math.sqrt(d))
    err = np.abs(f64(lse) - want).max()
    assert err <= TOL[dt], f"max |lse err| {err:.3e}"


def test_lse_merges_two_key_sets_into_the_whole():
    """The use the log-sum-exp is for.  Under full causal attention the rows
    of the second half read keys 0..i; split those keys into the first half
    (every such row reads all of it: computed here in float64 with its
    log-sum-exp) and the second half's own keys (the kernel's forward over
    the second half of the sequence alone, with its log-sum-exp).  Merging
    the two results with weights exp(lse_x - lse) must give the kernel's
    forward over the whole sequence, and the merged log-sum-exp its lse."""
    say("lse merge")
    B, Hq, Hkv, N, d = 1, 4, 1, 192, 64
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, torch.float32, seed=11)
    half = N // 2
    full, lse_full = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=N, return_lse=True)
    # second half on its own: its rows read keys half..i only
    o2, l2 = swa.attn_fwd(q[:, :, half:].contiguous().to(DEV), k[:, :, half:].contiguous().to(DEV),
                          v[:, :, half:].contiguous().to(DEV), window=N, return_lse=True)
    torch.cuda.synchronize()
    # first half's keys for those rows: every row reads all of 0..half-1
    qf, kf, vf = f64(q), f64(k), f64(v)
    s1 = np.einsum("hid,jd->hij", qf[0, :, half:], kf[0, 0, :half]) / math.sqrt(d)
    m1 = s1.max(-1, keepdims=True)
    e1 = np.exp(s1 - m1)
    l1 = (m1[..., 0] + np.log(e1.sum(-1)))
    o1 = (e1 / e1.sum(-1, keepdims=True)) @ vf[0, 0, :half]
    L = np.logaddexp(l1, f64(l2)[0])
    merged = np.exp(l1 - L)[..., None] * o1 + np.exp(f64(l2)[0] - L)[..., None] * f64(o2)[0]
    assert np.abs(merged - f64(full)[0, :, half:]).max() <= 2e-5
    assert np.abs(L - f64(lse_full)[0, :, half:]).max() <= 2e-5
