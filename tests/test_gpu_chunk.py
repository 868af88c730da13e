"""GPU parity of the rolling-cache prefill path: ring append (bit-exact
against the oracle) and chunked prefill over the ring history (against the
float64 oracle, and chunk by chunk against the oracle's whole-sequence
prefill).  Tolerances as for the band kernel: fp32 max |err| <= 1e-5; bf16
max |err| <= 1.5e-2 and mean |err| <= 1e-3.  Each case prints its name
before it touches the GPU."""
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


def _dt(name):
    return torch.float32 if name == "f32" else torch.bfloat16


def _read_slots(p0, W):
    """Ring slots a chunk starting after p0 cached positions reads."""
    n = min(p0, W - 1)
    return {oracle.ring_slot(t, W) for t in range(p0 - n + 1, p0 + 1)}


def _nan_unread(kr, vr, p0s, W):
    for b, p in enumerate(p0s):
        used = _read_slots(p, W)
        for s in range(W):
            if s not in used:
                kr[b, :, s] = float("nan")
                vr[b, :, s] = float("nan")


# ---------------------------------------------------------------- ring append
@pytest.mark.parametrize("dtype,d,W,T,p0s", [
    ("bf16", 128, 64, 1, [0, 63, 64, 1000]),
    ("bf16", 128, 64, 100, [0, 5, 64]),       # chunk longer than the ring: last 64 rows survive
    ("bf16", 64, 100, 37, [90, 0, 12345]),    # wraps around the end of the ring
    ("f32", 64, 33, 33, [0, 1, 32]),
    ("f32", 128, 4096, 300, [4000, 0]),
])
def test_ring_append_bit_exact(dtype, d, W, T, p0s):
    say(f"ring_append {dtype} d={d} W={W} T={T} p0={p0s}")
    dt = _dt(dtype)
    B, Hkv = len(p0s), 3
    g = torch.Generator().manual_seed(W * 7 + T)
    k = torch.randn(B, Hkv, T, d, generator=g).to(dt)
    v = torch.randn(B, Hkv, T, d, generator=g).to(dt)
    kr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
    vr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
    p0 = torch.tensor(p0s, dtype=torch.int32)
    want_k, want_v = oracle.ring_append(f64(kr), f64(vr), f64(k), f64(v), p0s, W)
    krd, vrd = kr.to(DEV), vr.to(DEV)
    swa.ring_append(k.to(DEV), v.to(DEV), p0.to(DEV), krd, vrd)
    torch.cuda.synchronize()
    assert np.array_equal(f64(krd), want_k)
    assert np.array_equal(f64(vrd), want_v)


# ---------------------------------------------------------------- chunked prefill
@pytest.mark.parametrize("dtype,d,G,W,T,p0s", [
    ("f32", 64, 1, 32, 100, [0, 7, 31, 32, 500]),
    ("f32", 128, 4, 128, 129, [0, 127, 128, 300]),
    ("bf16", 128, 4, 256, 300, [0, 1, 255, 256, 10000]),
    ("bf16", 64, 2, 100, 1, [0, 1, 99, 100, 101, 777]),   # one new token per sequence
    ("bf16", 128, 8, 64, 200, [3, 64]),                   # chunk longer than the window
    ("bf16", 64, 1, 1, 17, [0, 5]),                       # window 1: each row reads itself only
    ("f32", 64, 2, 1000, 70, [0, 999, 2500]),
    # 8-wave kernel: d = 64, history lengths not multiples of the 64-key tile
    ("bf16", 64, 4, 200, 150, [0, 2, 70, 199, 200, 5000]),
    # 8-wave kernel: the history wraps around the ring's end inside a tile
    ("bf16", 128, 4, 1000, 130, [0, 999, 1500, 2500]),
    # 8-wave kernel: a history of exactly two tiles (no placeholder keys)
    ("bf16", 128, 4, 129, 100, [128, 129, 1000]),
    # 8-wave kernel with several head groups per KV head (6 and 16 query heads)
    ("bf16", 64, 6, 300, 280, [0, 150, 299, 5000]),
    ("bf16", 128, 6, 200, 260, [0, 77, 1000]),
    ("bf16", 128, 16, 257, 270, [0, 300, 1000]),
    ("bf16", 64, 16, 90, 300, [5, 89]),
])
def test_chunk_prefill_vs_oracle(dtype, d, G, W, T, p0s):
    say(f"chunk_prefill {dtype} d={d} G={G} W={W} T={T} p0={p0s}")
    dt = _dt(dtype)
    B, Hkv = len(p0s), 2
    Hq = G * Hkv
    g = torch.Generator().manual_seed(1000 * G + W + T)
    q = torch.randn(B, Hq, T, d, generator=g).to(dt)
    k = torch.randn(B, Hkv, T, d, generator=g).to(dt)
    v = torch.randn(B, Hkv, T, d, generator=g).to(dt)
    kr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
    vr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
    _nan_unread(kr, vr, p0s, W)  # slots the step must not read hold NaN
    p0 = torch.tensor(p0s, dtype=torch.int32)
    out = swa.chunk_prefill(q.to(DEV), k.to(DEV), v.to(DEV), kr.to(DEV), vr.to(DEV), p0.to(DEV))
    torch.cuda.synchronize()
    want = oracle.chunk_prefill(f64(q), f64(k), f64(v), f64(kr), f64(vr), p0s, W, 1 / math.sqrt(d))
    check(out, want, dt, f"{dtype} W={W} T={T}")


@pytest.mark.parametrize("dtype,W,chunks", [
    ("f32", 64, [1, 37, 64, 200, 5, 130]),
    ("bf16", 256, [300, 1, 255, 512, 2]),
    ("f32", 16, [16, 16, 3, 40]),
])
def test_chunked_sequence_equals_whole_prefill(dtype, W, chunks):
    """Attend, then append, chunk after chunk through the HIP path; the rows
    match the oracle's prefill of the whole sequence."""
    say(f"chunked sequence {dtype} W={W} chunks={chunks}")
    dt = _dt(dtype)
    B, Hq, Hkv, d = 2, 4, 2, 64
    L = sum(chunks)
    q, k, v = inputs.random_qkv(B, Hq, Hkv, L, d, dt, seed=W + L)
    whole = oracle.attn_fwd(f64(q), f64(k), f64(v), W)
    kr = torch.full((B, Hkv, W, d), float("nan"), dtype=dt, device=DEV)
    vr = torch.full((B, Hkv, W, d), float("nan"), dtype=dt, device=DEV)
    p0 = 0
    outs = []
    for T in chunks:
        sl = slice(p0, p0 + T)
        qc, kc, vc = (x[:, :, sl].contiguous().to(DEV) for x in (q, k, v))
        pd = torch.full((B,), p0, dtype=torch.int32, device=DEV)
        outs.append(swa.chunk_prefill(qc, kc, vc, kr, vr, pd))
        swa.ring_append(kc, vc, pd, kr, vr)
        p0 += T
    torch.cuda.synchronize()
    check(torch.cat(outs, 2), whole, dt, "chunked vs whole")


def test_one_token_chunk_matches_decode():
    """A one-token chunk before its append reads the same keys as the decode
    step after it (both kernels, fp32)."""
    say("one-token chunk vs decode")
    B, Hq, Hkv, d, W = 3, 8, 2, 128, 96
    g = torch.Generator().manual_seed(5)
    q = torch.randn(B, Hq, 1, d, generator=g)
    k = torch.randn(B, Hkv, 1, d, generator=g)
    v = torch.randn(B, Hkv, 1, d, generator=g)
    kr = torch.randn(B, Hkv, W, d, generator=g).to(DEV)
    vr = torch.randn(B, Hkv, W, d, generator=g).to(DEV)
    p0 = torch.tensor([0, 40, 5000], dtype=torch.int32, device=DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = swa.chunk_prefill(qd, kd, vd, kr, vr, p0)
    swa.ring_append(kd, vd, p0, kr, vr)
    b = swa.decode(qd[:, :, 0].contiguous(), kr, vr, p0 + 1)
    torch.cuda.synchronize()
    assert (a[:, :, 0] - b).abs().max().item() <= 1e-5


def test_chunk_config_full_parity():
    """The benchmarked chunk workload at full size: every output element of
    every (sequence, head) against the float64 oracle (one (sequence, head)
    per task on the host's cores), written into a NaN-filled buffer so a row
    the kernel never writes fails."""
    cfg = inputs.CHUNK
    say(f"{cfg.name} (whole output)")
    q, k, v, kr, vr, p0 = inputs.chunk_inputs(cfg)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    swa.chunk_prefill(q.to(DEV), k.to(DEV), v.to(DEV), kr.to(DEV), vr.to(DEV), p0.to(DEV), out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out
    qf, kf, vf, krf, vrf = (x.float().numpy() for x in (q, k, v, kr, vr))
    G, scale = cfg.Hq // cfg.Hkv, 1 / math.sqrt(cfg.d)

    def want(bh):
        b, h = bh
        g = slice(h // G, h // G + 1)
        return oracle.chunk_prefill(qf[b:b + 1, h:h + 1], kf[b:b + 1, g], vf[b:b + 1, g], krf[b:b + 1, g],
                                    vrf[b:b + 1, g], [cfg.p0[b]], cfg.window, scale)[0, 0]

    st = full_parity.compare_heads([(b, h) for b in range(cfg.B) for h in range(cfg.Hq)],
                                   lambda bh: got[bh[0], bh[1]], want)
    print(f"{cfg.name}: {st.count} elements, max |err| {st.max_err:.3e}, mean {st.mean_err:.3e}", flush=True)
    full_parity.assert_bf16(st, cfg.name)
