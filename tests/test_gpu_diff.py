"""GPU parity of differential sliding-window attention, (A1 - lam*A2) V,
against the float64 oracle: the bf16 one-pass kernel (windows under 512:
both maps in one workgroup over one tile stream; group sizes 1 to 8, d 64
and 128, ragged ends, W = 1 and W >= N small N, and a Mistral-shaped
workload with W = 256 in full) and the two-launch path (fp32, and bf16 from
W = 512 on, including the benchmark's W = 4096 workload in full); plus the
identities the entry point must keep: lam = 0 equals the single band map
bitwise, and identical Q/K pairs give (1 - lam) times it."""
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


def _inputs(B, Hq, Hkv, N, d, dt, seed):
    q1, k1, v = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed)
    q2, k2, _ = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed + 1000)
    g = torch.Generator().manual_seed(seed)
    lam = 0.5 + 0.3 * torch.rand(Hq, generator=g)  # the pages' typical range 0.5-0.8
    return q1, k1, q2, k2, v, lam


@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,d,W", [
    ("f32", 1, 2, 1, 200, 64, 33),
    ("f32", 2, 4, 2, 130, 128, 64),
    ("bf16", 1, 8, 2, 1000, 128, 256),   # one pass: 4 heads per KV head, one query block per map
    ("bf16", 2, 4, 4, 333, 64, 100),     # one pass: one head per KV head, 4 blocks per map
    ("bf16", 1, 4, 1, 77, 128, 4096),    # window beyond the sequence (two launches): the pages' causal form
    ("bf16", 1, 4, 1, 77, 128, 300),     # the same rows in one pass (W >= N)
    ("bf16", 1, 4, 2, 700, 128, 300),    # two heads per KV head
    ("bf16", 1, 16, 2, 400, 128, 130),   # 8 heads per KV head: two head groups
    ("bf16", 2, 6, 2, 260, 64, 1),       # 3 heads per KV head, window 1
    ("bf16", 1, 2, 2, 1, 64, 5),         # one token
    ("bf16", 1, 8, 4, 2049, 64, 2049),   # full causal, ragged end
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


@pytest.mark.parametrize("window", [4096, 256], ids=["two_launch_w4096", "one_pass_w256"])
def test_diff_mistral_workload_full_parity(window):
    """The benchmark's differential leg (Mistral-shaped: B=1, 32/8 heads,
    d=128, N=16384; the second Q/K pair the position-reversed first pair,
    lam = linspace(0.5, 0.8) over the heads) at its W = 4096 (two launches)
    and at W = 256 (one pass): every output element against the float64
    oracle (one head per task on the host's cores), in a NaN-filled buffer."""
    cfg = inputs.MISTRAL
    say(f"diff mistral-shaped workload W={window} (whole output)")
    q, k, v = inputs.prefill_inputs(cfg)
    q2, k2 = q.flip(2).contiguous(), k.flip(2).contiguous()
    lam = torch.linspace(0.5, 0.8, cfg.Hq)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    swa.diff_attn_fwd(*(x.to(DEV) for x in (q, k, q2, k2, v, lam)), window=window, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out
    qf, kf, q2f, k2f, vf = (x.float().numpy() for x in (q, k, q2, k2, v))
    G, lamd = cfg.Hq // cfg.Hkv, lam.double().numpy()

    def want(bh):
        _, h = bh
        g = slice(h // G, h // G + 1)
        return oracle.diff_attn_fwd(qf[:, h:h + 1], kf[:, g], q2f[:, h:h + 1], k2f[:, g], vf[:, g],
                                    lamd[h:h + 1], window, 1 / math.sqrt(cfg.d))[0, 0]

    st = full_parity.compare_heads([(0, h) for h in range(cfg.Hq)], lambda bh: got[0, bh[1]], want)
    print(f"diff mistral W={window}: {st.count} elements, max |err| {st.max_err:.3e}, mean {st.mean_err:.3e}",
          flush=True)
    full_parity.assert_bf16(st, f"diff mistral W={window}")
