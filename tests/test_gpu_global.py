"""GPU parity of the causal local window plus global tokens against the
float64 oracle (fp32 and bf16; one global token such as a leading [CLS], a
few scattered ones, global positions at the end, several sequences), and
the identities the entry point keeps: no global positions equals the band
bitwise; global rows equal full causal rows; global keys on a stride grid
give the other rows the local + strided result."""
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


def run(q, k, v, W, g):
    gi = torch.tensor(g, dtype=torch.int32, device=DEV)
    out = swa.attn_fwd_global(q.to(DEV), k.to(DEV), v.to(DEV), W, gi)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype,B,Hq,Hkv,N,d,W,g", [
    ("f32", 1, 2, 1, 300, 64, 32, [0]),                        # a leading [CLS]-like token
    ("f32", 2, 4, 2, 257, 128, 64, [0, 100, 101, 256]),
    ("bf16", 1, 8, 2, 1000, 128, 128, [0, 7, 500, 999]),
    ("bf16", 2, 4, 4, 333, 64, 50, [3, 64, 65, 128, 200, 332]),
    ("bf16", 1, 16, 2, 4096, 128, 256, [0, 1000, 2048, 4095]),  # long global rows: several decode splits
    ("f32", 1, 4, 1, 130, 64, 1, list(range(0, 130, 13))),     # window 1
    # bf16 with an even head group and at most 64 positions: the 8-wave
    # kernel, its compact tile below the band and global keys in its edge
    # tiles (2, 4 and 8 query heads per KV head, d 64 and 128, ragged ends)
    ("bf16", 1, 4, 2, 1200, 64, 100, [5, 70, 71, 130, 640, 641, 700, 1199]),
    ("bf16", 2, 8, 4, 777, 128, 200, list(range(3, 777, 61))),
    ("bf16", 1, 8, 1, 900, 128, 64, [0, 1, 63, 64, 65, 127, 128, 300, 450, 899]),
    ("bf16", 1, 16, 2, 1500, 64, 300, list(range(0, 1500, 97))),
    ("bf16", 1, 4, 1, 5000, 128, 257, list(range(7, 5000, 78))[:64]),   # 64 positions: the 8-wave limit
    ("bf16", 1, 4, 1, 5000, 128, 257, list(range(7, 5000, 76))[:65]),   # 65: the 4-wave kernel
])
def test_global_vs_oracle(dtype, B, Hq, Hkv, N, d, W, g):
    say(f"global {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} W={W} g={g}")
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, dt, seed=N + W + len(g))
    out = run(q, k, v, W, g)
    want = oracle.attn_fwd_global(f64(q), f64(k), f64(v), W, g)
    check(out, want, dt, f"W={W} g={g}")


def test_global_none_is_the_band_bitwise():
    say("global ng=0")
    for dt in (torch.float32, torch.bfloat16):
        q, k, v = inputs.random_qkv(1, 8, 2, 300, 128, dt, seed=8)
        a = swa.attn_fwd_global(q.to(DEV), k.to(DEV), v.to(DEV), 40, torch.zeros(0, dtype=torch.int32, device=DEV))
        b = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=40)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_global_rows_are_full_causal_rows_and_stride_grid_is_strided():
    say("global rows / stride grid")
    N, s = 600, 64
    g = list(range(0, N, s))
    q, k, v = inputs.random_qkv(1, 4, 2, N, 64, torch.float32, seed=9)
    out = run(q, k, v, 30, g)
    full = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=N)
    strided = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=30, stride=s)
    torch.cuda.synchronize()
    assert (out[:, :, g] - full[:, :, g]).abs().max().item() <= 1e-5
    rows = [i for i in range(N) if i % s]
    assert (out[:, :, rows] - strided[:, :, rows]).abs().max().item() <= 1e-5


def test_global_leg_full_parity():
    """The benchmark's global-token leg (Mistral shape: B 1, 32/8 heads,
    N 16384, d 128, W 4096, position 0 and every 1024th global), every
    output element against the float64 oracle, written into a NaN-filled
    buffer so that unwritten rows fail."""
    import math
    from tolerances import BF16_MAX
    import full_parity
    cfg = inputs.MISTRAL
    say(f"{cfg.name} with 16 global positions (whole output)")
    q, k, v = inputs.prefill_inputs(cfg)
    g = [0] + list(range(1024, cfg.N, 1024))
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    swa.attn_fwd_global(q.to(DEV), k.to(DEV), v.to(DEV), cfg.window, torch.tensor(g, dtype=torch.int32, device=DEV),
                        out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    G, scale = cfg.Hq // cfg.Hkv, 1 / math.sqrt(cfg.d)
    st = full_parity.compare_heads(
        [(0, h) for h in range(cfg.Hq)],
        lambda bh: got[0, bh[1]],
        lambda bh: oracle.attn_fwd_global(qf[:, bh[1]:bh[1] + 1], kf[:, bh[1] // G:bh[1] // G + 1],
                                          vf[:, bh[1] // G:bh[1] // G + 1], cfg.window, g, scale)[0, 0], BF16_MAX)
    print(f"global leg: {st.count} elements, max |err| {st.max_err:.3e}, mean {st.mean_err:.3e}", flush=True)
    full_parity.assert_bf16(st, "global leg")
