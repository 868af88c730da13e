"""Degenerate and boundary cases of every entry point, against the float64
oracle: one-token sequences, window 1, one global position, one-token chunks
over empty and very long histories, positions near the int32 limit, grids
with many sequences, and the head groupings the 8-wave kernel takes."""
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


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_one_token_sequences(dt):
    say(f"N=1 everywhere {dt}")
    q, k, v = inputs.random_qkv(3, 8, 2, 1, 128, dt, seed=51)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    outs = {
        "band": swa.attn_fwd(qd, kd, vd, window=7),
        "strided": swa.attn_fwd(qd, kd, vd, window=1, stride=3),
        "two_sided": swa.attn_fwd_two_sided(qd, kd, vd, 5, 5),
        "global": swa.attn_fwd_global(qd, kd, vd, 4, torch.zeros(1, dtype=torch.int32, device=DEV)),
        "diff": swa.diff_attn_fwd(qd, kd, qd, kd, vd, torch.full((8,), 0.5, device=DEV), 3),
    }
    torch.cuda.synchronize()
    # a single key: every variant returns V (the difference (1 - lam) V)
    want = np.repeat(f64(v), 4, axis=1)
    for name, o in outs.items():
        w = 0.5 * want if name == "diff" else want
        check(o, w, dt, name)


def test_many_sequences_and_the_8_wave_grouping():
    """B = 24 sequences, 16 query heads over 2 KV heads (8 per group: the
    8-wave kernel with 8 heads and one position block), ragged N."""
    say("B=24 G=8 ragged")
    q, k, v = inputs.random_qkv(24, 16, 2, 77, 64, torch.bfloat16, seed=52)
    out = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=20)
    torch.cuda.synchronize()
    check(out, oracle.attn_fwd(f64(q), f64(k), f64(v), 20), torch.bfloat16, "B=24")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_chunk_edges(dt):
    """One-token chunks with window 1 and window larger than the history,
    over an empty history and over one near the int32 limit."""
    say(f"chunk edges {dt}")
    B, Hq, Hkv, d = 3, 4, 2, 64
    for W, p0s in ((1, [0, 5, 2 ** 31 - 10]), (50, [0, 49, 2 ** 31 - 100])):
        g = torch.Generator().manual_seed(W)
        q = torch.randn(B, Hq, 1, d, generator=g).to(dt)
        k = torch.randn(B, Hkv, 1, d, generator=g).to(dt)
        v = torch.randn(B, Hkv, 1, d, generator=g).to(dt)
        kr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
        vr = torch.randn(B, Hkv, W, d, generator=g).to(dt)
        p0 = torch.tensor(p0s, dtype=torch.int32)
        out = swa.chunk_prefill(q.to(DEV), k.to(DEV), v.to(DEV), kr.to(DEV), vr.to(DEV), p0.to(DEV))
        krd, vrd = kr.to(DEV), vr.to(DEV)
        swa.ring_append(k.to(DEV), v.to(DEV), p0.to(DEV), krd, vrd)
        torch.cuda.synchronize()
        want = oracle.chunk_prefill(f64(q), f64(k), f64(v), f64(kr), f64(vr), p0s, W, 1 / math.sqrt(d))
        check(out, want, dt, f"W={W}")
        wk, wv = oracle.ring_append(f64(kr), f64(vr), f64(k), f64(v), p0s, W)
        assert np.array_equal(f64(krd), wk) and np.array_equal(f64(vrd), wv)


def test_decode_position_near_the_int32_limit():
    say("decode pos near 2^31")
    B, Hq, Hkv, d, W = 2, 8, 2, 128, 96
    g = torch.Generator().manual_seed(53)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    kr = torch.randn(B, Hkv, W, d, generator=g).to(torch.bfloat16)
    vr = torch.randn(B, Hkv, W, d, generator=g).to(torch.bfloat16)
    pos = torch.tensor([2 ** 31 - 1, 2 ** 31 - 97], dtype=torch.int32)
    out = swa.decode(q.to(DEV), kr.to(DEV), vr.to(DEV), pos.to(DEV))
    torch.cuda.synchronize()
    check(out, oracle.decode(f64(q), f64(kr), f64(vr), pos.numpy().astype(np.int64), W, 1 / math.sqrt(d)),
          torch.bfloat16, "pos")


def test_global_all_positions_and_last_position():
    say("global: every position, and only the last one")
    q, k, v = inputs.random_qkv(2, 4, 2, 70, 64, torch.float32, seed=54)
    for g in (list(range(70)), [69]):
        gi = torch.tensor(g, dtype=torch.int32, device=DEV)
        out = swa.attn_fwd_global(q.to(DEV), k.to(DEV), v.to(DEV), 5, gi)
        torch.cuda.synchronize()
        check(out, oracle.attn_fwd_global(f64(q), f64(k), f64(v), 5, g), torch.float32, f"ng={len(g)}")


def test_key_value_arrays_beyond_2_gib():
    """K and V of one head just past 2 GiB each (N = 2^23 + 100 rows of d=128
    bf16): the 8-wave kernel addresses an array with 32-bit byte offsets, so
    such shapes run on the 4-wave kernel, whose copies address rows by index.
    Sampled rows, the last ones beyond the 2 GiB offset included, against the
    oracle evaluated on each row's own key range; the same rows as a first
    chunk of a chunked prefill (no history, NaN ring) too."""
    N, d, W, Hq = 2 ** 23 + 100, 128, 64, 4
    say(f"N={N} Hq={Hq} Hkv=1 d={d} W={W} bf16 (~20 GiB on the device)")
    g = torch.Generator(device=DEV).manual_seed(55)
    q = torch.randn(1, Hq, N, d, generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn(1, 1, N, d, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(1, 1, N, d, generator=g, device=DEV).to(torch.bfloat16)
    assert k[0, 0].numel() * 2 >= 2 ** 31
    out = swa.attn_fwd(q, k, v, window=W)
    # the same rows as a first chunk (no history): chunk mode on the same path
    kr = torch.full((1, 1, W, d), float("nan"), device=DEV).to(torch.bfloat16)
    vr = torch.full((1, 1, W, d), float("nan"), device=DEV).to(torch.bfloat16)
    outc = swa.chunk_prefill(q, k, v, kr, vr, torch.zeros(1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 5000, 2 ** 22, 2 ** 23 - 1, 2 ** 23, 2 ** 23 + 37, N - 65, N - 2, N - 1]
    got, gotc, want = [], [], []
    for idx, i in enumerate(rows):
        h = idx % Hq
        lo = max(0, i - W + 1)
        qs = q[:, h:h + 1, i:i + 1].cpu().float().numpy()
        ks = k[:, :, lo:i + 1].cpu().float().numpy()
        vs = v[:, :, lo:i + 1].cpu().float().numpy()
        # the row's band is the whole slice: place the query at its last
        # position of a slice-length sequence
        L = i + 1 - lo
        qpad = np.zeros((1, 1, L, d))
        qpad[:, :, L - 1] = qs[:, :, 0]
        want.append(oracle.attn_fwd_rows(qpad, ks, vs, W, 0, 1 / math.sqrt(d), [(0, 0, L - 1)])[0])
        got.append(out[0, h, i].float().cpu())
        gotc.append(outc[0, h, i].float().cpu())
    del q, k, v, out, outc
    torch.cuda.empty_cache()
    check(torch.stack(got), np.stack(want), torch.bfloat16, "beyond 2 GiB")
    check(torch.stack(gotc), np.stack(want), torch.bfloat16, "beyond 2 GiB, chunk")


def test_key_split_with_every_score_very_negative():
    """bf16 local + strided with one query head per KV head runs the 4-wave
    kernel's key split.  With every score at about -277 in log2 units, the
    second key half of rows 0..31 meets no allowed key; merging the halves
    must give that half weight 0 (not underflow the other half to 0/0).
    All allowed keys have the same score, so every row is the mean of its
    allowed V rows."""
    say("key split, every score -192 (scale 3, q.k = -64)")
    N, d, W, stride = 200, 64, 40, 16
    q = torch.zeros(1, 2, N, d)
    q[..., 0] = 8.0
    k = torch.zeros(1, 2, N, d)
    k[..., 0] = -8.0
    _, _, v = inputs.random_qkv(1, 2, 2, N, d, torch.float32, seed=31)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    out = swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=W, stride=stride, scale=3.0)
    torch.cuda.synchronize()
    want = oracle.attn_fwd(f64(q), f64(k), f64(v), W, stride, 3.0)
    check(out, want, torch.bfloat16, "key split, very negative scores")
