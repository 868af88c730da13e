"""GPU parity of the band kernel where each persistent workgroup runs several
query blocks and streams from one into the next (shapes with more query
blocks than CUs): every output element against the float64 oracle, in
NaN-filled buffers.  Cases: ragged sequence ends, windows of one key (blocks
with fewer than three tiles, padded with copy-only steps), 2, 4 and 8 query
heads per KV head, the two-sided band, a negative scale (the sign enters
through the queries, also those a block takes over from its predecessor's
staging), the row log-sum-exp, blocks whose successor lies in another head
or sequence, and seeded random shapes of the same kind.  Tolerances as in the other
parity tests (bf16: 1.5e-2 max, 1e-3 mean; log-sum-exp 2.5e-3).  Each case
prints its parameters before it touches the GPU."""
import math
import sys

import numpy as np
import pytest
import torch

import full_parity
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


def _compare(got, want_of, B, Hq, what, tol=1.5e-2):
    st = full_parity.compare_heads([(b, h) for b in range(B) for h in range(Hq)], lambda bh: got[bh[0], bh[1]],
                                   want_of, tol=tol)
    print(f"{what}: {st.count} elements, max |err| {st.max_err:.3e}, mean {st.mean_err:.3e}", flush=True)
    return st


# (B, Hq, Hkv, N, d, window, right, scale; 0: 1/sqrt(d))
CASES = [
    (1, 8, 2, 32768 - 37, 128, 100, 0, 0),    # 4 heads per KV head, ragged end, 1024 blocks
    (2, 4, 2, 16384 + 5, 64, 1, 0, 0),        # 2 heads per KV head, one key: blocks of 1-2 tiles
    (1, 16, 2, 20000, 128, 700, 0, 0),        # 8 heads per KV head: 32-row blocks
    (3, 8, 4, 5000, 128, 64, 0, 0),           # successors in other heads and sequences
    (1, 8, 2, 20000, 128, 201, 150, 0),       # two-sided band
    (2, 8, 2, 9000 + 3, 128, 150, 0, -0.11),  # negative scale, 564 blocks, ragged end
    (1, 8, 4, 17000, 64, 64, 0, -0.2),        # negative scale, d = 64, 532 blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_N{}_d{}_W{}_r{}_s{}".format(*c))
def test_streamed_blocks_match_oracle(case):
    B, Hq, Hkv, N, d, W, right, sc = case
    say(f"streamed band {case}")
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, torch.bfloat16, seed=N % 1000 + W)
    G, scale = Hq // Hkv, sc if sc else 1 / math.sqrt(d)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    if right:
        swa.attn_fwd_two_sided(q.to(DEV), k.to(DEV), v.to(DEV), W - 1, right, scale=scale, out=out)
    else:
        swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=W, scale=scale, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()

    def want(bh):
        b, h = bh
        g = slice(h // G, h // G + 1)
        if right:
            return oracle.attn_fwd_two_sided(qf[b:b + 1, h:h + 1], kf[b:b + 1, g], vf[b:b + 1, g], W - 1, right,
                                             scale)[0, 0]
        return oracle.attn_fwd(qf[b:b + 1, h:h + 1], kf[b:b + 1, g], vf[b:b + 1, g], W, 0, scale)[0, 0]

    st = _compare(got, want, B, Hq, str(case))
    full_parity.assert_bf16(st, str(case))


def test_streamed_blocks_lse():
    """The row log-sum-exp written by the streamed blocks (and the output
    bitwise equal to the plain entry point's)."""
    B, Hq, Hkv, N, d, W = 1, 8, 2, 24000, 64, 300
    say(f"streamed band lse B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} W{W}")
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, torch.bfloat16, seed=77)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = swa.attn_fwd(qd, kd, vd, window=W, return_lse=True)
    plain = swa.attn_fwd(qd, kd, vd, window=W)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    got = lse.cpu().double().numpy()
    qf, kf = q.float().numpy(), k.float().numpy()
    G, scale = Hq // Hkv, 1 / math.sqrt(d)
    st = _compare(got, lambda bh: oracle.attn_lse(qf[:, bh[1]:bh[1] + 1], kf[:, bh[1] // G:bh[1] // G + 1], W, 0,
                                                  scale)[0, 0], B, Hq, "lse", tol=2.5e-3)
    assert st.nonfinite == 0 and st.over == 0, (st.max_err, st.worst)


def _random_stream_case(i):
    """Seeded random shape with more query blocks than workgroups (case i)."""
    rng = np.random.default_rng(777000 + i)
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([2, 4, 6, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 3))
    N = int(rng.integers(4000, 14001))
    # a window of one key or of at least 16 (smaller ones return near-copies
    # of V rows, which the flat bf16 bound does not cover)
    W = int(rng.choice([1, int(rng.integers(16, 1500))]))
    right = int(rng.choice([0, 0, 0, int(rng.integers(1, 400))]))
    scale = (1 / math.sqrt(d)) * float(rng.choice([1.0, 1.0, -1.0, 0.5]))
    return B, G * Hkv, Hkv, N, d, W, right, scale


@pytest.mark.parametrize("i", [1, 2, 4, 13, 17, 22])
def test_streamed_random_shapes(i):
    """Random shapes through the streamed path (ragged ends, 2-8 query heads
    per KV head, d 64 and 128, two-sided bands, negative scales), every output
    element against the oracle."""
    B, Hq, Hkv, N, d, W, right, scale = _random_stream_case(i)
    say(f"streamed random {i}: B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} W{W} right{right} scale{scale:.4f}")
    q, k, v = inputs.random_qkv(B, Hq, Hkv, N, d, torch.bfloat16, seed=i + 99)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    if right:
        swa.attn_fwd_two_sided(q.to(DEV), k.to(DEV), v.to(DEV), W - 1, right, scale=scale, out=out)
    else:
        swa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window=W, scale=scale, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    G = Hq // Hkv

    def want(bh):
        b, h = bh
        g = slice(h // G, h // G + 1)
        if right:
            return oracle.attn_fwd_two_sided(qf[b:b + 1, h:h + 1], kf[b:b + 1, g], vf[b:b + 1, g], W - 1, right,
                                             scale)[0, 0]
        return oracle.attn_fwd(qf[b:b + 1, h:h + 1], kf[b:b + 1, g], vf[b:b + 1, g], W, 0, scale)[0, 0]

    st = _compare(got, want, B, Hq, f"random {i}")
    full_parity.assert_bf16(st, f"random {i}")
