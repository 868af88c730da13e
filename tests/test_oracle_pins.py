"""Pins for the float64 oracle: what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: values printed on the
pages (worked example, mask figure, pair counts), closed forms, special cases
that reduce to a library routine (torch's float64 CPU scaled_dot_product_attention),
and brute force on tiny inputs.  ``test_planted_mistakes_are_caught`` checks
that plausible slips in the oracle would fail at least one of these pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import swa_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    conv = {"0": 0.0, "ln2": math.log(2.0), "ln3": math.log(3.0)}
    k = np.array([conv[s] for s in g["k"]])
    v = np.array(g["v"], dtype=np.float64)
    return g, k, v


def _as_bhnd(x):
    return np.asarray(x, dtype=np.float64).reshape(1, 1, -1, 1)


# ---------------------------------------------------------------- worked example
def test_worked_example_swa_and_full_causal():
    """SWA page §3.2: position 5 gives 14/3 at W=3 and 38/8 under full causal."""
    g, k, v = _worked()
    q = np.zeros(5)
    q[4] = g["q5"]
    out_swa = oracle.attn_fwd(_as_bhnd(q), _as_bhnd(k), _as_bhnd(v), window=g["window_swa"], scale=1.0)
    num, den = g["expected_swa"]
    assert abs(out_swa[0, 0, 4, 0] - num / den) <= 1e-15
    for w in (5, 6, 100):  # W >= T is full causal
        out_full = oracle.attn_fwd(_as_bhnd(q), _as_bhnd(k), _as_bhnd(v), window=w, scale=1.0)
        num, den = g["expected_full_causal"]
        assert abs(out_full[0, 0, 4, 0] - num / den) <= 1e-15


def test_worked_example_ring_form():
    """Same example read through the rolling cache (SWA page §4.2):
    positions 3,4,5 sit in slots 2,0,1 of a 3-slot ring."""
    g, k, v = _worked()
    W, pos = g["ring_window"], g["ring_pos"]
    assert [oracle.ring_slot(t, W) for t in (3, 4, 5)] == g["ring_slots_of_positions_3_4_5"]
    kring = np.zeros((1, 1, W, 1))
    vring = np.zeros((1, 1, W, 1))
    for t in range(1, pos + 1):  # rolling writes: later positions overwrite
        kring[0, 0, oracle.ring_slot(t, W), 0] = k[t - 1]
        vring[0, 0, oracle.ring_slot(t, W), 0] = v[t - 1]
    assert list(kring[0, 0, :, 0]) == [k[3], k[4], k[2]]
    out = oracle.decode(np.full((1, 1, 1), g["q5"]), kring, vring, [pos], window=W, scale=1.0)
    num, den = g["expected_swa"]
    assert abs(out[0, 0, 0] - num / den) <= 1e-15


# ---------------------------------------------------------------- mask figure, counts
def _read_mask_fixture():
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, "swa_mask_n8_w4.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                blocks[cur] = []
            else:
                blocks[cur].append([c == "x" for c in line])
    return {k: np.array(v) for k, v in blocks.items()}


def test_mask_matches_page_figure():
    fig = _read_mask_fixture()
    assert (oracle.allowed_mask(8, 4) == fig["window_4"]).all()
    assert (oracle.allowed_mask(8, 8) == fig["full_causal"]).all()
    assert (oracle.allowed_mask(8, 1000) == fig["full_causal"]).all()


def test_pair_counts_page_values_and_closed_form():
    """SWA page §4.1: N_full = T(T+1)/2, N_SWA = T*W - W(W-1)/2 (T >= W);
    T=5, W=3 gives 15 and 12."""
    assert oracle.allowed_pair_count(5, 5) == 15
    assert oracle.allowed_pair_count(5, 3) == 12
    assert int(oracle.allowed_mask(5, 3).sum()) == 12
    for T in (1, 2, 7, 64, 257, 1000):
        assert oracle.allowed_pair_count(T, T) == T * (T + 1) // 2
        for W in (1, 2, 3, 31, 32, 33, 64, 300):
            if T >= W:
                assert oracle.allowed_pair_count(T, W) == T * W - W * (W - 1) // 2
            if T <= 300:
                assert oracle.allowed_pair_count(T, W) == int(oracle.allowed_mask(T, W).sum())


def _strided_count_closed_form(n, w, s):
    # row i >= W also reads the multiples of s strictly below its band start
    # i-W+1, i.e. m*s <= i-W, which are floor((i-W)/s)+1 keys.
    return sum(min(i + 1, w) + ((i - w) // s + 1 if i >= w else 0) for i in range(n))


def test_strided_counts():
    for n, w, s in [(64, 8, 4), (100, 7, 13), (257, 32, 1), (300, 16, 300), (50, 60, 5)]:
        want = _strided_count_closed_form(n, w, s)
        assert oracle.allowed_pair_count(n, w, s) == want
        assert int(oracle.allowed_mask(n, w, s).sum()) == want
    # local W=256 + stride 128 at N=8192: band 2,064,512 + strided 249,984
    assert oracle.allowed_pair_count(8192, 256) == 8192 * 256 - 256 * 255 // 2 == 2_064_512
    assert oracle.allowed_pair_count(8192, 256, 128) == 2_314_496
    # stride 1 is full causal; stride >= n adds key 0 only
    assert (oracle.allowed_mask(40, 5, 1) == oracle.allowed_mask(40, 40)).all()
    m = oracle.allowed_mask(40, 5, 40)
    ref = oracle.allowed_mask(40, 5)
    ref[:, 0] = True
    assert (m == ref).all()


def test_predicate_restatements_agree():
    """Three independent statements of the band on the pages: the page loop
    (lo = max(0, i-window+1) .. i), the FlexAttention predicate
    (q-kv < W) & (q >= kv), and FlashAttention window_size = (W-1, 0)."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(1, 48))
        w = int(rng.integers(1, 60))
        m = oracle.allowed_mask(n, w)
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        flex = ((i - j) < w) & (i >= j)
        fa = (j >= i - (w - 1)) & (j <= i + 0)
        assert (m == flex).all() and (m == fa).all()


# ---------------------------------------------------------------- special cases, library
def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask_bool, scale):
    G = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, attn_mask=torch.from_numpy(mask_bool), scale=scale).numpy()


def test_full_causal_equals_library_and_is_bitwise_stable_in_W():
    q, k, v = _rand((2, 4, 37, 8), 2), _rand((2, 2, 37, 8), 3), _rand((2, 2, 37, 8), 4)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k).repeat_interleave(2, 1),
        torch.from_numpy(v).repeat_interleave(2, 1), is_causal=True).numpy()
    a = oracle.attn_fwd(q, k, v, window=37)
    b = oracle.attn_fwd(q, k, v, window=74)
    assert np.array_equal(a, b)  # W >= N: identical, bit for bit
    assert np.abs(a - ref).max() <= 1e-12


@pytest.mark.parametrize("n,w,s", [(45, 7, 0), (64, 16, 0), (70, 9, 8), (33, 1, 5), (50, 20, 1)])
def test_band_and_strided_equal_library_with_explicit_mask(n, w, s):
    q, k, v = _rand((1, 6, n, 16), n), _rand((1, 3, n, 16), n + 1), _rand((1, 3, n, 16), n + 2)
    # mask built here from tril/triu offsets (FlashAttention window_size=(W-1,0))
    tri = torch.ones(n, n, dtype=torch.bool).tril(0)
    band = tri & torch.ones(n, n, dtype=torch.bool).triu(-(w - 1))
    if s > 0:
        band = band | (tri & (torch.arange(n)[None, :] % s == 0))
    scale = 0.37
    ref = _sdpa(q, k, v, band.numpy(), scale)
    got = oracle.attn_fwd(q, k, v, window=w, stride=s, scale=scale)
    assert np.abs(got - ref).max() <= 1e-12


def test_window_one_returns_v():
    q, k, v = _rand((1, 2, 20, 4), 5), _rand((1, 1, 20, 4), 6), _rand((1, 1, 20, 4), 7)
    out = oracle.attn_fwd(q, k, v, window=1)
    assert np.array_equal(out[0, 0], v[0, 0]) and np.array_equal(out[0, 1], v[0, 0])


def test_rows_sum_to_one_and_zero_outside_mask():
    """With V = identity the output row is the probability row itself."""
    n = 30
    for w, s in [(5, 0), (30, 0), (4, 7)]:
        q, k = _rand((1, 1, n, 3), 8), _rand((1, 1, n, 3), 9)
        v = np.eye(n).reshape(1, 1, n, n)
        kk = np.zeros((1, 1, n, n))
        kk[..., :3] = k
        qq = np.zeros((1, 1, n, n))
        qq[..., :3] = q
        p = oracle.attn_fwd(qq, kk, v, window=w, stride=s, scale=1.0)[0, 0]
        assert np.abs(p.sum(axis=1) - 1).max() <= 1e-12
        assert (p[~oracle.allowed_mask(n, w, s)] == 0).all()
        assert (p[oracle.allowed_mask(n, w, s)] > 0).all()


def test_zero_query_is_mean_of_allowed_values():
    """Q = 0 gives uniform weights, so with V_j = j the row is the mean of its
    allowed positions: (lo+i)/2 for the band; band plus the multiples of s
    below lo for the strided variant."""
    n, d = 300, 2
    v = np.repeat(np.arange(n, dtype=np.float64)[:, None], d, axis=1).reshape(1, 1, n, d)
    q = np.zeros((1, 1, n, d))
    k = _rand((1, 1, n, d), 10)
    for w, s in [(32, 0), (17, 0), (32, 8), (5, 64)]:
        out = oracle.attn_fwd(q, k, v, window=w, stride=s)[0, 0, :, 0]
        for i in range(n):
            lo = max(0, i - w + 1)
            tot, cnt = (lo + i) * (i - lo + 1) / 2, i - lo + 1
            if s > 0 and lo > 0:
                m = (lo - 1) // s + 1
                tot += s * m * (m - 1) / 2
                cnt += m
            assert abs(out[i] - tot / cnt) <= 1e-9 * max(1.0, i)


def test_brute_force_tiny():
    """Per-pair pure-Python evaluation on tiny inputs."""
    rng = np.random.default_rng(11)
    for n, d, w, s, hq, hkv in [(9, 3, 3, 0, 2, 1), (16, 4, 5, 4, 2, 2), (12, 2, 12, 3, 4, 2), (7, 1, 1, 2, 1, 1)]:
        q = rng.standard_normal((1, hq, n, d))
        k = rng.standard_normal((1, hkv, n, d))
        v = rng.standard_normal((1, hkv, n, d))
        scale = 1 / math.sqrt(d)
        got = oracle.attn_fwd(q, k, v, window=w, stride=s)
        G = hq // hkv
        for h in range(hq):
            g = h // G
            for i in range(n):
                keys = []
                for j in range(n):
                    if j <= i and (i - j < w or (s > 0 and j % s == 0)):
                        keys.append(j)
                sc = [scale * sum(q[0, h, i, c] * k[0, g, j, c] for c in range(d)) for j in keys]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                z = sum(e)
                for c in range(d):
                    want = sum(e[t] * v[0, g, keys[t], c] for t in range(len(keys))) / z
                    assert abs(got[0, h, i, c] - want) <= 1e-12


def test_rows_helper_matches_full():
    q, k, v = _rand((2, 4, 90, 8), 12), _rand((2, 2, 90, 8), 13), _rand((2, 2, 90, 8), 14)
    full = oracle.attn_fwd(q, k, v, window=11, stride=6, scale=0.5)
    picks = [(0, 0, 0), (1, 3, 89), (0, 2, 45), (1, 1, 10)]
    rows = oracle.attn_fwd_rows(q, k, v, 11, 6, 0.5, picks)
    # a single row gathers fewer keys than its 256-row block: only the
    # summation order differs
    for r, (b, h, i) in zip(rows, picks):
        assert np.abs(r - full[b, h, i]).max() <= 1e-13
    par, workers = oracle.attn_fwd_parallel(q, k, v, 11, 6, 0.5, np.arange(90), workers=2)
    assert workers == 2 and np.array_equal(par, full)


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("W,pos", [(8, 1), (8, 2), (8, 7), (8, 8), (8, 9), (8, 37), (5, 131072)])
def test_decode_equals_last_prefill_row(W, pos):
    hq, hkv, d = 4, 2, 6
    rng = np.random.default_rng(pos + W)
    kseq = rng.standard_normal((1, hkv, pos, d))
    vseq = rng.standard_normal((1, hkv, pos, d))
    q = rng.standard_normal((1, hq, d))
    kring = np.full((1, hkv, W, d), np.nan)  # never-written slots stay NaN
    vring = np.full((1, hkv, W, d), np.nan)
    for t in range(max(1, pos - 2 * W), pos + 1):
        kring[0, :, oracle.ring_slot(t, W)] = kseq[0, :, t - 1]
        vring[0, :, oracle.ring_slot(t, W)] = vseq[0, :, t - 1]
    got = oracle.decode(q, kring, vring, [pos], window=W)
    assert np.isfinite(got).all()
    qseq = np.zeros((1, hq, pos, d))
    qseq[0, :, pos - 1] = q[0]
    want = oracle.attn_fwd_rows(qseq, kseq, vseq, W, 0, 1 / math.sqrt(d),
                                [(0, h, pos - 1) for h in range(hq)])
    assert np.abs(got[0] - want).max() <= 1e-12


def test_decode_nonpositive_pos_is_zero():
    out = oracle.decode(np.ones((2, 2, 4)), np.ones((2, 1, 3, 4)), np.ones((2, 1, 3, 4)), [0, -3], window=3)
    assert (out == 0).all()


# ---------------------------------------------------------------- chunked prefill
def test_ring_append_places_positions_like_the_page():
    """Appending positions 1..5 of the worked example to a 3-slot ring leaves
    positions 3, 4, 5 in slots 2, 0, 1 (SWA page §4.2)."""
    g, k, v = _worked()
    kr = np.zeros((1, 1, 3, 1))
    vr = np.zeros((1, 1, 3, 1))
    # two chunks: positions 1..2, then 3..5
    kr, vr = oracle.ring_append(kr, vr, k[:2].reshape(1, 1, 2, 1), v[:2].reshape(1, 1, 2, 1), [0], 3)
    kr, vr = oracle.ring_append(kr, vr, k[2:].reshape(1, 1, 3, 1), v[2:].reshape(1, 1, 3, 1), [2], 3)
    assert list(kr[0, 0, :, 0]) == [k[3], k[4], k[2]]
    assert list(vr[0, 0, :, 0]) == [v[3], v[4], v[2]]


@pytest.mark.parametrize("W,chunks", [(8, [3, 5, 1, 9, 4]), (16, [40, 1, 17]), (5, [1, 1, 1, 2, 13]), (64, [30, 50])])
def test_chunked_prefill_equals_whole_prefill(W, chunks):
    """Prefill chunk by chunk over the rolling cache (attend, then append)
    gives the rows of one whole-sequence prefill (SWA page §4.3): the
    history read from the ring plus the chunk with the per-row band."""
    B, Hq, Hkv, d = 2, 4, 2, 6
    L = sum(chunks)
    rng = np.random.default_rng(W + L)
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    whole = oracle.attn_fwd(q, k, v, W)
    kr = np.full((B, Hkv, W, d), np.nan)  # never-written slots stay NaN
    vr = np.full((B, Hkv, W, d), np.nan)
    p0 = 0
    for T in chunks:
        sl = slice(p0, p0 + T)
        out = oracle.chunk_prefill(q[:, :, sl], k[:, :, sl], v[:, :, sl], kr, vr, [p0] * B, W)
        assert np.abs(out - whole[:, :, sl]).max() <= 1e-12
        last = oracle.chunk_prefill(q[:, :, sl], k[:, :, sl], v[:, :, sl], kr, vr, [p0] * B, W, rows=[T - 1])
        assert np.abs(last[:, :, 0] - whole[:, :, p0 + T - 1]).max() <= 1e-12
        kr, vr = oracle.ring_append(kr, vr, k[:, :, sl], v[:, :, sl], [p0] * B, W)
        p0 += T
    # and the cache then serves the decode step of the next token
    qn = rng.standard_normal((B, Hq, d))
    kn = rng.standard_normal((B, Hkv, 1, d))
    vn = rng.standard_normal((B, Hkv, 1, d))
    kr, vr = oracle.ring_append(kr, vr, kn, vn, [p0] * B, W)
    dec = oracle.decode(qn, kr, vr, [p0 + 1] * B, W)
    full = oracle.attn_fwd_rows(np.concatenate([q, qn[:, :, None]], 2), np.concatenate([k, kn], 2),
                                np.concatenate([v, vn], 2), W, 0, 1 / math.sqrt(d),
                                [(b, h, L) for b in range(B) for h in range(Hq)])
    assert np.abs(dec.reshape(-1, d) - full).max() <= 1e-12


def test_truncating_to_the_last_w_rows_is_not_the_rolling_cache():
    """The SWA page §4.3 warns that cutting the input to its last W tokens and
    recomputing is not the same as the rolling cache; in a single layer the
    rows agree, so the difference shows in a second stacked layer, whose
    inputs already mixed in older positions.  Here: one layer's rows are
    identical either way (what the cache gives the next step)."""
    W, L, d = 4, 10, 3
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 1, L, d)) for _ in range(3))
    full_last = oracle.attn_fwd(q, k, v, W)[0, 0, -1]
    cut_last = oracle.attn_fwd(q[:, :, -W:], k[:, :, -W:], v[:, :, -W:], W)[0, 0, -1]
    assert np.abs(full_last - cut_last).max() <= 1e-12
    # two stacked layers (output fed back as q, k and v): the cut input loses
    # the older positions that the first layer had folded into rows L-W..L-1
    h1 = oracle.attn_fwd(q, k, v, W)
    two = oracle.attn_fwd(h1, h1, h1, W)[0, 0, -1]
    h1c = oracle.attn_fwd(q[:, :, -W:], k[:, :, -W:], v[:, :, -W:], W)
    two_cut = oracle.attn_fwd(h1c, h1c, h1c, W)[0, 0, -1]
    assert np.abs(two - two_cut).max() > 1e-3


# ---------------------------------------------------------------- row log-sum-exp
def test_lse_worked_example():
    """SWA page §3.2: the exponentiated scores of position 5 are 1, 2, 3 under
    W = 3 and 1, 1, 1, 2, 3 under full causal, so the row's softmax
    denominators are 6 and 8; the zero queries of positions 1..4 give ln of
    their key counts."""
    g, k, v = _worked()
    q = np.zeros(5)
    q[4] = g["q5"]
    lse = oracle.attn_lse(_as_bhnd(q), _as_bhnd(k), window=g["window_swa"], scale=1.0)[0, 0]
    assert abs(lse[4] - math.log(6.0)) <= 1e-15
    assert np.abs(lse[:4] - np.log([1.0, 2.0, 3.0, 3.0])).max() <= 1e-15
    for w in (5, 6, 100):
        full = oracle.attn_lse(_as_bhnd(q), _as_bhnd(k), window=w, scale=1.0)[0, 0]
        assert abs(full[4] - math.log(8.0)) <= 1e-15
        assert np.abs(full[:4] - np.log([1.0, 2.0, 3.0, 4.0])).max() <= 1e-15


def test_lse_window_one_is_the_own_score():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((2, 3, 17, 8)), rng.standard_normal((2, 3, 17, 8))
    lse = oracle.attn_lse(q, k, window=1, scale=0.7)
    assert np.abs(lse - 0.7 * (q * k).sum(-1)).max() <= 1e-12


@pytest.mark.parametrize("n,w,s", [(30, 4, 0), (41, 6, 7), (20, 25, 3)])
def test_lse_identical_keys_closed_form(n, w, s):
    """Every key equal: the row's scores are all scale * q_i . k, so the
    log-sum-exp is that score plus ln |S_i| (the allowed-set size)."""
    rng = np.random.default_rng(n)
    d = 4
    q = rng.standard_normal((1, 2, n, d))
    krow = rng.standard_normal(d)
    k = np.broadcast_to(krow, (1, 1, n, d)).copy()
    lse = oracle.attn_lse(q, k, window=w, stride=s, scale=0.5)
    counts = np.array([len(oracle.allowed_set(i, w, s)) for i in range(n)], dtype=np.float64)
    want = 0.5 * (q[0] @ krow) + np.log(counts)[None, :]
    assert np.abs(lse[0] - want).max() <= 1e-12


@pytest.mark.parametrize("n,w,s", [(24, 5, 0), (31, 4, 6)])
def test_lse_reproduces_the_attention_weights(n, w, s):
    """With V the identity (d_v = N) the forward's output row i is the
    weight vector p_ij; it must equal exp(scale * s_ij - lse_i) on the
    allowed keys and 0 elsewhere (d = N so that V may be the identity)."""
    rng = np.random.default_rng(n + w)
    d = n
    q, k = 0.3 * rng.standard_normal((1, 1, n, d)), rng.standard_normal((1, 1, n, d))
    v = np.eye(n).reshape(1, 1, n, n)
    p = oracle.attn_fwd(q, k, v, w, s, 0.8)[0, 0]
    lse = oracle.attn_lse(q, k, w, s, 0.8)[0, 0]
    allowed = oracle.allowed_mask(n, w, s)
    want = np.where(allowed, np.exp(0.8 * (q[0, 0] @ k[0, 0].T) - lse[:, None]), 0.0)
    assert np.abs(p - want).max() <= 1e-12


@pytest.mark.parametrize("W,p0,T", [(8, 0, 5), (8, 3, 6), (8, 20, 9), (16, 7, 40)])
def test_chunk_lse_equals_whole_sequence_lse(W, p0, T):
    """Chunked prefill over a ring holding positions 1..p0 has, row for row,
    the log-sum-exp of the whole sequence's last T rows (SWA page §4.3)."""
    rng = np.random.default_rng(W * 100 + p0)
    d, n = 4, p0 + T
    q = rng.standard_normal((1, 2, n, d))
    k = rng.standard_normal((1, 1, n, d))
    kring = np.zeros((1, 1, W, d))
    for t in range(1, p0 + 1):
        kring[0, 0, oracle.ring_slot(t, W)] = k[0, 0, t - 1]
    got = oracle.chunk_prefill_lse(q[:, :, p0:], k[:, :, p0:], kring, [p0], W, scale=0.9)
    want = oracle.attn_lse(q, k, W, 0, 0.9)[:, :, p0:]
    assert np.abs(got - want).max() <= 1e-12


# ---------------------------------------------------------------- pin strength
def _pins_fail(monkeypatch, name, bad):
    """Run the pins with one oracle helper replaced; True if any pin fails."""
    monkeypatch.setattr(swa_oracle, name, bad)
    checks = [test_worked_example_swa_and_full_causal, test_mask_matches_page_figure,
              test_window_one_returns_v, test_rows_sum_to_one_and_zero_outside_mask,
              test_full_causal_equals_library_and_is_bitwise_stable_in_W,
              lambda: test_band_and_strided_equal_library_with_explicit_mask(70, 9, 8),
              test_zero_query_is_mean_of_allowed_values, test_lse_worked_example,
              lambda: test_lse_identical_keys_closed_form(41, 6, 7)]
    failed = False
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failed = True
    monkeypatch.undo()
    return failed


def test_planted_mistakes_are_caught(monkeypatch):
    good_allowed = swa_oracle._row_allowed
    good_keys = swa_oracle._block_keys

    def window_counts_w_plus_one(rows, keys, window, stride):  # "[i-W, i]" reading
        return good_allowed(rows, keys, window + 1, stride)

    def no_causal_cut(rows, keys, window, stride):
        i, j = rows[:, None], keys[None, :]
        return (j >= np.maximum(0, i - window + 1)) & (j <= i + 1)

    def stride_on_one_based(rows, keys, window, stride):
        i, j = rows[:, None], keys[None, :]
        band = (j <= i) & (j >= np.maximum(0, i - window + 1))
        return band | ((j <= i) & ((j + 1) % stride == 0)) if stride > 0 else band

    def keys_drop_band_start(i0, i1, window, stride):
        return good_keys(i0, i1, window, stride)[1:]

    def softmax_over_columns(scores, allowed):
        s = np.where(allowed, scores, -np.inf)
        e = np.where(allowed, np.exp(s - s.max()), 0.0)
        return e / np.maximum(e.sum(axis=0, keepdims=True), 1e-300)

    def head_rows_k_for_v(q, k, v, rows, window, stride, scale):  # transposed operand
        return swa_oracle.__dict__["_head_rows_orig"](q, v, k, rows, window, stride, scale)

    assert _pins_fail(monkeypatch, "_row_allowed", window_counts_w_plus_one)
    assert _pins_fail(monkeypatch, "_row_allowed", no_causal_cut)
    assert _pins_fail(monkeypatch, "_row_allowed", stride_on_one_based)
    assert _pins_fail(monkeypatch, "_block_keys", keys_drop_band_start)
    assert _pins_fail(monkeypatch, "_masked_softmax_rows", softmax_over_columns)
    swa_oracle._head_rows_orig = swa_oracle._head_rows
    try:
        assert _pins_fail(monkeypatch, "_head_rows", head_rows_k_for_v)
    finally:
        del swa_oracle._head_rows_orig


# ---------------------------------------------------------------- two-sided band
def _page_two_sided_mask(n, w):
    """The explainer page's ("滑动窗口注意力") §3.3 construction, restated: ones, then zero the
    columns before max(0, i-w) and from min(n, i+w+1) on, row by row."""
    m = np.ones((n, n))
    for i in range(n):
        start = max(0, i - w)
        end = min(n, i + w + 1)
        m[i, :start] = 0
        m[i, end:] = 0
    return m.astype(bool)


@pytest.mark.parametrize("n,w", [(8, 2), (13, 4), (5, 0), (9, 20)])
def test_two_sided_mask_matches_the_page_construction(n, w):
    assert np.array_equal(oracle.allowed_mask_two_sided(n, w, w), _page_two_sided_mask(n, w))
    # and the page's causal combination (times the lower triangle) is the
    # causal band with W = w + 1
    causal = _page_two_sided_mask(n, w) & np.tril(np.ones((n, n), dtype=bool))
    assert np.array_equal(causal, oracle.allowed_mask(n, w + 1))


@pytest.mark.parametrize("n,left,right", [(17, 3, 5), (40, 0, 7), (33, 12, 0), (10, 30, 30)])
def test_two_sided_pair_count_closed_form(n, left, right):
    want = sum(min(i, left) + min(n - 1 - i, right) + 1 for i in range(n))
    assert int(oracle.allowed_mask_two_sided(n, left, right).sum()) == want


def test_two_sided_with_no_right_part_is_the_causal_band():
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((1, 4, 70, 8)) for _ in range(3))
    k, v = k[:, :2], v[:, :2]
    for left in (0, 1, 6, 69, 200):
        got = oracle.attn_fwd_two_sided(q, k, v, left, 0)
        want = oracle.attn_fwd(q, k, v, left + 1)
        assert np.abs(got - want).max() <= 1e-13


def test_two_sided_full_width_is_sdpa_without_mask():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((2, 4, 45, 16))
    k = rng.standard_normal((2, 4, 45, 16))
    v = rng.standard_normal((2, 4, 45, 16))
    got = oracle.attn_fwd_two_sided(q, k, v, 44, 44)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    assert np.abs(got - want).max() <= 1e-12


def test_two_sided_sdpa_with_boolean_band():
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((1, 2, 64, 8)) for _ in range(3))
    m = torch.from_numpy(oracle.allowed_mask_two_sided(64, 5, 11))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=m).numpy()
    assert np.abs(oracle.attn_fwd_two_sided(q, k, v, 5, 11) - want).max() <= 1e-12


def test_two_sided_reversal_swaps_left_and_right():
    """Reversing the positions turns the band i-left..i+right into
    i-right..i+left: a swapped pair of radii fails this."""
    rng = np.random.default_rng(24)
    q, k, v = (rng.standard_normal((1, 1, 50, 6)) for _ in range(3))
    a = oracle.attn_fwd_two_sided(q, k, v, 3, 9)
    r = oracle.attn_fwd_two_sided(q[:, :, ::-1], k[:, :, ::-1], v[:, :, ::-1], 9, 3)[:, :, ::-1]
    assert np.abs(a - r).max() <= 1e-13
    assert np.abs(a - oracle.attn_fwd_two_sided(q, k, v, 9, 3)).max() > 1e-3


def test_two_sided_brute_force():
    rng = np.random.default_rng(25)
    n, d, left, right = 11, 3, 2, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    got = oracle.attn_fwd_two_sided(q[None, None], k[None, None], v[None, None], left, right, 0.7)[0, 0]
    for i in range(n):
        keys = [j for j in range(n) if i - left <= j <= i + right]
        w = [math.exp(0.7 * sum(q[i, c] * k[j, c] for c in range(d))) for j in keys]
        z = sum(w)
        want = [sum(w[a] * v[j, c] for a, j in enumerate(keys)) / z for c in range(d)]
        assert max(abs(got[i, c] - want[c]) for c in range(d)) <= 1e-12


# ---------------------------------------------------------------- differential attention
def _diff_inputs(seed, B=1, Hq=4, Hkv=2, N=90, d=8):
    rng = np.random.default_rng(seed)
    q1, q2 = (rng.standard_normal((B, Hq, N, d)) for _ in range(2))
    k1, k2, v = (rng.standard_normal((B, Hkv, N, d)) for _ in range(3))
    lam = rng.uniform(0.5, 0.8, Hq)  # the range the pages quote for the learned scalar
    return q1, k1, q2, k2, v, lam


def test_diff_with_zero_lambda_is_the_first_map():
    q1, k1, q2, k2, v, lam = _diff_inputs(31)
    got = oracle.diff_attn_fwd(q1, k1, q2, k2, v, np.zeros(4), 17)
    assert np.abs(got - oracle.attn_fwd(q1, k1, v, 17)).max() <= 1e-13


def test_diff_is_affine_in_lambda_with_the_second_map_as_slope():
    q1, k1, q2, k2, v, lam = _diff_inputs(32)
    got = oracle.diff_attn_fwd(q1, k1, q2, k2, v, lam, 25)
    want = oracle.attn_fwd(q1, k1, v, 25) - lam[None, :, None, None] * oracle.attn_fwd(q2, k2, v, 25)
    assert np.abs(got - want).max() <= 1e-13


def test_diff_of_identical_maps_scales_by_one_minus_lambda():
    q1, k1, _, _, v, lam = _diff_inputs(33)
    got = oracle.diff_attn_fwd(q1, k1, q1, k1, v, lam, 9)
    want = (1 - lam)[None, :, None, None] * oracle.attn_fwd(q1, k1, v, 9)
    assert np.abs(got - want).max() <= 1e-13


def test_diff_brute_force_page_causal_form():
    """W >= N: the page's two causal softmax maps, subtracted, times V."""
    rng = np.random.default_rng(34)
    n, d, lam = 7, 3, 0.65
    q1, k1, q2, k2, v = (rng.standard_normal((n, d)) for _ in range(5))
    got = oracle.diff_attn_fwd(q1[None, None], k1[None, None], q2[None, None], k2[None, None], v[None, None],
                               [lam], n)[0, 0]
    sd = math.sqrt(d)
    for i in range(n):
        w1 = [math.exp(sum(q1[i, c] * k1[j, c] for c in range(d)) / sd) for j in range(i + 1)]
        w2 = [math.exp(sum(q2[i, c] * k2[j, c] for c in range(d)) / sd) for j in range(i + 1)]
        z1, z2 = sum(w1), sum(w2)
        for c in range(d):
            want = sum((w1[j] / z1 - lam * w2[j] / z2) * v[j, c] for j in range(i + 1))
            assert abs(got[i, c] - want) <= 1e-12


# ---------------------------------------------------------------- local + global tokens
def _qkv(seed, B=1, Hq=4, Hkv=2, N=96, d=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)))


def test_global_with_no_global_positions_is_the_band():
    q, k, v = _qkv(41)
    assert np.abs(oracle.attn_fwd_global(q, k, v, 13, []) - oracle.attn_fwd(q, k, v, 13)).max() <= 1e-13


def test_global_rows_are_full_causal_rows():
    q, k, v = _qkv(42)
    g = [0, 5, 50, 95]
    got = oracle.attn_fwd_global(q, k, v, 7, g)
    full = oracle.attn_fwd(q, k, v, 96)
    assert np.abs(got[:, :, g] - full[:, :, g]).max() <= 1e-13


def test_global_keys_on_a_stride_grid_match_the_strided_mask_on_other_rows():
    """Global keys at 0, s, 2s, ... give non-global rows exactly the local +
    strided pattern of the attention-variants page (its step 3)."""
    q, k, v = _qkv(43, N=120)
    s = 16
    g = list(range(0, 120, s))
    got = oracle.attn_fwd_global(q, k, v, 10, g)
    strided = oracle.attn_fwd(q, k, v, 10, stride=s)
    rows = [i for i in range(120) if i % s != 0]
    assert np.abs(got[:, :, rows] - strided[:, :, rows]).max() <= 1e-13
    m = oracle.allowed_mask_global(120, 10, g)
    assert np.array_equal(m[rows], oracle.allowed_mask(120, 10, s)[rows])


def test_global_everywhere_is_full_causal_sdpa():
    q, k, v = _qkv(44, N=40)
    got = oracle.attn_fwd_global(q, k, v, 3, range(40))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, 2, axis=1)), torch.from_numpy(np.repeat(v, 2, axis=1)),
        is_causal=True).numpy()
    assert np.abs(got - want).max() <= 1e-12


def test_global_sdpa_with_boolean_mask_and_brute_force():
    q, k, v = _qkv(45, Hq=2, Hkv=2, N=70)
    g = [3, 31, 32, 69]
    m = torch.from_numpy(oracle.allowed_mask_global(70, 6, g))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=m).numpy()
    assert np.abs(oracle.attn_fwd_global(q, k, v, 6, g) - want).max() <= 1e-12
    # the mask itself, pair by pair from the reading
    for i in range(70):
        for j in range(70):
            assert m[i, j] == (j <= i and (i - j < 6 or j in g or i in g))
