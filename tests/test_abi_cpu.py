"""Host-side checks that need no GPU: the built library loads, exports every
symbol the public header declares, and rejects bad arguments with the
documented codes before it launches anything."""
import ctypes
import os
import re

import pytest
import torch

import sparse_causal_attention_band_amd as swa
from sparse_causal_attention_band_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa_attn.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"SWA_API\s+[\w\s\*]+?\b(swa_\w+)\s*\(", text)


def test_header_declares_the_abi():
    names = _declared()
    assert sorted(names) == sorted(swa.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    L = swa.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_only_the_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", swa.LIB_PATH], capture_output=True, text=True).stdout
    text_syms = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert text_syms == sorted(_declared())


A = 1 << 12  # a fake, 16-byte aligned "device" address: never dereferenced


def _fwd(**kw):
    args = dict(q=A, k=A * 2, v=A * 3, out=A * 1024, B=1, Hq=4, Hkv=2, N=16, d=64, window=4, stride=0,
                scale=0.125, stream=None)
    args.update(kw)
    fn = swa.lib().swa_attn_fwd
    return fn(args["q"], args["k"], args["v"], args["out"], args["B"], args["Hq"], args["Hkv"], args["N"],
              args["d"], args["window"], args["stride"], args["scale"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -1), (dict(N=0), -1), (dict(Hq=0), -1), (dict(Hkv=0), -1), (dict(Hq=3, Hkv=2), -1),
    (dict(window=0), -1), (dict(window=-7), -1), (dict(d=32), -2), (dict(d=96), -2),
    (dict(q=None), -1), (dict(k=A + 8), -1), (dict(out=A + 2), -1), (dict(scale=0.0), -1),
    (dict(scale=float("inf")), -1), (dict(scale=float("nan")), -1), (dict(out=A), -1),
])
def test_fwd_rejects_bad_arguments(kw, code):
    rc = _fwd(**kw)
    assert rc == code
    assert swa.lib().swa_last_error().decode().startswith("swa_attn_fwd")


def _dec(**kw):
    ws = swa.lib().swa_decode_workspace_bytes(2, 8, 2, 128, 4096)
    assert ws > 0  # this shape is split, so it needs a workspace
    args = dict(q=A, kr=A * 2, vr=A * 3, pos=A * 4, out=A * 5, B=2, Hq=8, Hkv=2, d=128, scale=0.1,
                ws=A * 6, wsb=ws, window=4096, stream=None)
    args.update(kw)
    return swa.lib().swa_decode(args["q"], args["kr"], args["vr"], args["pos"], args["out"], args["B"],
                                args["Hq"], args["Hkv"], args["d"], args["scale"], args["ws"], args["wsb"],
                                args["window"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -1), (dict(Hq=6, Hkv=4), -1), (dict(window=0), -1), (dict(d=80), -2),
    (dict(Hq=6, Hkv=2), -2), (dict(Hq=32, Hkv=2), -2), (dict(pos=None), -1), (dict(pos=A + 2), -1),
    (dict(ws=None), -1), (dict(wsb=16), -1), (dict(kr=A + 4), -1), (dict(scale=0.0), -1),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert _dec(**kw) == code
    assert swa.lib().swa_last_error().decode().startswith("swa_decode")


def test_workspace_size_formula():
    L = swa.lib()
    # 256 or more (sequence, KV head) pairs: one split, no workspace
    assert L.swa_decode_workspace_bytes(64, 32, 8, 128, 4096) == 0
    assert L.swa_decode_workspace_bytes(1, 1, 1, 64, 1) == 0  # a single 64-slot tile cannot split
    # otherwise ceil(256 / pairs) splits of whole 64-slot tiles, each holding
    # d floats + (max, sum) per (sequence, query head)
    assert L.swa_decode_workspace_bytes(1, 1, 1, 64, 513) == 9 * 66 * 4       # 9 tiles, 9 splits
    assert L.swa_decode_workspace_bytes(10, 32, 8, 128, 4096) == 10 * 32 * 4 * 130 * 4  # 80 pairs -> 4 splits
    assert L.swa_decode_workspace_bytes(1, 3, 2, 64, 8) == 0
    assert L.swa_decode_workspace_bytes(1, 2, 1, 100, 8) == 0


def test_python_wrapper_refuses_host_tensors():
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        swa.attn_fwd(q, q, q, window=4)
    with pytest.raises(TypeError):
        swa.attn_fwd(q.half(), q.half(), q.half(), window=4)


def test_noalloc_decode_refuses_bad_arguments_before_launch():
    L = swa.lib()
    assert L.swa_decode_noalloc(A, A * 2, A * 3, A * 4, A * 5, 2, 6, 2, 128, 0.1, 64, None) == -2   # 3 heads per KV head
    assert L.swa_decode_noalloc(A, A * 2, A * 3, A * 4, A * 5, 2, 8, 2, 96, 0.1, 64, None) == -2    # d = 96
    assert L.swa_decode_noalloc(A, A * 2, A * 3, None, A * 5, 2, 8, 2, 128, 0.1, 64, None) == -1    # pos
    assert L.swa_decode_noalloc(A, A * 2, A * 3, A * 4, A * 5, 0, 8, 2, 128, 0.1, 64, None) == -1    # B
    assert L.swa_decode_noalloc(A + 2, A * 2, A * 3, A * 4, A * 5, 2, 8, 2, 128, 0.1, 64, None) == -1  # q aligned
    assert L.swa_decode_noalloc(A, A * 2, A * 3, A * 4, A * 5, 2, 8, 2, 128, 0.0, 64, None) == -1   # scale
    assert L.swa_last_error().decode().startswith("swa_decode_noalloc")


def test_noalloc_scratch_covers_every_split_plan():
    """The split plan splits only below 256 (sequence, KV head) pairs, so the
    partials of any supported shape fit the fixed scratch (the largest: 8
    heads per KV head, d = 128)."""
    L = swa.lib()
    text = open(HEADER).read()
    cap = int(re.search(r"#define SWA_DECODE_NOALLOC_SCRATCH_BYTES (\d+)", text).group(1))
    worst = 0
    for pairs in list(range(1, 520)) + [600, 1000, 4096]:
        for W in (1, 63, 64, 65, 1000, 4096, 131072):
            worst = max(worst, L.swa_decode_workspace_bytes(pairs, 8 * pairs, pairs, 128, W))
            for B, Hkv in ((pairs, 1), (1, pairs)):
                for G in (1, 2, 4, 8):
                    for d in (64, 128):
                        need = L.swa_decode_workspace_bytes(B, G * Hkv, Hkv, d, W)
                        assert need <= cap
                        worst = max(worst, need)
    assert 2_000_000 < worst <= cap  # the bound is tight to within a few per cent


def test_python_decode_refuses_a_wrong_shaped_out():
    """The decode kernel writes B * Hq * d elements into out: a smaller (or
    differently shaped) out is refused before any device work."""
    q = torch.zeros(2, 8, 64)
    ring = torch.zeros(2, 2, 16, 64)
    pos = torch.ones(2, dtype=torch.int32)
    for bad in (torch.zeros(2, 8, 32), torch.zeros(1, 8, 64), torch.zeros(2 * 8 * 64)):
        with pytest.raises(ValueError, match="out must have"):
            swa.decode(q, ring, ring, pos, out=bad)


def test_inputs_are_seeded_and_shaped():
    a = inputs.prefill_inputs(inputs.STRIDED, N=100)
    b = inputs.prefill_inputs(inputs.STRIDED, N=100)
    for x, y in zip(a, b):
        assert torch.equal(x, y) and x.dtype == torch.bfloat16
    assert a[0].shape == (1, 16, 100, 64)
    q, kr, vr, pos = inputs.decode_inputs(inputs.DECODE, B=8)
    assert q.shape == (8, 32, 128) and kr.shape == (8, 8, 4096, 128) and pos.dtype == torch.int32
    assert int(pos.min()) >= 1 and int(pos.max()) <= 131072
    m = inputs.prefill_inputs(inputs.MISTRAL, N=64)
    # Q and K carry the 0.5 factor, V does not
    assert float(m[0].float().std()) < 0.7 and float(m[2].float().std()) > 0.8


def test_two_sided_and_diff_reject_bad_arguments():
    L = swa.lib()
    base = (A, A * 2, A * 3, A * 1024, 1, 4, 2, 16, 64)
    assert L.swa_attn_fwd_two_sided(*base, -1, 3, 0.125, None) == -1
    assert L.swa_attn_fwd_two_sided(*base, 3, -2, 0.125, None) == -1
    assert L.swa_attn_fwd_two_sided(A, A * 2, A * 3, A * 1024, 1, 4, 2, 16, 96, 3, 3, 0.125, None) == -2
    assert L.swa_last_error().decode().startswith("swa_attn_fwd_two_sided")
    # lam missing, misaligned; out overlapping q2; bad window
    d = (A, A * 2, A * 3, A * 4, A * 5)
    assert L.swa_diff_attn_fwd(*d, None, A * 1024, 1, 4, 2, 16, 64, 8, 0.125, None) == -1
    assert L.swa_diff_attn_fwd(*d, A * 6 + 2, A * 1024, 1, 4, 2, 16, 64, 8, 0.125, None) == -1
    assert L.swa_diff_attn_fwd(*d, A * 6, A * 3, 1, 4, 2, 16, 64, 8, 0.125, None) == -1
    assert L.swa_diff_attn_fwd(*d, A * 6, A * 1024, 1, 4, 2, 16, 64, 0, 0.125, None) == -1
    assert L.swa_last_error().decode().startswith("swa_diff_attn_fwd")


def test_global_rejects_bad_arguments_and_sizes_its_workspace():
    L = swa.lib()
    args = lambda **kw: [kw.get(n, dflt) for n, dflt in (
        ("q", A), ("k", A * 2), ("v", A * 3), ("out", A * 1024), ("B", 1), ("Hq", 8), ("Hkv", 2), ("N", 4096),
        ("d", 128), ("window", 64), ("gidx", A * 5), ("ng", 4), ("scale", 0.1), ("ws", A * 6),
        ("wsb", 1 << 30), ("stream", None))]
    assert L.swa_attn_fwd_global(*args(gidx=None)) == -1
    assert L.swa_attn_fwd_global(*args(gidx=A * 5 + 2)) == -1
    assert L.swa_attn_fwd_global(*args(ng=-1)) == -1
    assert L.swa_attn_fwd_global(*args(ng=5000)) == -1            # more global positions than N
    assert L.swa_attn_fwd_global(*args(Hq=6, Hkv=2)) == -2        # 3 heads per KV head: no row kernel
    assert L.swa_attn_fwd_global(*args(wsb=16)) == -1
    assert L.swa_last_error().decode().startswith("swa_attn_fwd_global")
    # one (sequence, global row) entry per decode entry: 4 rows x 2 KV heads
    # = 8 pairs -> 32 splits (two 64-key tiles each over N = 4096 keys, so
    # that pairs x splits fill the 256 CUs), d + 2 floats each
    assert L.swa_attn_fwd_global_workspace_bytes(1, 8, 2, 4096, 128, 4) == 4 * 8 * 32 * 130 * 4
    assert L.swa_attn_fwd_global_workspace_bytes(1, 8, 2, 4096, 128, 0) == 0


def test_lse_entry_points_reject_bad_arguments():
    L = swa.lib()
    base = (A, A * 2, A * 3, A * 1024)
    sizes = (1, 4, 2, 16, 64, 4, 0, 0.125, None)
    assert L.swa_attn_fwd_lse(*base, None, *sizes) == -1              # lse missing
    assert L.swa_attn_fwd_lse(*base, A * 2048 + 2, *sizes) == -1      # misaligned
    assert L.swa_attn_fwd_lse(*base, A * 1024 + 64, *sizes) == -1     # inside out
    assert L.swa_last_error().decode().startswith("swa_attn_fwd_lse")
    assert L.swa_attn_fwd_lse_f32(*base, None, *sizes) == -1
    assert L.swa_last_error().decode().startswith("swa_attn_fwd_lse_f32")
    ch = (A, A * 2, A * 3, A * 4, A * 5, A * 6, A * 1024)
    csz = (1, 4, 2, 16, 64, 8, 0.125, None)
    assert L.swa_chunk_prefill_lse(*ch, None, *csz) == -1
    assert L.swa_chunk_prefill_lse(*ch, A * 2048 + 1, *csz) == -1
    assert L.swa_chunk_prefill_lse(*ch, A * 1024 + 4, *csz) == -1
    assert L.swa_last_error().decode().startswith("swa_chunk_prefill_lse")
    assert L.swa_chunk_prefill_lse_f32(*ch, None, *csz) == -1
