"""ctypes binding of ``libswa_attn.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
checks tensor dtype/shape/device on the Python side, allocates outputs with
torch (device memory), passes raw pointers and the current HIP stream, and
turns a non-zero return code into an exception.  There is no fallback: if
the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loads the HIP runtime first, so the library binds to that same runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswa_attn.so")

SWA_OK = 0
SWA_ERR_INVALID_ARG = -1
SWA_ERR_UNSUPPORTED = -2
SWA_ERR_HIP = -3

# name -> (restype, argtypes); mirrors include/swa_attn.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "swa_attn_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_attn_fwd_f32": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_attn_fwd_lse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_attn_fwd_lse_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _Z, _I, _P]),
    "swa_decode_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _Z, _I, _P]),
    "swa_attn_fwd_two_sided": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_attn_fwd_two_sided_f32": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_diff_attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_diff_attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_attn_fwd_global": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _F, _P, _Z, _P]),
    "swa_attn_fwd_global_f32": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _F, _P, _Z, _P]),
    "swa_attn_fwd_global_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "swa_chunk_prefill": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_chunk_prefill_f32": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_chunk_prefill_lse": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_chunk_prefill_lse_f32": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_ring_append": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "swa_ring_append_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "swa_decode_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "swa_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "swa_last_error": (ctypes.c_char_p, []),
}


class SwaError(RuntimeError):
    """A library entry point returned a non-zero code."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load the shared library (once); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python sparse_causal_attention_band_amd/build.py` first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != SWA_OK:
        raise SwaError(rc, lib().swa_last_error().decode())


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int, stride: int = 0,
             scale: float | None = None, out: torch.Tensor | None = None, return_lse: bool = False):
    """Causal sliding-window (optionally + strided) attention forward.

    q: [B, Hq, N, d], k/v: [B, Hkv, N, d], all bf16 (or all fp32) on one GPU.
    Returns out [B, Hq, N, d] in the input dtype.  scale defaults to 1/sqrt(d).
    With ``return_lse`` returns (out, lse), lse fp32 [B, Hq, N] the natural
    log of each row's softmax denominator.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    dtype, dev = q.dtype, q.device
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        fn = lib().swa_attn_fwd_lse if dtype == torch.bfloat16 else lib().swa_attn_fwd_lse_f32
        _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, k.shape[1], N, d,
                  int(window), int(stride), float(scale), _stream(dev)))
        return out, lse
    fn = lib().swa_attn_fwd if dtype == torch.bfloat16 else lib().swa_attn_fwd_f32
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, k.shape[1], N, d,
              int(window), int(stride), float(scale), _stream(dev)))
    return out


def attn_fwd_two_sided(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, left: int, right: int,
                       scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Two-sided band attention (no causal cut): row i reads keys i-left .. i+right.

    Shapes, dtypes and device as ``attn_fwd``.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    dtype, dev = q.dtype, q.device
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().swa_attn_fwd_two_sided if dtype == torch.bfloat16 else lib().swa_attn_fwd_two_sided_f32
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, k.shape[1], N, d,
              int(left), int(right), float(scale), _stream(dev)))
    return out


def diff_attn_fwd(q1: torch.Tensor, k1: torch.Tensor, q2: torch.Tensor, k2: torch.Tensor, v: torch.Tensor,
                  lam: torch.Tensor, window: int, scale: float | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Differential sliding-window attention: (A1 - lam[h] * A2) V.

    q1, q2: [B, Hq, N, d]; k1, k2, v: [B, Hkv, N, d]; lam: float32 [Hq] on
    the GPU.  All bf16 (or all fp32).
    """
    if q1.dim() != 4 or q2.shape != q1.shape or k1.dim() != 4 or k2.shape != k1.shape or v.shape != k1.shape:
        raise ValueError("q1/q2 must be [B, Hq, N, d] and k1/k2/v [B, Hkv, N, d]")
    B, Hq, N, d = q1.shape
    if k1.shape[0] != B or k1.shape[2] != N or k1.shape[3] != d:
        raise ValueError("k1, k2, v do not match q1")
    dtype, dev = q1.dtype, q1.device
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q1 must be bfloat16 or float32")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v")):
        _need(t, n, dtype, dev)
    _need(lam, "lam", torch.float32, dev)
    if lam.shape != (Hq,):
        raise ValueError("lam must be [Hq]")
    if out is None:
        out = torch.empty_like(q1)
    _need(out, "out", dtype, dev)
    if out.shape != q1.shape:
        raise ValueError("out must have q1's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().swa_diff_attn_fwd if dtype == torch.bfloat16 else lib().swa_diff_attn_fwd_f32
    _check(fn(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(), lam.data_ptr(),
              out.data_ptr(), B, Hq, k1.shape[1], N, d, int(window), float(scale), _stream(dev)))
    return out


def global_workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, ng: int) -> int:
    return int(lib().swa_attn_fwd_global_workspace_bytes(B, Hq, Hkv, N, d, ng))


def attn_fwd_global(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int, gidx: torch.Tensor,
                    scale: float | None = None, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Causal window plus global positions ``gidx`` (int32, sorted, distinct,
    on the GPU).  Shapes as ``attn_fwd``."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k, v do not match q")
    dtype, dev = q.dtype, q.device
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dtype, dev)
    _need(gidx, "gidx", torch.int32, dev)
    if gidx.dim() != 1:
        raise ValueError("gidx must be 1-D")
    ng = gidx.numel()
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = global_workspace_bytes(B, Hq, k.shape[1], N, d, ng)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().swa_attn_fwd_global if dtype == torch.bfloat16 else lib().swa_attn_fwd_global_f32
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, k.shape[1], N, d, int(window),
              gidx.data_ptr() if ng > 0 else None, ng, float(scale), ws_ptr or None, ws_bytes, _stream(dev)))
    return out


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, window: int) -> int:
    return int(lib().swa_decode_workspace_bytes(B, Hq, Hkv, d, window))


def decode(q: torch.Tensor, kring: torch.Tensor, vring: torch.Tensor, pos: torch.Tensor,
           scale: float | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step over a rolling window-slot cache.

    q: [B, Hq, d]; kring/vring: [B, Hkv, W, d] (window W = kring.shape[2]);
    pos: int32 [B] on the GPU, 1-based absolute position of each query token.
    """
    if q.dim() != 3 or kring.dim() != 4 or vring.shape != kring.shape:
        raise ValueError("q must be [B, Hq, d] and kring/vring [B, Hkv, W, d]")
    B, Hq, d = q.shape
    W = kring.shape[2]
    if kring.shape[0] != B or kring.shape[3] != d:
        raise ValueError("ring shape does not match q")
    if out is not None and (not isinstance(out, torch.Tensor) or out.shape != q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}")
    dtype, dev = q.dtype, q.device
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((q, "q"), (kring, "kring"), (vring, "vring")):
        _need(t, n, dtype, dev)
    _need(pos, "pos", torch.int32, dev)
    if pos.shape != (B,):
        raise ValueError("pos must be [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype, dev)
    need = decode_workspace_bytes(B, Hq, kring.shape[1], d, W)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the same GPU")
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().swa_decode if dtype == torch.bfloat16 else lib().swa_decode_f32
    _check(fn(q.data_ptr(), kring.data_ptr(), vring.data_ptr(), pos.data_ptr(), out.data_ptr(),
              B, Hq, kring.shape[1], d, float(scale), ws_ptr, ws_bytes, W, _stream(dev)))
    return out


def decode_noalloc(q: torch.Tensor, kring: torch.Tensor, vring: torch.Tensor, pos: torch.Tensor,
                   scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """``decode`` (bf16) through the entry point that allocates nothing: the
    split partials live in the library's per-device scratch, shared by every
    call on that GPU (calls that may overlap on one GPU race).  ``out`` must
    be given by callers that cannot allocate; when it is None it is
    allocated here, as in the other wrappers."""
    if q.dim() != 3 or kring.dim() != 4 or vring.shape != kring.shape:
        raise ValueError("q must be [B, Hq, d] and kring/vring [B, Hkv, W, d]")
    B, Hq, d = q.shape
    W = kring.shape[2]
    if kring.shape[0] != B or kring.shape[3] != d:
        raise ValueError("ring shape does not match q")
    if out is not None and (not isinstance(out, torch.Tensor) or out.shape != q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}")
    dev = q.device
    if q.dtype != torch.bfloat16:
        raise TypeError("decode_noalloc takes bfloat16 tensors")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((q, "q"), (kring, "kring"), (vring, "vring")):
        _need(t, n, torch.bfloat16, dev)
    _need(pos, "pos", torch.int32, dev)
    if pos.shape != (B,):
        raise ValueError("pos must be [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib().swa_decode_noalloc(q.data_ptr(), kring.data_ptr(), vring.data_ptr(), pos.data_ptr(),
                                    out.data_ptr(), B, Hq, kring.shape[1], d, float(scale), W, _stream(dev)))
    return out


def chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kring: torch.Tensor, vring: torch.Tensor,
                  p0: torch.Tensor, scale: float | None = None, out: torch.Tensor | None = None,
                  return_lse: bool = False):
    """A chunk of new tokens over the rolling-cache history plus itself.

    q: [B, Hq, T, d]; k, v: [B, Hkv, T, d]; kring, vring: [B, Hkv, W, d]
    holding positions up to p0 (int32 [B] on the GPU).  Call before
    ``ring_append`` of the same chunk.  With ``return_lse`` returns (out, lse),
    lse fp32 [B, Hq, T] as for ``attn_fwd``.
    """
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or kring.dim() != 4 or vring.shape != kring.shape:
        raise ValueError("q, k, v must be [B, H, T, d] and kring, vring [B, Hkv, W, d]")
    B, Hq, T, d = q.shape
    if k.shape[0] != B or k.shape[2] != T or k.shape[3] != d:
        raise ValueError("k, v do not match q")
    if kring.shape[0] != B or kring.shape[1] != k.shape[1] or kring.shape[3] != d:
        raise ValueError("rings do not match k, v")
    dtype, dev = q.dtype, q.device
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (kring, "kring"), (vring, "vring")):
        _need(t, n, dtype, dev)
    _need(p0, "p0", torch.int32, dev)
    if p0.shape != (B,):
        raise ValueError("p0 must be [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if return_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
        fn = lib().swa_chunk_prefill_lse if dtype == torch.bfloat16 else lib().swa_chunk_prefill_lse_f32
        _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), kring.data_ptr(), vring.data_ptr(), p0.data_ptr(),
                  out.data_ptr(), lse.data_ptr(), B, Hq, k.shape[1], T, d, kring.shape[2], float(scale),
                  _stream(dev)))
        return out, lse
    fn = lib().swa_chunk_prefill if dtype == torch.bfloat16 else lib().swa_chunk_prefill_f32
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), kring.data_ptr(), vring.data_ptr(), p0.data_ptr(),
              out.data_ptr(), B, Hq, k.shape[1], T, d, kring.shape[2], float(scale), _stream(dev)))
    return out


def ring_append(k: torch.Tensor, v: torch.Tensor, p0: torch.Tensor, kring: torch.Tensor, vring: torch.Tensor):
    """Write a chunk's K/V rows into the rolling cache in place (slot (p0+r) % W)."""
    if k.dim() != 4 or v.shape != k.shape or kring.dim() != 4 or vring.shape != kring.shape:
        raise ValueError("k, v must be [B, Hkv, T, d] and kring, vring [B, Hkv, W, d]")
    B, Hkv, T, d = k.shape
    if kring.shape[0] != B or kring.shape[1] != Hkv or kring.shape[3] != d:
        raise ValueError("rings do not match k, v")
    dtype, dev = k.dtype, k.device
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("k must be bfloat16 or float32")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t, n in ((k, "k"), (v, "v"), (kring, "kring"), (vring, "vring")):
        _need(t, n, dtype, dev)
    _need(p0, "p0", torch.int32, dev)
    if p0.shape != (B,):
        raise ValueError("p0 must be [B]")
    fn = lib().swa_ring_append if dtype == torch.bfloat16 else lib().swa_ring_append_f32
    _check(fn(k.data_ptr(), v.data_ptr(), p0.data_ptr(), kring.data_ptr(), vring.data_ptr(), B, Hkv, T, d,
              kring.shape[2], _stream(dev)))
