"""Python binding for libfattn (exact tiled attention on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfattn.so``.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or refuses a call,
an exception is raised.

Names mirror the C ABI in ``include/fattn.h``:
    fa_fwd(q, k, v, ...)        bf16 forward  -> (o, lse)
    fa_fwd_f32(q, k, v, ...)    fp32 forward  -> (o, lse)
    fa_fwd_local(q, k, v, window, ...)  bf16 sliding-window causal forward -> (o, lse)
    fa_fwd_fp8(q, k, v, descale_q, descale_k, descale_v, ...)  FP8 (e4m3) forward -> (o bf16, lse)
    fa_bwd(q, k, v, o, lse, dO, ...)  bf16 backward -> (dq, dk, dv)
    fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, ...)  the same backward with
                                the library's fixed device scratch (no workspace)
    fa_bwd_workspace_bytes(B, H, Hkv, N, d)
    fa_debug_counters(out[4], reset)   (counters_lib(), read_counters(): debug build)
    fa_status_string(status)
"""
from __future__ import annotations

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfattn.so")
# the same library built with the forward's device counters (debug build)
COUNTERS_LIB_PATH = os.path.join(PKG_DIR, "libfattn_counters.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_ERR_TOO_LARGE = -4

# C prototypes (kept in step with include/fattn.h)
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
PROTOTYPES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_local": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "fa_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "fa_debug_counters": (_I, [ctypes.POINTER(ctypes.c_ulonglong), _I]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
}

_lib = None


class FattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """The loaded libfattn with prototypes set.  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libfattn is not built ({LIB_PATH} missing); run "
                "`python -c 'import __graft_entry__ as g; g.build()'` or "
                "`python -m exact_tiled_attention_31_amd._build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def counters_lib() -> ctypes.CDLL:
    """The debug build (libfattn_counters.so) with prototypes set: the same C
    ABI, plus device counters in the bf16 forward that fa_debug_counters
    reads.  Raises if it is not built."""
    if not os.path.exists(COUNTERS_LIB_PATH):
        raise ImportError(f"{COUNTERS_LIB_PATH} is not built; run the build")
    h = ctypes.CDLL(COUNTERS_LIB_PATH)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    return h


def read_counters(handle: ctypes.CDLL, reset: bool = False) -> dict:
    """fa_debug_counters through `handle` as a dict."""
    out = (ctypes.c_ulonglong * 4)()
    st = handle.fa_debug_counters(out, int(bool(reset)))
    if st != FA_OK:
        raise FattnError(st, "fa_debug_counters")
    return dict(zip(("tiles_computed", "tiles_skipped", "tiles_masked", "reference_raises"),
                    (int(x) for x in out)))


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def fa_bwd_workspace_bytes(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, Hkv, N, d))


# ---------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _stream_of(t, stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/hip) tensor, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, H, Hkv, N, d


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _fwd(cname, dtype, q, k, v, o, lse, mode: int, scale, stream):
    """Shared marshalling; ``mode`` is the call's int argument after d (causal
    flag or window)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dtype)
    B, H, Hkv, N, d = _dims(q, k, v)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _need(o, "o", dtype, (B, H, N, d))
    _need(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = getattr(lib(), cname)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               B, H, Hkv, N, d, int(mode), float(scale),
                               _stream_of(q, stream))
    if st != FA_OK:
        raise FattnError(st, cname)
    return o, lse


def fa_fwd(q, k, v, o=None, lse=None, causal: bool = False, scale: float | None = None,
           stream=None):
    """bf16 forward.  q [B,H,N,d], k, v [B,Hkv,N,d] (torch.bfloat16, contiguous,
    on the GPU).  Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N]); o and lse are
    allocated when not given.  scale defaults to 1/sqrt(d)."""
    return _fwd("fa_fwd", _torch().bfloat16, q, k, v, o, lse, int(bool(causal)), scale, stream)


def fa_fwd_local(q, k, v, window: int, o=None, lse=None, scale: float | None = None,
                 stream=None):
    """bf16 local (sliding-window) causal forward: query i sees keys
    i - window + 1 .. i.  Same tensors and defaults as fa_fwd."""
    return _fwd("fa_fwd_local", _torch().bfloat16, q, k, v, o, lse, int(window), scale, stream)


def fa_fwd_fp8(q, k, v, descale_q: float, descale_k: float, descale_v: float, o=None, lse=None,
               causal: bool = False, scale: float | None = None, stream=None):
    """FP8 forward.  q [B,H,N,d], k, v [B,Hkv,N,d] hold OCP e4m3 codes
    (torch.uint8 or torch.float8_e4m3fn, contiguous, on the GPU) whose values
    are descale_x * e4m3(code).  Returns (o bf16 [B,H,N,d], lse fp32
    [B,H,N]), allocated when not given.  scale defaults to 1/sqrt(d)."""
    torch = _torch()
    allowed = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in allowed:
            raise TypeError(f"{name} must be torch.uint8 or torch.float8_e4m3fn codes")
        _need(t, name, t.dtype)
    B, H, Hkv, N, d = _dims(q, k, v)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, (B, H, N, d))
    _need(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                          int(bool(causal)), float(scale), float(descale_q), float(descale_k),
                          float(descale_v), _stream_of(q, stream))
    if st != FA_OK:
        raise FattnError(st, "fa_fwd_fp8")
    return o, lse


def fa_fwd_f32(q, k, v, o=None, lse=None, causal: bool = False, scale: float | None = None,
               stream=None):
    """fp32 forward (same contract as fa_fwd with torch.float32 tensors)."""
    return _fwd("fa_fwd_f32", _torch().float32, q, k, v, o, lse, int(bool(causal)), scale,
                stream)


def fa_bwd(q, k, v, o, lse, do, dq=None, dk=None, dv=None, workspace=None,
           causal: bool = False, scale: float | None = None, stream=None):
    """bf16 backward with recomputation.  Returns (dq, dk, dv), allocated
    when not given; ``workspace`` (a uint8 device tensor of at least
    fa_bwd_workspace_bytes bytes) is allocated when not given."""
    torch = _torch()
    bf = torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(t, name, bf)
    B, H, Hkv, N, d = _dims(q, k, v)
    _need(o, "o", bf, (B, H, N, d))
    _need(do, "do", bf, (B, H, N, d))
    _need(lse, "lse", torch.float32, (B, H, N))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", bf, (B, H, N, d))
    _need(dk, "dk", bf, (B, Hkv, N, d))
    _need(dv, "dv", bf, (B, Hkv, N, d))
    need = fa_bwd_workspace_bytes(B, H, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                      B, H, Hkv, N, d, int(bool(causal)), float(scale), _stream_of(q, stream))
    if st != FA_OK:
        raise FattnError(st, "fa_bwd")
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, causal: bool = False,
                   scale: float | None = None, stream=None):
    """fa_bwd through the allocation-free entry point: the caller passes the
    output tensors, and the per-row D terms go to the library's fixed device
    scratch (B*H*N <= 2^22).  Nothing is allocated here or in the library."""
    torch = _torch()
    bf = torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(t, name, bf)
    B, H, Hkv, N, d = _dims(q, k, v)
    _need(o, "o", bf, (B, H, N, d))
    _need(do, "do", bf, (B, H, N, d))
    _need(lse, "lse", torch.float32, (B, H, N))
    _need(dq, "dq", bf, (B, H, N, d))
    _need(dk, "dk", bf, (B, Hkv, N, d))
    _need(dv, "dv", bf, (B, Hkv, N, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                              _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d,
                              int(bool(causal)), float(scale), _stream_of(q, stream))
    if st != FA_OK:
        raise FattnError(st, "fa_bwd_noalloc")
    return dq, dk, dv


__all__ = ["fa_fwd", "fa_fwd_f32", "fa_fwd_local", "fa_fwd_fp8", "fa_bwd", "fa_bwd_noalloc",
           "fa_bwd_workspace_bytes", "fa_status_string", "counters_lib", "read_counters",
           "FattnError", "lib", "LIB_PATH", "PROTOTYPES",
           "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_TOO_LARGE"]
