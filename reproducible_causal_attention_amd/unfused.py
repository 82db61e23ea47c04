"""ctypes binding of libattn_unfused.so (include/attn_unfused.h): the unfused
attention baseline, for torch tensors.

Argument marshalling only: the GEMMs run in rocBLAS and the row kernels in the
library's HIP code.  Layouts as in ``attn``; bfloat16 or float16 only.  If the
library is missing the calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import attn as _attn
from . import build as _build

EXPORTED = (
    "attn_unfused_create", "attn_unfused_destroy", "attn_unfused_workspace_bytes",
    "attn_unfused_fwd", "attn_unfused_bwd", "attn_unfused_softmax_lse",
    "attn_unfused_probs_from_lse", "attn_unfused_softmax_bwd",
)

_lib = None


def library_path() -> str:
    return _build.UNFUSED_LIB_PATH


def load_library(path: str | None = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m reproducible_causal_attention_amd.build`; "
                           "there is no fallback path")
    lib = ctypes.CDLL(path)
    P, I, F, Z, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_longlong
    sizes = [I, I, I, I, I]
    lib.attn_unfused_create.argtypes = [ctypes.POINTER(P)]
    lib.attn_unfused_create.restype = I
    lib.attn_unfused_destroy.argtypes = [P]
    lib.attn_unfused_destroy.restype = None
    lib.attn_unfused_workspace_bytes.argtypes = [*sizes, I]
    lib.attn_unfused_workspace_bytes.restype = Z
    lib.attn_unfused_fwd.argtypes = [P, P, P, P, P, P, *sizes, F, I, I, P, Z, P]
    lib.attn_unfused_bwd.argtypes = [P, P, P, P, P, P, P, P, P, *sizes, F, I, I, P, Z, P]
    lib.attn_unfused_softmax_lse.argtypes = [P, P, P, L, I, F, I, I, P]
    lib.attn_unfused_probs_from_lse.argtypes = [P, P, P, L, I, F, I, I, P]
    lib.attn_unfused_softmax_bwd.argtypes = [P, P, P, L, I, I, I, P]
    for name in ("attn_unfused_fwd", "attn_unfused_bwd", "attn_unfused_softmax_lse",
                 "attn_unfused_probs_from_lse", "attn_unfused_softmax_bwd"):
        getattr(lib, name).restype = I
    if path == library_path():
        _lib = lib
    return lib


def _check(status: int):
    if status != _attn.ATTN_OK:
        raise _attn.AttnError(status, _attn.load_library().attn_status_string(status).decode())


class Context:
    """Owns a rocBLAS handle (attn_unfused_create); use from one thread at a time."""

    def __init__(self):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.attn_unfused_create(ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            torch.cuda.synchronize()
            self._lib.attn_unfused_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def workspace_bytes(B, T, Hq, Hkv, D, dtype_code) -> int:
    return int(load_library().attn_unfused_workspace_bytes(B, T, Hq, Hkv, D, dtype_code))


def _workspace(q, k, workspace):
    B, T, Hq, Hkv, D = _attn._shapes(q, k)
    n = workspace_bytes(B, T, Hq, Hkv, D, _attn._dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    return workspace


def fwd(ctx: Context, q, k, v, scale=None, causal=True, workspace=None):
    """Unfused forward: ``(o, lse)``."""
    lib = load_library()
    B, T, Hq, Hkv, D = _attn._shapes(q, k)
    scale = _attn.default_scale(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    ws = _workspace(q, k, workspace)
    _check(lib.attn_unfused_fwd(ctx.handle, _attn._ptr(q), _attn._ptr(k), _attn._ptr(v),
                                _attn._ptr(o), _attn._ptr(lse), B, T, Hq, Hkv, D, scale,
                                int(bool(causal)), _attn._dtype_code(q), _attn._ptr(ws),
                                ws.numel(), _attn._stream()))
    return o, lse


def bwd(ctx: Context, q, k, v, lse, dO, scale=None, causal=True, workspace=None):
    """Unfused backward: ``(dq, dk, dv)``."""
    lib = load_library()
    B, T, Hq, Hkv, D = _attn._shapes(q, k)
    scale = _attn.default_scale(D) if scale is None else float(scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = _workspace(q, k, workspace)
    _check(lib.attn_unfused_bwd(ctx.handle, _attn._ptr(q), _attn._ptr(k), _attn._ptr(v),
                                _attn._ptr(lse), _attn._ptr(dO), _attn._ptr(dq), _attn._ptr(dk),
                                _attn._ptr(dv), B, T, Hq, Hkv, D, scale, int(bool(causal)),
                                _attn._dtype_code(q), _attn._ptr(ws), ws.numel(),
                                _attn._stream()))
    return dq, dk, dv


def softmax_lse(s, scale, causal, dtype):
    """Row kernel alone: s [..., T, T] float32 -> (p in ``dtype``, lse [...T])."""
    lib = load_library()
    T = s.shape[-1]
    n_rows = s.numel() // T
    p = torch.empty(s.shape, dtype=dtype, device=s.device)
    lse = torch.empty(s.shape[:-1], dtype=torch.float32, device=s.device)
    _check(lib.attn_unfused_softmax_lse(_attn._ptr(s), _attn._ptr(p), _attn._ptr(lse), n_rows, T,
                                        float(scale), int(bool(causal)), _attn._dtype_code(p),
                                        _attn._stream()))
    return p, lse


def probs_from_lse(s, lse, scale, causal, dtype):
    lib = load_library()
    T = s.shape[-1]
    p = torch.empty(s.shape, dtype=dtype, device=s.device)
    _check(lib.attn_unfused_probs_from_lse(_attn._ptr(s), _attn._ptr(lse), _attn._ptr(p),
                                           s.numel() // T, T, float(scale), int(bool(causal)),
                                           _attn._dtype_code(p), _attn._stream()))
    return p


def softmax_bwd(p, dp, causal):
    lib = load_library()
    T = p.shape[-1]
    ds = torch.empty_like(p)
    _check(lib.attn_unfused_softmax_bwd(_attn._ptr(p), _attn._ptr(dp), _attn._ptr(ds),
                                        p.numel() // T, T, int(bool(causal)),
                                        _attn._dtype_code(p), _attn._stream()))
    return ds
