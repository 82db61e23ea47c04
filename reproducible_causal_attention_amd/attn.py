"""ctypes binding of libattn.so (include/attn.h) for torch tensors.

Argument marshalling only: every step of the attention path runs in the HIP
kernels of the library.  torch supplies device memory (``torch.empty``) and the
stream (``torch.cuda.current_stream()``).  If the library is missing the calls
raise; there is no fallback.

Layouts: q, o, dO, dq are [B, T, Hq, D]; k, v, dk, dv are [B, T, Hkv, D]
(contiguous, one dtype: bfloat16, float16 or float32; D = 64, or 128 for the
16-bit types); lse and delta are [B, Hq, T] float32.  The rotary variants take
cos and sin tables [T, D/2] float32 (bf16 / fp16 only).  Every wrapper checks
the shapes, dtypes and device of all its tensors against q before it hands a
pointer to the library, which sizes every buffer from q's shape.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

from . import build as _build

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2

EXPORTED = (
    "attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_preprocess",
    "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dkdv_dq", "attn_fwd_rope",
    "attn_bwd_rope_workspace_bytes", "attn_bwd_rope", "attn_status_string", "attn_build_info",
    "attn_bwd_noalloc",
)

# Bytes of the per-GPU array attn_bwd_noalloc keeps its delta rows in
# (ATTN_NOALLOC_SCRATCH_BYTES in include/attn.h).
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _build.LIB_PATH


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m reproducible_causal_attention_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sizes = [I, I, I, I, I]
    lib.attn_fwd.argtypes = [P, P, P, P, P, *sizes, F, I, I, P]
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, *sizes, F, I, I, P, Z, P]
    lib.attn_bwd_workspace_bytes.argtypes = [*sizes, I]
    lib.attn_bwd_workspace_bytes.restype = Z
    lib.attn_bwd_preprocess.argtypes = [P, P, P, I, I, I, I, I, P]
    lib.attn_bwd_dkdv.argtypes = [P, P, P, P, P, P, P, P, *sizes, F, I, I, P]
    lib.attn_bwd_dq.argtypes = [P, P, P, P, P, P, P, *sizes, F, I, I, P]
    lib.attn_bwd_dkdv_dq.argtypes = [P, P, P, P, P, P, P, P, P, *sizes, F, I, I, P]
    lib.attn_fwd_rope.argtypes = [P, P, P, P, P, P, P, *sizes, F, I, I, P]
    lib.attn_bwd_rope_workspace_bytes.argtypes = [*sizes, I]
    lib.attn_bwd_rope_workspace_bytes.restype = Z
    lib.attn_bwd_rope.argtypes = [P, P, P, P, P, P, P, P, P, P, P, *sizes, F, I, I, P, Z, P]
    lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, *sizes, F, I, I, P]
    for name in ("attn_fwd", "attn_bwd", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq",
                 "attn_bwd_dkdv_dq", "attn_fwd_rope", "attn_bwd_rope", "attn_bwd_noalloc"):
        getattr(lib, name).restype = I
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_build_info.argtypes = []
    lib.attn_build_info.restype = ctypes.c_char_p
    if path == library_path():
        _lib = lib
    return lib


def build_info() -> str:
    return load_library().attn_build_info().decode()


def _check(status: int):
    if status != ATTN_OK:
        lib = load_library()
        raise AttnError(status, lib.attn_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16, torch.float16 or torch.float32")


def _ptr(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _shapes(q, k, v=None, *, o=None, dO=None, lse=None, delta=None):
    """(B, T, Hq, Hkv, D) from q and k, after checking every given tensor against them.

    The C ABI sizes every buffer from these five numbers, so a tensor of another
    shape, dtype or device would be read or written out of its bounds: raise
    ValueError instead.  q, k, v, o, dO share q's dtype and device; k and v are
    [B, T, Hkv, D]; o and dO are q's shape; lse and delta are [B, Hq, T] float32.
    """
    if not isinstance(q, torch.Tensor) or not isinstance(k, torch.Tensor):
        raise ValueError("q and k must be torch tensors")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, T, Hq, D] and k, v [B, T, Hkv, D]")
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    kv_shape = (B, T, Hkv, D)
    checks = [("k", k, kv_shape)]
    if v is not None:
        checks.append(("v", v, kv_shape))
    for name, t in (("o", o), ("dO", dO)):
        if t is not None:
            checks.append((name, t, tuple(q.shape)))
    for name, t, shape in checks:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} is {t.dtype} but q is {q.dtype}: all inputs share one dtype")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device} but q is on {q.device}")
    for name, t in (("lse", lse), ("delta", delta)):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if tuple(t.shape) != (B, Hq, T) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 of shape {(B, Hq, T)}, "
                             f"got {t.dtype} {tuple(t.shape)}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device} but q is on {q.device}")
    return B, T, Hq, Hkv, D


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _workspace(workspace, nbytes: int, device):
    """The caller's workspace (any dtype, sized in bytes; the library checks the
    size), or a new one of ``nbytes`` bytes on ``device``."""
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError(f"workspace must be a tensor on {device}")
    return workspace


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def fwd(q, k, v, scale=None, causal=True):
    """Forward: returns ``(o [B,T,Hq,D], lse [B,Hq,T] float32)``."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq, Hkv, D,
                        scale, int(bool(causal)), _dtype_code(q), _stream()))
    return o, lse


def workspace_bytes(B, T, Hq, Hkv, D, dtype_code) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, T, Hq, Hkv, D, dtype_code))


def bwd(q, k, v, o, lse, dO, scale=None, causal=True, workspace=None):
    """Backward of sum(o * dO): returns ``(dq, dk, dv)``."""
    B, T, Hq, Hkv, D = _shapes(q, k, v, o=o, dO=dO, lse=lse)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = workspace_bytes(B, T, Hq, Hkv, D, _dtype_code(q))
    workspace = _workspace(workspace, nbytes, q.device)
    _check(lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                        _ptr(dk), _ptr(dv), B, T, Hq, Hkv, D, scale, int(bool(causal)),
                        _dtype_code(q), _ptr(workspace), _nbytes(workspace), _stream()))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dO, scale=None, causal=True):
    """``bwd`` through attn_bwd_noalloc (delta in the library's per-GPU array, no
    workspace): returns ``(dq, dk, dv)``, bitwise those of ``bwd``."""
    B, T, Hq, Hkv, D = _shapes(q, k, v, o=o, dO=dO, lse=lse)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, T, Hq, Hkv, D, scale,
                                int(bool(causal)), _dtype_code(q), _stream()))
    return dq, dk, dv


def bwd_preprocess(o, dO):
    """delta = rowsum(dO * o) as [B, Hq, T] float32."""
    if not isinstance(o, torch.Tensor) or o.dim() != 4:
        raise ValueError("o must be [B, T, Hq, D]")
    _shapes(o, o, o, dO=dO)
    B, T, Hq, D = o.shape
    lib = load_library()
    delta = torch.empty((B, Hq, T), dtype=torch.float32, device=o.device)
    _check(lib.attn_bwd_preprocess(_ptr(o), _ptr(dO), _ptr(delta), B, T, Hq, D,
                                   _dtype_code(o), _stream()))
    return delta


def bwd_dkdv(q, k, v, dO, lse, delta, scale=None, causal=True):
    B, T, Hq, Hkv, D = _shapes(q, k, v, dO=dO, lse=lse, delta=delta)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    _check(lib.attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta),
                             _ptr(dk), _ptr(dv), B, T, Hq, Hkv, D, scale, int(bool(causal)),
                             _dtype_code(q), _stream()))
    return dk, dv


def bwd_dq(q, k, v, dO, lse, delta, scale=None, causal=True):
    B, T, Hq, Hkv, D = _shapes(q, k, v, dO=dO, lse=lse, delta=delta)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    dq = torch.empty_like(q)
    _check(lib.attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta),
                           _ptr(dq), B, T, Hq, Hkv, D, scale, int(bool(causal)),
                           _dtype_code(q), _stream()))
    return dq


def bwd_dkdv_dq(q, k, v, dO, lse, delta, scale=None, causal=True):
    """dK/dV and dQ co-launched in one grid: returns ``(dq, dk, dv)``, bitwise those
    of ``bwd_dkdv`` and ``bwd_dq``."""
    B, T, Hq, Hkv, D = _shapes(q, k, v, dO=dO, lse=lse, delta=delta)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib.attn_bwd_dkdv_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, T, Hq, Hkv, D, scale,
                                int(bool(causal)), _dtype_code(q), _stream()))
    return dq, dk, dv


def _tables(cos, sin, T, D):
    for t in (cos, sin):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or tuple(t.shape) != (T, D // 2):
            raise ValueError(f"rotary tables must be float32 [T, D/2] = [{T}, {D // 2}]")
    return _ptr(cos), _ptr(sin)


def fwd_rope(q, k, v, cos, sin, scale=None, causal=True):
    """Forward with rotary embedding of q and k (adjacent pairs, tables [T, D/2]):
    returns ``(o, lse)``."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    pc, ps = _tables(cos, sin, T, D)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(lib.attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), pc, ps, _ptr(o), _ptr(lse), B, T, Hq,
                             Hkv, D, scale, int(bool(causal)), _dtype_code(q), _stream()))
    return o, lse


def rope_workspace_bytes(B, T, Hq, Hkv, D, dtype_code) -> int:
    return int(load_library().attn_bwd_rope_workspace_bytes(B, T, Hq, Hkv, D, dtype_code))


def bwd_rope(q, k, v, o, lse, dO, cos, sin, scale=None, causal=True, workspace=None):
    """Backward of ``fwd_rope``: ``(dq, dk, dv)`` with respect to the unrotated q, k, v."""
    B, T, Hq, Hkv, D = _shapes(q, k, v, o=o, dO=dO, lse=lse)
    lib = load_library()
    scale = default_scale(D) if scale is None else float(scale)
    pc, ps = _tables(cos, sin, T, D)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = rope_workspace_bytes(B, T, Hq, Hkv, D, _dtype_code(q))
    workspace = _workspace(workspace, nbytes, q.device)
    _check(lib.attn_bwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), pc, ps,
                             _ptr(dq), _ptr(dk), _ptr(dv), B, T, Hq, Hkv, D, scale,
                             int(bool(causal)), _dtype_code(q), _ptr(workspace), _nbytes(workspace),
                             _stream()))
    return dq, dk, dv
