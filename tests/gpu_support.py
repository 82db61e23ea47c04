"""Helpers shared by the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI, compare with the oracle, hash outputs."""
from __future__ import annotations

import contextlib
import ctypes
import hashlib
import sys

import numpy as np
import pytest
import torch

import oracle
from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import workloads as W

# Tolerances, max |gpu - ref| / max |ref| per tensor (lse: absolute, in nats).
TOL = {
    "f32": {"o": 1e-4, "lse": 1e-4, "dq": 1e-3, "dk": 1e-3, "dv": 1e-3, "delta": 1e-4},
    "bf16": {"o": 2e-2, "lse": 2e-2, "dq": 2e-2, "dk": 2e-2, "dv": 2e-2, "delta": 2e-2},
    # fp16 rounds to 11 significant bits (bf16: 8): the errors measured at
    # 1x512 and 4x1024 are ~8x below bf16's (<= 6e-4); 2e-3 keeps a 3x margin.
    "f16": {"o": 2e-3, "lse": 2e-3, "dq": 2e-3, "dk": 2e-3, "dv": 2e-3, "delta": 2e-3},
}


def say(*args):
    """Name the case before each GPU step, flushed, so a crash still identifies it."""
    print("[gpu-case]", *args, file=sys.stderr, flush=True)


def to_device(inp: W.Inputs):
    dev = torch.device("cuda:0")
    out = []
    for name in ("q", "k", "v", "dO"):
        a = getattr(inp, name)
        if inp.workload.dtype == "bf16":
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        elif inp.workload.dtype == "f16":
            t = torch.from_numpy(a.view(np.int16)).view(torch.float16)
        else:
            t = torch.from_numpy(a)
        out.append(t.to(dev))
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(inp: W.Inputs, tensors=None):
    """fwd + bwd on the GPU; returns dict of device tensors."""
    w = inp.workload
    q, k, v, dO = tensors if tensors is not None else to_device(inp)
    o, lse = A.fwd(q, k, v, w.scale, w.causal)
    delta = A.bwd_preprocess(o, dO)
    dq, dk, dv = A.bwd(q, k, v, o, lse, dO, w.scale, w.causal)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv}


def rel_err(a, b):
    den = max(float(np.max(np.abs(b))), 1e-30)
    return float(np.max(np.abs(a - b))) / den


GRADS = ("dq", "dk", "dv")


def check_against(gpu: dict, ref: dict, dtype: str, where=""):
    """Assert every tensor in ``ref`` is within tolerance; return the errors.

    Errors are max |gpu - ref| / max |ref| per tensor (lse: absolute).  A gradient
    whose exact value is (close to) zero everywhere -- dq and dk of a single token,
    for instance -- is measured against 1e-3 of the largest gradient reference
    instead, so rounding noise in a cancelling sum is not divided by zero.
    """
    grad_scale = max((float(np.max(np.abs(ref[n]))) for n in GRADS if n in ref), default=0.0)
    errs = {}
    for name, r in ref.items():
        g = gpu[name]
        assert g.shape == r.shape, (name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{where}: non-finite values in {name}"
        if name == "lse":
            e = float(np.max(np.abs(g - r)))
        else:
            den = float(np.max(np.abs(r)))
            if name in GRADS:
                den = max(den, 1e-3 * grad_scale)
            e = float(np.max(np.abs(g - r))) / max(den, 1e-30)
        errs[name] = e
    bad = {n: e for n, e in errs.items() if e > TOL[dtype][n]}
    assert not bad, f"{where}: out of tolerance {bad} (all errors {errs})"
    return errs


def oracle_full(inp: W.Inputs):
    w = inp.workload
    q, k, v, dO = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    o, lse = oracle.ref_fwd(q, k, v, w.scale, w.causal)
    dq, dk, dv, delta = oracle.ref_bwd(q, k, v, dO, w.scale, w.causal)
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv}


def sampled_units(w: W.Workload, n: int = 3):
    """Deterministic (b, g) units: first, last and one in the middle."""
    units = [(0, 0), (w.B - 1, w.Hkv - 1), (w.B // 2, w.Hkv // 2)]
    seen = []
    for u in units:
        if u not in seen:
            seen.append(u)
    return seen[:n]


def check_units(inp: W.Inputs, gpu_np: dict, units, where=""):
    """Compare the GPU result with the oracle on sampled (batch, KV-group) units."""
    w = inp.workload
    q, k, v, dO = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    G = w.G
    errs = []
    for b, g in units:
        o_r, lse_r = oracle.ref_fwd_group(q, k, v, w.scale, w.causal, b, g)
        dq_r, dk_r, dv_r, dl_r = oracle.ref_bwd_group(q, k, v, dO, w.scale, w.causal, b, g)
        hs = slice(g * G, (g + 1) * G)
        gpu_u = {"o": gpu_np["o"][b, :, hs], "lse": gpu_np["lse"][b, hs],
                 "delta": gpu_np["delta"][b, hs], "dq": gpu_np["dq"][b, :, hs],
                 "dk": gpu_np["dk"][b, :, g], "dv": gpu_np["dv"][b, :, g]}
        ref_u = {"o": o_r, "lse": lse_r, "delta": dl_r, "dq": dq_r, "dk": dk_r, "dv": dv_r}
        errs.append(check_against(gpu_u, ref_u, w.dtype, f"{where} unit b={b} g={g}"))
    return errs


def sha256_outputs(gpu: dict) -> str:
    h = hashlib.sha256()
    for name in ("o", "lse", "dq", "dk", "dv"):
        t = gpu[name].contiguous()
        h.update(t.view(torch.uint8).cpu().numpy().tobytes() if t.dtype != torch.bfloat16
                 else t.view(torch.int16).cpu().numpy().tobytes())
    return h.hexdigest()


def as_numpy(gpu: dict) -> dict:
    return {n: to_f64(t) for n, t in gpu.items()}


def unit_rows(T: int):
    """Query rows checked in every unit: tile and block edges, the middle, the last."""
    return sorted({r for r in (0, 31, 32, 127, 128, T // 2 + 5, T - 1) if 0 <= r < T})


def check_every_unit(inp: W.Inputs, gpu_np: dict, where="", n_keys: int = 32):
    """Every (batch, KV-group) unit against the row-wise oracle.

    For each unit: o, lse, delta and dq of the rows of ``unit_rows`` of every
    query head of the group (``oracle.ref_query_rows``), dk and dv of the last
    ``n_keys`` keys of the KV head (``oracle.ref_key_rows``), each to the
    tolerances of ``check_against`` relative to the checked rows; and the two
    exact-math column sums over all T keys of the unit -- sum_j dv_j equals the sum
    of dO over the group's query rows (rows of P sum to one) and sum_j dk_j = 0
    (shifting every key by one vector leaves P unchanged) -- to the dtype's
    tolerance relative to sum |dO| and to the largest column sum of |dk|.  A unit
    computed for the wrong (batch, group) slot, or not at all, fails here.
    """
    w = inp.workload
    q, k, v, dO = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    G, T = w.G, w.T
    rows = unit_rows(T)
    keys = list(range(max(0, T - n_keys), T))
    tol = TOL[w.dtype]["dv"]
    worst = {}
    for b in range(w.B):
        for g in range(w.Hkv):
            ref_u = {"o": [], "lse": [], "delta": [], "dq": []}
            gpu_u = {"o": [], "lse": [], "delta": [], "dq": []}
            for h in range(g * G, (g + 1) * G):
                r = oracle.ref_query_rows(q, k, v, dO, w.scale, w.causal, b, h, rows)
                for n in ref_u:
                    ref_u[n].append(r[n])
                gpu_u["o"].append(gpu_np["o"][b, rows, h])
                gpu_u["dq"].append(gpu_np["dq"][b, rows, h])
                gpu_u["lse"].append(gpu_np["lse"][b, h, rows])
                gpu_u["delta"].append(gpu_np["delta"][b, h, rows])
            ref_u = {n: np.concatenate(a) for n, a in ref_u.items()}
            gpu_u = {n: np.concatenate(a) for n, a in gpu_u.items()}
            ref_u["dk"], ref_u["dv"] = oracle.ref_key_rows(q, k, v, dO, w.scale, w.causal, b, g, keys)
            gpu_u["dk"], gpu_u["dv"] = gpu_np["dk"][b, keys, g], gpu_np["dv"][b, keys, g]
            errs = check_against(gpu_u, ref_u, w.dtype, f"{where} unit b={b} g={g}")
            dO_g = dO[b, :, g * G:(g + 1) * G]
            want = dO_g.sum(axis=(0, 1))
            got = gpu_np["dv"][b, :, g].sum(axis=0)
            errs["dv_colsum"] = float(np.max(np.abs(got - want)) / np.abs(dO_g).sum(axis=(0, 1)).max())
            dk_u = gpu_np["dk"][b, :, g]
            errs["dk_colsum"] = float(np.max(np.abs(dk_u.sum(axis=0))) / np.abs(dk_u).sum(axis=0).max())
            assert errs["dv_colsum"] <= tol and errs["dk_colsum"] <= tol, (where, b, g, errs)
            for n, e in errs.items():
                worst[n] = max(worst.get(n, 0.0), e)
    return worst


def loaded_hip_runtime():
    """The HIP runtime library this process already uses (torch's and the attention
    library's), so a stream created through it is valid for both."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("libamdhip64 is not loaded")


@contextlib.contextmanager
def cu_masked_stream(mask_kind: str):
    """Make the current torch stream one that may use only some CUs: "first-half-cus"
    or "first-16-cus".  Skips the test if the runtime refuses the mask."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    words = (n_cu + 31) // 32
    if mask_kind == "first-half-cus":
        mask = [0xFFFFFFFF] * (words // 2) + [0] * (words - words // 2)
    elif mask_kind == "first-16-cus":
        mask = [0x0000FFFF] + [0] * (words - 1)
    else:
        raise ValueError(mask_kind)
    hip = loaded_hip_runtime()
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    handle = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), words, (ctypes.c_uint32 * words)(*mask))
    if rc != 0:
        hip.hipGetErrorString.restype = ctypes.c_char_p
        hip.hipGetLastError()  # the failed call leaves its error pending
        pytest.skip(f"hipExtStreamCreateWithCUMask failed: {rc} {hip.hipGetErrorString(rc).decode()}")
    try:
        with torch.cuda.stream(torch.cuda.ExternalStream(handle.value)):
            yield
    finally:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        hip.hipStreamDestroy(handle)
