"""The Python binding checks every tensor against q before any pointer reaches the
library (which sizes all buffers from q's shape).  The checks come before the
device check, so they run here on CPU tensors; a call that passes them would
then be refused for being on the CPU, so nothing is ever launched."""
import pytest
import torch

from reproducible_causal_attention_amd import attn as A

B, T, HQ, HKV, D = 2, 16, 6, 2, 64
BF = torch.bfloat16


def z(*shape, dtype=BF):
    return torch.zeros(*shape, dtype=dtype)


def good():
    return dict(q=z(B, T, HQ, D), k=z(B, T, HKV, D), v=z(B, T, HKV, D), o=z(B, T, HQ, D),
                dO=z(B, T, HQ, D), lse=z(B, HQ, T, dtype=torch.float32),
                delta=z(B, HQ, T, dtype=torch.float32))


BAD = [
    ("k_short_T", "k", z(B, T - 1, HKV, D)),
    ("k_other_D", "k", z(B, T, HKV, 128)),
    ("k_other_B", "k", z(B + 1, T, HKV, D)),
    ("v_short_T", "v", z(B, T - 1, HKV, D)),
    ("v_other_heads", "v", z(B, T, HKV + 1, D)),
    ("v_fp32", "v", z(B, T, HKV, D, dtype=torch.float32)),
    ("k_fp16", "k", z(B, T, HKV, D, dtype=torch.float16)),
    ("v_3d", "v", z(B, T, HKV * D)),
    ("v_not_tensor", "v", [0.0]),
]


def _call(fn, a):
    if fn == "fwd":
        return A.fwd(a["q"], a["k"], a["v"])
    if fn == "bwd":
        return A.bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"])
    if fn == "bwd_dkdv":
        return A.bwd_dkdv(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"])
    if fn == "bwd_dq":
        return A.bwd_dq(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"])
    if fn == "bwd_dkdv_dq":
        return A.bwd_dkdv_dq(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"])
    if fn == "fwd_rope":
        t = torch.zeros(T, D // 2)
        return A.fwd_rope(a["q"], a["k"], a["v"], t, t)
    if fn == "bwd_rope":
        t = torch.zeros(T, D // 2)
        return A.bwd_rope(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], t, t)
    raise AssertionError(fn)


FNS = ["fwd", "bwd", "bwd_dkdv", "bwd_dq", "bwd_dkdv_dq", "fwd_rope", "bwd_rope"]


@pytest.mark.parametrize("fn", FNS)
@pytest.mark.parametrize("name,key,bad", BAD, ids=[b[0] for b in BAD])
def test_kv_mismatch_is_refused(fn, name, key, bad):
    a = good()
    a[key] = bad
    with pytest.raises(ValueError):
        _call(fn, a)


BAD_BWD = [
    ("o_short_T", "o", z(B, T - 1, HQ, D)),
    ("o_fp32", "o", z(B, T, HQ, D, dtype=torch.float32)),
    ("dO_other_heads", "dO", z(B, T, HQ - 1, D)),
    ("dO_fp16", "dO", z(B, T, HQ, D, dtype=torch.float16)),
    ("lse_bf16", "lse", z(B, HQ, T)),
    ("lse_transposed", "lse", z(B, T, HQ, dtype=torch.float32)),
    ("lse_short", "lse", z(B, HQ, T - 1, dtype=torch.float32)),
    ("delta_fp64", "delta", z(B, HQ, T, dtype=torch.float64)),
    ("delta_short", "delta", z(B, HQ - 1, T, dtype=torch.float32)),
]


@pytest.mark.parametrize("fn", ["bwd", "bwd_dkdv", "bwd_dq", "bwd_dkdv_dq", "bwd_rope"])
@pytest.mark.parametrize("name,key,bad", BAD_BWD, ids=[b[0] for b in BAD_BWD])
def test_backward_operand_mismatch_is_refused(fn, name, key, bad):
    a = good()
    uses = {"bwd": ("o", "dO", "lse"), "bwd_rope": ("o", "dO", "lse"),
            "bwd_dkdv": ("dO", "lse", "delta"), "bwd_dq": ("dO", "lse", "delta"),
            "bwd_dkdv_dq": ("dO", "lse", "delta")}[fn]
    if key not in uses:
        pytest.skip(f"{fn} takes no {key}")
    a[key] = bad
    with pytest.raises(ValueError):
        _call(fn, a)


def test_preprocess_checks_dO_against_o():
    with pytest.raises(ValueError):
        A.bwd_preprocess(z(B, T, HQ, D), z(B, T - 1, HQ, D))
    with pytest.raises(ValueError):
        A.bwd_preprocess(z(B, T, HQ, D), z(B, T, HQ, D, dtype=torch.float16))
    with pytest.raises(ValueError):
        A.bwd_preprocess(z(B, T, HQ * D), z(B, T, HQ * D))


@pytest.mark.parametrize("fn", FNS)
def test_consistent_cpu_tensors_reach_the_device_check(fn):
    """Matching shapes pass the checks and are then refused as CPU tensors."""
    with pytest.raises(ValueError, match="on the GPU"):
        _call(fn, good())


def test_rope_tables_are_checked():
    a = good()
    t = torch.zeros(T, D // 2)
    with pytest.raises(ValueError, match="rotary tables"):
        A.fwd_rope(a["q"], a["k"], a["v"], torch.zeros(T - 1, D // 2), t)
    with pytest.raises(ValueError, match="rotary tables"):
        A.fwd_rope(a["q"], a["k"], a["v"], t, torch.zeros(T, D // 2, dtype=torch.float64))
