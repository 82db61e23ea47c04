"""The unfused-baseline library on the CPU: it loads, exports what
include/attn_unfused.h declares, and rejects bad arguments before it touches
the context or the GPU.  No call here passes validation."""
import os
import re

import pytest

from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import unfused as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_unfused.h")
BASE, MB = 1 << 40, 1 << 20
FAKE_CTX = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(attn_unfused_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(U.library_path()):
        pytest.fail("libattn_unfused.so is not built: run __graft_entry__.build()")
    return U.load_library()


def test_header_matches_binding():
    assert declared_functions() == sorted(U.EXPORTED)


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_workspace_bytes(lib):
    f = lib.attn_unfused_workspace_bytes
    n = 4 * 12 * 1024 * 1024
    m = 4 * 12 * 1024 * 64
    # S, P, dS; per-head dk, dv partials (float32); k, v repeated to 12 heads (16-bit)
    assert f(4, 1024, 12, 4, 64, A.ATTN_BF16) == 4 * n + 2 * n + 2 * n + 4 * m + 4 * m + 2 * m + 2 * m
    # S 392 -> 512, P and dS 196 -> 256 each, partials 3584 each, repeated k, v 1792 each
    assert f(1, 7, 2, 1, 64, A.ATTN_F16) == 512 + 256 + 256 + 3584 + 3584 + 1792 + 1792
    assert f(1, 7, 2, 1, 64, A.ATTN_F32) == 0   # 16-bit only
    assert f(1, 7, 3, 2, 64, A.ATTN_BF16) == 0  # Hq not a multiple of Hkv
    assert f(1, 7, 2, 1, 60, A.ATTN_BF16) == 0  # D not a multiple of 8
    assert f(1, 7, 2, 1, 128, A.ATTN_BF16) > 0  # D = 128 is fine here
    assert f(1, 1 << 17, 1, 1, 64, A.ATTN_BF16) == 0


def fwd_call(lib, **over):
    a = dict(ctx=FAKE_CTX, q=BASE, k=BASE + 16 * MB, v=BASE + 32 * MB, o=BASE + 48 * MB,
             lse=BASE + 64 * MB, B=1, T=128, Hq=4, Hkv=2, D=64, scale=0.125, causal=1,
             dtype=A.ATTN_BF16, ws=BASE + 80 * MB, ws_bytes=1 << 30, stream=None)
    a.update(over)
    return lib.attn_unfused_fwd(a["ctx"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"],
                                a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["dtype"],
                                a["ws"], a["ws_bytes"], a["stream"])


FWD_ERRORS = [
    ("null_ctx", dict(ctx=None), A.ATTN_ERR_INVALID_ARG),
    ("null_q", dict(q=None), A.ATTN_ERR_INVALID_ARG),
    ("misaligned_v", dict(v=BASE + 32 * MB + 2), A.ATTN_ERR_INVALID_ARG),
    ("f32", dict(dtype=A.ATTN_F32), A.ATTN_ERR_UNSUPPORTED),
    ("head_dim_60", dict(D=60), A.ATTN_ERR_UNSUPPORTED),
    ("head_dim_512", dict(D=512), A.ATTN_ERR_UNSUPPORTED),
    ("workspace_too_small", dict(ws_bytes=1000), A.ATTN_ERR_INVALID_ARG),
    ("o_overlaps_workspace", dict(o=BASE + 80 * MB + 4096), A.ATTN_ERR_INVALID_ARG),
    ("lse_overlaps_q", dict(lse=BASE + 16), A.ATTN_ERR_INVALID_ARG),
    ("causal_2", dict(causal=2), A.ATTN_ERR_INVALID_ARG),
    ("T_too_long", dict(T=(1 << 16) + 1), A.ATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,over,want", FWD_ERRORS, ids=[e[0] for e in FWD_ERRORS])
def test_fwd_validation(lib, name, over, want):
    assert fwd_call(lib, **over) == want


def bwd_call(lib, **over):
    a = dict(ctx=FAKE_CTX, q=BASE, k=BASE + 16 * MB, v=BASE + 32 * MB, lse=BASE + 64 * MB,
             dO=BASE + 48 * MB, dq=BASE + 96 * MB, dk=BASE + 112 * MB, dv=BASE + 128 * MB,
             B=1, T=128, Hq=4, Hkv=2, D=64, scale=0.125, causal=1, dtype=A.ATTN_BF16,
             ws=BASE + 144 * MB, ws_bytes=1 << 30, stream=None)
    a.update(over)
    return lib.attn_unfused_bwd(a["ctx"], a["q"], a["k"], a["v"], a["lse"], a["dO"], a["dq"],
                                a["dk"], a["dv"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                a["scale"], a["causal"], a["dtype"], a["ws"], a["ws_bytes"],
                                a["stream"])


BWD_ERRORS = [
    ("null_ctx", dict(ctx=None), A.ATTN_ERR_INVALID_ARG),
    ("null_dv", dict(dv=None), A.ATTN_ERR_INVALID_ARG),
    ("dq_overlaps_dk", dict(dq=BASE + 112 * MB + 64), A.ATTN_ERR_INVALID_ARG),
    ("dk_overlaps_lse", dict(dk=BASE + 64 * MB), A.ATTN_ERR_INVALID_ARG),
    ("workspace_too_small", dict(ws_bytes=4096), A.ATTN_ERR_INVALID_ARG),
    ("scale_nan", dict(scale=float("nan")), A.ATTN_ERR_INVALID_ARG),
    ("groups_do_not_divide", dict(Hq=5), A.ATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,over,want", BWD_ERRORS, ids=[e[0] for e in BWD_ERRORS])
def test_bwd_validation(lib, name, over, want):
    assert bwd_call(lib, **over) == want


def test_row_kernels_validate(lib):
    # rows not a multiple of T, p overlapping s, 32-bit type, null lse
    assert lib.attn_unfused_softmax_lse(BASE, BASE + 16 * MB, BASE + 32 * MB, 100, 64, 0.125, 1,
                                        A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    assert lib.attn_unfused_softmax_lse(BASE, BASE + 1024, BASE + 32 * MB, 128, 64, 0.125, 1,
                                        A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    assert lib.attn_unfused_softmax_lse(BASE, BASE + 16 * MB, BASE + 32 * MB, 128, 64, 0.125, 1,
                                        A.ATTN_F32, None) == A.ATTN_ERR_UNSUPPORTED
    assert lib.attn_unfused_probs_from_lse(BASE, None, BASE + 32 * MB, 128, 64, 0.125, 1,
                                           A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    assert lib.attn_unfused_softmax_bwd(BASE, BASE + 16 * MB, BASE + 16 * MB + 256, 128, 64, 1,
                                        A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    assert lib.attn_unfused_softmax_bwd(BASE, BASE + 16 * MB, BASE + 32 * MB, 128, 64, 3,
                                        A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no fallback"):
        U.load_library(str(tmp_path / "libattn_unfused.so"))
