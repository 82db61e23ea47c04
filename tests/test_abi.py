"""The C-ABI library on the CPU: it loads, exports every function include/attn.h
declares, and its host-side validator rejects bad arguments before touching the
GPU.  No call here passes validation, so nothing is ever launched."""
import ctypes
import os
import re

import pytest

from reproducible_causal_attention_amd import attn as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.library_path()):
        pytest.fail("libattn.so is not built: run __graft_entry__.build()")
    return A.load_library()


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(A.EXPORTED)


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_build_info_names_arch_and_tiles(lib):
    info = A.build_info()
    assert "arch=gfx950" in info and "revision=" in info and "fwd_bf16{" in info


def test_status_strings(lib):
    for code in range(4):
        assert lib.attn_status_string(code).decode().startswith(
            ("ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_HIP")[code])
    assert b"unknown" in lib.attn_status_string(99)


def test_workspace_bytes(lib):
    f = lib.attn_bwd_workspace_bytes
    assert f(4, 1024, 12, 4, 64, A.ATTN_BF16) == 4 * 12 * 1024 * 4
    assert f(1, 7, 3, 1, 64, A.ATTN_F32) == 256  # 84 bytes rounded up to 256
    assert f(1, 7, 3, 2, 64, A.ATTN_F32) == 0    # Hq not a multiple of Hkv
    assert f(1, 7, 3, 1, 32, A.ATTN_F32) == 0    # unsupported head dim
    assert f(0, 7, 3, 1, 64, A.ATTN_F32) == 0


# Fake device addresses: the validator only does arithmetic on them.
BASE = 1 << 40
MB = 1 << 20


def fwd_args(**over):
    a = dict(q=BASE, k=BASE + 16 * MB, v=BASE + 32 * MB, o=BASE + 48 * MB, lse=BASE + 64 * MB,
             B=1, T=128, Hq=4, Hkv=2, D=64, scale=0.125, causal=1, dtype=A.ATTN_BF16, stream=None)
    a.update(over)
    return a


def call_fwd(lib, a):
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"], a["Hq"],
                        a["Hkv"], a["D"], a["scale"], a["causal"], a["dtype"], a["stream"])


FWD_ERRORS = [
    ("null_q", dict(q=None), A.ATTN_ERR_INVALID_ARG),
    ("null_lse", dict(lse=None), A.ATTN_ERR_INVALID_ARG),
    ("misaligned_k", dict(k=BASE + 16 * MB + 8), A.ATTN_ERR_INVALID_ARG),
    ("zero_batch", dict(B=0), A.ATTN_ERR_INVALID_ARG),
    ("negative_T", dict(T=-3), A.ATTN_ERR_INVALID_ARG),
    ("zero_heads", dict(Hkv=0), A.ATTN_ERR_INVALID_ARG),
    ("groups_do_not_divide", dict(Hq=5, Hkv=2), A.ATTN_ERR_INVALID_ARG),
    ("causal_not_boolean", dict(causal=2), A.ATTN_ERR_INVALID_ARG),
    ("scale_nan", dict(scale=float("nan")), A.ATTN_ERR_INVALID_ARG),
    ("scale_inf", dict(scale=float("inf")), A.ATTN_ERR_INVALID_ARG),
    ("T_too_long", dict(T=(1 << 24) + 1), A.ATTN_ERR_INVALID_ARG),
    ("too_many_tiles", dict(B=1 << 14, T=1 << 16, Hq=8, Hkv=8), A.ATTN_ERR_INVALID_ARG),
    ("batch_element_too_large", dict(B=1, T=1 << 20, Hq=128, Hkv=128), A.ATTN_ERR_INVALID_ARG),
    ("head_dim_96", dict(D=96), A.ATTN_ERR_UNSUPPORTED),
    ("f32_head_dim_128", dict(D=128, dtype=A.ATTN_F32), A.ATTN_ERR_UNSUPPORTED),
    ("unknown_dtype", dict(dtype=7), A.ATTN_ERR_UNSUPPORTED),
    ("unknown_dtype_but_overlap", dict(dtype=7, o=BASE + 64), A.ATTN_ERR_INVALID_ARG),
    ("o_overlaps_q", dict(o=BASE + 64), A.ATTN_ERR_INVALID_ARG),
    ("lse_overlaps_o", dict(lse=BASE + 48 * MB + 16), A.ATTN_ERR_INVALID_ARG),
    ("o_overlaps_v_tail", dict(o=BASE + 32 * MB + 128 * 2 * 64 * 2 - 16), A.ATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,over,want", FWD_ERRORS, ids=[e[0] for e in FWD_ERRORS])
def test_fwd_validation(lib, name, over, want):
    assert call_fwd(lib, fwd_args(**over)) == want


def test_adjacent_buffers_are_not_overlap(lib):
    """o starting exactly where v ends is legal, one element earlier is not.  An
    unknown dtype (checked after the overlap rule, 2-byte elements for the
    sizes) keeps every call from launching."""
    v_end = BASE + 32 * MB + 1 * 128 * 2 * 64 * 2
    assert call_fwd(lib, fwd_args(o=v_end, dtype=7)) == A.ATTN_ERR_UNSUPPORTED
    assert call_fwd(lib, fwd_args(o=v_end - 16, dtype=7)) == A.ATTN_ERR_INVALID_ARG


def bwd_call(lib, **over):
    a = dict(q=BASE, k=BASE + 16 * MB, v=BASE + 32 * MB, o=BASE + 48 * MB, lse=BASE + 64 * MB,
             dO=BASE + 80 * MB, dq=BASE + 96 * MB, dk=BASE + 112 * MB, dv=BASE + 128 * MB,
             B=1, T=128, Hq=4, Hkv=2, D=64, scale=0.125, causal=1, dtype=A.ATTN_BF16,
             ws=BASE + 144 * MB, ws_bytes=4 * 128 * 4, stream=None)
    a.update(over)
    return lib.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"], a["dk"],
                        a["dv"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                        a["causal"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


BWD_ERRORS = [
    ("null_workspace", dict(ws=None), A.ATTN_ERR_INVALID_ARG),
    ("workspace_too_small", dict(ws_bytes=4 * 128 * 4 - 1), A.ATTN_ERR_INVALID_ARG),
    ("null_dO", dict(dO=None), A.ATTN_ERR_INVALID_ARG),
    ("dq_overlaps_dk", dict(dq=BASE + 112 * MB + 32), A.ATTN_ERR_INVALID_ARG),
    ("dv_overlaps_o", dict(dv=BASE + 48 * MB), A.ATTN_ERR_INVALID_ARG),
    ("workspace_overlaps_lse", dict(ws=BASE + 64 * MB + 256), A.ATTN_ERR_INVALID_ARG),
    ("dk_overlaps_workspace", dict(dk=BASE + 144 * MB + 16), A.ATTN_ERR_INVALID_ARG),
    ("misaligned_dq", dict(dq=BASE + 96 * MB + 2), A.ATTN_ERR_INVALID_ARG),
    ("groups_do_not_divide", dict(Hq=3, Hkv=2), A.ATTN_ERR_INVALID_ARG),
    ("head_dim_32", dict(D=32), A.ATTN_ERR_UNSUPPORTED),
    ("scale_nan", dict(scale=float("nan")), A.ATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,over,want", BWD_ERRORS, ids=[e[0] for e in BWD_ERRORS])
def test_bwd_validation(lib, name, over, want):
    assert bwd_call(lib, **over) == want


def noalloc_call(lib, **over):
    a = dict(q=BASE, k=BASE + 16 * MB, v=BASE + 32 * MB, o=BASE + 48 * MB, lse=BASE + 64 * MB,
             dO=BASE + 80 * MB, dq=BASE + 96 * MB, dk=BASE + 112 * MB, dv=BASE + 128 * MB,
             B=1, T=128, Hq=4, Hkv=2, D=64, scale=0.125, causal=1, dtype=A.ATTN_BF16, stream=None)
    a.update(over)
    return lib.attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"],
                                a["dk"], a["dv"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                a["scale"], a["causal"], a["dtype"], a["stream"])


# Buffers 4 GiB apart, so that large shapes do not overlap.
GB4 = 1 << 32
BIG = dict(q=BASE, k=BASE + GB4, v=BASE + 2 * GB4, o=BASE + 3 * GB4, lse=BASE + 4 * GB4,
           dO=BASE + 5 * GB4, dq=BASE + 6 * GB4, dk=BASE + 7 * GB4, dv=BASE + 8 * GB4)

NOALLOC_ERRORS = [
    ("null_dq", dict(dq=None), A.ATTN_ERR_INVALID_ARG),
    ("dv_overlaps_o", dict(dv=BASE + 48 * MB), A.ATTN_ERR_INVALID_ARG),
    ("groups_do_not_divide", dict(Hq=3, Hkv=2), A.ATTN_ERR_INVALID_ARG),
    ("head_dim_32", dict(D=32), A.ATTN_ERR_UNSUPPORTED),
    ("causal_2", dict(causal=2), A.ATTN_ERR_INVALID_ARG),
    # delta of 2 x 4 x 2^20 rows = 32 MiB, beyond the 16 MiB scratch array
    ("beyond_scratch", dict(BIG, B=2, T=1 << 20, Hq=4, Hkv=4), A.ATTN_ERR_INVALID_ARG),
    ("beyond_scratch_f32", dict(BIG, B=1, T=1 << 20, Hq=5, Hkv=5, dtype=A.ATTN_F32),
     A.ATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,over,want", NOALLOC_ERRORS, ids=[e[0] for e in NOALLOC_ERRORS])
def test_bwd_noalloc_validation(lib, name, over, want):
    """attn_bwd_noalloc applies attn_bwd's checks and the scratch size limit, all on
    the host before any HIP call."""
    assert noalloc_call(lib, **over) == want


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", text)
    assert m, "ATTN_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == A.NOALLOC_SCRATCH_BYTES


def test_step_entry_points_validate(lib):
    # preprocess: delta overlapping dO
    assert lib.attn_bwd_preprocess(BASE, BASE + 16 * MB, BASE + 16 * MB + 64, 1, 128, 4, 64,
                                   A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    assert lib.attn_bwd_preprocess(BASE, BASE + 16 * MB, BASE + 32 * MB, 1, 128, 4, 48,
                                   A.ATTN_BF16, None) == A.ATTN_ERR_UNSUPPORTED
    # dkdv: dk == dv
    assert lib.attn_bwd_dkdv(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB, BASE + 64 * MB,
                             BASE + 80 * MB, BASE + 96 * MB, BASE + 96 * MB, 1, 128, 4, 2, 64,
                             0.125, 1, A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    # dkdv: null delta
    assert lib.attn_bwd_dkdv(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB, BASE + 64 * MB,
                             None, BASE + 96 * MB, BASE + 112 * MB, 1, 128, 4, 2, 64,
                             0.125, 1, A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    # dq: dq overlapping delta
    assert lib.attn_bwd_dq(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB, BASE + 64 * MB,
                           BASE + 80 * MB, BASE + 80 * MB + 16, 1, 128, 4, 2, 64, 0.125, 1,
                           A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    # dq: causal out of range
    assert lib.attn_bwd_dq(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB, BASE + 64 * MB,
                           BASE + 80 * MB, BASE + 96 * MB, 1, 128, 4, 2, 64, 0.125, -1,
                           A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    # dkdv_dq: dq overlapping dk
    assert lib.attn_bwd_dkdv_dq(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB,
                                BASE + 64 * MB, BASE + 80 * MB, BASE + 96 * MB,
                                BASE + 96 * MB + 64, BASE + 112 * MB, 1, 128, 4, 2, 64, 0.125, 1,
                                A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    # dkdv_dq: dv overlapping an input (delta)
    assert lib.attn_bwd_dkdv_dq(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB,
                                BASE + 64 * MB, BASE + 80 * MB, BASE + 96 * MB, BASE + 112 * MB,
                                BASE + 80 * MB, 1, 128, 4, 2, 64, 0.125, 1,
                                A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    # dkdv_dq: null dv, Hq not a multiple of Hkv
    assert lib.attn_bwd_dkdv_dq(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB,
                                BASE + 64 * MB, BASE + 80 * MB, BASE + 96 * MB, BASE + 112 * MB,
                                None, 1, 128, 4, 2, 64, 0.125, 1,
                                A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG
    assert lib.attn_bwd_dkdv_dq(BASE, BASE + 16 * MB, BASE + 32 * MB, BASE + 48 * MB,
                                BASE + 64 * MB, BASE + 80 * MB, BASE + 96 * MB, BASE + 112 * MB,
                                BASE + 128 * MB, 1, 128, 4, 3, 64, 0.125, 1,
                                A.ATTN_BF16, None) == A.ATTN_ERR_INVALID_ARG


def test_rope_workspace_bytes(lib):
    f = lib.attn_bwd_rope_workspace_bytes
    # delta (4*12*1024 float32) + q' (4*1024*12*64 bf16) + k' (4*1024*4*64 bf16)
    assert f(4, 1024, 12, 4, 64, A.ATTN_BF16) == 4 * 12 * 1024 * 4 + 4 * 1024 * 12 * 128 + 4 * 1024 * 4 * 128
    # 84 + 2688 + 896 bytes, each rounded up to 256
    assert f(1, 7, 3, 1, 64, A.ATTN_F16) == 256 + 2816 + 1024
    assert f(1, 7, 3, 1, 64, A.ATTN_F32) == 0    # rotary variants are 16-bit only
    assert f(1, 7, 3, 2, 64, A.ATTN_BF16) == 0


def fwd_rope_call(lib, **over):
    a = dict(q=BASE, k=BASE + 16 * MB, v=BASE + 32 * MB, cos=BASE + 160 * MB, sin=BASE + 176 * MB,
             o=BASE + 48 * MB, lse=BASE + 64 * MB, B=1, T=128, Hq=4, Hkv=2, D=64, scale=0.125,
             causal=1, dtype=A.ATTN_BF16, stream=None)
    a.update(over)
    return lib.attn_fwd_rope(a["q"], a["k"], a["v"], a["cos"], a["sin"], a["o"], a["lse"], a["B"],
                             a["T"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["dtype"],
                             a["stream"])


FWD_ROPE_ERRORS = [
    ("f32", dict(dtype=A.ATTN_F32), A.ATTN_ERR_UNSUPPORTED),
    ("null_cos", dict(cos=None), A.ATTN_ERR_INVALID_ARG),
    ("misaligned_sin", dict(sin=BASE + 176 * MB + 4), A.ATTN_ERR_INVALID_ARG),
    ("o_overlaps_cos", dict(o=BASE + 160 * MB + 128 * 32 * 4 - 16), A.ATTN_ERR_INVALID_ARG),
    ("lse_overlaps_sin", dict(lse=BASE + 176 * MB), A.ATTN_ERR_INVALID_ARG),
    ("head_dim_96", dict(D=96), A.ATTN_ERR_UNSUPPORTED),
    ("groups_do_not_divide", dict(Hq=3), A.ATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,over,want", FWD_ROPE_ERRORS, ids=[e[0] for e in FWD_ROPE_ERRORS])
def test_fwd_rope_validation(lib, name, over, want):
    assert fwd_rope_call(lib, **over) == want


def test_rope_tables_end_where_they_should(lib):
    """o starting right after the cos table ([T, 32] float32) is not overlap, one
    float earlier it is; float32 (unsupported by the rotary entry points, and
    checked after the overlap rule) keeps the calls from launching."""
    end = BASE + 160 * MB + 128 * 32 * 4
    assert fwd_rope_call(lib, o=end, dtype=A.ATTN_F32) == A.ATTN_ERR_UNSUPPORTED
    assert fwd_rope_call(lib, o=end - 16, dtype=A.ATTN_F32) == A.ATTN_ERR_INVALID_ARG


def bwd_rope_call(lib, **over):
    a = dict(q=BASE, k=BASE + 16 * MB, v=BASE + 32 * MB, o=BASE + 48 * MB, lse=BASE + 64 * MB,
             dO=BASE + 80 * MB, cos=BASE + 160 * MB, sin=BASE + 176 * MB, dq=BASE + 96 * MB,
             dk=BASE + 112 * MB, dv=BASE + 128 * MB, B=1, T=128, Hq=4, Hkv=2, D=64, scale=0.125,
             causal=1, dtype=A.ATTN_BF16, ws=BASE + 144 * MB, ws_bytes=None, stream=None)
    a.update(over)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.attn_bwd_rope_workspace_bytes(1, 128, 4, 2, 64, A.ATTN_BF16)
    return lib.attn_bwd_rope(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["cos"], a["sin"],
                             a["dq"], a["dk"], a["dv"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"],
                             a["scale"], a["causal"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


BWD_ROPE_ERRORS = [
    ("f32", dict(dtype=A.ATTN_F32), A.ATTN_ERR_UNSUPPORTED),
    ("workspace_too_small", dict(ws_bytes=512 + 65536 + 32768 - 1), A.ATTN_ERR_INVALID_ARG),
    ("plain_bwd_workspace_is_too_small", dict(ws_bytes=4 * 128 * 4), A.ATTN_ERR_INVALID_ARG),
    ("null_sin", dict(sin=None), A.ATTN_ERR_INVALID_ARG),
    ("workspace_overlaps_cos", dict(ws=BASE + 160 * MB - 65536), A.ATTN_ERR_INVALID_ARG),
    ("dk_overlaps_sin", dict(dk=BASE + 176 * MB + 256), A.ATTN_ERR_INVALID_ARG),
    ("scale_inf", dict(scale=float("inf")), A.ATTN_ERR_INVALID_ARG),
    ("head_dim_32", dict(D=32), A.ATTN_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,over,want", BWD_ROPE_ERRORS, ids=[e[0] for e in BWD_ROPE_ERRORS])
def test_bwd_rope_validation(lib, name, over, want):
    assert bwd_rope_call(lib, **over) == want


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.fwd(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous())


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no fallback"):
        A.load_library(str(tmp_path / "libattn.so"))
