"""GPU parity of the rotary-embedding variants (attn_fwd_rope, attn_bwd_rope)
against the fp64 oracle (oracle.ref_fwd_rope / ref_bwd_rope), plus properties
that need no oracle: identity tables reproduce the plain entry points bit for
bit, and repeated calls give the same bits.

The kernels round the rotated q', k' to the input type before the products (as
an unfused rotation that stores its result would); the oracle rotates the
rounded inputs exactly.  That extra rounding is half a unit in the last place of
each rotated element: inside the per-dtype tolerances of the plain path (used
unchanged) for unit-variance inputs.  Where the scores reach tens (the peaked
8 x 4096 workload) it moves lse by ~0.02 nats, so there the oracle is given
the same rounded q', k'."""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import TOL, as_numpy, check_against, cu_masked_stream, say, to_device
from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def tables(T, D=64, base=10000.0):
    c, s = W.rope_tables(T, D, base)
    dev = torch.device("cuda:0")
    return torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev), c, s


def run_rope(w, tensors, ct, st):
    q, k, v, dO = tensors
    o, lse = A.fwd_rope(q, k, v, ct, st, w.scale, w.causal)
    dq, dk, dv = A.bwd_rope(q, k, v, o, lse, dO, ct, st, w.scale, w.causal)
    delta = A.bwd_preprocess(o, dO)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv}


def oracle_rope(inp, c, s):
    w = inp.workload
    q, k, v, dO = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    o, lse = oracle.ref_fwd_rope(q, k, v, c, s, w.scale, w.causal)
    dq, dk, dv, delta = oracle.ref_bwd_rope(q, k, v, dO, c, s, w.scale, w.causal)
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("name", ["gqa-1x512", "gqa-1x512-f16", "gqa-4x1024"])
def test_rope_full_parity(name):
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    ct, st, c, s = tables(w.T)
    say("rope full parity", name, w.label())
    gpu = as_numpy(run_rope(w, to_device(inp), ct, st))
    print(name, check_against(gpu, oracle_rope(inp, c, s), w.dtype, "rope " + name))


ROPE_EDGES = [
    # (B, T, Hq, Hkv, dtype, causal, base)
    (1, 1, 2, 1, "bf16", True, 10000.0),     # one token: the rotation of position 0 is the identity
    (2, 7, 6, 2, "bf16", True, 10000.0),     # shorter than one tile
    (1, 129, 12, 4, "bf16", True, 10000.0),  # one row past a tile boundary
    (2, 1000, 6, 3, "bf16", True, 10000.0),  # ragged tail over several tiles
    (1, 333, 12, 1, "f16", True, 10000.0),   # all query heads on one KV head
    (2, 77, 6, 2, "bf16", False, 10000.0),   # non-causal, ragged
    (1, 300, 4, 2, "bf16", True, 100.0),     # fast-turning angles: every pair rotates far
]


@pytest.mark.parametrize("case", ROPE_EDGES,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}/{c[3]}{c[4]}{'c' if c[5] else 'n'}b{int(c[6])}"
                              for c in ROPE_EDGES])
def test_rope_edge_parity(case):
    B, T, Hq, Hkv, dtype, causal, base = case
    w = W.custom(B, T, Hq, Hkv, 64, dtype, seed=2000 + T, causal=causal)
    inp = W.generate(w)
    ct, st, c, s = tables(T, 64, base)
    say("rope edge parity", w.label(), "base", base)
    gpu = as_numpy(run_rope(w, to_device(inp), ct, st))
    check_against(gpu, oracle_rope(inp, c, s), dtype, "rope " + w.label())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_identity_tables_give_the_plain_path(dtype):
    """cos = 1, sin = 0 rotates nothing.  The backward of the rotary path (its
    preparation kernel and the shared dK/dV + dQ grid) then returns the values of
    attn_bwd exactly when both are given the same forward outputs.  The forwards
    are different kernels at head dim 64 (the plain one stages K/V by load-to-LDS
    and has no register pass in which to rotate K, the rotary one rotates K in its
    register-staged loads), each with its own fixed summation order, so they agree
    to the rounding of the dtype rather than bitwise: o within the dtype's
    tolerance relative to max |o|, lse within it in nats."""
    w = W.custom(2, 333, 12, 4, 64, dtype, seed=77)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    ones = torch.ones((w.T, 32), dtype=torch.float32, device=q.device)
    zeros = torch.zeros_like(ones)
    tol = TOL[dtype]["o"]
    say("rope identity tables", w.label())
    for causal in (True, False):
        o, lse = A.fwd(q, k, v, w.scale, causal)
        o2, lse2 = A.fwd_rope(q, k, v, ones, zeros, w.scale, causal)
        dq, dk, dv = A.bwd(q, k, v, o, lse, dO, w.scale, causal)
        dq2, dk2, dv2 = A.bwd_rope(q, k, v, o, lse, dO, ones, zeros, w.scale, causal)
        torch.cuda.synchronize()
        e_o = float((o.float() - o2.float()).abs().max() / o.float().abs().max())
        e_l = float((lse - lse2).abs().max())
        assert e_o <= tol and e_l <= tol, (causal, e_o, e_l)
        for n, a, b in (("dq", dq, dq2), ("dk", dk, dk2), ("dv", dv, dv2)):
            assert torch.equal(a, b), (n, causal)


def test_rope_is_bitwise_repeatable():
    w = W.WORKLOADS["gqa-4x1024"]
    inp = W.generate(w)
    ts = to_device(inp)
    ct, st, _, _ = tables(w.T)
    say("rope repeatability", w.label())
    first = run_rope(w, ts, ct, st)
    for _ in range(3):
        again = run_rope(w, ts, ct, st)
        for n in first:
            assert torch.equal(first[n], again[n]), n


def test_rope_same_bits_under_a_cu_mask():
    """The rotary path on 16 CUs gives the bits it gives on all of them: each
    workgroup of the co-launched backward then runs a long list of dQ units whose
    epilogues also read the rotation tables."""
    w = W.WORKLOADS["gqa-4x1024"]
    inp = W.generate(w)
    ts = to_device(inp)
    ct, st, _, _ = tables(w.T)
    say("rope CU-mask invariance", w.label())
    want = run_rope(w, ts, ct, st)
    with cu_masked_stream("first-16-cus"):
        got = run_rope(w, ts, ct, st)
    for n in want:
        assert torch.equal(want[n], got[n]), n


def round_to_dtype(x, dtype):
    """fp64 values rounded to the 16-bit input type (via float32, nearest-even)."""
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)


def test_rope_sampled_units_at_4096():
    """8 x 4096 with rotary positions up to 4095, checked on sampled (batch, KV
    group) units of the full launch.  This workload's softmax is peaked (scores
    of tens), where rounding q', k' to bf16 moves a score by a few hundredths --
    the kernel's documented semantics, not an error of the attention -- so the
    oracle is given the same rounded q', k' (rotated exactly, then rounded) and
    the plain path's tolerances apply unchanged."""
    w = W.WORKLOADS["gqa-8x4096-peaked"]
    inp = W.generate(w)
    ct, st, c, s = tables(w.T)
    say("rope sampled units", w.label())
    gpu = as_numpy(run_rope(w, to_device(inp), ct, st))
    q, k, v, dO = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    qr = round_to_dtype(oracle.apply_rope(q, c, s), w.dtype)
    kr = round_to_dtype(oracle.apply_rope(k, c, s), w.dtype)
    G = w.G
    for b, g in [(0, 0), (w.B - 1, w.Hkv - 1)]:
        o_r, lse_r = oracle.ref_fwd_group(qr, kr, v, w.scale, w.causal, b, g)
        dq_r, dk_r, dv_r, dl_r = oracle.ref_bwd_group(qr, kr, v, dO, w.scale, w.causal, b, g)
        # map the gradients of this unit back through the rotation transpose
        dq_r = oracle.apply_rope_transpose(dq_r[None], c, s)[0]
        dk_r = oracle.apply_rope_transpose(dk_r[None, :, None], c, s)[0, :, 0]
        hs = slice(g * G, (g + 1) * G)
        gpu_u = {"o": gpu["o"][b, :, hs], "lse": gpu["lse"][b, hs], "delta": gpu["delta"][b, hs],
                 "dq": gpu["dq"][b, :, hs], "dk": gpu["dk"][b, :, g], "dv": gpu["dv"][b, :, g]}
        ref_u = {"o": o_r, "lse": lse_r, "delta": dl_r, "dq": dq_r, "dk": dk_r, "dv": dv_r}
        print(check_against(gpu_u, ref_u, w.dtype, f"rope 8x4096 unit b={b} g={g}"))


def test_rope_at_4096_against_the_unrounded_oracle():
    """The rotary path at 8 x 4096 against the plain rotary oracle (q and k rotated
    exactly, never rounded), with the kernel's rounding of q', k' to bf16 bounded
    rather than handed to the oracle.

    The kernel rotates each pair in float32 (two fmas: absolute error below
    2^-22 times the pair's norm) and rounds to nearest bf16 (relative error at
    most u = 2^-8), so each rotated element is within u a_d of the exact one,
    a_d = |x'_d| + 2^-14 |pair|; that moves the score s_ij = scale <q'_i, k'_j>
    by at most
        E_ij = scale (2u + u^2) sum_d a(q'_i)_d a(k'_j)_d,
    and the log-sum-exp of a row moves by at most the largest move of its scores,
    so |lse_gpu - lse_exact| <= 2e-2 (the plain bf16 tolerance) + max_{j <= i} E_ij
    row by row.  o, dq, dk, dv change with P, by a factor exp(ds - dlse) per
    probability; the rounding errors are independent with standard deviation
    about u / sqrt(3) of each element, so a score moves by about
        sigma = scale (u / sqrt(3)) sqrt(2 max_ij sum_d (q'_id k'_jd)^2)
    and these are compared at 2e-2 + 6 sigma relative to max |ref|."""
    w = W.WORKLOADS["gqa-8x4096-peaked"]
    inp = W.generate(w)
    ct, st, c, s = tables(w.T)
    say("rope vs unrounded oracle", w.label())
    gpu = as_numpy(run_rope(w, to_device(inp), ct, st))
    q, k, v, dO = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    qr, kr = oracle.apply_rope(q, c, s), oracle.apply_rope(k, c, s)  # exact, not rounded
    u = 2.0 ** -8

    def mag(x):  # a_d: |x'_d| plus 2^-14 times the norm of its rotary pair
        pair = np.sqrt(x[..., 0::2] ** 2 + x[..., 1::2] ** 2)
        return np.abs(x) + 2.0 ** -14 * np.repeat(pair, 2, axis=-1)

    G, T = w.G, w.T
    causal_mask = np.tril(np.ones((T, T), dtype=bool))
    for b, g in [(0, 0), (w.B - 1, w.Hkv - 1)]:
        o_r, lse_r = oracle.ref_fwd_group(qr, kr, v, w.scale, w.causal, b, g)
        dq_r, dk_r, dv_r, _ = oracle.ref_bwd_group(qr, kr, v, dO, w.scale, w.causal, b, g)
        dq_r = oracle.apply_rope_transpose(dq_r[None], c, s)[0]
        dk_r = oracle.apply_rope_transpose(dk_r[None, :, None], c, s)[0, :, 0]
        ka = mag(kr[b, :, g])
        sigma = 0.0
        for hh in range(G):
            h = g * G + hh
            qa = mag(qr[b, :, h])
            E = w.scale * (2 * u + u * u) * np.where(causal_mask, qa @ ka.T, 0.0).max(axis=1)
            err = np.abs(gpu["lse"][b, h] - lse_r[hh])
            assert np.all(err <= 2e-2 + E), (b, h, float(err.max()), float(E.max()))
            sq = np.where(causal_mask, (qa * qa) @ (ka * ka).T, 0.0).max()
            sigma = max(sigma, w.scale * (u / np.sqrt(3.0)) * np.sqrt(2.0 * sq))
        tol = 2e-2 + 6.0 * sigma
        hs = slice(g * G, (g + 1) * G)
        for name, a, r in (("o", gpu["o"][b, :, hs], o_r), ("dq", gpu["dq"][b, :, hs], dq_r),
                           ("dk", gpu["dk"][b, :, g], dk_r), ("dv", gpu["dv"][b, :, g], dv_r)):
            e = float(np.max(np.abs(a - r)) / np.max(np.abs(r)))
            print(f"rope unrounded b={b} g={g} {name}: {e:.4g} (tolerance {tol:.4g})")
            assert e <= tol, (b, g, name, e, tol)
