"""GPU tests of the unfused baseline (libattn_unfused.so): parity with the fp64
oracle (the same tolerances as the fused path), bitwise repeatability, and
each row kernel against a plain float32 torch reference of the same step on
the same input."""
import numpy as np
import pytest
import torch

from gpu_support import as_numpy, check_against, oracle_full, say, to_device
from reproducible_causal_attention_amd import unfused as U
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = U.Context()
    yield c
    c.close()


def run_unfused(ctx, w, tensors):
    q, k, v, dO = tensors
    o, lse = U.fwd(ctx, q, k, v, w.scale, w.causal)
    dq, dk, dv = U.bwd(ctx, q, k, v, lse, dO, w.scale, w.causal)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def oracle_no_delta(inp):
    ref = oracle_full(inp)
    ref.pop("delta")
    return ref


@pytest.mark.parametrize("name", ["gqa-1x512", "gqa-1x512-f16", "gqa-4x1024", "gqa-4x1024-noncausal"])
def test_unfused_parity(ctx, name):
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    say("unfused parity", name, w.label())
    gpu = as_numpy(run_unfused(ctx, w, to_device(inp)))
    print(name, check_against(gpu, oracle_no_delta(inp), w.dtype, "unfused " + name))


UNFUSED_EDGES = [
    # (B, T, Hq, Hkv, dtype, causal)
    (1, 1, 2, 1, "bf16", True),      # a single token
    (2, 7, 6, 2, "bf16", True),      # T not a multiple of 4: scalar row path
    (1, 130, 12, 4, "bf16", True),   # ragged, scalar row path
    (2, 77, 6, 2, "f16", False),     # non-causal, ragged
    (1, 333, 12, 1, "f16", True),    # one KV head for all query heads
    (3, 200, 4, 4, "bf16", True),    # MHA
]


@pytest.mark.parametrize("case", UNFUSED_EDGES,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}/{c[3]}{c[4]}{'c' if c[5] else 'n'}" for c in UNFUSED_EDGES])
def test_unfused_edge_parity(ctx, case):
    B, T, Hq, Hkv, dtype, causal = case
    w = W.custom(B, T, Hq, Hkv, 64, dtype, seed=3000 + T, causal=causal)
    inp = W.generate(w)
    say("unfused edge parity", w.label())
    gpu = as_numpy(run_unfused(ctx, w, to_device(inp)))
    check_against(gpu, oracle_no_delta(inp), dtype, "unfused " + w.label())


def test_unfused_head_dim_128(ctx):
    """The unfused path is not tied to D = 64 (rocBLAS GEMMs, row kernels over T)."""
    w = W.custom(1, 256, 8, 2, 128, "bf16", seed=31, scale=128 ** -0.5)
    inp = W.generate(w)
    say("unfused D=128", w.label())
    gpu = as_numpy(run_unfused(ctx, w, to_device(inp)))
    check_against(gpu, oracle_no_delta(inp), "bf16", "unfused D=128")


def test_unfused_is_bitwise_repeatable(ctx):
    w = W.WORKLOADS["gqa-4x1024"]
    inp = W.generate(w)
    ts = to_device(inp)
    say("unfused repeatability", w.label())
    first = run_unfused(ctx, w, ts)
    for _ in range(2):
        again = run_unfused(ctx, w, ts)
        for n in first:
            assert torch.equal(first[n], again[n]), n


def _rand_scores(shape, seed, std=3.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).cuda()


def _mask(T, causal, device):
    if not causal:
        return torch.ones((T, T), dtype=torch.bool, device=device)
    return torch.tril(torch.ones((T, T), dtype=torch.bool, device=device))


# T = 64, 256: one register chunk per lane; 600: three, the last partly past T;
# 2048: eight; 130 and 1: the looped kernels (T not a multiple of 4); 2100 and
# 4096: the looped kernels with 16-byte accesses (T beyond the register rows).
@pytest.mark.parametrize("T,causal,dtype", [(64, True, torch.bfloat16), (130, True, torch.float16),
                                            (256, False, torch.bfloat16), (1, True, torch.bfloat16),
                                            (600, True, torch.float16), (2048, True, torch.bfloat16),
                                            (2100, False, torch.bfloat16), (4096, True, torch.float16)])
def test_row_kernels_against_torch(T, causal, dtype):
    """softmax_lse, probs_from_lse and softmax_bwd against float32 torch on the
    same scores: lse within 1e-5 nats, probabilities within a half-unit of the
    16-bit type (plus the exp rounding), dS within a unit of the 16-bit type."""
    say("unfused row kernels", T, causal, dtype)
    scale = 0.3
    shape = (2, 3, T, T) if T <= 1024 else (1, 1, T, T)
    s = _rand_scores(shape, 100 + T)
    mask = _mask(T, causal, s.device)
    x = torch.where(mask, s * scale, torch.tensor(float("-inf"), device=s.device))
    lse_ref = torch.logsumexp(x, dim=-1)
    p_ref = torch.exp(x - lse_ref[..., None])
    p, lse = U.softmax_lse(s, scale, causal, dtype)
    p2 = U.probs_from_lse(s, lse, scale, causal, dtype)
    torch.cuda.synchronize()
    assert float((lse - lse_ref).abs().max()) < 1e-5
    ulp = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    floor = 2.0 ** -24  # fp16 subnormal spacing: tiny probabilities lose relative precision
    for name, got in (("softmax_lse", p), ("probs_from_lse", p2)):
        excess = (got.float() - p_ref).abs() - (ulp * p_ref + floor)
        assert float(excess[mask.expand_as(excess)].max()) <= 0, name
        assert torch.all(got.float()[~mask.expand_as(got)] == 0), name
    dp = _rand_scores(shape, 200 + T, std=1.0)
    ds = U.softmax_bwd(p, dp, causal)
    torch.cuda.synchronize()
    pf = p.float()
    delta = (pf * torch.where(mask, dp, torch.zeros_like(dp))).sum(-1, keepdim=True)
    ds_ref = torch.where(mask, pf * (dp - delta), torch.zeros_like(dp))
    tol = ulp * float(ds_ref.abs().max()) + 1e-6
    assert float((ds.float() - ds_ref).abs().max()) < tol
    assert torch.all(ds.float()[~mask.expand_as(ds)] == 0)


def test_unfused_close_to_fused(ctx):
    """Both paths approximate the same attention: their outputs agree to the
    bf16 tolerance (they are not bitwise equal: the arithmetic differs)."""
    from reproducible_causal_attention_amd import attn as A
    w = W.WORKLOADS["gqa-1x512"]
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("unfused vs fused", w.label())
    o, lse = A.fwd(q, k, v, w.scale, True)
    dq, dk, dv = A.bwd(q, k, v, o, lse, dO, w.scale, True)
    u = run_unfused(ctx, w, (q, k, v, dO))
    torch.cuda.synchronize()
    for n, a in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        b = u[n]
        rel = float((a.float() - b.float()).abs().max() / a.float().abs().max())
        assert rel < 2e-2, (n, rel)
    assert float((lse - u["lse"]).abs().max()) < 1e-2
