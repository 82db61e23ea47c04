"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances (max |gpu - ref| / max |ref| per tensor; lse as an absolute error in
nats): float32 -- o and lse 1e-4, dq/dk/dv 1e-3; bfloat16 -- 2e-2 for every
tensor, against an oracle fed the bf16-rounded inputs widened exactly."""
import numpy as np
import pytest
import torch

from gpu_support import (as_numpy, check_against, check_every_unit, check_units, oracle_full,
                         run_gpu, sampled_units, say, to_device)
from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny-f32", "gqa-1x512", "gqa-4x1024", "gqa-1x512-f16",
                                  "gqa-4x1024-f16", "gqa-4x1024-noncausal"])
def test_workload_full_parity(name):
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    say("full parity", name, w.label())
    gpu = as_numpy(run_gpu(inp))
    errs = check_against(gpu, oracle_full(inp), w.dtype, name)
    print(name, errs)


@pytest.mark.parametrize("name", ["mha-32x1024", "gqa-8x4096-peaked"])
def test_workload_sampled_parity(name):
    """Full-size launch: three (batch, KV-group) units against the full oracle, and
    every unit against the row-wise oracle on fixed rows and the last keys, plus
    its exact column sums of dk and dv."""
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    say("sampled parity", name, w.label())
    gpu = as_numpy(run_gpu(inp))
    for n, a in gpu.items():
        assert np.all(np.isfinite(a)), (name, n)
    print(name, check_units(inp, gpu, sampled_units(w), name))
    say("every-unit parity", name, w.B * w.Hkv, "units")
    print(name, "every unit:", check_every_unit(inp, gpu, name))


EDGE_CASES = [
    # (B, T, Hq, Hkv, dtype, causal, q_std)
    (1, 1, 2, 1, "bf16", True, 1.0),      # a single token
    (2, 7, 6, 2, "bf16", True, 1.0),      # shorter than one tile
    (1, 129, 12, 4, "bf16", True, 1.0),   # one row past a tile boundary
    (2, 1000, 6, 3, "bf16", True, 1.0),   # ragged tail, several tiles
    (1, 333, 12, 1, "bf16", True, 2.0),   # all query heads on one KV head
    (3, 200, 1, 1, "bf16", True, 1.0),    # single head
    (1, 256, 4, 4, "bf16", False, 1.0),   # non-causal, tile multiple
    (2, 77, 6, 2, "bf16", False, 1.0),    # non-causal, ragged
    (1, 1, 2, 2, "f32", True, 1.0),
    (1, 100, 4, 2, "f32", True, 1.0),
    (2, 65, 3, 1, "f32", False, 1.0),
    (1, 300, 2, 2, "f32", True, 3.0),
    (1, 1, 2, 1, "f16", True, 1.0),
    (2, 1000, 6, 3, "f16", True, 1.0),
    (1, 333, 12, 1, "f16", True, 3.0),    # peaked softmax in fp16
    (2, 77, 6, 2, "f16", False, 1.0),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}/{c[3]}{c[4]}{'c' if c[5] else 'n'}" for c in EDGE_CASES])
def test_edge_case_parity(case):
    B, T, Hq, Hkv, dtype, causal, q_std = case
    w = W.custom(B, T, Hq, Hkv, 64, dtype, seed=1000 + T, q_std=q_std, causal=causal)
    inp = W.generate(w)
    say("edge parity", w.label())
    gpu = as_numpy(run_gpu(inp))
    check_against(gpu, oracle_full(inp), dtype, w.label())


@pytest.mark.parametrize("shape", [(1, 1408, 24, 8), (3, 1024, 12, 4)],
                         ids=["paired-order-264-workgroups", "group-count-12-fallback"])
def test_forward_unit_orders(shape):
    """Forward grids of 257..512 workgroups: 264 with 8 KV groups (the paired
    order, one shared CU per XCD) and 288 with 12 (not a multiple of 8: the
    plain heaviest-first order)."""
    B, T, Hq, Hkv = shape
    w = W.custom(B, T, Hq, Hkv, 64, "bf16", seed=61 + T)
    inp = W.generate(w)
    say("forward unit order", w.label())
    gpu = as_numpy(run_gpu(inp))
    check_against(gpu, oracle_full(inp), "bf16", w.label())


def test_scale_other_than_default():
    w = W.custom(1, 160, 4, 2, 64, "bf16", seed=7, scale=0.3)
    inp = W.generate(w)
    say("scale 0.3", w.label())
    gpu = as_numpy(run_gpu(inp))
    check_against(gpu, oracle_full(inp), "bf16", "scale=0.3")


def test_outputs_are_overwritten_not_accumulated():
    """The ABI overwrites o, lse, dq, dk, dv: NaN-filled output buffers give the same bits."""
    w = W.custom(1, 200, 6, 2, 64, "bf16", seed=11)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("overwrite", w.label())
    ref = run_gpu(inp, (q, k, v, dO))
    lib = A.load_library()
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 6, 200), float("nan"), device=q.device)
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    ws = torch.full((A.workspace_bytes(1, 200, 6, 2, 64, A.ATTN_BF16),), 255, dtype=torch.uint8, device=q.device)
    s = torch.cuda.current_stream().cuda_stream
    assert lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        1, 200, 6, 2, 64, w.scale, 1, A.ATTN_BF16, s) == 0
    assert lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        dO.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), 1, 200, 6, 2,
                        64, w.scale, 1, A.ATTN_BF16, ws.data_ptr(), ws.numel(), s) == 0
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(t, ref[name]), name


@pytest.mark.parametrize("name", ["gqa-4x1024", "mha-32x1024"])
def test_every_unit_writes_its_outputs(name):
    """Output buffers filled with NaN before the launches: every element of o,
    lse, dq, dk, dv comes out finite and equal to a run into fresh buffers, so
    every workgroup's unit (at these sizes the forward's paired order and the
    co-launched backward's per-workgroup unit lists are in play) wrote its part
    exactly once."""
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("every unit writes", w.label())
    ref = run_gpu(inp, (q, k, v, dO))
    lib = A.load_library()
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full((w.B, w.Hq, w.T), nan, device=q.device)
    dq, dk, dv = torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan)
    ws = torch.full((A.workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, A.ATTN_BF16),), 255,
                    dtype=torch.uint8, device=q.device)
    s = torch.cuda.current_stream().cuda_stream
    shp = (w.B, w.T, w.Hq, w.Hkv, w.D, w.scale, int(w.causal), A.ATTN_BF16)
    assert lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        *shp, s) == 0
    assert lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        dO.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *shp,
                        ws.data_ptr(), ws.numel(), s) == 0
    torch.cuda.synchronize()
    for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t.float()).all()), n
        assert torch.equal(t, ref[n]), n


def test_steps_compose_to_bwd():
    """attn_bwd == preprocess, then dkdv, then dq through the step entry points (bitwise)."""
    w = W.WORKLOADS["gqa-1x512"]
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("steps compose", w.label())
    o, lse = A.fwd(q, k, v, w.scale, True)
    dq, dk, dv = A.bwd(q, k, v, o, lse, dO, w.scale, True)
    delta = A.bwd_preprocess(o, dO)
    dk2, dv2 = A.bwd_dkdv(q, k, v, dO, lse, delta, w.scale, True)
    dq2 = A.bwd_dq(q, k, v, dO, lse, delta, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


@pytest.mark.parametrize("name", ["gqa-1x512", "tiny-f32", "gqa-4x1024"])
def test_colaunched_backward_equals_two_launches(name):
    """dK/dV and dQ in one grid give bitwise the results of the two launches."""
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("co-launched backward", w.label())
    o, lse = A.fwd(q, k, v, w.scale, True)
    delta = A.bwd_preprocess(o, dO)
    dq, dk, dv = A.bwd_dkdv_dq(q, k, v, dO, lse, delta, w.scale, True)
    dk2, dv2 = A.bwd_dkdv(q, k, v, dO, lse, delta, w.scale, True)
    dq2 = A.bwd_dq(q, k, v, dO, lse, delta, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


@pytest.mark.parametrize("shape", [(3, 333, 6, 2), (1, 65, 12, 4), (2, 200, 4, 4)])
def test_colaunched_backward_odd_grids(shape):
    """Odd unit counts: the dQ part not a multiple of 8 (XCD lists of different lengths), odd
    key-block counts (a middle block), non-causal."""
    B, T, Hq, Hkv = shape
    w = W.custom(B, T, Hq, Hkv, 64, "bf16", seed=41 + T)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    for causal in (True, False):
        say("co-launched backward", w.label(), "causal" if causal else "full")
        o, lse = A.fwd(q, k, v, w.scale, causal)
        delta = A.bwd_preprocess(o, dO)
        dq, dk, dv = A.bwd_dkdv_dq(q, k, v, dO, lse, delta, w.scale, causal)
        dk2, dv2 = A.bwd_dkdv(q, k, v, dO, lse, delta, w.scale, causal)
        dq2 = A.bwd_dq(q, k, v, dO, lse, delta, w.scale, causal)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
