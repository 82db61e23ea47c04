"""Head dimension 128 (16-bit types): the same kernels instantiated for 128-wide
rows, checked against the fp64 oracle with the tolerances of the 64-wide path;
the co-launched backward against its two separate launches (bitwise); the
rotary variants; repeatability."""
import pytest
import torch

import oracle
from gpu_support import as_numpy, check_against, oracle_full, run_gpu, say, to_device
from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5

D128_CASES = [
    # (B, T, Hq, Hkv, dtype, causal)
    (1, 512, 8, 2, "bf16", True),
    (4, 1024, 12, 4, "bf16", True),    # the headline shape at D = 128
    (2, 333, 4, 4, "f16", True),       # ragged, MHA
    (1, 200, 6, 2, "bf16", False),     # non-causal
    (1, 1, 2, 1, "bf16", True),        # a single token
    (2, 77, 12, 1, "f16", True),       # one KV head for all query heads, shorter than a tile
    (1, 1000, 4, 2, "bf16", True),     # ragged tail over many tiles
]


@pytest.mark.parametrize("case", D128_CASES,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}/{c[3]}{c[4]}{'c' if c[5] else 'n'}" for c in D128_CASES])
def test_d128_parity(case):
    B, T, Hq, Hkv, dtype, causal = case
    w = W.custom(B, T, Hq, Hkv, 128, dtype, seed=4000 + T, scale=SCALE, causal=causal)
    inp = W.generate(w)
    say("D=128 parity", w.label())
    gpu = as_numpy(run_gpu(inp))
    print(w.label(), check_against(gpu, oracle_full(inp), dtype, "D=128 " + w.label()))


@pytest.mark.parametrize("shape", [(4, 1024, 12, 4), (3, 333, 6, 2)])
def test_d128_colaunch_equals_two_launches(shape):
    B, T, Hq, Hkv = shape
    w = W.custom(B, T, Hq, Hkv, 128, "bf16", seed=51 + T, scale=SCALE)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    for causal in (True, False):
        say("D=128 co-launch", w.label(), causal)
        o, lse = A.fwd(q, k, v, w.scale, causal)
        delta = A.bwd_preprocess(o, dO)
        dq, dk, dv = A.bwd_dkdv_dq(q, k, v, dO, lse, delta, w.scale, causal)
        dk2, dv2 = A.bwd_dkdv(q, k, v, dO, lse, delta, w.scale, causal)
        dq2 = A.bwd_dq(q, k, v, dO, lse, delta, w.scale, causal)
        dq3, dk3, dv3 = A.bwd(q, k, v, o, lse, dO, w.scale, causal)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
        assert torch.equal(dq, dq3) and torch.equal(dk, dk3) and torch.equal(dv, dv3)


def test_d128_repeatable():
    w = W.custom(4, 1024, 12, 4, 128, "bf16", seed=77, scale=SCALE)
    inp = W.generate(w)
    ts = to_device(inp)
    say("D=128 repeatability", w.label())
    first = run_gpu(inp, ts)
    for _ in range(3):
        again = run_gpu(inp, ts)
        for n in first:
            assert torch.equal(first[n], again[n]), n


@pytest.mark.parametrize("case", [(1, 512, 8, 2, "bf16"), (2, 130, 4, 4, "f16")])
def test_d128_rope_parity(case):
    B, T, Hq, Hkv, dtype = case
    w = W.custom(B, T, Hq, Hkv, 128, dtype, seed=5000 + T, scale=SCALE)
    inp = W.generate(w)
    c, s = W.rope_tables(T, 128)
    q, k, v, dO = to_device(inp)
    ct, st = torch.from_numpy(c).to(q.device), torch.from_numpy(s).to(q.device)
    say("D=128 rope parity", w.label())
    o, lse = A.fwd_rope(q, k, v, ct, st, w.scale, True)
    dq, dk, dv = A.bwd_rope(q, k, v, o, lse, dO, ct, st, w.scale, True)
    torch.cuda.synchronize()
    gpu = as_numpy({"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv})
    qd, kd, vd, dOd = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    o_r, lse_r = oracle.ref_fwd_rope(qd, kd, vd, c, s, w.scale, True)
    dq_r, dk_r, dv_r, _ = oracle.ref_bwd_rope(qd, kd, vd, dOd, c, s, w.scale, True)
    ref = {"o": o_r, "lse": lse_r, "dq": dq_r, "dk": dk_r, "dv": dv_r}
    print(check_against(gpu, ref, dtype, "D=128 rope " + w.label()))
