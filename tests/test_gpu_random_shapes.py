"""GPU parity over a fixed, seeded sample of shapes, dtypes, masks and scales.

Each case draws batch size, sequence length (ragged, from a single token up to
several tiles), KV heads, group size, head dim (128 only for the 16-bit types),
dtype, causal flag, the spread of q and the softmax scale, and compares every
output with the fp64 oracle at the tolerances of the other parity tests.  The
scale cases include the degenerate ones the interface accepts: 0 (every visible
key weighted equally), negative (the ordering of the scores reversed, which the
forward handles with the minimum of the raw scores), and large positive (a
nearly one-hot softmax)."""
import numpy as np
import pytest

from gpu_support import as_numpy, check_against, oracle_full, run_gpu, say
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _draw_cases(n, seed=20261202):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        dtype = ["bf16", "f16", "f32"][int(rng.integers(3))]
        D = 128 if dtype != "f32" and rng.random() < 0.3 else 64
        Hkv = int(rng.integers(1, 5))
        G = int(rng.integers(1, 7))
        T = int(rng.choice([1, 2, 31, 33, 64, 97, 128, 129, 255, 300, 511, 640]))
        B = int(rng.integers(1, 4))
        causal = bool(rng.random() < 0.7)
        q_std = float(rng.choice([0.5, 1.0, 2.0, 3.0]))
        scale = float(rng.uniform(0.05, 0.3)) * (1 if D == 64 else 0.7)
        cases.append((B, T, G * Hkv, Hkv, D, dtype, causal, q_std, round(scale, 4), 7000 + i))
    return cases


CASES = _draw_cases(24) + [
    # (B, T, Hq, Hkv, D, dtype, causal, q_std, scale, seed): degenerate scales
    (2, 200, 6, 2, 64, "bf16", True, 1.0, 0.0, 7100),
    (1, 300, 4, 1, 64, "bf16", True, 1.0, -0.125, 7101),
    (2, 129, 6, 3, 64, "f16", False, 1.0, -0.2, 7102),
    (1, 160, 4, 2, 128, "bf16", True, 1.0, -0.0884, 7103),
    (1, 100, 2, 2, 64, "f32", True, 1.0, -0.125, 7104),
    (1, 100, 2, 1, 64, "f32", False, 1.0, 0.0, 7105),
    (1, 257, 8, 2, 64, "bf16", True, 1.0, 1.0, 7106),   # scores of order 8: nearly one-hot rows
]


def _id(c):
    B, T, Hq, Hkv, D, dtype, causal, q_std, scale, seed = c
    return f"B{B}T{T}H{Hq}/{Hkv}D{D}{dtype}{'c' if causal else 'n'}s{scale}q{q_std}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_parity(case):
    B, T, Hq, Hkv, D, dtype, causal, q_std, scale, seed = case
    w = W.custom(B, T, Hq, Hkv, D, dtype, seed=seed, q_std=q_std, scale=scale, causal=causal)
    inp = W.generate(w)
    say("random-shape parity", w.label(), "scale", scale, "q_std", q_std)
    gpu = as_numpy(run_gpu(inp))
    print(w.label(), check_against(gpu, oracle_full(inp), dtype, _id(case)))
