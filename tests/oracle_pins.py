"""Pins for the CPU oracle: facts fixed by the mathematics, not by the oracle.

Each ``pin_*`` takes the implementation under test (forward and/or backward
callables with the signatures of ``oracle.ref_fwd`` / ``oracle.ref_bwd``) and
raises ``AssertionError`` if it disagrees with a fact that does not depend on
that implementation: brute force, finite differences, closed forms, symmetry
invariants and an independent library routine.  ``test_oracle_pins.py`` runs
them on the oracle; ``test_oracle_mutations.py`` runs them on copies of the
oracle with planted mistakes and checks that some pin fails.

The operation is the causal softmax attention that the fused flash-attention
kernel of "Training a 100M transformer in pure Rust: RustingBrain vs PyTorch
and TensorFlow" (section "Step 2: fused flash attention") computes, with the
grouped-query shape of that page's section "The setup".
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from oracle import brute

TINY_SHAPES = [  # (B, T, Hq, Hkv, D)
    (1, 5, 4, 2, 3),
    (2, 4, 2, 2, 4),
    (1, 6, 3, 1, 2),
]


def rand(shape, seed, std=1.0):
    return std * np.random.default_rng(seed).standard_normal(shape)


def tiny_inputs(B, T, Hq, Hkv, D, seed):
    return (rand((B, T, Hq, D), seed), rand((B, T, Hkv, D), seed + 1),
            rand((B, T, Hkv, D), seed + 2), rand((B, T, Hq, D), seed + 3))


def rel_err(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    den = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / den


# ----------------------------------------------------------------------------
# brute force
# ----------------------------------------------------------------------------

def pin_brute(fwd, bwd, tol=1e-12):
    """Vectorised oracle == pure-Python fsum loops on tiny shapes, causal and full."""
    for n, (B, T, Hq, Hkv, D) in enumerate(TINY_SHAPES):
        for causal in (True, False):
            q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 10 * n + 7)
            scale = 0.37
            o, lse = fwd(q, k, v, scale, causal)
            bo, blse = brute.brute_fwd(q, k, v, scale, causal)
            assert rel_err(o, bo) < tol, ("o", B, T, Hq, Hkv, D, causal)
            assert rel_err(lse, blse) < tol, ("lse", B, T, Hq, Hkv, D, causal)
            dq, dk, dv, _ = bwd(q, k, v, dO, scale, causal)
            bdq, bdk, bdv, _ = brute.brute_bwd(q, k, v, dO, scale, causal)
            for name, a, b in (("dq", dq, bdq), ("dk", dk, bdk), ("dv", dv, bdv)):
                assert rel_err(a, b) < tol, (name, B, T, Hq, Hkv, D, causal)


# ----------------------------------------------------------------------------
# finite differences of L = sum(o * dO)
# ----------------------------------------------------------------------------

def pin_finite_differences(fwd, bwd, h=1e-6, tol=1e-7):
    """Analytic gradients == central differences of L = sum(o * dO)."""
    for causal in (True, False):
        B, T, Hq, Hkv, D = 1, 5, 4, 2, 3
        q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 101 if causal else 202)
        scale = 0.61

        def loss(q_, k_, v_):
            return float(np.sum(fwd(q_, k_, v_, scale, causal)[0] * dO))

        dq, dk, dv, _ = bwd(q, k, v, dO, scale, causal)
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            args = [q, k, v]
            fd = np.zeros_like(args[which])
            for idx in np.ndindex(*args[which].shape):
                plus = [a.copy() for a in args]
                minus = [a.copy() for a in args]
                plus[which][idx] += h
                minus[which][idx] -= h
                fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
            assert rel_err(grad, fd) < tol, (("dq", "dk", "dv")[which], causal, rel_err(grad, fd))


# ----------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------

def pin_row0(fwd):
    """Under the causal mask query 0 sees only key 0: o_0 = v_0, lse_0 = scale*<q_0,k_0>."""
    B, T, Hq, Hkv, D = 2, 7, 6, 3, 5
    q, k, v, _ = tiny_inputs(B, T, Hq, Hkv, D, 5)
    scale = 0.8
    o, lse = fwd(q, k, v, scale, True)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            assert np.array_equal(o[b, 0, h], v[b, 0, g]) or rel_err(o[b, 0, h], v[b, 0, g]) < 1e-15
            expect = scale * math.fsum(q[b, 0, h, d] * k[b, 0, g, d] for d in range(D))
            assert abs(lse[b, h, 0] - expect) <= 1e-14 * max(1.0, abs(expect))


def pin_zero_queries(fwd, bwd):
    """Q = 0 makes every visible score 0: o_i is the mean of v_0..v_i, lse_i = ln(i+1),
    and the key gradient vanishes (dS multiplies q, which is zero)."""
    B, T, Hq, Hkv, D = 1, 9, 4, 2, 3
    _, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 11)
    q = np.zeros((B, T, Hq, D))
    o, lse = fwd(q, k, v, 0.5, True)
    counts = np.arange(1, T + 1, dtype=np.float64)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        prefix_mean = np.cumsum(v[0, :, g], axis=0) / counts[:, None]
        assert rel_err(o[0, :, h], prefix_mean) < 1e-14
        assert np.max(np.abs(lse[0, h] - np.log(counts))) < 1e-14
    _, dk, _, _ = bwd(q, k, v, dO, 0.5, True)
    assert np.max(np.abs(dk)) == 0.0


def pin_single_token(fwd, bwd):
    """T = 1: o = v; dq = dk = 0; dv = sum of dO over the query heads of the group."""
    B, T, Hq, Hkv, D = 3, 1, 6, 2, 4
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 21)
    G = Hq // Hkv
    for causal in (True, False):
        o, lse = fwd(q, k, v, 0.3, causal)
        assert rel_err(o, np.repeat(v, G, axis=2)) < 1e-15
        dq, dk, dv, _ = bwd(q, k, v, dO, 0.3, causal)
        assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15
        assert rel_err(dv, dO.reshape(B, T, Hkv, G, D).sum(axis=3)) < 1e-14


def pin_constant_values(fwd, bwd):
    """All value rows equal c: o_i = c for every row and dq = dk = 0 (dP_ij is constant
    along j, so dS = P * (dP - delta) vanishes)."""
    B, T, Hq, Hkv, D = 1, 6, 2, 1, 3
    q, k, _, dO = tiny_inputs(B, T, Hq, Hkv, D, 31)
    c = np.array([0.25, -1.5, 3.0])
    v = np.broadcast_to(c, (B, T, Hkv, D)).copy()
    for causal in (True, False):
        o, _ = fwd(q, k, v, 0.9, causal)
        assert np.max(np.abs(o - c)) < 1e-14
        dq, dk, _, _ = bwd(q, k, v, dO, 0.9, causal)
        assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


def pin_log_scores_example(fwd, bwd):
    """A worked example with rational probabilities, derived by hand.

    D = 1, scale = 1, q_i = 1, k_j = ln(j+1), v_j = j, dO_i = 1, causal.
    Scores are s_ij = ln(j+1), so P_ij = (j+1) / S_i with S_i = (i+1)(i+2)/2:
      lse_i = ln(S_i);
      o_i   = sum_{j<=i} j(j+1) / S_i = 2i/3;
      dv_j  = sum_{i>=j} P_ij = 2(j+1) sum_{i>=j} (1/(i+1) - 1/(i+2))
            = 2 - 2(j+1)/(T+1)                      (telescoping);
      dS_ij = P_ij (j - o_i), so
      dk_j  = sum_{i>=j} P_ij (j - 2i/3)   and   dq_i = sum_{j<=i} P_ij (j - 2i/3) ln(j+1),
    evaluated here with exact fractions for the rational parts.
    """
    T = 12
    q = np.ones((1, T, 1, 1))
    k = np.log(np.arange(1, T + 1, dtype=np.float64)).reshape(1, T, 1, 1)
    v = np.arange(T, dtype=np.float64).reshape(1, T, 1, 1)
    dO = np.ones((1, T, 1, 1))
    o, lse = fwd(q, k, v, 1.0, True)
    dq, dk, dv, _ = bwd(q, k, v, dO, 1.0, True)

    def P(i, j):
        return Fraction(2 * (j + 1), (i + 1) * (i + 2))

    for i in range(T):
        assert abs(o[0, i, 0, 0] - 2.0 * i / 3.0) < 1e-13
        assert abs(lse[0, 0, i] - math.log((i + 1) * (i + 2) / 2)) < 1e-13
        want_dq = math.fsum(float(P(i, j) * (j - Fraction(2 * i, 3))) * math.log(j + 1)
                            for j in range(i + 1))
        assert abs(dq[0, i, 0, 0] - want_dq) < 1e-13
    for j in range(T):
        assert abs(dv[0, j, 0, 0] - float(2 - Fraction(2 * (j + 1), T + 1))) < 1e-13
        want_dk = float(sum(P(i, j) * (j - Fraction(2 * i, 3)) for i in range(j, T)))
        assert abs(dk[0, j, 0, 0] - want_dk) < 1e-13


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def pin_probabilities(probs):
    """Rows of P sum to 1; entries above the diagonal are exactly 0 under the mask."""
    B, T, Hq, Hkv, D = 1, 8, 3, 1, 4
    q, k, _, _ = tiny_inputs(B, T, Hq, Hkv, D, 41)
    for h in range(Hq):
        p = probs(q, k, 0.7, True, 0, h)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-14
        assert np.all(p[np.triu_indices(T, 1)] == 0.0)
        assert np.all(p[np.tril_indices(T)] > 0.0)
        pf = probs(q, k, 0.7, False, 0, h)
        assert np.max(np.abs(pf.sum(axis=1) - 1.0)) < 1e-14


def pin_linear_in_values(fwd):
    """o(a V1 + b V2) = a o(V1) + b o(V2)."""
    B, T, Hq, Hkv, D = 2, 6, 4, 2, 3
    q, k, v1, _ = tiny_inputs(B, T, Hq, Hkv, D, 51)
    v2 = rand(v1.shape, 52)
    a, b = 1.75, -0.5
    o12, _ = fwd(q, k, a * v1 + b * v2, 0.4, True)
    o1, _ = fwd(q, k, v1, 0.4, True)
    o2, _ = fwd(q, k, v2, 0.4, True)
    assert rel_err(o12, a * o1 + b * o2) < 1e-13


def pin_key_translation(fwd, bwd):
    """Adding one vector c to every key adds scale*<q_i, c> to row i of the scores,
    which the softmax removes: o and dq are unchanged (dq because the rows of dS sum
    to zero), lse shifts by scale*<q_i, c>, and sum_j dk_j = 0 for every (b, g)."""
    B, T, Hq, Hkv, D = 2, 5, 4, 2, 3
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 61)
    c = np.array([0.3, -1.1, 2.0])
    scale = 0.45
    for causal in (True, False):
        o, lse = fwd(q, k, v, scale, causal)
        o2, lse2 = fwd(q, k + c, v, scale, causal)
        assert rel_err(o2, o) < 1e-12
        shift = scale * np.einsum("bthd,d->bht", q, c)
        assert np.max(np.abs(lse2 - lse - shift)) < 1e-12
        dq, dk, _, _ = bwd(q, k, v, dO, scale, causal)
        dq2, _, _, _ = bwd(q, k + c, v, dO, scale, causal)
        assert rel_err(dq2, dq) < 1e-11
        assert np.max(np.abs(dk.sum(axis=1))) < 1e-12 * max(1.0, np.max(np.abs(dk)))


def pin_gradient_sums(bwd):
    """sum_j dv_j = sum over the group's heads of sum_i dO_i (rows of P sum to 1), and
    <dq, q> over the group equals <dk, k> (scores are bilinear in q and k)."""
    B, T, Hq, Hkv, D = 2, 6, 6, 2, 3
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 71)
    G = Hq // Hkv
    for causal in (True, False):
        dq, dk, dv, _ = bwd(q, k, v, dO, 0.55, causal)
        for b in range(B):
            for g in range(Hkv):
                heads = slice(g * G, (g + 1) * G)
                want = dO[b, :, heads].sum(axis=(0, 1))
                assert np.max(np.abs(dv[b, :, g].sum(axis=0) - want)) < 1e-12
                lhs = float(np.sum(dq[b, :, heads] * q[b, :, heads]))
                rhs = float(np.sum(dk[b, :, g] * k[b, :, g]))
                assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def pin_gqa_is_repeated_mha(fwd, bwd):
    """GQA(Hq, Hkv) == MHA on K, V repeat-interleaved to Hq heads; dk, dv of the GQA
    call are the sums over each group of the MHA gradients."""
    B, T, Hq, Hkv, D = 2, 5, 6, 2, 3
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 81)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    for causal in (True, False):
        o, lse = fwd(q, k, v, 0.6, causal)
        o_m, lse_m = fwd(q, kr, vr, 0.6, causal)
        assert rel_err(o, o_m) < 1e-15 and rel_err(lse, lse_m) < 1e-15
        dq, dk, dv, _ = bwd(q, k, v, dO, 0.6, causal)
        dq_m, dk_m, dv_m, _ = bwd(q, kr, vr, dO, 0.6, causal)
        assert rel_err(dq, dq_m) < 1e-14
        assert rel_err(dk, dk_m.reshape(B, T, Hkv, G, D).sum(axis=3)) < 1e-13
        assert rel_err(dv, dv_m.reshape(B, T, Hkv, G, D).sum(axis=3)) < 1e-13


def pin_library_sdpa(fwd, bwd):
    """Cross-check against torch's scaled_dot_product_attention in float64 on the CPU
    (a different code path: agreement is evidence, not identity)."""
    import torch
    B, T, Hq, Hkv, D = 2, 17, 6, 3, 8
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 91)
    G = Hq // Hkv
    for causal in (True, False):
        tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_(True)
        tk = torch.tensor(np.repeat(k, G, axis=2)).permute(0, 2, 1, 3).requires_grad_(True)
        tv = torch.tensor(np.repeat(v, G, axis=2)).permute(0, 2, 1, 3).requires_grad_(True)
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                              scale=0.33)
        to.backward(torch.tensor(dO).permute(0, 2, 1, 3))
        o, _ = fwd(q, k, v, 0.33, causal)
        dq, dk, dv, _ = bwd(q, k, v, dO, 0.33, causal)
        assert rel_err(o, to.detach().permute(0, 2, 1, 3).numpy()) < 1e-12
        assert rel_err(dq, tq.grad.permute(0, 2, 1, 3).numpy()) < 1e-12
        dk_t = tk.grad.permute(0, 2, 1, 3).numpy().reshape(B, T, Hkv, G, D).sum(axis=3)
        dv_t = tv.grad.permute(0, 2, 1, 3).numpy().reshape(B, T, Hkv, G, D).sum(axis=3)
        assert rel_err(dk, dk_t) < 1e-12 and rel_err(dv, dv_t) < 1e-12


def pin_delta(bwd, fwd):
    """delta_i = <dO_i, o_i> of the forward output (the softmax-backward row term)."""
    B, T, Hq, Hkv, D = 1, 7, 4, 2, 3
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 97)
    o, _ = fwd(q, k, v, 0.5, True)
    _, _, _, delta = bwd(q, k, v, dO, 0.5, True)
    want = np.array([[[math.fsum(dO[0, i, h, d] * o[0, i, h, d] for d in range(D))
                       for i in range(T)] for h in range(Hq)]])
    assert np.max(np.abs(delta - want)) < 1e-13


ALL_PINS = [
    ("brute", lambda f, b, p: pin_brute(f, b)),
    ("finite_differences", lambda f, b, p: pin_finite_differences(f, b)),
    ("row0", lambda f, b, p: pin_row0(f)),
    ("zero_queries", lambda f, b, p: pin_zero_queries(f, b)),
    ("single_token", lambda f, b, p: pin_single_token(f, b)),
    ("constant_values", lambda f, b, p: pin_constant_values(f, b)),
    ("log_scores_example", lambda f, b, p: pin_log_scores_example(f, b)),
    ("probabilities", lambda f, b, p: pin_probabilities(p)),
    ("linear_in_values", lambda f, b, p: pin_linear_in_values(f)),
    ("key_translation", lambda f, b, p: pin_key_translation(f, b)),
    ("gradient_sums", lambda f, b, p: pin_gradient_sums(b)),
    ("gqa_is_repeated_mha", lambda f, b, p: pin_gqa_is_repeated_mha(f, b)),
    ("library_sdpa", lambda f, b, p: pin_library_sdpa(f, b)),
    ("delta", lambda f, b, p: pin_delta(b, f)),
]
