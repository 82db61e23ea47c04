"""Pins of the rotary-embedding oracle (oracle/rope.py) against facts fixed by the
mathematics: a hand-rotated example, the identity at angle 0, orthogonality and
the relative-position property of exact tables, central finite differences
through the whole rotated attention, pure-Python loops, and the reduction to
plain attention.  Each pin takes the functions under test, so the mutation
tests can run them on planted mistakes."""
import math

import numpy as np

from oracle import brute
from oracle_pins import rand, rel_err, tiny_inputs


def exact_tables(T, D, base=10000.0):
    """fp64 tables of the rotary angles t * base^(-2i/D), [T, D/2]."""
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(T, dtype=np.float64)[:, None] * base ** (-2.0 * i / D)[None, :]
    return np.cos(ang), np.sin(ang)


def pin_hand_rotation(apply, apply_t):
    """e_0 and e_1 at an angle a become (cos a, sin a) and (-sin a, cos a); the
    transpose maps them back."""
    a = 0.7
    cos = np.array([[1.0, 1.0], [math.cos(a), 1.0]])
    sin = np.array([[0.0, 0.0], [math.sin(a), 0.0]])
    x = np.zeros((1, 2, 1, 4))
    x[0, 1, 0, 0] = 1.0
    y = apply(x, cos, sin)
    assert np.allclose(y[0, 1, 0], [math.cos(a), math.sin(a), 0, 0], atol=1e-15), y[0, 1, 0]
    x[0, 1, 0, 0], x[0, 1, 0, 1] = 0.0, 1.0
    y = apply(x, cos, sin)
    assert np.allclose(y[0, 1, 0], [-math.sin(a), math.cos(a), 0, 0], atol=1e-15), y[0, 1, 0]
    assert np.allclose(apply_t(y, cos, sin), x, atol=1e-15)
    # position 0 has angle 0: unchanged
    assert np.array_equal(y[0, 0], x[0, 0])


def pin_orthogonal(apply, apply_t):
    """With exact tables each rotation keeps norms and its transpose undoes it."""
    T, D = 9, 8
    cos, sin = exact_tables(T, D)
    x = rand((2, T, 3, D), 5)
    y = apply(x, cos, sin)
    assert rel_err(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1)) < 1e-14
    assert rel_err(apply_t(y, cos, sin), x) < 1e-14


def pin_relative_position(apply):
    """<R_i q, R_j k> depends on j - i only: shifting both positions by s keeps it."""
    T, D = 12, 6
    cos, sin = exact_tables(T, D, base=50.0)
    qv, kv = rand((D,), 11), rand((D,), 12)
    x = np.zeros((1, T, 2, D))
    x[0, :, 0] = qv
    x[0, :, 1] = kv
    y = apply(x, cos, sin)
    dots = y[0, :, 0] @ y[0, :, 1].T  # [i, j]
    for s in (1, 3):
        assert rel_err(dots[s:, s:], dots[:T - s, :T - s]) < 1e-12


def pin_rope_finite_differences(fwd_r, bwd_r, h=1e-6, tol=1e-7):
    """dq, dk, dv == central differences of sum(o * dO) through the rotation, for
    arbitrary (non-orthogonal) tables, where only the transpose is the gradient."""
    for causal in (True, False):
        B, T, Hq, Hkv, D = 1, 4, 2, 1, 4
        q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 303 if causal else 404)
        cos, sin = rand((T, D // 2), 31), rand((T, D // 2), 32)
        scale = 0.53

        def loss(q_, k_, v_):
            return float(np.sum(fwd_r(q_, k_, v_, cos, sin, scale, causal)[0] * dO))

        dq, dk, dv, _ = bwd_r(q, k, v, dO, cos, sin, scale, causal)
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


def _brute_rotate(x, cos, sin):
    B, T, H, D = x.shape
    out = np.zeros_like(x)
    for b in range(B):
        for t in range(T):
            for hh in range(H):
                for i in range(D // 2):
                    c, s = float(cos[t][i]), float(sin[t][i])
                    a, bb = float(x[b, t, hh, 2 * i]), float(x[b, t, hh, 2 * i + 1])
                    out[b, t, hh, 2 * i] = a * c - bb * s
                    out[b, t, hh, 2 * i + 1] = a * s + bb * c
    return out


def pin_rope_brute(fwd_r):
    """Scalar loops: rotate element by element, then the pure-Python attention."""
    B, T, Hq, Hkv, D = 1, 5, 4, 2, 4
    q, k, v, _ = tiny_inputs(B, T, Hq, Hkv, D, 55)
    cos, sin = exact_tables(T, D, base=7.0)
    o, lse = fwd_r(q, k, v, cos, sin, 0.45, True)
    bo, blse = brute.brute_fwd(_brute_rotate(q, cos, sin), _brute_rotate(k, cos, sin), v, 0.45, True)
    assert rel_err(o, bo) < 1e-12 and rel_err(lse, blse) < 1e-12


def pin_identity_tables(fwd_r, bwd_r, fwd, bwd):
    """cos = 1, sin = 0 everywhere: the rotated attention is the plain one."""
    B, T, Hq, Hkv, D = 2, 6, 4, 2, 4
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 77)
    cos, sin = np.ones((T, D // 2)), np.zeros((T, D // 2))
    for a, b in zip(fwd_r(q, k, v, cos, sin, 0.3, True), fwd(q, k, v, 0.3, True)):
        assert rel_err(a, b) < 1e-15
    for a, b in zip(bwd_r(q, k, v, dO, cos, sin, 0.3, True), bwd(q, k, v, dO, 0.3, True)):
        assert rel_err(a, b) < 1e-15


ROPE_PINS = [
    ("hand_rotation", lambda m: pin_hand_rotation(m.apply_rope, m.apply_rope_transpose)),
    ("orthogonal", lambda m: pin_orthogonal(m.apply_rope, m.apply_rope_transpose)),
    ("relative_position", lambda m: pin_relative_position(m.apply_rope)),
    ("finite_differences", lambda m: pin_rope_finite_differences(m.ref_fwd_rope, m.ref_bwd_rope)),
    ("brute", lambda m: pin_rope_brute(m.ref_fwd_rope)),
    ("identity_tables", lambda m: pin_identity_tables(m.ref_fwd_rope, m.ref_bwd_rope, m.ref_fwd, m.ref_bwd)),
]
