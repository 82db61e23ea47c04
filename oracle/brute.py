"""Pure-Python scalar-loop attention for tiny inputs (T, D of a few dozen).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

This is a second, independent statement of the same definition as
``oracle.attention`` (the textbook causal softmax attention that the fused
kernel of "Training a 100M transformer in pure Rust: RustingBrain vs PyTorch
and TensorFlow", section "Step 2: fused flash attention", computes): every
sum is an exactly rounded ``math.fsum`` over Python floats, every score is
formed element by element, and no array library is involved.  It exists to
pin the vectorised oracle (matrix products, masking by index arrays, the
max-shifted log-sum-exp) against loops a reader can check by eye.
"""
from __future__ import annotations

import math


def _lists(x):
    return x.tolist() if hasattr(x, "tolist") else x


def _shape(q, k):
    B, T, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, T, Hq, Hkv, D


def _row(qr, k, b, g, i, T, scale, causal):
    """Visible key indices and their scores for query row ``i``."""
    js = [j for j in range(T) if (j <= i or not causal)]
    s = [scale * math.fsum(qr[d] * k[b][j][g][d] for d in range(len(qr))) for j in js]
    return js, s


def _lse(s):
    m = max(s)
    return m + math.log(math.fsum(math.exp(x - m) for x in s))


def brute_fwd(q, k, v, scale, causal=True):
    """Returns nested lists ``(o[B][T][Hq][D], lse[B][Hq][T])``."""
    q, k, v = _lists(q), _lists(k), _lists(v)
    B, T, Hq, Hkv, D = _shape(q, k)
    G = Hq // Hkv
    o = [[[[0.0] * D for _ in range(Hq)] for _ in range(T)] for _ in range(B)]
    lse = [[[0.0] * T for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                js, s = _row(q[b][i][h], k, b, g, i, T, scale, causal)
                L = _lse(s)
                lse[b][h][i] = L
                p = [math.exp(x - L) for x in s]
                for d in range(D):
                    o[b][i][h][d] = math.fsum(pj * v[b][j][g][d] for pj, j in zip(p, js))
    return o, lse


def brute_bwd(q, k, v, dO, scale, causal=True):
    """Returns nested lists ``(dq, dk, dv, delta)`` of the gradient of sum(o*dO)."""
    q, k, v, dO = _lists(q), _lists(k), _lists(v), _lists(dO)
    B, T, Hq, Hkv, D = _shape(q, k)
    G = Hq // Hkv
    o, lse = brute_fwd(q, k, v, scale, causal)
    dq = [[[[0.0] * D for _ in range(Hq)] for _ in range(T)] for _ in range(B)]
    delta = [[[0.0] * T for _ in range(Hq)] for _ in range(B)]
    # Terms of dk and dv are gathered per (b, g, j, d) and summed once with fsum.
    dk_terms = [[[[[] for _ in range(D)] for _ in range(Hkv)] for _ in range(T)] for _ in range(B)]
    dv_terms = [[[[[] for _ in range(D)] for _ in range(Hkv)] for _ in range(T)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                js, s = _row(q[b][i][h], k, b, g, i, T, scale, causal)
                p = [math.exp(x - lse[b][h][i]) for x in s]
                dOr = dO[b][i][h]
                dl = math.fsum(dOr[d] * o[b][i][h][d] for d in range(D))
                delta[b][h][i] = dl
                ds = []
                for pj, j in zip(p, js):
                    dp = math.fsum(dOr[d] * v[b][j][g][d] for d in range(D))
                    ds.append(pj * (dp - dl))
                for d in range(D):
                    dq[b][i][h][d] = scale * math.fsum(dsj * k[b][j][g][d] for dsj, j in zip(ds, js))
                for pj, dsj, j in zip(p, ds, js):
                    for d in range(D):
                        dk_terms[b][j][g][d].append(scale * dsj * q[b][i][h][d])
                        dv_terms[b][j][g][d].append(pj * dOr[d])
    dk = [[[[math.fsum(dk_terms[b][j][g][d]) for d in range(D)] for g in range(Hkv)]
           for j in range(T)] for b in range(B)]
    dv = [[[[math.fsum(dv_terms[b][j][g][d]) for d in range(D)] for g in range(Hkv)]
           for j in range(T)] for b in range(B)]
    return dq, dk, dv, delta
