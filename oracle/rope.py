"""fp64 oracle: rotary position embedding of q and k ahead of the attention.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  The product path
never imports this module.

"Training a 100M transformer in pure Rust: RustingBrain vs PyTorch and
TensorFlow", section "The setup", lists rotary positions among the model's
parts and prints nothing more: no convention, base or table.  The reading
taken (listed in the design doc) is the original rotary formulation: at position t
each adjacent pair of dimensions (2i, 2i+1) of a query or key vector is
rotated by the angle t * theta_i,

    x'[2i]   = x[2i] cos(t, i) - x[2i+1] sin(t, i)
    x'[2i+1] = x[2i] sin(t, i) + x[2i+1] cos(t, i),

with the cos / sin tables ([T, D/2], float32) supplied by the caller, the same
positions 0 .. T-1 for queries and keys, and v not rotated.  Attention then
runs on the rotated q', k' (oracle.attention), and the chain rule gives the
input gradients through the transpose of each 2x2 rotation:

    dq[2i]   =  dq'[2i] cos + dq'[2i+1] sin
    dq[2i+1] = -dq'[2i] sin + dq'[2i+1] cos            (same for dk).

The transpose is the exact gradient whatever the table values are, so it is
used even where float32 tables make cos^2 + sin^2 differ from 1 by rounding.
"""
from __future__ import annotations

import numpy as np

from .attention import ref_bwd, ref_fwd


def _pairs(x):
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % 2:
        raise ValueError("head_dim must be even")
    return x[..., 0::2], x[..., 1::2]


def _tables(cos, sin, T):
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    if c.shape != s.shape or c.shape[0] < T:
        raise ValueError("cos and sin must be [>= T, D/2]")
    # broadcast over [B, T, H, D/2]
    return c[None, :T, None, :], s[None, :T, None, :]


def apply_rope(x, cos, sin):
    """x [B, T, H, D] -> x' (each adjacent pair rotated by its position's angle)."""
    a, b = _pairs(x)
    c, s = _tables(cos, sin, a.shape[1])
    out = np.empty(np.shape(x), dtype=np.float64)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def apply_rope_transpose(y, cos, sin):
    """The transpose of apply_rope: maps a gradient wrt x' to the gradient wrt x."""
    a, b = _pairs(y)
    c, s = _tables(cos, sin, a.shape[1])
    out = np.empty(np.shape(y), dtype=np.float64)
    out[..., 0::2] = a * c + b * s
    out[..., 1::2] = -a * s + b * c
    return out


def ref_fwd_rope(q, k, v, cos, sin, scale, causal=True):
    """(o, lse) of attention on the rotated q and k."""
    return ref_fwd(apply_rope(q, cos, sin), apply_rope(k, cos, sin), v, scale, causal)


def ref_bwd_rope(q, k, v, dO, cos, sin, scale, causal=True):
    """(dq, dk, dv, delta): gradients of sum(o * dO) wrt the unrotated q, k and v."""
    dq_r, dk_r, dv, delta = ref_bwd(apply_rope(q, cos, sin), apply_rope(k, cos, sin), v, dO,
                                    scale, causal)
    return apply_rope_transpose(dq_r, cos, sin), apply_rope_transpose(dk_r, cos, sin), dv, delta
