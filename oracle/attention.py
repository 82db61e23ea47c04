"""fp64 numpy oracle: causal (grouped-query) scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  The product path
never imports this module.

What is computed
----------------
The pages name the computation but do not print its formulas.  "Training a
100M transformer in pure Rust: RustingBrain vs PyTorch and TensorFlow",
section "Step 1: measure before changing anything", names the unfused
kernels ``causal_softmax_lse``, ``causal_softmax_bwd`` and
``causal_probs_from_lse`` and the [seq_len, seq_len] fp32 score matrix they
write and read back; section "Step 2: fused flash attention" replaces them by
one fused causal flash-attention forward and backward.  Section "The setup"
fixes the shapes that matter here: grouped-query attention with 12 query
heads, 4 KV heads and head_dim 64.  A fused kernel computes exactly what the
unfused chain computes, so this oracle is the plain textbook definition,
written out with the full score matrix (one batch element and head at a time
to bound memory):

    s[i, j]  = scale * <q[i], k[j]>,      masked to -inf where j > i (causal)
    lse[i]   = log(sum_j exp(s[i, j]))     (natural log, per query row)
    P[i, j]  = exp(s[i, j] - lse[i])      ("probs from lse")
    o[i]     = sum_j P[i, j] v[j]

and its analytic gradients for a cotangent dO (the gradient of sum(o * dO)):

    delta[i] = <dO[i], o[i]>
    dP[i, j] = <dO[i], v[j]>
    dS[i, j] = P[i, j] * (dP[i, j] - delta[i])     (softmax backward)
    dq[i]    = scale * sum_j dS[i, j] k[j]
    dk[j]    = scale * sum_{heads h of the group} sum_i dS[i, j] q[i]
    dv[j]    =         sum_{heads h of the group} sum_i P[i, j] dO[i]

Readings where the pages are silent (each listed in the design doc):
  * layout: q, o, dO, dq are [B, T, Hq, D]; k, v, dk, dv are [B, T, Hkv, D];
    lse and delta are [B, Hq, T];
  * query head h reads KV head h // (Hq // Hkv) (consecutive groups);
  * causal keeps the diagonal (key j is visible to query i iff j <= i), with
    T_q == T_k == T and no offset;
  * lse is in natural log.

All arithmetic is float64.  Inputs are converted to float64 on entry; for
bf16 inputs the caller passes the already-rounded values widened exactly.
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head ``h``: consecutive groups of Hq // Hkv."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, T, H, D]")
    B, T, Hq, D = q.shape
    if k.shape[:2] != (B, T) or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("k and v must be [B, T, Hkv, D] matching q")
    Hkv = k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, T, Hq, Hkv, D


def _scores(qh, kh, scale, causal):
    """Scaled scores of one (batch, head): [T, T] with the causal mask applied."""
    s = scale * (qh @ kh.T)
    if causal:
        T = s.shape[0]
        s[np.triu_indices(T, 1)] = -np.inf
    return s


def _softmax_lse(s):
    """Row-wise log-sum-exp and probabilities of a masked score matrix."""
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p, lse


def ref_probs(q, k, scale, causal=True, b=0, h=0):
    """The [T, T] probability matrix P of batch element ``b``, query head ``h``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Hq, Hkv = q.shape[2], k.shape[2]
    g = kv_head_of(h, Hq, Hkv)
    p, _ = _softmax_lse(_scores(q[b, :, h, :], k[b, :, g, :], scale, causal))
    return p


def ref_fwd(q, k, v, scale, causal=True):
    """Forward pass.  Returns ``(o [B,T,Hq,D], lse [B,Hq,T])`` in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hq, Hkv, D = _check(q, k, v)
    o = np.empty((B, T, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            p, lse[b, h] = _softmax_lse(_scores(q[b, :, h], k[b, :, g], scale, causal))
            o[b, :, h] = p @ v[b, :, g]
    return o, lse


def ref_bwd(q, k, v, dO, scale, causal=True):
    """Backward pass of ``sum(o * dO)``.

    Returns ``(dq, dk, dv, delta)`` in float64; ``delta`` is [B, Hq, T] and is
    computed from the oracle's own float64 forward output.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, T, Hq, Hkv, D = _check(q, k, v)
    if dO.shape != q.shape:
        raise ValueError("dO must have the shape of q")
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.empty((B, Hq, T), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            qh, kh, vh, dOh = q[b, :, h], k[b, :, g], v[b, :, g], dO[b, :, h]
            p, _ = _softmax_lse(_scores(qh, kh, scale, causal))
            oh = p @ vh
            delta[b, h] = (dOh * oh).sum(axis=1)
            dp = dOh @ vh.T
            ds = p * (dp - delta[b, h][:, None])
            dq[b, :, h] = scale * (ds @ kh)
            dk[b, :, g] += scale * (ds.T @ qh)
            dv[b, :, g] += p.T @ dOh
    return dq, dk, dv, delta


def _group_slices(q, k, v, b, g):
    B, T, Hq, Hkv, D = _check(q, k, v)
    G = Hq // Hkv
    return q[b:b + 1, :, g * G:(g + 1) * G], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1]


def ref_fwd_group(q, k, v, scale, causal, b, g):
    """Forward of one (batch element, KV-head group) unit.

    Returns ``(o [T, G, D], lse [G, T])`` for the G query heads that read KV
    head ``g`` of batch element ``b``.  Units are independent, so this equals
    the corresponding slice of :func:`ref_fwd`; it lets large workloads be
    checked on sampled units.
    """
    qs, ks, vs = _group_slices(q, k, v, b, g)
    o, lse = ref_fwd(qs, ks, vs, scale, causal)
    return o[0], lse[0]


def ref_bwd_group(q, k, v, dO, scale, causal, b, g):
    """Backward of one (batch element, KV-head group) unit.

    Returns ``(dq [T, G, D], dk [T, D], dv [T, D], delta [G, T])``.
    """
    qs, ks, vs = _group_slices(q, k, v, b, g)
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    dOs = dO[b:b + 1, :, g * G:(g + 1) * G]
    dq, dk, dv, delta = ref_bwd(qs, ks, vs, dOs, scale, causal)
    return dq[0], dk[0, :, 0], dv[0, :, 0], delta[0]


def _row_stats(q, k, v, dO, scale, causal, b, h, i):
    """One query row of head ``h``: the definitions above for row ``i`` alone.

    Returns ``(p, o_i, lse_i, delta_i, ds, n)``: the probabilities and dS of the
    row over its ``n`` visible keys (``i + 1`` under the causal mask, else T).
    Cost O(T * D), so long sequences can be checked row by row.
    """
    Hq, Hkv, T = q.shape[2], k.shape[2], q.shape[1]
    g = kv_head_of(h, Hq, Hkv)
    n = i + 1 if causal else T
    kh = np.asarray(k[b, :n, g], dtype=np.float64)
    vh = np.asarray(v[b, :n, g], dtype=np.float64)
    qi = np.asarray(q[b, i, h], dtype=np.float64)
    dOi = np.asarray(dO[b, i, h], dtype=np.float64) if dO is not None else None
    s = scale * (kh @ qi)
    m = s.max()
    lse = m + np.log(np.exp(s - m).sum())
    p = np.exp(s - lse)
    o = p @ vh
    if dOi is None:
        return p, o, lse, None, None, n
    delta = float(dOi @ o)
    ds = p * (vh @ dOi - delta)
    return p, o, lse, delta, ds, n


def ref_query_rows(q, k, v, dO, scale, causal, b, h, rows):
    """o, lse, delta and dq of the listed query rows of (batch ``b``, head ``h``).

    Same definitions as :func:`ref_fwd` and :func:`ref_bwd`, evaluated one row
    at a time (a row of causal attention needs only its own query and the keys
    it sees), so the cost is O(len(rows) * T * D) instead of O(T^2 * D).
    Returns a dict of float64 arrays: ``o`` and ``dq`` [len(rows), D], ``lse``
    and ``delta`` [len(rows)].
    """
    D = q.shape[3]
    out = {"o": np.empty((len(rows), D)), "lse": np.empty(len(rows)),
           "delta": np.empty(len(rows)), "dq": np.empty((len(rows), D))}
    g = kv_head_of(h, q.shape[2], k.shape[2])
    for r, i in enumerate(rows):
        _, o, lse, delta, ds, n = _row_stats(q, k, v, dO, scale, causal, b, h, i)
        out["o"][r], out["lse"][r], out["delta"][r] = o, lse, delta
        out["dq"][r] = scale * (ds @ np.asarray(k[b, :n, g], dtype=np.float64))
    return out


def ref_key_rows(q, k, v, dO, scale, causal, b, g, keys):
    """dk and dv of the listed key rows of (batch ``b``, KV head ``g``).

    dk_j and dv_j sum over every query row that sees key j (rows i >= j under
    the causal mask, else all rows) of every query head of the group; each such
    row's probabilities come from its own full row (:func:`_row_stats`).  The
    cost is O(rows seen * T * D), small for keys near the end of a causal
    sequence.  Returns ``(dk, dv)`` as float64 [len(keys), D].
    """
    T, Hq, Hkv, D = q.shape[1], q.shape[2], k.shape[2], q.shape[3]
    G = Hq // Hkv
    keys = list(keys)
    first = min(keys) if causal else 0
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for h in range(g * G, (g + 1) * G):
        for i in range(first, T):
            p, _, _, _, ds, n = _row_stats(q, k, v, dO, scale, causal, b, h, i)
            qi = np.asarray(q[b, i, h], dtype=np.float64)
            dOi = np.asarray(dO[b, i, h], dtype=np.float64)
            for r, j in enumerate(keys):
                if j < n:  # key j is visible to row i
                    dk[r] += scale * ds[j] * qi
                    dv[r] += p[j] * dOi
    return dk, dv
