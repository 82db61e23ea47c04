"""The oracle against facts fixed by the mathematics (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("name,pin", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_oracle_pin(name, pin):
    pin(oracle.ref_fwd, lambda *a: oracle.ref_bwd(*a), oracle.ref_probs)


def test_group_units_equal_full_result():
    """The per-(batch, KV-group) entry points used for sampled checks of large
    workloads return exactly the slices of the full computation."""
    import numpy as np
    from oracle_pins import tiny_inputs
    B, T, Hq, Hkv, D = 2, 6, 6, 3, 4
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 3)
    o, lse = oracle.ref_fwd(q, k, v, 0.4, True)
    dq, dk, dv, delta = oracle.ref_bwd(q, k, v, dO, 0.4, True)
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            og, lg = oracle.ref_fwd_group(q, k, v, 0.4, True, b, g)
            assert np.array_equal(og, o[b, :, g * G:(g + 1) * G])
            assert np.array_equal(lg, lse[b, g * G:(g + 1) * G])
            dqg, dkg, dvg, dlg = oracle.ref_bwd_group(q, k, v, dO, 0.4, True, b, g)
            assert np.array_equal(dqg, dq[b, :, g * G:(g + 1) * G])
            assert np.array_equal(dkg, dk[b, :, g])
            assert np.array_equal(dvg, dv[b, :, g])
            assert np.array_equal(dlg, delta[b, g * G:(g + 1) * G])


@pytest.mark.parametrize("causal", [True, False])
def test_row_entry_points_equal_full_result(causal):
    """The row-at-a-time entry points used for sampled checks of long sequences
    agree with the full computation (a second, independent evaluation of the
    same definitions: one row's scores, softmax and products alone)."""
    import numpy as np
    from oracle_pins import rel_err, tiny_inputs
    B, T, Hq, Hkv, D = 2, 37, 6, 2, 8
    q, k, v, dO = tiny_inputs(B, T, Hq, Hkv, D, 5)
    scale = 0.3
    o, lse = oracle.ref_fwd(q, k, v, scale, causal)
    dq, dk, dv, delta = oracle.ref_bwd(q, k, v, dO, scale, causal)
    rows = [0, 1, 17, 31, 32, 36]
    for b in range(B):
        for h in (0, 3, 5):
            r = oracle.ref_query_rows(q, k, v, dO, scale, causal, b, h, rows)
            assert rel_err(r["o"], o[b, rows, h]) < 1e-12
            assert np.max(np.abs(r["lse"] - lse[b, h, rows])) < 1e-12
            assert np.max(np.abs(r["delta"] - delta[b, h, rows])) < 1e-12
            assert rel_err(r["dq"], dq[b, rows, h]) < 1e-12
        for g in range(Hkv):
            keys = [0, 5, 30, 35, 36] if not causal else [29, 33, 36]
            dk_r, dv_r = oracle.ref_key_rows(q, k, v, dO, scale, causal, b, g, keys)
            assert rel_err(dk_r, dk[b, keys, g]) < 1e-12
            assert rel_err(dv_r, dv[b, keys, g]) < 1e-12
