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
