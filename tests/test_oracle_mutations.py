"""Plant plausible mistakes in copies of the oracle (CPU only) and check that at
least one pin fails for each: evidence that the pins can tell a wrong oracle
from a right one.  The oracle module itself is never modified on disk."""
import inspect
import textwrap

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle_pins import ALL_PINS


def _mutant(func_name, old, new):
    """Compile a copy of ``oracle.attention.<func_name>`` with one textual edit."""
    src = textwrap.dedent(inspect.getsource(getattr(A, func_name)))
    assert old in src, (func_name, old)
    ns = dict(vars(A))
    exec(compile(src.replace(old, new, 1), f"<mutant {func_name}>", "exec"), ns)
    return ns




MUTATIONS = [
    # (id, function, old text, new text)
    ("mask_hides_diagonal", "_scores", "np.triu_indices(T, 1)", "np.triu_indices(T, 0)"),
    ("mask_wrong_side", "_scores", "np.triu_indices(T, 1)", "np.tril_indices(T, -1)"),
    ("scale_dropped", "_scores", "s = scale * (qh @ kh.T)", "s = (qh @ kh.T)"),
    ("log2_lse", "_softmax_lse", "m + np.log(", "m + np.log2("),
    ("max_not_subtracted_in_probs", "_softmax_lse", "np.exp(s - lse[:, None])", "np.exp(s - m[:, None])"),
    ("gqa_modulo_mapping", "kv_head_of", "return h // (Hq // Hkv)", "return h % Hkv"),
    ("delta_dropped", "ref_bwd", "ds = p * (dp - delta[b, h][:, None])", "ds = p * dp"),
    ("dq_unscaled", "ref_bwd", "dq[b, :, h] = scale * (ds @ kh)", "dq[b, :, h] = (ds @ kh)"),
    ("dk_transposed_operand", "ref_bwd", "scale * (ds.T @ qh)", "scale * (ds @ qh)"),
    ("dv_uses_ds", "ref_bwd", "p.T @ dOh", "ds.T @ dOh"),
    ("dk_overwrites_group", "ref_bwd", "dk[b, :, g] += ", "dk[b, :, g] = "),
    ("delta_from_values", "ref_bwd", "(dOh * oh).sum(axis=1)", "(dOh * vh).sum(axis=1)"),
    ("o_uses_scores", "ref_fwd", "o[b, :, h] = p @ v[b, :, g]", "o[b, :, h] = np.exp(_scores(q[b, :, h], k[b, :, g], scale, causal)) @ v[b, :, g]"),
]


@pytest.mark.parametrize("mid,func,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_some_pin_catches_mutation(mid, func, old, new):
    ns = _mutant(func, old, new)
    # Re-create the public entry points inside the mutated namespace, except the
    # one that was mutated itself, so they call the mutated helper.
    for name in ("ref_fwd", "ref_bwd", "ref_probs"):
        if name != func:
            exec(compile(textwrap.dedent(inspect.getsource(getattr(A, name))), "<rebound>", "exec"), ns)
    fwd, bwd, probs = ns["ref_fwd"], ns["ref_bwd"], ns["ref_probs"]
    failed = []
    with np.errstate(all="ignore"):
        for name, pin in ALL_PINS:
            if name == "finite_differences" and failed:
                continue  # already caught; skip the slowest pin
            try:
                pin(fwd, bwd, probs)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                failed.append(name)
    assert failed, f"no pin catches mutation {mid}"
