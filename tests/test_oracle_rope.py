"""The rotary-embedding oracle against its pins, and planted mistakes that some
pin must catch (CPU only).  The oracle module is never modified on disk."""
import inspect
import textwrap
import types

import pytest

from oracle import rope as R
from oracle_rope_pins import ROPE_PINS


@pytest.mark.parametrize("name,pin", ROPE_PINS, ids=[n for n, _ in ROPE_PINS])
def test_rope_pin(name, pin):
    pin(R)


def _mutant_module(func_name, old, new):
    """A namespace like oracle.rope with one function recompiled from an edited copy;
    the public entry points are recompiled in it so they call the mutant."""
    ns = dict(vars(R))
    src = textwrap.dedent(inspect.getsource(getattr(R, func_name)))
    assert old in src, (func_name, old)
    exec(compile(src.replace(old, new, 1), f"<mutant {func_name}>", "exec"), ns)
    for name in ("apply_rope", "apply_rope_transpose", "ref_fwd_rope", "ref_bwd_rope"):
        if name != func_name:
            exec(compile(textwrap.dedent(inspect.getsource(getattr(R, name))), f"<{name}>", "exec"), ns)
    return types.SimpleNamespace(**ns)


ROPE_MUTATIONS = [
    ("sin_sign_flipped", "apply_rope", "out[..., 0::2] = a * c - b * s", "out[..., 0::2] = a * c + b * s"),
    ("pairs_swapped_roles", "apply_rope", "out[..., 1::2] = a * s + b * c", "out[..., 1::2] = b * s + a * c + 0 * a"),
    ("backward_not_transposed", "ref_bwd_rope", "return apply_rope_transpose(dq_r, cos, sin)", "return apply_rope(dq_r, cos, sin)"),
    ("dk_not_rotated_back", "ref_bwd_rope", "apply_rope_transpose(dk_r, cos, sin), dv", "dk_r, dv"),
    ("values_rotated", "ref_fwd_rope", "apply_rope(k, cos, sin), v,", "apply_rope(k, cos, sin), apply_rope(v, cos, sin),"),
    ("keys_not_rotated", "ref_fwd_rope", "apply_rope(k, cos, sin), v,", "k, v,"),
    ("half_split_pairs", "_pairs", "return x[..., 0::2], x[..., 1::2]", "return x[..., :x.shape[-1] // 2], x[..., x.shape[-1] // 2:]"),
]


@pytest.mark.parametrize("mid,func,old,new", ROPE_MUTATIONS, ids=[m[0] for m in ROPE_MUTATIONS])
def test_some_rope_pin_catches_mutation(mid, func, old, new):
    m = _mutant_module(func, old, new)
    caught = []
    for name, pin in ROPE_PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(name)
    assert caught, f"no pin catches {mid}"
