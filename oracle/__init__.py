"""CPU oracle for fused causal (grouped-query) scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, helpers or constants); the only module both
sides use is the seeded input generator, which holds none of the method's
arithmetic.

``attention``  vectorised numpy fp64 implementation (materialises the score
               matrix one (batch, head) at a time), plus row-at-a-time
               entry points for sampled rows of very long sequences.
``brute``      pure-Python scalar loops with ``math.fsum``, for tiny inputs.
``rope``       rotary position embedding of q and k ahead of the attention.
"""
from .attention import (  # noqa: F401
    kv_head_of,
    ref_fwd,
    ref_bwd,
    ref_probs,
    ref_fwd_group,
    ref_bwd_group,
    ref_query_rows,
    ref_key_rows,
)
from .brute import brute_fwd, brute_bwd  # noqa: F401
from .rope import apply_rope, apply_rope_transpose, ref_fwd_rope, ref_bwd_rope  # noqa: F401
