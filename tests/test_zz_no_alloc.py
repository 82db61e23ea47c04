"""attn_bwd_noalloc (delta in the library's per-GPU scratch array) against attn_bwd
(delta in a caller workspace), through the C ABI: bitwise-equal dq, dk, dv on two
calls in a row, the second on a smaller problem, then at the scratch array's
largest size, and the oracle's tolerance on the small problem.  A call beyond the
array's size is refused before anything is launched."""
import pytest
import torch

from gpu_support import as_numpy, check_against, oracle_full, say, to_device
from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _both(q, k, v, dO, scale, causal):
    o, lse = A.fwd(q, k, v, scale, causal)
    want = A.bwd(q, k, v, o, lse, dO, scale, causal)
    got = A.bwd_noalloc(q, k, v, o, lse, dO, scale, causal)
    torch.cuda.synchronize()
    return o, lse, want, got


def test_noalloc_equals_bwd_on_two_calls_larger_then_smaller():
    w1 = W.WORKLOADS["gqa-4x1024"]
    w2 = W.custom(1, 300, 6, 2, 64, "bf16", seed=71)
    for w in (w1, w2):
        inp = W.generate(w)
        say("noalloc vs attn_bwd", w.label())
        q, k, v, dO = to_device(inp)
        o, lse, want, got = _both(q, k, v, dO, w.scale, w.causal)
        for name, a, b in zip(("dq", "dk", "dv"), want, got):
            assert torch.equal(a, b), (w.name, name)
        if w is w2:  # the oracle's bar on the smaller problem
            delta = A.bwd_preprocess(o, dO)
            torch.cuda.synchronize()
            gpu = {"o": o, "lse": lse, "delta": delta, "dq": got[0], "dk": got[1], "dv": got[2]}
            check_against(as_numpy(gpu), oracle_full(inp), "bf16", w.label())


def test_noalloc_at_the_scratch_limit_and_beyond():
    """B * Hq * T = 4,194,304 rows fill the 16 MiB array exactly; one more query head
    group is refused."""
    B, T, Hq, Hkv, D = 8, 4096, 128, 16, 64
    assert B * Hq * T * 4 == A.NOALLOC_SCRATCH_BYTES
    g = torch.Generator(device="cuda").manual_seed(5)
    mk = lambda h: torch.randn(B, T, h, D, device="cuda", generator=g).to(torch.bfloat16)
    q, k, v, dO = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    say("noalloc at the limit", (B, T, Hq, Hkv, D))
    _, _, want, got = _both(q, k, v, dO, 0.125, True)
    for name, a, b in zip(("dq", "dk", "dv"), want, got):
        assert torch.equal(a, b), name
    del q, k, v, dO, want, got
    q, k, v, dO = mk(Hq + 8), mk(Hkv + 1), mk(Hkv + 1), mk(Hq + 8)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq + 8, T, device="cuda")
    with pytest.raises(A.AttnError) as e:
        A.bwd_noalloc(q, k, v, o, lse, dO, 0.125, True)
    assert e.value.status == A.ATTN_ERR_INVALID_ARG


def test_noalloc_in_a_sequence_of_differently_sized_calls():
    """The array keeps the last call's contents: calls of different sizes, each checked
    bitwise against attn_bwd on its own workspace."""
    for i, (B, T, Hq, Hkv) in enumerate([(2, 700, 6, 2), (1, 65, 12, 4), (3, 129, 4, 4)]):
        w = W.custom(B, T, Hq, Hkv, 64, "bf16", seed=80 + i)
        q, k, v, dO = to_device(W.generate(w))
        say("noalloc sequence", w.label())
        _, _, want, got = _both(q, k, v, dO, w.scale, True)
        for name, a, b in zip(("dq", "dk", "dv"), want, got):
            assert torch.equal(a, b), (w.label(), name)
