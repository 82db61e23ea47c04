"""A whole step (forward, then backward) captured in a HIP graph through torch and
replayed: every replay gives the bits of the eager step.  The library records no
memset and allocates nothing, so the captured nodes are its kernels (the
co-launched backward sizes its grid from the device's CU count at capture
time).  Replays are separated by unrelated eager work and synchronizations."""
import pytest
import torch

from gpu_support import run_gpu, say, to_device
from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(4, 1024, 12, 4, 64), (3, 333, 6, 2, 64), (1, 300, 8, 2, 128)],
                         ids=["gqa-4x1024", "ragged-3x333", "d128-1x300"])
def test_step_graph_replays_match_eager(shape):
    B, T, Hq, Hkv, D = shape
    w = W.custom(B, T, Hq, Hkv, D, "bf16", seed=90 + T, scale=D ** -0.5)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("graph replay", w.label())
    eager = run_gpu(inp, (q, k, v, dO))

    side = torch.cuda.Stream()  # default priority; warm up off the capture stream
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            o, lse = A.fwd(q, k, v, w.scale, w.causal)
            A.bwd(q, k, v, o, lse, dO, w.scale, w.causal)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o, lse = A.fwd(q, k, v, w.scale, w.causal)
        dq, dk, dv = A.bwd(q, k, v, o, lse, dO, w.scale, w.causal)
    for r in range(3):
        x = torch.randn(512, 512, device=q.device)
        (x @ x).sum().item()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            assert torch.equal(t, eager[name]), (r, name)
    del graph
    torch.cuda.synchronize()
