"""GPU reproducibility: bitwise-identical outputs across repeated runs, streams,
concurrent load, CU masks, batch and head slicing, and (forward, dq) sequence
prefixes.

Repeated runs of one build on one device must give identical SHA-256 over the
raw bytes of o, lse, dq, dk, dv (in that order)."""
import pytest
import torch

from gpu_support import cu_masked_stream, run_gpu, say, sha256_outputs, to_device
from reproducible_causal_attention_amd import attn as A
from reproducible_causal_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["gqa-8x4096-peaked", "gqa-4x1024", "tiny-f32", "gqa-1x512",
                                  "mha-32x1024", "gqa-4x1024-f16"])
def test_ten_runs_identical_hashes(name):
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    tensors = to_device(inp)
    say("10-run hash", name)
    hashes = [sha256_outputs(run_gpu(inp, tensors)) for _ in range(10)]
    print(name, hashes[0])
    assert len(set(hashes)) == 1, hashes


def test_same_bits_on_another_stream_and_under_load():
    w = W.WORKLOADS["gqa-4x1024"]
    inp = W.generate(w)
    tensors = to_device(inp)
    say("stream/load invariance", w.name)
    want = sha256_outputs(run_gpu(inp, tensors))
    side = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(side):
        got_side = sha256_outputs(run_gpu(inp, tensors))
    assert got_side == want
    # A long unrelated kernel on another stream competes for the compute units.
    busy = torch.cuda.Stream()
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.float32)
    with torch.cuda.stream(busy):
        for _ in range(4):
            a = a @ a.T * 1e-4
    got_load = sha256_outputs(run_gpu(inp, tensors))
    torch.cuda.synchronize()
    assert got_load == want


@pytest.mark.parametrize("name", ["gqa-4x1024", "gqa-1x512"])
@pytest.mark.parametrize("mask_kind", ["first-half-cus", "first-16-cus"])
def test_same_bits_under_cu_masks(mask_kind, name):
    """Identical bits when the stream may use only half of the CUs, or only 16 (then
    every workgroup of the co-launched backward runs a long list of units, so each
    dQ unit but the first starts on copies its predecessor issued; at 1x512 the
    forward's one-per-CU 64-row workgroups then queue several to a CU).
    (A mask enabling every other CU is refused by the runtime on MI355X.)"""
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    tensors = to_device(inp)
    say("CU-mask invariance", name, mask_kind)
    want = sha256_outputs(run_gpu(inp, tensors))
    with cu_masked_stream(mask_kind):
        got = sha256_outputs(run_gpu(inp, tensors))
    assert got == want


@pytest.mark.parametrize("shape", [(4, 700, 6, 2), (4, 700, 4, 4)],
                         ids=["gqa-split-dkdv-units", "mha-per-wave-dkdv-units"])
def test_batch_invariance(shape):
    """Element b computed alone equals slice b of the batched call, bitwise (with
    three query heads per KV head the dK/dV work is split over the eight waves of a
    unit; with one, each wave owns a pair of key blocks)."""
    B, T, Hq, Hkv = shape
    w = W.custom(B, T, Hq, Hkv, 64, "bf16", seed=21)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("batch invariance", w.label())
    full = run_gpu(inp, (q, k, v, dO))
    for b in (0, 3):
        one = run_gpu(inp, tuple(t[b:b + 1].contiguous() for t in (q, k, v, dO)))
        for name in ("o", "dq", "dk", "dv"):
            assert torch.equal(one[name][0], full[name][b]), (b, name)
        assert torch.equal(one["lse"][0], full["lse"][b]), (b, "lse")


def test_forward_forms_give_the_same_bits_on_peaked_scores():
    """The 64-wide forward takes, by the number W of 128-row query tiles, 4-wave
    workgroups of 64 rows (32-row waves, one workgroup per CU) when 2W is at most
    the CU count, 8-wave workgroups of 128 rows (32-row waves) when W is at most
    twice it, and 4-wave workgroups of 128 rows (64-row waves) beyond.  The batch
    sizes below put one input through all three forms; q is scaled so that row
    maxima keep growing along the keys and blocks take the slow path (redone per
    32-row query block in every form).  The slices must agree bitwise."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    T, Hq, Hkv = 1024, 12, 4
    per_b = (T // 128) * Hq                       # 128-row tiles per batch element
    b_one = 1                                     # 2 W <= n_cu
    b_two = max(2, n_cu // per_b + 1)             # W in (n_cu, 2 n_cu]
    b_big = 2 * n_cu // per_b + 1                 # W > 2 n_cu
    assert 2 * b_one * per_b <= n_cu < b_two * per_b <= 2 * n_cu < b_big * per_b, (n_cu, b_two, b_big)
    w = W.custom(b_big, T, Hq, Hkv, 64, "bf16", seed=31, q_std=4.0)
    inp = W.generate(w)
    q, k, v, _ = to_device(inp)
    say("forward forms", w.label(), "batches", b_one, b_two, b_big)
    o_big, lse_big = A.fwd(q, k, v, w.scale, True)
    for bs in (b_two, b_one):
        o, lse = A.fwd(*(t[:bs].contiguous() for t in (q, k, v)), w.scale, True)
        torch.cuda.synchronize()
        assert torch.equal(o, o_big[:bs]), bs
        assert torch.equal(lse, lse_big[:bs]), bs
    assert torch.isfinite(o_big.float()).all()


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_forward_forms_agree_on_a_ragged_length(causal):
    """At T = 1000 (not a multiple of the 64- or 128-row query tiles) the batch
    sizes below take the three 64-wide forward forms (64-row workgroups for one
    element, 8-wave workgroups of 128 rows for a few, 4-wave workgroups of 64-row
    waves for many); every row must come out with the same bits in each, the rows
    of the last, partial tile and the masked key blocks past each row included."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    T, Hq, Hkv = 1000, 12, 4
    per_b = -(-T // 128) * Hq                     # 128-row tiles per batch element
    b_two = max(2, n_cu // (2 * per_b) + 1)       # 2 W > n_cu, W <= 2 n_cu
    b_big = 2 * n_cu // per_b + 1                 # W > 2 n_cu
    assert 2 * per_b <= n_cu < 2 * b_two * per_b and b_two * per_b <= 2 * n_cu < b_big * per_b
    w = W.custom(b_big, T, Hq, Hkv, 64, "bf16", seed=32, q_std=2.0, causal=causal)
    inp = W.generate(w)
    q, k, v, _ = to_device(inp)
    say("forward forms, ragged", w.label(), "batches", 1, b_two, b_big)
    o_big, lse_big = A.fwd(q, k, v, w.scale, causal)
    for bs in (b_two, 1):
        o, lse = A.fwd(*(t[:bs].contiguous() for t in (q, k, v)), w.scale, causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o_big[:bs]), bs
        assert torch.equal(lse, lse_big[:bs]), bs


@pytest.mark.parametrize("D", [64, 128])
def test_forward_tile_size_does_not_change_bits(D):
    """The forward picks 128-key tiles for grids of at most 512 workgroups and
    64-key tiles above: a batch of 8 at T = 1024 (768 workgroups, 64-key
    tiles) and its elements computed alone (96 workgroups, 128-key tiles)
    give the same bits, as both visit a row's 32-key blocks in the same order."""
    w = W.custom(8, 1024, 12, 4, D, "bf16", seed=24, scale=D ** -0.5)
    inp = W.generate(w)
    q, k, v, _ = to_device(inp)
    say("tile-size invariance", w.label())
    o_full, lse_full = A.fwd(q, k, v, w.scale, True)
    for b in (0, 7):
        o_one, lse_one = A.fwd(*(t[b:b + 1].contiguous() for t in (q, k, v)), w.scale, True)
        torch.cuda.synchronize()
        assert torch.equal(o_one[0], o_full[b]), b
        assert torch.equal(lse_one[0], lse_full[b]), b


@pytest.mark.parametrize("shape", [(2, 513, 12, 4), (2, 513, 8, 8)],
                         ids=["gqa-split-dkdv-units", "mha-per-wave-dkdv-units"])
def test_kv_group_invariance(shape):
    """One KV-head group computed alone equals its slice of the call, bitwise
    (the head-parallel split of a sharded run)."""
    B, T, Hq, Hkv = shape
    w = W.custom(B, T, Hq, Hkv, 64, "bf16", seed=22)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("group invariance", w.label())
    full = run_gpu(inp, (q, k, v, dO))
    G = Hq // Hkv
    for g in (0, Hkv - 1):
        hs = slice(g * G, (g + 1) * G)
        part = run_gpu(inp, (q[:, :, hs].contiguous(), k[:, :, g:g + 1].contiguous(),
                             v[:, :, g:g + 1].contiguous(), dO[:, :, hs].contiguous()))
        assert torch.equal(part["o"], full["o"][:, :, hs])
        assert torch.equal(part["lse"], full["lse"][:, hs])
        assert torch.equal(part["dq"], full["dq"][:, :, hs])
        assert torch.equal(part["dk"][:, :, 0], full["dk"][:, :, g])
        assert torch.equal(part["dv"][:, :, 0], full["dv"][:, :, g])


@pytest.mark.parametrize("t", [300, 512, 1])
def test_prefix_invariance(t):
    """o, lse and dq of the first t rows do not depend on rows after t (causal)."""
    w = W.custom(1, 1024, 6, 2, 64, "bf16", seed=23)
    inp = W.generate(w)
    q, k, v, dO = to_device(inp)
    say("prefix invariance", t)
    full = run_gpu(inp, (q, k, v, dO))
    pre = run_gpu(inp, tuple(x[:, :t].contiguous() for x in (q, k, v, dO)))
    assert torch.equal(pre["o"], full["o"][:, :t])
    assert torch.equal(pre["lse"], full["lse"][:, :, :t])
    assert torch.equal(pre["dq"], full["dq"][:, :t])
