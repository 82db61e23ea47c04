"""Seeded synthetic attention inputs, shared by the tests, the bench and the oracle.

This module holds none of the attention arithmetic: it draws i.i.d. normal
numbers, rounds them to the storage dtype and widens stored values for the
oracle.  Nothing here imports the oracle or the HIP library.

Workloads
---------
The pages train on synthetic token IDs because throughput does not depend on
the content ("Training a 100M transformer in pure Rust: RustingBrain vs
PyTorch and TensorFlow", section "The setup"), and measure no attention on a
public dataset.  The attention inputs here are therefore i.i.d. normal values
at the pages' shapes:

* ``gqa-4x1024``  -- one attention layer of that page's 101.7M decoder
  (d_model 768, 12 query heads, 4 KV heads, head_dim 64) at its 4 x 1024
  batch shape (section "Limitations" quotes the 4 x 1024 runs);
* ``gqa-1x512``   -- the same layer at the page's 1 x 512 shape (section
  "The result");
* ``mha-32x1024`` -- the profile configuration of "rust-trainer", section
  "Full-step profiling" (B=32, T=1024, 24 heads of 64);
* ``tiny-f32``    -- a tiny fp32 multi-head case the oracle finishes at once;
* ``gqa-8x4096-peaked`` -- a long-sequence stress case whose queries are
  drawn with standard deviation 3 so that the softmax is peaked;
* ``gqa-1x512-f16``, ``gqa-4x1024-f16`` -- the same shapes with float16 storage
  (the adjacent input type: the same dense peak as bf16);
* ``gqa-4x1024-noncausal`` -- the headline shape without the causal mask;
* ``gqa-4x1024-d128`` -- the headline shape with 128-wide heads (scale 1/sqrt(128)).

Generation recipe: ``numpy.random.Generator(PCG64(seed))``; ``standard_normal``
in float64 (in float32 for workloads marked ``draw_f32``, a faster draw used
for test shapes of half a billion elements) drawn in the order Q, K, V, dO,
each in C order of its [B, T, H, D] shape; Q multiplied by ``q_std``; cast to float32; for bf16
workloads rounded to bfloat16 with round-to-nearest-even (float16 workloads:
numpy's float32 -> float16 conversion, also round-to-nearest-even).  The oracle
sees the stored values widened exactly to float64.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "f32", "bf16" or "f16"
    seed: int
    q_std: float = 1.0
    scale: float = 0.125
    causal: bool = True
    description: str = ""
    draw_f32: bool = False  # draw in float32 (faster; used by the largest test shapes)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def causal_pairs(self) -> int:
        """Unmasked (query, key) pairs summed over batch and query heads."""
        per_head = self.T * (self.T + 1) // 2 if self.causal else self.T * self.T
        return self.B * self.Hq * per_head

    @property
    def fwd_flops(self) -> float:
        """Algorithmic forward flops: 4*D per unmasked pair (QK^T and PV)."""
        return 4.0 * self.D * self.causal_pairs

    @property
    def bwd_flops(self) -> float:
        """Algorithmic backward flops: 10*D per unmasked pair (S, dP, dV, dK, dQ)."""
        return 10.0 * self.D * self.causal_pairs

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def label(self) -> str:
        return (f"B{self.B}_T{self.T}_Hq{self.Hq}_Hkv{self.Hkv}_D{self.D}_{self.dtype}"
                f"{'_causal' if self.causal else '_full'}")


WORKLOADS = {
    "tiny-f32": Workload("tiny-f32", 1, 128, 2, 2, 64, "f32", seed=1,
                         description="tiny fp32 causal multi-head"),
    "gqa-1x512": Workload("gqa-1x512", 1, 512, 12, 4, 64, "bf16", seed=2,
                          description="bf16 causal GQA 12/4, 1 x 512"),
    "gqa-4x1024": Workload("gqa-4x1024", 4, 1024, 12, 4, 64, "bf16", seed=3,
                           description="bf16 causal GQA 12/4, 4 x 1024 (one decoder layer)"),
    "mha-32x1024": Workload("mha-32x1024", 32, 1024, 24, 24, 64, "bf16", seed=4,
                            description="bf16 causal MHA 24 heads, 32 x 1024"),
    "gqa-8x4096-peaked": Workload("gqa-8x4096-peaked", 8, 4096, 12, 4, 64, "bf16", seed=5,
                                  q_std=3.0,
                                  description="bf16 causal GQA 12/4, 8 x 4096, Q ~ N(0, 9)"),
    "gqa-1x512-f16": Workload("gqa-1x512-f16", 1, 512, 12, 4, 64, "f16", seed=6,
                              description="fp16 causal GQA 12/4, 1 x 512"),
    "gqa-4x1024-f16": Workload("gqa-4x1024-f16", 4, 1024, 12, 4, 64, "f16", seed=3,
                               description="fp16 causal GQA 12/4, 4 x 1024"),
    "gqa-4x1024-noncausal": Workload("gqa-4x1024-noncausal", 4, 1024, 12, 4, 64, "bf16", seed=3,
                                     causal=False,
                                     description="bf16 GQA 12/4, 4 x 1024, no causal mask"),
    "gqa-4x1024-d128": Workload("gqa-4x1024-d128", 4, 1024, 12, 4, 128, "bf16", seed=3,
                                scale=128 ** -0.5,
                                description="bf16 causal GQA 12/4, 4 x 1024, head dim 128"),
}


def custom(B, T, Hq, Hkv, D=64, dtype="bf16", seed=0, q_std=1.0, scale=0.125,
           causal=True, name="custom", draw_f32=False) -> Workload:
    return Workload(name, B, T, Hq, Hkv, D, dtype, seed, q_std, scale, causal,
                    draw_f32=draw_f32)


def rope_tables(T: int, D: int, base: float = 10000.0):
    """Caller-side rotary tables: cos and sin of t * base^(-2i/D) for positions
    t < T and pairs i < D/2, computed in float64 and stored as float32 [T, D/2]
    (the form the kernels and the oracle both take as an input)."""
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(T, dtype=np.float64)[:, None] * np.power(base, -2.0 * i / D)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# --------------------------------------------------------------------------
# bfloat16 storage helpers (storage format only, not attention arithmetic)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  Inputs here are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Stored inputs of one workload.

    For ``bf16`` and ``f16`` workloads the arrays are ``uint16`` bit patterns;
    for ``f32`` they are ``float32``.  Shapes: q, dO [B,T,Hq,D]; k, v [B,T,Hkv,D].
    """
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dO: np.ndarray

    def as_float64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.workload.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        if self.workload.dtype == "f16":
            return a.view(np.float16).astype(np.float64)
        return a.astype(np.float64)


def generate(w: Workload) -> Inputs:
    """Draw the seeded inputs of workload ``w`` (recipe in the module docstring)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    qshape = (w.B, w.T, w.Hq, w.D)
    kshape = (w.B, w.T, w.Hkv, w.D)
    out = {}
    for name, shape in (("q", qshape), ("k", kshape), ("v", kshape), ("dO", qshape)):
        a = rng.standard_normal(shape, dtype=np.float32 if w.draw_f32 else np.float64)
        if name == "q" and w.q_std != 1.0:
            a *= w.q_std
        a = a.astype(np.float32)
        if w.dtype == "bf16":
            out[name] = f32_to_bf16_bits(a)
        elif w.dtype == "f16":
            out[name] = a.astype(np.float16).view(np.uint16)
        else:
            out[name] = a
    return Inputs(w, **out)
