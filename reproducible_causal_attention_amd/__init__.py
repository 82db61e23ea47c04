"""Reproducible fused causal (grouped-query) attention for MI355X (gfx950).

The compute path is the HIP library ``libattn.so`` behind the C ABI declared
in ``include/attn.h``; :mod:`.attn` only marshals torch tensors into it and
raises if the library is missing.  :mod:`.workloads` draws seeded synthetic
inputs.
"""
