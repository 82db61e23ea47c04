"""Ahead-of-time build of the libraries for gfx950 with hipcc (no JIT, no torch extension).

``python -m reproducible_causal_attention_amd.build`` or ``build()`` compiles every
HIP source directly under ``csrc/`` into ``libattn.so`` (the fused path) and the
sources under ``csrc/unfused/`` into ``libattn_unfused.so`` (the unfused
baseline, linked against rocBLAS), next to this file.  Both are always rebuilt,
so a stale binary never survives a source change.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
UNFUSED_LIB_PATH = os.path.join(PKG_DIR, "libattn_unfused.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # Packed fp32 VALU instructions are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _revision() -> str:
    try:
        rev = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                             capture_output=True, text=True, timeout=10).stdout.strip()
        dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--", "reproducible_causal_attention_amd/csrc", "include"],
                               capture_output=True, text=True, timeout=10).stdout.strip()
        return (rev or "unknown") + ("-dirty" if dirty else "")
    except (OSError, subprocess.SubprocessError):
        return "unknown"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def unfused_sources():
    return sorted(glob.glob(os.path.join(CSRC, "unfused", "*.hip")))


def _compile(srcs, out, extra, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, f'-DATTN_GIT_REV="{_revision()}"',
           f"-I{os.path.join(ROOT, 'include')}", *srcs, *extra, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = True) -> str:
    """Compile libattn.so and libattn_unfused.so; raises ``RuntimeError`` with the
    compiler output on failure.  Returns the path of libattn.so."""
    _compile(sources(), LIB_PATH, [], verbose)
    _compile(unfused_sources(), UNFUSED_LIB_PATH, ["-L/opt/rocm/lib", "-lrocblas"], verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(), file=sys.stderr)
