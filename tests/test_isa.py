"""Checks of the gfx950 assembly the kernels compile to (CPU only: hipcc emits the
device assembly without a GPU).

* No packed fp32 VALU instructions: the build turns the feature off, and this
  confirms that the compiler honoured it for every kernel.
* No scalar-cache writes: every store goes through the vector memory path.
* m0 is written only inside the kernels' own load-to-LDS asm blocks, each write
  immediately followed by its load, and no compiler-generated instruction reads or
  writes m0.  hipcc warns that an asm clobber of m0 may not be preserved; this
  shows there is no compiler-held value in m0 for those blocks to overwrite.
* No scratch memory in the 16-bit (MFMA) kernels: a register spill there would
  be a silent slowdown of the hot path.  The fp32 VALU forward, used for small
  fp32 problems only, is exempt.
"""
import concurrent.futures
import os
import re
import subprocess
import tempfile

import pytest

from reproducible_causal_attention_amd import build

CSRC = build.CSRC
SOURCES = build.sources() + build.unfused_sources()


def _assemble(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in build.HIP_FLAGS if f != "-shared"]
    cmd = [build.HIPCC, *flags, f"-I{os.path.join(build.ROOT, 'include')}",
           "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (src, r.stderr[-2000:])
    return src, open(out).read()


@pytest.fixture(scope="module")
def assembly():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            return dict(ex.map(lambda s: _assemble(s, d), SOURCES))


def _code_lines(text):
    """(line, inside_inline_asm) for every instruction line, comments dropped."""
    inside = False
    for raw in text.splitlines():
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
            continue
        if s.startswith(";;#ASMEND"):
            inside = False
            continue
        s = s.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        yield s, inside


def test_every_source_is_checked():
    names = {os.path.basename(s) for s in SOURCES}
    assert {"fwd64.hip", "bwd_dkdv_dq.hip", "bwd_dq.hip", "bwd_dkdv.hip", "bwd_pre.hip"} <= names


def test_no_packed_fp32(assembly):
    pat = re.compile(r"^v_pk_(fma|mul|add)_f32\b")
    bad = [(os.path.basename(f), s) for f, t in assembly.items() for s, _ in _code_lines(t) if pat.match(s)]
    assert not bad, bad[:10]


def test_no_scalar_cache_writes(assembly):
    pat = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")
    bad = [(os.path.basename(f), s) for f, t in assembly.items() for s, _ in _code_lines(t) if pat.match(s)]
    assert not bad, bad[:10]


def test_m0_only_in_the_load_to_lds_blocks(assembly):
    m0 = re.compile(r"\bm0\b")
    n_blocks = 0
    for f, text in assembly.items():
        lines = list(_code_lines(text))
        for i, (s, inside) in enumerate(lines):
            if not m0.search(s):
                continue
            assert inside, (os.path.basename(f), s)
            assert s.startswith("s_mov_b32 m0,"), (os.path.basename(f), s)
            # the block's next instructions: optional s_nop, then the load into LDS
            rest = [x for x, _ in lines[i + 1:i + 3] if not x.startswith("s_nop")]
            assert rest and rest[0].startswith("buffer_load_") and rest[0].endswith(" lds"), \
                (os.path.basename(f), s, rest[:1])
            n_blocks += 1
    assert n_blocks > 0  # the forward and the backward bodies use load-to-LDS copies


def test_no_scratch_in_16_bit_kernels(assembly):
    bad = []
    for f, text in assembly.items():
        kernel = None
        for raw in text.splitlines():
            s = raw.strip()
            if s.startswith(".amdhsa_kernel "):
                kernel = s.split()[1]
            m = re.match(r"\.amdhsa_private_segment_fixed_size (\d+)", s)
            if m and int(m.group(1)) != 0 and "f32_kernel" not in kernel:
                bad.append((os.path.basename(f), kernel, int(m.group(1))))
    assert not bad, bad
