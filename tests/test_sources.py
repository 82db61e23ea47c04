"""Static checks of the sources, on the CPU: the HIP path and the oracle stay
apart, and two code patterns known to go wrong on this toolchain are absent."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "reproducible_causal_attention_amd")
CSRC = os.path.join(PKG, "csrc")


def _files(d, exts):
    for dirpath, _, names in os.walk(d):
        for n in names:
            if n.endswith(exts):
                yield os.path.join(dirpath, n)


def _strip_comments(text):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.sub(r"//[^\n]*", "", text)


def test_no_bit_cast_of_a_vector_element():
    """clang's __builtin_bit_cast applied to a vector element (v[e]) reads element
    0 whatever e is; the kernels pass such elements through bits_to_float (by
    value) instead.  This once rotated every 4-pair group of the rotary forward
    by its first pair's angle."""
    pat = re.compile(r"__builtin_bit_cast\s*\(\s*[\w:]+\s*,\s*[\w.]+(\s*\[[^\]]*\])+\s*\)")
    bad = []
    for f in _files(CSRC, (".hip", ".hpp")):
        for m in pat.finditer(_strip_comments(open(f).read())):
            bad.append((os.path.basename(f), m.group(0)))
    assert not bad, bad


def test_no_hand_written_packed_fp32():
    bad = []
    for f in _files(CSRC, (".hip", ".hpp")):
        text = _strip_comments(open(f).read())
        for op in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"):
            if op in text:
                bad.append((os.path.basename(f), op))
    assert not bad, bad


def test_package_does_not_use_the_oracle():
    """The product path never imports, links or includes anything under oracle/."""
    bad = []
    for f in _files(PKG, (".py", ".hip", ".hpp", ".h", ".cpp")):
        code = _strip_comments(open(f).read()) if not f.endswith(".py") else open(f).read()
        if f.endswith(".py"):
            code = re.sub(r'""".*?"""', "", code, flags=re.S)
            code = re.sub(r"#[^\n]*", "", code)
        if re.search(r"\boracle\b", code):
            bad.append(os.path.relpath(f, ROOT))
    assert not bad, bad
