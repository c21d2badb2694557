"""Checks of the generated gfx950 code (CPU only; needs hipcc, which cross-compiles).

An `if (masked) x = -inf;` inside a fully unrolled loop once compiled, for one kernel, to a
divergent branch with nothing in it -- `s_and_saveexec_b64 sA, ...` directly followed by the
restore `s_or_b64 exec, exec, sA` -- with the masked store gone, so that kernel returned wrong
results.  The masks are now written as selects; this scan keeps any such empty branch from coming
back unnoticed in any kernel of the library.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_self_attention_amd", "csrc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _device_asm(src, out):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
                    os.path.join(CSRC, src), "-o", out], check=True, capture_output=True)
    return open(out).read()


def empty_branches(asm):
    """(function, count) of if-blocks whose body is empty: saveexec straight into the exec restore."""
    func, prev, hits = None, None, {}
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            func, prev = m.group(1), None
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")):
            continue
        m2 = re.match(r"s_or_b64 exec, exec, (s\[\d+:\d+\])", t)
        if m2 and prev is not None:
            m1 = re.match(r"s_and_saveexec_b64 (s\[\d+:\d+\]),", prev)
            if m1 and m1.group(1) == m2.group(1):
                hits[func] = hits.get(func, 0) + 1
        prev = t
    return hits


def test_scanner_finds_an_empty_branch():
    asm = "_Zfoo:\n\ts_and_saveexec_b64 s[8:9], s[6:7]\n\ts_or_b64 exec, exec, s[8:9]\n\ts_endpgm\n"
    assert empty_branches(asm) == {"_Zfoo": 1}
    asm_ok = "_Zfoo:\n\ts_and_saveexec_b64 s[8:9], s[6:7]\n\tv_mov_b32 v2, s14\n\ts_or_b64 exec, exec, s[8:9]\n"
    assert empty_branches(asm_ok) == {}


@pytest.mark.parametrize("src", SOURCES)
def test_no_empty_divergent_branches(src, tmp_path):
    hits = empty_branches(_device_asm(src, str(tmp_path / (src + ".s"))))
    assert not hits, f"{src}: empty if-blocks in {hits}"
