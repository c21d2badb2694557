"""Checks of the generated gfx950 code (CPU only; needs hipcc, which cross-compiles).

An `if (masked) x = -inf;` inside a fully unrolled loop once compiled, for one kernel, to a
divergent branch with nothing in it -- `s_and_saveexec_b64 sA, ...` directly followed by the
restore `s_or_b64 exec, exec, sA` -- with the masked store gone, so that kernel returned wrong
results.  The masks are now written as selects; this scan keeps any such empty branch from coming
back unnoticed in any kernel of the library.

The kernels are also held to their register budgets: no kernel spills vector registers or uses
scratch memory (the prefill kernels hold 251-255 of the 256 VGPRs a wave has at two waves per
SIMD; a spill there moves data through memory on every tile).
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


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """Assembly of every source, compiled once (in parallel) for the tests of this module."""
    from concurrent.futures import ThreadPoolExecutor
    d = tmp_path_factory.mktemp("asm")
    srcs = [s for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, str(d / (s + ".s"))), srcs))
    return dict(zip(srcs, texts))


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
def test_no_empty_divergent_branches(src, device_asm):
    hits = empty_branches(device_asm[src])
    assert not hits, f"{src}: empty if-blocks in {hits}"


def kernel_resources(asm):
    """{kernel: {field: int}} from the code object metadata of the assembly (fields after `.name`)."""
    out = {}
    names = list(re.finditer(r"^\s*\.name:\s+(_Z\S+)\s*$", asm, re.M))
    for i, m in enumerate(names):
        end = names[i + 1].start() if i + 1 < len(names) else len(asm)
        block = asm[m.end():end]
        fields = {}
        for key in ("private_segment_fixed_size", "vgpr_count", "vgpr_spill_count", "sgpr_spill_count"):
            f = re.search(r"\." + key + r":\s+(\d+)", block)
            if f:
                fields[key] = int(f.group(1))
        out[m.group(1)] = fields
    return out


def test_resource_parser_reads_a_metadata_entry():
    asm = ("  - .args: []\n    .name: _Zk1\n    .private_segment_fixed_size: 16\n    .vgpr_count: 256\n"
           "    .vgpr_spill_count: 3\n  - .args:\n      - .name: q\n    .name: _Zk2\n"
           "    .private_segment_fixed_size: 0\n    .vgpr_count: 64\n    .vgpr_spill_count: 0\n")
    r = kernel_resources(asm)
    assert r["_Zk1"] == {"private_segment_fixed_size": 16, "vgpr_count": 256, "vgpr_spill_count": 3}
    assert r["_Zk2"]["vgpr_spill_count"] == 0 and r["_Zk2"]["vgpr_count"] == 64


@pytest.mark.parametrize("src", [s for s in SOURCES if s != "attn_api.hip"])
def test_no_register_spills_or_scratch(src, device_asm):
    res = kernel_resources(device_asm[src])
    assert res, f"{src}: no kernels found in the metadata"
    bad = {k: v for k, v in res.items()
           if v.get("vgpr_spill_count", 0) != 0 or v.get("private_segment_fixed_size", 0) != 0
           or v.get("vgpr_count", 0) > 512}
    assert not bad, f"{src}: kernels spilling or using scratch: {bad}"
