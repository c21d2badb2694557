"""The C ABI's host code (argument validation, size queries, dispatch up to the first launch)
under AddressSanitizer and UBSan: tests/test_abi.py runs in a child process against a build of
libattn.so whose attn_api.hip host code is instrumented (build.build_host_sanitized), with the
ASan runtime preloaded.  Any report fails the test.  No GPU is used: the ABI tests launch
nothing."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_under_asan_and_ubsan(tmp_path):
    from transformer_self_attention_amd import build
    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env.update(ATTN_LIBRARY=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={tmp_path}/ubsan")
    res = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = {p.name: p.read_text() for p in tmp_path.iterdir()}
    detail = res.stdout[-4000:] + res.stderr[-2000:] + "".join(r[:3000] for r in reports.values())
    assert res.returncode == 0, detail
    assert not reports, detail
    assert " passed" in res.stdout
