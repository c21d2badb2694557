import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# With ATTN_CHECKED_RUN=1 (tests/test_gpu_checked.py sets it, with ATTN_LIBRARY pointing at the
# index-checked build), every GPU test ends by reading the words of failed index checks: any set
# bit fails the test.
import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _checked_build_sites(request):
    yield
    if os.environ.get("ATTN_CHECKED_RUN") != "1" or request.node.get_closest_marker("gpu") is None:
        return
    import torch
    from transformer_self_attention_amd import lib
    torch.cuda.synchronize()
    words = lib.checked_sites()
    assert words is not None, "ATTN_CHECKED_RUN=1 but the loaded library is not the checked build"
    files = ("rope", "cache", "prefill_bf16", "prefill_f32", "decode", "decode_wide")
    failed = {f: [i for i in range(32) if w >> i & 1] for f, w in zip(files, words) if w}
    assert not failed, f"failed index checks (file: sites): {failed}"


# ---- helpers shared by the GPU tests -------------------------------------------------------
import numpy as np  # noqa: E402

BF16_MAX_ABS = 2e-2     # parity bars for bf16 inputs (max and mean absolute error vs fp64 oracle)
BF16_MEAN_ABS = 1e-3
F32_MAX_ABS = 1e-5      # parity bar for fp32 inputs


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def to_np(t):
    import torch
    return t.detach().to("cpu", dtype=torch.float64).numpy()


def err_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    e = np.abs(got - ref)
    return float(e.max()), float(e.mean())


def assert_bf16_parity(got, ref, what=""):
    mx, mean = err_stats(got, ref)
    print(f"    {what} max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= BF16_MAX_ABS, f"{what}: max abs error {mx} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean abs error {mean} > {BF16_MEAN_ABS}"


def assert_f32_parity(got, ref, what="", tol=F32_MAX_ABS):
    mx, mean = err_stats(got, ref)
    print(f"    {what} max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= tol, f"{what}: max abs error {mx} > {tol}"
