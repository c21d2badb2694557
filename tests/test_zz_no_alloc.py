"""attn_decode_noalloc (the decode whose split partials live in the library's static per-GPU
buffer) against attn_decode with a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, each equal bit for bit to
attn_decode on the same inputs (the two share their kernels) and within the bf16 bars of the fp64
oracle.  The first call splits a multi-query cache into 8 parts (8.5 MB of partials in the
buffer), the second a smaller grouped-query cache into fewer: stale partials of the first call
must not leak into the second.
"""

import numpy as np
import pytest
import torch

import oracle
from conftest import assert_bf16_parity, banner, to_np
from transformer_self_attention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from transformer_self_attention_amd import lib as _lib
    return _lib


def _case(lib, name, B, Hq, Hkv, S, seed, n_split):
    wl = inputs.Workload(name, B=B, Hq=Hq, Hkv=Hkv, S=S, D=128, dtype="bf16", seed=seed, kind="decode")
    d = inputs.make_decode(wl)
    q, kc, vc = d.q.torch("cuda"), d.k_cache.torch("cuda"), d.v_cache.torch("cuda")
    cl = torch.from_numpy(d.cache_len).cuda()
    qp = torch.from_numpy(d.q_pos).cuda()
    tab = lib.make_rope_table(int(d.q_pos.max()) + 1, 128)
    need = lib.decode_workspace_bytes(B, Hq, Hkv, S, 128, n_split)
    assert need <= lib.NOALLOC_SCRATCH_BYTES
    banner(f"decode_noalloc {name}: B={B} Hq={Hq} Hkv={Hkv} S={S} n_split={n_split} "
           f"({lib.decode_num_splits(B, Hq, Hkv, S, 128, n_split)} splits, {need} B of partials)")
    return d, (q, kc, vc, cl, qp, tab)


def _check(lib, d, args, n_split):
    q, kc, vc, cl, qp, tab = args
    lse_a = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    o_a = lib.decode_noalloc(q, kc, vc, cl, qp, tab, n_split=n_split, lse=lse_a, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_b = lib.decode(q, kc, vc, cl, qp, tab, n_split=n_split, lse=lse_b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b), "attn_decode_noalloc differs from attn_decode"
    assert torch.equal(lse_a, lse_b)
    ref, _ = oracle.decode(d.q.f64(), d.k_cache.f32, d.v_cache.f32, d.cache_len, d.q_pos)
    assert_bf16_parity(to_np(o_a), ref, "o (noalloc) vs oracle")


def test_noalloc_two_calls_second_smaller(lib):
    d1, a1 = _case(lib, "mqa", B=32, Hq=64, Hkv=1, S=8192, seed=7, n_split=0)
    d2, a2 = _case(lib, "gqa_small", B=4, Hq=16, Hkv=2, S=1000, seed=71, n_split=3)
    _check(lib, d1, a1, 0)
    _check(lib, d2, a2, 3)


def test_noalloc_rejects_partials_beyond_the_buffer(lib):
    """64 splits of the multi-query cache need 68 MB of partials: refused before any launch."""
    banner("decode_noalloc: too many partials -> ATTN_ERR_UNSUPPORTED")
    B, Hq, Hkv, S = 32, 64, 1, 8192
    assert lib.decode_workspace_bytes(B, Hq, Hkv, S, 128, 64) > lib.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, 1, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, S, 128), dtype=torch.bfloat16, device="cuda")
    cl = torch.full((B,), S, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, 1, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.AttnError) as ei:
        lib.decode_noalloc(q, kc, kc, cl, None, None, n_split=64, out=out)
    assert ei.value.status == lib.ATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call wrote its output"
