"""Decode with more than 16 query heads per KV head (multi-query attention and other wide
groups) on the GPU, against the fp64 oracle.

The query heads of one KV head are taken 16 per wave and up to 64 per workgroup, which reads
each K/V tile once into LDS for all of them.  Covered: group sizes that leave a partial group
of 16 (17, 20, 48) or need two workgroups per KV head (128), head dims 64 and 128, one split
(o written directly) and several (merge pass), windows (with the rows outside the visible
range poisoned with NaN, which must never be read), no RoPE, empty caches, bf16 and fp32
outputs and the LSE.
"""

import numpy as np
import pytest
import torch

import oracle
from conftest import assert_bf16_parity, banner, err_stats, to_np
from transformer_self_attention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_self_attention_amd import lib as L
    return L


CASES = [
    # B, Hq, Hkv, S, D, lens, q_pos offset, n_split, window, rope, out dtype
    (2, 17, 1, 300, 128, [300, 150], 2, 0, None, True, torch.float32),
    (2, 20, 1, 333, 128, [333, 1], 0, 2, None, True, torch.bfloat16),
    (2, 48, 1, 700, 128, [700, 64], 1, 0, None, True, torch.float32),
    (2, 128, 1, 500, 128, [500, 499], 3, 0, None, True, torch.float32),
    (3, 64, 1, 1000, 64, [1000, 65, 0], 0, 0, None, True, torch.float32),
    (2, 64, 2, 2000, 128, [2000, 1500], 0, 1, None, True, torch.bfloat16),
    (2, 64, 1, 2000, 128, [2000, 1777], 5, 7, 300, True, torch.float32),
    (4, 32, 1, 1200, 128, [1200, 1100, 65, 64], 0, 0, 100, False, torch.float32),
    (2, 64, 1, 999, 64, [999, 998], -1, 3, 0, True, torch.float32),
    (2, 96, 3, 4100, 128, [4100, 4099], 0, 0, 2048, True, torch.bfloat16),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,lens,qoff,n_split,W,rope,out_dtype", CASES)
def test_decode_wide_groups(lib, B, Hq, Hkv, S, D, lens, qoff, n_split, W, rope, out_dtype):
    banner(f"wide decode B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} lens={lens} qoff={qoff} n_split={n_split} "
           f"W={W} rope={rope} out={out_dtype}")
    wl = inputs.Workload("w", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=7000 + Hq + S, kind="decode")
    lens = np.array(lens, np.int32)
    qpos = np.maximum(lens + qoff, 0).astype(np.int32)
    d = inputs.make_decode(wl, cache_len=lens, q_pos=qpos)
    kc, vc = d.k_cache.torch("cuda"), d.v_cache.torch("cuda")
    # rows no query may read: before the window and past the cache length
    nan = torch.tensor(inputs.BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).item()
    for b in range(B):
        lo = max(int(qpos[b]) - W, 0) if W is not None else 0
        kc[b, :, :lo] = nan
        vc[b, :, :lo] = nan
        kc[b, :, int(lens[b]):] = nan
        vc[b, :, int(lens[b]):] = nan
    tab = lib.make_rope_table(int(qpos.max()) + 1, D) if rope else None
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    o = lib.decode(d.q.torch("cuda"), kc, vc, torch.from_numpy(lens).cuda(), torch.from_numpy(qpos).cuda(), tab,
                   n_split=n_split, window=W, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(d.q.f64(), d.k_cache.f32, d.v_cache.f32, lens, qpos,
                                 rope_base=10000.0 if rope else None, window=W)
    got = to_np(o)
    assert np.all(np.isfinite(got))
    empty = np.isneginf(ref_lse)
    assert np.all(got[empty] == 0.0)
    assert_bf16_parity(got, ref, "o")
    got_lse = to_np(lse)
    assert np.all(np.isneginf(got_lse[empty]))
    assert err_stats(got_lse[~empty], ref_lse[~empty])[0] < 2e-2


def test_decode_wide_split_counts(lib):
    """The same multi-query step with 1 (o written directly), 2, 8 and 16 splits (merge pass)."""
    wl = inputs.Workload("w", B=4, Hq=64, Hkv=1, S=3000, D=128, dtype="bf16", seed=7100, kind="decode")
    d = inputs.make_decode(wl)
    tab = lib.make_rope_table(int(d.q_pos.max()) + 1, 128)
    args = (d.q.torch("cuda"), d.k_cache.torch("cuda"), d.v_cache.torch("cuda"),
            torch.from_numpy(d.cache_len).cuda(), torch.from_numpy(d.q_pos).cuda(), tab)
    ref, _ = oracle.decode(d.q.f64(), d.k_cache.f32, d.v_cache.f32, d.cache_len, d.q_pos)
    for ns in (1, 2, 8, 16):
        banner(f"wide decode B=4 Hq=64 Hkv=1 S=3000 n_split={ns}")
        o = lib.decode(*args, n_split=ns, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_bf16_parity(to_np(o), ref, f"o (n_split={ns})")


@pytest.mark.parametrize("B,Hq,Hkv,S,bs,lens,n_split,W", [
    (3, 64, 1, 1000, 16, [1000, 517, 0], 0, None),
    (2, 48, 2, 2050, 32, [2050, 2049], 3, None),
    (2, 64, 1, 4096, 64, [4096, 4000], 0, 700),
    (3, 20, 1, 900, 128, [900, 130, 1], 2, 64),
])
def test_decode_wide_paged(lib, B, Hq, Hkv, S, bs, lens, n_split, W):
    """The paged cache: blocks scattered over the pool; blocks wholly before every window are
    released (NaN, table entries -1 or out of range).  Equal, bit for bit, to the contiguous
    decode of the same cache."""
    banner(f"wide decode paged B={B} Hq={Hq} Hkv={Hkv} S={S} bs={bs} lens={lens} n_split={n_split} W={W}")
    wl = inputs.Workload("w", B=B, Hq=Hq, Hkv=Hkv, S=S, D=128, dtype="bf16", seed=7200 + bs + S, kind="decode")
    lens = np.array(lens, np.int32)
    pd = inputs.make_paged_decode(wl, block_size=bs, cache_len=lens, q_pos=lens)
    kp, vp, bt = pd.k_pages.bits.copy(), pd.v_pages.bits.copy(), pd.block_table.copy()
    if W is not None:
        for b in range(B):
            # only rows from the window start on are read
            first_needed = max(int(lens[b]) - W, 0) // bs
            for j in range(first_needed):
                kp[bt[b, j]] = inputs.BF16_NAN_BITS
                vp[bt[b, j]] = inputs.BF16_NAN_BITS
                bt[b, j] = -1 if j % 2 else 10 ** 8
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    tab = lib.make_rope_table(int(lens.max()) + 1, 128)
    cl = torch.from_numpy(lens).cuda()
    qp = torch.from_numpy(lens.copy()).cuda()
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    o = lib.decode_paged(pd.q.torch("cuda"), to_dev(kp), to_dev(vp), torch.from_numpy(bt).cuda(), cl, qp, tab,
                         n_split=n_split, window=W, out_dtype=torch.float32, lse=lse)
    d = pd.contiguous
    lc = torch.empty_like(lse)
    oc = lib.decode(d.q.torch("cuda"), d.k_cache.torch("cuda"), d.v_cache.torch("cuda"), cl, qp, tab,
                    n_split=n_split, window=W, out_dtype=torch.float32, lse=lc)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc), "paged and contiguous decode differ"
    ref, ref_lse = oracle.decode(pd.q.f64(), d.k_cache.f32, d.v_cache.f32, lens, lens, window=W)
    assert_bf16_parity(to_np(o), ref, "paged o")
    empty = np.isneginf(ref_lse)
    assert np.all(np.isneginf(to_np(lse)[empty]))


def test_decode_wide_groups_cache_over_2gib(lib):
    """A sequence's cache over 2 GiB (S_max > 2^23 rows at D = 128): the wide kernel's 32-bit
    offsets do not reach, so the query heads go 16 per workgroup through the narrow kernel.  Only
    the first cache_len rows hold data; the rest is never read (left as NaN)."""
    B, Hq, Hkv, D, L = 2, 32, 1, 128, 2500
    S_max = (1 << 23) + 256
    banner(f"wide groups, cache over 2 GiB: B={B} Hq={Hq} Hkv={Hkv} S_max={S_max} L={L}")
    wl = inputs.Workload("w", B=B, Hq=Hq, Hkv=Hkv, S=L, D=D, dtype="bf16", seed=7300, kind="decode")
    lens = np.array([L, L - 777], np.int32)
    d = inputs.make_decode(wl, cache_len=lens, q_pos=lens)
    nan = torch.tensor(inputs.BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).item()
    kc = torch.full((B, Hkv, S_max, D), nan, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B, Hkv, S_max, D), nan, dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        kc[b, :, :lens[b]] = d.k_cache.torch("cuda")[b, :, :lens[b]]
        vc[b, :, :lens[b]] = d.v_cache.torch("cuda")[b, :, :lens[b]]
    tab = lib.make_rope_table(L + 1, D)
    cl = torch.from_numpy(lens).cuda()
    o = lib.decode(d.q.torch("cuda"), kc, vc, cl, cl.clone(), tab, out_dtype=torch.float32)
    torch.cuda.synchronize()
    del kc, vc
    ref, _ = oracle.decode(d.q.f64(), d.k_cache.f32, d.v_cache.f32, lens, lens)
    assert_bf16_parity(to_np(o), ref, "o (cache over 2 GiB)")


def test_decode_wide_groups_pool_over_2gib(lib):
    """A paged pool over 2 GiB with the sequences' blocks at its far end (byte offsets past
    2^31): the narrow kernel again, with 64-bit addresses.  Equal to the contiguous decode."""
    B, Hq, Hkv, S, D, bs = 2, 64, 1, 1000, 128, 16
    banner(f"wide groups, pool over 2 GiB: B={B} Hq={Hq} Hkv={Hkv} S={S} bs={bs}")
    wl = inputs.Workload("w", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=7400, kind="decode")
    lens = np.array([S, 321], np.int32)
    pd = inputs.make_paged_decode(wl, block_size=bs, cache_len=lens, q_pos=lens)
    n_small = pd.k_pages.shape[0]
    n_big = (1 << 31) // (Hkv * bs * D * 2) + 4096            # 2 GiB + 16 MiB per pool
    off = n_big - n_small                                     # the used blocks at the end
    nan = torch.tensor(inputs.BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).item()
    kp = torch.full((n_big, Hkv, bs, D), nan, dtype=torch.bfloat16, device="cuda")
    vp = torch.full((n_big, Hkv, bs, D), nan, dtype=torch.bfloat16, device="cuda")
    kp[off:] = pd.k_pages.torch("cuda")
    vp[off:] = pd.v_pages.torch("cuda")
    bt = torch.from_numpy(pd.block_table + off).cuda()
    tab = lib.make_rope_table(S + 1, D)
    cl = torch.from_numpy(lens).cuda()
    o = lib.decode_paged(pd.q.torch("cuda"), kp, vp, bt, cl, cl.clone(), tab, out_dtype=torch.float32)
    torch.cuda.synchronize()
    del kp, vp
    ref, _ = oracle.decode(pd.q.f64(), pd.contiguous.k_cache.f32, pd.contiguous.v_cache.f32, lens, lens)
    assert_bf16_parity(to_np(o), ref, "paged o (pool over 2 GiB)")
