"""Chunked prefill with a chunk start per sequence (attn_prefill_chunk_varpos).

What is checked, on seeded inputs (inputs.make_chunk draws the chunk and the whole cache):
  * with every start equal to p, the call gives attn_prefill_chunk's result with pos0 = p bit
    for bit (output, LSE, both caches), with a larger pos0_max so that the fp16 key copy is laid
    out differently;
  * ragged starts: each sequence against the fp64 oracle run on that sequence alone
    (oracle.append_to_cache, oracle.attention_with_cache at its own start) at the bf16 bars; the
    cache rows outside each sequence's chunk are untouched, bit for bit, and the appended rows
    match the oracle's bf16-rounded rotation;
  * starts outside [0, pos0_max]: those sequences get NaN output rows and LSE and keep their
    cache bit for bit, while the other sequences of the batch still match the oracle;
  * into a shuffled block pool (attn_prefill_chunk_paged_varpos): the same outputs as the
    contiguous call bit for bit and the same cache contents in table order, each valid sequence
    against the oracle; with equal starts, attn_prefill_chunk_paged's result bit for bit.
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


def _chunk(B, Hq, Hkv, Sq, S_max, D, seed):
    wl = inputs.Workload("v", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=seed, kind="chunk",
                         pos0=0, S_max=S_max)
    return inputs.make_chunk(wl)


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


def _varpos(lib, c, starts, pos0_max, *, rope=True, window=None, out_dtype=torch.bfloat16):
    wl = c.wl
    tab = lib.make_rope_table(wl.S_max, wl.D) if rope else None
    kc, vc = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    p0 = torch.tensor(starts, dtype=torch.int32, device="cuda")
    lse = torch.empty((wl.B, wl.Hq, wl.S), dtype=torch.float32, device="cuda")
    o = lib.prefill_chunk_varpos(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"), kc, vc, p0,
                                 pos0_max, tab, window=window, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    return o, lse, kc, vc


@pytest.mark.parametrize("B,Hq,Hkv,Sq,S_max,D,p,pos0_max,rope,window", [
    (2, 8, 2, 77, 300, 128, 100, 150, True, None),
    (1, 4, 4, 130, 260, 64, 70, 100, True, 40),
    (2, 8, 2, 150, 400, 128, 37, 200, False, None),
    (2, 16, 2, 200, 500, 128, 0, 300, True, None),
])
def test_equal_starts_match_prefill_chunk(lib, B, Hq, Hkv, Sq, S_max, D, p, pos0_max, rope, window):
    banner(f"prefill_chunk_varpos == prefill_chunk: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} D={D} p={p} "
           f"pos0_max={pos0_max} rope={rope} window={window}")
    c = _chunk(B, Hq, Hkv, Sq, S_max, D, seed=Sq + p)
    for out_dtype in (torch.bfloat16, torch.float32):
        o, lse, kc, vc = _varpos(lib, c, [p] * B, pos0_max, rope=rope, window=window, out_dtype=out_dtype)
        tab = lib.make_rope_table(S_max, D) if rope else None
        kc2, vc2 = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
        lse2 = torch.empty_like(lse)
        o2 = lib.prefill_chunk(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"), kc2, vc2, p, tab,
                               window=window, out_dtype=out_dtype, lse=lse2)
        torch.cuda.synchronize()
        assert torch.equal(o, o2), f"output differs ({out_dtype})"
        assert torch.equal(lse, lse2), f"LSE differs ({out_dtype})"
        assert torch.equal(kc, kc2) and torch.equal(vc, vc2), f"caches differ ({out_dtype})"


def _check_sequence(c, b, p, got_o, got_lse, got_k, got_v, *, rope, window, what):
    """Sequence b against the oracle run on it alone, chunk at p."""
    Sq = c.wl.S
    base = 10000.0 if rope else None
    sl = slice(b, b + 1)
    kc0, vc0 = c.k_cache.f64()[sl], c.v_cache.f64()[sl]
    ref_k, ref_v = oracle.append_to_cache(kc0, vc0, c.k_new.f64()[sl], c.v_new.f64()[sl], p, rope_base=base)
    ref, ref_lse = oracle.attention_with_cache(c.q.f64()[sl], ref_k, ref_v, p, rope_base=base, window=window)
    # cache: rows outside the chunk untouched; values copied; keys the oracle's bf16 rounding
    # (the GPU rotates in fp32 first: one rounding step apart at most)
    S_max = kc0.shape[2]
    outside = np.r_[0:p, p + Sq:S_max]
    gk, gv = _bits(got_k)[sl], _bits(got_v)[sl]
    bk, bv = c.k_cache.bits.view(np.int16)[sl], c.v_cache.bits.view(np.int16)[sl]
    assert np.array_equal(gk[:, :, outside], bk[:, :, outside]), f"{what}: K rows outside the chunk changed"
    assert np.array_equal(gv[:, :, outside], bv[:, :, outside]), f"{what}: V rows outside the chunk changed"
    assert np.array_equal(gv[:, :, p:p + Sq], c.v_new.bits.view(np.int16)[sl]), f"{what}: V rows not copied"
    kn = to_np(got_k)[sl][:, :, p:p + Sq]
    exact = oracle.rope(c.k_new.f64()[sl], p + np.arange(Sq)) if rope else c.k_new.f64()[sl]
    assert np.all(np.abs(kn - exact) <= np.abs(exact) * 2.0 ** -8 + 2e-6), f"{what}: appended keys"
    assert_bf16_parity(to_np(got_o)[sl], ref, f"{what} o")
    assert err_stats(to_np(got_lse)[sl], ref_lse)[0] < 2e-2, f"{what} lse"


@pytest.mark.parametrize("B,Hq,Hkv,Sq,S_max,D,starts,pos0_max,rope,window", [
    (4, 8, 2, 70, 420, 128, [0, 37, 200, 350], 350, True, None),    # ragged, one at the bound
    (3, 4, 4, 129, 400, 64, [5, 271, 64], 271, True, 90),            # D = 64, window, tile crossings
    (3, 8, 1, 1, 300, 128, [0, 150, 299], 299, True, None),          # one new token each (MQA)
    (2, 8, 2, 64, 256, 128, [64, 0], 192, False, None),              # no RoPE, below the bound
    (2, 16, 2, 300, 1000, 128, [513, 17], 700, True, None),          # several query blocks
])
def test_ragged_starts_against_oracle(lib, B, Hq, Hkv, Sq, S_max, D, starts, pos0_max, rope, window):
    banner(f"prefill_chunk_varpos B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} D={D} starts={starts} pos0_max={pos0_max} "
           f"rope={rope} window={window}")
    c = _chunk(B, Hq, Hkv, Sq, S_max, D, seed=7 * Sq + sum(starts))
    o, lse, kc, vc = _varpos(lib, c, starts, pos0_max, rope=rope, window=window)
    for b, p in enumerate(starts):
        _check_sequence(c, b, p, o, lse, kc, vc, rope=rope, window=window, what=f"seq {b} (start {p})")


def test_starts_out_of_range(lib):
    """Sequences 1 and 2 have starts outside [0, pos0_max]: NaN rows and LSE, caches untouched;
    sequences 0 and 3 are still exact."""
    B, Hq, Hkv, Sq, S_max, D, pos0_max = 4, 8, 2, 50, 200, 128, 150
    starts = [10, -1, pos0_max + 1, 100]
    banner(f"prefill_chunk_varpos with starts {starts}, pos0_max={pos0_max}")
    c = _chunk(B, Hq, Hkv, Sq, S_max, D, seed=99)
    for out_dtype in (torch.bfloat16, torch.float32):
        o, lse, kc, vc = _varpos(lib, c, starts, pos0_max, out_dtype=out_dtype)
        for b in (1, 2):
            assert torch.isnan(o[b].float()).all(), f"seq {b}: output not NaN ({out_dtype})"
            assert torch.isnan(lse[b]).all(), f"seq {b}: LSE not NaN"
            assert np.array_equal(_bits(kc)[b], c.k_cache.bits.view(np.int16)[b]), f"seq {b}: K cache changed"
            assert np.array_equal(_bits(vc)[b], c.v_cache.bits.view(np.int16)[b]), f"seq {b}: V cache changed"
        for b in (0, 3):
            _check_sequence(c, b, starts[b], o, lse, kc, vc, rope=True, window=None,
                            what=f"seq {b} (start {starts[b]}, {out_dtype})")


def _gather_bits(pool_bits, table, bs, S):
    """Contiguous [B, Hkv, S, D] view of a pool's slots in table order."""
    B, nb = table.shape
    blocks = pool_bits[table.ravel()]                      # [B*nb, Hkv, bs, D]
    Hkv, D = blocks.shape[1], blocks.shape[3]
    seq = blocks.reshape(B, nb, Hkv, bs, D).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, nb * bs, D)
    return seq[:, :, :S]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,S_max,D,bs,starts,pos0_max,window,rope", [
    (4, 8, 2, 70, 420, 128, 16, [0, 37, 200, 350], 350, None, True),
    (3, 4, 4, 129, 400, 64, 32, [5, 271, 64], 271, 90, True),
    (2, 8, 2, 64, 256, 128, 16, [64, 0], 192, None, False),
    (4, 8, 2, 50, 200, 128, 16, [10, -1, 151, 100], 150, None, True),    # two starts out of range
])
def test_paged_varpos_equals_contiguous_varpos(lib, B, Hq, Hkv, Sq, S_max, D, bs, starts, pos0_max, window, rope):
    """The same ragged chunk into a shuffled block pool (attn_prefill_chunk_paged_varpos) and into the
    contiguous cache (attn_prefill_chunk_varpos): outputs and LSE equal bit for bit (NaN rows
    included), and the pool's slots, read in table order, equal the contiguous cache."""
    banner(f"paged varpos == contiguous varpos: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} D={D} bs={bs} starts={starts} "
           f"pos0_max={pos0_max} window={window} rope={rope}")
    wl = inputs.Workload("v", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=11 * Sq + bs, kind="chunk",
                         pos0=0, S_max=S_max)
    pc = inputs.make_paged_chunk(wl, block_size=bs)
    c = pc.chunk
    o, lse, kc, vc = _varpos(lib, c, starts, pos0_max, rope=rope, window=window, out_dtype=torch.float32)
    tab = lib.make_rope_table(S_max, D) if rope else None
    kp, vp = pc.k_pages.torch("cuda"), pc.v_pages.torch("cuda")
    bt = torch.from_numpy(pc.block_table).cuda()
    p0 = torch.tensor(starts, dtype=torch.int32, device="cuda")
    lp = torch.empty_like(lse)
    op = lib.prefill_chunk_paged_varpos(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"), kp, vp, bt,
                                        p0, pos0_max, tab, window=window, out_dtype=torch.float32, lse=lp)
    torch.cuda.synchronize()
    same_o = torch.equal(torch.nan_to_num(op, nan=7.0), torch.nan_to_num(o, nan=7.0))
    same_l = torch.equal(torch.nan_to_num(lp, nan=7.0), torch.nan_to_num(lse, nan=7.0))
    assert same_o and torch.equal(torch.isnan(op), torch.isnan(o)), "paged and contiguous outputs differ"
    assert same_l and torch.equal(torch.isnan(lp), torch.isnan(lse)), "paged and contiguous LSE differ"
    gk = _gather_bits(kp.cpu().view(torch.int16).numpy(), pc.block_table, bs, S_max)
    gv = _gather_bits(vp.cpu().view(torch.int16).numpy(), pc.block_table, bs, S_max)
    assert np.array_equal(gk, _bits(kc)), "pool keys differ from the contiguous cache"
    assert np.array_equal(gv, _bits(vc)), "pool values differ from the contiguous cache"
    for b, p in enumerate(starts):
        if 0 <= p <= pos0_max:
            _check_sequence(c, b, p, op, lp, kc, vc, rope=rope, window=window, what=f"paged seq {b} (start {p})")
        else:
            assert torch.isnan(op[b]).all() and torch.isnan(lp[b]).all(), f"seq {b}: not NaN"


def test_paged_varpos_equal_starts_match_paged_chunk(lib):
    B, Hq, Hkv, Sq, S_max, D, bs, p, pos0_max = 2, 8, 2, 77, 300, 128, 16, 100, 150
    banner(f"paged varpos == paged chunk at equal starts p={p} (pos0_max={pos0_max})")
    wl = inputs.Workload("v", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=123, kind="chunk", pos0=0,
                         S_max=S_max)
    pc = inputs.make_paged_chunk(wl, block_size=bs)
    c = pc.chunk
    tab = lib.make_rope_table(S_max, D)
    bt = torch.from_numpy(pc.block_table).cuda()
    q, kn, vn = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    kp1, vp1 = pc.k_pages.torch("cuda"), pc.v_pages.torch("cuda")
    kp2, vp2 = pc.k_pages.torch("cuda"), pc.v_pages.torch("cuda")
    l1 = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    o1 = lib.prefill_chunk_paged_varpos(q, kn, vn, kp1, vp1, bt, torch.full((B,), p, dtype=torch.int32, device="cuda"),
                                        pos0_max, tab, lse=l1)
    o2 = lib.prefill_chunk_paged(q, kn, vn, kp2, vp2, bt, p, tab, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "outputs differ"
    assert torch.equal(kp1.view(torch.int16), kp2.view(torch.int16)) and \
        torch.equal(vp1.view(torch.int16), vp2.view(torch.int16)), "pools differ"
