"""Append only (attn_cache_append, attn_cache_append_paged) and the serving loop it completes.

What is checked, on seeded inputs:
  * each sequence's new rows against oracle.append_to_cache at its own position (keys within one
    bf16 rounding of the exact rotation and equal to the oracle's rounding for >99% of values;
    values copied bit for bit); every other row untouched; a sequence whose position is out of
    range untouched; the paged pool, read in table order, equal to the contiguous cache;
  * the cache after an append equals the cache after attn_prefill_chunk appends the same chunk,
    bit for bit;
  * a serving loop on a paged pool: prompts of different lengths through
    attn_prefill_chunk_paged_varpos, then decode steps (append the new token at each
    sequence's position, then attn_decode_paged with cache_len = position + 1), every output
    against the fp64 oracle run on the oracle's own cache.
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


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


def _gather_bits(pool_bits, table, bs, S):
    B, nb = table.shape
    blocks = pool_bits[table.ravel()]
    Hkv, D = blocks.shape[1], blocks.shape[3]
    return blocks.reshape(B, nb, Hkv, bs, D).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, nb * bs, D)[:, :, :S]


@pytest.mark.parametrize("B,Hkv,Sq,S_max,D,bs,positions,rope", [
    (3, 2, 1, 300, 128, 16, [0, 77, 299], True),        # one token each (a decode step), last row
    (3, 2, 5, 256, 64, 32, [3, 252, 100], True),          # D = 64; one position out of range (252 + 5 > 256)
    (2, 4, 17, 400, 128, 16, [383, 16], False),           # no RoPE; several rows across a block edge
    (4, 1, 2, 128, 128, 16, [-1, 0, 126, 64], True),      # MQA-sized head count; a negative position
])
def test_append_against_oracle(lib, B, Hkv, Sq, S_max, D, bs, positions, rope):
    banner(f"cache_append B={B} Hkv={Hkv} Sq={Sq} S_max={S_max} D={D} bs={bs} positions={positions} rope={rope}")
    wl = inputs.Workload("a", B=B, Hq=Hkv, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=31 * Sq + D, kind="chunk",
                         pos0=0, S_max=S_max)
    pc = inputs.make_paged_chunk(wl, block_size=bs)
    c = pc.chunk
    tab = lib.make_rope_table(S_max, D) if rope else None
    kn, vn = c.k_new.torch("cuda"), c.v_new.torch("cuda")
    kc, vc = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    kp, vp = pc.k_pages.torch("cuda"), pc.v_pages.torch("cuda")
    bt = torch.from_numpy(pc.block_table).cuda()
    pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
    lib.cache_append(kn, vn, kc, vc, pos, tab)
    lib.cache_append_paged(kn, vn, kp, vp, bt, pos, tab)
    torch.cuda.synchronize()
    gk = _gather_bits(_bits(kp), pc.block_table, bs, S_max)
    gv = _gather_bits(_bits(vp), pc.block_table, bs, S_max)
    assert np.array_equal(gk, _bits(kc)) and np.array_equal(gv, _bits(vc)), "paged and contiguous appends differ"
    base = 10000.0 if rope else None
    for b, p in enumerate(positions):
        before_k, before_v = c.k_cache.bits.view(np.int16)[b], c.v_cache.bits.view(np.int16)[b]
        if p < 0 or p + Sq > S_max:
            assert np.array_equal(_bits(kc)[b], before_k) and np.array_equal(_bits(vc)[b], before_v), \
                f"seq {b} (position {p} out of range) was written"
            continue
        outside = np.r_[0:p, p + Sq:S_max]
        assert np.array_equal(_bits(kc)[b][:, outside], before_k[:, outside]), f"seq {b}: K rows outside changed"
        assert np.array_equal(_bits(vc)[b][:, outside], before_v[:, outside]), f"seq {b}: V rows outside changed"
        assert np.array_equal(_bits(vc)[b][:, p:p + Sq], c.v_new.bits.view(np.int16)[b]), f"seq {b}: V not copied"
        sl = slice(b, b + 1)
        ref_k, _ = oracle.append_to_cache(c.k_cache.f64()[sl], c.v_cache.f64()[sl], c.k_new.f64()[sl],
                                          c.v_new.f64()[sl], p, rope_base=base)
        exact = oracle.rope(c.k_new.f64()[sl], p + np.arange(Sq)) if rope else c.k_new.f64()[sl]
        got = to_np(kc)[sl][:, :, p:p + Sq]
        assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8 + 2e-6), f"seq {b}: appended keys"
        assert np.mean(got == ref_k[:, :, p:p + Sq]) > 0.99, f"seq {b}: keys differ from the oracle's rounding"


def test_append_equals_the_chunk_append(lib):
    """attn_cache_append writes what attn_prefill_chunk writes into the cache, bit for bit."""
    B, Hq, Hkv, Sq, S_max, D, p = 2, 8, 2, 77, 300, 128, 100
    banner(f"cache_append == the append of prefill_chunk (Sq={Sq} at {p})")
    wl = inputs.Workload("a", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=5, kind="chunk", pos0=p,
                         S_max=S_max)
    c = inputs.make_chunk(wl)
    tab = lib.make_rope_table(S_max, D)
    kc1, vc1 = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    kc2, vc2 = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    lib.cache_append(c.k_new.torch("cuda"), c.v_new.torch("cuda"), kc1, vc1,
                     torch.full((B,), p, dtype=torch.int32, device="cuda"), tab)
    lib.prefill_chunk(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"), kc2, vc2, p, tab)
    torch.cuda.synchronize()
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "keys differ"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "values differ"


def test_serving_loop_prompts_then_decode_steps(lib):
    """Three sequences with prompts of 300, 77 and 512 tokens, each written by a chunk call with a
    start per sequence (0 for that sequence, out of range for the others, which stay untouched),
    then 3 decode steps: append the new token at each sequence's position, then decode."""
    B, Hq, Hkv, D, bs, S_max = 3, 16, 2, 128, 16, 640
    prompt = [300, 77, 512]
    banner(f"serving loop on a paged pool: prompts {prompt}, then 3 decode steps (B={B} Hq={Hq} Hkv={Hkv})")
    rng = np.random.Generator(np.random.PCG64(77))

    def bf16(shape):
        return inputs.Tensor(rng.standard_normal(shape).astype(np.float32), "bf16")

    max_blocks = S_max // bs
    num_blocks = B * max_blocks + 4
    perm = rng.permutation(num_blocks)[:B * max_blocks]
    table_np = perm.reshape(B, max_blocks).astype(np.int32)
    bt = torch.from_numpy(table_np).cuda()
    kp = torch.zeros((num_blocks, Hkv, bs, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    tab = lib.make_rope_table(S_max, D)
    ref_k = np.zeros((B, Hkv, S_max, D))
    ref_v = np.zeros((B, Hkv, S_max, D))
    # prompts: one chunk per sequence, each written with a start per sequence of 0 (others out of
    # range, so untouched), so that every sequence has its own prompt length
    for b in range(B):
        q, k, v = bf16((B, Hq, prompt[b], D)), bf16((B, Hkv, prompt[b], D)), bf16((B, Hkv, prompt[b], D))
        starts = torch.tensor([0 if i == b else -1 for i in range(B)], dtype=torch.int32, device="cuda")
        o = lib.prefill_chunk_paged_varpos(q.torch("cuda"), k.torch("cuda"), v.torch("cuda"), kp, vp, bt, starts,
                                           S_max - prompt[b], tab, out_dtype=torch.float32)
        torch.cuda.synchronize()
        sl = slice(b, b + 1)
        rk, rv = oracle.append_to_cache(ref_k[sl], ref_v[sl], k.f64()[sl], v.f64()[sl], 0)
        ref_k[sl], ref_v[sl] = rk, rv
        ref, _ = oracle.attention_with_cache(q.f64()[sl], rk, rv, 0)
        assert_bf16_parity(to_np(o)[sl], ref, f"prompt of sequence {b}")
        assert torch.isnan(o[[i for i in range(B) if i != b]]).all(), "sequences out of range not NaN"
    pos = np.array(prompt, dtype=np.int32)
    for step in range(3):
        q1, k1, v1 = bf16((B, Hq, 1, D)), bf16((B, Hkv, 1, D)), bf16((B, Hkv, 1, D))
        pos_t = torch.from_numpy(pos).cuda()
        lib.cache_append_paged(k1.torch("cuda"), v1.torch("cuda"), kp, vp, bt, pos_t, tab)
        cache_len = torch.from_numpy(pos + 1).cuda()
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        o = lib.decode_paged(q1.torch("cuda"), kp, vp, bt, cache_len, pos_t, tab, out_dtype=torch.float32, lse=lse)
        torch.cuda.synchronize()
        for b in range(B):
            sl = slice(b, b + 1)
            rk, rv = oracle.append_to_cache(ref_k[sl], ref_v[sl], k1.f64()[sl], v1.f64()[sl], int(pos[b]))
            ref_k[sl], ref_v[sl] = rk, rv
            ref, ref_lse = oracle.attention_with_cache(q1.f64()[sl], rk, rv, int(pos[b]))
            assert_bf16_parity(to_np(o)[sl], ref, f"step {step} seq {b} (position {pos[b]})")
            assert err_stats(to_np(lse)[sl], ref_lse[..., 0])[0] < 2e-2
        pos = pos + 1
