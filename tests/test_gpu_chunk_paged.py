"""Chunked prefill against a paged KV cache (attn_prefill_chunk_paged) on the GPU.

What is checked, on seeded inputs (inputs.make_paged_chunk: the cache of make_chunk cut into
blocks scattered over a pool):
  * the pool after the call equals, bit for bit, the contiguous cache after attn_prefill_chunk
    on the same inputs, read back through the block table; pool slots of no sequence keep their
    NaN; the output and LSE are the contiguous call's, bit for bit;
  * the output against oracle.attention_with_cache on the oracle's own paged append, with the
    bf16 bars;
  * with a window, blocks wholly before the first query's window are never read, nor are
    their table entries (NaN data, entries -1 or out of range);
  * a serving loop on one pool: chunks, then a paged decode step.
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


def _wl(B, Hq, Hkv, Sq, S_max, D, pos0, seed):
    return inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=seed, kind="chunk",
                           pos0=pos0, S_max=S_max)


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _gather_bits(pool_bits, table, bs, n):
    """[B, Hkv, n, D] bits of the first n tokens, read through the block table."""
    B = table.shape[0]
    out = np.empty((B, pool_bits.shape[1], n, pool_bits.shape[3]), dtype=pool_bits.dtype)
    for b in range(B):
        for t in range(n):
            out[b, :, t] = pool_bits[table[b, t // bs], :, t % bs]
    return out


@pytest.mark.parametrize("B,Hq,Hkv,Sq,pos0,S_max,D,bs,W,rope", [
    (2, 8, 2, 100, 37, 150, 128, 16, None, True),     # pos0 and Sq not block or tile multiples
    (1, 16, 2, 64, 64, 128, 128, 32, None, True),
    (2, 4, 4, 33, 0, 40, 64, 16, None, True),          # first chunk of a prompt, D = 64
    (3, 12, 3, 77, 200, 300, 128, 64, 90, True),      # window
    (2, 8, 1, 50, 130, 200, 128, 128, None, False),   # no RoPE, MQA-like
    (1, 64, 8, 256, 1000, 1300, 128, 16, 300, True),  # GQA 8 heads per KV head, window
])
def test_paged_chunk_against_contiguous_and_oracle(lib, B, Hq, Hkv, Sq, pos0, S_max, D, bs, W, rope):
    banner(f"paged chunk B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} pos0={pos0} S_max={S_max} D={D} bs={bs} W={W} "
           f"rope={rope}")
    wl = _wl(B, Hq, Hkv, Sq, S_max, D, pos0, seed=9000 + Sq + pos0)
    p = inputs.make_paged_chunk(wl, block_size=bs)
    c = p.chunk
    tab = lib.make_rope_table(S_max, D) if rope else None
    q, kn, vn = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    kp, vp = p.k_pages.torch("cuda"), p.v_pages.torch("cuda")
    bt = torch.from_numpy(p.block_table).cuda()
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    o = lib.prefill_chunk_paged(q, kn, vn, kp, vp, bt, pos0, tab, window=W, out_dtype=torch.float32, lse=lse)
    # the same chunk on the contiguous cache
    kc, vc = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    lc = torch.empty_like(lse)
    oc = lib.prefill_chunk(q, kn, vn, kc, vc, pos0, tab, window=W, out_dtype=torch.float32, lse=lc)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc), "paged and contiguous chunk outputs differ"
    kp_bits = kp.cpu().view(torch.int16).numpy()
    vp_bits = vp.cpu().view(torch.int16).numpy()
    n = -(-S_max // bs) * bs
    gk = _gather_bits(kp_bits, p.block_table, bs, S_max)
    gv = _gather_bits(vp_bits, p.block_table, bs, S_max)
    assert np.array_equal(gk, kc.cpu().view(torch.int16).numpy()), "pool keys differ from the contiguous cache"
    assert np.array_equal(gv, vc.cpu().view(torch.int16).numpy()), "pool values differ from the contiguous cache"
    # slots of no sequence: still NaN
    used = np.zeros(p.k_pages.shape[0], bool)
    used[p.block_table.ravel()] = True
    assert np.all(kp_bits[~used] == np.int16(inputs.BF16_NAN_BITS))
    tail = n - S_max
    if tail:
        last = p.block_table[:, -1]
        assert np.all(kp_bits[last, :, bs - tail:] == np.int16(inputs.BF16_NAN_BITS))
    # against the oracle's own paged append
    base = 10000.0 if rope else None
    rk, rv = oracle.append_to_cache_paged(p.k_pages.f64(), p.v_pages.f64(), p.block_table, c.k_new.f64(),
                                          c.v_new.f64(), pos0, rope_base=base)
    ck, cv = oracle.gather_pages(rk, rv, p.block_table, pos0 + Sq)
    ref, ref_lse = oracle.attention_with_cache(c.q.f64(), ck, cv, pos0, rope_base=base, window=W)
    assert_bf16_parity(to_np(o), ref, "paged chunk o")
    assert err_stats(to_np(lse), ref_lse)[0] < 2e-2


def test_paged_chunk_window_skips_released_blocks(lib):
    """Blocks wholly before the first query's window start hold NaN and their table entries are
    -1 or out of range: the result equals the contiguous call's, bit for bit."""
    B, Hq, Hkv, Sq, pos0, S_max, D, bs, W = 2, 8, 2, 64, 700, 800, 128, 16, 200
    banner(f"paged chunk, released blocks before the window: pos0={pos0} W={W} bs={bs}")
    wl = _wl(B, Hq, Hkv, Sq, S_max, D, pos0, seed=9100)
    p = inputs.make_paged_chunk(wl, block_size=bs)
    c = p.chunk
    kp_bits, vp_bits, table = p.k_pages.bits.copy(), p.v_pages.bits.copy(), p.block_table.copy()
    first_seen = pos0 - W                      # the first query's window start
    for b in range(B):
        for j in range(first_seen // bs):      # blocks wholly before it
            kp_bits[table[b, j]] = inputs.BF16_NAN_BITS
            vp_bits[table[b, j]] = inputs.BF16_NAN_BITS
            table[b, j] = -1 if j % 2 else 10 ** 8
    tab = lib.make_rope_table(S_max, D)
    q, kn, vn = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    o = lib.prefill_chunk_paged(q, kn, vn, _dev(kp_bits), _dev(vp_bits), torch.from_numpy(table).cuda(), pos0,
                                tab, window=W, out_dtype=torch.float32)
    oc = lib.prefill_chunk(q, kn, vn, c.k_cache.torch("cuda"), c.v_cache.torch("cuda"), pos0, tab, window=W,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, oc)
    assert np.all(np.isfinite(to_np(o)))


def test_paged_serving_loop(lib):
    """One pool: a 300-token prompt in chunks of 128, 100 and 72, then a decode step of every
    sequence against the pool, each stage against the oracle's own evolving pool."""
    B, Hq, Hkv, D, bs, S_max = 2, 16, 4, 128, 16, 320
    banner("paged serving loop: chunks 128 + 100 + 72, then decode")
    wl = _wl(B, Hq, Hkv, 300, S_max, D, 0, seed=9200)
    p = inputs.make_paged_chunk(wl, block_size=bs)
    c = p.chunk
    tab = lib.make_rope_table(S_max + 1, D)
    kp, vp = p.k_pages.torch("cuda"), p.v_pages.torch("cuda")
    bt = torch.from_numpy(p.block_table).cuda()
    rk, rv = p.k_pages.f64(), p.v_pages.f64()
    q_all, kn_all, vn_all = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    pos0 = 0
    for Sq in (128, 100, 72):
        sl = slice(pos0, pos0 + Sq)
        o = lib.prefill_chunk_paged(q_all[:, :, sl].contiguous(), kn_all[:, :, sl].contiguous(),
                                    vn_all[:, :, sl].contiguous(), kp, vp, bt, pos0, tab, out_dtype=torch.float32)
        torch.cuda.synchronize()
        rk, rv = oracle.append_to_cache_paged(rk, rv, p.block_table, c.k_new.f64()[:, :, sl], c.v_new.f64()[:, :, sl],
                                              pos0)
        ck, cv = oracle.gather_pages(rk, rv, p.block_table, pos0 + Sq)
        ref, _ = oracle.attention_with_cache(c.q.f64()[:, :, sl], ck, cv, pos0)
        assert_bf16_parity(to_np(o), ref, f"chunk at {pos0}")
        pos0 += Sq
    # one decode step per sequence at position 300 against the 300 cached tokens
    dq = inputs.make_decode(inputs.Workload("d", B=B, Hq=Hq, Hkv=Hkv, S=1, D=D, dtype="bf16", seed=9201,
                                            kind="decode"))
    cl = torch.full((B,), pos0, dtype=torch.int32, device="cuda")
    od = lib.decode_paged(dq.q.torch("cuda"), kp, vp, bt, cl, cl.clone(), tab, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_d, _ = oracle.decode_paged(dq.q.f64(), rk, rv, p.block_table, [pos0] * B, [pos0] * B)
    assert_bf16_parity(to_np(od), ref_d, "decode after the chunks")
