"""Chunked prefill against a KV cache (attn_prefill_chunk) against the fp64 oracle.

What is checked, on seeded inputs (inputs.make_chunk):
  * the cache after the call: rows [pos0, pos0+Sq) hold the chunk's keys rotated at their
    absolute positions and rounded to bf16 (within one bf16 rounding of the oracle's fp64
    rotation: the GPU rotates in fp32 first), values copied bit for bit; every other row is
    untouched, bit for bit;
  * the output and LSE against oracle.attention_with_cache on the oracle's own cache, with the
    bf16 bars (max abs <= 2e-2, mean abs <= 1e-3);
  * a serving loop: a cache filled by several chunks, then one decode step, each stage against
    the oracle's own evolving cache;
  * the chunk workload at full size, in the launch configuration the benchmark times, on
    sampled rows.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from conftest import BF16_MAX_ABS, assert_bf16_parity, banner, err_stats, to_np
from transformer_self_attention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_self_attention_amd import lib as L
    return L


def _wl(B, Hq, Hkv, Sq, S_max, D, pos0, seed=0, check_rows=0):
    return inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=seed, kind="chunk",
                           check_rows=check_rows, pos0=pos0, S_max=S_max)


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


def run_chunk(lib, c, *, rope=True, out_dtype=None, kc=None, vc=None, pos0=None, q=None, kn=None, vn=None):
    wl = c.wl
    pos0 = wl.pos0 if pos0 is None else pos0
    tab = lib.make_rope_table(wl.S_max, wl.D) if rope else None
    kc = c.k_cache.torch("cuda") if kc is None else kc
    vc = c.v_cache.torch("cuda") if vc is None else vc
    q = c.q.torch("cuda") if q is None else q
    kn = c.k_new.torch("cuda") if kn is None else kn
    vn = c.v_new.torch("cuda") if vn is None else vn
    Sq = q.shape[2]
    lse = torch.empty((wl.B, wl.Hq, Sq), dtype=torch.float32, device="cuda")
    o = lib.prefill_chunk(q, kn, vn, kc, vc, pos0, tab, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    return o, lse, kc, vc


def check_cache(got_k, got_v, before_k, before_v, ref_k, pos0, Sq, what):
    """Rows outside the chunk untouched; V copied; K within one bf16 rounding of the fp64 value."""
    S_max = before_k.shape[2]
    outside = np.r_[0:pos0, pos0 + Sq:S_max]
    gk, gv = _bits(got_k), _bits(got_v)
    assert np.array_equal(gk[:, :, outside], before_k[:, :, outside]), f"{what}: K rows outside the chunk changed"
    assert np.array_equal(gv[:, :, outside], before_v[:, :, outside]), f"{what}: V rows outside the chunk changed"
    k_new_rows = to_np(got_k)[:, :, pos0:pos0 + Sq]
    ref = ref_k[:, :, pos0:pos0 + Sq]
    # fp32 rotation then one RNE rounding to 8 significant bits: within 2^-8 relative of the exact
    # value, plus the fp32 rotation's own error (a few 2^-24 of |x0 c| + |x1 s| <= ~10 for N(0,1)
    # inputs), which dominates where the two products cancel
    err = np.abs(k_new_rows - ref)
    bad = err > np.abs(ref) * 2.0 ** -8 + 2e-6
    if bad.any():
        idx = np.argwhere(bad)
        for i in idx[:8]:
            t = tuple(i)
            print(f"    {what}: K[{t}] (row {pos0 + t[2]}) got {k_new_rows[t]!r} exact {ref[t]!r}", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} appended key values off by more than one rounding"
    exact = np.mean(k_new_rows == oracle.round_bf16(ref))
    print(f"    {what}: appended keys equal to the oracle's rounding: {exact:.5f}", flush=True)
    assert exact > 0.99


@pytest.mark.parametrize("B,Hq,Hkv,Sq,S_max,D,pos0,rope", [
    (2, 8, 2, 77, 300, 128, 100, True),      # ragged chunk, GQA, pos0 not a tile multiple
    (1, 4, 4, 130, 200, 64, 70, True),       # MHA, D = 64
    (1, 16, 2, 200, 260, 128, 0, True),      # pos0 = 0: an ordinary prefill whose keys are kept
    (2, 8, 8, 1, 500, 128, 333, True),       # one new token (the decode shape)
    (1, 8, 1, 64, 128, 128, 64, True),       # MQA (one KV head); the chunk fills the cache
    (2, 8, 2, 150, 400, 128, 37, False),     # no RoPE: keys copied, exact bf16 products
    (1, 8, 2, 300, 1000, 128, 513, True),    # several query blocks after a long prefix
])
def test_chunk_against_oracle(lib, B, Hq, Hkv, Sq, S_max, D, pos0, rope):
    banner(f"prefill_chunk B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} S_max={S_max} D={D} pos0={pos0} rope={rope}")
    c = inputs.make_chunk(_wl(B, Hq, Hkv, Sq, S_max, D, pos0, seed=Sq + pos0))
    before_k = c.k_cache.bits.view(np.int16)
    before_v = c.v_cache.bits.view(np.int16)
    base = 10000.0 if rope else None
    ref_k, ref_v = oracle.append_to_cache(c.k_cache.f64(), c.v_cache.f64(), c.k_new.f64(), c.v_new.f64(), pos0,
                                          rope_base=base)
    ref_k_exact = ref_k.copy()
    if rope:   # exact rotated values (before rounding), for the one-rounding bound
        ref_k_exact[:, :, pos0:pos0 + Sq] = oracle.rope(c.k_new.f64(), pos0 + np.arange(Sq))
    ref, ref_lse = oracle.attention_with_cache(c.q.f64(), ref_k, ref_v, pos0, rope_base=base)
    for out_dtype in (torch.bfloat16, torch.float32):
        o, lse, kc, vc = run_chunk(lib, c, rope=rope, out_dtype=out_dtype)
        check_cache(kc, vc, before_k, before_v, ref_k_exact, pos0, Sq, f"cache ({out_dtype})")
        assert np.array_equal(_bits(vc)[:, :, pos0:pos0 + Sq], c.v_new.bits.view(np.int16))
        assert_bf16_parity(to_np(o), ref, f"o ({out_dtype})")
        assert err_stats(to_np(lse), ref_lse)[0] < 2e-2


def test_chunks_then_decode_serving_loop(lib):
    """Fill a cache with three chunks (first at pos0 = 0), then decode the next token; every
    stage against the oracle's own cache."""
    B, Hq, Hkv, D, S_max = 2, 16, 2, 128, 640
    bounds = [(0, 200), (200, 333), (333, 600)]
    banner(f"serving loop: chunks {bounds}, then decode at 600 (B={B} Hq={Hq} Hkv={Hkv})")
    total = inputs.make_chunk(_wl(B, Hq, Hkv, 600, S_max, D, 0, seed=77))
    tab = lib.make_rope_table(S_max + 1, D)
    kc = torch.zeros((B, Hkv, S_max, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ref_k = np.zeros((B, Hkv, S_max, D))
    ref_v = np.zeros((B, Hkv, S_max, D))
    q_all, k_all, v_all = total.q.torch("cuda"), total.k_new.torch("cuda"), total.v_new.torch("cuda")
    for a, e in bounds:
        q = q_all[:, :, a:e].contiguous()
        kn = k_all[:, :, a:e].contiguous()
        vn = v_all[:, :, a:e].contiguous()
        o = lib.prefill_chunk(q, kn, vn, kc, vc, a, tab, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref_k, ref_v = oracle.append_to_cache(ref_k, ref_v, total.k_new.f64()[:, :, a:e],
                                              total.v_new.f64()[:, :, a:e], a)
        ref, _ = oracle.attention_with_cache(total.q.f64()[:, :, a:e], ref_k, ref_v, a)
        assert_bf16_parity(to_np(o), ref, f"chunk [{a}, {e})")
    # cache contents: keys within one rounding step of the oracle's, values exact
    got_k = to_np(kc)
    assert np.all(np.abs(got_k - ref_k) <= np.abs(ref_k) * 2.0 ** -7 + 2e-6)
    assert np.array_equal(to_np(vc), ref_v)
    # the next token, decoded against the cache the chunks built
    d = inputs.make_decode(inputs.Workload("d", B=B, Hq=Hq, Hkv=Hkv, S=1, D=D, dtype="bf16", seed=78,
                                           kind="decode"))
    cl = torch.full((B,), 600, dtype=torch.int32, device="cuda")
    qp = torch.full((B,), 600, dtype=torch.int32, device="cuda")
    od = lib.decode(d.q.torch("cuda"), kc, vc, cl, qp, tab, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_d, _ = oracle.decode(d.q.f64(), ref_k, ref_v, [600] * B, [600] * B)
    assert_bf16_parity(to_np(od), ref_d, "decode after chunks")


def test_chunk_config_full_size(lib):
    """The chunk workload at full size (last 2048 tokens of an 8192-token GQA prompt, 6144
    cached), as the benchmark launches it; sampled rows against the oracle."""
    wl = inputs.WORKLOADS["chunk"]
    banner("prefill_chunk full config B=1 Hq=64 Hkv=8 Sq=2048 pos0=6144 S_max=8192 (sampled rows)")
    c = inputs.make_chunk(wl)
    before_k = c.k_cache.bits.view(np.int16)
    before_v = c.v_cache.bits.view(np.int16)
    o, lse, kc, vc = run_chunk(lib, c)
    ref_k, ref_v = oracle.append_to_cache(c.k_cache.f64(), c.v_cache.f64(), c.k_new.f64(), c.v_new.f64(),
                                          wl.pos0)
    exact_k = ref_k.copy()
    exact_k[:, :, wl.pos0:wl.pos0 + wl.S] = oracle.rope(c.k_new.f64(), wl.pos0 + np.arange(wl.S))
    check_cache(kc, vc, before_k, before_v, exact_k, wl.pos0, wl.S, "cache")
    ref, ref_lse = oracle.attention_with_cache(c.q.f64(), ref_k, ref_v, wl.pos0, rows=c.rows)
    got = to_np(o)
    got_rows = np.stack([got[:, h, c.rows[h]] for h in range(wl.Hq)], axis=1)
    got_lse = to_np(lse)
    lse_rows = np.stack([got_lse[:, h, c.rows[h]] for h in range(wl.Hq)], axis=1)
    mx, _ = err_stats(got_rows, ref)
    assert mx <= BF16_MAX_ABS
    # the bf16 output itself carries one rounding (up to 2^-9 relative): the mean bar is checked
    # against the exact result rounded to bf16
    assert_bf16_parity(got_rows, oracle.round_bf16(ref), "o (sampled rows)")
    assert err_stats(lse_rows, ref_lse)[0] < 2e-2


def test_chunk_pos0_zero_matches_prefill(lib):
    """A chunk at pos0 = 0 into an empty cache is an ordinary causal prefill (whose keys are
    then kept): same rows as attn_prefill, up to the bf16 rounding of the stored keys."""
    B, Hq, Hkv, S, D = 1, 8, 2, 257, 128
    banner(f"prefill_chunk pos0=0 vs prefill S={S}")
    c = inputs.make_chunk(_wl(B, Hq, Hkv, S, S, D, 0, seed=3))
    o_chunk, _, _, _ = run_chunk(lib, c, out_dtype=torch.float32)
    tab = lib.make_rope_table(S, D)
    ws = torch.empty(lib.prefill_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    o_pre = lib.prefill(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"), tab, out_dtype=torch.float32,
                        workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(c.q.f64(), c.k_new.f64(), c.v_new.f64())
    assert_bf16_parity(to_np(o_pre), ref, "prefill")
    assert_bf16_parity(to_np(o_chunk), ref, "chunk at pos0 = 0 (keys rounded to bf16 in the cache)")
    assert np.abs(to_np(o_chunk) - to_np(o_pre)).max() < 1e-2
