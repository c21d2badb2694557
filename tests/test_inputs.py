"""The seeded input generator: rounding, determinism and the long-context key structure (CPU)."""

import numpy as np
import torch

from transformer_self_attention_amd import inputs


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        # exact ties between two bf16 values: low 16 bits == 0x8000
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0], dtype=np.float32),
    ])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_prefill_draw_is_deterministic_and_ordered():
    wl = inputs.WORKLOADS["mha"]
    a = inputs.make_prefill(wl, S=64, B=1)
    b = inputs.make_prefill(wl, S=64, B=1)
    assert np.array_equal(a.q.bits, b.q.bits) and np.array_equal(a.v.bits, b.v.bits)
    # Q, K, V come from one stream in that order
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    q = rng.standard_normal(a.q.f32.size).astype(np.float32)
    k = rng.standard_normal(a.k.f32.size).astype(np.float32)
    assert np.array_equal(inputs.f32_to_bf16_bits(q).reshape(a.q.shape), a.q.bits)
    assert np.array_equal(inputs.f32_to_bf16_bits(k).reshape(a.k.shape), a.k.bits)


def test_chunked_draw_equals_single_draw():
    rng1 = np.random.Generator(np.random.PCG64(5))
    rng2 = np.random.Generator(np.random.PCG64(5))
    one = rng1.standard_normal(1000).astype(np.float32)
    chunked = inputs._normal32(rng2, (1000,), chunk=64)
    assert np.array_equal(one, chunked)


def test_long_context_big_keys_scaled_by_8_exactly():
    wl = inputs.WORKLOADS["long"]
    small = inputs.make_prefill(wl, S=2000)
    nbig = int(round(0.01 * 2000))
    assert small.big_keys.shape == (1, 8, nbig)
    # rebuild the unscaled K from the same stream and compare row by row
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    _ = rng.standard_normal(1 * 32 * 2000 * 128)
    k = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(
        rng.standard_normal(1 * 8 * 2000 * 128).astype(np.float32))).reshape(1, 8, 2000, 128)
    for h in range(8):
        big = set(small.big_keys[0, h].tolist())
        assert len(big) == nbig
        for j in range(2000):
            want = k[0, h, j] * (8.0 if j in big else 1.0)
            assert np.array_equal(small.k.f32[0, h, j], want.astype(np.float32))


def test_sampled_rows_include_edges():
    wl = inputs.WORKLOADS["gqa"]
    p = inputs.make_prefill(wl, S=1024)
    assert p.rows.shape == (64, 256)
    for r in p.rows:
        assert len(set(r.tolist())) == 256
        assert {0, 1, 1022, 1023} <= set(r.tolist())


def test_workload_work_counts():
    g = inputs.WORKLOADS["gqa"]
    assert g.prefill_flops() == 2 * 64 * 8192 ** 2 * 128
    d = inputs.WORKLOADS["decode"]
    assert d.decode_kv_bytes() == 1 << 30


def test_chunk_workload_and_draw_order():
    c = inputs.WORKLOADS["chunk"]
    assert (c.B, c.Hq, c.Hkv, c.S, c.D, c.pos0, c.S_max) == (1, 64, 8, 2048, 128, 6144, 8192)
    # at pos0 = 0 the count is the ordinary causal prefill's
    import dataclasses
    assert dataclasses.replace(c, pos0=0).chunk_flops() == 2 * 64 * 2048 ** 2 * 128
    assert c.chunk_flops() == 4 * 64 * 128 * (6144 * 2048 + 2048 ** 2 / 2)
    small = dataclasses.replace(c, S=40, S_max=100, pos0=30, check_rows=8)
    a = inputs.make_chunk(small)
    b = inputs.make_chunk(small)
    assert np.array_equal(a.k_cache.bits, b.k_cache.bits) and np.array_equal(a.rows, b.rows)
    # draw order q, k_new, v_new, k_cache, v_cache from one PCG64 stream
    rng = np.random.Generator(np.random.PCG64(small.seed))
    q = rng.standard_normal((1, 64, 40, 128)).astype(np.float32)
    assert np.array_equal(a.q.f32, inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(q)))
    rng.standard_normal((1, 8, 40, 128))
    rng.standard_normal((1, 8, 40, 128))
    kc = rng.standard_normal((1, 8, 100, 128)).astype(np.float32)
    assert np.array_equal(a.k_cache.f32, inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(kc)))
    assert a.rows.shape == (64, 8)


def test_paged_decode_layout():
    """Each table entry points at the pool block holding those tokens; other slots are NaN."""
    wl = inputs.Workload("d", B=3, Hq=8, Hkv=2, S=70, D=16, dtype="bf16", seed=9, kind="decode")
    pd = inputs.make_paged_decode(wl, block_size=16, spare_blocks=4)
    d = pd.contiguous
    assert pd.block_table.shape == (3, 5) and pd.k_pages.shape == (19, 2, 16, 16)
    assert len(set(pd.block_table.ravel().tolist())) == 15
    for b in range(3):
        for t in range(70):
            blk = pd.block_table[b, t // 16]
            assert np.array_equal(pd.k_pages.bits[blk, :, t % 16], d.k_cache.bits[b, :, t])
            assert np.array_equal(pd.v_pages.bits[blk, :, t % 16], d.v_cache.bits[b, :, t])
    used = np.zeros(19, bool)
    used[pd.block_table.ravel()] = True
    assert np.all(np.isnan(pd.k_pages.f32[~used]))
    assert np.all(np.isnan(pd.k_pages.f32[pd.block_table[:, 4], :, 6:]))   # tail of the last block
    # same draws as the contiguous generator
    d2 = inputs.make_decode(wl)
    assert np.array_equal(d.k_cache.bits, d2.k_cache.bits) and np.array_equal(d.q.bits, d2.q.bits)


def test_window_work_counts():
    import dataclasses
    swa = inputs.WORKLOADS["swa"]
    S, W = 32768, 4096
    assert swa.prefill_flops() == 4 * 32 * 128 * (S * S / 2 - (S - W - 1) * (S - W) / 2)
    # a window covering every key counts like plain causal
    assert dataclasses.replace(swa, window=S - 1).prefill_flops() == 2 * 32 * S * S * 128
    assert dataclasses.replace(swa, window=-1).prefill_flops() == 2 * 32 * S * S * 128
    # brute count of visible pairs (i - W <= j <= i) on a small case matches within the diagonal convention
    s, w = 50, 7
    pairs = sum(1 for i in range(s) for j in range(s) if i - w <= j <= i)
    small = dataclasses.replace(swa, S=s, window=w, B=1, Hq=1, D=1)
    assert abs(small.prefill_flops() / 4 - pairs) <= s / 2     # S^2/2 convention vs S(S+1)/2 exact
    assert inputs.WORKLOADS["swa_decode"].decode_kv_bytes() == (1 << 30) // 2
