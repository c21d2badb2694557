"""Pins of the oracle's KV-cache functions (CPU only): bfloat16 rounding of stored keys, the
append of a chunk to the cache, and a chunk of queries attending to the cache with the causal
mask aligned at the bottom right, and decode against a paged cache.

Passages: the KV cache of "Transformer internals: attention without the mysticism"
(ninaddeshpande.com), "The KV cache and the memory wall" (earlier tokens' keys and values are
stored and reused); chunked prefill as named on "Multi-Head Attention & Rotary Position
Embeddings (RoPE)" (learnllm.online), "Prefill vs Decode Latency & Memory Wall Waterfall"; the
causal mask of the same page's PyTorch listing; the paged cache of "Building Self-Attention and
Transformer Engines" (codingpancake.com), section 6.2, for decode and for a chunk appended into
the blocks.
"""

import math

import numpy as np
import pytest

from oracle import (append_to_cache, append_to_cache_paged, attention, attention_with_cache, decode, decode_paged,
                    gather_pages, rope, round_bf16)
from transformer_self_attention_amd import inputs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------------------
# bfloat16 rounding (8 significant bits, ties to even)
# --------------------------------------------------------------------------------------
def test_round_bf16_special_values():
    u = 2.0 ** -8
    cases = {
        1.0: 1.0,
        1.0 + u: 1.0,                       # halfway between 1 and 1 + 2^-7: to even (1)
        1.0 + 3 * u: 1.0 + 4 * u,           # halfway between 1 + 2^-7 and 1 + 2^-6: to even
        1.0 + 1.5 * u: 1.0 + 2 * u,         # above halfway
        -(1.0 + 3 * u): -(1.0 + 4 * u),     # sign symmetric
        255.5: 256.0,                       # 255 needs 8 bits; 255.5 ties to 256 (even)
        257.0: 256.0,                       # 257 needs 9 bits; halfway, to even (256)
        259.0: 260.0,
        0.0: 0.0,
        3.0 * 2.0 ** -100: 3.0 * 2.0 ** -100,
    }
    for x, want in cases.items():
        assert round_bf16(np.array([x]))[0] == want, (x, round_bf16(np.array([x]))[0], want)
    assert np.isinf(round_bf16(np.array([np.inf]))[0])


def test_round_bf16_matches_bit_rounding_of_float32():
    """On float32 inputs the frexp form agrees with integer rounding of the float32 bit pattern."""
    x = (np.random.default_rng(5).standard_normal(200000) * np.exp2(np.random.default_rng(6).integers(-30, 30, 200000))).astype(np.float32)
    want = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(round_bf16(x.astype(np.float64)), want)


def test_round_bf16_is_idempotent_and_nearest():
    x = _rand(50000, 7) * 10
    r = round_bf16(x)
    assert np.array_equal(round_bf16(r), r)
    # |x - r| <= half a unit in the 8th significant bit
    _, e = np.frexp(x)
    assert np.all(np.abs(x - r) <= np.ldexp(1.0, e - 9) * (1 + 1e-15))


# --------------------------------------------------------------------------------------
# Appending a chunk
# --------------------------------------------------------------------------------------
def test_append_writes_only_the_chunk_rows():
    B, Hkv, S_max, Sq, D, pos0 = 2, 3, 40, 7, 16, 9
    kc, vc = _rand((B, Hkv, S_max, D), 1), _rand((B, Hkv, S_max, D), 2)
    kn, vn = _rand((B, Hkv, Sq, D), 3), _rand((B, Hkv, Sq, D), 4)
    k2, v2 = append_to_cache(kc, vc, kn, vn, pos0)
    outside = np.r_[0:pos0, pos0 + Sq:S_max]
    assert np.array_equal(k2[:, :, outside], kc[:, :, outside])
    assert np.array_equal(v2[:, :, outside], vc[:, :, outside])
    assert np.array_equal(v2[:, :, pos0:pos0 + Sq], vn)
    # keys: rotated at their absolute positions, then rounded to bf16
    want = round_bf16(rope(kn, pos0 + np.arange(Sq)))
    assert np.array_equal(k2[:, :, pos0:pos0 + Sq], want)
    # rotation preserves each pair's length up to the bf16 rounding
    n_new = np.linalg.norm(kn.reshape(B, Hkv, Sq, D // 2, 2), axis=-1)
    n_rot = np.linalg.norm(k2[:, :, pos0:pos0 + Sq].reshape(B, Hkv, Sq, D // 2, 2), axis=-1)
    assert np.allclose(n_rot, n_new, rtol=2 ** -7)
    with pytest.raises(ValueError):
        append_to_cache(kc, vc, kn, vn, S_max - Sq + 1)


def test_append_without_rope_is_a_copy_of_bf16_values():
    B, Hkv, S_max, Sq, D = 1, 2, 20, 5, 8
    kn = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(_rand((B, Hkv, Sq, D), 5).astype(np.float32)))
    k2, _ = append_to_cache(np.zeros((B, Hkv, S_max, D)), np.zeros((B, Hkv, S_max, D)), kn,
                            np.zeros((B, Hkv, Sq, D)), 3, rope_base=None)
    assert np.array_equal(k2[:, :, 3:8], kn)


# --------------------------------------------------------------------------------------
# Chunk of queries against the cache
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("pos0,Sq", [(0, 12), (5, 7), (11, 1), (1, 11)])
def test_chunk_equals_full_prefill_rows_without_rope(pos0, Sq):
    """Without RoPE the appended keys are copied exactly, so the chunk's rows are rows
    pos0 .. pos0+Sq-1 of the ordinary causal prefill over the whole sequence."""
    B, Hq, Hkv, D = 2, 6, 3, 16
    S = pos0 + Sq
    q, k, v = _rand((B, Hq, S, D), 10), _rand((B, Hkv, S, D), 11), _rand((B, Hkv, S, D), 12)
    full, lfull = attention(q, k, v, causal=True, rope_base=None)
    kc = np.zeros((B, Hkv, S + 3, D))
    vc = np.zeros((B, Hkv, S + 3, D))
    kc[:, :, :pos0], vc[:, :, :pos0] = k[:, :, :pos0], v[:, :, :pos0]
    # k values are not bf16 here, so append without rounding them: write the chunk directly
    kc[:, :, pos0:S], vc[:, :, pos0:S] = k[:, :, pos0:], v[:, :, pos0:]
    o, lse = attention_with_cache(q[:, :, pos0:], kc, vc, pos0, rope_base=None)
    assert np.allclose(o, full[:, :, pos0:], atol=1e-13)
    assert np.allclose(lse, lfull[:, :, pos0:], atol=1e-13)


def test_chunk_rows_equal_decode():
    """Chunk row i is the decode of that query at position pos0+i against the first pos0+i+1
    cache rows (a separate oracle function with no mask)."""
    B, Hq, Hkv, S_max, Sq, D, pos0 = 2, 8, 2, 30, 6, 16, 13
    kc, vc = _rand((B, Hkv, S_max, D), 20), _rand((B, Hkv, S_max, D), 21)
    q, kn, vn = _rand((B, Hq, Sq, D), 22), _rand((B, Hkv, Sq, D), 23), _rand((B, Hkv, Sq, D), 24)
    k2, v2 = append_to_cache(kc, vc, kn, vn, pos0)
    o, lse = attention_with_cache(q, k2, v2, pos0)
    for i in range(Sq):
        od, ld = decode(q[:, :, i:i + 1], k2, v2, [pos0 + i + 1] * B, [pos0 + i] * B)
        assert np.allclose(o[:, :, i], od[:, :, 0], atol=1e-13)
        assert np.allclose(lse[:, :, i], ld, atol=1e-13)


def test_chunk_matches_torch_sdpa_with_explicit_mask():
    import torch
    import torch.nn.functional as F
    B, Hq, Hkv, S_max, Sq, D, pos0 = 2, 8, 4, 50, 9, 32, 23
    kc, vc = _rand((B, Hkv, S_max, D), 30), _rand((B, Hkv, S_max, D), 31)
    q, kn, vn = _rand((B, Hq, Sq, D), 32), _rand((B, Hkv, Sq, D), 33), _rand((B, Hkv, Sq, D), 34)
    k2, v2 = append_to_cache(kc, vc, kn, vn, pos0)
    o, lse = attention_with_cache(q, k2, v2, pos0)
    Sk = pos0 + Sq
    qt = torch.from_numpy(rope(q, pos0 + np.arange(Sq)))
    kt = torch.from_numpy(k2[:, :, :Sk]).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v2[:, :, :Sk]).repeat_interleave(Hq // Hkv, dim=1)
    visible = torch.arange(Sk)[None, :] <= (pos0 + torch.arange(Sq))[:, None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=visible)
    assert np.allclose(o, ref.numpy(), atol=1e-12)
    scores = (qt @ kt.transpose(-1, -2)) / math.sqrt(D)
    ref_lse = torch.logsumexp(scores.masked_fill(~visible, float("-inf")), dim=-1)
    assert np.allclose(lse, ref_lse.numpy(), atol=1e-12)


def _brute_chunk(q, kc, vc, pos0, base):
    """Scalar loops: rotate each query pair at pos0+i, score against the stored keys 0..pos0+i."""
    B, Hq, Sq, D = q.shape
    G = Hq // kc.shape[1]
    o = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for i in range(Sq):
                m = pos0 + i
                qi = list(q[b, h, i])
                for p in range(D // 2):
                    ang = m * base ** (-(2.0 * p) / D)
                    c, s = math.cos(ang), math.sin(ang)
                    qi[2 * p], qi[2 * p + 1] = (q[b, h, i, 2 * p] * c - q[b, h, i, 2 * p + 1] * s,
                                                q[b, h, i, 2 * p] * s + q[b, h, i, 2 * p + 1] * c)
                sc = [sum(qi[d] * kc[b, kv, j, d] for d in range(D)) / math.sqrt(D) for j in range(m + 1)]
                mx = max(sc)
                den = sum(math.exp(x - mx) for x in sc)
                for j, x in enumerate(sc):
                    w = math.exp(x - mx) / den
                    for d in range(D):
                        o[b, h, i, d] += w * vc[b, kv, j, d]
    return o


def test_chunk_brute_force_tiny():
    B, Hq, Hkv, S_max, Sq, D, pos0 = 1, 4, 2, 16, 4, 8, 6
    kc, vc = _rand((B, Hkv, S_max, D), 40), _rand((B, Hkv, S_max, D), 41)
    q, kn, vn = _rand((B, Hq, Sq, D), 42), _rand((B, Hkv, Sq, D), 43), _rand((B, Hkv, Sq, D), 44)
    k2, v2 = append_to_cache(kc, vc, kn, vn, pos0)
    o, _ = attention_with_cache(q, k2, v2, pos0)
    assert np.allclose(o, _brute_chunk(q, k2, v2, pos0, 10000.0), atol=1e-13)


def test_chunks_in_sequence_build_the_same_cache():
    """Appending a sequence in chunks gives the same cache as appending it at once."""
    B, Hkv, S, D = 1, 2, 23, 16
    k, v = _rand((B, Hkv, S, D), 50), _rand((B, Hkv, S, D), 51)
    z = np.zeros((B, Hkv, S, D))
    whole = append_to_cache(z, z, k, v, 0)
    kc, vc = z, z
    for a, e in ((0, 5), (5, 6), (6, 17), (17, 23)):
        kc, vc = append_to_cache(kc, vc, k[:, :, a:e], v[:, :, a:e], a)
    assert np.array_equal(kc, whole[0]) and np.array_equal(vc, whole[1])


# --------------------------------------------------------------------------------------
# Paged KV cache (codingpancake.com section 6.2: fixed-size physical blocks and a block table)
# --------------------------------------------------------------------------------------
def _pages_from_contiguous(kc, vc, bs, perm, extra_blocks=3):
    """Scatter a contiguous cache [B, Hkv, S, D] into physical blocks: block j of sequence b goes
    to physical block perm[b * nb + j]; returns the pools and the block table."""
    B, Hkv, S, D = kc.shape
    nb = -(-S // bs)
    nblk = B * nb + extra_blocks
    kp = np.full((nblk, Hkv, bs, D), np.nan)
    vp = np.full((nblk, Hkv, bs, D), np.nan)
    bt = np.empty((B, nb), dtype=np.int64)
    for b in range(B):
        for j in range(nb):
            phys = int(perm[b * nb + j])
            bt[b, j] = phys
            n = min(bs, S - j * bs)
            kp[phys, :, :n] = kc[b, :, j * bs:j * bs + n]
            vp[phys, :, :n] = vc[b, :, j * bs:j * bs + n]
    return kp, vp, bt


@pytest.mark.parametrize("bs,shuffle", [(16, False), (16, True), (32, True), (4, True)])
def test_paged_decode_equals_contiguous_decode(bs, shuffle):
    B, Hq, Hkv, S, D = 3, 8, 2, 80, 16
    kc, vc, q = _rand((B, Hkv, S, D), 60), _rand((B, Hkv, S, D), 61), _rand((B, Hq, 1, D), 62)
    nb = -(-S // bs)
    perm = np.random.default_rng(63).permutation(B * nb + 3) if shuffle else np.arange(B * nb + 3)
    kp, vp, bt = _pages_from_contiguous(kc, vc, bs, perm)
    lens = [80, 37, 1]
    qpos = [80, 40, 3]
    o, lse = decode_paged(q, kp, vp, bt, lens, qpos)
    o_ref, lse_ref = decode(q, kc, vc, lens, qpos)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    # unused pool slots hold NaN: none of them is read
    assert np.all(np.isfinite(o))


def test_paged_decode_ignores_table_entries_past_the_length():
    B, Hq, Hkv, S, D, bs = 2, 4, 1, 64, 8, 16
    kc, vc, q = _rand((B, Hkv, S, D), 70), _rand((B, Hkv, S, D), 71), _rand((B, Hq, 1, D), 72)
    kp, vp, bt = _pages_from_contiguous(kc, vc, bs, np.arange(B * 4 + 3))
    bt[0, 2:] = 10 ** 9        # sequence 0 uses 2 blocks (length 20 -> blocks 0, 1)
    bt[1, 1:] = -5             # sequence 1 uses 1 block (length 16)
    o, _ = decode_paged(q, kp, vp, bt, [20, 16], [20, 16])
    o_ref, _ = decode(q, kc, vc, [20, 16], [20, 16])
    assert np.array_equal(o, o_ref)


def test_paged_decode_brute_force_tiny():
    """Scalar loops reading the blocks directly (no contiguous cache is formed)."""
    Hq, Hkv, D, bs = 4, 2, 8, 4
    kp, vp = _rand((7, Hkv, bs, D), 80), _rand((7, Hkv, bs, D), 81)
    q = _rand((1, Hq, 1, D), 82)
    bt = np.array([[5, 0, 3]])
    L, pos = 10, 12
    o, _ = decode_paged(q, kp, vp, bt, [L], [pos])
    G = Hq // Hkv
    for h in range(Hq):
        kv = h // G
        qi = list(q[0, h, 0])
        for p in range(D // 2):
            ang = pos * 10000.0 ** (-(2.0 * p) / D)
            c, s = math.cos(ang), math.sin(ang)
            qi[2 * p], qi[2 * p + 1] = q[0, h, 0, 2 * p] * c - q[0, h, 0, 2 * p + 1] * s, \
                q[0, h, 0, 2 * p] * s + q[0, h, 0, 2 * p + 1] * c
        sc = [sum(qi[d] * kp[bt[0, t // bs], kv, t % bs, d] for d in range(D)) / math.sqrt(D) for t in range(L)]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        den = sum(w)
        want = [sum(w[t] / den * vp[bt[0, t // bs], kv, t % bs, d] for t in range(L)) for d in range(D)]
        assert np.allclose(o[0, h, 0], want, atol=1e-13)


# --------------------------------------------------------------------------------------
# A chunk appended into a paged cache
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("bs,pos0,Sq", [(4, 0, 9), (4, 6, 7), (8, 13, 3), (16, 5, 30)])
def test_paged_append_equals_contiguous_append(bs, pos0, Sq):
    """Writing the chunk into the blocks and reading the blocks back in table order gives the
    contiguous cache after the contiguous append; pool slots of no sequence stay as they were."""
    B, Hkv, D = 2, 3, 8
    S = pos0 + Sq + 5
    nb = -(-S // bs)
    kc, vc = _rand((B, Hkv, S, D), 90), _rand((B, Hkv, S, D), 91)
    kn, vn = _rand((B, Hkv, Sq, D), 92), _rand((B, Hkv, Sq, D), 93)
    perm = np.random.default_rng(94).permutation(B * nb + 2)
    kp, vp, bt = _pages_from_contiguous(kc, vc, bs, perm)
    kp2, vp2 = append_to_cache_paged(kp, vp, bt, kn, vn, pos0)
    kc2, vc2 = append_to_cache(kc, vc, kn, vn, pos0)
    gk, gv = gather_pages(kp2, vp2, bt, S)
    assert np.array_equal(gk, kc2) and np.array_equal(gv, vc2)
    spare = perm[B * nb:]
    assert np.array_equal(kp2[spare], kp[spare], equal_nan=True)
    # only the chunk's slots changed
    changed = np.argwhere(np.any(kp2 != kp, axis=(1, 3)) & ~np.isnan(kp).any(axis=(1, 3)))
    want = {(int(bt[b, t // bs]), t % bs) for b in range(B) for t in range(pos0, pos0 + Sq)}
    assert {(int(i), int(j)) for i, j in changed} <= want


def test_paged_append_brute_force_tiny():
    """Scalar loops: the rotated, bf16-rounded key of token t lands in its block's slot."""
    Hkv, D, bs = 1, 4, 2
    kp, vp = np.zeros((5, Hkv, bs, D)), np.zeros((5, Hkv, bs, D))
    bt = np.array([[3, 0, 4]])
    kn, vn = _rand((1, Hkv, 3, D), 95), _rand((1, Hkv, 3, D), 96)
    kp2, vp2 = append_to_cache_paged(kp, vp, bt, kn, vn, 2)     # tokens 2, 3, 4
    for i, t in enumerate((2, 3, 4)):
        blk, slot = int(bt[0, t // bs]), t % bs
        x = list(kn[0, 0, i])
        for p in range(D // 2):
            ang = t * 10000.0 ** (-(2.0 * p) / D)
            c, s = math.cos(ang), math.sin(ang)
            x[2 * p], x[2 * p + 1] = kn[0, 0, i, 2 * p] * c - kn[0, 0, i, 2 * p + 1] * s, \
                kn[0, 0, i, 2 * p] * s + kn[0, 0, i, 2 * p + 1] * c
        assert np.array_equal(kp2[blk, 0, slot], round_bf16(np.array(x)))
        assert np.array_equal(vp2[blk, 0, slot], vn[0, 0, i])
    assert np.all(kp2[3] == 0) and np.all(kp2[1] == 0)   # the blocks of tokens 0, 1 and no token: untouched
