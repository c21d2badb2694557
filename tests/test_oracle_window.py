"""Pins of the oracle's sliding window (CPU only).

Passage: "Building Self-Attention and Transformer Engines" (codingpancake.com), section 6.4: a
token attends only to the W tokens before it.  Reading: the query at position p sees the keys at
positions p - W .. p, on top of the causal mask.
"""

import math

import numpy as np
import pytest

from oracle import append_to_cache, attention, attention_with_cache, decode, decode_paged, rope


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_window_zero_attends_to_itself_only():
    """W = 0: each row sees only its own key, so its output is its own value row, exactly."""
    q, k, v = _rand((2, 4, 19, 16), 1), _rand((2, 2, 19, 16), 2), _rand((2, 2, 19, 16), 3)
    o, lse = attention(q, k, v, window=0)
    assert np.array_equal(o, np.repeat(v, 2, axis=1))
    qr, kr = rope(q, np.arange(19)), rope(k, np.arange(19))
    own = np.einsum("bhsd,bhsd->bhs", qr, np.repeat(kr, 2, axis=1)) / 4.0
    assert np.allclose(lse, own, atol=1e-13)


def test_window_covering_everything_is_plain_causal():
    q, k, v = _rand((1, 4, 30, 8), 4), _rand((1, 4, 30, 8), 5), _rand((1, 4, 30, 8), 6)
    o0, l0 = attention(q, k, v)
    for W in (29, 30, 1000):
        o1, l1 = attention(q, k, v, window=W)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    o2, _ = attention(q, k, v, window=28)        # row 29 loses key 0: differs there only
    assert np.array_equal(o2[:, :, :29], o0[:, :, :29]) and not np.allclose(o2[:, :, 29], o0[:, :, 29])


def test_window_one_is_two_key_softmax():
    """W = 1: row i (i >= 1) mixes v_{i-1} and v_i with weights from its two scores."""
    q, k, v = _rand((1, 1, 6, 4), 7), _rand((1, 1, 6, 4), 8), _rand((1, 1, 6, 4), 9)
    o, _ = attention(q, k, v, window=1, rope_base=None)
    for i in range(1, 6):
        s0 = q[0, 0, i] @ k[0, 0, i - 1] / 2.0
        s1 = q[0, 0, i] @ k[0, 0, i] / 2.0
        a = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.allclose(o[0, 0, i], a * v[0, 0, i - 1] + (1 - a) * v[0, 0, i], atol=1e-14)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])


def test_window_matches_torch_sdpa_band_mask():
    import torch
    import torch.nn.functional as F
    B, Hq, Hkv, S, D, W = 2, 8, 2, 45, 16, 7
    q, k, v = _rand((B, Hq, S, D), 10), _rand((B, Hkv, S, D), 11), _rand((B, Hkv, S, D), 12)
    o, lse = attention(q, k, v, window=W)
    qt, kt = torch.from_numpy(rope(q, np.arange(S))), torch.from_numpy(rope(k, np.arange(S)))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    band = (j <= i) & (j >= i - W)
    ref = F.scaled_dot_product_attention(qt, kt.repeat_interleave(4, 1), torch.from_numpy(v).repeat_interleave(4, 1),
                                         attn_mask=band)
    assert np.allclose(o, ref.numpy(), atol=1e-12)
    sc = (qt @ kt.repeat_interleave(4, 1).transpose(-1, -2)) / math.sqrt(D)
    assert np.allclose(lse, torch.logsumexp(sc.masked_fill(~band, float("-inf")), -1).numpy(), atol=1e-12)


def test_window_brute_force_tiny():
    B, Hq, Hkv, S, D, W = 1, 2, 1, 9, 4, 3
    q, k, v = _rand((B, Hq, S, D), 13), _rand((B, Hkv, S, D), 14), _rand((B, Hkv, S, D), 15)
    o, _ = attention(q, k, v, window=W, rope_base=None)
    for h in range(Hq):
        for i in range(S):
            js = [j for j in range(S) if i - W <= j <= i]
            sc = [sum(q[0, h, i, d] * k[0, 0, j, d] for d in range(D)) / 2.0 for j in js]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            want = [sum(w[t] * v[0, 0, j, d] for t, j in enumerate(js)) / sum(w) for d in range(D)]
            assert np.allclose(o[0, h, i], want, atol=1e-14)


def test_window_decode_equals_prefill_row():
    B, Hq, Hkv, S, D, W = 2, 4, 2, 40, 16, 11
    q, k, v = _rand((B, Hq, S, D), 16), _rand((B, Hkv, S, D), 17), _rand((B, Hkv, S, D), 18)
    o, lse = attention(q, k, v, window=W)
    kc = rope(k, np.arange(S))
    for P in (0, 5, 11, 12, 39):
        od, ld = decode(q[:, :, P:P + 1], kc, v, [P + 1] * B, [P] * B, window=W)
        assert np.allclose(od[:, :, 0], o[:, :, P], atol=1e-13)
        assert np.allclose(ld, lse[:, :, P], atol=1e-13)


def test_window_decode_with_nothing_visible_is_empty():
    q, kc, vc = _rand((2, 4, 1, 8), 19), _rand((2, 2, 10, 8), 20), _rand((2, 2, 10, 8), 21)
    o, lse = decode(q, kc, vc, [10, 10], [30, 14], window=5)   # window [25, 30] / [9, 14]
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    o1, _ = decode(q[1:], kc[1:, :, 9:10], vc[1:, :, 9:10], [1], [14])
    assert np.allclose(o[1], o1[0], atol=1e-14)


def test_window_chunk_rows_equal_full_prefill_rows():
    B, Hq, Hkv, D, pos0, Sq, W = 1, 4, 2, 16, 17, 9, 6
    S = pos0 + Sq
    q, k, v = _rand((B, Hq, S, D), 22), _rand((B, Hkv, S, D), 23), _rand((B, Hkv, S, D), 24)
    full, lfull = attention(q, k, v, rope_base=None, window=W)
    kc, vc = np.zeros((B, Hkv, S, D)), np.zeros((B, Hkv, S, D))
    kc[:, :, :pos0], vc[:, :, :pos0] = k[:, :, :pos0], v[:, :, :pos0]
    kc, vc = append_to_cache(kc, vc, k[:, :, pos0:], v[:, :, pos0:], pos0, rope_base=None)
    # k is not bf16 here: put the exact values back (the append rounds keys to bf16)
    kc[:, :, pos0:] = k[:, :, pos0:]
    o, lse = attention_with_cache(q[:, :, pos0:], kc, vc, pos0, rope_base=None, window=W)
    assert np.allclose(o, full[:, :, pos0:], atol=1e-13) and np.allclose(lse, lfull[:, :, pos0:], atol=1e-13)


def test_window_paged_decode_equals_contiguous():
    B, Hq, Hkv, S, D, bs, W = 2, 4, 1, 64, 8, 16, 20
    kc, vc, q = _rand((B, Hkv, S, D), 25), _rand((B, Hkv, S, D), 26), _rand((B, Hq, 1, D), 27)
    kp = kc.reshape(B, Hkv, 4, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * 4, Hkv, bs, D)
    vp = vc.reshape(B, Hkv, 4, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * 4, Hkv, bs, D)
    bt = np.arange(B * 4).reshape(B, 4)
    o, _ = decode_paged(q, kp, vp, bt, [64, 50], [64, 50], window=W)
    o_ref, _ = decode(q, kc, vc, [64, 50], [64, 50], window=W)
    assert np.array_equal(o, o_ref)


def test_window_rejects_bad_use():
    q = _rand((1, 1, 4, 4), 28)
    with pytest.raises(ValueError):
        attention(q, q, q, causal=False, window=2)
    with pytest.raises(ValueError):
        attention(q, q, q, window=-1)
