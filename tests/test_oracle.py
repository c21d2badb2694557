"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it checks.  A plausible slip in the oracle -- a dropped
scale, the rotation turned the wrong way, a wrong frequency index, the mask off by one,
the wrong KV head for a query head, a transposed operand -- fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import attention, decode, rope, rope_frequencies

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------------------
# Problem 1 (devthesis section 5): softmax of [16, 8, 0] unscaled and scaled by sqrt(64).
# Realised through the attention oracle: one query, three keys, V = identity rows, so the
# output row is the weight vector.
# --------------------------------------------------------------------------------------
def _problem1_attention(D, q_scale):
    q = np.zeros((1, 1, 1, D))
    q[0, 0, 0, 0] = q_scale
    k = np.zeros((1, 1, 3, D))
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 1, 0] = 0.5
    v = np.zeros((1, 1, 3, D))
    for j in range(3):
        v[0, 0, j, j] = 1.0
    # one query against 3 keys: use decode (no mask, every cached key visible)
    o, lse = decode(q, k, v, [3], [0], rope_base=None)
    return o[0, 0, 0, :3], lse[0, 0]


def test_problem1_scaled_softmax():
    g = _golden("problem1_softmax.json")
    w, lse = _problem1_attention(D=g["d_k"], q_scale=16.0)       # z = [16, 8, 0], / sqrt(64)
    assert np.allclose(w, g["scaled_softmax_printed_5dp"], atol=5e-6, rtol=0)
    assert np.allclose(w, g["scaled_softmax_printed_4dp"], atol=5e-5, rtol=0)
    # the page prints the normaliser sum(exp(s)) = 11.107338 -> lse = ln of it
    assert abs(lse - math.log(g["scaled_exp_sum_printed"])) < 1e-7
    # page's slope A1 (1 - A1) = 0.22269, formed from its rounded A1 and cut (not rounded) to
    # 5 decimals: one unit of the last printed digit
    assert abs(w[0] * (1 - w[0]) - g["scaled_gradient_printed"]) < 1e-5
    assert abs(w.sum() - 1.0) < 1e-15


def test_problem1_unscaled_softmax():
    g = _golden("problem1_softmax.json")
    # D = 4 scales by 1/2, so q = 32 e_0 gives the unscaled logits [16, 8, 0] exactly
    w, _ = _problem1_attention(D=4, q_scale=32.0)
    for got, want, dec in zip(w, g["unscaled_softmax_printed"], g["unscaled_printed_decimals"]):
        assert abs(got - want) <= 0.5 * 10.0 ** (-dec) + 1e-15


# --------------------------------------------------------------------------------------
# Problem 2 (devthesis section 5): a full 2-token head, non-causal, no RoPE.
# --------------------------------------------------------------------------------------
def test_problem2_projection_fixture_consistent():
    g = _golden("problem2_mha.json")
    X = np.array(g["X"])
    assert np.array_equal(X @ np.array(g["W1_Q"]), g["Q1_printed"])
    assert np.array_equal(X @ np.array(g["W1_K"]), g["K1_printed"])
    assert np.array_equal(X @ np.array(g["W1_V"]), g["V1_printed"])
    assert np.array_equal(np.array(g["Q1_printed"]) @ np.array(g["K1_printed"]).T, g["S1_printed"])


def test_problem2_weights_and_output():
    g = _golden("problem2_mha.json")
    Q = np.array(g["Q1_printed"], dtype=np.float64)[None, None]
    K = np.array(g["K1_printed"], dtype=np.float64)[None, None]
    V = np.array(g["V1_printed"], dtype=np.float64)[None, None]
    # weights: V = I gives O = A
    A, _ = attention(Q, K, np.eye(2)[None, None], causal=False, rope_base=None)
    assert np.allclose(A[0, 0], g["A1_printed"], atol=5e-5, rtol=0)
    H, _ = attention(Q, K, V, causal=False, rope_base=None)
    # page multiplies its rounded A_1 by V_1 (entries up to 2): 2 x 5e-5 of rounding
    assert np.allclose(H[0, 0], g["H1_printed"], atol=1e-4 + 1e-12, rtol=0)


def test_problem2_causal_row0_is_v0():
    """Causal mask (learnllm.online listing): row 0 sees only key 0, so o_0 = v_0; row 1 sees both."""
    g = _golden("problem2_mha.json")
    Q = np.array(g["Q1_printed"], dtype=np.float64)[None, None]
    K = np.array(g["K1_printed"], dtype=np.float64)[None, None]
    V = np.array(g["V1_printed"], dtype=np.float64)[None, None]
    H, _ = attention(Q, K, V, causal=True, rope_base=None)
    assert np.array_equal(H[0, 0, 0], V[0, 0, 0])
    Hn, _ = attention(Q, K, V, causal=False, rope_base=None)
    assert np.allclose(H[0, 0, 1], Hn[0, 0, 1], atol=1e-15)


# --------------------------------------------------------------------------------------
# RoPE (devthesis section 3; Problem 3; academy.kwas.tech dim-8 example)
# --------------------------------------------------------------------------------------
def _rot(vec, pos, base=10000.0):
    x = np.asarray(vec, dtype=np.float64)[None, :]
    return rope(x, [pos], base)[0]


def test_rope_example_position0_identity():
    g = _golden("rope_dim8_example.json")
    a = np.array(g["token_vec_a"])
    assert np.array_equal(_rot(a, g["position_a"], g["base"]), a)


def test_rope_example_norms_preserved():
    g = _golden("rope_dim8_example.json")
    for vec, pos in ((g["token_vec_a"], 0), (g["token_vec_b"], g["position_b"]), (g["token_vec_b"], 12345)):
        v = np.array(vec)
        assert abs(np.linalg.norm(_rot(v, pos)) - np.linalg.norm(v)) < 1e-14
    # every pair keeps its own length (rotation acts per 2D slice)
    b = np.array(g["token_vec_b"])
    rb = _rot(b, g["position_b"])
    assert np.allclose(np.hypot(rb[0::2], rb[1::2]), np.hypot(b[0::2], b[1::2]), atol=1e-15)


def test_rope_example_relative_invariance():
    """<R_m q, R_n k> depends only on m - n (devthesis 'Relative Invariance Proof')."""
    g = _golden("rope_dim8_example.json")
    a = np.array(g["token_vec_a"])
    b = np.array(g["token_vec_b"])
    ref = _rot(a, 0) @ _rot(b, 5)
    for t in (1, 7, 100, 8191, 32767):
        assert abs(_rot(a, t) @ _rot(b, 5 + t) - ref) < 1e-12
    # and it does change with the distance (rotation is not the identity)
    assert abs(_rot(a, 0) @ _rot(b, 6) - ref) > 1e-3


def test_rope_problem3_closed_form():
    """Problem 3: <R_m q, R_n k> = A cos((m-n)θ) - B sin((m-n)θ), A = q.k, B = q2 k1 - q1 k2.

    The sign of the B term fixes the rotation direction (counter-clockwise)."""
    rng = np.random.default_rng(11)
    D = 16
    theta = 10000.0 ** (-2.0 * np.arange(D // 2) / D)          # devthesis: theta_i = 10000^(-2i/d_k)
    for _ in range(50):
        i = int(rng.integers(0, D // 2))
        m, n = (int(x) for x in rng.integers(0, 40000, size=2))
        q2 = rng.standard_normal(2)
        k2 = rng.standard_normal(2)
        qv = np.zeros(D)
        kvv = np.zeros(D)
        qv[2 * i:2 * i + 2] = q2
        kvv[2 * i:2 * i + 2] = k2
        got = _rot(qv, m) @ _rot(kvv, n)
        A = q2[0] * k2[0] + q2[1] * k2[1]
        Bc = q2[1] * k2[0] - q2[0] * k2[1]
        want = A * math.cos((m - n) * theta[i]) - Bc * math.sin((m - n) * theta[i])
        assert abs(got - want) < 1e-9


def test_rope_frequencies_geometric_from_one():
    """Pair 0 turns by exactly m radians; frequencies fall geometrically by 10000^(-2/d)
    (devthesis theta_i; codingpancake section 3.2: wavelengths from 2π to 10000·2π)."""
    for D in (8, 64, 128):
        x = np.zeros((D // 2, D))
        for i in range(D // 2):
            x[i, 2 * i] = 1.0
        # rotate each unit vector e_{2i} at position 1 and read the angle back
        rot = np.stack([_rot(x[i], 1) for i in range(D // 2)])
        ang = np.array([math.atan2(rot[i, 2 * i + 1], rot[i, 2 * i]) for i in range(D // 2)])
        assert abs(ang[0] - 1.0) < 1e-15
        ratio = ang[1:] / ang[:-1]
        assert np.allclose(ratio, 10000.0 ** (-2.0 / D), rtol=1e-12)
        assert np.allclose(rope_frequencies(D), ang, rtol=1e-12)


# --------------------------------------------------------------------------------------
# Softmax / attention invariants (devthesis section 1, learnllm.online listing)
# --------------------------------------------------------------------------------------
def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rows_sum_to_one():
    q, k = _rand((2, 4, 33, 16), 1), _rand((2, 2, 33, 16), 2)
    ones = np.ones((2, 2, 33, 16))
    o, _ = attention(q, k, ones, causal=True)
    assert np.allclose(o, 1.0, atol=1e-14)


def test_zero_q_gives_prefix_means():
    q = np.zeros((1, 2, 40, 8))
    k, v = _rand((1, 1, 40, 8), 3), _rand((1, 1, 40, 8), 4)
    o, lse = attention(q, k, v, causal=True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, 41)[:, None]
    for h in range(2):
        assert np.allclose(o[0, h], prefix, atol=1e-14)
        assert np.allclose(lse[0, h], np.log(np.arange(1, 41)), atol=1e-14)


def test_causal_row0_is_v0_random():
    q, k, v = _rand((2, 4, 9, 8), 5), _rand((2, 2, 9, 8), 6), _rand((2, 2, 9, 8), 7)
    o, _ = attention(q, k, v, causal=True)
    for h in range(4):
        assert np.allclose(o[:, h, 0], v[:, h // 2, 0], atol=1e-15)


def test_permutation_equivariance():
    """Attention(PX) = P Attention(X) without mask and position (devthesis section 3)."""
    q, k, v = _rand((1, 2, 12, 8), 8), _rand((1, 2, 12, 8), 9), _rand((1, 2, 12, 8), 10)
    perm = np.random.default_rng(0).permutation(12)
    o, _ = attention(q, k, v, causal=False, rope_base=None)
    op, _ = attention(q[:, :, perm], k[:, :, perm], v[:, :, perm], causal=False, rope_base=None)
    assert np.allclose(op, o[:, :, perm], atol=1e-14)


def test_score_variance_unit():
    """Var(q.k / sqrt(d_k)) = 1 for unit-variance components (devthesis variance analysis)."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((20000, 128))
    k = rng.standard_normal((20000, 128))
    s = np.sum(q * k, axis=1) / math.sqrt(128)
    assert abs(s.var() - 1.0) < 0.05


# --------------------------------------------------------------------------------------
# Library routine: torch's CPU SDPA in float64 (the page's recommended API)
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [(2, 4, 4, 37, 16, True), (1, 8, 2, 64, 32, True),
                                                 (2, 6, 3, 19, 8, False), (1, 4, 1, 50, 16, True)])
def test_matches_torch_sdpa_float64(B, Hq, Hkv, S, D, causal):
    import torch
    import torch.nn.functional as F
    q, k, v = _rand((B, Hq, S, D), 20), _rand((B, Hkv, S, D), 21), _rand((B, Hkv, S, D), 22)
    o, lse = attention(q, k, v, causal=causal, rope_base=10000.0)
    qt = torch.from_numpy(rope(q, np.arange(S)))
    kt = torch.from_numpy(rope(k, np.arange(S)))
    ref = F.scaled_dot_product_attention(qt, kt, torch.from_numpy(v), is_causal=causal, enable_gqa=True)
    assert np.allclose(o, ref.numpy(), atol=1e-12)
    # lse cross-check via logsumexp of explicitly formed scores
    G = Hq // Hkv
    scores = torch.einsum("bhsd,bhtd->bhst", qt, kt.repeat_interleave(G, dim=1)) / math.sqrt(D)
    if causal:
        scores = scores.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    assert np.allclose(lse, torch.logsumexp(scores, dim=-1).numpy(), atol=1e-12)


def test_gqa_head_mapping_is_floor_division():
    """Query head h reads KV head h // G (the reading taken; the pages' formula is lost)."""
    B, Hq, Hkv, S, D = 1, 8, 2, 10, 8
    q, v = _rand((B, Hq, S, D), 30), _rand((B, Hkv, S, D), 31)
    k = _rand((B, Hkv, S, D), 32)
    o, _ = attention(q, k, v, causal=True)
    for h in range(Hq):
        o1, _ = attention(q[:, h:h + 1], k[:, h // 4:h // 4 + 1], v[:, h // 4:h // 4 + 1], causal=True)
        assert np.allclose(o[:, h:h + 1], o1, atol=1e-15)


def test_sampled_rows_equal_full():
    q, k, v = _rand((1, 4, 30, 8), 40), _rand((1, 2, 30, 8), 41), _rand((1, 2, 30, 8), 42)
    full, lfull = attention(q, k, v)
    rows = np.array([[0, 3, 29], [1, 2, 28], [5, 6, 7], [0, 1, 29]])
    part, lpart = attention(q, k, v, rows=rows)
    for h in range(4):
        assert np.allclose(part[0, h], full[0, h, rows[h]], atol=1e-15)
        assert np.allclose(lpart[0, h], lfull[0, h, rows[h]], atol=1e-15)


def test_pos0_shift_does_not_change_output():
    """RoPE makes scores depend only on m - n, so shifting every position leaves attention unchanged."""
    q, k, v = _rand((1, 2, 24, 16), 50), _rand((1, 2, 24, 16), 51), _rand((1, 2, 24, 16), 52)
    o0, _ = attention(q, k, v, pos0=0)
    o1, _ = attention(q, k, v, pos0=1000)
    assert np.allclose(o0, o1, atol=1e-12)


# --------------------------------------------------------------------------------------
# Brute force: scalar loops, written independently of the vectorised oracle
# --------------------------------------------------------------------------------------
def _brute(q, k, v, causal, base):
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv

    def rot(vec, m):
        out = list(vec)
        for i in range(D // 2):
            ang = m * base ** (-(2.0 * i) / D)
            c, s = math.cos(ang), math.sin(ang)
            out[2 * i] = vec[2 * i] * c - vec[2 * i + 1] * s
            out[2 * i + 1] = vec[2 * i] * s + vec[2 * i + 1] * c
        return out

    o = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for i in range(S):
                qi = rot(q[b, h, i], i)
                sc = []
                for j in range(S):
                    if causal and j > i:
                        continue
                    kj = rot(k[b, kv, j], j)
                    sc.append((j, sum(qi[d] * kj[d] for d in range(D)) / math.sqrt(D)))
                mx = max(s for _, s in sc)
                den = sum(math.exp(s - mx) for _, s in sc)
                for j, s in sc:
                    w = math.exp(s - mx) / den
                    for d in range(D):
                        o[b, h, i, d] += w * v[b, kv, j, d]
    return o


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_tiny(causal):
    q, k, v = _rand((2, 4, 11, 8), 60), _rand((2, 2, 11, 8), 61), _rand((2, 2, 11, 8), 62)
    o, _ = attention(q, k, v, causal=causal)
    assert np.allclose(o, _brute(q, k, v, causal, 10000.0), atol=1e-13)


# --------------------------------------------------------------------------------------
# Decode (ninaddeshpande.com, KV cache): one query per sequence against the stored cache
# --------------------------------------------------------------------------------------
def test_decode_equals_prefill_last_row():
    """Decode of row P against the rotated cache K[0..P] equals prefill row P."""
    B, Hq, Hkv, S, D = 2, 8, 2, 21, 16
    q, k, v = _rand((B, Hq, S, D), 70), _rand((B, Hkv, S, D), 71), _rand((B, Hkv, S, D), 72)
    o, lse = attention(q, k, v, causal=True)
    k_cache = rope(k, np.arange(S))                    # cache stores rotated keys
    for P in (0, 7, S - 1):
        od, ld = decode(q[:, :, P:P + 1], k_cache, v, [P + 1] * B, [P] * B)
        assert np.allclose(od[:, :, 0], o[:, :, P], atol=1e-13)
        assert np.allclose(ld, lse[:, :, P], atol=1e-13)


def test_decode_matches_torch_sdpa():
    import torch
    import torch.nn.functional as F
    B, Hq, Hkv, S, D = 3, 8, 2, 40, 16
    q, kc, vc = _rand((B, Hq, 1, D), 80), _rand((B, Hkv, S, D), 81), _rand((B, Hkv, S, D), 82)
    lens = [40, 17, 1]
    qpos = [40, 17, 5]
    o, _ = decode(q, kc, vc, lens, qpos)
    for b in range(B):
        qt = torch.from_numpy(rope(q[b], [qpos[b]]))[None]
        L = lens[b]
        ref = F.scaled_dot_product_attention(qt, torch.from_numpy(kc[b:b + 1, :, :L]),
                                             torch.from_numpy(vc[b:b + 1, :, :L]), enable_gqa=True)
        assert np.allclose(o[b], ref[0].numpy(), atol=1e-12)


def test_decode_empty_cache_is_zero():
    q, kc, vc = _rand((2, 4, 1, 8), 90), _rand((2, 2, 6, 8), 91), _rand((2, 2, 6, 8), 92)
    o, lse = decode(q, kc, vc, [0, -3], [0, 0])
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
