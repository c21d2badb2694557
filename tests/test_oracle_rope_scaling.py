"""Pins of the oracle's RoPE frequency scalings (CPU only).

The pages name Position Interpolation, NTK-aware scaling and YaRN as ways to stretch RoPE past
the trained context ("Transformer internals: attention without the mysticism",
ninaddeshpande.com, "Rotary positional embeddings (RoPE)"; devthesis.com Problem 3,
"Superiority for Context Window Extension") without giving formulas; the oracle follows the
published definitions, pinned here by their closed forms and special cases.
"""

import math

import numpy as np
import pytest

from oracle import RopeScaling, attention, decode, rope, rope_angles, rope_frequencies


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("kind", ["pi", "ntk", "yarn"])
def test_factor_one_is_plain_rope(kind):
    x = _rand((3, 17, 64), 1)
    pos = np.arange(100, 117)
    assert np.allclose(rope(x, pos, scaling=RopeScaling(kind, 1.0)), rope(x, pos), atol=1e-14, rtol=0)


def test_pi_divides_positions():
    x = _rand((2, 9, 32), 2)
    pos = np.arange(0, 90, 10)
    assert np.array_equal(rope(x, pos, scaling=RopeScaling("pi", 4.0)), rope(x, pos / 4.0))
    ang, amp = rope_angles(32, [8], scaling=RopeScaling("pi", 4.0))
    assert ang[0, 0] == 2.0 and amp == 1.0                    # pair 0 turns by m / s radians


def test_ntk_keeps_highest_and_divides_lowest_frequency():
    D, s = 128, 8.0
    ang, amp = rope_angles(D, [1], scaling=RopeScaling("ntk", s))
    theta = rope_frequencies(D)
    assert ang[0, 0] == 1.0 and amp == 1.0
    assert math.isclose(ang[0, -1], theta[-1] / s, rel_tol=1e-13)
    ratio = ang[0, 1:] / ang[0, :-1]                          # still a geometric sequence
    assert np.allclose(ratio, (10000.0 * s ** (D / (D - 2.0))) ** (-2.0 / D), rtol=1e-13)


def test_yarn_ramp_and_temperature():
    D, s, L = 128, 4.0, 4096
    sc = RopeScaling("yarn", s, original_max_pos=L, beta_fast=32.0, beta_slow=1.0)
    ang, amp = rope_angles(D, [1], scaling=sc)
    theta = rope_frequencies(D)
    r = L * theta / (2 * math.pi)                              # rotations over the trained context
    fast, slow = r >= 32.0, r <= 1.0
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    assert np.array_equal(ang[0, fast], theta[fast])           # many rotations: kept
    assert np.allclose(ang[0, slow], theta[slow] / s, rtol=1e-15)  # under one rotation: interpolated
    mid = ~fast & ~slow
    g = (r[mid] - 1.0) / 31.0
    assert np.allclose(ang[0, mid], (1 - g) * theta[mid] / s + g * theta[mid], rtol=1e-15)
    ratio = ang[0] / theta
    assert np.all(np.diff(ratio) <= 1e-15)                     # from 1 down to 1/s along the pairs
    assert math.isclose(amp, 0.1 * math.log(4.0) + 1.0) and math.isclose(amp, 1.1386294361119890)
    # rotated vectors are scaled by the temperature factor, pair by pair
    x = _rand((5, D), 3)
    xr = rope(x, np.arange(5), scaling=sc)
    n0 = np.linalg.norm(x.reshape(5, D // 2, 2), axis=-1)
    n1 = np.linalg.norm(xr.reshape(5, D // 2, 2), axis=-1)
    assert np.allclose(n1, amp * n0, rtol=1e-14)


@pytest.mark.parametrize("sc", [RopeScaling("pi", 3.0), RopeScaling("ntk", 5.0), RopeScaling("yarn", 8.0, 2048)])
def test_scaled_rope_stays_relative(sc):
    """Scores depend on m - n only, under every scaling (rotations plus a uniform amplitude)."""
    q, k = _rand((1, 64), 4), _rand((1, 64), 5)
    a = float((rope(q, [7], scaling=sc) @ rope(k, [3], scaling=sc).T)[0, 0])
    b = float((rope(q, [1007], scaling=sc) @ rope(k, [1003], scaling=sc).T)[0, 0])
    assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-12)


def test_attention_and_decode_take_the_scaling():
    """Decode of row P against keys rotated with the same scaling equals prefill row P."""
    sc = RopeScaling("yarn", 4.0, original_max_pos=64)
    B, Hq, Hkv, S, D = 1, 4, 2, 30, 32
    q, k, v = _rand((B, Hq, S, D), 6), _rand((B, Hkv, S, D), 7), _rand((B, Hkv, S, D), 8)
    o, _ = attention(q, k, v, rope_scaling=sc)
    o_plain, _ = attention(q, k, v)
    assert not np.allclose(o, o_plain)
    kc = rope(k, np.arange(S), scaling=sc)
    for P in (0, 13, 29):
        od, _ = decode(q[:, :, P:P + 1], kc, v, [P + 1], [P], rope_scaling=sc)
        assert np.allclose(od[:, :, 0], o[:, :, P], atol=1e-13)


def test_bad_scalings_rejected():
    with pytest.raises(ValueError):
        rope_angles(8, [1], scaling=RopeScaling("pi", 0.5))
    with pytest.raises(ValueError):
        rope_angles(8, [1], scaling=RopeScaling("linear", 2.0))
