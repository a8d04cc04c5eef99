"""Pins of the oracle's elementwise pieces and projections against closed forms,
identities and brute force."""
import math

import numpy as np
import pytest

from oracle import concat_target_states, ctx_kv, ctx_proj, rms_norm, rope, silu


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 16))
    assert np.allclose(rope(x, np.zeros(5), 1e6), x, atol=0, rtol=0)
    y = rope(x, np.arange(5) * 977, 1e6)
    half = 8
    assert np.allclose(x[:, :half] ** 2 + x[:, half:] ** 2, y[:, :half] ** 2 + y[:, half:] ** 2,
                       rtol=1e-13, atol=1e-13)


def test_rope_closed_form_pairs_and_frequencies():
    # D = 2: a single pair with inverse frequency theta^0 = 1 -> angle = position.
    for p in (0, 1, 5, 12345):
        assert np.allclose(rope(np.array([1.0, 0.0]), p, 1e6), [math.cos(p), math.sin(p)],
                           rtol=0, atol=1e-12)
        assert np.allclose(rope(np.array([0.0, 1.0]), p, 1e6), [-math.sin(p), math.cos(p)],
                           rtol=0, atol=1e-12)
    # D = 4: dimension 1 pairs with dimension 3 (i with i + D/2) at theta^(-1/2).
    theta, p = 10000.0, 7
    y = rope(np.array([0.0, 1.0, 0.0, 0.0]), p, theta)
    w = p * theta ** -0.5
    assert np.allclose(y, [0.0, math.cos(w), 0.0, math.sin(w)], rtol=0, atol=1e-12)


def test_rope_relative_position():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=64), rng.normal(size=64)
    for m, n in ((10, 3), (1000, 999), (40000, 17)):
        lhs = np.dot(rope(q, m, 1e6), rope(k, n, 1e6))
        rhs = np.dot(rope(q, m - n, 1e6), k)
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs))


def test_rms_norm_closed_forms():
    w = np.array([1.0, 2.0, -0.5, 3.0])
    c, eps = 3.0, 1e-6
    assert np.allclose(rms_norm(np.full(4, c), w, eps), c / math.sqrt(c * c + eps) * w,
                       rtol=1e-15, atol=0)
    rng = np.random.default_rng(2)
    x = rng.normal(size=(3, 32))
    y = rms_norm(x, np.ones(32), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    assert np.allclose(rms_norm(7.5 * x, np.ones(32), 0.0), y, rtol=1e-13)
    assert np.allclose(rms_norm(x, w.repeat(8), 0.0), y * w.repeat(8), rtol=1e-13)


def test_silu_closed_forms():
    assert silu(np.array(0.0)) == 0.0
    assert abs(silu(np.array(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    z = np.linspace(-8, 8, 33)
    assert np.allclose(silu(z) - silu(-z), z, rtol=0, atol=1e-13)
    assert abs(silu(np.array(40.0)) - 40.0) < 1e-12


def test_ctx_proj_matches_naive_loop_and_concat_order():
    rng = np.random.default_rng(3)
    states = rng.normal(size=(3, 5, 4))             # 3 target layers, 5 rows, 4 wide
    X = concat_target_states(states)
    assert X.shape == (5, 12)
    assert np.array_equal(X[:, 4:8], states[1])
    W = rng.normal(size=(6, 12))
    C = ctx_proj(X, W)
    naive = np.zeros((5, 6))
    for i in range(5):
        for j in range(6):
            for k in range(12):
                naive[i, j] += X[i, k] * W[j, k]
    assert np.allclose(C, naive, rtol=1e-13, atol=1e-13)
    # A W_proj that copies target layer 2 returns that layer's states.
    sel = np.zeros((4, 12))
    sel[:, 8:12] = np.eye(4)
    assert np.array_equal(ctx_proj(X, sel), states[2])


def test_ctx_kv_layout_positions_and_packing():
    rng = np.random.default_rng(4)
    Hkv, D, H = 2, 8, 16
    layers = [{"wk": rng.normal(size=(Hkv * D, H)), "wv": rng.normal(size=(Hkv * D, H))}
              for _ in range(2)]
    C1, C2 = rng.normal(size=(5, H)), rng.normal(size=(3, H))
    packed = np.concatenate([C1, C2])
    pos = np.array([0, 1, 2, 3, 4, 0, 1, 2])        # positions restart per sequence
    ks, vs = ctx_kv(packed, layers, pos, Hkv, D, 1e6)
    k1, v1 = ctx_kv(C1, layers, np.arange(5), Hkv, D, 1e6)
    k2, v2 = ctx_kv(C2, layers, np.arange(3), Hkv, D, 1e6)
    for l in range(2):
        assert ks[l].shape == (Hkv, 8, D)
        assert np.allclose(ks[l], np.concatenate([k1[l], k2[l]], axis=1), rtol=0, atol=1e-14)
        assert np.allclose(vs[l], np.concatenate([v1[l], v2[l]], axis=1), rtol=0, atol=1e-14)
        # head-major, V unrotated; K of the first row (position 0) is unrotated too
        raw_k = packed @ layers[l]["wk"].T
        raw_v = packed @ layers[l]["wv"].T
        for g in range(Hkv):
            assert np.allclose(vs[l][g], raw_v[:, g * D:(g + 1) * D], rtol=0, atol=1e-14)
            assert np.allclose(ks[l][g, 0], raw_k[0, g * D:(g + 1) * D], rtol=0, atol=1e-14)
            assert np.allclose(ks[l][g, 5], raw_k[5, g * D:(g + 1) * D], rtol=0, atol=1e-14)
            assert not np.allclose(ks[l][g, 1], raw_k[1, g * D:(g + 1) * D])
