"""Pins of the oracle's dual-source block attention: the brute-force dense-mask
form on tiny inputs, textbook special cases and closed forms, and the pages'
visibility rule (NeMo RL "DFlash Draft Body", How It Works, step 3; cooking-agi
"DFlash: drafting, verification, and speed", One DFlash generation cycle)."""
import math

import numpy as np
import pytest

from oracle import block_attention, block_attn_call, dense_mask_attention, rope


def _case(rng, nb=3, bs=3, Hq=4, Hkv=2, D=8, S=10, rows=2):
    T = rows * S
    q = rng.normal(size=(nb, bs, Hq, D))
    kb = rng.normal(size=(nb, bs, Hkv, D))
    vb = rng.normal(size=(nb, bs, Hkv, D))
    ck = rng.normal(size=(Hkv, T, D))
    cv = rng.normal(size=(Hkv, T, D))
    return q, kb, vb, ck, cv


def test_gathered_equals_dense_mask_brute_force():
    rng = np.random.default_rng(10)
    q, kb, vb, ck, cv = _case(rng, nb=4)
    base = np.array([0, 0, 10, 10])
    anchor = np.array([0, 7, 9, -1])
    a = block_attention(q, kb, vb, ck, cv, base, anchor)
    b = dense_mask_attention(q, kb, vb, ck, cv, base, anchor)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    assert (a[3] == 0).all()


def _textbook_causal_last(qrow, keys, vals):
    # Full causal self-attention over a sequence; return the last query's output.
    L, D = keys.shape
    qs = np.zeros((L, D))
    qs[-1] = qrow
    s = qs @ keys.T / math.sqrt(D)
    s = np.where(np.tril(np.ones((L, L), bool)), s, -np.inf)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return (p @ vals)[-1]


def test_block_size_one_is_causal_attention():
    rng = np.random.default_rng(11)
    q, kb, vb, ck, cv = _case(rng, nb=1, bs=1, Hq=2, Hkv=2, S=12, rows=1)
    a = 9
    out = block_attention(q, kb, vb, ck, cv, [0], [a])
    for h in range(2):
        keys = np.concatenate([ck[h, :a], kb[0, :, h]])
        vals = np.concatenate([cv[h, :a], vb[0, :, h]])
        ref = _textbook_causal_last(q[0, 0, h], keys, vals)
        assert np.allclose(out[0, 0, h], ref, rtol=0, atol=1e-13)


def test_anchor_zero_is_in_block_attention():
    rng = np.random.default_rng(12)
    q, kb, vb, ck, cv = _case(rng, nb=1, bs=4, Hq=1, Hkv=1)
    out = block_attention(q, kb, vb, ck, cv, [0], [0])
    s = q[0, :, 0] @ kb[0, :, 0].T / math.sqrt(8)
    p = np.exp(s) / np.exp(s).sum(1, keepdims=True)
    assert np.allclose(out[0, :, 0], p @ vb[0, :, 0], rtol=0, atol=1e-13)


def test_zero_query_averages_visible_values():
    rng = np.random.default_rng(13)
    q, kb, vb, ck, cv = _case(rng, nb=2, bs=3)
    q[:] = 0.0
    base, anchor = np.array([0, 10]), np.array([5, 2])
    out = block_attention(q, kb, vb, ck, cv, base, anchor)
    for n in range(2):
        for h in range(4):
            g = h // 2
            vis = np.concatenate([cv[g, base[n]:base[n] + anchor[n]], vb[n, :, g]])
            assert np.allclose(out[n, :, h], vis.mean(0), rtol=0, atol=1e-13)


def test_identical_values_returned():
    rng = np.random.default_rng(14)
    q, kb, vb, ck, cv = _case(rng)
    row = rng.normal(size=8)
    vb[:] = row
    cv[:] = row
    out = block_attention(q, kb, vb, ck, cv, [0, 0, 10], [3, 0, 8])
    assert np.allclose(out, np.broadcast_to(row, out.shape), rtol=0, atol=1e-13)


def test_two_key_closed_form_pins_scale():
    # One query, one context key, one block key: weights are a logistic split.
    D = 16
    rng = np.random.default_rng(15)
    q = rng.normal(size=(1, 1, 1, D))
    kb, vb = rng.normal(size=(1, 1, 1, D)), rng.normal(size=(1, 1, 1, D))
    ck, cv = rng.normal(size=(1, 1, D)), rng.normal(size=(1, 1, D))
    out = block_attention(q, kb, vb, ck, cv, [0], [1])[0, 0, 0]
    z = (q[0, 0, 0] @ ck[0, 0] - q[0, 0, 0] @ kb[0, 0, 0]) / math.sqrt(D)
    w = 1.0 / (1.0 + math.exp(-z))
    assert np.allclose(out, w * cv[0, 0] + (1 - w) * vb[0, 0, 0], rtol=0, atol=1e-14)


def test_gqa_head_grouping():
    # With Hq = 4, Hkv = 2 heads 0,1 read KV head 0 only; poisoning KV head 1
    # must not reach them (a modulo mapping would).
    rng = np.random.default_rng(16)
    q, kb, vb, ck, cv = _case(rng)
    clean = block_attention(q, kb, vb, ck, cv, [0, 0, 10], [4, 6, 2])
    kb[:, :, 1] = np.nan
    ck[1] = np.nan
    out = block_attention(q, kb, vb, ck, cv, [0, 0, 10], [4, 6, 2])
    assert np.array_equal(out[:, :, :2], clean[:, :, :2])
    assert np.isnan(out[:, :, 2:]).all()


def test_mha_special_case():
    rng = np.random.default_rng(17)
    q, kb, vb, ck, cv = _case(rng, Hq=2, Hkv=2)
    out = block_attention(q, kb, vb, ck, cv, [0, 0, 10], [4, 6, 2])
    ref = dense_mask_attention(q, kb, vb, ck, cv, [0, 0, 10], [4, 6, 2])
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_information_boundary():
    # Context at or after the anchor, other sequences and other blocks are never read.
    rng = np.random.default_rng(18)
    q, kb, vb, ck, cv = _case(rng, nb=3)
    base, anchor = np.array([0, 0, 10]), np.array([4, 7, 3])
    ref = block_attention(q, kb, vb, ck, cv, base, anchor)
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[:, 4:10] += 100.0
    cv2[:, 4:10] -= 50.0
    ck2[:, 10:] = np.nan
    kb2, vb2 = kb.copy(), vb.copy()
    kb2[1:] = np.nan
    vb2[1:] = np.nan
    out = block_attention(q, kb2, vb2, ck2, cv2, base, anchor)
    assert np.array_equal(out[0], ref[0])


def test_block_attn_call_rotation_and_zeroing():
    rng = np.random.default_rng(19)
    nb, bs, Hq, Hkv, D = 2, 4, 4, 2, 8
    q = rng.normal(size=(nb * bs, Hq * D))
    k = rng.normal(size=(nb * bs, Hkv * D))
    v = rng.normal(size=(nb * bs, Hkv * D))
    ck, cv = rng.normal(size=(Hkv, 20, D)), rng.normal(size=(Hkv, 20, D))
    base, anchor = np.array([0, 10]), np.array([8, -1])
    valid = np.array([1, 1, 0, 1, 1, 1, 1, 1])
    out = block_attn_call(q, k, v, ck, cv, base, anchor, valid, bs, Hq, Hkv, D, 1e4)
    pos = 8 + np.arange(bs)
    q4 = rope(q.reshape(nb, bs, Hq, D)[:1], pos[None, :, None], 1e4)
    k4 = rope(k.reshape(nb, bs, Hkv, D)[:1], pos[None, :, None], 1e4)
    ref = block_attention(q4, k4, v.reshape(nb, bs, Hkv, D)[:1], ck, cv, base[:1], anchor[:1])
    ref = ref.reshape(bs, Hq * D)
    assert np.allclose(out[[0, 1, 3]], ref[[0, 1, 3]], rtol=0, atol=1e-13)
    assert (out[2] == 0).all() and (out[4:] == 0).all()
