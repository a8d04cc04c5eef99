"""Pins of the plan oracle against what the pages fix (NeMo RL "DFlash Draft
Body", How It Works, steps 1, 2 and 4) and against brute force. The exact
SplitMix64 finaliser constants are parity unpinned: the pages print no
known-answer vector; the finaliser is pinned only as a bijection with full
avalanche, and the increment by its definition from the golden ratio."""
import random
from math import isqrt

import numpy as np
import pytest

from oracle import build_plan, eligible_anchors, position_key, row_key, splitmix64

MASK64 = (1 << 64) - 1


def _inv_xorshift(z, s):
    x = z
    for _ in range(64 // s + 1):
        x = z ^ (x >> s)
    return x & MASK64


def _splitmix64_inverse(y):
    # Undo each step of the finaliser: x ^= x >> s is invertible by iteration,
    # multiplication by an odd constant by its inverse modulo 2^64.
    z = _inv_xorshift(y, 31)
    z = (z * pow(0x94D049BB133111EB, -1, 1 << 64)) & MASK64
    z = _inv_xorshift(z, 27)
    z = (z * pow(0xBF58476D1CE4E5B9, -1, 1 << 64)) & MASK64
    z = _inv_xorshift(z, 30)
    return (z - 0x9E3779B97F4A7C15) & MASK64


def test_mixer_is_a_bijection():
    r = random.Random(7)
    for _ in range(2000):
        x = r.getrandbits(64)
        assert _splitmix64_inverse(splitmix64(x)) == x
    for x in (0, 1, MASK64, 1 << 63):
        assert _splitmix64_inverse(splitmix64(x)) == x


def test_mixer_avalanche():
    r = random.Random(11)
    flips = []
    for _ in range(300):
        x = r.getrandbits(64)
        y = splitmix64(x)
        for bit in range(64):
            flips.append(bin(y ^ splitmix64(x ^ (1 << bit))).count("1"))
    mean = sum(flips) / len(flips)
    assert 31.0 < mean < 33.0
    assert min(flips) >= 8


def test_mixer_increment_is_the_golden_gamma():
    # SplitMix64's increment is the odd integer nearest 2^64 / phi (phi the golden
    # ratio), derived here with exact integer square roots. The xor-shift-multiply
    # finaliser is a bijection that maps 0 to 0, so the oracle's output is 0 for
    # exactly one state: the negated increment.
    S = isqrt(5 << 256)                          # floor(sqrt(5) * 2^128)
    num = S - (1 << 128)                         # 2^64 / phi = (sqrt(5) - 1) / 2 * 2^64 = num / 2^65
    lo = num >> 65
    frac2 = num - (lo << 65)                     # fractional part, times 2^65
    cands = [c for c in (lo - 1, lo, lo + 1, lo + 2) if c & 1]
    gamma = min(cands, key=lambda c: abs((c << 65) - num))
    assert lo < gamma + 2 and 0 < frac2
    assert splitmix64((-gamma) & MASK64) == 0
    assert splitmix64((-gamma + 1) & MASK64) != 0 and splitmix64((-gamma - 1) & MASK64) != 0


def _rand_mask(rng, B, S, p_one):
    return (rng.random((B, S)) < p_one).astype(np.uint8)


@pytest.mark.parametrize("B,S,N,bs,p_one", [(3, 40, 5, 4, 0.8), (2, 200, 16, 16, 1.0),
                                            (4, 25, 30, 3, 0.5), (1, 2, 3, 8, 1.0)])
def test_plan_structure(B, S, N, bs, p_one):
    rng = np.random.default_rng(B * 1000 + S)
    mask = _rand_mask(rng, B, S, p_one)
    ids = np.arange(B) + 100
    anchors, pos, valid, loss, num = build_plan(mask, ids, step=3, seed=9, anchors_per_row=N,
                                                block_size=bs)
    for b in range(B):
        elig = eligible_anchors(mask[b])
        n = num[b]
        assert n == min(N, len(elig))
        chosen = [int(a) for a in anchors[b, :n]]
        assert all(a in elig for a in chosen)
        assert chosen == sorted(set(chosen))
        assert (anchors[b, n:] == -1).all()
        # The chosen anchors are exactly the n smallest (key, position) pairs.
        rk = row_key(9, ids[b], 3)
        keys = {a: position_key(rk, a) for a in elig}
        brute = sorted(elig, key=lambda a: (keys[a], a))[:n]
        assert sorted(brute) == chosen
        for i in range(N):
            a = int(anchors[b, i])
            for k in range(bs):
                if a < 0:
                    assert pos[b, i, k] == -1 and valid[b, i, k] == 0 and loss[b, i, k] == 0
                    continue
                p = a + k
                assert pos[b, i, k] == p
                exp_valid = p < S and mask[b, p] == 1
                assert valid[b, i, k] == int(exp_valid)
                assert loss[b, i, k] == int(exp_valid and k >= 1)
            if a >= 0:
                assert valid[b, i, 0] == 1 and loss[b, i, 0] == 0     # anchor computed, no loss
                assert valid[b, i, 1] == 1                              # valid window


def test_plan_deterministic_and_keyed():
    rng = np.random.default_rng(5)
    mask = _rand_mask(rng, 4, 300, 0.9)
    mask[1] = mask[0]
    ids = np.array([7, 7, 8, 9])
    p1 = build_plan(mask, ids, step=11, seed=123, anchors_per_row=8, block_size=4)
    p2 = build_plan(mask.copy(), ids.copy(), step=11, seed=123, anchors_per_row=8, block_size=4)
    for x, y in zip(p1, p2):
        assert np.array_equal(x, y)
    anchors = p1[0]
    assert np.array_equal(anchors[0], anchors[1])      # equal sample id and mask -> equal anchors
    assert not np.array_equal(anchors[0], anchors[2])
    for kw in ({"step": 12}, {"seed": 124}):
        args = dict(step=11, seed=123)
        args.update(kw)
        other = build_plan(mask, ids, anchors_per_row=8, block_size=4, **args)[0]
        assert not np.array_equal(other[0], anchors[0])


def test_plan_row_index_does_not_matter():
    # Randomness depends on (seed, sample id, step), not on where a row sits.
    rng = np.random.default_rng(6)
    mask = _rand_mask(rng, 3, 120, 0.95)
    ids = np.array([4, 5, 6])
    a = build_plan(mask, ids, 0, 1, 6, 4)[0]
    perm = [2, 0, 1]
    b = build_plan(mask[perm], ids[perm], 0, 1, 6, 4)[0]
    assert np.array_equal(a[perm], b)


def test_plan_no_valid_window():
    mask = np.zeros((3, 30), np.uint8)
    mask[1, ::2] = 1                      # isolated valid positions: no window
    mask[2, 29] = 1                       # valid last position only: no successor
    anchors, pos, valid, loss, num = build_plan(mask, [0, 1, 2], 0, 0, 4, 5)
    assert (num == 0).all() and (anchors == -1).all() and (pos == -1).all()
    assert valid.sum() == 0 and loss.sum() == 0


def test_plan_window_at_end_and_overflow():
    S = 10
    mask = np.zeros((1, S), np.uint8)
    mask[0, S - 2:] = 1                    # only window: anchor S-2
    anchors, pos, valid, loss, num = build_plan(mask, [0], 0, 0, 3, 4)
    assert num[0] == 1 and anchors[0, 0] == S - 2
    assert list(valid[0, 0]) == [1, 1, 0, 0]
    assert list(loss[0, 0]) == [0, 1, 0, 0]
    assert list(pos[0, 0]) == [S - 2, S - 1, S, S + 1]


def test_plan_negative_ids_and_huge_seed():
    mask = np.ones((2, 50), np.uint8)
    a = build_plan(mask, [-1, -(2 ** 63)], step=-5, seed=(1 << 64) - 1, anchors_per_row=4,
                   block_size=2)[0]
    assert (a >= 0).all()


def test_plan_anchor_positions_uniform():
    # Over many steps, single anchors over an all-valid row are uniform (chi^2).
    S, steps = 64, 6300
    mask = np.ones((1, S), np.uint8)
    counts = np.zeros(S - 1)
    for step in range(steps):
        rk = row_key(2024, 0, step)
        a = min(range(S - 1), key=lambda x: (position_key(rk, x), x))
        counts[a] += 1
    expected = steps / (S - 1)
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 62 + 6 * np.sqrt(2 * 62)
