"""Pins of the draft-loss oracle (angelspec "DFlash", How it works, "Loss":
cross-entropy with an exponential positional decay favouring early block
positions; NeMo RL "DFlash Draft Body", step 4: the loss mask)."""
import math

import numpy as np

import oracle


def test_uniform_logits_give_log_vocab():
    rng = np.random.default_rng(0)
    V, H = 37, 8
    h = rng.standard_normal((5, H))
    ce = oracle.lm_head_ce_rows(h, np.zeros((V, H)), rng.integers(0, V, 5))
    assert np.allclose(ce, math.log(V), rtol=0, atol=1e-14)


def test_two_token_vocabulary_closed_form():
    for z0, z1 in [(0.3, -1.2), (5.0, 5.0), (-40.0, 2.0)]:
        z = np.array([[z0, z1]])
        assert abs(oracle.token_ce(z, [0])[0] - math.log1p(math.exp(z1 - z0))) < 1e-13
        assert abs(oracle.token_ce(z, [1])[0] - math.log1p(math.exp(z0 - z1))) < 1e-13


def test_shift_invariance_and_dominant_logit():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((3, 50))
    t = np.array([4, 0, 49])
    assert np.allclose(oracle.token_ce(z, t), oracle.token_ce(z + 123.0, t), atol=1e-12)
    big = np.zeros((1, 1000))
    big[0, 7] = 1000.0
    assert oracle.token_ce(big, [7])[0] == 0.0
    assert abs(oracle.token_ce(big, [3])[0] - 1000.0) < 1e-9


def test_decay_weights():
    w = oracle.position_weights(10, 4, 3.0)
    k = np.arange(10) % 4
    assert w[1] == 1.0 and w[5] == 1.0
    assert abs(w[2] - math.exp(-1 / 3.0)) < 1e-15 and abs(w[7] - math.exp(-2 / 3.0)) < 1e-15
    assert (np.diff(w[1:4]) < 0).all()                      # earlier positions weigh more
    assert np.allclose(w, np.exp(-(k - 1) / 3.0))


def test_decayed_mean_two_rows_and_limits():
    rng = np.random.default_rng(2)
    V, H, bs, tau = 20, 6, 4, 2.5
    h = rng.standard_normal((bs, H))
    W = rng.standard_normal((V, H))
    t = rng.integers(0, V, bs)
    ce_all = oracle.lm_head_ce_rows(h, W, t)
    ce, loss = oracle.lm_head_ce(h, W, t, np.array([0, 1, 1, 0]), bs, tau)
    a = math.exp(-1.0 / tau)
    assert abs(loss - (ce_all[1] + a * ce_all[2]) / (1 + a)) < 1e-12
    assert ce[0] == 0.0 and ce[3] == 0.0 and abs(ce[1] - ce_all[1]) < 1e-12
    _, plain = oracle.lm_head_ce(h, W, t, np.array([0, 1, 1, 1]), bs, 1e300)   # no decay: plain mean
    assert abs(plain - ce_all[1:].mean()) < 1e-12
    ce0, zero = oracle.lm_head_ce(h, W, t, np.zeros(bs), bs, tau)
    assert zero == 0.0 and (ce0 == 0).all()


def _ce_case(seed):
    rng = np.random.default_rng(seed)
    rows, H, V, bs = 12, 6, 9, 4
    h = rng.standard_normal((rows, H))
    W = rng.standard_normal((V, H))
    t = rng.integers(0, V, rows)
    t[5] = V + 3                                 # a target outside the vocabulary: the row does not count
    m = np.ones(rows, np.uint8)
    m[[0, 4, 8]] = 0                             # the anchors of the three blocks
    return h, W, t, m, bs, 2.5


def test_ce_backward_matches_finite_differences():
    h, W, t, m, bs, tau = _ce_case(0)
    g = oracle.lm_head_ce_backward(h, W, t, m, bs, tau)
    eps = 1e-6
    for i in range(h.size):
        flat = h.reshape(-1)
        old = flat[i]
        flat[i] = old + eps
        lp = oracle.lm_head_ce(h, W, t, m, bs, tau)[1]
        flat[i] = old - eps
        lm = oracle.lm_head_ce(h, W, t, m, bs, tau)[1]
        flat[i] = old
        assert abs((lp - lm) / (2 * eps) - g.reshape(-1)[i]) < 1e-8, i
    assert (g[[0, 4, 5, 8]] == 0).all()          # rows that do not count pass nothing back


def test_ce_backward_closed_forms():
    h, W, t, m, bs, tau = _ce_case(1)
    g = oracle.lm_head_ce_backward(h, W, t, m, bs, tau)
    assert np.allclose(oracle.lm_head_ce_backward(h, W, t, m, bs, tau, d_loss=-3.0), -3.0 * g, rtol=1e-13, atol=0)
    # One selected row, identity head (vocabulary = hidden): dL/dh = p - onehot(t), exactly the softmax
    # gradient, since z = h.
    H = 5
    hh = np.array([[0.2, -1.0, 0.7, 0.0, 1.5]])
    gi = oracle.lm_head_ce_backward(hh, np.eye(H), np.array([2]), np.array([1]), 4, 1.0)
    p = np.exp(hh[0]) / np.exp(hh[0]).sum()
    p[2] -= 1.0
    assert np.allclose(gi[0], p, rtol=0, atol=1e-15)
    # Nothing selected: zero gradient.
    assert (oracle.lm_head_ce_backward(h, W, t, np.zeros_like(m), bs, tau) == 0).all()
