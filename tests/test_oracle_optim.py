"""Pins of oracle.adamw_step (the optimizer step after the body's backward;
NeMo RL "DFlash Draft Body", How It Works, step 1; AdamW as published by
Loshchilov and Hutter with Kingma and Ba's bias correction).

Each check is a closed form the update must reduce to, chosen so that the
plausible mistakes (no bias correction, weight decay coupled into the gradient,
swapped moment rates, eps under the square root, decay applied after the step)
each fail one of them; test_planted_mistakes_are_caught plants them."""
import inspect
import re

import numpy as np
import pytest

import oracle.optim as optim

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def test_first_step_is_a_normalised_sign_step():
    # m_hat = g and v_hat = g^2 after one step: w1 = w0 - lr g / (|g| + eps);
    # gradients near eps show eps added outside the square root.
    rng = np.random.default_rng(0)
    w0 = rng.normal(size=64)
    g = rng.normal(size=64) * np.array([1.0, 1e-8, 3e-8, 1e3] * 16)
    w1, m, v = optim.adamw_step(w0, g, np.zeros(64), np.zeros(64), 1, LR, B1, B2, EPS, 0.0)
    np.testing.assert_allclose(w1, w0 - LR * g / (np.abs(g) + EPS), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, (1 - B1) * g, rtol=1e-15)
    np.testing.assert_allclose(v, (1 - B2) * g * g, rtol=1e-15)


def test_decay_alone_scales_the_weights():
    # g = 0: the moments stay zero and only the decoupled decay acts.
    w0 = np.linspace(-2, 2, 33)
    w1, m, v = optim.adamw_step(w0, np.zeros(33), np.zeros(33), np.zeros(33), 1, LR, B1, B2, EPS, 0.1)
    np.testing.assert_array_equal(m, 0)
    np.testing.assert_array_equal(v, 0)
    np.testing.assert_allclose(w1, w0 * (1 - LR * 0.1), rtol=1e-15, atol=0)


def test_constant_gradient_moves_a_fixed_amount_each_step():
    # Bias correction makes m_hat = g and v_hat = g^2 exactly under a constant
    # gradient, whatever the step: T steps move by T lr g / (|g| + eps).
    g = np.array([0.5, -2.0, 1e-3])
    w, m, v = np.zeros(3), np.zeros(3), np.zeros(3)
    for t in range(1, 8):
        w, m, v = optim.adamw_step(w, g, m, v, t, LR, B1, B2, EPS, 0.0)
    np.testing.assert_allclose(w, -7 * LR * g / (np.abs(g) + EPS), rtol=1e-12)


def test_two_steps_weigh_the_gradients_by_their_rates():
    # After g1 then g2: m_hat = (b1 g1 + g2) / (1 + b1), v_hat = (b2 g1^2 + g2^2) / (1 + b2).
    b1, b2 = 0.5, 0.75
    g1, g2 = np.array([1.0, -3.0]), np.array([4.0, 2.0])
    w, m, v = optim.adamw_step(np.zeros(2), g1, np.zeros(2), np.zeros(2), 1, 1.0, b1, b2, 0.0, 0.0)
    w2, _, _ = optim.adamw_step(np.zeros(2), g2, m, v, 2, 1.0, b1, b2, 0.0, 0.0)
    m_hat = (b1 * g1 + g2) / (1 + b1)
    v_hat = (b2 * g1 ** 2 + g2 ** 2) / (1 + b2)
    np.testing.assert_allclose(w2, -m_hat / np.sqrt(v_hat), rtol=1e-14)


def test_decay_comes_before_the_step():
    # One step with both: w1 = w0 (1 - lr wd) - lr g / (|g| + eps).
    w0, g = np.array([3.0, -1.0]), np.array([0.2, 0.7])
    w1, _, _ = optim.adamw_step(w0, g, np.zeros(2), np.zeros(2), 1, 0.1, B1, B2, EPS, 0.5)
    np.testing.assert_allclose(w1, w0 * (1 - 0.05) - 0.1 * g / (np.abs(g) + EPS), rtol=1e-14)


PLANTS = {
    "no bias correction": [("m_hat = m / (1.0 - beta1 ** step)", "m_hat = m")],
    "decay coupled into the gradient": [("w = w * (1.0 - lr * weight_decay)", "g = g + weight_decay * w")],
    "swapped moment rates": [("m = beta1 * m + (1.0 - beta1) * g", "m = beta2 * m + (1.0 - beta2) * g")],
    "eps under the square root": [("np.sqrt(v_hat) + eps", "np.sqrt(v_hat + eps)")],
    "decay after the step": [("w = w * (1.0 - lr * weight_decay)", "pass"),
                             ("return w, m, v", "return w * (1.0 - lr * weight_decay), m, v")],
}


@pytest.mark.parametrize("name", sorted(PLANTS))
def test_planted_mistakes_are_caught(name):
    src = inspect.getsource(optim)
    for old, new in PLANTS[name]:
        assert old in src
        src = src.replace(old, new)
    ns = {}
    exec(compile(src, "planted_optim", "exec"), ns)
    bad = ns["adamw_step"]
    saved = optim.adamw_step
    optim.adamw_step = bad
    try:
        failed = 0
        for test in (test_first_step_is_a_normalised_sign_step, test_decay_alone_scales_the_weights,
                     test_constant_gradient_moves_a_fixed_amount_each_step,
                     test_two_steps_weigh_the_gradients_by_their_rates, test_decay_comes_before_the_step):
            try:
                test()
            except AssertionError:
                failed += 1
        assert failed > 0, f"planted mistake not caught: {name}"
    finally:
        optim.adamw_step = saved
