"""Pins of the verification oracle (cooking-agi deep dive "DFlash: drafting,
verification, and speed": greedy verification and its worked example, and
speculative sampling's acceptance / [p - q]_+ replacement rule)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_worked_example_from_the_page():
    g = json.load(open(os.path.join(HERE, "golden", "verify_greedy_example.json")))
    emitted, accepted = oracle.verify_greedy_block(g["draft"], g["target_choices"])
    assert emitted == g["emitted"] and accepted == g["accepted"]


@pytest.mark.parametrize("gamma", [0, 1, 2, 3, 4])
def test_greedy_brute_force_characterisation(gamma):
    # Every block over a 3-token vocabulary. The output is pinned by properties
    # that determine it uniquely: the kept proposals agree with the target, the
    # first disagreement (if any) ends the block, and the emitted tokens are the
    # target's choices up to and including the one after the kept prefix.
    for draft in itertools.product(range(3), repeat=gamma):
        for choices in itertools.product(range(3), repeat=gamma + 1):
            out, n = oracle.verify_greedy_block(list(draft), list(choices))
            assert 0 <= n <= gamma
            assert list(draft[:n]) == list(choices[:n])
            assert n == gamma or draft[n] != choices[n]
            assert out == list(choices[:n + 1])


def test_greedy_eos_ends_the_block_without_bonus():
    out, n = oracle.verify_greedy_block([5, 7, 9], [5, 7, 9, 4], eos_token=7)
    assert out == [5, 7] and n == 2
    out, n = oracle.verify_greedy_block([5, 8, 9], [5, 7, 9, 4], eos_token=8)   # eos proposed but rejected
    assert out == [5, 7] and n == 1
    out, n = oracle.verify_greedy_block([5, 7, 9], [5, 7, 9, 4], eos_token=3)
    assert out == [5, 7, 9, 4] and n == 3
    with pytest.raises(ValueError):
        oracle.verify_greedy_block([1, 2], [1, 2])


def test_argmax_takes_the_first_of_equal_maxima():
    logits = np.array([[0.5, 2.0, 2.0, -1.0], [3.0, 3.0, 3.0, 3.0], [-5.0, -4.0, -4.5, -4.0]])
    assert oracle.target_choices_from_logits(logits).tolist() == [1, 0, 1]


def test_inverse_cdf_draw_definition():
    w = np.array([0.0, 0.2, 0.0, 0.5, 0.3])
    assert oracle.inverse_cdf_draw(w, 0.0) == 1                 # first token with positive weight
    assert oracle.inverse_cdf_draw(w, 0.199) == 1
    assert oracle.inverse_cdf_draw(w, 0.2) == 3                 # the boundary belongs to the next token
    assert oracle.inverse_cdf_draw(w, 0.7 - 1e-9) == 3
    assert oracle.inverse_cdf_draw(w, 0.999999) == 4
    assert oracle.inverse_cdf_draw(w * 7.0, 0.5) == 3           # unnormalised weights
    rng = np.random.default_rng(0)
    for _ in range(200):                                        # linear scan on random cases
        w = rng.random(9) * (rng.random(9) < 0.7)
        if w.sum() == 0:
            continue
        u = rng.random()
        acc, t = 0.0, None
        for i, x in enumerate(w):
            acc += x
            if acc > u * w.sum():
                t = i
                break
        assert oracle.inverse_cdf_draw(w, u) == t
        assert w[t] > 0


def _chi2_ok(counts, probs, n):
    exp = probs * n
    keep = exp > 0
    assert counts[~keep].sum() == 0                             # impossible tokens never appear
    chi2 = float((((counts - exp) ** 2)[keep] / exp[keep]).sum())
    dof = int(keep.sum()) - 1
    return chi2 < dof + 6.0 * np.sqrt(2.0 * dof)                 # ~4 sigma


@pytest.mark.parametrize("case", ["random", "disjoint", "peaked"])
def test_speculative_sampling_emits_target_distribution(case):
    # The guarantee the page's acceptance rule exists for: with y ~ q accepted
    # with probability min(1, p(y)/q(y)) and replacements drawn from
    # [p - q]_+, the first emitted token is distributed exactly as p.
    rng = np.random.default_rng({"random": 1, "disjoint": 2, "peaked": 3}[case])
    V = 6
    if case == "random":
        p, q = rng.random(V), rng.random(V)
    elif case == "disjoint":
        p = np.array([0.0, 0.0, 0.0, 0.5, 0.3, 0.2])
        q = np.array([0.4, 0.4, 0.2, 0.0, 0.0, 0.0])
    else:
        p = np.array([0.9, 0.02, 0.02, 0.02, 0.02, 0.02])
        q = np.array([0.02, 0.02, 0.02, 0.02, 0.02, 0.9])
    p = (p / p.sum()).astype(np.float32)
    q = (q / q.sum()).astype(np.float32)
    n = 40000
    ys = rng.choice(V, size=n, p=q.astype(np.float64) / q.astype(np.float64).sum())
    ua = rng.random(n).astype(np.float32)
    ud = rng.random(n).astype(np.float32)
    P = np.stack([p, p])                                          # gamma = 1: position 0 and the bonus
    Q = q[None, :]
    counts = np.zeros(V)
    for t in range(n):
        out, _, _ = oracle.verify_sample_block([int(ys[t])], P, Q, [float(ua[t])], float(ud[t]))
        counts[out[0]] += 1
    assert _chi2_ok(counts, p.astype(np.float64), n), counts / n


def test_speculative_sampling_special_cases():
    V = 5
    p = np.array([[0.1, 0.2, 0.3, 0.25, 0.15]] * 3, np.float32)
    q = p[:2].copy()
    # q = p: every proposal is accepted, then the bonus comes from p at the last position.
    out, n, info = oracle.verify_sample_block([2, 4], p, q, [0.999, 0.5], 0.05)
    assert n == 2 and out[:2] == [2, 4] and info["kind"] == "bonus"
    assert out[2] == oracle.inverse_cdf_draw(p[2], 0.05) == 0
    # p(y) = 0: always rejected; the replacement never lands where p <= q.
    p2 = np.array([[0.0, 0.5, 0.5, 0.0, 0.0], [0.2] * 5], np.float32)
    q2 = np.array([[0.6, 0.4, 0.0, 0.0, 0.0]], np.float32)
    for u in np.linspace(0.0, 0.999, 25):
        out, n, info = oracle.verify_sample_block([0], p2, q2, [0.0], float(u))
        assert n == 0 and info["kind"] == "residual"
        assert out[0] in (1, 2) and p2[0, out[0]] > q2[0, out[0]]
    # An accepted end-of-sequence proposal ends the block with no draw.
    out, n, info = oracle.verify_sample_block([3, 1], p, q, [0.0, 0.0], 0.5, eos_token=3)
    assert out == [3] and n == 1 and info["kind"] == "eos"
    # Acceptance threshold: accepted iff u * q(y) < p(y).
    assert oracle.accept_proposal(0.5, 0.3, 0.6) is False         # 0.3 == 0.3: not strictly below
    assert oracle.accept_proposal(0.49, 0.3, 0.6) is True
    assert oracle.accept_proposal(0.0, 0.0, 0.6) is False
    assert oracle.accept_proposal(0.99, 0.7, 0.1) is True         # p > q: always accepted


def test_batched_forms_match_blockwise():
    rng = np.random.default_rng(4)
    B, g, V = 5, 3, 7
    logits = rng.standard_normal((B, g + 1, V))
    choices = oracle.target_choices_from_logits(logits)
    draft = choices[:, :g].copy()
    draft[1, 1] = (draft[1, 1] + 1) % V
    draft[3, 0] = (draft[3, 0] + 2) % V
    em, num, acc = oracle.verify_greedy(draft, logits)
    assert acc.tolist() == [3, 1, 3, 0, 3] and num.tolist() == [4, 2, 4, 1, 4]
    for b in range(B):
        out, a = oracle.verify_greedy_block(draft[b].tolist(), choices[b].tolist())
        assert em[b, :len(out)].tolist() == out and (em[b, len(out):] == -1).all()
