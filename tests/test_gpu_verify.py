"""dflash_verify_greedy / dflash_verify_sample vs the verification oracle
(cooking-agi deep dive "DFlash: drafting, verification, and speed": greedy
verification and its worked example; speculative sampling's acceptance and
[p - q]_+ redraw), at the inference shape (64 requests, gamma 15, vocabulary
151936) and on edge cases. Token outputs are integers: bit-exact, except that
a draw whose target lands within rounding of a CDF boundary may pick either
neighbour (both are valid; checked)."""
import json
import os

import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
VOCAB = 151936


def _outs(B, g, dev="cuda"):
    return (torch.full((B, g + 1), -7, dtype=torch.int32, device=dev),
            torch.full((B,), -7, dtype=torch.int32, device=dev), torch.full((B,), -7, dtype=torch.int32, device=dev))


def _greedy(draft, logits, eos=-1):
    B, g1, _ = logits.shape
    em, num, acc = _outs(B, g1 - 1)
    d.dflash_verify_greedy(draft, logits, em, num, acc, eos_token=eos)
    torch.cuda.synchronize()
    return em.cpu().numpy(), num.cpu().numpy(), acc.cpu().numpy()


def test_greedy_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "verify_greedy_example.json")))
    V = 128
    logits = torch.zeros((1, 5, V), dtype=torch.float32)
    for i, c in enumerate(g["target_choices"]):
        logits[0, i, c] = 1.0
    draft = torch.tensor([g["draft"]], dtype=torch.int32, device="cuda")
    em, num, acc = _greedy(draft, logits.cuda())
    assert em[0, :num[0]].tolist() == g["emitted"] and acc[0] == g["accepted"]
    assert (em[0, num[0]:] == -1).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_greedy_inference_shape(dtype):
    B, g, V = 64, 15, VOCAB
    gen = torch.Generator(device="cuda").manual_seed(11)
    logits = torch.randn((B, g + 1, V), generator=gen, device="cuda").to(dtype)
    choices = oracle.target_choices_from_logits(logits.float().cpu().numpy())
    rng = np.random.default_rng(12)
    n = rng.integers(0, g + 1, size=B)
    draft = rng.integers(0, V, size=(B, g))
    for b in range(B):
        draft[b, :n[b]] = choices[b, :n[b]]
        if n[b] < g and draft[b, n[b]] == choices[b, n[b]]:
            draft[b, n[b]] = (choices[b, n[b]] + 1) % V
    em, num, acc = _greedy(torch.tensor(draft, dtype=torch.int32, device="cuda"), logits)
    ref_em, ref_num, ref_acc = oracle.verify_greedy(draft, logits.float().cpu().numpy())
    assert np.array_equal(acc, ref_acc) and np.array_equal(acc, n)
    assert np.array_equal(num, ref_num) and np.array_equal(em, ref_em)


def test_greedy_ties_eos_and_small_shapes():
    rng = np.random.default_rng(13)
    for B, g, V, eos in [(7, 5, 3, -1), (5, 6, 9, 2), (3, 0, 4, -1), (4, 3, 1, -1), (9, 8, 1000, 5)]:
        logits = rng.integers(-2, 3, size=(B, g + 1, V)).astype(np.float32)   # many exact ties
        choices = oracle.target_choices_from_logits(logits)
        draft = choices[:, :g].copy() if g else np.zeros((B, 0), np.int64)
        for b in range(B):
            if g and rng.random() < 0.6:
                k = rng.integers(0, g)
                draft[b, k] = rng.integers(0, V)
        em, num, acc = _greedy(torch.tensor(draft, dtype=torch.int32, device="cuda"),
                               torch.tensor(logits, device="cuda"), eos)
        ref = oracle.verify_greedy(draft, logits, None if eos < 0 else eos)
        assert np.array_equal(em, ref[0]) and np.array_equal(num, ref[1]) and np.array_equal(acc, ref[2]), (B, g, V)


def _probs(gen, shape, temp):
    return torch.softmax(torch.randn(shape, generator=gen, device="cuda") * temp, dim=-1).float().contiguous()


def _sample(draft, p, q, ua, ud, eos=-1):
    B, g1, _ = p.shape
    em, num, acc = _outs(B, g1 - 1)
    d.dflash_verify_sample(draft, p, q, ua, ud, em, num, acc, eos_token=eos)
    torch.cuda.synchronize()
    return em.cpu().numpy(), num.cpu().numpy(), acc.cpu().numpy()


def _check_sample(draft, p, q, ua, ud, eos=-1):
    em, num, acc = _sample(torch.tensor(draft, dtype=torch.int32, device="cuda"), p, q, ua, ud, eos)
    P, Q = p.cpu().numpy(), q.cpu().numpy()
    UA, UD = ua.cpu().numpy(), ud.cpu().numpy()
    ref_em, ref_num, ref_acc, infos = oracle.verify_sample(draft, P, Q, UA, UD, None if eos < 0 else eos)
    assert np.array_equal(acc, ref_acc) and np.array_equal(num, ref_num)
    for b in range(draft.shape[0]):
        k = num[b] - 1
        assert np.array_equal(em[b, :k], ref_em[b, :k]) and (em[b, num[b]:] == -1).all()
        if em[b, k] != ref_em[b, k]:
            # Only a draw may differ, and only across a boundary within fp64 rounding.
            w = infos[b]["weights"]
            csum = np.cumsum(w)
            t = float(UD[b]) * csum[-1]
            lo, hi = sorted((int(em[b, k]), int(ref_em[b, k])))
            assert w[em[b, k]] > 0 and abs(csum[lo] - t) <= 1e-12 * csum[-1], (b, lo, hi)
    return acc, infos


def test_sample_inference_shape():
    B, g, V = 64, 15, VOCAB
    gen = torch.Generator(device="cuda").manual_seed(21)
    p = _probs(gen, (B, g + 1, V), 3.0)
    q = _probs(gen, (B, g, V), 3.0)
    q[:8] = p[:8, :g]                                   # q = p: every proposal accepted -> bonus draws
    q[8:16] = 0.5 * q[8:16] + 0.5 * p[8:16, :g]         # close proposals: long accepted prefixes
    draft = torch.multinomial(q.reshape(-1, V), 1, generator=gen).reshape(B, g).cpu().numpy()
    ua = torch.rand((B, g), generator=gen, device="cuda")
    ud = torch.rand((B,), generator=gen, device="cuda")
    acc, infos = _check_sample(draft, p, q, ua, ud)
    kinds = {i["kind"] for i in infos}
    assert "bonus" in kinds and "residual" in kinds
    assert (acc[:8] == g).all()


def test_sample_edge_cases():
    gen = torch.Generator(device="cuda").manual_seed(31)
    # Disjoint supports: every proposal rejected; proposals outside the vocabulary rejected.
    V = 10
    p = torch.zeros((4, 3, V), device="cuda")
    p[:, :, 5:] = 0.2
    q = torch.zeros((4, 2, V), device="cuda")
    q[:, :, :5] = 0.2
    draft = np.array([[1, 2], [3, 4], [-1, 4], [V + 3, 0]])
    ua = torch.rand((4, 2), generator=gen, device="cuda")
    ud = torch.rand((4,), generator=gen, device="cuda")
    acc, infos = _check_sample(draft, p, q, ua, ud)
    assert (acc == 0).all()
    # gamma = 0: the bonus draw only; eos accepted first.
    p0 = _probs(gen, (6, 1, 50), 1.0)
    q0 = torch.zeros((6, 0, 50), device="cuda")
    _check_sample(np.zeros((6, 0), np.int64), p0, q0, torch.zeros((6, 0), device="cuda"),
                  torch.rand((6,), generator=gen, device="cuda"))
    p1 = _probs(gen, (5, 4, 30), 1.0)
    draft = np.array([[3, 7, 7], [7, 1, 2], [1, 2, 3], [7, 7, 7], [0, 0, 7]])
    ua = torch.zeros((5, 3), device="cuda")             # u = 0: accepted wherever p(y) > 0
    _check_sample(draft, p1, p1[:, :3].contiguous(), ua, torch.rand((5,), generator=gen, device="cuda"), eos=7)
    # [p - q]_+ = 0 at a rejected position (p = q there but u pushes past 1 is impossible,
    # so force a rejection with p(y) = 0 = q(y)): the draw falls back to p.
    p2 = torch.full((2, 2, 8), 0.125, device="cuda")
    p2[:, 0, 3] = 0.0
    p2[:, 0, 4] = 0.25
    q2 = p2[:, :1].clone()
    _check_sample(np.array([[3], [3]]), p2, q2, torch.zeros((2, 1), device="cuda"),
                  torch.tensor([0.1, 0.9], device="cuda"))


def test_sample_output_is_distributed_as_target():
    # The guarantee itself, on the GPU: 20000 one-proposal blocks with y ~ q.
    V, B = 6, 20000
    gen = torch.Generator(device="cuda").manual_seed(41)
    pv = torch.tensor([0.30, 0.05, 0.25, 0.0, 0.15, 0.25], device="cuda")
    qv = torch.tensor([0.10, 0.40, 0.10, 0.20, 0.10, 0.10], device="cuda")
    p = pv.expand(B, 2, V).contiguous()
    q = qv.expand(B, 1, V).contiguous()
    draft = torch.multinomial(qv.expand(B, V), 1, replacement=True, generator=gen).to(torch.int32)
    ua = torch.rand((B, 1), generator=gen, device="cuda")
    ud = torch.rand((B,), generator=gen, device="cuda")
    em, num, acc = _sample(draft, p, q, ua, ud)
    counts = np.bincount(em[:, 0], minlength=V).astype(np.float64)
    exp = pv.cpu().numpy().astype(np.float64) * B
    assert counts[3] == 0                               # p = 0: never emitted
    keep = exp > 0
    chi2 = float((((counts - exp) ** 2)[keep] / exp[keep]).sum())
    dof = int(keep.sum()) - 1
    assert chi2 < dof + 6.0 * np.sqrt(2.0 * dof), counts / B
