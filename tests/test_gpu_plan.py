"""GPU plan vs the oracle plan, bit-exact (NeMo RL "DFlash Draft Body", How It
Works, steps 1, 2 and 4)."""
import json
import os

import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _run(mask_np, ids_np, step, seed, N, bs):
    dev = "cuda"
    B, S = mask_np.shape
    mask = torch.from_numpy(mask_np.astype(np.uint8)).to(dev)
    ids = torch.from_numpy(np.asarray(ids_np, np.int64)).to(dev)
    a = torch.full((B, N), 7, dtype=torch.int32, device=dev)
    p = torch.full((B, N, bs), 7, dtype=torch.int32, device=dev)
    v = torch.full((B, N, bs), 7, dtype=torch.uint8, device=dev)
    lm = torch.full((B, N, bs), 7, dtype=torch.uint8, device=dev)
    num = torch.full((B,), 7, dtype=torch.int32, device=dev)
    base = torch.full((B * N,), 7, dtype=torch.int64, device=dev)
    d.dflash_build_plan(mask, ids, step, seed, N, bs, a, p, v, lm, num, base)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (a, p, v, lm, num, base)]


CASES = [
    # B, S, N, bs, fraction valid, step, seed
    (3, 40, 5, 4, 0.8, 3, 9),
    (2, 200, 16, 16, 1.0, 0, 0),
    (4, 25, 30, 3, 0.5, 1, 2),          # fewer eligible windows than N
    (1, 2, 3, 8, 1.0, 0, 5),            # shortest sequence with a window
    (2, 1, 2, 4, 1.0, 0, 5),            # no window at all
    (3, 5000, 64, 16, 0.97, 17, 123),   # several positions per thread
    (8, 4096, 32, 16, 1.0, 0, 0),       # 5-layer body workload shape
    (1, 32768, 512, 16, 1.0, 0, 0),     # long-context workload shape
    (2, 3000, 0, 16, 1.0, 0, 0),        # no anchors requested
    (2, 70000, 100, 1, 0.9, 5, 2 ** 64 - 1),
]


@pytest.mark.parametrize("B,S,N,bs,p_one,step,seed", CASES)
def test_plan_bit_exact(B, S, N, bs, p_one, step, seed):
    rng = np.random.default_rng(B * 7919 + S)
    mask = (rng.random((B, S)) < p_one).astype(np.uint8)
    ids = rng.integers(-50, 50, size=B)
    got = _run(mask, ids, step, seed, N, bs)
    ref = oracle.build_plan(mask, ids, step, seed, N, bs)
    for name, g, r in zip(("anchors", "positions", "valid", "loss_mask", "num_anchors"), got, ref):
        assert np.array_equal(g, r), name
    assert np.array_equal(got[5], np.repeat(np.arange(B) * S, N))


def test_plan_edge_rows_and_duplicate_ids():
    S = 300
    mask = np.ones((5, S), np.uint8)
    mask[1] = 0                          # no valid window
    mask[2, ::2] = 0                     # isolated valid positions: no window
    mask[3, :S - 2] = 0                  # a single window at the very end
    ids = np.array([7, 8, 9, 10, 7])     # rows 0 and 4 share an id and a mask
    got = _run(mask, ids, 4, 77, 10, 16)
    ref = oracle.build_plan(mask, ids, 4, 77, 10, 16)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    assert np.array_equal(got[0][0], got[0][4])
    assert got[4][1] == 0 and got[4][2] == 0 and got[4][3] == 1


def test_plan_tiny_fixture_and_determinism():
    with open(os.path.join(HERE, "golden", "c1_plan.json")) as f:
        g = json.load(f)
    S, bs, N = g["seq_len"], g["block_size"], g["anchors_per_row"]
    mask = np.ones((1, S), np.uint8)
    got = _run(mask, [g["sample_id"]], g["step"], g["seed"], N, bs)
    assert got[0].tolist() == g["anchors"]
    assert got[2].tolist() == g["valid"] and got[3].tolist() == g["loss_mask"]
    again = _run(mask, [g["sample_id"]], g["step"], g["seed"], N, bs)
    for x, y in zip(got, again):
        assert np.array_equal(x, y)
