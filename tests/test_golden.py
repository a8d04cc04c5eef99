"""Regression fixture for the tiny fp32 workload's plan, written by
tests/golden/make_golden.py from the oracle only."""
import json
import os

import numpy as np

from oracle import build_plan

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c1_plan_fixture():
    with open(os.path.join(HERE, "golden", "c1_plan.json")) as f:
        g = json.load(f)
    S, bs, N = g["seq_len"], g["block_size"], g["anchors_per_row"]
    anchors, _, valid, loss, _ = build_plan(np.ones((1, S), np.uint8), [g["sample_id"]], g["step"],
                                            g["seed"], N, bs)
    assert anchors.tolist() == g["anchors"]
    assert valid.tolist() == g["valid"] and loss.tolist() == g["loss_mask"]
    assert max(g["anchors"][0]) >= S - bs + 1          # one anchor overflows the sequence end
    for seed in range(g["seed"]):                       # and it is the smallest such seed
        a = build_plan(np.ones((1, S), np.uint8), [0], 0, seed, N, bs)[0]
        assert a.max() < S - bs + 1
