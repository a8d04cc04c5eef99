"""Writes tests/golden/c1_plan.json using the oracle only.

The tiny fp32 workload (batch 1, target seq 128, block 8, 4 anchors) asks for
one anchor drawn near the sequence end, so that overflow positions are
invalid. The plan stays a pure function of (mask, sample id, step, seed): the
seed used is the smallest seed >= 0 (sample id 0, step 0, all-valid mask)
whose plan has an anchor >= S - block_size + 1.
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import build_plan  # noqa: E402

S, BS, N = 128, 8, 4


def main():
    mask = np.ones((1, S), np.uint8)
    seed = 0
    while True:
        anchors = build_plan(mask, [0], 0, seed, N, BS)[0]
        if anchors.max() >= S - BS + 1:
            break
        seed += 1
    anchors, positions, valid, loss, num = build_plan(mask, [0], 0, seed, N, BS)
    out = dict(seq_len=S, block_size=BS, anchors_per_row=N, sample_id=0, step=0, seed=seed,
               anchors=anchors.tolist(), valid=valid.tolist(), loss_mask=loss.tolist())
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_plan.json")
    with open(path, "w") as f:
        json.dump(out, f)
        f.write("\n")
    print(path, seed, anchors.tolist())


if __name__ == "__main__":
    main()
