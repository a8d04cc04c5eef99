"""dflash_adamw_step vs oracle.adamw_step (the optimizer step after the body's
backward; NeMo RL "DFlash Draft Body", How It Works, step 1; AdamW as published,
the reading taken for the optimizer the pages leave unnamed).

Tolerance: every operation of the update is one fp32 rounding of an fp64
quantity (a few units of 2^-24 each), so after three steps the master weights
and both moments agree with the fp64 oracle to rel-L2 1e-6 and to 1e-6 of each
tensor's largest magnitude. The working copy is the master rounded to its dtype,
bit for bit (round to nearest even on both sides)."""
import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle
from tests.helpers import np64

pytestmark = pytest.mark.gpu
HP = dict(lr=3e-3, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.05)


def _cmp(gpu, ref, what):
    g = np64(gpu)
    err = g - ref
    scale = float(np.abs(ref).max()) or 1.0
    rel = float(np.sqrt((err * err).sum()) / (np.sqrt((ref * ref).sum()) or 1.0))
    assert rel <= 1e-6, f"{what}: rel-L2 {rel:.3e}"
    assert float(np.abs(err).max()) <= 1e-6 * scale, f"{what}: max-abs {np.abs(err).max():.3e}"


def _run(sizes, dtype, steps=3, copies=True, seed=0):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    tdt = torch.bfloat16 if dtype == d.DFLASH_BF16 else torch.float32
    ts, refs = [], []
    for i, n in enumerate(sizes):
        w0 = torch.randn(n, generator=gen, device="cuda")
        t = {"master": w0.clone(), "exp_avg": torch.zeros(n, device="cuda"),
             "exp_avg_sq": torch.zeros(n, device="cuda"), "grad": torch.empty(n, device="cuda")}
        if copies and i % 3 != 2:                    # some tensors keep no working copy
            t["weight"] = torch.full((n,), float("nan"), device="cuda", dtype=tdt)
        ts.append(t)
        refs.append([np64(w0), np.zeros(n), np.zeros(n)])
    for step in range(1, steps + 1):
        for t, r in zip(ts, refs):
            n = t["master"].numel()
            g = torch.randn(n, generator=gen, device="cuda") * (0.1 if step % 2 else 10.0)
            if n > 5:
                g[::5] = 0.0                         # zero gradients: decay only, no division by zero
            t["grad"].copy_(g)
            r[0], r[1], r[2] = oracle.adamw_step(r[0], np64(g), r[1], r[2], step, **HP)
        d.dflash_adamw_step(dtype, ts, step=step, **HP)
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(ts, refs)):
            if t["master"].numel() == 0:
                continue
            _cmp(t["master"], r[0], f"tensor {i} master, step {step}")
            _cmp(t["exp_avg"], r[1], f"tensor {i} exp_avg, step {step}")
            _cmp(t["exp_avg_sq"], r[2], f"tensor {i} exp_avg_sq, step {step}")
            if "weight" in t:
                assert torch.equal(t["weight"], t["master"].to(tdt)), f"tensor {i} working copy, step {step}"


@pytest.mark.parametrize("dtype", [d.DFLASH_BF16, d.DFLASH_F32])
def test_ragged_tensors_three_steps(dtype):
    # Empty, shorter than a vector, a vector tail, one and several workgroups.
    _run([0, 1, 3, 4, 7, 2048, 4096, 4097, 3 * 4096 + 5, 300001], dtype)


def test_many_tensors_over_several_launches():
    # More tensors than one launch carries, with working copies on most of them.
    _run([1000 + 37 * i for i in range(21)], d.DFLASH_BF16, steps=2, seed=1)


def test_no_working_copies_and_nothing_to_do():
    _run([513, 4096], d.DFLASH_BF16, steps=2, copies=False, seed=2)
    d.dflash_adamw_step(d.DFLASH_BF16, [], step=1, **HP)
    torch.cuda.synchronize()
