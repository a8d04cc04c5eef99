"""Anchor plan oracle (test infrastructure only; see the package docstring).

Follows NeMo RL "DFlash Draft Body", How It Works:
  step 1 -- an anchor is a valid position; the plan records which draft
            positions belong to each anchor; identical mask, sample ids,
            optimizer step and seed give an identical plan; rows with equal
            sample ids get equal anchors; a sample with no valid window
            contributes no draft loss;
  step 2 -- a block is one anchor followed by gamma draft positions;
  step 4 -- the loss mask leaves out the anchor and invalid positions.
and the angelspec "DFlash" page, How it works, "Anchor sampling": block starts
are sampled across the sequence.

The pages fix the properties, not the sampler. The reading used here (the one
the HIP kernel also implements, written separately there):
  * keys come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014): its increment-and-finalise
    step, applied to 64-bit words with wrap-around;
  * row key = mix(mix(mix(seed) xor sample_id) xor step), position key =
    mix(row key xor a) -- so the row's randomness depends only on
    (seed, sample id, step), never on the row index;
  * an anchor a is eligible when mask[a] and mask[a + 1] are both set
    (a valid window holds at least one valid draft position);
  * the n = min(N, #eligible) eligible positions with the smallest
    (key, position) pairs are chosen, then listed in ascending position order,
    padded with -1;
  * positions = a + k, valid = (a + k < S) and mask[a + k], loss_mask = valid
    and k >= 1; empty slots have position -1 and valid = loss_mask = 0.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(x: int) -> int:
    """One SplitMix64 output for state x: add the golden-ratio increment, then
    the two xor-shift-multiply rounds and the final xor-shift."""
    z = (int(x) + GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def _u64(v: int) -> int:
    """Two's-complement view of a signed 64-bit integer."""
    return int(v) & MASK64


def row_key(seed: int, sample_id: int, step: int) -> int:
    return splitmix64(splitmix64(splitmix64(_u64(seed)) ^ _u64(sample_id)) ^ _u64(step))


def position_key(rkey: int, a: int) -> int:
    return splitmix64(rkey ^ _u64(a))


def eligible_anchors(mask_row) -> list:
    m = [int(v) != 0 for v in mask_row]
    return [a for a in range(len(m) - 1) if m[a] and m[a + 1]]


def build_plan(mask, sample_ids, step: int, seed: int, anchors_per_row: int, block_size: int):
    """Returns (anchors [B,N] i32, positions [B,N,bs] i32, valid [B,N,bs] u8,
    loss_mask [B,N,bs] u8, num_anchors [B] i32)."""
    mask = np.asarray(mask)
    B, S = mask.shape
    N, bs = int(anchors_per_row), int(block_size)
    anchors = np.full((B, N), -1, dtype=np.int32)
    positions = np.full((B, N, bs), -1, dtype=np.int32)
    valid = np.zeros((B, N, bs), dtype=np.uint8)
    loss_mask = np.zeros((B, N, bs), dtype=np.uint8)
    num = np.zeros((B,), dtype=np.int32)
    for b in range(B):
        rk = row_key(seed, int(sample_ids[b]), step)
        ranked = sorted((position_key(rk, a), a) for a in eligible_anchors(mask[b]))
        chosen = sorted(a for _, a in ranked[:N])
        num[b] = len(chosen)
        for n, a in enumerate(chosen):
            anchors[b, n] = a
            for k in range(bs):
                p = a + k
                positions[b, n, k] = p
                ok = p < S and mask[b, p] != 0
                valid[b, n, k] = 1 if ok else 0
                loss_mask[b, n, k] = 1 if (ok and k >= 1) else 0
    return anchors, positions, valid, loss_mask, num
