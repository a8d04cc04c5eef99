"""Verification oracle (test infrastructure only; see the package docstring).

Follows the cooking-agi deep dive "DFlash: drafting, verification, and speed":
  * "Why can't later correct guesses simply stay?" -- greedy verification keeps
    the longest prefix of the draft that agrees with the target's choices; at
    the first disagreement the target's own choice is emitted instead and the
    cycle ends; when every proposal agrees, the target's extra (bonus) choice
    after the block is emitted too. An accepted end-of-sequence token ends the
    cycle without a bonus. The page's worked example pins this.
  * "Sampling with temperature is not argmax matching" -- speculative
    sampling accepts a proposal y ~ q with probability min(1, p(y)/q(y)); on
    rejection a replacement is drawn from [p - q]_+ renormalised.

Readings taken where the pages leave a step open (the HIP kernels implement
the same readings, written separately there):
  * the target's choice at a position is the argmax of its logits, ties going
    to the smallest token id;
  * random numbers are inputs: u_accept[i] in [0, 1) decides proposal i
    (accepted iff u_accept[i] * q(y) < p(y), with the product rounded to fp32,
    which is min(1, p/q) > u without a division); u_draw in [0, 1) drives the
    one draw a cycle makes (the replacement, or the bonus token when every
    proposal is accepted);
  * a draw from weights w over the vocabulary returns the smallest token t
    whose running sum of w exceeds u_draw * sum(w) (inverse CDF); when
    [p - q]_+ sums to zero the replacement is drawn from p;
  * the bonus token after a fully accepted block is drawn from p at the
    position after the block;
  * a proposal outside the vocabulary is rejected.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


def verify_greedy_block(draft: Sequence[int], target_choices: Sequence[int],
                        eos_token: Optional[int] = None) -> Tuple[List[int], int]:
    """Emitted tokens and number of accepted proposals for one block.

    target_choices[i] is the target's choice after the prefix ending at draft
    position i - 1; the last entry is the bonus choice after the whole block.
    accepted n = length of the longest prefix on which draft and choices agree;
    emitted = that prefix followed by the target's choice right after it (the
    replacement, or the bonus when n = gamma). If the kept prefix holds the
    end-of-sequence token, everything after its first occurrence is dropped."""
    if len(target_choices) != len(draft) + 1:
        raise ValueError("one target choice per proposal, plus the bonus choice")
    g = len(draft)
    agree = [int(draft[i]) == int(target_choices[i]) for i in range(g)]
    n = agree.index(False) if False in agree else g
    kept = [int(t) for t in draft[:n]]
    if eos_token is not None and eos_token in kept:
        e = kept.index(eos_token) + 1
        return kept[:e], e
    return kept + [int(target_choices[n])], n


def target_choices_from_logits(logits: np.ndarray) -> np.ndarray:
    """argmax over the vocabulary (first index among equal maxima), per position."""
    return np.argmax(np.asarray(logits, dtype=np.float64), axis=-1)


def verify_greedy(draft: np.ndarray, logits: np.ndarray, eos_token: Optional[int] = None):
    """Batched greedy verification: draft [B, gamma], logits [B, gamma + 1, V].
    Returns (emitted [B, gamma + 1] padded with -1, num_emitted [B], accepted [B])."""
    draft = np.asarray(draft)
    B, g = draft.shape
    choices = target_choices_from_logits(logits)
    emitted = np.full((B, g + 1), -1, dtype=np.int64)
    num = np.zeros(B, dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    for b in range(B):
        out, a = verify_greedy_block(draft[b].tolist(), choices[b].tolist(), eos_token)
        emitted[b, :len(out)] = out
        num[b], acc[b] = len(out), a
    return emitted, num, acc


def inverse_cdf_draw(weights: np.ndarray, u: float) -> int:
    """Smallest t with sum(weights[:t + 1]) > u * sum(weights), in fp64."""
    w = np.asarray(weights, dtype=np.float64)
    csum = np.cumsum(w)
    total = csum[-1]
    target = float(u) * total
    return int(np.searchsorted(csum, target, side="right"))


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """[p - q]_+ in fp64 (unnormalised; the draw normalises)."""
    return np.maximum(np.asarray(p, np.float64) - np.asarray(q, np.float64), 0.0)


def accept_proposal(u: float, p_y: float, q_y: float) -> bool:
    """min(1, p(y)/q(y)) > u, evaluated as fp32(u * q(y)) < p(y)."""
    return bool(np.float32(np.float32(u) * np.float32(q_y)) < np.float32(p_y))


def verify_sample_block(draft: Sequence[int], p: np.ndarray, q: np.ndarray, u_accept: Sequence[float],
                        u_draw: float, eos_token: Optional[int] = None) -> Tuple[List[int], int, dict]:
    """One block of speculative sampling. p [gamma + 1, V] target probabilities,
    q [gamma, V] proposal probabilities. Returns (emitted, accepted, info) where
    info names the distribution the last token came from (for the tests)."""
    emitted: List[int] = []
    g = len(draft)
    V = p.shape[-1]
    for i in range(g):
        y = int(draft[i])
        if 0 <= y < V and accept_proposal(u_accept[i], p[i, y], q[i, y]):
            emitted.append(y)
            if eos_token is not None and y == eos_token:
                return emitted, i + 1, {"kind": "eos", "position": i}
            continue
        w = residual_weights(p[i], q[i])
        if w.sum() > 0.0:
            emitted.append(inverse_cdf_draw(w, u_draw))
            return emitted, i, {"kind": "residual", "position": i, "weights": w}
        w = np.asarray(p[i], np.float64)
        emitted.append(inverse_cdf_draw(w, u_draw))
        return emitted, i, {"kind": "p", "position": i, "weights": w}
    w = np.asarray(p[g], np.float64)
    emitted.append(inverse_cdf_draw(w, u_draw))
    return emitted, g, {"kind": "bonus", "position": g, "weights": w}


def verify_sample(draft: np.ndarray, p: np.ndarray, q: np.ndarray, u_accept: np.ndarray, u_draw: np.ndarray,
                  eos_token: Optional[int] = None):
    """Batched speculative sampling: draft [B, gamma], p [B, gamma + 1, V], q [B, gamma, V],
    u_accept [B, gamma], u_draw [B]. Returns (emitted [B, gamma + 1] padded with -1,
    num_emitted [B], accepted [B], infos)."""
    draft = np.asarray(draft)
    B, g = draft.shape
    emitted = np.full((B, g + 1), -1, dtype=np.int64)
    num = np.zeros(B, dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    infos = []
    for b in range(B):
        out, a, info = verify_sample_block(draft[b].tolist(), p[b], q[b], u_accept[b], float(u_draw[b]),
                                           eos_token)
        emitted[b, :len(out)] = out
        num[b], acc[b] = len(out), a
        infos.append(info)
    return emitted, num, acc, infos
