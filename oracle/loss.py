"""Draft-loss oracle (test infrastructure only; see the package docstring).

Follows the angelspec "DFlash" page, How it works, "Loss": cross-entropy of the
draft's predictions against the ground-truth tokens, with an exponential
positional decay that gives earlier positions of a block more weight; the
same page, Configuration: the draft's lm_head comes from the target model. NeMo
RL "DFlash Draft Body", How It Works, step 4: the caller's loss mask leaves out
the anchor and invalid positions.

Readings taken where the pages leave a step open (the HIP kernels implement
the same readings, written separately there):
  * logits of a block row = h W_lm^T (the body's output row, no further norm;
    W_lm is [vocab, hidden]);
  * the weight of in-block position k is exp(-(k - 1) / tau), k = row index
    modulo block_size; tau is a caller parameter (the pages give no value), and
    the first draft position (k = 1) has weight 1;
  * the loss is the weighted mean sum(m w CE) / sum(m w) over rows with loss
    mask m = 1, and 0 when no row is selected.
"""
from __future__ import annotations

import math

import numpy as np


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """log(sum(exp(z))) along the last axis, shifted by the row maximum."""
    z = np.asarray(z, np.float64)
    mx = z.max(axis=-1, keepdims=True)
    return (mx + np.log(np.exp(z - mx).sum(axis=-1, keepdims=True)))[..., 0]


def token_ce(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Cross-entropy -log softmax(z)[y] = logsumexp(z) - z[y] per row."""
    z = np.asarray(logits, np.float64)
    t = np.asarray(targets, np.int64)
    return logsumexp_rows(z) - z[np.arange(z.shape[0]), t]


def position_weights(rows: int, block_size: int, tau: float) -> np.ndarray:
    k = np.arange(rows) % block_size
    return np.exp(-(k - 1.0) / float(tau))


def lm_head_ce(hidden: np.ndarray, lm_head: np.ndarray, targets: np.ndarray, loss_mask: np.ndarray,
               block_size: int, tau: float):
    """Per-row CE [rows] (0 where the mask is 0) and the decayed weighted-mean loss."""
    h = np.asarray(hidden, np.float64)
    W = np.asarray(lm_head, np.float64)
    m = np.asarray(loss_mask).astype(bool)
    ce = np.zeros(h.shape[0], np.float64)
    if m.any():
        ce[m] = token_ce(h[m] @ W.T, np.asarray(targets)[m])
    w = position_weights(h.shape[0], block_size, tau) * m
    den = w.sum()
    loss = float((w * ce).sum() / den) if den > 0 else 0.0
    return ce, loss


def lm_head_ce_rows(hidden_rows: np.ndarray, lm_head: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """CE of a few selected rows (no mask, no weights): for sampled checks."""
    z = np.asarray(hidden_rows, np.float64) @ np.asarray(lm_head, np.float64).T
    return token_ce(z, targets)
