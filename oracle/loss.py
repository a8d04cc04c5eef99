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
    mask m = 1, and 0 when no row is selected;
  * a row whose target lies outside the vocabulary does not count (m = 0).
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
    """Per-row CE [rows] (0 where the row does not count) and the decayed weighted-mean loss."""
    h = np.asarray(hidden, np.float64)
    W = np.asarray(lm_head, np.float64)
    t = np.asarray(targets, np.int64)
    m = np.asarray(loss_mask).astype(bool) & (t >= 0) & (t < W.shape[0])
    ce = np.zeros(h.shape[0], np.float64)
    if m.any():
        ce[m] = token_ce(h[m] @ W.T, t[m])
    w = position_weights(h.shape[0], block_size, tau) * m
    den = w.sum()
    loss = float((w * ce).sum() / den) if den > 0 else 0.0
    return ce, loss


def lm_head_ce_rows(hidden_rows: np.ndarray, lm_head: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """CE of a few selected rows (no mask, no weights): for sampled checks."""
    z = np.asarray(hidden_rows, np.float64) @ np.asarray(lm_head, np.float64).T
    return token_ce(z, targets)


def lm_head_ce_backward(hidden: np.ndarray, lm_head: np.ndarray, targets: np.ndarray, loss_mask: np.ndarray,
                        block_size: int, tau: float, d_loss: float = 1.0) -> np.ndarray:
    """Gradient of lm_head_ce's loss with respect to the hidden rows (angelspec
    "DFlash", Configuration: the LM head is the target's and stays frozen, so
    the hidden rows are what the loss differentiates). With c_r = m_r w_r / sum(m w)
    (0 for rows that do not count) and p_r = softmax(z_r):
        dL/dz_r      = d_loss c_r (p_r - onehot(targets[r]))
        dL/dhidden_r = dL/dz_r W_lm
    Rows whose target is outside [0, vocab) do not count (as in the forward)."""
    h = np.asarray(hidden, np.float64)
    W = np.asarray(lm_head, np.float64)
    t = np.asarray(targets, np.int64)
    V = W.shape[0]
    m = np.asarray(loss_mask).astype(bool) & (t >= 0) & (t < V)
    w = position_weights(h.shape[0], block_size, tau) * m
    den = w.sum()
    dh = np.zeros_like(h)
    if den <= 0:
        return dh
    rows = np.nonzero(m)[0]
    z = h[rows] @ W.T
    p = np.exp(z - logsumexp_rows(z)[:, None])
    p[np.arange(len(rows)), t[rows]] -= 1.0
    dz = (float(d_loss) * w[rows] / den)[:, None] * p
    dh[rows] = dz @ W
    return dh
