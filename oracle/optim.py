"""AdamW update of the draft's trainable tensors -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
the oracle; the HIP library never calls it and shares no code with it.

NeMo RL "DFlash Draft Body", How It Works, step 1, and Scope: the draft body is
trained, one optimizer step after each backward. The pages name no optimizer.
The reading taken is AdamW: Adam's moment estimates with bias correction
(Kingma and Ba, "Adam: A Method for Stochastic Optimization", ICLR 2015,
Algorithm 1) with the weight decay decoupled from the gradient (Loshchilov and
Hutter, "Decoupled Weight Decay Regularization", ICLR 2019, Algorithm 2),
applied in the order PyTorch's torch.optim.AdamW uses: the decay first, then
the moments, then the step. Plain numpy in fp64.
"""
from __future__ import annotations

import numpy as np


def adamw_step(w, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float):
    """One update at step number `step` (1 for the first) of weights w with
    gradient g and moment estimates m, v; returns the new (w, m, v) in fp64."""
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    w = w * (1.0 - lr * weight_decay)                 # decoupled weight decay
    m = beta1 * m + (1.0 - beta1) * g                 # first moment
    v = beta2 * v + (1.0 - beta2) * g * g             # second (raw) moment
    m_hat = m / (1.0 - beta1 ** step)                 # bias corrections
    v_hat = v / (1.0 - beta2 ** step)
    w = w - lr * m_hat / (np.sqrt(v_hat) + eps)
    return w, m, v
