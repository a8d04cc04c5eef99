"""Backward of the dual-source block attention (test infrastructure only; see
the package docstring).

The forward it differentiates is block_attention / block_attn_call (NeMo RL
"DFlash Draft Body", How It Works, step 3: a block reads the target prefix
before its anchor and all positions of its own block; angelspec "DFlash",
How it works: the projected target states are attended alongside the draft
tokens' own K/V). Training runs the body with an optimizer step (NeMo RL,
DFlash Draft Body, Scope), so these gradients are what a training step
needs from this layer.

For one block and query head, with K, V the block's visible keys and values
(context rows before the anchor, then the block's own rows), s = q K^T / sqrt(D),
p = softmax(s), o = p V, and an upstream gradient dO of o:
    dV = p^T dO,  dp = dO V^T,  ds = p * (dp - rowsum(dO * o)),
    dq = ds K / sqrt(D),  dK = ds^T q / sqrt(D),
each key's dK and dV summed over every query head of its KV group (and, for
context rows, over every block that reads them). block_attn_call rotates q and
the block's k at anchor + k before this and zeroes the output rows of invalid
positions; its backward therefore drops dO on those rows and rotates dq and dk
back (RoPE is orthogonal: its transpose is the rotation by the opposite angle).
Context K gradients are returned in the rotated frame the cache stores.
"""
from __future__ import annotations

import math

import numpy as np

from .body import rope


def block_attention_backward(q, kb, vb, ctx_k, ctx_v, base, anchor, d_out):
    """q [nb, bs, Hq, D], kb / vb [nb, bs, Hkv, D] (q, kb rotated), ctx_k / ctx_v [Hkv, T, D],
    d_out [nb, bs, Hq, D]. Returns (dq, dkb, dvb, d_ctx_k, d_ctx_v) in the same shapes."""
    q = np.asarray(q, np.float64)
    kb = np.asarray(kb, np.float64)
    vb = np.asarray(vb, np.float64)
    ctx_k = np.asarray(ctx_k, np.float64)
    ctx_v = np.asarray(ctx_v, np.float64)
    dO = np.asarray(d_out, np.float64)
    nb, bs, Hq, D = q.shape
    Hkv = kb.shape[2]
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dkb = np.zeros_like(kb)
    dvb = np.zeros_like(vb)
    dck = np.zeros_like(ctx_k)
    dcv = np.zeros_like(ctx_v)
    scale = 1.0 / math.sqrt(D)
    for n in range(nb):
        a = int(anchor[n])
        if a < 0:
            continue
        b0 = int(base[n])
        for h in range(Hq):
            g = h // G
            K = np.concatenate([ctx_k[g, b0:b0 + a], kb[n, :, g]], axis=0)
            V = np.concatenate([ctx_v[g, b0:b0 + a], vb[n, :, g]], axis=0)
            s = q[n, :, h] @ K.T * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ V
            do = dO[n, :, h]
            dV = p.T @ do
            dp = do @ V.T
            ds = p * (dp - (do * o).sum(axis=1, keepdims=True))
            dq[n, :, h] = ds @ K * scale
            dK = ds.T @ q[n, :, h] * scale
            dck[g, b0:b0 + a] += dK[:a]
            dkb[n, :, g] += dK[a:]
            dcv[g, b0:b0 + a] += dV[:a]
            dvb[n, :, g] += dV[a:]
    return dq, dkb, dvb, dck, dcv


def block_attn_call_backward(q, k_blk, v_blk, ctx_k, ctx_v, base, anchor, valid, block_size: int,
                             num_q_heads: int, num_kv_heads: int, head_dim: int, theta: float, d_out):
    """Gradients of block_attn_call with respect to its inputs: q [R, Hq*D] and
    k_blk / v_blk [R, Hkv*D] before RoPE, ctx_k (rotated) / ctx_v [Hkv, T, D];
    d_out [R, Hq*D]. Returns (dq, dk_blk, dv_blk, d_ctx_k, d_ctx_v)."""
    R = q.shape[0]
    nb = R // block_size
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    q4 = np.asarray(q, np.float64).reshape(nb, block_size, Hq, D)
    k4 = np.asarray(k_blk, np.float64).reshape(nb, block_size, Hkv, D)
    v4 = np.asarray(v_blk, np.float64).reshape(nb, block_size, Hkv, D)
    pos = np.asarray(anchor, np.int64)[:, None] + np.arange(block_size)[None, :]
    qr = rope(q4, pos[:, :, None], theta)
    kr = rope(k4, pos[:, :, None], theta)
    keep = np.asarray(valid, bool).reshape(R) & np.repeat(np.asarray(anchor) >= 0, block_size)
    dO = np.where(keep[:, None], np.asarray(d_out, np.float64), 0.0).reshape(nb, block_size, Hq, D)
    dqr, dkr, dvb, dck, dcv = block_attention_backward(qr, kr, v4, ctx_k, ctx_v, base, anchor, dO)
    dq = rope(dqr, -pos[:, :, None], theta)            # transpose of the rotation
    dk = rope(dkr, -pos[:, :, None], theta)
    return (dq.reshape(R, Hq * D), dk.reshape(R, Hkv * D), dvb.reshape(R, Hkv * D), dck, dcv)


def ctx_grad_rows(d_ctx_k, d_ctx_v, positions, num_kv_heads: int, head_dim: int, theta: float):
    """Per-row gradient of every layer's context K and V, back in the
    un-rotated projection space: for layer l, row t,
        Gk_l[t] = RoPE^T(dKc_l[:, t, :], positions[t])  (rotation by the opposite angle),
        Gv_l[t] = dVc_l[:, t, :],
    each flattened head-major to [Hkv*D]. d_ctx_k / d_ctx_v are lists over layers
    of [Hkv, T, D]. Returns (Gk, Gv), lists of [T, Hkv*D]."""
    pos = np.asarray(positions, np.int64)
    Gk, Gv = [], []
    for dk, dv in zip(d_ctx_k, d_ctx_v):
        dk = np.asarray(dk, np.float64).transpose(1, 0, 2)          # [T, Hkv, D]
        dv = np.asarray(dv, np.float64).transpose(1, 0, 2)
        T = dk.shape[0]
        Gk.append(rope(dk, -pos[:, None], theta).reshape(T, num_kv_heads * head_dim))
        Gv.append(dv.reshape(T, num_kv_heads * head_dim))
    return Gk, Gv


def ctx_hidden_grad(d_ctx_k, d_ctx_v, positions, layers, num_kv_heads: int, head_dim: int, theta: float):
    """dC = sum_l Gk_l Wk_l + Gv_l Wv_l [T, H] (the rows of C are independent, so
    any subset of rows with their positions gives those rows of dC; any subset
    of the weights' columns gives those columns)."""
    Gk, Gv = ctx_grad_rows(d_ctx_k, d_ctx_v, positions, num_kv_heads, head_dim, theta)
    dC = 0.0
    for l, W in enumerate(layers):
        dC = dC + Gk[l] @ np.asarray(W["wk"], np.float64) + Gv[l] @ np.asarray(W["wv"], np.float64)
    return dC


def ctx_proj_backward(X, positions, layers, d_ctx_k, d_ctx_v, num_kv_heads: int, head_dim: int, theta: float):
    """Gradients through the context path (ctx_proj, then ctx_kv of every layer;
    NeMo RL "DFlash Draft Body", Scope: training updates W_proj; angelspec
    "DFlash", How it works: the target's hidden states are projected into every
    layer's K/V). With C = X W_proj^T, Kc_l = RoPE(C Wk_l^T), Vc_l = C Wv_l^T and
    upstream gradients dKc_l, dVc_l:
        dC = sum_l Gk_l Wk_l + Gv_l Wv_l     [T, H]
        dW_proj = dC^T X                       [H, L_t*H_t]
    Returns (dC, dW_proj)."""
    X = np.asarray(X, np.float64)
    dC = ctx_hidden_grad(d_ctx_k, d_ctx_v, positions, layers, num_kv_heads, head_dim, theta)
    return dC, dC.T @ X
