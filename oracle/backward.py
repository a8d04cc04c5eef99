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

from .body import block_attn_call, rms_norm, rope, silu


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


def ctx_kv_weight_grads(C, positions, d_ctx_k, d_ctx_v, num_kv_heads: int, head_dim: int, theta: float):
    """The context path's share of every layer's Wk and Wv gradient (angelspec
    "DFlash", How it works: the projected target context enters each draft
    layer's K/V through that layer's own projections). With Kc_l = RoPE(C Wk_l^T)
    and Vc_l = C Wv_l^T:
        dWk_l = Gk_l^T C,   dWv_l = Gv_l^T C      [Hkv*D, H]
    with Gk_l, Gv_l as in ctx_grad_rows. The block rows' share comes from
    body_backward; a training step adds the two. Returns (dWk list, dWv list)."""
    C = np.asarray(C, np.float64)
    Gk, Gv = ctx_grad_rows(d_ctx_k, d_ctx_v, positions, num_kv_heads, head_dim, theta)
    return [g.T @ C for g in Gk], [g.T @ C for g in Gv]


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


# ---------------------------------------------------------------------------
# The draft body's backward: every layer weight, the block embeddings and the
# context caches (NeMo RL "DFlash Draft Body", How It Works, step 1 and Scope:
# the body is trained with an optimizer step; step 3: the layers the body runs).
# The forward differentiated is body_forward (body.py): per layer, with the
# same readings as there (pre-norm decoder layer, no biases, invalid rows evolve
# like the others inside the body, only the returned rows are zeroed):
#     x = RMSNorm(h) w_a;  q, k, v = x Wq^T, x Wk^T, x Wv^T
#     h1 = h + Attn(q, k, v) Wo^T
#     y = RMSNorm(h1) w_m;  g = y Wg^T, u_p = y Wu^T,  u = SiLU(g) u_p
#     h' = h1 + u Wd^T
# and out = h_L on kept rows (valid, non-empty block), zero elsewhere.


def rms_norm_backward(x, w, eps: float, dy):
    """Gradients of y = x * r * w, r = (mean(x^2) + eps)^(-1/2) per row, given dy:
        dx = r (dy w) - x r^3 (sum_j dy_j w_j x_j) / H
        dw = sum over rows of dy x r
    Returns (dx, dw)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    dy = np.asarray(dy, np.float64)
    H = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    dyw = dy * w
    dot = np.sum(dyw * x, axis=-1, keepdims=True)
    dx = r * dyw - x * (r ** 3) * dot / H
    dw = np.sum(dy * x * r, axis=0)
    return dx, dw


def swiglu_backward(g, up, du):
    """Gradients of u = SiLU(g) * up, SiLU(g) = g * s, s = sigmoid(g):
        dg = du * up * s (1 + g (1 - s)),   dup = du * SiLU(g).
    Returns (dg, dup)."""
    g = np.asarray(g, np.float64)
    up = np.asarray(up, np.float64)
    du = np.asarray(du, np.float64)
    s = 1.0 / (1.0 + np.exp(-g))
    return du * up * s * (1.0 + g * (1.0 - s)), du * g * s


def _f64(W):
    return {k: np.asarray(v, np.float64) for k, v in W.items()}


def _layer_attention(x, W, ctx_k, ctx_v, base, anchor, cfg):
    bs = int(cfg["block_size"])
    R = x.shape[0]
    q, k, v = x @ W["wq"].T, x @ W["wk"].T, x @ W["wv"].T
    every_row = np.ones(R, np.uint8)          # inside the body no row's output is zeroed
    o = block_attn_call(q, k, v, ctx_k, ctx_v, base, anchor, every_row, bs, int(cfg["num_q_heads"]),
                        int(cfg["num_kv_heads"]), int(cfg["head_dim"]), float(cfg["rope_theta"]))
    return q, k, v, o


def layer_forward(h, W, ctx_k, ctx_v, base, anchor, cfg):
    """One draft layer on the residual stream h [R, H] -> h' [R, H] (the loop body
    of body_forward, written out with its intermediates). ctx_k / ctx_v: this
    layer's caches [Hkv, T, D] (K rotated)."""
    W = _f64(W)
    eps = float(cfg["rms_eps"])
    h = np.asarray(h, np.float64)
    x = rms_norm(h, W["attn_norm"], eps)
    q, k, v, o = _layer_attention(x, W, np.asarray(ctx_k, np.float64), np.asarray(ctx_v, np.float64),
                                  base, anchor, cfg)
    h1 = h + o @ W["wo"].T
    y = rms_norm(h1, W["mlp_norm"], eps)
    g, up = y @ W["w_gate"].T, y @ W["w_up"].T
    u = silu(g) * up
    return h1 + u @ W["w_down"].T


def layer_backward(h, W, ctx_k, ctx_v, base, anchor, cfg, dh_out):
    """Backward of layer_forward given dh_out = dL/dh'. Recomputes the layer's
    intermediates from its input h, then applies the chain rule from the output
    back to the input:
        d_w_down = dh'^T u,            du = dh' Wd
        dg, dup  = swiglu_backward(g, up, du)
        d_w_gate = dg^T y, d_w_up = dup^T y,   dy = dg Wg + dup Wu
        dh1      = dh' + RMSNorm backward of (h1, w_m) at dy      (-> d_mlp_norm)
        d_wo     = dh1^T o,            do = dh1 Wo
        dq, dk, dv, dKc, dVc = block_attn_call_backward(..., do)  (every row kept)
        d_wq = dq^T x, d_wk = dk^T x, d_wv = dv^T x,   dx = dq Wq + dk Wk + dv Wv
        dh       = dh1 + RMSNorm backward of (h, w_a) at dx       (-> d_attn_norm)
    Returns (dh, grads, d_ctx_k, d_ctx_v): grads holds d_<name> for every weight
    of the layer in its own shape; d_ctx_k (rotated frame) and d_ctx_v are
    [Hkv, T, D] like the caches."""
    W = _f64(W)
    eps = float(cfg["rms_eps"])
    bs, Hq, Hkv, D = (int(cfg["block_size"]), int(cfg["num_q_heads"]), int(cfg["num_kv_heads"]),
                      int(cfg["head_dim"]))
    h = np.asarray(h, np.float64)
    ctx_k = np.asarray(ctx_k, np.float64)
    ctx_v = np.asarray(ctx_v, np.float64)
    dh2 = np.asarray(dh_out, np.float64)
    # Forward, keeping what the backward reads.
    x = rms_norm(h, W["attn_norm"], eps)
    q, k, v, o = _layer_attention(x, W, ctx_k, ctx_v, base, anchor, cfg)
    h1 = h + o @ W["wo"].T
    y = rms_norm(h1, W["mlp_norm"], eps)
    g, up = y @ W["w_gate"].T, y @ W["w_up"].T
    u = silu(g) * up
    # MLP.
    d_w_down = dh2.T @ u
    du = dh2 @ W["w_down"]
    dg, dup = swiglu_backward(g, up, du)
    d_w_gate, d_w_up = dg.T @ y, dup.T @ y
    dy = dg @ W["w_gate"] + dup @ W["w_up"]
    dh1_norm, d_mlp_norm = rms_norm_backward(h1, W["mlp_norm"], eps, dy)
    dh1 = dh2 + dh1_norm
    # Attention.
    d_wo = dh1.T @ o
    do = dh1 @ W["wo"]
    every_row = np.ones(h.shape[0], np.uint8)
    dq, dk, dv, dck, dcv = block_attn_call_backward(q, k, v, ctx_k, ctx_v, base, anchor, every_row, bs, Hq,
                                                    Hkv, D, float(cfg["rope_theta"]), do)
    d_wq, d_wk, d_wv = dq.T @ x, dk.T @ x, dv.T @ x
    dx = dq @ W["wq"] + dk @ W["wk"] + dv @ W["wv"]
    dh_norm, d_attn_norm = rms_norm_backward(h, W["attn_norm"], eps, dx)
    grads = dict(attn_norm=d_attn_norm, wq=d_wq, wk=d_wk, wv=d_wv, wo=d_wo, mlp_norm=d_mlp_norm,
                 w_gate=d_w_gate, w_up=d_w_up, w_down=d_w_down)
    return dh1 + dh_norm, grads, dck, dcv


def _kept_rows(anchor, valid, bs: int):
    anchor = np.asarray(anchor, np.int64)
    return np.asarray(valid, bool).reshape(-1) & np.repeat(anchor >= 0, bs)


def body_forward_layers(emb, layers, ctx_k, ctx_v, base, anchor, valid, cfg):
    """body_forward as a chain of layer_forward calls. Returns (out, hs) with
    hs[l] the residual stream entering layer l (hs[0] = emb)."""
    h = np.asarray(emb, np.float64)
    hs = []
    for l, W in enumerate(layers):
        hs.append(h)
        h = layer_forward(h, W, ctx_k[l], ctx_v[l], base, anchor, cfg)
    keep = _kept_rows(anchor, valid, int(cfg["block_size"]))
    return np.where(keep[:, None], h, 0.0), hs


def body_backward(emb, layers, ctx_k, ctx_v, base, anchor, valid, cfg, d_out):
    """Gradients of body_forward given d_out = dL/dout [R, H]: the returned rows'
    mask passes d_out to the last layer's output (zero rows pass nothing), then
    layer_backward runs from the last layer to the first. Returns
    (d_emb, grads, d_ctx_k, d_ctx_v), the last three lists over layers."""
    _, hs = body_forward_layers(emb, layers, ctx_k, ctx_v, base, anchor, valid, cfg)
    keep = _kept_rows(anchor, valid, int(cfg["block_size"]))
    dh = np.where(keep[:, None], np.asarray(d_out, np.float64), 0.0)
    L = len(layers)
    grads, dcks, dcvs = [None] * L, [None] * L, [None] * L
    for l in reversed(range(L)):
        dh, grads[l], dcks[l], dcvs[l] = layer_backward(hs[l], layers[l], ctx_k[l], ctx_v[l], base, anchor,
                                                        cfg, dh)
    return dh, grads, dcks, dcvs
