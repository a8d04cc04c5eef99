"""fp64 oracle of the DFlash draft body (test infrastructure only; see the
package docstring). Plain numpy; a matmul is the only library primitive used.

What is computed, and where the pages state it:
  * angelspec "DFlash" page, How it works, "Dual-source KV context": the target
    model's multi-layer hidden states are projected (W_proj) into the attention
    key/value space and attended to together with the draft tokens' own K/V.
  * same page, Configuration: the target layers given by target_layer_ids are
    the context, concatenated in that order; rope_theta is a model parameter.
  * NeMo RL "DFlash Draft Body", How It Works, step 3: the body projects the
    target states and runs the block embeddings through draft decoder layers;
    inside a layer a block reads the target prefix before its anchor and every
    position of its own block, never another block; attention produces outputs
    for block positions only.
  * same page, step 4: one hidden state per block position, zero for invalid
    positions; the anchor row is computed (it is only left out of the loss).
  * cooking-agi "DFlash: drafting, verification, and speed", One DFlash
    generation cycle: target context features enter every draft layer's K/V; a
    predicted block must not read target features that contain its future.

Readings where the pages are silent (the same ones the HIP path takes):
  * prefix visibility is strict: context keys j < a; prefix positions are not
    filtered by the mask;
  * all block positions (valid or not) are keys and queries in every layer,
    bidirectionally inside the block; only the returned rows are zeroed;
  * no normalisation between W_proj and the per-layer K/V projections;
  * the draft layer is a pre-norm decoder layer: RMSNorm -> Q/K/V -> RoPE ->
    attention -> o_proj -> residual, RMSNorm -> SwiGLU MLP -> residual; no
    biases, no q/k norm, no final norm; eps 1e-6;
  * RoPE pairs dimension i with i + D/2, inverse frequency theta^(-2i/D);
    context row j sits at position j of its sequence, block row k at a + k;
  * grouped-query attention maps query head h to KV head floor(h / (Hq/Hkv));
    scores are scaled by 1/sqrt(D);
  * Linear weights are [out, in] and y = x W^T.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np


def concat_target_states(states) -> np.ndarray:
    """[L_t, T, H_t] (one slab per target layer, in target_layer_ids order)
    -> X [T, L_t * H_t]."""
    states = np.asarray(states, dtype=np.float64)
    return np.concatenate([states[i] for i in range(states.shape[0])], axis=-1)


def ctx_proj(X: np.ndarray, w_proj: np.ndarray) -> np.ndarray:
    """C = X W_proj^T: the concatenated target states in the draft hidden space."""
    return np.asarray(X, np.float64) @ np.asarray(w_proj, np.float64).T


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotary embedding of x [..., D] at integer positions pos (broadcast over
    x[..., 0]). Pair (i, i + D/2) is rotated by angle pos * theta^(-2i/D)."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    half = D // 2
    ang = np.asarray(pos, np.float64)[..., None] * rope_inv_freq(D, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def ctx_kv(C: np.ndarray, layers: Sequence[Dict[str, np.ndarray]], positions,
           num_kv_heads: int, head_dim: int, theta: float):
    """Per draft layer l: Kc_l = RoPE(C Wk_l^T) at each row's position, Vc_l = C Wv_l^T,
    both returned head-major [Hkv, T, D]."""
    T = C.shape[0]
    ks, vs = [], []
    pos = np.asarray(positions)
    for W in layers:
        k = (C @ np.asarray(W["wk"], np.float64).T).reshape(T, num_kv_heads, head_dim)
        v = (C @ np.asarray(W["wv"], np.float64).T).reshape(T, num_kv_heads, head_dim)
        k = rope(k, pos[:, None], theta)
        ks.append(np.ascontiguousarray(k.transpose(1, 0, 2)))
        vs.append(np.ascontiguousarray(v.transpose(1, 0, 2)))
    return ks, vs


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def block_attention(q, kb, vb, ctx_k, ctx_v, base, anchor) -> np.ndarray:
    """Dual-source attention in gathered form.

    q [nb, bs, Hq, D] and kb [nb, bs, Hkv, D] already rotated; vb [nb, bs, Hkv, D];
    ctx_k / ctx_v [Hkv, T, D] (K rotated); block n reads ctx rows
    base[n] .. base[n] + anchor[n] - 1 and the bs rows of its own block.
    Blocks with anchor < 0 are empty and return zeros.
    """
    q = np.asarray(q, np.float64)
    nb, bs, Hq, D = q.shape
    Hkv = kb.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for n in range(nb):
        a = int(anchor[n])
        if a < 0:
            continue
        b0 = int(base[n])
        for h in range(Hq):
            g = h // G
            K = np.concatenate([ctx_k[g, b0:b0 + a], kb[n, :, g]], axis=0)
            V = np.concatenate([ctx_v[g, b0:b0 + a], vb[n, :, g]], axis=0)
            p = _softmax_rows(q[n, :, h] @ K.T / math.sqrt(D))
            out[n, :, h] = p @ V
    return out


def dense_mask_attention(q, kb, vb, ctx_k, ctx_v, base, anchor) -> np.ndarray:
    """Brute force: one key axis [all T context rows | all nb*bs block rows] per
    KV head with an explicit boolean visibility mask and a textbook masked
    softmax, looped query by query. Used only on tiny inputs to pin
    block_attention's gathering."""
    q = np.asarray(q, np.float64)
    nb, bs, Hq, D = q.shape
    Hkv = kb.shape[2]
    T = ctx_k.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for n in range(nb):
        if int(anchor[n]) < 0:
            continue
        for k in range(bs):
            for h in range(Hq):
                g = h // G
                keys, vals, vis = [], [], []
                for j in range(T):
                    keys.append(ctx_k[g, j]); vals.append(ctx_v[g, j])
                    vis.append(int(base[n]) <= j < int(base[n]) + int(anchor[n]))
                for n2 in range(nb):
                    for k2 in range(bs):
                        keys.append(kb[n2, k2, g]); vals.append(vb[n2, k2, g])
                        vis.append(n2 == n)
                keys = np.array(keys); vals = np.array(vals); vis = np.array(vis)
                scores = np.array([np.dot(q[n, k, h], key) for key in keys]) / math.sqrt(D)
                scores = np.where(vis, scores, -np.inf)
                w = np.exp(scores - scores[vis].max())
                w = np.where(vis, w, 0.0)
                out[n, k, h] = (w[:, None] * vals).sum(0) / w.sum()
    return out


def block_attn_call(q, k_blk, v_blk, ctx_k, ctx_v, base, anchor, valid, block_size: int,
                    num_q_heads: int, num_kv_heads: int, head_dim: int, theta: float):
    """The standalone attention call: q [nb*bs, Hq*D] and k_blk / v_blk
    [nb*bs, Hkv*D] before RoPE; block row k of block n is rotated at anchor + k;
    returns [nb*bs, Hq*D] with rows of invalid positions (and of empty blocks)
    set to zero."""
    R = q.shape[0]
    nb = R // block_size
    q4 = np.asarray(q, np.float64).reshape(nb, block_size, num_q_heads, head_dim)
    k4 = np.asarray(k_blk, np.float64).reshape(nb, block_size, num_kv_heads, head_dim)
    v4 = np.asarray(v_blk, np.float64).reshape(nb, block_size, num_kv_heads, head_dim)
    pos = np.asarray(anchor, np.int64)[:, None] + np.arange(block_size)[None, :]
    q4 = rope(q4, pos[:, :, None], theta)
    k4 = rope(k4, pos[:, :, None], theta)
    o = block_attention(q4, k4, v4, np.asarray(ctx_k, np.float64), np.asarray(ctx_v, np.float64),
                        base, anchor).reshape(R, num_q_heads * head_dim)
    keep = np.asarray(valid, bool).reshape(R) & np.repeat(np.asarray(anchor) >= 0, block_size)
    return np.where(keep[:, None], o, 0.0)


def _body(emb, layers, ctx_k, ctx_v, base, anchor, valid, cfg, attention, zero_invalid_each_layer):
    bs = int(cfg["block_size"])
    Hq, Hkv, D = int(cfg["num_q_heads"]), int(cfg["num_kv_heads"]), int(cfg["head_dim"])
    theta, eps = float(cfg["rope_theta"]), float(cfg["rms_eps"])
    emb = np.asarray(emb, np.float64)
    R, H = emb.shape
    nb = R // bs
    anchor = np.asarray(anchor, np.int64)
    keep = np.asarray(valid, bool).reshape(R) & np.repeat(anchor >= 0, bs)
    pos = anchor[:, None] + np.arange(bs)[None, :]
    h = emb.copy()
    for l, W in enumerate(layers):
        W = {k: np.asarray(v, np.float64) for k, v in W.items()}
        x = rms_norm(h, W["attn_norm"], eps)
        q = (x @ W["wq"].T).reshape(nb, bs, Hq, D)
        k = (x @ W["wk"].T).reshape(nb, bs, Hkv, D)
        v = (x @ W["wv"].T).reshape(nb, bs, Hkv, D)
        q = rope(q, pos[:, :, None], theta)
        k = rope(k, pos[:, :, None], theta)
        o = attention(q, k, v, np.asarray(ctx_k[l], np.float64), np.asarray(ctx_v[l], np.float64),
                      base, anchor).reshape(R, Hq * D)
        h = h + o @ W["wo"].T
        y = rms_norm(h, W["mlp_norm"], eps)
        h = h + (silu(y @ W["w_gate"].T) * (y @ W["w_up"].T)) @ W["w_down"].T
        if zero_invalid_each_layer:
            h = np.where(keep[:, None], h, 0.0)
    return np.where(keep[:, None], h, 0.0)


def body_forward(emb, layers: List[Dict[str, np.ndarray]], ctx_k, ctx_v, base, anchor, valid,
                 cfg: Dict[str, float], zero_invalid_each_layer: bool = False) -> np.ndarray:
    """The draft body over nb blocks: emb [nb*bs, H] -> out [nb*bs, H].

    cfg holds block_size, num_q_heads, num_kv_heads, head_dim, rope_theta, rms_eps.
    ctx_k[l] / ctx_v[l] are [Hkv, T, D] (K already rotated), base[n] is the first
    context row of block n's sequence and anchor[n] its anchor (-1: empty block).
    zero_invalid_each_layer=True is the rejected alternative reading (invalid rows
    forced to zero after every layer), kept to show where the readings differ.
    """
    return _body(emb, layers, ctx_k, ctx_v, base, anchor, valid, cfg, block_attention,
                 zero_invalid_each_layer)


def body_forward_dense(emb, layers, ctx_k, ctx_v, base, anchor, valid, cfg) -> np.ndarray:
    """body_forward with the brute-force dense-mask attention (tiny inputs only)."""
    return _body(emb, layers, ctx_k, ctx_v, base, anchor, valid, cfg, dense_mask_attention, False)
