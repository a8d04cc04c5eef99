"""A whole training step's gradients, pinned end to end (NeMo RL "DFlash Draft
Body", How It Works, steps 1-4, and Scope: the body is trained with an
optimizer step; angelspec "DFlash", How it works: the projected target context
enters every draft layer's K/V through that layer's own projections, and the
decayed cross-entropy loss).

The loss of one step is a function of every trainable tensor: W_proj and each
layer's weights reach it through the block rows and, for Wk and Wv, also
through the context K/V. Central differences of that composite loss (the
forward oracles chained: ctx_proj, ctx_kv, body_forward, lm_head_ce) must equal
the sum of the oracle's backward pieces: body_backward (block rows),
ctx_kv_weight_grads (the context's share of Wk and Wv) and ctx_proj_backward
(W_proj). Leaving the context's share out fails here."""
import numpy as np
import pytest

import oracle

EPS = 1e-6
CFG = dict(block_size=4, num_q_heads=2, num_kv_heads=1, head_dim=8, rope_theta=100.0, rms_eps=1e-5)
H, I, T, HT, LT, V = 16, 24, 9, 6, 2, 11


def _case():
    rng = np.random.default_rng(7)
    Hq, Hkv, D, bs = 2, 1, 8, 4

    def mat(o, i):
        return rng.standard_normal((o, i)) / np.sqrt(i)
    layers = [dict(attn_norm=1.0 + 0.2 * rng.standard_normal(H), wq=mat(Hq * D, H), wk=mat(Hkv * D, H),
                   wv=mat(Hkv * D, H), wo=mat(H, Hq * D), mlp_norm=1.0 + 0.2 * rng.standard_normal(H),
                   w_gate=mat(I, H), w_up=mat(I, H), w_down=mat(H, I)) for _ in range(2)]
    return dict(
        layers=layers,
        w_proj=mat(H, LT * HT),
        X=rng.standard_normal((T, LT * HT)),
        emb=rng.standard_normal((3 * bs, H)),
        base=np.array([0, 0, 0]),
        anchor=np.array([3, 7, -1]),
        valid=np.array([1, 1, 0, 1, 1, 0, 1, 0, 1, 1, 1, 1], np.uint8),
        w_lm=mat(V, H),
        targets=rng.integers(0, V, 3 * bs),
        loss_mask=(np.arange(3 * bs) % bs != 0).astype(np.uint8),
        pos=np.arange(T),
    )


def _loss(c):
    C = oracle.ctx_proj(c["X"], c["w_proj"])
    ck, cv = oracle.ctx_kv(C, c["layers"], c["pos"], CFG["num_kv_heads"], CFG["head_dim"], CFG["rope_theta"])
    out = oracle.body_forward(c["emb"], c["layers"], ck, cv, c["base"], c["anchor"], c["valid"], CFG)
    return oracle.lm_head_ce(out, c["w_lm"], c["targets"], c["loss_mask"], CFG["block_size"], 3.0)[1]


def _grads(c):
    hkv, D, th = CFG["num_kv_heads"], CFG["head_dim"], CFG["rope_theta"]
    C = oracle.ctx_proj(c["X"], c["w_proj"])
    ck, cv = oracle.ctx_kv(C, c["layers"], c["pos"], hkv, D, th)
    out = oracle.body_forward(c["emb"], c["layers"], ck, cv, c["base"], c["anchor"], c["valid"], CFG)
    d_out = oracle.lm_head_ce_backward(out, c["w_lm"], c["targets"], c["loss_mask"], CFG["block_size"], 3.0)
    d_emb, grads, dck, dcv = oracle.body_backward(c["emb"], c["layers"], ck, cv, c["base"], c["anchor"],
                                                  c["valid"], CFG, d_out)
    dWk, dWv = oracle.ctx_kv_weight_grads(C, c["pos"], dck, dcv, hkv, D, th)
    _, dWp = oracle.ctx_proj_backward(c["X"], c["pos"], c["layers"], dck, dcv, hkv, D, th)
    total = [dict(g) for g in grads]
    for l in range(len(total)):
        total[l]["wk"] = grads[l]["wk"] + dWk[l]
        total[l]["wv"] = grads[l]["wv"] + dWv[l]
    return d_emb, total, dWp, (dWk, dWv)


def _central(c, arr, idx):
    flat = arr.reshape(-1)
    old = flat[idx]
    flat[idx] = old + EPS
    lp = _loss(c)
    flat[idx] = old - EPS
    lm = _loss(c)
    flat[idx] = old
    return (lp - lm) / (2 * EPS)


@pytest.mark.parametrize("name", ["wk", "wv", "wq", "w_down", "attn_norm"])
def test_layer_weight_gradients_of_the_whole_step(name):
    c = _case()
    _, total, _, _ = _grads(c)
    rng = np.random.default_rng(1)
    for l in range(2):
        W = c["layers"][l][name]
        for idx in rng.choice(W.size, size=min(12, W.size), replace=False):
            num = _central(c, W, int(idx))
            ana = float(total[l][name].reshape(-1)[idx])
            assert abs(num - ana) <= 1e-7 + 1e-5 * abs(ana), f"layer {l} {name}[{idx}]: {num} vs {ana}"


def test_context_share_of_wk_wv_is_needed():
    # The context's share is not small: without it the Wk / Wv gradients miss
    # the central differences by far more than the bar above.
    c = _case()
    _, total, _, (dWk, dWv) = _grads(c)
    assert np.abs(dWk[0]).max() > 1e-3 and np.abs(dWv[1]).max() > 1e-3
    num = _central(c, c["layers"][0]["wv"], int(np.argmax(np.abs(dWv[0]))))
    body_only = float((total[0]["wv"] - dWv[0]).reshape(-1)[int(np.argmax(np.abs(dWv[0])))])
    assert abs(num - body_only) > 100 * (1e-7 + 1e-5 * abs(num))


def test_w_proj_and_embedding_gradients_of_the_whole_step():
    c = _case()
    d_emb, _, dWp, _ = _grads(c)
    rng = np.random.default_rng(2)
    for arr, grad, what in ((c["w_proj"], dWp, "W_proj"), (c["emb"], d_emb, "embeddings")):
        for idx in rng.choice(arr.size, size=12, replace=False):
            num = _central(c, arr, int(idx))
            ana = float(grad.reshape(-1)[idx])
            assert abs(num - ana) <= 1e-7 + 1e-5 * abs(ana), f"{what}[{idx}]: {num} vs {ana}"
