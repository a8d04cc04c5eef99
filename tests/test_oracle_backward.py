"""Pins of the attention-backward oracle against finite differences of the
forward oracle (NeMo RL "DFlash Draft Body", How It Works, step 3; Scope:
training runs the body with an optimizer step). Central differences of
L = sum(d_out * block_attn_call(...)) in fp64 must match every analytic
gradient component, including context rows read by several blocks and the
rows of invalid positions (keys for the others, no output of their own)."""
import numpy as np

import oracle
from oracle.backward import block_attention_backward, block_attn_call_backward


def _case(seed):
    rng = np.random.default_rng(seed)
    nb, bs, Hq, Hkv, D, T = 3, 4, 4, 2, 8, 14
    q = rng.standard_normal((nb * bs, Hq * D))
    k = rng.standard_normal((nb * bs, Hkv * D))
    v = rng.standard_normal((nb * bs, Hkv * D))
    ck = rng.standard_normal((Hkv, T, D))
    cv = rng.standard_normal((Hkv, T, D))
    base = [0, 0, 7]
    anchor = [5, 7, 6]                            # blocks 0 and 1 share context rows 0..4
    valid = np.ones(nb * bs, np.uint8)
    valid[6] = 0                                  # an invalid position: its key still counts
    dO = rng.standard_normal((nb * bs, Hq * D))
    return q, k, v, ck, cv, base, anchor, valid, dO, (bs, Hq, Hkv, D, 1e4)


def _loss(q, k, v, ck, cv, base, anchor, valid, dO, dims):
    bs, Hq, Hkv, D, theta = dims
    o = oracle.block_attn_call(q, k, v, ck, cv, base, anchor, valid, bs, Hq, Hkv, D, theta)
    return float((dO * o).sum())


def test_gradients_match_finite_differences():
    q, k, v, ck, cv, base, anchor, valid, dO, dims = _case(0)
    bs, Hq, Hkv, D, theta = dims
    grads = block_attn_call_backward(q, k, v, ck, cv, base, anchor, valid, bs, Hq, Hkv, D, theta, dO)
    args = [q, k, v, ck, cv]
    eps = 1e-6
    for which, (x, g) in enumerate(zip(args, grads)):
        num = np.zeros_like(x)
        flat, nflat = x.reshape(-1), num.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            lp = _loss(*args, base, anchor, valid, dO, dims)
            flat[i] = old - eps
            lm = _loss(*args, base, anchor, valid, dO, dims)
            flat[i] = old
            nflat[i] = (lp - lm) / (2 * eps)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-7), (which, np.abs(g - num).max())


def test_structure_of_the_gradients():
    q, k, v, ck, cv, base, anchor, valid, dO, dims = _case(1)
    bs, Hq, Hkv, D, theta = dims
    dq, dk, dv, dck, dcv = block_attn_call_backward(q, k, v, ck, cv, base, anchor, valid, bs, Hq, Hkv, D,
                                                    theta, dO)
    assert (dq[6] == 0).all()                     # no output at an invalid position -> no dq
    assert np.abs(dk[6]).sum() > 0 and np.abs(dv[6]).sum() > 0   # but it is a key of its block
    # rows that no block reads get nothing
    assert (dck[:, 13:] == 0).all() and (dcv[:, 13:] == 0).all()     # block 2 reads rows 7..12 only
    # empty block: no gradient anywhere from it
    anchor2 = [5, -1, 6]
    g2 = block_attn_call_backward(q, k, v, ck, cv, base, anchor2, valid, bs, Hq, Hkv, D, theta, dO)
    assert (g2[0][4:8] == 0).all() and (g2[1][4:8] == 0).all() and (g2[2][4:8] == 0).all()
    # dV sums p over queries: with dO = 1 everywhere, every block's dV rows sum to bs*G per value dim
    nb = q.shape[0] // bs
    q4 = oracle.rope(q.reshape(nb, bs, Hq, D), (np.array(anchor)[:, None] + np.arange(bs))[:, :, None], theta)
    k4 = oracle.rope(k.reshape(nb, bs, Hkv, D), (np.array(anchor)[:, None] + np.arange(bs))[:, :, None], theta)
    ones = np.ones((nb, bs, Hq, D))
    _, _, dvb, _, dcv1 = block_attention_backward(q4, k4, v.reshape(nb, bs, Hkv, D), ck, cv, base, anchor, ones)
    total = dvb.sum(axis=(0, 1)) + dcv1.sum(axis=1)       # [Hkv, D]
    assert np.allclose(total, nb * bs * (Hq // Hkv))


# ---------------------------------------------------------------- context path
def _ctx_case(seed):
    rng = np.random.default_rng(seed)
    T, K_in, H, Hkv, D, L = 6, 10, 8, 2, 4, 2
    X = rng.standard_normal((T, K_in))
    w_proj = rng.standard_normal((H, K_in))
    layers = [{"wk": rng.standard_normal((Hkv * D, H)), "wv": rng.standard_normal((Hkv * D, H))} for _ in range(L)]
    pos = rng.integers(0, 50, T)
    gk = [rng.standard_normal((Hkv, T, D)) for _ in range(L)]
    gv = [rng.standard_normal((Hkv, T, D)) for _ in range(L)]
    return X, w_proj, layers, pos, gk, gv, (Hkv, D, 1e4)


def _ctx_loss_of_c(C, layers, pos, gk, gv, dims):
    Hkv, D, theta = dims
    ks, vs = oracle.ctx_kv(C, layers, pos, Hkv, D, theta)
    return sum(float((a * b).sum()) for a, b in zip(ks + vs, gk + gv))


def _ctx_loss(w_proj, X, layers, pos, gk, gv, dims):
    return _ctx_loss_of_c(oracle.ctx_proj(X, w_proj), layers, pos, gk, gv, dims)


def test_ctx_backward_matches_directional_differences():
    # The context path is linear in W_proj and in C, so a central difference
    # along any direction E equals <grad, E> up to rounding.
    X, w_proj, layers, pos, gk, gv, dims = _ctx_case(2)
    dC, dW = oracle.ctx_proj_backward(X, pos, layers, gk, gv, *dims)
    rng = np.random.default_rng(3)
    for _ in range(3):
        E = rng.standard_normal(w_proj.shape)
        h = 1e-3
        num = (_ctx_loss(w_proj + h * E, X, layers, pos, gk, gv, dims)
               - _ctx_loss(w_proj - h * E, X, layers, pos, gk, gv, dims)) / (2 * h)
        assert abs(num - float((dW * E).sum())) <= 1e-9 * max(1.0, abs(num))
        Ec = rng.standard_normal(dC.shape)
        C = oracle.ctx_proj(X, w_proj)
        num_c = (_ctx_loss_of_c(C + h * Ec, layers, pos, gk, gv, dims)
                 - _ctx_loss_of_c(C - h * Ec, layers, pos, gk, gv, dims)) / (2 * h)
        assert abs(num_c - float((dC * Ec).sum())) <= 1e-9 * max(1.0, abs(num_c))


def test_ctx_backward_entrywise():
    X, w_proj, layers, pos, gk, gv, dims = _ctx_case(4)
    _, dW = oracle.ctx_proj_backward(X, pos, layers, gk, gv, *dims)
    num = np.zeros_like(w_proj)
    for i in range(w_proj.shape[0]):
        for j in range(w_proj.shape[1]):
            E = np.zeros_like(w_proj)
            E[i, j] = 1.0
            num[i, j] = (_ctx_loss(w_proj + E, X, layers, pos, gk, gv, dims)
                         - _ctx_loss(w_proj - E, X, layers, pos, gk, gv, dims)) / 2
    assert np.allclose(dW, num, rtol=1e-10, atol=1e-9)


def test_ctx_grad_rows_undo_the_rotation():
    # At position 0 RoPE is the identity; at any position the rotated-back
    # gradient keeps each pair's norm.
    rng = np.random.default_rng(5)
    gk = [rng.standard_normal((2, 3, 8))]
    gv = [rng.standard_normal((2, 3, 8))]
    Gk, Gv = oracle.ctx_grad_rows(gk, gv, [0, 7, 123], 2, 8, 1e4)
    assert np.allclose(Gk[0][0], gk[0][:, 0, :].reshape(-1))
    a = Gk[0].reshape(3, 2, 2, 4)
    b = gk[0].transpose(1, 0, 2).reshape(3, 2, 2, 4)
    assert np.allclose((a * a).sum(axis=2), (b * b).sum(axis=2))
    assert np.allclose(Gv[0], gv[0].transpose(1, 0, 2).reshape(3, -1))


def test_ctx_kv_weight_grads_entrywise():
    # The context path is linear in each Wk_l and Wv_l: a central difference of
    # step 1 over one entry is that entry's gradient exactly (up to rounding).
    X, w_proj, layers, pos, gk, gv, dims = _ctx_case(6)
    C = oracle.ctx_proj(X, w_proj)
    dWk, dWv = oracle.ctx_kv_weight_grads(C, pos, gk, gv, *dims)
    for l in range(len(layers)):
        for kind, grad in (("wk", dWk[l]), ("wv", dWv[l])):
            num = np.zeros_like(grad)
            for i in range(grad.shape[0]):
                for j in range(grad.shape[1]):
                    plus = [dict(L) for L in layers]
                    minus = [dict(L) for L in layers]
                    E = np.zeros_like(layers[l][kind])
                    E[i, j] = 1.0
                    plus[l][kind] = layers[l][kind] + E
                    minus[l][kind] = layers[l][kind] - E
                    num[i, j] = (_ctx_loss_of_c(C, plus, pos, gk, gv, dims)
                                 - _ctx_loss_of_c(C, minus, pos, gk, gv, dims)) / 2
            assert np.allclose(grad, num, rtol=1e-10, atol=1e-9), f"layer {l} {kind}"
