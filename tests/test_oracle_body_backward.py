"""Pins of the body-backward oracle (NeMo RL "DFlash Draft Body", How It Works,
step 1 and Scope: the body is trained with an optimizer step; step 3: the draft
decoder layers). Every analytic gradient is checked against central finite
differences of the forward oracle body_forward, which is an independent loop
(body.py), on a two-layer case whose blocks hold invalid rows (they evolve
like the others inside the body, only the returned rows are zeroed) and one
empty block. RMSNorm and SwiGLU backward are pinned on their own, entry by
entry, so that a dropped term shows up where it is made."""
import numpy as np
import pytest

import oracle
from oracle.backward import (body_backward, body_forward_layers, layer_backward, layer_forward,
                             rms_norm_backward, swiglu_backward)

EPS = 1e-6


def _central(f, x, idx):
    """Central difference of scalar f() with respect to x.flat[idx] (x edited in place)."""
    flat = x.reshape(-1)
    old = flat[idx]
    flat[idx] = old + EPS
    lp = f()
    flat[idx] = old - EPS
    lm = f()
    flat[idx] = old
    return (lp - lm) / (2 * EPS)


def test_rms_norm_backward_every_entry():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 10))
    x[1] *= 1e-2                                # a row where eps matters
    w = 1.0 + 0.3 * rng.standard_normal(10)
    dy = rng.standard_normal((3, 10))
    eps = 1e-3
    dx, dw = rms_norm_backward(x, w, eps, dy)
    f = lambda: float((dy * oracle.rms_norm(x, w, eps)).sum())
    for i in range(x.size):
        assert abs(_central(f, x, i) - dx.reshape(-1)[i]) < 1e-7
    for i in range(w.size):
        assert abs(_central(f, w, i) - dw[i]) < 1e-7


def test_swiglu_backward_every_entry():
    rng = np.random.default_rng(1)
    g = 3.0 * rng.standard_normal((4, 6))
    g[0, 0], g[0, 1] = 0.0, -40.0               # SiLU'(0) = 1/2; a saturated negative gate
    up = rng.standard_normal((4, 6))
    du = rng.standard_normal((4, 6))
    dg, dup = swiglu_backward(g, up, du)
    f = lambda: float((du * oracle.silu(g) * up).sum())
    for i in range(g.size):
        assert abs(_central(f, g, i) - dg.reshape(-1)[i]) < 1e-7
        assert abs(_central(f, up, i) - dup.reshape(-1)[i]) < 1e-7
    assert dg[0, 0] == pytest.approx(0.5 * du[0, 0] * up[0, 0])
    assert abs(dg[0, 1]) < 1e-15


CFG = dict(block_size=4, num_q_heads=2, num_kv_heads=1, head_dim=8, rope_theta=100.0, rms_eps=1e-5)
H, I, T = 16, 24, 9


def _case(seed):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 2, 1, 8, 4

    def mat(o, i):
        return rng.standard_normal((o, i)) / np.sqrt(i)
    layers = [dict(attn_norm=1.0 + 0.2 * rng.standard_normal(H), wq=mat(Hq * D, H), wk=mat(Hkv * D, H),
                   wv=mat(Hkv * D, H), wo=mat(H, Hq * D), mlp_norm=1.0 + 0.2 * rng.standard_normal(H),
                   w_gate=mat(I, H), w_up=mat(I, H), w_down=mat(H, I)) for _ in range(2)]
    ck = [rng.standard_normal((Hkv, T, D)) for _ in range(2)]
    cv = [rng.standard_normal((Hkv, T, D)) for _ in range(2)]
    emb = rng.standard_normal((3 * bs, H))
    base = np.array([0, 0, 0])
    anchor = np.array([3, 7, -1])               # two blocks share context rows 0..2; one empty block
    valid = np.ones(3 * bs, np.uint8)
    valid[[2, 5, 7]] = 0                        # invalid rows inside both live blocks
    d_out = rng.standard_normal((3 * bs, H))
    return layers, ck, cv, emb, base, anchor, valid, d_out


def test_layer_chain_equals_body_forward():
    layers, ck, cv, emb, base, anchor, valid, _ = _case(2)
    out, hs = body_forward_layers(emb, layers, ck, cv, base, anchor, valid, CFG)
    ref = oracle.body_forward(emb, layers, ck, cv, base, anchor, valid, CFG)
    assert np.abs(out - ref).max() < 1e-12
    assert np.array_equal(hs[0], emb)
    assert np.abs(hs[1] - layer_forward(emb, layers[0], ck[0], cv[0], base, anchor, CFG)).max() == 0.0


def test_body_backward_matches_finite_differences():
    layers, ck, cv, emb, base, anchor, valid, d_out = _case(3)
    d_emb, grads, dck, dcv = body_backward(emb, layers, ck, cv, base, anchor, valid, CFG, d_out)
    f = lambda: float((d_out * oracle.body_forward(emb, layers, ck, cv, base, anchor, valid, CFG)).sum())
    rng = np.random.default_rng(4)

    def check(x, g, what, k=None):
        idx = range(x.size) if k is None else rng.choice(x.size, k, replace=False)
        scale = max(float(np.abs(g).max()), 1e-3)
        for i in idx:
            num = _central(f, x, int(i))
            assert abs(num - g.reshape(-1)[int(i)]) < 1e-6 * scale + 1e-8, (what, int(i), num, g.reshape(-1)[i])

    check(emb, d_emb, "emb")
    for l in range(2):
        for name in ("attn_norm", "mlp_norm"):
            check(layers[l][name], grads[l][name], f"{name} {l}")
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            assert grads[l][name].shape == layers[l][name].shape
            check(layers[l][name], grads[l][name], f"{name} {l}", k=24)
        check(ck[l], dck[l], f"ctx_k {l}")
        check(cv[l], dcv[l], f"ctx_v {l}")


def test_body_backward_structure():
    layers, ck, cv, emb, base, anchor, valid, d_out = _case(5)
    d_emb, grads, dck, dcv = body_backward(emb, layers, ck, cv, base, anchor, valid, CFG, d_out)
    # An empty block passes nothing back and reads nothing.
    assert (d_emb[8:12] == 0).all()
    # Context rows at or after the largest anchor are read by no block.
    for l in range(2):
        assert (dck[l][:, 7:] == 0).all() and (dcv[l][:, 7:] == 0).all()
    # Invalid rows receive a gradient: they feed their blocks' later layers.
    assert np.abs(d_emb[[2, 5, 7]]).min() > 0
    # d_out on rows the body returns as zero changes nothing.
    d2 = d_out.copy()
    d2[[2, 5, 7]] += 7.0
    d2[8:] -= 3.0
    d_emb2, grads2, _, _ = body_backward(emb, layers, ck, cv, base, anchor, valid, CFG, d2)
    assert np.array_equal(d_emb, d_emb2)
    assert all(np.array_equal(grads[l][k], grads2[l][k]) for l in range(2) for k in grads[l])


def test_single_layer_backward_is_linear_in_dh():
    layers, ck, cv, emb, base, anchor, valid, d_out = _case(6)
    a = layer_backward(emb, layers[0], ck[0], cv[0], base, anchor, CFG, d_out)
    b = layer_backward(emb, layers[0], ck[0], cv[0], base, anchor, CFG, 2.5 * d_out)
    assert np.allclose(b[0], 2.5 * a[0], rtol=1e-12, atol=1e-12)
    assert all(np.allclose(b[1][k], 2.5 * a[1][k], rtol=1e-12, atol=1e-12) for k in a[1])


# Plausible mistakes, planted in a copy of the backward oracle: each must make
# its gradients disagree with the central differences somewhere.
MUTATIONS = [
    ("    dx = r * dyw - x * (r ** 3) * dot / H", "    dx = r * dyw"),                      # RMSNorm term dropped
    ("    dh1 = dh2 + dh1_norm", "    dh1 = dh1_norm"),                                    # residual path dropped
    ('    dy = dg @ W["w_gate"] + dup @ W["w_up"]', '    dy = dg @ W["w_gate"]'),          # up branch dropped
    ("    d_wq, d_wk, d_wv = dq.T @ x, dk.T @ x, dv.T @ x",
     "    d_wq, d_wk, d_wv = dq.T @ x, dv.T @ x, dk.T @ x"),                              # operands swapped
    ("    return du * up * s * (1.0 + g * (1.0 - s)), du * g * s",
     "    return du * up * s, du * g * s"),                                                # SiLU' incomplete
    ("    return dh1 + dh_norm, grads, dck, dcv", "    return dh1 - dh_norm, grads, dck, dcv"),   # sign
    ("    d_w_down = dh2.T @ u", "    d_w_down = dh2.T @ (g * up)"),                        # wrong activation
]


@pytest.mark.parametrize("k", range(len(MUTATIONS)))
def test_planted_mistakes_are_caught(k):
    import types
    import oracle.backward as ob
    old, new = MUTATIONS[k]
    src = open(ob.__file__).read()
    assert old in src
    mod = types.ModuleType("oracle._planted")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new, 1), "planted", "exec"), mod.__dict__)
    layers, ck, cv, emb, base, anchor, valid, d_out = _case(3)
    d_emb, grads, dck, dcv = mod.body_backward(emb, layers, ck, cv, base, anchor, valid, CFG, d_out)
    f = lambda: float((d_out * oracle.body_forward(emb, layers, ck, cv, base, anchor, valid, CFG)).sum())
    checks = [(emb, d_emb)] + [(layers[l][n], grads[l][n]) for l in (1, 0) for n in
                               ("w_down", "w_gate", "w_up", "wo", "wq", "wk", "wv", "attn_norm", "mlp_norm")]
    rng = np.random.default_rng(9)
    for x, g in checks:
        scale = max(float(np.abs(g).max()), 1e-3)
        for i in rng.choice(x.size, min(x.size, 12), replace=False):
            if abs(_central(f, x, int(i)) - g.reshape(-1)[int(i)]) > 1e-6 * scale + 1e-8:
                return
    pytest.fail(f"planted mistake not caught: {new.strip()}")
