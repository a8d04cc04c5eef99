"""Pins of the oracle's draft body: its composition against the brute-force
dense-mask body, special cases with closed forms, and the pages' invariants
(NeMo RL "DFlash Draft Body", How It Works, steps 3-4 and the closing note on
block independence; cooking-agi "DFlash: drafting, verification, and speed",
One DFlash generation cycle, on the information boundary). Whole-body values
beyond this composition are parity unpinned: the pages print no worked example."""
import numpy as np
import pytest

from oracle import body_forward, body_forward_dense, ctx_kv, ctx_proj, concat_target_states


def _cfg(bs=4, Hq=4, Hkv=2, D=8):
    return dict(block_size=bs, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, rope_theta=1e4,
                rms_eps=1e-6)


def _layers(rng, n_l, H, Hq, Hkv, D, I):
    out = []
    for _ in range(n_l):
        out.append(dict(
            attn_norm=1 + 0.1 * rng.normal(size=H), mlp_norm=1 + 0.1 * rng.normal(size=H),
            wq=rng.normal(size=(Hq * D, H)) / np.sqrt(H), wk=rng.normal(size=(Hkv * D, H)) / np.sqrt(H),
            wv=rng.normal(size=(Hkv * D, H)) / np.sqrt(H), wo=rng.normal(size=(H, Hq * D)) / np.sqrt(Hq * D),
            w_gate=rng.normal(size=(I, H)) / np.sqrt(H), w_up=rng.normal(size=(I, H)) / np.sqrt(H),
            w_down=rng.normal(size=(H, I)) / np.sqrt(I)))
    return out


def _setup(seed=0, n_l=2, nb=3, S=12, rows=2, H=16):
    rng = np.random.default_rng(seed)
    cfg = _cfg()
    layers = _layers(rng, n_l, H, 4, 2, 8, 24)
    T = rows * S
    states = rng.normal(size=(2, T, 10))
    C = ctx_proj(concat_target_states(states), rng.normal(size=(H, 20)) / np.sqrt(20))
    pos = np.tile(np.arange(S), rows)
    ck, cv = ctx_kv(C, layers, pos, 2, 8, 1e4)
    emb = rng.normal(size=(nb * 4, H))
    base = np.array([0, 0, S])[:nb]
    anchor = np.array([3, 10, 0])[:nb]
    valid = np.ones(nb * 4, np.uint8)
    valid[6:8] = 0                        # block 1 at anchor 10 overflows S = 12
    return rng, cfg, layers, ck, cv, emb, base, anchor, valid


def test_body_equals_dense_mask_body():
    _, cfg, layers, ck, cv, emb, base, anchor, valid = _setup()
    a = body_forward(emb, layers, ck, cv, base, anchor, valid, cfg)
    b = body_forward_dense(emb, layers, ck, cv, base, anchor, valid, cfg)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_invalid_rows_and_empty_blocks_are_zero():
    _, cfg, layers, ck, cv, emb, base, anchor, valid = _setup()
    anchor = anchor.copy()
    anchor[2] = -1
    out = body_forward(emb, layers, ck, cv, base, anchor, valid, cfg)
    assert (out[6:8] == 0).all() and (out[8:12] == 0).all()
    assert (np.abs(out[:6]) > 0).all()


def test_zero_output_projections_return_embeddings():
    _, cfg, layers, ck, cv, emb, base, anchor, valid = _setup()
    for W in layers:
        W["wo"] = np.zeros_like(W["wo"])
        W["w_down"] = np.zeros_like(W["w_down"])
    out = body_forward(emb, layers, ck, cv, base, anchor, valid, cfg)
    keep = valid.astype(bool)
    assert np.array_equal(out[keep], emb[keep])


def test_information_boundary_and_block_independence():
    _, cfg, layers, ck, cv, emb, base, anchor, valid = _setup()
    ref = body_forward(emb, layers, ck, cv, base, anchor, valid, cfg)
    ck2 = [k.copy() for k in ck]
    cv2 = [v.copy() for v in cv]
    for l in range(len(ck)):
        ck2[l][:, 3:] += 10.0            # block 0 (anchor 3, base 0) must not see rows >= 3
        cv2[l][:, 3:] = np.nan
    emb2 = emb.copy()
    emb2[4:] = np.nan                     # other blocks
    out = body_forward(emb2, layers, ck2, cv2, base, anchor, valid, cfg)
    assert np.array_equal(out[:4], ref[:4])


def test_permuting_blocks_permutes_outputs():
    _, cfg, layers, ck, cv, emb, base, anchor, valid = _setup()
    ref = body_forward(emb, layers, ck, cv, base, anchor, valid, cfg).reshape(3, 4, -1)
    perm = [2, 0, 1]
    out = body_forward(emb.reshape(3, 4, -1)[perm].reshape(12, -1), layers, ck, cv, base[perm],
                       anchor[perm], valid.reshape(3, 4)[perm].reshape(-1), cfg).reshape(3, 4, -1)
    assert np.array_equal(out, ref[perm])


def test_zeroing_reading_matters_only_inside_multilayer_blocks():
    # The reading taken: only returned rows are zeroed. The rejected reading
    # (zero invalid rows after every layer) agrees for one layer and differs
    # for two layers when a block has invalid rows.
    for n_l, same in ((1, True), (2, False)):
        _, cfg, layers, ck, cv, emb, base, anchor, valid = _setup(n_l=n_l)
        a = body_forward(emb, layers, ck, cv, base, anchor, valid, cfg)
        b = body_forward(emb, layers, ck, cv, base, anchor, valid, cfg, zero_invalid_each_layer=True)
        assert np.allclose(a[:4], b[:4], rtol=0, atol=0)                # block 0 fully valid
        assert np.allclose(a[4:6], b[4:6], rtol=0, atol=1e-15) == same  # block 1 has invalid rows


# --- Closed forms of one draft layer's composition -------------------------
# The workload lists the layer as RMSNorm -> QKV -> RoPE -> attention -> o_proj
# (residual), then RMSNorm -> SwiGLU MLP (residual); NeMo RL "DFlash Draft
# Body", How It Works, step 3 runs the blocks through these draft decoder
# layers. With every embedding row equal to c * 1, every norm weight a constant
# and the V / o_proj / gate / up / down matrices constant, every quantity in the
# layer is a scalar per component and the output has a closed form written out
# below by hand. The wq / wk matrices stay random: all V rows a block can see
# are equal, so the softmax weights (and RoPE) cannot change the result.
# Swapping w_gate with w_up, or attn_norm with mlp_norm, changes that closed
# form, so either swap in the oracle fails these tests.

def _scalar_layer(rng, H, Hq, Hkv, D, I, alpha, mu, beta, omega, g, u, delta):
    return dict(
        attn_norm=np.full(H, alpha), mlp_norm=np.full(H, mu),
        wq=rng.normal(size=(Hq * D, H)), wk=rng.normal(size=(Hkv * D, H)),
        wv=np.full((Hkv * D, H), beta / H), wo=np.full((H, Hq * D), omega / (Hq * D)),
        w_gate=np.full((I, H), g / H), w_up=np.full((I, H), u / H), w_down=np.full((H, I), delta / I))


def _scalar_layer_expected(c, alpha, mu, beta, omega, g, u, delta, eps):
    s0 = c / np.sqrt(c * c + eps)                 # RMSNorm of a constant row, before its weight
    v = beta * (s0 * alpha)                        # every V row, every component
    h1 = c + omega * v                             # attention output = v; o_proj adds omega * v
    s1 = h1 / np.sqrt(h1 * h1 + eps)
    gate, up = g * s1 * mu, u * s1 * mu
    return h1 + delta * (gate / (1.0 + np.exp(-gate))) * up


@pytest.mark.parametrize("alpha,mu,g,u", [
    (1.3, 0.6, 1.5, -0.7),       # generic: both swaps change the result
    (0.0, 0.9, 1.5, -0.7),       # zero attention norm: q = k = v = 0, the attention adds nothing
    (0.9, 0.0, 1.5, -0.7),       # zero MLP norm: gate = up = 0, the MLP adds nothing
    (1.1, 0.8, -60.0, 2.0),      # gate driven far negative: SiLU(gate) ~ 0, the MLP vanishes
])
def test_layer_composition_closed_form(alpha, mu, g, u):
    rng = np.random.default_rng(7)
    H, Hq, Hkv, D, I, bs = 16, 4, 2, 8, 24, 4
    cfg = _cfg(bs=bs, Hq=Hq, Hkv=Hkv, D=D)
    c, beta, omega, delta = 0.8, 0.9, 1.7, 1.2
    layer = _scalar_layer(rng, H, Hq, Hkv, D, I, alpha, mu, beta, omega, g, u, delta)
    # Two blocks: anchor 0 (no context) and anchor 5, whose context V rows are
    # set equal to the block's own V so that the closed form still holds.
    s0 = c / np.sqrt(c * c + cfg["rms_eps"])
    ck = [rng.normal(size=(Hkv, 8, D))]
    cv = [np.full((Hkv, 8, D), beta * s0 * alpha)]
    emb = np.full((2 * bs, H), c)
    out = body_forward(emb, [layer], ck, cv, np.array([0, 0]), np.array([0, 5]),
                       np.ones(2 * bs, np.uint8), cfg)
    want = _scalar_layer_expected(c, alpha, mu, beta, omega, g, u, delta, cfg["rms_eps"])
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)
    # The swapped compositions give different values for these parameters.
    swapped_mlp = _scalar_layer_expected(c, alpha, mu, beta, omega, u, g, delta, cfg["rms_eps"])
    swapped_norms = _scalar_layer_expected(c, mu, alpha, beta, omega, g, u, delta, cfg["rms_eps"])
    assert abs(swapped_norms - want) > 1e-3
    if mu != 0.0:                # with a zero MLP norm both MLP orders add exactly nothing
        assert abs(swapped_mlp - want) > 1e-3


def test_two_layer_composition_closed_form():
    # The second layer reads the first layer's residual stream: applying the
    # scalar closed form twice (with each layer's own constants) gives the body.
    rng = np.random.default_rng(8)
    H, Hq, Hkv, D, I, bs = 16, 4, 2, 8, 24, 4
    cfg = _cfg(bs=bs, Hq=Hq, Hkv=Hkv, D=D)
    p1 = dict(alpha=1.3, mu=0.6, beta=0.9, omega=1.7, g=1.5, u=-0.7, delta=1.2)
    p2 = dict(alpha=0.7, mu=1.4, beta=-0.5, omega=0.8, g=-0.4, u=1.1, delta=0.9)
    layers = [_scalar_layer(rng, H, Hq, Hkv, D, I, **p1), _scalar_layer(rng, H, Hq, Hkv, D, I, **p2)]
    c = 0.8
    emb = np.full((bs, H), c)
    ck = [np.zeros((Hkv, 1, D))] * 2
    out = body_forward(emb, layers, ck, ck, np.array([0]), np.array([0]), np.ones(bs, np.uint8), cfg)
    h1 = _scalar_layer_expected(c, eps=cfg["rms_eps"], **p1)
    want = _scalar_layer_expected(h1, eps=cfg["rms_eps"], **p2)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)
