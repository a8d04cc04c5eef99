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
