"""dflash_ctx_proj_backward vs the oracle's context-path backward (NeMo RL
"DFlash Draft Body", Scope: training updates W_proj; angelspec "DFlash", How it
works: the target states reach every layer's K/V through W_proj and that
layer's own Wk / Wv). The oracle is pinned by central differences of the
forward context path. With C given, the context path's share of every Wk / Wv
gradient (G^T C) is added to the caller's buffers; C here is a seeded input of
its own (the product does not depend on how C was made), and the buffers start
from seeded values so that "added" is what is checked.

Tolerance: fp32 configs multiply in fp32 (rel-L2 1e-5, max-abs 1e-4 of the
reference's RMS). With bf16 configs the packed gradient G and dC each enter
their product rounded once to bf16 (unit 2^-9), with fp32 sums; every dC and
dW_proj element is a long sum of products carrying at most one such rounding
per factor, so its error stays a few units of 2^-9 relative to the values'
scale: rel-L2 1e-2 and max-abs 5e-2 of the reference's RMS."""
import math

import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle
from dflash_synth import WORKLOADS, Rng, layer_weights, scaled
from tests.helpers import compare, np64

pytestmark = pytest.mark.gpu


def _tol(w, ref):
    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    if w.dtype == "f32":
        return dict(rel_l2=1e-5, max_abs=1e-4 * rms)
    return dict(rel_l2=1e-2, max_abs=5e-2 * rms)


def _inputs(w, T, ctx_total, seed):
    rng = Rng(seed, "cuda")
    kin = w.num_target_layers * w.target_hidden
    X = rng.normal("cb.x", (T, kin), dtype=w.torch_dtype)
    pos = rng.integers("cb.pos", 0, 9000, (T,)).to(torch.int32)
    layers = [layer_weights(w, rng, l) for l in range(w.num_layers)]
    Hkv, D = w.num_kv_heads, w.head_dim
    gk = [rng.normal(f"cb.gk{l}", (Hkv, ctx_total, D), dtype=torch.float32) for l in range(w.num_layers)]
    gv = [rng.normal(f"cb.gv{l}", (Hkv, D, ctx_total), dtype=torch.float32) for l in range(w.num_layers)]
    return X, pos, layers, gk, gv


def _kv_inputs(w, T, seed):
    """C [T, H] (config dtype) and the starting Wk / Wv gradients [Hkv*D, H] (f32)."""
    rng = Rng(seed, "cuda")
    kvd = w.num_kv_heads * w.head_dim
    C = rng.normal("cb.c", (T, w.hidden), dtype=w.torch_dtype)
    wk0 = [rng.normal(f"cb.wk0_{l}", (kvd, w.hidden), dtype=torch.float32) for l in range(w.num_layers)]
    wv0 = [rng.normal(f"cb.wv0_{l}", (kvd, w.hidden), dtype=torch.float32) for l in range(w.num_layers)]
    return C, wk0, wv0


def _gpu(w, X, pos, layers, gk, gv, T, ctx_total, row_offset, with_dc=True, kv=None):
    cfg = d.config_from_workload(w)
    kin = w.num_target_layers * w.target_hidden
    dW = torch.full((w.hidden, kin), float("nan"), dtype=torch.float32, device="cuda")
    dC = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda") if with_dc else None
    ws = torch.empty(d.dflash_ctx_proj_backward_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    extra = {}
    if kv is not None:
        C, wk0, wv0 = kv
        extra = dict(ctx_hidden=C, d_wk=[t.clone() for t in wk0], d_wv=[t.clone() for t in wv0])
    d.dflash_ctx_proj_backward(cfg, X, kin, w.target_hidden, T, pos, layers, gk, gv, ctx_total, row_offset, dW,
                               dC, ws, **extra)
    torch.cuda.synchronize()
    if kv is not None:
        return dW, dC, extra["d_wk"], extra["d_wv"]
    return dW, dC


def _oracle_slices(gk, gv, lo, hi):
    return ([np64(g[:, lo:hi]) for g in gk], [np64(g[:, :, lo:hi]).transpose(0, 2, 1) for g in gv])


def _layers64(layers):
    return [{"wk": np64(L["wk"]), "wv": np64(L["wv"])} for L in layers]


@pytest.mark.parametrize("w,T,ctx_total,row_offset", [
    (WORKLOADS["c1"], 100, 128, 5),                    # fp32, ragged rows, offset into the cache
    (scaled(WORKLOADS["c2"], hidden=256, num_kv_heads=2, num_q_heads=4, num_layers=2, num_target_layers=2,
            target_hidden=256), 200, 300, 37),          # bf16, rows not a multiple of 64
    (scaled(WORKLOADS["c2"], hidden=512, num_kv_heads=2, num_q_heads=8, num_layers=3, num_target_layers=3,
            target_hidden=384), 640, 640, 0),           # bf16, several row tiles, whole cache
])
def test_all_elements(w, T, ctx_total, row_offset):
    X, pos, layers, gk, gv = _inputs(w, T, ctx_total, seed=T)
    dW, dC = _gpu(w, X, pos, layers, gk, gv, T, ctx_total, row_offset)
    gk_o, gv_o = _oracle_slices(gk, gv, row_offset, row_offset + T)
    dC_ref, dW_ref = oracle.ctx_proj_backward(np64(X), pos.cpu().numpy(), _layers64(layers), gk_o, gv_o,
                                              w.num_kv_heads, w.head_dim, w.rope_theta)
    compare(dC, dC_ref, _tol(w, dC_ref), "dC")
    compare(dW, dW_ref, _tol(w, dW_ref), "dW_proj")


@pytest.mark.parametrize("w,T,ctx_total,row_offset", [
    (WORKLOADS["c1"], 100, 128, 5),                    # fp32, ragged rows, offset into the cache
    (scaled(WORKLOADS["c2"], hidden=256, num_kv_heads=2, num_q_heads=4, num_layers=2, num_target_layers=2,
            target_hidden=256), 200, 300, 37),          # bf16, rows not a multiple of 64
    (scaled(WORKLOADS["c2"], hidden=512, num_kv_heads=2, num_q_heads=8, num_layers=3, num_target_layers=3,
            target_hidden=384), 640, 640, 0),           # bf16, several row tiles, whole cache
])
def test_kv_weight_grads_all_elements(w, T, ctx_total, row_offset):
    X, pos, layers, gk, gv = _inputs(w, T, ctx_total, seed=T)
    kv = _kv_inputs(w, T, seed=T + 1)
    dW, dC, dwk, dwv = _gpu(w, X, pos, layers, gk, gv, T, ctx_total, row_offset, kv=kv)
    gk_o, gv_o = _oracle_slices(gk, gv, row_offset, row_offset + T)
    dC_ref, dW_ref = oracle.ctx_proj_backward(np64(X), pos.cpu().numpy(), _layers64(layers), gk_o, gv_o,
                                              w.num_kv_heads, w.head_dim, w.rope_theta)
    compare(dC, dC_ref, _tol(w, dC_ref), "dC")                       # unchanged by the extra product
    compare(dW, dW_ref, _tol(w, dW_ref), "dW_proj")
    sk, sv = oracle.ctx_kv_weight_grads(np64(kv[0]), pos.cpu().numpy(), gk_o, gv_o, w.num_kv_heads, w.head_dim,
                                        w.rope_theta)
    for l in range(w.num_layers):
        compare(dwk[l] - kv[1][l], sk[l], _tol(w, sk[l]), f"dWk layer {l} (added share)")
        compare(dwv[l] - kv[2][l], sv[l], _tol(w, sv[l]), f"dWv layer {l} (added share)")


def test_kv_weight_grads_no_rows_leave_buffers():
    w = scaled(WORKLOADS["c2"], hidden=256, num_kv_heads=2, num_q_heads=4, num_layers=1, num_target_layers=2,
               target_hidden=256)
    X, pos, layers, gk, gv = _inputs(w, 1, 16, seed=3)
    kv = _kv_inputs(w, 1, seed=4)
    dW, _, dwk, dwv = _gpu(w, X, pos, layers, gk, gv, 0, 16, 0, with_dc=False, kv=kv)
    assert (dW == 0).all()
    assert torch.equal(dwk[0], kv[1][0]) and torch.equal(dwv[0], kv[2][0])


def test_no_rows_gives_zero_gradient():
    w = scaled(WORKLOADS["c2"], hidden=256, num_kv_heads=2, num_q_heads=4, num_layers=1, num_target_layers=2,
               target_hidden=256)
    X, pos, layers, gk, gv = _inputs(w, 1, 16, seed=3)
    dW, _ = _gpu(w, X, pos, layers, gk, gv, 0, 16, 0, with_dc=False)
    assert (dW == 0).all()


def test_full_size_sampled():
    # The 5-layer training shape: 8 x 4096 context rows, 5 x 4096 target
    # features, hidden 4096, 8 KV heads of 128.
    w = WORKLOADS["c3"]
    T = w.batch * w.seq_len
    X, pos, layers, gk, gv = _inputs(w, T, T, seed=7)
    kv = _kv_inputs(w, T, seed=8)
    dW, dC, dwk, dwv = _gpu(w, X, pos, layers, gk, gv, T, T, 0, kv=kv)
    assert torch.isfinite(dW).all() and torch.isfinite(dC).all()
    lay = _layers64(layers)
    pos_h = pos.cpu().numpy()
    Hkv, D, th = w.num_kv_heads, w.head_dim, w.rope_theta
    # Whole rows of dC.
    rows = np.array([0, 1, 63, 64, 4095, 20001, T - 1])
    gk_r = [np64(g[:, torch.from_numpy(rows).cuda()]) for g in gk]
    gv_r = [np64(g[:, :, torch.from_numpy(rows).cuda()]).transpose(0, 2, 1) for g in gv]
    ref_rows = oracle.ctx_hidden_grad(gk_r, gv_r, pos_h[rows], lay, Hkv, D, th)
    compare(dC[torch.from_numpy(rows).cuda()], ref_rows, _tol(w, ref_rows), "dC rows")
    # dW_proj entries: whole columns of dC from the oracle (row chunks), then dC^T X.
    cols = np.array([0, 5, 2047, 4095])
    ks = np.array([0, 1, 4095, 4096, 12345, 20479])
    lay_c = [{"wk": L["wk"][:, cols], "wv": L["wv"][:, cols]} for L in lay]
    dc_cols = np.zeros((T, len(cols)))
    # Whole columns of every layer's added Wk / Wv share: G^T C[:, cols], summed over row chunks.
    sk = [np.zeros((Hkv * D, len(cols))) for _ in range(w.num_layers)]
    sv = [np.zeros((Hkv * D, len(cols))) for _ in range(w.num_layers)]
    cols_t = torch.from_numpy(cols).cuda()
    for r0 in range(0, T, 4096):
        sl = slice(r0, r0 + 4096)
        gk_c = [np64(g[:, sl]) for g in gk]
        gv_c = [np64(g[:, :, sl]).transpose(0, 2, 1) for g in gv]
        dc_cols[sl] = oracle.ctx_hidden_grad(gk_c, gv_c, pos_h[sl], lay_c, Hkv, D, th)
        ak, av = oracle.ctx_kv_weight_grads(np64(kv[0][sl][:, cols_t]), pos_h[sl], gk_c, gv_c, Hkv, D, th)
        for l in range(w.num_layers):
            sk[l] += ak[l]
            sv[l] += av[l]
    for l in range(w.num_layers):
        compare(dwk[l][:, cols_t] - kv[1][l][:, cols_t], sk[l], _tol(w, sk[l]), f"dWk layer {l} columns")
        compare(dwv[l][:, cols_t] - kv[2][l][:, cols_t], sv[l], _tol(w, sv[l]), f"dWv layer {l} columns")
    Xk = np64(X[:, torch.from_numpy(ks).cuda()])
    ref = dc_cols.T @ Xk
    got = dW[torch.from_numpy(cols).cuda()][:, torch.from_numpy(ks).cuda()]
    compare(got, ref, _tol(w, ref), "dW_proj entries")
