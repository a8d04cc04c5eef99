"""dflash_lm_head_ce vs the draft-loss oracle (angelspec "DFlash", How it
works, Loss: cross-entropy with an exponential positional decay favouring
early block positions; NeMo RL "DFlash Draft Body", step 4: loss mask).

Tolerance: logits are fp32 sums of exact bf16 (or fp32) products, the
softmax statistics use fp32 exp/log; the CE of a row is O(log V) ~ 12, and
the fp32 error of every step is below 1e-6 of that, so CE values must agree
with the fp64 oracle to rel-L2 1e-5 and max-abs 1e-4 (fp32 inputs: 1e-6 / 1e-5)."""
import math

import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle
from dflash_synth import WORKLOADS, Rng, scaled
from tests.helpers import compare, np64

pytestmark = pytest.mark.gpu
CE_TOL = dict(rel_l2=1e-5, max_abs=1e-4)
CE_TOL_F32 = dict(rel_l2=1e-6, max_abs=1e-5)


def _inputs(w, rows, vocab, seed, dev="cuda"):
    rng = Rng(seed, dev)
    h = rng.normal("lm.hidden", (rows, w.hidden), dtype=w.torch_dtype)
    W = rng.normal("lm.head", (vocab, w.hidden), std=1 / math.sqrt(w.hidden), dtype=w.torch_dtype)
    t = rng.integers("lm.targets", 0, vocab - 1, (rows,)).to(torch.int32)
    k = torch.arange(rows, device=dev) % w.block_size
    mask = (k != 0).to(torch.uint8)                     # the anchor row of every block is excluded
    return h, W, t, mask


def _run(w, h, W, t, mask, tau):
    cfg = d.config_from_workload(w)
    rows, vocab = h.shape[0], W.shape[0]
    ce = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    loss = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    ws = torch.empty(d.dflash_lm_head_ce_workspace_size(rows, vocab), dtype=torch.uint8, device="cuda")
    d.dflash_lm_head_ce(cfg, h, W, t, mask, tau, ce, loss, ws)
    torch.cuda.synchronize()
    return ce, float(loss.item())


SMALL = scaled(WORKLOADS["c3"], hidden=256, num_q_heads=4, num_kv_heads=2, intermediate=512, num_layers=1)


@pytest.mark.parametrize("w,rows,vocab,tol", [
    (SMALL, 48, 1000, CE_TOL),                          # ragged vocabulary (not a multiple of 128)
    (SMALL, 300, 4099, CE_TOL),                         # ragged rows and vocabulary
    (WORKLOADS["c1"], 32, 777, CE_TOL_F32),
])
def test_all_rows_small(w, rows, vocab, tol):
    h, W, t, mask = _inputs(w, rows, vocab, seed=rows + vocab)
    t[5] = -1                                           # targets outside the vocabulary: excluded rows
    t[9] = vocab
    tau = 3.0
    ce, loss = _run(w, h, W, t, mask, tau)
    ref_ce, ref_loss = oracle.lm_head_ce(np64(h), np64(W), t.cpu().numpy(), mask.cpu().numpy(), w.block_size, tau)
    compare(ce, ref_ce, tol, "row CE")
    keep = mask.clone()
    keep[5] = 0
    keep[9] = 0
    assert (ce.cpu()[keep.cpu() == 0] == 0).all()
    assert abs(loss - ref_loss) <= tol["max_abs"]


def test_full_size_block_rows_sampled():
    # The 5-layer training shape: 256 blocks of 16 rows, hidden 4096, vocabulary 151936.
    w = WORKLOADS["c3"]
    rows, vocab, tau = w.num_blocks * w.block_size, 151936, 7.0
    h, W, t, mask = _inputs(w, rows, vocab, seed=5)
    ce, loss = _run(w, h, W, t, mask, tau)
    ce_h = ce.cpu().numpy().astype(np.float64)
    m = mask.cpu().numpy().astype(bool)
    assert np.isfinite(ce_h).all() and (ce_h[~m] == 0).all() and (ce_h[m] > 0).all()
    sample = np.array([1, 2, 15, 17, 1000, 2049, 4094, 4095])
    Wd = np64(W)
    ref = oracle.lm_head_ce_rows(np64(h[torch.from_numpy(sample).cuda()]), Wd, t.cpu().numpy()[sample])
    compare(torch.from_numpy(ce_h[sample]), ref, CE_TOL, "sampled row CE")
    # The loss is the decayed weighted mean of the row CEs the kernel produced.
    wts = oracle.position_weights(rows, w.block_size, tau) * m
    assert abs(loss - float((wts * ce_h).sum() / wts.sum())) <= 1e-9 * abs(loss)


def test_no_selected_rows_gives_zero_loss():
    w = SMALL
    h, W, t, mask = _inputs(w, 32, 500, seed=9)
    ce, loss = _run(w, h, W, t, torch.zeros_like(mask), 2.0)
    assert loss == 0.0 and (ce.cpu() == 0).all()


# ---------------------------------------------------------------- backward
# dflash_lm_head_ce_backward vs oracle.lm_head_ce_backward (pinned by central
# differences of the loss). fp32: every step is fp32, so the forward's fp32 bar
# relative to the gradient's scale. bf16: dz is rounded to bf16 once before its
# product with W_lm and d_hidden once on output, each a relative 2^-9; the
# softmax and both accumulations are fp32: rel-L2 1e-2 and max-abs 2e-2 of the
# largest magnitude hold that with room.
GRAD_TOL = dict(rel_l2=1e-2, max_rel=2e-2)
GRAD_TOL_F32 = dict(rel_l2=1e-5, max_rel=1e-4)


def _cmp_rel(gpu, ref, tol, what):
    g = np64(gpu).reshape(ref.shape)
    assert np.isfinite(g).all(), what
    err = g - ref
    rel = float(np.sqrt((err * err).sum()) / (np.sqrt((ref * ref).sum()) or 1.0))
    scale = float(np.abs(ref).max())
    assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3e}"
    assert float(np.abs(err).max()) <= tol["max_rel"] * scale, f"{what}: max-abs {np.abs(err).max():.3e} vs {scale:.3e}"


def _run_bwd(w, h, W, t, mask, tau, ce, d_loss=1.0, W_t=None):
    cfg = d.config_from_workload(w)
    rows, vocab = h.shape[0], W.shape[0]
    dh = torch.full_like(h, float("nan"))
    ws = torch.empty(d.dflash_lm_head_ce_backward_workspace_size(cfg, rows, vocab), dtype=torch.uint8, device="cuda")
    d.dflash_lm_head_ce_backward(cfg, h, W, t, mask, tau, ce, d_loss, dh, ws, lm_head_t=W_t)
    torch.cuda.synchronize()
    return dh


@pytest.mark.parametrize("w,rows,vocab,tol", [
    (SMALL, 48, 1000, GRAD_TOL),
    (SMALL, 300, 4099, GRAD_TOL),
    (WORKLOADS["c1"], 32, 777, GRAD_TOL_F32),
])
def test_backward_all_rows_small(w, rows, vocab, tol):
    h, W, t, mask = _inputs(w, rows, vocab, seed=rows + vocab + 1)
    t[5] = -1
    t[9] = vocab
    tau = 3.0
    ce, _ = _run(w, h, W, t, mask, tau)
    dh = _run_bwd(w, h, W, t, mask, tau, ce)
    ref = oracle.lm_head_ce_backward(np64(h), np64(W), t.cpu().numpy(), mask.cpu().numpy(), w.block_size, tau)
    _cmp_rel(dh, ref, tol, "d_hidden")
    skip = (mask == 0).cpu().numpy()
    skip[[5, 9]] = True
    assert (dh.cpu()[torch.from_numpy(skip)] == 0).all()
    # Linear in d_loss: doubling it doubles every element exactly; zero gives zeros.
    assert torch.equal(_run_bwd(w, h, W, t, mask, tau, ce, 2.0), 2 * dh)
    assert (_run_bwd(w, h, W, t, mask, tau, ce, 0.0) == 0).all()


def test_backward_full_size_sampled_blocks():
    # 4096 block rows x vocabulary 151936 x hidden 4096. The oracle differentiates
    # three whole blocks (so each row keeps its in-block position); its
    # normaliser covers only those rows, so its result is rescaled by the ratio
    # of that normaliser to the one over all rows.
    w = WORKLOADS["c3"]
    rows, vocab, tau = w.num_blocks * w.block_size, 151936, 7.0
    h, W, t, mask = _inputs(w, rows, vocab, seed=6)
    ce, _ = _run(w, h, W, t, mask, tau)
    dh = _run_bwd(w, h, W, t, mask, tau, ce)
    bs = w.block_size
    blocks = [0, 131, 255]
    idx = np.concatenate([np.arange(n * bs, (n + 1) * bs) for n in blocks])
    m_all = mask.cpu().numpy()
    wts = oracle.position_weights(rows, bs, tau) * (m_all != 0)
    sub = torch.from_numpy(idx).cuda()
    ref = oracle.lm_head_ce_backward(np64(h[sub]), np64(W), t.cpu().numpy()[idx], m_all[idx], bs, tau)
    ref *= wts[idx].sum() / wts.sum()
    _cmp_rel(dh[sub], ref, GRAD_TOL, "sampled d_hidden")
    assert torch.isfinite(dh.float()).all()


# ---------------------------------------------------------------- kept logits
# dflash_lm_head_ce_train keeps the fp32 logits; dflash_lm_head_ce_backward_saved
# takes the gradient from them. The forward runs the same GEMM and reductions as
# dflash_lm_head_ce, so the row CEs and the loss are bit-identical; the logits are
# fp32 sums of exact products, within the forward's bar of hidden W^T in fp64.
# The saved backward recovers lse = row_ce + z_target with the forward's own
# target logit, where the recomputing backward recomputes that logit as a dot
# product (a different fp32 summation order, ~1e-6 apart): the two d_hidden agree
# to that, i.e. up to a bf16 rounding of dz flipping now and then (rel-L2 1e-3),
# and each meets the oracle's bar.
SAVED_VS_RECOMPUTE = dict(rel_l2=1e-3, max_rel=1e-2)


def _run_train(w, h, W, t, mask, tau):
    cfg = d.config_from_workload(w)
    rows, vocab = h.shape[0], W.shape[0]
    ce = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    loss = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    ws = torch.empty(d.dflash_lm_head_ce_workspace_size(rows, vocab), dtype=torch.uint8, device="cuda")
    nbytes = d.dflash_lm_head_ce_logits_size(rows, vocab)
    ldl = (vocab + 63) // 64 * 64
    assert nbytes == rows * ldl * 4
    logits = torch.full((rows, ldl), float("nan"), dtype=torch.float32, device="cuda")
    d.dflash_lm_head_ce_train(cfg, h, W, t, mask, tau, ce, loss, logits, ws)
    torch.cuda.synchronize()
    return ce, float(loss.item()), logits


def _transposed_head(w, W):
    cfg = d.config_from_workload(w)
    W_t = torch.full((d.dflash_lm_head_transpose_size(cfg, W.shape[0]),), 255, dtype=torch.uint8, device="cuda")
    d.dflash_lm_head_transpose(cfg, W, W_t)
    torch.cuda.synchronize()
    return W_t


def _run_bwd_saved(w, rows, logits, W, t, mask, tau, ce, d_loss=1.0, W_t=None):
    cfg = d.config_from_workload(w)
    vocab, H = W.shape
    dh = torch.full((rows, H), float("nan"), dtype=W.dtype, device="cuda")
    ws = torch.empty(d.dflash_lm_head_ce_backward_workspace_size(cfg, rows, vocab), dtype=torch.uint8, device="cuda")
    d.dflash_lm_head_ce_backward_saved(cfg, rows, logits, W, t, mask, tau, ce, d_loss, dh, ws, lm_head_t=W_t)
    torch.cuda.synchronize()
    return dh


@pytest.mark.parametrize("w,rows,vocab,tol", [
    (SMALL, 48, 1000, GRAD_TOL),
    (SMALL, 300, 4099, GRAD_TOL),
    (WORKLOADS["c1"], 32, 777, GRAD_TOL_F32),
])
def test_kept_logits_small(w, rows, vocab, tol):
    h, W, t, mask = _inputs(w, rows, vocab, seed=rows + vocab + 2)
    t[5] = -1
    t[9] = vocab
    tau = 3.0
    ce, loss = _run(w, h, W, t, mask, tau)
    ce2, loss2, logits = _run_train(w, h, W, t, mask, tau)
    assert torch.equal(ce, ce2) and loss == loss2
    ref_z = np64(h) @ np64(W).T
    compare(logits[:, :vocab], ref_z, dict(rel_l2=1e-5, max_abs=1e-4) if w.dtype == "bf16" else CE_TOL_F32,
            "kept logits")
    dh = _run_bwd(w, h, W, t, mask, tau, ce)
    dh2 = _run_bwd_saved(w, rows, logits, W, t, mask, tau, ce)
    _cmp_rel(dh2, np64(dh), SAVED_VS_RECOMPUTE if w.dtype == "bf16" else GRAD_TOL_F32, "saved vs recomputed")
    skip = (mask == 0).cpu().numpy()
    skip[[5, 9]] = True
    assert (dh2.cpu()[torch.from_numpy(skip)] == 0).all()
    ref = oracle.lm_head_ce_backward(np64(h), np64(W), t.cpu().numpy(), mask.cpu().numpy(), w.block_size, tau)
    _cmp_rel(dh2, ref, tol, "d_hidden from kept logits")
    assert torch.equal(_run_bwd_saved(w, rows, logits, W, t, mask, tau, ce, 2.0), 2 * dh2)
    # A kept transposed head gives the same bytes, and holds W_lm^T with zero padding columns.
    W_t = _transposed_head(w, W)
    assert torch.equal(_run_bwd_saved(w, rows, logits, W, t, mask, tau, ce, W_t=W_t), dh2)
    assert torch.equal(_run_bwd(w, h, W, t, mask, tau, ce, W_t=W_t), dh)
    H, vp = W.shape[1], (vocab + 63) // 64 * 64
    Wt = W_t.view(W.dtype).reshape(H, vp)
    assert torch.equal(Wt[:, :vocab], W.t()) and (Wt[:, vocab:] == 0).all()


def test_kept_logits_full_size():
    # The training shape: 4096 block rows x vocabulary 151936 x hidden 4096.
    w = WORKLOADS["c3"]
    rows, vocab, tau = w.num_blocks * w.block_size, 151936, 7.0
    h, W, t, mask = _inputs(w, rows, vocab, seed=8)
    ce, loss = _run(w, h, W, t, mask, tau)
    ce2, loss2, logits = _run_train(w, h, W, t, mask, tau)
    assert torch.equal(ce, ce2) and loss == loss2
    sample = torch.tensor([0, 1, 2047, 4095], device="cuda")
    compare(logits[sample, :vocab], np64(h[sample]) @ np64(W).T, dict(rel_l2=1e-5, max_abs=1e-4), "kept logits rows")
    dh = _run_bwd(w, h, W, t, mask, tau, ce)
    dh2 = _run_bwd_saved(w, rows, logits, W, t, mask, tau, ce)
    _cmp_rel(dh2, np64(dh), SAVED_VS_RECOMPUTE, "saved vs recomputed")
