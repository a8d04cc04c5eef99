"""One whole training step through the library, against the oracle's chain
(NeMo RL "DFlash Draft Body", How It Works, steps 1-4 and Scope: the body is
trained with an optimizer step; angelspec "DFlash", How it works, Loss, and
Configuration: the LM head is the target's, frozen).

GPU: dflash_build_plan -> dflash_ctx_proj_train (keeps C) ->
dflash_body_forward_train -> dflash_lm_head_ce_train (keeps the logits) ->
dflash_lm_head_ce_backward_saved (with the head transposed once by
dflash_lm_head_transpose) -> dflash_body_backward ->
dflash_ctx_proj_backward (adds the context path's share of every Wk / Wv
gradient), the chain the benchmark's training step runs. Oracle: build_plan,
ctx_proj/ctx_kv, body_forward, lm_head_ce, lm_head_ce_backward, body_backward,
ctx_kv_weight_grads, ctx_proj_backward, each pinned on its own and their sum by
central differences of a whole step's loss. Targets are the sequence's own
tokens at each block position.

Tolerance: fp32 chains every fp32 step: rel-L2 1e-5 of each gradient's scale.
bf16: the tolerance of the body backward (rel-L2 3e-2, max-abs 6e-2 of the
largest magnitude), whose analysis covers the extra bf16 rounding of d_out and
of the context gradients on their way to W_proj."""
import math

import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle
from dflash_synth import WORKLOADS, Rng, make_training_inputs, scaled
from tests.helpers import TrainingRun, layers64, np64, oracle_cfg

pytestmark = pytest.mark.gpu
NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def _cmp(gpu, ref, tol, what):
    g = np64(gpu).reshape(ref.shape)
    assert np.isfinite(g).all(), what
    err = g - ref
    rel = float(np.sqrt((err * err).sum()) / (np.sqrt((ref * ref).sum()) or 1.0))
    assert rel <= tol[0], f"{what}: rel-L2 {rel:.3e}"
    assert float(np.abs(err).max()) <= tol[1] * float(np.abs(ref).max()), what


def _case(name):
    """(workload, (rel-L2, max-abs fraction), vocabulary) of the two training cases."""
    if name == "f32":
        return scaled(WORKLOADS["c1"], batch=2, num_layers=2, anchors_per_row=4), (1e-5, 1e-4), 301
    w = scaled(WORKLOADS["c3"], batch=2, seq_len=160, num_target_layers=2, target_hidden=128, hidden=256,
               num_q_heads=4, num_kv_heads=2, intermediate=512, num_layers=2, block_size=16, anchors_per_row=4,
               seed=91)
    return w, (3e-2, 6e-2), 999


def _setup(w, vocab, seed):
    """Seeded inputs of a training step: states, embeddings, weights, a shorter last row, tokens, frozen head."""
    dev = "cuda"
    mask = torch.ones((w.batch, w.seq_len), dtype=torch.uint8, device=dev)
    mask[-1, w.seq_len - w.seq_len // 5:] = 0                   # a shorter last row
    inp = make_training_inputs(w, dev, plan_seed=seed, mask=mask)
    rng = Rng(seed + 100, dev)
    tokens = rng.integers("train.tokens", 0, vocab - 1, (w.batch, w.seq_len)).to(torch.int32)
    W_lm = rng.normal("train.lm_head", (vocab, w.hidden), std=1 / math.sqrt(w.hidden), dtype=w.torch_dtype)
    cfg = d.config_from_workload(w)
    W_t = torch.empty(d.dflash_lm_head_transpose_size(cfg, vocab), dtype=torch.uint8, device=dev)
    d.dflash_lm_head_transpose(cfg, W_lm, W_t)                   # the head is frozen: transposed once
    return dict(inp=inp, tokens=tokens, W_lm=W_lm, W_t=W_t)


def _step(w, vocab, tau, setup):
    """The GPU chain over the setup's inputs, with the weights its tensors hold now."""
    dev = "cuda"
    inp, tokens, W_lm = setup["inp"], setup["tokens"], setup["W_lm"]
    run = TrainingRun(d, w, inp)
    run.plan()
    cfg, bs, R, H, L = run.cfg, w.block_size, w.num_blocks * w.block_size, w.hidden, w.num_layers
    C = torch.empty((run.T, H), dtype=w.torch_dtype, device=dev)
    d.dflash_ctx_proj_train(cfg, inp["states"], w.target_hidden, run.T * w.target_hidden, run.T, run.ctx_pos,
                            inp["w_proj"], inp["layers"], run.ctx_k, run.ctx_v, run.T, 0, C, run.ws)
    pos = run.positions.reshape(-1).long().clamp(0, w.seq_len - 1)
    row = torch.arange(R, device=dev) // (bs * w.anchors_per_row)
    targets = tokens[row, pos].contiguous()
    loss_mask = run.loss_mask.reshape(-1).contiguous()
    reserve = torch.empty(d.dflash_body_train_reserve_size(cfg, w.num_blocks), dtype=torch.uint8, device=dev)
    d.dflash_body_forward_train(cfg, w.num_blocks, inp["emb"], inp["layers"], run.ctx_k, run.ctx_v, run.T,
                                run.base, run.anchors.reshape(-1), run.valid.reshape(-1), run.out, reserve, run.ws)
    ce = torch.empty(R, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    ws = torch.empty(d.dflash_lm_head_ce_workspace_size(R, vocab), dtype=torch.uint8, device=dev)
    logits = torch.empty(d.dflash_lm_head_ce_logits_size(R, vocab), dtype=torch.uint8, device=dev)
    d.dflash_lm_head_ce_train(cfg, run.out, W_lm, targets, loss_mask, tau, ce, loss, logits, ws)
    d_out = torch.empty_like(run.out)
    ws = torch.empty(d.dflash_lm_head_ce_backward_workspace_size(cfg, R, vocab), dtype=torch.uint8, device=dev)
    d.dflash_lm_head_ce_backward_saved(cfg, R, logits, W_lm, targets, loss_mask, tau, ce, 1.0, d_out, ws,
                                       lm_head_t=setup["W_t"])
    grads = [{k: torch.empty(tuple(v.shape), dtype=torch.float32, device=dev) for k, v in Lw.items()}
             for Lw in inp["layers"]]
    dck = [torch.empty((w.num_kv_heads, run.T, w.head_dim), dtype=torch.float32, device=dev) for _ in range(L)]
    dcv = [torch.empty((w.num_kv_heads, w.head_dim, run.T), dtype=torch.float32, device=dev) for _ in range(L)]
    demb = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = torch.empty(d.dflash_body_backward_workspace_size(cfg, w.num_blocks), dtype=torch.uint8, device=dev)
    d.dflash_body_backward(cfg, w.num_blocks, reserve, inp["layers"], run.ctx_k, run.ctx_v, run.T, run.base,
                           run.anchors.reshape(-1), run.valid.reshape(-1), d_out, demb, grads, dck, dcv, ws)
    Kt = w.num_target_layers * w.target_hidden
    dW = torch.empty((H, Kt), dtype=torch.float32, device=dev)
    ws = torch.empty(d.dflash_ctx_proj_backward_workspace_size(cfg, run.T), dtype=torch.uint8, device=dev)
    d.dflash_ctx_proj_backward(cfg, inp["states"], w.target_hidden, run.T * w.target_hidden, run.T, run.ctx_pos,
                               inp["layers"], dck, dcv, run.T, 0, dW, None, ws, ctx_hidden=C,
                               d_wk=[g["wk"] for g in grads], d_wv=[g["wv"] for g in grads])
    torch.cuda.synchronize()
    return dict(inp=inp, run=run, W_lm=W_lm, targets=targets, loss_mask=loss_mask, loss=float(loss.item()),
                grads=grads, demb=demb, dW=dW)


def _oracle(w, s, tau, layers=None, w_proj=None):
    """The oracle's chain over the same seeded inputs; layers / w_proj (fp64) replace the
    weights the inputs were made with (the oracle's own update of them, for a later step)."""
    inp, run = s["inp"], s["run"]
    bs, S, N = w.block_size, w.seq_len, w.anchors_per_row
    plan = oracle.build_plan(inp["mask"].cpu().numpy(), inp["sample_ids"].cpu().numpy(), inp["step"],
                             inp["plan_seed"], N, bs)
    anchors = plan[0].reshape(-1)
    valid = plan[2].reshape(-1)
    assert np.array_equal(run.anchors.cpu().numpy().reshape(-1), anchors)
    layers = layers64(inp["layers"]) if layers is None else layers
    X = oracle.concat_target_states(np64(inp["states"]))
    pos = np.arange(w.batch * S) % S
    C = oracle.ctx_proj(X, np64(inp["w_proj"]) if w_proj is None else w_proj)
    ck, cv = oracle.ctx_kv(C, layers, pos, w.num_kv_heads, w.head_dim, w.rope_theta)
    base = np.arange(len(anchors)) // N * S
    cfg = oracle_cfg(w)
    emb = np64(inp["emb"])
    out = oracle.body_forward(emb, layers, ck, cv, base, anchors, valid, cfg)
    t = s["targets"].cpu().numpy()
    m = s["loss_mask"].cpu().numpy()
    _, loss = oracle.lm_head_ce(out, np64(s["W_lm"]), t, m, bs, tau)
    d_out = oracle.lm_head_ce_backward(out, np64(s["W_lm"]), t, m, bs, tau)
    d_emb, grads, dck, dcv = oracle.body_backward(emb, layers, ck, cv, base, anchors, valid, cfg, d_out)
    dWk, dWv = oracle.ctx_kv_weight_grads(C, pos, dck, dcv, w.num_kv_heads, w.head_dim, w.rope_theta)
    for l in range(w.num_layers):
        grads[l]["wk"] = grads[l]["wk"] + dWk[l]
        grads[l]["wv"] = grads[l]["wv"] + dWv[l]
    _, dW = oracle.ctx_proj_backward(X, pos, layers, dck, dcv, w.num_kv_heads, w.head_dim, w.rope_theta)
    return loss, d_emb, grads, dW


@pytest.mark.parametrize("name", ["f32", "bf16"])
def test_training_step_matches_the_oracle_chain(name):
    w, tol, vocab = _case(name)
    tau = 4.0
    s = _step(w, vocab, tau, _setup(w, vocab, 13))
    loss, d_emb, grads, dW = _oracle(w, s, tau)
    assert abs(s["loss"] - loss) <= (1e-5 if name == "f32" else 1e-2) * abs(loss)
    _cmp(s["demb"], d_emb, tol, "d_block_embeds")
    for l in range(w.num_layers):
        for k in NAMES:
            _cmp(s["grads"][l][k], grads[l][k], tol, f"layer {l} d_{k}")
    _cmp(s["dW"], dW, tol, "d_w_proj")


def _adam_tensor(weight, grad):
    return {"master": weight.float().reshape(-1).clone(), "exp_avg": torch.zeros(weight.numel(), device="cuda"),
            "exp_avg_sq": torch.zeros(weight.numel(), device="cuda"), "grad": grad.reshape(-1),
            "weight": weight.reshape(-1)}


@pytest.mark.parametrize("name", ["f32", "bf16"])
def test_second_step_after_the_optimizer(name):
    """Two training steps with the AdamW step between them (NeMo RL "DFlash Draft
    Body", How It Works, step 1: the body is trained with an optimizer step): the
    second step's forward reads the working copies the optimizer wrote. The oracle
    updates its own weights from its own gradients (fp64) and rounds them to the
    config dtype, as a working copy is; the second step's loss and gradients are
    compared at the first step's bar. The first step moves an entry by
    lr * g / (|g| + eps); with eps = lr its derivative in g is at most 1, so the
    two sides' gradient differences carry over to the weights at most one for
    one (with eps near zero, an entry whose tiny gradient differs in sign between
    the two sides would move by +-lr)."""
    w, tol, vocab = _case(name)
    tau = 4.0
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-3, weight_decay=0.01)
    setup = _setup(w, vocab, 17)
    inp = setup["inp"]
    lay0, wp0 = layers64(inp["layers"]), np64(inp["w_proj"])        # before the update
    s1 = _step(w, vocab, tau, setup)
    _, _, g1, dW1 = _oracle(w, s1, tau)
    tensors = [_adam_tensor(Lw[k], G[k]) for Lw, G in zip(inp["layers"], s1["grads"]) for k in NAMES]
    tensors.append(_adam_tensor(inp["w_proj"], s1["dW"]))
    d.dflash_adamw_step(s1["run"].cfg.dtype, tensors, step=1, **hp)
    torch.cuda.synchronize()

    def update(w0, g):
        w1, _, _ = oracle.adamw_step(w0, g, np.zeros_like(w0), np.zeros_like(w0), 1, **hp)
        return np64(torch.from_numpy(w1).to(w.torch_dtype))
    lay1 = [{k: update(L[k], G[k]) for k in NAMES} for L, G in zip(lay0, g1)]
    wp1 = update(wp0, dW1)
    if name == "f32":                                  # the working copies themselves, against the oracle's
        for l in range(w.num_layers):
            for k in NAMES:
                _cmp(inp["layers"][l][k] - torch.from_numpy(lay0[l][k]).cuda(), lay1[l][k] - lay0[l][k],
                     (1e-4, 1e-3), f"layer {l} {k} update")
    s2 = _step(w, vocab, tau, setup)
    loss, d_emb, grads, dW = _oracle(w, s2, tau, layers=lay1, w_proj=wp1)
    assert abs(s2["loss"] - loss) <= (1e-5 if name == "f32" else 1e-2) * abs(loss)
    _cmp(s2["demb"], d_emb, tol, "step 2 d_block_embeds")
    for l in range(w.num_layers):
        for k in NAMES:
            _cmp(s2["grads"][l][k], grads[l][k], tol, f"step 2 layer {l} d_{k}")
    _cmp(s2["dW"], dW, tol, "step 2 d_w_proj")
