"""Context projection and the full draft body on the GPU vs the oracle
(angelspec "DFlash", How it works and Configuration; NeMo RL "DFlash Draft
Body", How It Works, steps 1-4), from the tiny fp32 workload to sampled
blocks of the full-size bf16 workloads, plus the pages' invariants."""
import json
import os

import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle
from dflash_synth import WORKLOADS, make_inference_inputs, make_training_inputs, scaled
from tests.helpers import (TrainingRun, compare, layers64, np64, oracle_cfg, oracle_row_context,
                           oracle_training_blocks, tol_for, workspace)

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _c1_seed():
    with open(os.path.join(HERE, "golden", "c1_plan.json")) as f:
        return json.load(f)["seed"]


def _check_plan(run):
    w = run.w
    ref = oracle.build_plan(run.inp["mask"].cpu().numpy(), run.inp["sample_ids"].cpu().numpy(),
                            run.inp["step"], run.inp["plan_seed"], w.anchors_per_row, w.block_size)
    assert np.array_equal(run.anchors.cpu().numpy(), ref[0])
    assert np.array_equal(run.valid.cpu().numpy(), ref[2])
    return ref


def _check_ctx(run, rows):
    """Context K/V of the given cache rows vs the oracle (computed for those rows only)."""
    w, inp = run.w, run.inp
    S = w.seq_len
    layers = layers64(inp["layers"])
    X = oracle.concat_target_states(np64(inp["states"][:, rows]))
    C = oracle.ctx_proj(X, np64(inp["w_proj"]))
    ck, cv = oracle.ctx_kv(C, layers, np.asarray(rows) % S, w.num_kv_heads, w.head_dim, w.rope_theta)
    tol = tol_for(w)
    for l in range(w.num_layers):
        compare(run.ctx_k[l][:, rows], ck[l], tol, f"ctx_k layer {l}")
        compare(run.ctx_v[l][:, :, rows], cv[l].transpose(0, 2, 1), tol, f"ctx_v layer {l}")


def test_tiny_fp32_end_to_end():
    w = WORKLOADS["c1"]
    inp = make_training_inputs(w, "cuda", plan_seed=_c1_seed())
    run = TrainingRun(d, w, inp).run()
    anchors, _, valid, _, _ = _check_plan(run)
    assert anchors.max() >= w.seq_len - w.block_size + 1          # one block overflows the end
    _check_ctx(run, np.arange(w.seq_len))
    ref = oracle_training_blocks(w, inp, anchors, valid, range(w.num_blocks))
    compare(run.out, ref, tol_for(w), "body")
    zero = torch.from_numpy(valid.reshape(-1) == 0).cuda()
    assert zero.any() and (run.out[zero] == 0).all()


SMALL_BF16 = scaled(WORKLOADS["c3"], batch=2, seq_len=300, num_target_layers=2, target_hidden=128,
                    hidden=256, num_q_heads=4, num_kv_heads=2, intermediate=512, num_layers=2,
                    block_size=16, anchors_per_row=6, seed=77)


def test_small_bf16_multilayer_ragged():
    w = SMALL_BF16
    mask = torch.ones((2, 300), dtype=torch.uint8, device="cuda")
    mask[1, 250:] = 0                                             # short second row
    mask[0, 100:110] = 0
    inp = make_training_inputs(w, "cuda", plan_seed=3, mask=mask)
    run = TrainingRun(d, w, inp).run()
    anchors, _, valid, _, _ = _check_plan(run)
    _check_ctx(run, np.arange(2 * w.seq_len))
    ref = oracle_training_blocks(w, inp, anchors, valid, range(w.num_blocks))
    compare(run.out, ref, tol_for(w), "body")


def _invalid_rows_case(w):
    """Blocks with short prefixes and invalid rows inside them: 3 blocks per
    sequence at anchors near the start, each with invalid positions spread over
    the block (including its last row). Empty blocks fill the rest."""
    B, N, bs = w.batch, w.anchors_per_row, w.block_size
    anchors = np.full((B, N), -1, np.int32)
    valid = np.zeros((B, N, bs), np.uint8)
    for b in range(B):
        for i, a in enumerate([1 + b, 6 + 3 * b, 19 + b][:N]):
            anchors[b, i] = a
            valid[b, i] = 1
            valid[b, i, [2 + i, 5, bs - 1]] = 0
    return anchors, valid


def _attention_zeroing_invalid(valid, bs):
    keep = np.asarray(valid, bool).reshape(-1, bs)[:, :, None, None]

    def att(q, k, v, ck, cv, base, anchor):
        return np.where(keep, oracle.block_attention(q, k, v, ck, cv, base, anchor), 0.0)
    return att


@pytest.mark.parametrize("name", ["c1x2", "small_bf16"])
def test_multilayer_invalid_rows_keep_evolving(name):
    # Inside a multi-layer body an invalid row keeps its attention output and
    # evolves like any other row; only the returned rows are zeroed. With short
    # prefixes the block's own rows carry much of each query's attention, so
    # the reading where attention zeroes invalid rows in every layer differs
    # far beyond the tolerance (checked on the oracle here).
    w = scaled(WORKLOADS["c1"], num_layers=2, anchors_per_row=4) if name == "c1x2" else SMALL_BF16
    inp = make_training_inputs(w, "cuda")
    run = TrainingRun(d, w, inp)
    run.plan()
    anchors, valid = _invalid_rows_case(w)
    run.anchors.copy_(torch.from_numpy(anchors))
    run.valid.copy_(torch.from_numpy(valid))
    run.ctx_proj()
    run.body()
    torch.cuda.synchronize()
    blocks = [n for n in range(w.num_blocks) if anchors.reshape(-1)[n] >= 0]
    ref = oracle_training_blocks(w, inp, anchors, valid, blocks)
    rows = torch.from_numpy(np.concatenate([np.arange(n * w.block_size, (n + 1) * w.block_size)
                                            for n in blocks])).cuda()
    compare(run.out[rows], ref, tol_for(w), "body with invalid rows")
    empty = torch.from_numpy(np.repeat(anchors.reshape(-1) < 0, w.block_size)).cuda()
    assert (run.out[empty] == 0).all()
    # The rejected reading, on the oracle: the first sequence's blocks.
    b0 = [n for n in blocks if n < w.anchors_per_row]
    bs = w.block_size
    layers = layers64(inp["layers"])
    ck, cv = oracle_row_context(w, inp, 0, int(anchors.max()), layers)
    e = np.concatenate([np64(inp["emb"][n * bs:(n + 1) * bs]) for n in b0])
    a = anchors.reshape(-1)[b0]
    v = np.concatenate([valid.reshape(-1)[n * bs:(n + 1) * bs] for n in b0])
    alt = oracle.body._body(e, layers, ck, cv, np.zeros(len(b0), np.int64), a, v, oracle_cfg(w),
                            _attention_zeroing_invalid(v, bs), False)
    mine = ref[: len(b0) * bs]
    assert np.linalg.norm(alt - mine) > 4 * tol_for(w)["rel_l2"] * np.linalg.norm(mine)


def test_concat_and_stacked_layouts_agree():
    w = SMALL_BF16
    inp = make_training_inputs(w, "cuda")
    run = TrainingRun(d, w, inp)
    run.ctx_proj()
    k1 = [t.clone() for t in run.ctx_k]
    X = torch.cat([inp["states"][i] for i in range(w.num_target_layers)], dim=-1).contiguous()
    Kt = w.num_target_layers * w.target_hidden
    d.dflash_ctx_proj(run.cfg, X, Kt, w.target_hidden, run.T, run.ctx_pos, inp["w_proj"], inp["layers"],
                      run.ctx_k, run.ctx_v, run.T, 0, run.ws)
    torch.cuda.synchronize()
    for a, b in zip(k1, run.ctx_k):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["c1", "small_bf16"])
def test_ctx_proj_train_keeps_c(name):
    """dflash_ctx_proj_train writes the caches of dflash_ctx_proj bit for bit and
    keeps C = X W_proj^T (angelspec "DFlash", How it works)."""
    w = WORKLOADS["c1"] if name == "c1" else SMALL_BF16
    inp = make_training_inputs(w, "cuda")
    run = TrainingRun(d, w, inp)
    run.ctx_proj()
    k1, v1 = [t.clone() for t in run.ctx_k], [t.clone() for t in run.ctx_v]
    for t in run.ctx_k + run.ctx_v:
        t.fill_(7.0)
    C = torch.full((run.T, w.hidden), float("nan"), dtype=w.torch_dtype, device="cuda")
    d.dflash_ctx_proj_train(run.cfg, inp["states"], w.target_hidden, run.T * w.target_hidden, run.T, run.ctx_pos,
                            inp["w_proj"], inp["layers"], run.ctx_k, run.ctx_v, run.T, 0, C, run.ws)
    torch.cuda.synchronize()
    for a, b in zip(k1 + v1, run.ctx_k + run.ctx_v):
        assert torch.equal(a, b)
    X = oracle.concat_target_states(np64(inp["states"]))
    compare(C, oracle.ctx_proj(X, np64(inp["w_proj"])), tol_for(w), "kept C")


def test_one_layer_bf16_full_size():
    w = WORKLOADS["c2"]
    inp = make_training_inputs(w, "cuda")
    run = TrainingRun(d, w, inp).run()
    anchors, _, valid, _, _ = _check_plan(run)
    _check_ctx(run, np.array([0, 1, 2047, 2048, 5000, 8191]))
    ref = oracle_training_blocks(w, inp, anchors, valid, range(w.num_blocks))
    compare(run.out, ref, tol_for(w), "body (all 1024 rows)")
    # Every reduction order is fixed, so a rerun is bit-identical.
    first = run.out.clone()
    run.body()
    torch.cuda.synchronize()
    assert torch.equal(run.out, first)


def _spread(order, k):
    """k positions spread evenly over an ordering (first and last included)."""
    idx = np.unique(np.round(np.linspace(0, len(order) - 1, k)).astype(int))
    return [int(order[i]) for i in idx]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["c3", "c4"])
def test_five_layer_full_size_sampled(name):
    # Full-size 5-layer bodies. Compared blocks are spread over the whole anchor
    # order and include the longest prefixes: for the 5-layer workload the
    # largest-anchor block of every row plus 24 spread blocks, for the
    # long-context workload its 8 largest anchors plus 16 spread blocks, so
    # split prefixes, pipelined tiles and the combine step all run inside the
    # compared blocks. The oracle projects its own context from the target
    # states; for sequence 0 of the 5-layer workload every cache row of every
    # layer is compared as well.
    w = WORKLOADS[name]
    inp = make_training_inputs(w, "cuda")
    run = TrainingRun(d, w, inp).run()
    anchors, _, valid, _, _ = _check_plan(run)
    flat = anchors.reshape(-1)
    N, bs = w.anchors_per_row, w.block_size
    order = np.argsort(flat, kind="stable")
    if name == "c3":
        must = {int(b * N + np.argmax(flat[b * N:(b + 1) * N])) for b in range(w.batch)}
        want = 32
    else:
        must = set(int(n) for n in order[-8:])
        want = 24
    k = want - len(must)
    while len(must | set(_spread(order, k))) < want:
        k += 1
    blocks = sorted(must | set(_spread(order, k)))
    layers = layers64(inp["layers"])
    contexts = {}
    if name == "c3":
        contexts[0] = oracle_row_context(w, inp, 0, w.seq_len, layers)
        tol = tol_for(w)
        for l in range(w.num_layers):                             # every row of sequence 0
            compare(run.ctx_k[l][:, :w.seq_len], contexts[0][0][l], tol, f"ctx_k layer {l} sequence 0")
            compare(run.ctx_v[l][:, :, :w.seq_len], contexts[0][1][l].transpose(0, 2, 1), tol,
                    f"ctx_v layer {l} sequence 0")
    else:
        _check_ctx(run, np.array([0, 3, 4095, 16384, w.seq_len - 1]))
    rows = np.concatenate([np.arange(n * bs, (n + 1) * bs) for n in blocks])
    ref = oracle_training_blocks(w, inp, anchors, valid, blocks, contexts, layers)
    rel, mx = compare(run.out[torch.from_numpy(rows).cuda()], ref, tol_for(w),
                      f"{name} blocks {blocks}")
    print(f"{name}: {len(blocks)} blocks, anchors {sorted(int(flat[n]) for n in blocks)}, "
          f"rel-L2 {rel:.3e}, max-abs {mx:.3e}", flush=True)
    # Every row of the full output is finite and invalid rows are exactly zero.
    assert torch.isfinite(run.out.float()).all()
    zero = torch.from_numpy(valid.reshape(-1) == 0).cuda()
    assert (run.out[zero] == 0).all()


def test_ragged_cache_body_sampled():
    w = WORKLOADS["c5"]
    inp = make_inference_inputs(w, "cuda")
    cfg = d.config_from_workload(w)
    out = torch.empty((w.num_blocks * w.block_size, w.hidden), dtype=torch.bfloat16, device="cuda")
    ws = workspace(d, cfg, w.num_blocks, 0, "cuda")
    d.dflash_body_forward(cfg, w.num_blocks, inp["emb"], inp["layers"], inp["ctx_k"], inp["ctx_v"],
                          inp["total"], inp["block_ctx_base"], inp["block_anchor"], inp["block_valid"],
                          out, ws)
    torch.cuda.synchronize()
    lens = inp["lengths"].cpu().numpy()
    offs = inp["offsets"].cpu().numpy()
    layers = layers64(inp["layers"])
    bs = w.block_size
    for r in [int(np.argmin(lens)), int(np.argmax(lens)), 7]:
        lo, hi = int(offs[r]), int(offs[r + 1])
        ck = [np64(k[:, lo:hi]) for k in inp["ctx_k"]]
        cv = [np64(v[:, :, lo:hi]).transpose(0, 2, 1) for v in inp["ctx_v"]]
        ref = oracle.body_forward(np64(inp["emb"][r * bs:(r + 1) * bs]), layers, ck, cv, [0],
                                  [int(lens[r])], np.ones(bs, np.uint8), oracle_cfg(w))
        compare(out[r * bs:(r + 1) * bs], ref, tol_for(w), f"request {r} (prefix {lens[r]})")



@pytest.mark.parametrize("batch", [7, 45, 170])
def test_full_width_ragged_rows(batch):
    # One full-width layer (hidden 4096, 32/8 heads, intermediate 12288) over
    # 112, 720 and 2720 block rows: row counts that end inside a tile of every
    # GEMM shape the body picks at this width (128x128 with 8 waves, 128x192,
    # 256x192, 256x256 and plain 128x128), so the last request's rows sit in a
    # ragged tail of each product.
    w = scaled(WORKLOADS["c5"], batch=batch, num_layers=1, min_prefix=1, max_prefix=600, seed=2000 + batch)
    inp = make_inference_inputs(w, "cuda")
    cfg = d.config_from_workload(w)
    out = torch.full((w.num_blocks * w.block_size, w.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = workspace(d, cfg, w.num_blocks, 0, "cuda")
    d.dflash_body_forward(cfg, w.num_blocks, inp["emb"], inp["layers"], inp["ctx_k"], inp["ctx_v"],
                          inp["total"], inp["block_ctx_base"], inp["block_anchor"], inp["block_valid"],
                          out, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    lens = inp["lengths"].cpu().numpy()
    offs = inp["offsets"].cpu().numpy()
    layers = layers64(inp["layers"])
    bs = w.block_size
    for r in sorted({0, int(np.argmax(lens)), batch - 2, batch - 1}):
        lo, hi = int(offs[r]), int(offs[r + 1])
        ck = [np64(k[:, lo:hi]) for k in inp["ctx_k"]]
        cv = [np64(v[:, :, lo:hi]).transpose(0, 2, 1) for v in inp["ctx_v"]]
        ref = oracle.body_forward(np64(inp["emb"][r * bs:(r + 1) * bs]), layers, ck, cv, [0],
                                  [int(lens[r])], np.ones(bs, np.uint8), oracle_cfg(w))
        compare(out[r * bs:(r + 1) * bs], ref, tol_for(w), f"{batch} requests: request {r} (prefix {lens[r]})")

def test_body_invariants_bit_exact():
    w = SMALL_BF16
    inp = make_training_inputs(w, "cuda", plan_seed=5)
    run = TrainingRun(d, w, inp).run()
    ref = run.out.clone()
    run.body()
    torch.cuda.synchronize()
    assert torch.equal(run.out, ref)                              # deterministic
    anchors = run.anchors.cpu().numpy().reshape(-1)
    n = int(np.argmin(np.where(anchors >= 0, anchors, 1 << 30)))   # block with the smallest anchor
    a = int(anchors[n])
    b = n // w.anchors_per_row
    S, bs = w.seq_len, w.block_size
    for l in range(w.num_layers):                                 # context at or after the anchor
        run.ctx_k[l][:, b * S + a: (b + 1) * S] += 5.0
        run.ctx_v[l][:, :, b * S + a: (b + 1) * S] = float("nan")
    emb = inp["emb"]
    saved = emb.clone()
    emb[: n * bs] = float("nan")                                  # every other block's embeddings
    emb[(n + 1) * bs:] = float("nan")
    run.body()
    torch.cuda.synchronize()
    assert torch.equal(run.out[n * bs:(n + 1) * bs], ref[n * bs:(n + 1) * bs])
    emb.copy_(saved)
