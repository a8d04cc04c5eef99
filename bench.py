"""Benchmark of the DFlash draft-body forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM:
  training-shaped workloads: anchor plan -> context projection (W_proj and every
  layer's context K/V) -> draft body (all layers);
  inference-shaped workload (ragged prefixes, cached context K/V): draft body.

Prints one JSON line. `value` is block positions per second (every block slot
counted). The roofline object describes the kernel with the largest share of
the step time, timed live with HIP events recorded by the library around each
of its launches on the launch stream; the cpu_baseline object is the fp64
oracle timed on this host on a bounded sample of the same workload.

    python bench.py [--workload c3] [--steps 20] [--warmup 5] [--gpus 1]

The JSON line also carries `configs`: the one-layer, 5-layer, long-context and
ragged-cache workloads each timed the same way (step time with median, p10 and
p90 over per-step events, the step's roofline and MFMA fractions, the dominant
kernel's fraction), so every workload's bar is on record in one run.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft block-positions/sec for 5-layer DFlash body forward; % bf16 MFMA / HBM roofline"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}     # dense MI355X matrix peaks
PEAK_HBM_GBS = 8000.0
PEAK_VALU_F32_TFLOPS = 157.3                          # fp32 vector units (FMA = 2 flops)

DESCR = {
    "c1": "tiny fp32 single-layer body: batch 1, target seq 128, 2x256 target layers -> 256, 4/2 heads x 64, block 8, 4 anchors",
    "c2": "one draft layer, bf16: batch 4, target seq 2048, 5x4096 target layers -> 4096, 32/8 heads x 128, block 16, 16 anchors/row",
    "c3": "full 5-layer draft body, bf16: batch 8, target seq 4096, 5x4096 target layers -> 4096, 32/8 heads x 128, SwiGLU 12288, block 16, 32 anchors/row",
    "c4": "long-context 5-layer body, bf16: batch 1, target seq 32768, 512 anchors, block 16",
    "c5": "inference drafting, bf16: 64 requests, prefixes U{1024..16384} with cached per-layer context K/V, one block of 16 per request, 5 layers",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- GPU runner
class Runner:
    def __init__(self, d, w, device="cuda"):
        import torch
        from dflash_synth import make_inference_inputs, make_training_inputs
        self.d, self.w, self.torch = d, w, torch
        self.cfg = d.config_from_workload(w)
        bs, H = w.block_size, w.hidden
        if w.inference:
            self.inp = make_inference_inputs(w, device)
            self.T = self.inp["total"]
            self.base, self.anchor = self.inp["block_ctx_base"], self.inp["block_anchor"]
            self.valid = self.inp["block_valid"]
            self.ctx_k, self.ctx_v = self.inp["ctx_k"], self.inp["ctx_v"]
            ctx_rows = 0
        else:
            self.inp = make_training_inputs(w, device)
            B, S, N = w.batch, w.seq_len, w.anchors_per_row
            self.T = B * S
            self.anchors = torch.empty((B, N), dtype=torch.int32, device=device)
            self.positions = torch.empty((B, N, bs), dtype=torch.int32, device=device)
            self.valid3 = torch.empty((B, N, bs), dtype=torch.uint8, device=device)
            self.loss_mask = torch.empty((B, N, bs), dtype=torch.uint8, device=device)
            self.num = torch.empty((B,), dtype=torch.int32, device=device)
            self.base = torch.empty((B * N,), dtype=torch.int64, device=device)
            self.anchor = self.anchors.view(-1)
            self.valid = self.valid3.view(-1)
            self.ctx_pos = torch.arange(S, dtype=torch.int32, device=device).repeat(B)
            self.ctx_k = [torch.empty((w.num_kv_heads, self.T, w.head_dim), dtype=w.torch_dtype, device=device)
                          for _ in range(w.num_layers)]
            self.ctx_v = [torch.empty((w.num_kv_heads, w.head_dim, self.T), dtype=w.torch_dtype, device=device)
                          for _ in range(w.num_layers)]
            ctx_rows = self.T
        self.out = torch.empty((w.num_blocks * bs, H), dtype=w.torch_dtype, device=device)
        self.ws = torch.empty(d.dflash_workspace_size(self.cfg, w.num_blocks, ctx_rows), dtype=torch.uint8,
                              device=device)

    def step(self):
        d, w, i = self.d, self.w, self.inp
        if not w.inference:
            d.dflash_build_plan(i["mask"], i["sample_ids"], i["step"], i["plan_seed"], w.anchors_per_row,
                                w.block_size, self.anchors, self.positions, self.valid3, self.loss_mask,
                                self.num, self.base)
            d.dflash_ctx_proj(self.cfg, i["states"], w.target_hidden, self.T * w.target_hidden, self.T,
                              self.ctx_pos, i["w_proj"], i["layers"], self.ctx_k, self.ctx_v, self.T, 0,
                              self.ws)
        d.dflash_body_forward(self.cfg, w.num_blocks, i["emb"], i["layers"], self.ctx_k, self.ctx_v, self.T,
                              self.base, self.anchor, self.valid, self.out, self.ws)

    def anchors_np(self):
        return self.anchor.cpu().numpy().astype("int64")

    def bases_np(self):
        return self.base.cpu().numpy().astype("int64")


# ----------------------------------------------------------------------------- algorithmic counts
def kernel_counts(w, anchors, bases):
    """Algorithmic flops and HBM bytes per launch, and launches per step, for each
    kernel. GEMMs: 2*M*N*K flops, each operand read once and the output written
    once. Attention: 4*D flops per (query head, block row, visible key); bytes:
    every context K and V row that some block can see, once per KV head (blocks
    of one sequence share their prefix), each block's own K and V, plus q in and
    out. Its bound is whichever of the two takes longer at peak: the MFMA where
    many blocks share a sequence's prefix, HBM where each request has its own."""
    import numpy as np
    eb = 4 if w.dtype == "f32" else 2
    bs, H, D, I = w.block_size, w.hidden, w.head_dim, w.intermediate
    Hq, Hkv, L = w.num_q_heads, w.num_kv_heads, w.num_layers
    nb = w.num_blocks
    R = nb * bs
    a = np.asarray(anchors, np.int64)
    live = a >= 0
    keys = (a[live] + bs).astype(np.float64)
    c = {}

    def gemm(name, M, N, K, extra_bytes=0.0, launches=1):
        c[name] = dict(flops=2.0 * M * N * K, bytes=float(eb * (M * K + N * K + M * N) + extra_bytes),
                       launches=launches, bound="mfma")

    if not w.inference:
        T = w.batch * w.seq_len
        Kt = w.num_target_layers * w.target_hidden
        gemm("ctx_proj", T, H, Kt)
        gemm("ctx_kv", T, L * 2 * Hkv * D, H)
    gemm("qkv", R, (Hq + 2 * Hkv) * D, H, launches=L)
    gemm("o_proj", R, H, Hq * D, extra_bytes=R * H * (8 - eb), launches=L)
    gemm("gate_up", R, 2 * I, H, extra_bytes=-R * I * eb, launches=L)
    gemm("down", R, H, I, extra_bytes=R * H * (8 - eb), launches=L)
    b = np.asarray(bases, np.int64)[live]
    ctx_rows = sum(int(a[live][b == u].max()) for u in np.unique(b))
    att_flops = float(4.0 * D * Hq * bs * keys.sum())
    att_bytes = float(Hkv * (ctx_rows + bs * int(live.sum())) * 2 * D * eb + 2 * R * Hq * D * eb)
    c["attention"] = dict(flops=att_flops, bytes=att_bytes, launches=L,
                          bound="mfma" if att_flops / (PEAK_MFMA_TFLOPS[w.dtype] * 1e12)
                          >= att_bytes / (PEAK_HBM_GBS * 1e9) else "hbm")
    c["rmsnorm"] = dict(flops=float(3.0 * R * H), bytes=float(R * H * (4 + eb)), launches=2 * L, bound="hbm")
    # Merge of split prefixes: at most every query row of every head in and out
    # once in fp32 (an upper bound; no splits -> no work).
    c["attn_combine"] = dict(flops=0.0, bytes=float(2 * R * Hq * D * 4), launches=L, bound="hbm")
    if not w.inference:
        c["plan"] = dict(flops=0.0, bytes=float(w.batch * w.seq_len + 10 * nb * bs), launches=1, bound="hbm")
    return c


def roofline_entry(name, cnt, avg_ms, dtype):
    t = avg_ms / 1e3
    if cnt["bound"] == "mfma":
        ach = cnt["flops"] / t / 1e12
        peak = PEAK_MFMA_TFLOPS[dtype]
        return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4)}
    ach = cnt["bytes"] / t / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


def step_roofline_ms(counts, dtype):
    tot = 0.0
    for cnt in counts.values():
        f = cnt["flops"] / (PEAK_MFMA_TFLOPS[dtype] * 1e12)
        b = cnt["bytes"] / (PEAK_HBM_GBS * 1e9)
        tot += max(f, b) * cnt["launches"]
    return tot * 1e3


# ----------------------------------------------------------------------------- steps next to the path
def hook_ms(d, torch, kernels, fn, reps=10):
    """Device time per call of fn, summed over the given library kernels, from
    the library's own HIP events on the launch stream (host overhead excluded)."""
    fn()
    torch.cuda.synchronize()
    total = 0.0
    for name, per_call in kernels:
        d.dflash_profile_start(name, per_call * reps)
        for _ in range(reps):
            fn()
        times = d.dflash_profile_stop(per_call * reps)
        total += sum(times) / reps
    return total


def next_rows(d, torch, device="cuda"):
    """Time the steps around the body at the inference shape (64 requests,
    gamma + 1 = 16 verified positions each, the 5-layer dimensions):
    ctx_append = one cycle's projection of 1024 newly verified target states into
    every layer's context cache (scattered rows), with its MFMA roofline;
    verify_greedy / verify_sample = verification of the 64 drafted blocks over a
    151936-token vocabulary, with their HBM rooflines; and, on the training
    side, lm_head_ce = LM head + decayed cross-entropy over the 5-layer body's
    4096 block rows (151936 x 4096 head), attn_backward = one layer's
    dual-source attention backward at the training shape,
    ctx_proj_backward = dW_proj and the context path's share of every layer's
    Wk / Wv gradient through every layer's context K/V over the 32768 context
    rows, lm_head_ce_backward = the loss gradient with respect to
    the 4096 block rows, body_backward = the body's training forward and
    backward, each with its MFMA roofline; and train_step = one whole training
    step of the 5-layer workload, end to end."""
    import math as _m
    from dflash_synth import WORKLOADS, Rng, layer_weights
    w = WORKLOADS["c5"]
    cfg = d.config_from_workload(w)
    out = {}
    R, g1, cap = w.batch, w.block_size, 2048
    rows = R * g1
    K = w.num_target_layers * w.target_hidden
    rng = Rng(2024, device)
    X = rng.normal("append.states", (rows, K))
    w_proj = rng.normal("append.w_proj", (w.hidden, K), std=1 / _m.sqrt(K))
    layers = [layer_weights(w, rng, l) for l in range(w.num_layers)]
    total = R * cap
    ck = [torch.empty((w.num_kv_heads, total, w.head_dim), dtype=torch.bfloat16, device=device)
          for _ in range(w.num_layers)]
    cv = [torch.empty((w.num_kv_heads, w.head_dim, total), dtype=torch.bfloat16, device=device)
          for _ in range(w.num_layers)]
    lens = rng.integers("append.len", 0, cap - g1, (R,))
    j = torch.arange(g1, device=device)
    pos = (lens[:, None] + j[None, :]).reshape(-1).to(torch.int32)
    dst = (torch.arange(R, device=device)[:, None] * cap + lens[:, None] + j[None, :]).reshape(-1)
    ws = torch.empty(d.dflash_workspace_size(cfg, 0, rows), dtype=torch.uint8, device=device)
    ms = hook_ms(d, torch, [("ctx_proj", 1), ("ctx_kv", 1)],
                 lambda: d.dflash_ctx_append(cfg, X, K, w.target_hidden, rows, pos, dst, w_proj, layers, ck, cv,
                                             total, ws))
    flops = 2.0 * rows * w.hidden * K + 2.0 * rows * (w.num_layers * 2 * w.num_kv_heads * w.head_dim) * w.hidden
    ach = flops / (ms / 1e3) / 1e12
    out["ctx_append"] = {"rows": rows, "ms": round(ms, 4), "rows_per_s": round(rows / (ms / 1e3), 1),
                         "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_MFMA_TFLOPS["bf16"],
                                      "unit": "TFLOP/s", "frac": round(ach / PEAK_MFMA_TFLOPS["bf16"], 4)}}
    del ck, cv

    # Verification of one cycle's blocks (64 requests, gamma 15, vocabulary 151936).
    B, g, V = R, g1 - 1, 151936
    gen = torch.Generator(device=device).manual_seed(7)
    draft = torch.randint(0, V, (B, g), generator=gen, device=device, dtype=torch.int32)
    em = torch.empty((B, g + 1), dtype=torch.int32, device=device)
    num = torch.empty((B,), dtype=torch.int32, device=device)
    acc = torch.empty((B,), dtype=torch.int32, device=device)
    logits = torch.randn((B, g + 1, V), generator=gen, device=device).to(torch.bfloat16)
    ms = hook_ms(d, torch, [("verify", 1)], lambda: d.dflash_verify_greedy(draft, logits, em, num, acc))
    byt = logits.numel() * 2.0
    out["verify_greedy"] = {"blocks": B, "gamma": g, "vocab": V, "ms": round(ms, 4),
                            "roofline": {"bound": "hbm", "achieved": round(byt / (ms / 1e3) / 1e9, 1),
                                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                         "frac": round(byt / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}}
    del logits
    p = torch.softmax(torch.randn((B, g + 1, V), generator=gen, device=device) * 3.0, dim=-1)
    q = torch.softmax(torch.randn((B, g, V), generator=gen, device=device) * 3.0, dim=-1)
    ua = torch.rand((B, g), generator=gen, device=device)
    ud = torch.rand((B,), generator=gen, device=device)
    ms = hook_ms(d, torch, [("verify", 1)], lambda: d.dflash_verify_sample(draft, p, q, ua, ud, em, num, acc))
    # Algorithmic bytes: the accept lookups, then one p row and one q row per
    # request (the draw position), read twice (sum, then the crossing walk).
    byt = B * g * 8.0 + B * 2 * 2 * V * 4.0
    out["verify_sample"] = {"blocks": B, "gamma": g, "vocab": V, "ms": round(ms, 4),
                            "roofline": {"bound": "hbm", "achieved": round(byt / (ms / 1e3) / 1e9, 1),
                                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                         "frac": round(byt / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}}
    del p, q
    # Training side: LM head + decayed CE over the 5-layer body's 4096 block rows.
    wt = WORKLOADS["c3"]
    cfg3 = d.config_from_workload(wt)
    rows = wt.num_blocks * wt.block_size
    hid = torch.randn((rows, wt.hidden), generator=gen, device=device).to(torch.bfloat16)
    W = (torch.randn((V, wt.hidden), generator=gen, device=device) / _m.sqrt(wt.hidden)).to(torch.bfloat16)
    tg = torch.randint(0, V, (rows,), generator=gen, device=device, dtype=torch.int32)
    lm = (torch.arange(rows, device=device) % wt.block_size != 0).to(torch.uint8)
    ce = torch.empty((rows,), dtype=torch.float32, device=device)
    loss = torch.empty((1,), dtype=torch.float64, device=device)
    ws2 = torch.empty(d.dflash_lm_head_ce_workspace_size(rows, V), dtype=torch.uint8, device=device)
    call = lambda: d.dflash_lm_head_ce(cfg3, hid, W, tg, lm, 7.0, ce, loss, ws2)
    ms_gemm = hook_ms(d, torch, [("lm_head", 1)], call)
    ms = ms_gemm + hook_ms(d, torch, [("lm_ce", 1)], call)
    flops = 2.0 * rows * V * wt.hidden
    out["lm_head_ce"] = {"rows": rows, "vocab": V, "hidden": wt.hidden, "ms": round(ms, 4),
                         "lm_head_gemm_ms": round(ms_gemm, 4),
                         "roofline": {"bound": "mfma", "achieved": round(flops / (ms / 1e3) / 1e12, 2),
                                      "peak": PEAK_MFMA_TFLOPS["bf16"], "unit": "TFLOP/s",
                                      "frac": round(flops / (ms / 1e3) / 1e12 / PEAK_MFMA_TFLOPS["bf16"], 4)}}
    # Its backward (the gradient of the loss with respect to the hidden rows):
    # two products of 2 * rows * V * H flops each (logits again, then dz W_lm).
    dh = torch.empty_like(hid)
    ws5 = torch.empty(d.dflash_lm_head_ce_backward_workspace_size(cfg3, rows, V), dtype=torch.uint8, device=device)
    call = lambda: d.dflash_lm_head_ce_backward(cfg3, hid, W, tg, lm, 7.0, ce, 1.0, dh, ws5)
    parts = {k: hook_ms(d, torch, [(k, 1)], call) for k in ("lm_bwd_prep", "lm_bwd_dz", "lm_bwd_dh")}
    ms = sum(parts.values())
    ach = 2 * flops / (ms / 1e3) / 1e12
    out["lm_head_ce_backward"] = {"rows": rows, "vocab": V, "hidden": wt.hidden, "ms": round(ms, 4),
                                  **{k + "_ms": round(v, 4) for k, v in parts.items()},
                                  "roofline": {"bound": "mfma", "achieved": round(ach, 2),
                                               "peak": PEAK_MFMA_TFLOPS["bf16"], "unit": "TFLOP/s",
                                               "frac": round(ach / PEAK_MFMA_TFLOPS["bf16"], 4)}}
    # The training pair that keeps the fp32 logits: the forward's GEMM also
    # stores them, and the backward takes dz from them in one elementwise pass
    # (rows x V fp32 read, rows x V bf16 written), then the one product dz W_lm.
    logits = torch.empty(d.dflash_lm_head_ce_logits_size(rows, V), dtype=torch.uint8, device=device)
    call = lambda: d.dflash_lm_head_ce_train(cfg3, hid, W, tg, lm, 7.0, ce, loss, logits, ws2)
    ms_gemm = hook_ms(d, torch, [("lm_head", 1)], call)
    ms = ms_gemm + hook_ms(d, torch, [("lm_ce", 1)], call)
    out["lm_head_ce_train"] = {"ms": round(ms, 4), "lm_head_gemm_ms": round(ms_gemm, 4),
                               "logits_bytes": logits.numel()}
    # The head is frozen: its transpose is formed once (dflash_lm_head_transpose) and kept.
    W_t = torch.empty(d.dflash_lm_head_transpose_size(cfg3, V), dtype=torch.uint8, device=device)
    d.dflash_lm_head_transpose(cfg3, W, W_t)
    call = lambda: d.dflash_lm_head_ce_backward_saved(cfg3, rows, logits, W, tg, lm, 7.0, ce, 1.0, dh, ws5,
                                                      lm_head_t=W_t)
    parts = {k: hook_ms(d, torch, [(k, 1)], call) for k in ("lm_bwd_prep", "lm_bwd_dz", "lm_bwd_dh")}
    ms = sum(parts.values())
    dz_bytes = rows * ((V + 63) // 64 * 64) * (4 + 2)
    out["lm_head_ce_backward_saved"] = {
        "ms": round(ms, 4), **{k + "_ms": round(v, 4) for k, v in parts.items()},
        "dz_pass": {"bound": "hbm", "achieved": round(dz_bytes / (parts["lm_bwd_dz"] / 1e3) / 1e9, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(dz_bytes / (parts["lm_bwd_dz"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(flops / (ms / 1e3) / 1e12, 2),
                     "peak": PEAK_MFMA_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(flops / (ms / 1e3) / 1e12 / PEAK_MFMA_TFLOPS["bf16"], 4)}}
    del hid, W, dh, ws5, logits, W_t
    # Training side: backward of one layer's dual-source attention at the
    # training shape (8 sequences of 4096, 32 blocks each at random anchors).
    T = wt.batch * wt.seq_len
    nb, bs, Hq, Hkv, D = wt.num_blocks, wt.block_size, wt.num_q_heads, wt.num_kv_heads, wt.head_dim
    anc = torch.cat([torch.randperm(wt.seq_len - bs - 1, generator=gen, device=device)[:wt.anchors_per_row] + 1
                     for _ in range(wt.batch)]).to(torch.int32)
    base = (torch.arange(nb, device=device) // wt.anchors_per_row * wt.seq_len).to(torch.int64)
    val = torch.ones((nb * bs,), dtype=torch.uint8, device=device)
    mk = lambda *shape: torch.randn(shape, generator=gen, device=device).to(torch.bfloat16)
    qa, ka, va, oa, doa = mk(nb * bs, Hq * D), mk(nb * bs, Hkv * D), mk(nb * bs, Hkv * D), mk(nb * bs, Hq * D), \
        mk(nb * bs, Hq * D)
    cka, cva = mk(Hkv, T, D), mk(Hkv, D, T)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=device)
    grads = (f32(nb * bs, Hq * D), f32(nb * bs, Hkv * D), f32(nb * bs, Hkv * D), f32(Hkv, T, D), f32(Hkv, D, T))
    ws3 = torch.empty(d.dflash_block_attn_backward_workspace_size(cfg3, nb), dtype=torch.uint8, device=device)
    ms = hook_ms(d, torch, [("attn_bwd", 1)],
                 lambda: d.dflash_block_attn_backward(cfg3, nb, qa, ka, va, cka, cva, T, base, anc, val, oa, doa,
                                                      *grads, ws3))
    # Algorithmic flops: five products of bs x keys x D per query head (scores,
    # dO V^T, dq, dk, dv), keys = anchor + bs.
    keys = float((anc.to(torch.float64) + bs).sum().item())
    flops = 10.0 * bs * D * Hq * keys
    ach = flops / (ms / 1e3) / 1e12
    out["attn_backward"] = {"blocks": nb, "ctx_total": T, "ms": round(ms, 4),
                            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_MFMA_TFLOPS["bf16"],
                                         "unit": "TFLOP/s", "frac": round(ach / PEAK_MFMA_TFLOPS["bf16"], 4)}}
    del qa, ka, va, oa, doa, cka, cva, grads, ws3
    # Training side: gradient of W_proj through the context path (every layer's
    # context K/V gradient -> dC -> dW_proj) over the 32768 context rows, and
    # the path's share of every layer's Wk / Wv gradient (G^T C).
    Kin = wt.num_target_layers * wt.target_hidden
    X3 = mk(T, Kin)
    C3 = mk(T, wt.hidden)
    dkv3 = [f32(Hkv * D, wt.hidden).zero_() for _ in range(2 * wt.num_layers)]
    pos3 = (torch.arange(T, device=device) % wt.seq_len).to(torch.int32)
    layers3 = [layer_weights(wt, Rng(2025, device), l) for l in range(wt.num_layers)]
    gk3 = [torch.randn((Hkv, T, D), generator=gen, device=device) for _ in range(wt.num_layers)]
    gv3 = [torch.randn((Hkv, D, T), generator=gen, device=device) for _ in range(wt.num_layers)]
    dW3 = torch.empty((wt.hidden, Kin), dtype=torch.float32, device=device)
    ws4 = torch.empty(d.dflash_ctx_proj_backward_workspace_size(cfg3, T), dtype=torch.uint8, device=device)
    call = lambda: d.dflash_ctx_proj_backward(cfg3, X3, Kin, wt.target_hidden, T, pos3, layers3, gk3, gv3, T, 0,
                                              dW3, None, ws4, ctx_hidden=C3, d_wk=dkv3[:wt.num_layers],
                                              d_wv=dkv3[wt.num_layers:])
    parts = {k: hook_ms(d, torch, [(k, n)], call)
             for k, n in (("ctx_bwd_pack", 2), ("ctx_bwd_dc", 1), ("ctx_bwd_dw", 1), ("ctx_bwd_dkv", 1))}
    ms = sum(parts.values())
    kg = 2 * wt.num_layers * Hkv * D
    flops = 2.0 * T * wt.hidden * kg + 2.0 * wt.hidden * Kin * T + 2.0 * kg * wt.hidden * T
    ach = flops / (ms / 1e3) / 1e12
    out["ctx_proj_backward"] = {"rows": T, "ms": round(ms, 4), **{k + "_ms": round(v, 4) for k, v in parts.items()},
                                "roofline": {"bound": "mfma", "achieved": round(ach, 2),
                                             "peak": PEAK_MFMA_TFLOPS["bf16"], "unit": "TFLOP/s",
                                             "frac": round(ach / PEAK_MFMA_TFLOPS["bf16"], 4)}}
    del X3, dW3, ws4, C3, dkv3
    out["body_backward"] = body_backward_row(d, torch, wt, cfg3, layers3, anc, base, val, gk3, gv3, mk, f32)
    del gk3, gv3, layers3
    torch.cuda.empty_cache()
    out["train_step"] = train_step_row(d, torch, wt, V, device)
    return out


class TrainingBuffers:
    """Inputs, outputs and workspaces of one training step of a training-shaped
    workload, and the step itself as the library's calls in order. The targets
    (the caller's ground-truth tokens at each block position) are gathered with
    torch from a synthetic token sequence, as a caller would."""

    def __init__(self, d, torch, w, vocab, device):
        import math as _m
        from dflash_synth import Rng, make_training_inputs
        self.d, self.torch, self.w, self.vocab = d, torch, w, vocab
        B, S, N, bs, L = w.batch, w.seq_len, w.anchors_per_row, w.block_size, w.num_layers
        self.inp = inp = make_training_inputs(w, device)
        self.cfg = cfg = d.config_from_workload(w)
        rng = Rng(4321, device)
        self.tokens = rng.integers("train.tokens", 0, vocab - 1, (B, S)).to(torch.int32)
        self.lm_head = rng.normal("train.lm_head", (vocab, w.hidden), std=1 / _m.sqrt(w.hidden),
                                  dtype=w.torch_dtype)
        nb, R, T, H = w.num_blocks, w.num_blocks * bs, B * S, w.hidden
        e = lambda *shape, dt=torch.float32: torch.empty(shape, dtype=dt, device=device)
        u8 = lambda n: torch.empty(n, dtype=torch.uint8, device=device)
        self.anchors, self.positions = e(B, N, dt=torch.int32), e(B, N, bs, dt=torch.int32)
        self.valid, self.loss_mask = e(B, N, bs, dt=torch.uint8), e(B, N, bs, dt=torch.uint8)
        self.num, self.base = e(B, dt=torch.int32), e(nb, dt=torch.int64)
        self.ctx_pos = (torch.arange(T, device=device) % S).to(torch.int32)
        self.ck = [e(w.num_kv_heads, T, w.head_dim, dt=w.torch_dtype) for _ in range(L)]
        self.cv = [e(w.num_kv_heads, w.head_dim, T, dt=w.torch_dtype) for _ in range(L)]
        self.out, self.d_out = e(R, H, dt=w.torch_dtype), e(R, H, dt=w.torch_dtype)
        self.C = e(T, H, dt=w.torch_dtype)          # C = X W_proj^T, kept for the Wk / Wv gradients
        self.ws = u8(d.dflash_workspace_size(cfg, nb, T))
        self.reserve = u8(d.dflash_body_train_reserve_size(cfg, nb))
        self.ce, self.loss = e(R), e(1, dt=torch.float64)
        self.ws_lm = u8(d.dflash_lm_head_ce_workspace_size(R, vocab))
        self.ws_lmb = u8(d.dflash_lm_head_ce_backward_workspace_size(cfg, R, vocab))
        self.logits = u8(d.dflash_lm_head_ce_logits_size(R, vocab))
        # The LM head is frozen: its transpose for the loss backward is formed once.
        self.lm_head_t = u8(d.dflash_lm_head_transpose_size(cfg, vocab))
        d.dflash_lm_head_transpose(cfg, self.lm_head, self.lm_head_t)
        self.grads = [{k: e(*v.shape) for k, v in Lw.items()} for Lw in inp["layers"]]
        self.dck = [e(w.num_kv_heads, T, w.head_dim) for _ in range(L)]
        self.dcv = [e(w.num_kv_heads, w.head_dim, T) for _ in range(L)]
        self.demb = e(R, H)
        self.ws_bb = u8(d.dflash_body_backward_workspace_size(cfg, nb))
        self.Kt = w.num_target_layers * w.target_hidden
        self.dW = e(H, self.Kt)
        self.ws_cb = u8(d.dflash_ctx_proj_backward_workspace_size(cfg, T))
        self.row_of = torch.arange(R, device=device) // (bs * N)
        # Optimizer state of every trainable tensor (each layer's weights and
        # W_proj): fp32 master copies and moments; the working copies are the
        # config-dtype weights the forward reads.
        pairs = [(Lw[k], G[k]) for Lw, G in zip(inp["layers"], self.grads) for k in Lw]
        pairs.append((inp["w_proj"], self.dW))
        self.opt = [{"master": wt.float().reshape(-1).clone(), "exp_avg": e(wt.numel()),
                     "exp_avg_sq": e(wt.numel()), "grad": gr.reshape(-1), "weight": wt.reshape(-1)}
                    for wt, gr in pairs]
        for t in self.opt:
            t["exp_avg"].zero_()
            t["exp_avg_sq"].zero_()
        self.params = sum(t["master"].numel() for t in self.opt)
        self.opt_step = 0

    def step(self):
        """Runs the step; returns events recorded before and after each stage."""
        d, torch, w, i = self.d, self.torch, self.w, self.inp
        cfg, T, nb, V = self.cfg, self.w.batch * self.w.seq_len, self.w.num_blocks, self.vocab
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(9)]
        ev[0].record()
        d.dflash_build_plan(i["mask"], i["sample_ids"], i["step"], i["plan_seed"], w.anchors_per_row, w.block_size,
                            self.anchors, self.positions, self.valid, self.loss_mask, self.num, self.base)
        ev[1].record()
        d.dflash_ctx_proj_train(cfg, i["states"], w.target_hidden, T * w.target_hidden, T, self.ctx_pos,
                                i["w_proj"], i["layers"], self.ck, self.cv, T, 0, self.C, self.ws)
        ev[2].record()
        anc, val = self.anchors.reshape(-1), self.valid.reshape(-1)
        d.dflash_body_forward_train(cfg, nb, i["emb"], i["layers"], self.ck, self.cv, T, self.base, anc, val, self.out,
                                    self.reserve, self.ws)
        ev[3].record()
        pos = self.positions.reshape(-1).long().clamp(0, w.seq_len - 1)
        targets = self.tokens[self.row_of, pos].contiguous()
        lm = self.loss_mask.reshape(-1)
        d.dflash_lm_head_ce_train(cfg, self.out, self.lm_head, targets, lm, 7.0, self.ce, self.loss, self.logits,
                                  self.ws_lm)
        ev[4].record()
        d.dflash_lm_head_ce_backward_saved(cfg, self.out.shape[0], self.logits, self.lm_head, targets, lm, 7.0,
                                           self.ce, 1.0, self.d_out, self.ws_lmb, lm_head_t=self.lm_head_t)
        ev[5].record()
        d.dflash_body_backward(cfg, nb, self.reserve, i["layers"], self.ck, self.cv, T, self.base, anc, val,
                               self.d_out, self.demb, self.grads, self.dck, self.dcv, self.ws_bb)
        ev[6].record()
        d.dflash_ctx_proj_backward(cfg, i["states"], w.target_hidden, T * w.target_hidden, T, self.ctx_pos,
                                   i["layers"], self.dck, self.dcv, T, 0, self.dW, None, self.ws_cb,
                                   ctx_hidden=self.C, d_wk=[g["wk"] for g in self.grads],
                                   d_wv=[g["wv"] for g in self.grads])
        ev[7].record()
        self.opt_step += 1
        d.dflash_adamw_step(cfg.dtype, self.opt, lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01,
                            step=self.opt_step)
        ev[8].record()
        return ev


def train_step_row(d, torch, w, vocab, device, reps=3):
    """One whole training step of the 5-layer training workload through the
    library, timed end to end with events on the launch stream: plan, context
    projection (keeping C), training forward (reserve space), LM head + decayed
    CE keeping its logits, its backward from them (the frozen head transposed
    once, outside the step), body backward, the context path's backward (W_proj,
    and its share of every Wk / Wv gradient), and the AdamW step over every
    layer weight and W_proj (fp32 master copies and moments; it writes the bf16
    weights the next step's forward reads). Synthetic inputs of the workload's
    shapes; targets are random tokens at the block positions; frozen synthetic
    LM head of the given vocabulary. Also the events between the stages."""
    bufs = TrainingBuffers(d, torch, w, vocab, device)
    marks = bufs.step()                       # warm-up
    torch.cuda.synchronize()
    names = ["plan", "ctx_proj", "forward_train", "lm_head_ce", "lm_head_ce_backward", "body_backward",
             "ctx_proj_backward", "optimizer"]
    acc = [0.0] * len(names)
    total = 0.0
    for _ in range(reps):
        marks = bufs.step()
        torch.cuda.synchronize()
        ts = [marks[i].elapsed_time(marks[i + 1]) for i in range(len(names))]
        acc = [a + t for a, t in zip(acc, ts)]
        total += marks[0].elapsed_time(marks[-1])
    ms = total / reps
    opt_ms = acc[-1] / reps
    opt_bytes = bufs.params * (4 + 3 * 4 + 3 * 4 + (2 if w.dtype == "bf16" else 4))
    return {"blocks": w.num_blocks, "layers": w.num_layers, "vocab": vocab, "ms": round(ms, 3),
            "stages_ms": {n: round(a / reps, 3) for n, a in zip(names, acc)},
            "block_positions_per_s": round(w.num_blocks * w.block_size / (ms / 1e3), 1),
            "optimizer": {"params": bufs.params, "bytes": opt_bytes,
                          "roofline": {"bound": "hbm", "achieved": round(opt_bytes / (opt_ms / 1e3) / 1e9, 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": round(opt_bytes / (opt_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}}}


def body_backward_row(d, torch, wt, cfg, layers, anc, base, val, d_ctx_k, d_ctx_v, mk, f32, reps=5):
    """The body's training step at the 5-layer training shape (256 blocks at
    random anchors over 8 sequences of 4096 positions): dflash_body_forward_train
    (keeping every layer's activations in the reserve space), then
    dflash_body_backward (every gradient). Wall times from events around the calls on the launch stream;
    per-class device times from the library's hook. Rooflines: the weight-
    gradient GEMMs (contraction over the 4096 rows) and the activation-gradient
    GEMMs, each 2 * R * (H I + 2 I H + H nq + nqkv H) flops per layer."""
    T = wt.batch * wt.seq_len
    nb, bs, L = wt.num_blocks, wt.block_size, wt.num_layers
    R, H, I = nb * bs, wt.hidden, wt.intermediate
    nq, nk = wt.num_q_heads * wt.head_dim, wt.num_kv_heads * wt.head_dim
    cks = [mk(wt.num_kv_heads, T, wt.head_dim) for _ in range(L)]
    cvs = [mk(wt.num_kv_heads, wt.head_dim, T) for _ in range(L)]
    emb, dout = mk(R, H), mk(R, H)
    outb = torch.empty_like(emb)
    demb = f32(R, H)
    reserve = torch.empty(d.dflash_body_train_reserve_size(cfg, nb), dtype=torch.uint8, device=emb.device)
    grads = [{k: f32(*v.shape) for k, v in Lw.items()} for Lw in layers]
    ws = torch.empty(d.dflash_workspace_size(cfg, nb, 0), dtype=torch.uint8, device=emb.device)
    wsb = torch.empty(d.dflash_body_backward_workspace_size(cfg, nb), dtype=torch.uint8, device=emb.device)
    fwd = lambda: d.dflash_body_forward_train(cfg, nb, emb, layers, cks, cvs, T, base, anc, val, outb, reserve,
                                              ws)
    bwd = lambda: d.dflash_body_backward(cfg, nb, reserve, layers, cks, cvs, T, base, anc, val, dout, demb, grads,
                                         d_ctx_k, d_ctx_v, wsb)

    def wall(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    ms_f, ms_b = wall(fwd), wall(bwd)
    # Hook scopes per backward call: 4 pack scopes per layer + the output mask,
    # 4 GEMMs of each gradient kind per layer, 2 norms per layer, the attention backward.
    per_call = {"bwd_pack": 4 * L + 1, "bwd_data": 4 * L, "bwd_weight": 4 * L, "bwd_norm": 2 * L, "attn_bwd": L}
    parts = {k: hook_ms(d, torch, [(k, n)], bwd, reps=3) for k, n in per_call.items()}
    gemm_flops = L * 2.0 * R * (H * I + 2 * I * H + H * nq + (nq + 2 * nk) * H)
    peak = PEAK_MFMA_TFLOPS["bf16"]

    def roof(ms):
        ach = gemm_flops / (ms / 1e3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4)}
    return {"blocks": nb, "layers": L, "rows": R, "ctx_total": T, "ms": round(ms_b, 4),
            "forward_train_ms": round(ms_f, 4), "parts_ms": {k: round(v, 4) for k, v in parts.items()},
            "roofline": roof(parts["bwd_weight"]), "roofline_data_grads": roof(parts["bwd_data"])}


# ----------------------------------------------------------------------------- CPU oracle sample
def cpu_baseline(w, runner, anchors, budget_rows=None, budget_blocks=None):
    """The fp64 oracle on a bounded sample of the workload, scaled to block positions/s.

    Training-shaped: the context projection of `rows` target rows and the body of
    `blocks` blocks (evenly spaced over the plan's anchors, each with its full
    prefix of context K/V), extrapolated to the step's rows and blocks.
    Inference-shaped: the body of `blocks` requests over their cached context."""
    import numpy as np
    import torch
    import oracle

    def np64(t):
        return t.detach().to("cpu", torch.float64).numpy()

    inp = runner.inp
    cfg = dict(block_size=w.block_size, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
               head_dim=w.head_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps)
    layers = [{k: np64(v) for k, v in L.items()} for L in inp["layers"]]
    bs = w.block_size
    t_ctx = 0.0
    sample = {}
    if w.inference:
        nblk = budget_blocks or 4
        lens = inp["lengths"].cpu().numpy()
        offs = inp["offsets"].cpu().numpy()
        pick = np.linspace(0, w.batch - 1, nblk).round().astype(int)
        data = []
        for r in pick:
            lo, hi = int(offs[r]), int(offs[r + 1])
            data.append((np64(inp["emb"][r * bs:(r + 1) * bs]), [np64(k[:, lo:hi]) for k in inp["ctx_k"]],
                         [np64(v[:, :, lo:hi]).transpose(0, 2, 1) for v in inp["ctx_v"]], int(lens[r])))
        t0 = time.perf_counter()
        for e, ck, cv, a in data:
            oracle.body_forward(e, layers, ck, cv, [0], [a], np.ones(bs, np.uint8), cfg)
        t_body = time.perf_counter() - t0
        t_est = t_body * w.num_blocks / nblk
        sample["what"] = f"body of {nblk} of {w.num_blocks} requests (prefixes {sorted(int(lens[r]) for r in pick)})"
    else:
        rows = budget_rows or 1024
        nblk = budget_blocks or 4
        w_proj = np64(inp["w_proj"])
        states = np64(inp["states"][:, :rows])
        t0 = time.perf_counter()
        C = oracle.ctx_proj(oracle.concat_target_states(states), w_proj)
        oracle.ctx_kv(C, layers, np.arange(rows) % w.seq_len, w.num_kv_heads, w.head_dim, w.rope_theta)
        t_ctx = time.perf_counter() - t0
        order = np.argsort(anchors, kind="stable")
        pick = order[np.linspace(0, len(order) - 1, nblk).round().astype(int)]
        gen = np.random.default_rng(0)
        data = []
        for n in pick:
            a = int(anchors[n])
            ck = [gen.standard_normal((w.num_kv_heads, max(a, 1), w.head_dim)) for _ in range(w.num_layers)]
            cv = [gen.standard_normal((w.num_kv_heads, max(a, 1), w.head_dim)) for _ in range(w.num_layers)]
            data.append((np64(inp["emb"][n * bs:(n + 1) * bs]), ck, cv, a))
        t0 = time.perf_counter()
        for e, ck, cv, a in data:
            oracle.body_forward(e, layers, ck, cv, [0], [a], np.ones(bs, np.uint8), cfg)
        t_body = time.perf_counter() - t0
        T = w.batch * w.seq_len
        t_est = t_ctx * T / rows + t_body * w.num_blocks / nblk
        sample["what"] = (f"context projection of {rows} of {T} target rows + body of {nblk} of {w.num_blocks} "
                          f"blocks (anchors {sorted(int(anchors[n]) for n in pick)}), scaled to the whole step")
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max([p.get("num_threads", 1) for p in libs] or [1])
        if libs:
            blas = ", ".join(f"{p.get('internal_api', '?')} {p.get('version', '?')}" for p in libs)
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    value = w.num_blocks * bs / t_est
    return {"value": round(value, 3), "unit": "block-positions/s", "cores": int(cores), "kind": "oracle",
            "blas": blas, "numpy": np.__version__, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": sample["what"], "sample_seconds": round(t_ctx + t_body, 2)}


# ----------------------------------------------------------------------------- timing
def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def measure(d, torch, w, steps, warmup, breakdown=True):
    """Build one workload's inputs, warm up, then time `steps` steps: HIP events
    around the whole loop (the reported step time) and around each step
    (median, p10, p90), with the dominant kernel's launches timed by the
    library's own events over the same region. Returns the figures and the runner."""
    runner = Runner(d, w)
    torch.cuda.synchronize()
    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    anchors = runner.anchors_np()
    counts = kernel_counts(w, anchors, runner.bases_np())

    # Per-kernel time shares: each kernel in turn, over a couple of steps.
    per_kernel = {}
    if breakdown:
        for name in counts:
            launches = counts[name]["launches"]
            reps = 2
            d.dflash_profile_start(name, launches * reps)
            for _ in range(reps):
                runner.step()
            times = d.dflash_profile_stop(launches * reps)
            if times:
                per_kernel[name] = sum(times) / reps
        dominant = max(per_kernel, key=per_kernel.get)
    else:
        dominant = "ctx_proj" if not w.inference else "attention"

    n_dom = counts[dominant]["launches"] * steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    d.dflash_profile_start(dominant, n_dom)
    ev[0].record()
    for i in range(steps):
        runner.step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    dom_times = d.dflash_profile_stop(n_dom)
    dom_avg = sum(dom_times) / len(dom_times)

    positions = w.num_blocks * w.block_size
    roof = roofline_entry(dominant, counts[dominant], dom_avg, w.dtype)
    t_roof = step_roofline_ms(counts, w.dtype)
    flops = sum(c["flops"] * c["launches"] for c in counts.values())
    med = _pct(per_step, 50)
    res = {
        "ms_per_step": ms, "ms_median": med, "ms_p10": _pct(per_step, 10), "ms_p90": _pct(per_step, 90),
        "value": positions / (ms / 1e3), "positions": positions, "dominant": dominant, "dom_avg_ms": dom_avg,
        "dom_launches": len(dom_times), "roofline": roof, "roofline_ms": t_roof, "flops": flops,
        "counts": counts, "per_kernel": per_kernel, "anchors": anchors,
    }
    return res, runner


def long_context_views(w, res):
    """Three labelled figures for the long-context workload. (i) The per-block
    prefix-stream model: every block streams its own prefix of context K and V
    from HBM in every layer (the bytes a kernel without shared tiles would
    move), as a fraction of HBM peak over the step and over attention alone;
    (ii) the algorithmic MFMA fraction of the step; (iii) the attention kernel's
    measured DRAM traffic rate, from the committed rocprofv3 counter file when
    it matches the current sources."""
    import numpy as np
    a = np.asarray(res["anchors"], np.int64)
    eb = 2 if w.dtype == "bf16" else 4
    stream = float(a[a >= 0].sum()) * w.num_kv_heads * 2 * w.head_dim * eb * w.num_layers
    att_ms = res["per_kernel"].get("attention")
    views = {
        "per_block_stream_bytes": stream,
        "per_block_stream_hbm_frac_step": round(stream / (PEAK_HBM_GBS * 1e9) / (res["ms_per_step"] / 1e3), 4),
        "algorithmic_mfma_frac_step": round(res["flops"] / (PEAK_MFMA_TFLOPS[w.dtype] * 1e12)
                                            / (res["ms_per_step"] / 1e3), 4),
    }
    if att_ms:
        views["per_block_stream_hbm_frac_attention"] = round(
            stream / (PEAK_HBM_GBS * 1e9) / (att_ms / 1e3), 4)
    return views


def config_summary(w, res):
    out = {"workload": w.name, "ms_per_step": round(res["ms_per_step"], 4),
           "ms_median": round(res["ms_median"], 4), "ms_p10": round(res["ms_p10"], 4),
           "ms_p90": round(res["ms_p90"], 4), "block_positions_per_s": round(res["value"], 1),
           "step_roofline_frac": round(res["roofline_ms"] / res["ms_per_step"], 4),
           "step_mfma_frac": round(res["flops"] / (PEAK_MFMA_TFLOPS[w.dtype] * 1e12)
                                   / (res["ms_per_step"] / 1e3), 4),
           "dominant_kernel": res["dominant"], "dominant_frac": res["roofline"]["frac"],
           "dominant_bound": res["roofline"]["bound"],
           "kernel_ms_per_step": {k: round(v, 4) for k, v in res["per_kernel"].items()}}
    if w.name == "c4":
        out["long_context_views"] = long_context_views(w, res)
    return out


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(DESCR))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the steps next to the path")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' summaries")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_draft_model_build_amd as d
    from dflash_synth import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    w = WORKLOADS[args.workload]
    log(f"workload {w.name}: building inputs")
    res, runner = measure(d, torch, w, args.steps, args.warmup, breakdown=not args.no_breakdown)
    ms = res["ms_per_step"]
    log("kernel ms/step: " + ", ".join(f"{k} {v:.3f}" for k, v in res["per_kernel"].items()))
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (median {res['ms_median']:.3f}, p10 {res['ms_p10']:.3f}, "
        f"p90 {res['ms_p90']:.3f}); {res['dominant']} avg {res['dom_avg_ms']:.4f} ms over "
        f"{res['dom_launches']} launches")

    roof = dict(res["roofline"])
    from bench_traffic import load as load_traffic
    roof["traffic"] = load_traffic(w.name, res["dominant"])
    roof["launches_timed"] = res["dom_launches"]
    t_roof = res["roofline_ms"]
    result = {
        "metric": METRIC, "value": round(res["value"], 1), "unit": "block-positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {DESCR[w.name]}", "num_blocks": w.num_blocks,
                   "block_size": w.block_size, "layers": w.num_layers, "block_positions": res["positions"]},
        "roofline": roof,
        "ms_per_step_stats": {"median": round(res["ms_median"], 4), "p10": round(res["ms_p10"], 4),
                              "p90": round(res["ms_p90"], 4), "events": "one HIP event pair per step"},
        "step_roofline": {"roofline_ms": round(t_roof, 4), "frac": round(t_roof / ms, 4),
                          "flops": res["flops"],
                          "model": "sum over kernels of max(flops / MFMA peak, bytes / HBM peak)"},
        "kernel_ms_per_step": {k: round(v, 4) for k, v in res["per_kernel"].items()},
    }
    if w.name == "c4":
        result["long_context_views"] = long_context_views(w, res)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a CPU sample")
        budgets = {"c1": (128, 4), "c2": (8192, 32), "c3": (8192, 48), "c4": (4096, 12), "c5": (None, 24)}
        r, b = budgets[w.name]
        cpu = cpu_baseline(w, runner, res["anchors"], r, b)
    del runner
    torch.cuda.empty_cache()
    if not args.no_configs:
        # The other bf16 workloads (one-layer, long-context, ragged-cache), each
        # measured the same way, so the per-workload bars are on record.
        configs = {}
        for name in ("c2", "c3", "c4", "c5"):
            if name == w.name:
                configs[name] = config_summary(w, res)
                continue
            log(f"workload {name}: building inputs")
            r2, run2 = measure(d, torch, WORKLOADS[name], args.steps, args.warmup)
            configs[name] = config_summary(WORKLOADS[name], r2)
            log(f"workload {name}: {r2['ms_per_step']:.3f} ms/step (median {r2['ms_median']:.3f})")
            del run2
            torch.cuda.empty_cache()
        result["configs"] = configs
    if not args.no_next:
        log("timing the steps next to the path (inference shape)")
        result["next_rows"] = next_rows(d, torch)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
