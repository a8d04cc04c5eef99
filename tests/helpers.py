"""Shared plumbing for the parity tests: run the HIP path through the C ABI on
seeded inputs, and run the oracle on the same bytes (copied to the host)."""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
from dflash_synth import Workload

BF16_TOL = dict(rel_l2=1e-2, max_abs=5e-2)
F32_TOL = dict(rel_l2=1e-5, max_abs=1e-4)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def tol_for(w: Workload):
    return F32_TOL if w.dtype == "f32" else BF16_TOL


def compare(gpu: torch.Tensor, ref: np.ndarray, tol, what: str = ""):
    g = np64(gpu).reshape(ref.shape)
    err = g - ref
    denom = math.sqrt(float((ref * ref).sum())) or 1.0
    rel = math.sqrt(float((err * err).sum())) / denom
    mx = float(np.abs(err).max()) if err.size else 0.0
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3e} > {tol['rel_l2']}"
    assert mx <= tol["max_abs"], f"{what}: max-abs {mx:.3e} > {tol['max_abs']}"
    return rel, mx


def oracle_cfg(w: Workload) -> Dict[str, float]:
    return dict(block_size=w.block_size, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                head_dim=w.head_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps)


def layers64(layers: Sequence[Dict[str, torch.Tensor]]) -> List[Dict[str, np.ndarray]]:
    return [{k: np64(v) for k, v in L.items()} for L in layers]


def workspace(lib, cfg, num_blocks: int, ctx_rows: int, device) -> torch.Tensor:
    n = lib.dflash_workspace_size(cfg, num_blocks, ctx_rows)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=device)


class TrainingRun:
    """Plan + context projection + body on the GPU for a training-shaped workload."""

    def __init__(self, lib, w: Workload, inputs: Dict[str, object], device="cuda"):
        self.lib, self.w, self.inp, self.device = lib, w, inputs, device
        B, S, N, bs = w.batch, w.seq_len, w.anchors_per_row, w.block_size
        self.cfg = lib.config_from_workload(w)
        d = device
        self.anchors = torch.empty((B, N), dtype=torch.int32, device=d)
        self.positions = torch.empty((B, N, bs), dtype=torch.int32, device=d)
        self.valid = torch.empty((B, N, bs), dtype=torch.uint8, device=d)
        self.loss_mask = torch.empty((B, N, bs), dtype=torch.uint8, device=d)
        self.num = torch.empty((B,), dtype=torch.int32, device=d)
        self.base = torch.empty((B * N,), dtype=torch.int64, device=d)
        T = B * S
        self.T = T
        self.ctx_pos = torch.arange(S, dtype=torch.int32, device=d).repeat(B)
        self.ctx_k = [torch.empty((w.num_kv_heads, T, w.head_dim), dtype=w.torch_dtype, device=d)
                      for _ in range(w.num_layers)]
        self.ctx_v = [torch.empty((w.num_kv_heads, w.head_dim, T), dtype=w.torch_dtype, device=d)
                      for _ in range(w.num_layers)]
        self.out = torch.empty((w.num_blocks * bs, w.hidden), dtype=w.torch_dtype, device=d)
        self.ws = workspace(lib, self.cfg, w.num_blocks, T, d)

    def plan(self):
        i = self.inp
        self.lib.dflash_build_plan(i["mask"], i["sample_ids"], i["step"], i["plan_seed"],
                                   self.w.anchors_per_row, self.w.block_size, self.anchors,
                                   self.positions, self.valid, self.loss_mask, self.num, self.base)

    def ctx_proj(self):
        w, i = self.w, self.inp
        st = i["states"]                       # [L_t, T, H_t]
        self.lib.dflash_ctx_proj(self.cfg, st, w.target_hidden, self.T * w.target_hidden, self.T,
                                 self.ctx_pos, i["w_proj"], i["layers"], self.ctx_k, self.ctx_v, self.T,
                                 0, self.ws)

    def body(self):
        w, i = self.w, self.inp
        self.lib.dflash_body_forward(self.cfg, w.num_blocks, i["emb"], i["layers"], self.ctx_k,
                                     self.ctx_v, self.T, self.base, self.anchors.reshape(-1),
                                     self.valid.reshape(-1), self.out, self.ws)

    def run(self):
        self.plan()
        self.ctx_proj()
        self.body()
        torch.cuda.synchronize()
        return self


def oracle_row_context(w: Workload, inputs, b: int, rows: int, layers=None):
    """Oracle context K/V (per layer, [Hkv, rows, D], K rotated) of the first
    `rows` positions of training sequence b, projected from the target states."""
    S = w.seq_len
    layers = layers64(inputs["layers"]) if layers is None else layers
    rows = max(int(rows), 1)
    states = np64(inputs["states"][:, b * S: b * S + rows])
    C = oracle.ctx_proj(oracle.concat_target_states(states), np64(inputs["w_proj"]))
    del states
    return oracle.ctx_kv(C, layers, np.arange(rows), w.num_kv_heads, w.head_dim, w.rope_theta)


def oracle_training_blocks(w: Workload, inputs, anchors: np.ndarray, valid: np.ndarray,
                           blocks: Sequence[int], contexts: Optional[Dict[int, tuple]] = None,
                           layers=None) -> np.ndarray:
    """Oracle body outputs [len(blocks)*bs, H] for the chosen blocks of a
    training-shaped workload. Only the context rows each block can read are
    projected (rows [0, max anchor) of the rows involved), unless `contexts`
    already holds sequence b's oracle context K/V (from oracle_row_context)
    covering those rows."""
    bs, N = w.block_size, w.anchors_per_row
    layers = layers64(inputs["layers"]) if layers is None else layers
    emb = inputs["emb"]
    by_row: Dict[int, List[int]] = {}
    for n in blocks:
        by_row.setdefault(n // N, []).append(n)
    result = {}
    for b, ns in by_row.items():
        amax = max(int(anchors.reshape(-1)[n]) for n in ns)
        if contexts is not None and b in contexts and contexts[b][0][0].shape[1] >= amax:
            ck, cv = contexts[b]
        else:
            ck, cv = oracle_row_context(w, inputs, b, amax, layers)
        e = np.concatenate([np64(emb[n * bs:(n + 1) * bs]) for n in ns])
        a = np.array([int(anchors.reshape(-1)[n]) for n in ns])
        v = np.concatenate([valid.reshape(-1)[n * bs:(n + 1) * bs] for n in ns])
        o = oracle.body_forward(e, layers, ck, cv, np.zeros(len(ns), np.int64), a, v, oracle_cfg(w))
        for i, n in enumerate(ns):
            result[n] = o[i * bs:(i + 1) * bs]
    return np.concatenate([result[n] for n in blocks])
