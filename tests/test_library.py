"""Host-side checks of libdflash that need no GPU: the library loads, exports
every symbol include/dflash.h declares, sizes workspaces, and rejects bad
arguments before enqueueing anything (only failing calls are made here)."""
import ctypes
import os
import re

import pytest

import block_draft_model_build_amd as d
from dflash_synth import WORKLOADS, scaled

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    declared = _declared()
    assert set(declared) == set(d.EXPORTED)
    lib = ctypes.CDLL(d.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_config_checks():
    for w in WORKLOADS.values():
        assert d.dflash_check_config(d.config_from_workload(w)) == d.DFLASH_OK
    c3 = WORKLOADS["c3"]
    bad = [
        (dict(head_dim=64), d.DFLASH_ERR_UNSUPPORTED),          # bf16 rows must be 256 bytes
        (dict(num_q_heads=30), d.DFLASH_ERR_INVALID_ARG),       # not a multiple of kv heads
        (dict(block_size=17), d.DFLASH_ERR_UNSUPPORTED),        # bs * G > 64
        (dict(block_size=0), d.DFLASH_ERR_INVALID_ARG),
        (dict(hidden=4000), d.DFLASH_ERR_UNSUPPORTED),
        (dict(num_layers=17), d.DFLASH_ERR_UNSUPPORTED),
        (dict(rope_theta=0.0), d.DFLASH_ERR_INVALID_ARG),
    ]
    for change, status in bad:
        assert d.dflash_check_config(d.config_from_workload(scaled(c3, **change))) == status, change
    assert d.dflash_workspace_size(d.config_from_workload(scaled(c3, head_dim=64)), 4, 4) == 0


def test_workspace_size_grows_with_work():
    c = d.config_from_workload(WORKLOADS["c3"])
    a = d.dflash_workspace_size(c, 64, 0)
    b = d.dflash_workspace_size(c, 256, 0)
    e = d.dflash_workspace_size(c, 256, 32768)
    assert 0 < a < b <= e
    assert a % 256 == 0 and b % 256 == 0


def test_status_strings():
    for s in range(6):
        assert d.dflash_status_string(s)
    assert "scratch" in d.dflash_status_string(d.DFLASH_ERR_SCRATCH_LIMIT)
    assert "workspace" in d.dflash_status_string(d.DFLASH_ERR_WORKSPACE)


def _lib():
    return d.library()


def test_rejects_bad_arguments_before_launch():
    lib = _lib()
    cfg = d.config_from_workload(WORKLOADS["c2"])
    fake = 1 << 20                               # 16-byte-aligned non-null value; never dereferenced
    P = ctypes.c_void_p
    # plan: negative sizes, missing outputs
    assert lib.dflash_build_plan(P(fake), -1, 10, P(fake), 0, 0, 4, 4, P(fake), P(fake), P(fake),
                                 P(fake), P(fake), None, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_build_plan(P(fake), 2, 10, P(fake), 0, 0, 4, 0, P(fake), P(fake), P(fake),
                                 P(fake), P(fake), None, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_build_plan(P(fake), 2, 10, None, 0, 0, 4, 4, P(fake), P(fake), P(fake),
                                 P(fake), P(fake), None, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_build_plan(None, 0, 10, None, 0, 0, 4, 4, None, None, None, None, None, None,
                                 None) == d.DFLASH_OK                       # empty batch: no-op
    # attention: null output, workspace too small or misaligned
    args = [ctypes.byref(cfg), 4, P(fake), P(fake), P(fake), P(fake), P(fake), 100, P(fake),
            P(fake), P(fake)]
    assert lib.dflash_block_attn(*args, None, P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_block_attn(*args, P(fake), P(fake), 16, None) == d.DFLASH_ERR_WORKSPACE
    assert lib.dflash_block_attn(*args, P(fake), P(fake + 16), 1 << 40, None) == d.DFLASH_ERR_WORKSPACE
    assert lib.dflash_block_attn(*args, P(fake), None, 1 << 40, None) == d.DFLASH_ERR_WORKSPACE
    misaligned = [ctypes.byref(cfg), 4, P(fake), P(fake), P(fake), P(fake + 2), P(fake), 100,
                  P(fake), P(fake), P(fake)]
    assert lib.dflash_block_attn(*misaligned, P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    # q, k_blk, v_blk (positions 2-4) and out are read and written with 16-byte accesses
    for pos in (2, 3, 4):
        bad = list(args)
        bad[pos] = P(fake + 8)
        assert lib.dflash_block_attn(*bad, P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_block_attn(*args, P(fake + 8), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    # ctx projection: rows past the cache, bad strides
    lw = (d.DFlashLayerWeights * 1)()
    for f in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
        setattr(lw[0], f, fake)
    ptrs = (ctypes.c_void_p * 1)(fake)
    assert lib.dflash_ctx_proj(ctypes.byref(cfg), P(fake), 20480, 4096, 100, P(fake), P(fake), lw,
                               ptrs, ptrs, 50, 0, P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_proj(ctypes.byref(cfg), P(fake), 20481, 4096, 10, P(fake), P(fake), lw,
                               ptrs, ptrs, 50, 0, P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_proj(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), P(fake), lw,
                               ptrs, ptrs, 50, 0, P(fake), 1024, None) == d.DFLASH_ERR_WORKSPACE
    # incremental append: null scatter rows, bad stride, small workspace; truncate: bad sizes
    assert lib.dflash_ctx_append(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), None, P(fake), lw,
                                 ptrs, ptrs, 50, P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_append(ctypes.byref(cfg), P(fake), 20481, 4096, 10, P(fake), P(fake), P(fake), lw,
                                 ptrs, ptrs, 50, P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_append(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), P(fake), P(fake), lw,
                                 ptrs, ptrs, 50, P(fake), 1024, None) == d.DFLASH_ERR_WORKSPACE
    assert lib.dflash_ctx_append(ctypes.byref(cfg), None, 0, 0, 0, None, None, None, None, None, None, 0,
                                 None, 0, None) == d.DFLASH_OK                     # nothing to append
    # allocation-free append: same checks; inputs past the static scratch are
    # refused before anything touches the device (hidden 4096 bf16: 4096 rows fit)
    assert lib.dflash_ctx_append_noalloc(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), None, P(fake),
                                         lw, ptrs, ptrs, 50, None) == d.DFLASH_ERR_INVALID_ARG
    limit = d.DFLASH_NOALLOC_SCRATCH_BYTES // (cfg.hidden * 2)
    assert limit == 4096
    assert lib.dflash_ctx_append_noalloc(ctypes.byref(cfg), P(fake), 20480, 4096, limit + 1, P(fake), P(fake),
                                         P(fake), lw, ptrs, ptrs, 50, None) == d.DFLASH_ERR_SCRATCH_LIMIT
    assert lib.dflash_ctx_append_noalloc(ctypes.byref(cfg), None, 0, 0, 0, None, None, None, None, None, None,
                                         0, None) == d.DFLASH_OK                   # nothing to append
    assert lib.dflash_ctx_truncate(P(fake), P(fake), -1, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_truncate(None, P(fake), 3, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_truncate(None, None, 0, None) == d.DFLASH_OK
    # verification: bad sizes, unknown dtype, missing outputs; empty batch is a no-op
    assert lib.dflash_verify_greedy(P(fake), P(fake), 1, -1, 3, 10, -1, P(fake), P(fake), P(fake),
                                    None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_verify_greedy(P(fake), P(fake), 7, 2, 3, 10, -1, P(fake), P(fake), P(fake),
                                    None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_verify_greedy(P(fake), P(fake), 1, 2, 3, 0, -1, P(fake), P(fake), P(fake),
                                    None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_verify_greedy(None, P(fake), 1, 2, 3, 10, -1, P(fake), P(fake), P(fake),
                                    None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_verify_greedy(None, None, 1, 0, 3, 10, -1, None, None, None, None) == d.DFLASH_OK
    assert lib.dflash_verify_sample(P(fake), P(fake), None, P(fake), P(fake), 2, 3, 10, -1, P(fake),
                                    P(fake), P(fake), None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_verify_sample(P(fake), P(fake), P(fake), P(fake), P(fake), 2, 3, 1 << 30, -1,
                                    P(fake), P(fake), P(fake), None) == d.DFLASH_ERR_UNSUPPORTED
    assert lib.dflash_verify_sample(None, None, None, None, None, 0, 3, 10, -1, None, None, None,
                                    None) == d.DFLASH_OK
    # LM head + CE: bad tau, bad vocab, small workspace
    assert lib.dflash_lm_head_ce(ctypes.byref(cfg), 16, P(fake), P(fake), 100, P(fake), P(fake), 0.0, P(fake),
                                 P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_lm_head_ce(ctypes.byref(cfg), 16, P(fake), P(fake), 0, P(fake), P(fake), 2.0, P(fake),
                                 P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_lm_head_ce(ctypes.byref(cfg), 16, P(fake), P(fake), 100, P(fake), P(fake), 2.0, P(fake),
                                 P(fake), P(fake), 64, None) == d.DFLASH_ERR_WORKSPACE
    assert d.dflash_lm_head_ce_workspace_size(16, 100) > 0 and d.dflash_lm_head_ce_workspace_size(-1, 100) == 0
    # kept logits: null or small buffer; their size; the saved backward's checks
    assert d.dflash_lm_head_ce_logits_size(16, 100) == 16 * 128 * 4
    assert d.dflash_lm_head_ce_logits_size(-1, 100) == 0 and d.dflash_lm_head_ce_logits_size(16, 0) == 0
    assert lib.dflash_lm_head_ce_train(ctypes.byref(cfg), 16, P(fake), P(fake), 100, P(fake), P(fake), 2.0, P(fake),
                                       P(fake), None, 1 << 40, P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_lm_head_ce_train(ctypes.byref(cfg), 16, P(fake), P(fake), 100, P(fake), P(fake), 2.0, P(fake),
                                       P(fake), P(fake), 16 * 128 * 4 - 1, P(fake), 1 << 40,
                                       None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_lm_head_ce_train(ctypes.byref(cfg), 16, P(fake), P(fake), 100, P(fake), P(fake), 2.0, P(fake),
                                       P(fake), P(fake), 1 << 40, P(fake), 64, None) == d.DFLASH_ERR_WORKSPACE
    saved = lambda logits, head_t, head_t_bytes, tau, ws_bytes, rows=16: lib.dflash_lm_head_ce_backward_saved(
        ctypes.byref(cfg), rows, logits, 1 << 40, P(fake), head_t, head_t_bytes, 100, P(fake), P(fake), tau,
        P(fake), 1.0, P(fake), P(fake), ws_bytes, None)
    assert saved(None, None, 0, 2.0, 1 << 40) == d.DFLASH_ERR_INVALID_ARG
    assert saved(P(fake), None, 0, 0.0, 1 << 40) == d.DFLASH_ERR_INVALID_ARG
    assert saved(P(fake), None, 0, 2.0, 64) == d.DFLASH_ERR_WORKSPACE
    assert saved(None, None, 0, 2.0, 0, rows=0) == d.DFLASH_OK
    # a kept transposed head: its size; small or misaligned buffers are refused
    tsize = d.dflash_lm_head_transpose_size(cfg, 100)
    assert tsize == cfg.hidden * 128 * (2 if cfg.dtype == d.DFLASH_BF16 else 4)
    assert d.dflash_lm_head_transpose_size(cfg, 0) == 0
    assert saved(P(fake), P(fake), tsize - 1, 2.0, 1 << 40) == d.DFLASH_ERR_INVALID_ARG
    assert saved(P(fake), P(fake + 8), tsize, 2.0, 1 << 40) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_lm_head_ce_backward(ctypes.byref(cfg), 16, P(fake), P(fake), P(fake), tsize - 1, 100, P(fake),
                                          P(fake), 2.0, P(fake), 1.0, P(fake), P(fake), 1 << 40,
                                          None) == d.DFLASH_ERR_INVALID_ARG
    transpose = lambda head, vocab, out, nbytes: lib.dflash_lm_head_transpose(ctypes.byref(cfg), head, vocab, out,
                                                                             nbytes, None)
    assert transpose(P(fake), 100, P(fake), tsize - 1) == d.DFLASH_ERR_INVALID_ARG
    assert transpose(P(fake), 100, None, tsize) == d.DFLASH_ERR_INVALID_ARG
    assert transpose(None, 100, P(fake), tsize) == d.DFLASH_ERR_INVALID_ARG
    assert transpose(P(fake), 100, P(fake + 8), tsize) == d.DFLASH_ERR_INVALID_ARG
    assert transpose(P(fake), 0, P(fake), tsize) == d.DFLASH_ERR_INVALID_ARG
    # optimizer step: dtype, step, rates, eps, sizes, null or misaligned arrays; empty calls
    T = d.DFlashAdamWTensor
    good = (T * 1)(T(fake, fake, fake, fake, fake, 100))
    args = lambda **k: dict(dict(dt=d.DFLASH_BF16, n=1, t=good, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0,
                                 step=1), **k)
    def adam(a):
        return lib.dflash_adamw_step(a["dt"], a["n"], a["t"], a["lr"], a["b1"], a["b2"], a["eps"], a["wd"],
                                     a["step"], None)
    for bad in (dict(dt=7), dict(n=-1), dict(step=0), dict(lr=-1.0), dict(b1=1.0), dict(b2=-0.1),
                dict(eps=0.0), dict(wd=-1.0), dict(t=None)):
        assert adam(args(**bad)) == d.DFLASH_ERR_INVALID_ARG, bad
    assert adam(args(t=(T * 1)(T(fake, fake, fake, fake, fake, -1)))) == d.DFLASH_ERR_INVALID_ARG
    assert adam(args(t=(T * 1)(T(None, fake, fake, fake, fake, 4)))) == d.DFLASH_ERR_INVALID_ARG
    assert adam(args(t=(T * 1)(T(fake, fake + 4, fake, fake, fake, 4)))) == d.DFLASH_ERR_INVALID_ARG
    assert adam(args(t=(T * 1)(T(fake, fake, fake, fake, fake + 8, 4)))) == d.DFLASH_ERR_INVALID_ARG
    assert adam(args(n=0, t=None)) == d.DFLASH_OK
    assert adam(args(t=(T * 1)(T(None, None, None, None, None, 0)))) == d.DFLASH_OK
    # attention backward: negative sizes, a null gradient, a small workspace, nothing to do
    F = [P(fake)] * 3
    assert lib.dflash_block_attn_backward(ctypes.byref(cfg), -1, *F, P(fake), P(fake), 64, *F, P(fake), P(fake),
                                          *F, P(fake), P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_block_attn_backward(ctypes.byref(cfg), 4, *F, P(fake), P(fake), 64, *F, P(fake), P(fake),
                                          P(fake), None, P(fake), P(fake), P(fake), P(fake), 1 << 40,
                                          None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_block_attn_backward(ctypes.byref(cfg), 4, *F, P(fake), P(fake), 64, *F, P(fake), P(fake),
                                          *F, P(fake), P(fake), P(fake), 64, None) == d.DFLASH_ERR_WORKSPACE
    assert lib.dflash_block_attn_backward(ctypes.byref(cfg), 0, *([None] * 5), 0, *([None] * 10), None, 0,
                                          None) == d.DFLASH_OK
    assert d.dflash_block_attn_backward_workspace_size(cfg, 4) > 0
    assert d.dflash_block_attn_backward_workspace_size(cfg, -1) == 0
    # context-path backward: rows past the cache, null output, unsupported width, small workspace
    G = (ctypes.c_void_p * cfg.num_layers)(*([fake] * cfg.num_layers))
    assert lib.dflash_ctx_proj_backward(ctypes.byref(cfg), P(fake), 20480, 4096, 100, P(fake), lw, G, G, 50, 0,
                                        P(fake), None, None, None, None, P(fake), 1 << 40,
                                        None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_proj_backward(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), lw, G, G, 50, 0,
                                        None, None, None, None, None, P(fake), 1 << 40,
                                        None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_proj_backward(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), lw, G, G, 50, 0,
                                        P(fake), None, None, None, None, P(fake), 64,
                                        None) == d.DFLASH_ERR_WORKSPACE
    # with C for the K/V weight gradients: their arrays are required and aligned
    assert lib.dflash_ctx_proj_backward(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), lw, G, G, 50, 0,
                                        P(fake), None, P(fake), None, G, P(fake), 1 << 40,
                                        None) == d.DFLASH_ERR_INVALID_ARG
    Gbad = (ctypes.c_void_p * cfg.num_layers)(*([fake + 4] * cfg.num_layers))
    assert lib.dflash_ctx_proj_backward(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), lw, G, G, 50, 0,
                                        P(fake), None, P(fake), G, Gbad, P(fake), 1 << 40,
                                        None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_proj_backward(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), lw, G, G, 50, 0,
                                        P(fake), None, P(fake + 8), G, G, P(fake), 1 << 40,
                                        None) == d.DFLASH_ERR_INVALID_ARG
    # the training context projection needs its C buffer
    assert lib.dflash_ctx_proj_train(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), P(fake), lw, G, G, 50,
                                     0, None, P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    assert lib.dflash_ctx_proj_train(ctypes.byref(cfg), P(fake), 20480, 4096, 10, P(fake), P(fake), lw, G, G, 50,
                                     0, P(fake + 8), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    odd = d.config_from_workload(scaled(WORKLOADS["c2"], target_hidden=4032))
    assert lib.dflash_ctx_proj_backward(ctypes.byref(odd), P(fake), 5 * 4032, 4032, 10, P(fake), lw, G, G, 50, 0,
                                        P(fake), None, None, None, None, P(fake), 1 << 40,
                                        None) == d.DFLASH_ERR_UNSUPPORTED
    assert d.dflash_ctx_proj_backward_workspace_size(cfg, 100) > d.dflash_ctx_proj_backward_workspace_size(cfg, 10)
    # body: misaligned embeddings (16-byte reads), a null weight
    w_up = lw[0].w_up
    assert lib.dflash_body_forward(ctypes.byref(cfg), 4, P(fake + 8), lw, ptrs, ptrs, 100, P(fake),
                                   P(fake), P(fake), P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    lw[0].w_up = None
    assert lib.dflash_body_forward(ctypes.byref(cfg), 4, P(fake), lw, ptrs, ptrs, 100, P(fake),
                                   P(fake), P(fake), P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_INVALID_ARG
    lw[0].w_up = w_up
    # unsupported config is reported before anything else
    bad = d.config_from_workload(scaled(WORKLOADS["c2"], head_dim=64))
    assert lib.dflash_body_forward(ctypes.byref(bad), 4, P(fake), lw, ptrs, ptrs, 100, P(fake),
                                   P(fake), P(fake), P(fake), P(fake), 1 << 40, None) == d.DFLASH_ERR_UNSUPPORTED


def test_body_training_entry_points_reject_bad_arguments():
    # Checked on the host before anything is enqueued, so no GPU is needed.
    lib = d.library()
    fake = 1 << 20
    P = ctypes.c_void_p
    c3 = WORKLOADS["c3"]
    cfg = d.config_from_workload(c3)
    L = c3.num_layers
    lw = (d.DFlashLayerWeights * L)()
    for i in range(L):
        for f in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            setattr(lw[i], f, fake)
    grads = (d.DFlashLayerGrads * L)()
    for i in range(L):
        for f in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            setattr(grads[i], f, fake)
    ptrs = (ctypes.c_void_p * L)(*([fake] * L))
    big = 1 << 44
    # training forward: a null, small or misaligned reserve
    need = d.dflash_body_train_reserve_size(cfg, 4)
    assert need > 0 and d.dflash_body_train_reserve_size(cfg, -1) == 0

    def fwd(res=P(fake), nbytes=need, nbw=big):
        return lib.dflash_body_forward_train(ctypes.byref(cfg), 4, P(fake), lw, ptrs, ptrs, 100, P(fake), P(fake),
                                             P(fake), P(fake), res, nbytes, P(fake), nbw, None)
    assert fwd(res=None) == d.DFLASH_ERR_INVALID_ARG
    assert fwd(nbytes=need - 1) == d.DFLASH_ERR_WORKSPACE
    assert fwd(res=P(fake + 16)) == d.DFLASH_ERR_WORKSPACE
    assert fwd(nbw=64) == d.DFLASH_ERR_WORKSPACE

    def bwd(c=cfg, nb=4, hs=P(fake), rb=big, g=grads, dout=P(fake), demb=None, ws=P(fake), nbytes=big):
        return lib.dflash_body_backward(ctypes.byref(c), nb, hs, rb, lw, ptrs, ptrs, 100, P(fake), P(fake), P(fake),
                                        dout, demb, g, ptrs, ptrs, ws, nbytes, None)
    assert bwd(nb=-1) == d.DFLASH_ERR_INVALID_ARG
    assert bwd(hs=None) == d.DFLASH_ERR_INVALID_ARG
    assert bwd(dout=None) == d.DFLASH_ERR_INVALID_ARG
    assert bwd(demb=P(fake + 8)) == d.DFLASH_ERR_INVALID_ARG
    assert bwd(g=None) == d.DFLASH_ERR_INVALID_ARG
    w_up = grads[2].w_up
    grads[2].w_up = None
    assert bwd() == d.DFLASH_ERR_INVALID_ARG
    grads[2].w_up = w_up
    assert bwd(nbytes=64) == d.DFLASH_ERR_WORKSPACE
    assert bwd(rb=need - 1) == d.DFLASH_ERR_WORKSPACE
    assert bwd(ws=P(fake + 16)) == d.DFLASH_ERR_WORKSPACE
    # shapes outside the backward's envelope: intermediate not a multiple of 128, hidden > 8192
    for change in (dict(intermediate=12288 + 64), dict(hidden=8192 + 128)):
        odd = d.config_from_workload(scaled(c3, **change))
        assert d.dflash_check_config(odd) == d.DFLASH_OK, change
        assert bwd(c=odd) == d.DFLASH_ERR_UNSUPPORTED, change
        assert d.dflash_body_backward_workspace_size(odd, 4) == 0, change
    # the workspace grows with the blocks
    assert 0 < d.dflash_body_backward_workspace_size(cfg, 64) < d.dflash_body_backward_workspace_size(cfg, 256)


def test_product_path_does_not_reach_the_oracle():
    pkg = os.path.join(ROOT, "block_draft_model_build_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_vt_dma_offset_limit(tmp_path):
    # The attention kernel's direct-to-LDS V^T loads form a 32-bit lane offset
    # (15 * ctx_total + 15 * elems_per_chunk) * elem_bytes; the helper's limit
    # must be the largest cache length for which that offset still fits.
    import shutil
    import subprocess
    gxx = shutil.which("g++") or shutil.which("c++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "lim.cpp"
    src.write_text('#include <stdio.h>\n#include "dma_limits.h"\n'
                   'int main() { printf("%lld %lld\\n", (long long)dflash::vt_dma_max_ctx(2, 8),'
                   ' (long long)dflash::vt_dma_max_ctx(4, 4)); return 0; }\n')
    exe = tmp_path / "lim"
    subprocess.run([gxx, "-std=c++17", "-I", os.path.join(ROOT, "block_draft_model_build_amd", "csrc"),
                    str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    for lim, (eb, ec) in zip(got, ((2, 8), (4, 4))):
        off = lambda t: (15 * t + 15 * ec) * eb            # largest lane offset, in bytes
        assert off(lim) <= 2**32 - 1 < off(lim + 1)
    assert got[0] == 143_165_568
    # The kernel's guard uses the helper (and no other bound on ctx_total).
    att = open(os.path.join(ROOT, "block_draft_model_build_amd", "csrc", "attention.h")).read()
    guard = re.search(r"auto tile_dma_ok = \[&\]\(int t0\) \{(.*?)\};", att, flags=re.S).group(1)
    assert "vt_dma_max_ctx(EB, TT::EC)" in guard and "1 << 28" not in guard
