"""Python binding of libdflash: the DFlash draft-body forward on MI355X (gfx950).

Argument marshalling only. Every call goes to the C ABI declared in
include/dflash.h; all computation runs in the library's HIP kernels. Tensors
are torch tensors used as device buffers (their data pointers are passed);
the stream defaults to torch's current stream on the tensor's device.

The names mirror the C entry points:
  dflash_build_plan, dflash_ctx_proj, dflash_ctx_proj_train, dflash_ctx_append, dflash_ctx_append_noalloc,
  dflash_ctx_truncate,
  dflash_block_attn, dflash_body_forward, dflash_verify_greedy,
  dflash_verify_sample, dflash_lm_head_ce, dflash_lm_head_ce_workspace_size,
  dflash_lm_head_ce_backward, dflash_lm_head_ce_backward_workspace_size,
  dflash_lm_head_ce_train, dflash_lm_head_ce_logits_size, dflash_lm_head_ce_backward_saved,
  dflash_lm_head_transpose, dflash_lm_head_transpose_size,
  dflash_block_attn_backward, dflash_block_attn_backward_workspace_size,
  dflash_ctx_proj_backward, dflash_ctx_proj_backward_workspace_size,
  dflash_body_forward_train, dflash_body_train_reserve_size, dflash_body_backward,
  dflash_body_backward_workspace_size, dflash_adamw_step,
  dflash_workspace_size, dflash_check_config, dflash_status_string.

If libdflash.so is missing it is built in-tree with hipcc on first import; if
that fails, importing this package raises ImportError. There is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

(DFLASH_OK, DFLASH_ERR_INVALID_ARG, DFLASH_ERR_UNSUPPORTED, DFLASH_ERR_WORKSPACE, DFLASH_ERR_HIP,
 DFLASH_ERR_SCRATCH_LIMIT) = range(6)
DFLASH_NOALLOC_SCRATCH_BYTES = 32 << 20
DFLASH_F32, DFLASH_BF16 = 0, 1

EXPORTED = ("dflash_build_plan", "dflash_ctx_proj", "dflash_ctx_proj_train", "dflash_ctx_append",
            "dflash_ctx_append_noalloc",
            "dflash_ctx_truncate",
            "dflash_block_attn", "dflash_body_forward", "dflash_verify_greedy", "dflash_verify_sample",
            "dflash_lm_head_ce", "dflash_lm_head_ce_workspace_size",
            "dflash_lm_head_ce_backward", "dflash_lm_head_ce_backward_workspace_size",
            "dflash_lm_head_ce_train", "dflash_lm_head_ce_logits_size", "dflash_lm_head_ce_backward_saved",
            "dflash_lm_head_transpose", "dflash_lm_head_transpose_size",
            "dflash_block_attn_backward", "dflash_block_attn_backward_workspace_size",
            "dflash_ctx_proj_backward", "dflash_ctx_proj_backward_workspace_size",
            "dflash_body_forward_train", "dflash_body_train_reserve_size", "dflash_body_backward",
            "dflash_body_backward_workspace_size", "dflash_adamw_step",
            "dflash_workspace_size", "dflash_check_config", "dflash_status_string",
            "dflash_profile_start", "dflash_profile_stop")

# dflash_kernel ids for the measurement hook
KERNELS = {"plan": 0, "ctx_proj": 1, "ctx_kv": 2, "rmsnorm": 3, "qkv": 4, "attention": 5,
           "attn_combine": 6, "o_proj": 7, "gate_up": 8, "down": 9, "verify": 10,
           "lm_head": 11, "lm_ce": 12, "attn_bwd": 13,
           "ctx_bwd_pack": 14, "ctx_bwd_dc": 15, "ctx_bwd_dw": 16,
           "bwd_pack": 17, "bwd_data": 18, "bwd_weight": 19, "bwd_norm": 20,
           "lm_bwd_prep": 21, "lm_bwd_dz": 22, "lm_bwd_dh": 23, "ctx_bwd_dkv": 24}


class DFlashConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("num_target_layers", ctypes.c_int32), ("target_hidden", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_float)]


_LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


class DFlashLayerWeights(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _LAYER_FIELDS]


class DFlashLayerGrads(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _LAYER_FIELDS]


class DFlashAdamWTensor(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("master", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class DFlashError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {dflash_status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                            ctypes.c_size_t)
    CFG = ctypes.POINTER(DFlashConfig)
    lib.dflash_build_plan.argtypes = [P, I32, I32, P, I64, U64, I32, I32, P, P, P, P, P, P, P]
    lib.dflash_build_plan.restype = ctypes.c_int
    lib.dflash_ctx_proj.argtypes = [CFG, P, I64, I64, I64, P, P, P, P, P, I64, I64, P, SZ, P]
    lib.dflash_ctx_proj.restype = ctypes.c_int
    lib.dflash_ctx_proj_train.argtypes = [CFG, P, I64, I64, I64, P, P, P, P, P, I64, I64, P, P, SZ, P]
    lib.dflash_ctx_proj_train.restype = ctypes.c_int
    lib.dflash_ctx_append.argtypes = [CFG, P, I64, I64, I64, P, P, P, P, P, P, I64, P, SZ, P]
    lib.dflash_ctx_append.restype = ctypes.c_int
    lib.dflash_ctx_append_noalloc.argtypes = [CFG, P, I64, I64, I64, P, P, P, P, P, P, I64, P]
    lib.dflash_ctx_append_noalloc.restype = ctypes.c_int
    lib.dflash_ctx_truncate.argtypes = [P, P, I32, P]
    lib.dflash_ctx_truncate.restype = ctypes.c_int
    lib.dflash_block_attn.argtypes = [CFG, I32, P, P, P, P, P, I64, P, P, P, P, P, SZ, P]
    lib.dflash_block_attn.restype = ctypes.c_int
    lib.dflash_body_forward.argtypes = [CFG, I32, P, P, P, P, I64, P, P, P, P, P, SZ, P]
    lib.dflash_body_forward.restype = ctypes.c_int
    lib.dflash_verify_greedy.argtypes = [P, P, I32, I32, I32, I32, I32, P, P, P, P]
    lib.dflash_verify_greedy.restype = ctypes.c_int
    lib.dflash_verify_sample.argtypes = [P, P, P, P, P, I32, I32, I32, I32, P, P, P, P]
    lib.dflash_verify_sample.restype = ctypes.c_int
    lib.dflash_lm_head_ce.argtypes = [CFG, I32, P, P, I32, P, P, ctypes.c_double, P, P, P, SZ, P]
    lib.dflash_lm_head_ce.restype = ctypes.c_int
    lib.dflash_lm_head_ce_backward.argtypes = [CFG, I32, P, P, P, SZ, I32, P, P, ctypes.c_double, P,
                                               ctypes.c_double, P, P, SZ, P]
    lib.dflash_lm_head_transpose.argtypes = [CFG, P, I32, P, SZ, P]
    lib.dflash_lm_head_transpose.restype = ctypes.c_int
    lib.dflash_lm_head_transpose_size.argtypes = [CFG, I32]
    lib.dflash_lm_head_transpose_size.restype = ctypes.c_size_t
    lib.dflash_lm_head_ce_backward.restype = ctypes.c_int
    lib.dflash_lm_head_ce_backward_workspace_size.argtypes = [CFG, I32, I32]
    lib.dflash_lm_head_ce_backward_workspace_size.restype = ctypes.c_size_t
    lib.dflash_lm_head_ce_workspace_size.argtypes = [I32, I32]
    lib.dflash_lm_head_ce_workspace_size.restype = ctypes.c_size_t
    lib.dflash_lm_head_ce_train.argtypes = [CFG, I32, P, P, I32, P, P, ctypes.c_double, P, P, P, SZ, P, SZ, P]
    lib.dflash_lm_head_ce_train.restype = ctypes.c_int
    lib.dflash_lm_head_ce_logits_size.argtypes = [I32, I32]
    lib.dflash_lm_head_ce_logits_size.restype = ctypes.c_size_t
    lib.dflash_lm_head_ce_backward_saved.argtypes = [CFG, I32, P, SZ, P, P, SZ, I32, P, P, ctypes.c_double, P,
                                                     ctypes.c_double, P, P, SZ, P]
    lib.dflash_lm_head_ce_backward_saved.restype = ctypes.c_int
    lib.dflash_block_attn_backward.argtypes = [CFG, I32, P, P, P, P, P, I64, P, P, P, P, P, P, P, P, P, P, P,
                                               SZ, P]
    lib.dflash_block_attn_backward.restype = ctypes.c_int
    lib.dflash_block_attn_backward_workspace_size.argtypes = [CFG, I32]
    lib.dflash_block_attn_backward_workspace_size.restype = ctypes.c_size_t
    lib.dflash_ctx_proj_backward.argtypes = [CFG, P, I64, I64, I64, P, P, P, P, I64, I64, P, P, P, P, P, P, SZ,
                                             P]
    lib.dflash_ctx_proj_backward.restype = ctypes.c_int
    lib.dflash_body_forward_train.argtypes = [CFG, I32, P, P, P, P, I64, P, P, P, P, P, SZ, P, SZ, P]
    lib.dflash_body_forward_train.restype = ctypes.c_int
    lib.dflash_body_train_reserve_size.argtypes = [CFG, I32]
    lib.dflash_body_train_reserve_size.restype = ctypes.c_size_t
    lib.dflash_body_backward.argtypes = [CFG, I32, P, SZ, P, P, P, I64, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.dflash_body_backward.restype = ctypes.c_int
    lib.dflash_body_backward_workspace_size.argtypes = [CFG, I32]
    lib.dflash_body_backward_workspace_size.restype = ctypes.c_size_t
    lib.dflash_adamw_step.argtypes = [I32, I32, P, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_double, ctypes.c_double, I64, P]
    lib.dflash_adamw_step.restype = ctypes.c_int
    lib.dflash_ctx_proj_backward_workspace_size.argtypes = [CFG, I64]
    lib.dflash_ctx_proj_backward_workspace_size.restype = ctypes.c_size_t
    lib.dflash_workspace_size.argtypes = [CFG, I32, I64]
    lib.dflash_workspace_size.restype = ctypes.c_size_t
    lib.dflash_check_config.argtypes = [CFG]
    lib.dflash_check_config.restype = ctypes.c_int
    lib.dflash_profile_start.argtypes = [I32, I32]
    lib.dflash_profile_start.restype = ctypes.c_int
    lib.dflash_profile_stop.argtypes = [P, P]
    lib.dflash_profile_stop.restype = ctypes.c_int
    lib.dflash_status_string.argtypes = [ctypes.c_int]
    lib.dflash_status_string.restype = ctypes.c_char_p
    return lib


try:
    _lib = _load()
except Exception as exc:  # noqa: BLE001 - surface any build/load failure as ImportError
    raise ImportError(f"libdflash is not available ({LIB_PATH}): {exc}") from exc


def library() -> ctypes.CDLL:
    return _lib


# ----------------------------------------------------------------- marshalling helpers
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def make_config(hidden, num_q_heads, num_kv_heads, head_dim, intermediate, num_layers,
                num_target_layers, target_hidden, block_size, dtype, rope_theta=1e6,
                rms_eps=1e-6) -> DFlashConfig:
    dt = {"f32": DFLASH_F32, "bf16": DFLASH_BF16}.get(dtype, dtype)
    return DFlashConfig(hidden, num_q_heads, num_kv_heads, head_dim, intermediate, num_layers,
                        num_target_layers, target_hidden, block_size, int(dt), float(rope_theta),
                        float(rms_eps))


def config_from_workload(w) -> DFlashConfig:
    """Config from a workload description (attributes named as in DFlashConfig)."""
    return make_config(w.hidden, w.num_q_heads, w.num_kv_heads, w.head_dim, w.intermediate,
                       w.num_layers, w.num_target_layers, w.target_hidden, w.block_size, w.dtype,
                       w.rope_theta, w.rms_eps)


def _layers(layers: Sequence[Dict[str, object]]):
    arr = (DFlashLayerWeights * len(layers))()
    for i, L in enumerate(layers):
        for f in _LAYER_FIELDS:
            setattr(arr[i], f, _ptr(L.get(f)) if isinstance(L, dict) else _ptr(getattr(L, f)))
    return arr


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


def _check(fn, status):
    if status != DFLASH_OK:
        raise DFlashError(fn, status)


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


# ----------------------------------------------------------------- entry points
def dflash_status_string(status: int) -> str:
    return _lib.dflash_status_string(int(status)).decode()


def dflash_check_config(cfg: DFlashConfig) -> int:
    return _lib.dflash_check_config(ctypes.byref(cfg))


def dflash_workspace_size(cfg: DFlashConfig, num_blocks: int, ctx_rows: int) -> int:
    return _lib.dflash_workspace_size(ctypes.byref(cfg), int(num_blocks), int(ctx_rows))


def dflash_build_plan(mask, sample_ids, step: int, seed: int, anchors_per_row: int, block_size: int,
                      anchors, positions, valid, loss_mask, num_anchors, block_ctx_base=None,
                      stream=None) -> None:
    B, S = mask.shape
    s = _lib.dflash_build_plan(_ptr(mask), B, S, _ptr(sample_ids), int(step),
                               int(seed) & ((1 << 64) - 1), int(anchors_per_row), int(block_size),
                               _ptr(anchors), _ptr(positions), _ptr(valid), _ptr(loss_mask),
                               _ptr(num_anchors), _ptr(block_ctx_base), _stream(stream, mask))
    _check("dflash_build_plan", s)


def dflash_ctx_proj(cfg: DFlashConfig, target_states, ts_row_stride: int, ts_layer_stride: int,
                    num_rows: int, positions, w_proj, layers, ctx_k: List, ctx_v: List,
                    ctx_total: int, row_offset: int, workspace, stream=None) -> None:
    lw = _layers(layers)
    ck, cv = _ptr_array(ctx_k), _ptr_array(ctx_v)
    wp, wb = _ws(workspace)
    s = _lib.dflash_ctx_proj(ctypes.byref(cfg), _ptr(target_states), int(ts_row_stride),
                             int(ts_layer_stride), int(num_rows), _ptr(positions), _ptr(w_proj), lw,
                             ck, cv, int(ctx_total), int(row_offset), wp, wb,
                             _stream(stream, target_states))
    _check("dflash_ctx_proj", s)


def dflash_ctx_proj_train(cfg: DFlashConfig, target_states, ts_row_stride: int, ts_layer_stride: int,
                          num_rows: int, positions, w_proj, layers, ctx_k: List, ctx_v: List,
                          ctx_total: int, row_offset: int, ctx_hidden, workspace, stream=None) -> None:
    """dflash_ctx_proj that also writes C = X W_proj^T into ctx_hidden [num_rows, H] (config dtype)."""
    lw = _layers(layers)
    ck, cv = _ptr_array(ctx_k), _ptr_array(ctx_v)
    wp, wb = _ws(workspace)
    s = _lib.dflash_ctx_proj_train(ctypes.byref(cfg), _ptr(target_states), int(ts_row_stride),
                                   int(ts_layer_stride), int(num_rows), _ptr(positions), _ptr(w_proj), lw,
                                   ck, cv, int(ctx_total), int(row_offset), _ptr(ctx_hidden), wp, wb,
                                   _stream(stream, target_states))
    _check("dflash_ctx_proj_train", s)


def dflash_ctx_append(cfg: DFlashConfig, target_states, ts_row_stride: int, ts_layer_stride: int,
                      num_rows: int, positions, dst_rows, w_proj, layers, ctx_k: List, ctx_v: List,
                      ctx_total: int, workspace, stream=None) -> None:
    lw = _layers(layers)
    ck, cv = _ptr_array(ctx_k), _ptr_array(ctx_v)
    wp, wb = _ws(workspace)
    s = _lib.dflash_ctx_append(ctypes.byref(cfg), _ptr(target_states), int(ts_row_stride),
                               int(ts_layer_stride), int(num_rows), _ptr(positions), _ptr(dst_rows),
                               _ptr(w_proj), lw, ck, cv, int(ctx_total), wp, wb,
                               _stream(stream, target_states))
    _check("dflash_ctx_append", s)


def dflash_ctx_append_noalloc(cfg: DFlashConfig, target_states, ts_row_stride: int, ts_layer_stride: int,
                              num_rows: int, positions, dst_rows, w_proj, layers, ctx_k: List, ctx_v: List,
                              ctx_total: int, stream=None) -> None:
    lw = _layers(layers)
    ck, cv = _ptr_array(ctx_k), _ptr_array(ctx_v)
    s = _lib.dflash_ctx_append_noalloc(ctypes.byref(cfg), _ptr(target_states), int(ts_row_stride),
                                       int(ts_layer_stride), int(num_rows), _ptr(positions), _ptr(dst_rows),
                                       _ptr(w_proj), lw, ck, cv, int(ctx_total), _stream(stream, target_states))
    _check("dflash_ctx_append_noalloc", s)


def dflash_ctx_truncate(lengths, keep, n: int = None, stream=None) -> None:
    n = lengths.numel() if n is None else n
    s = _lib.dflash_ctx_truncate(_ptr(lengths), _ptr(keep), int(n), _stream(stream, lengths))
    _check("dflash_ctx_truncate", s)


def dflash_block_attn(cfg: DFlashConfig, num_blocks: int, q, k_blk, v_blk, ctx_k, ctx_v,
                      ctx_total: int, block_ctx_base, block_anchor, block_valid, out, workspace,
                      stream=None) -> None:
    wp, wb = _ws(workspace)
    s = _lib.dflash_block_attn(ctypes.byref(cfg), int(num_blocks), _ptr(q), _ptr(k_blk), _ptr(v_blk),
                               _ptr(ctx_k), _ptr(ctx_v), int(ctx_total), _ptr(block_ctx_base),
                               _ptr(block_anchor), _ptr(block_valid), _ptr(out), wp, wb,
                               _stream(stream, q))
    _check("dflash_block_attn", s)


def dflash_body_forward(cfg: DFlashConfig, num_blocks: int, block_embeds, layers, ctx_k: List,
                        ctx_v: List, ctx_total: int, block_ctx_base, block_anchor, block_valid, out,
                        workspace, stream=None) -> None:
    lw = _layers(layers)
    ck, cv = _ptr_array(ctx_k), _ptr_array(ctx_v)
    wp, wb = _ws(workspace)
    s = _lib.dflash_body_forward(ctypes.byref(cfg), int(num_blocks), _ptr(block_embeds), lw, ck, cv,
                                 int(ctx_total), _ptr(block_ctx_base), _ptr(block_anchor),
                                 _ptr(block_valid), _ptr(out), wp, wb, _stream(stream, block_embeds))
    _check("dflash_body_forward", s)


def dflash_verify_greedy(draft, target_logits, emitted, num_emitted, accepted, eos_token: int = -1,
                         stream=None) -> None:
    """draft [B, gamma] i32, target_logits [B, gamma + 1, V] bf16/f32 -> emitted [B, gamma + 1],
    num_emitted [B], accepted [B] (i32)."""
    import torch
    B, g1, V = target_logits.shape
    dt = DFLASH_BF16 if target_logits.dtype == torch.bfloat16 else DFLASH_F32
    s = _lib.dflash_verify_greedy(_ptr(draft), _ptr(target_logits), dt, int(B), int(g1 - 1), int(V),
                                  int(eos_token), _ptr(emitted), _ptr(num_emitted), _ptr(accepted),
                                  _stream(stream, target_logits))
    _check("dflash_verify_greedy", s)


def dflash_verify_sample(draft, p, q, u_accept, u_draw, emitted, num_emitted, accepted, eos_token: int = -1,
                         stream=None) -> None:
    """draft [B, gamma] i32, p [B, gamma + 1, V] f32, q [B, gamma, V] f32, u_accept [B, gamma] f32,
    u_draw [B] f32 -> emitted [B, gamma + 1], num_emitted [B], accepted [B] (i32)."""
    B, g1, V = p.shape
    s = _lib.dflash_verify_sample(_ptr(draft), _ptr(p), _ptr(q), _ptr(u_accept), _ptr(u_draw), int(B),
                                  int(g1 - 1), int(V), int(eos_token), _ptr(emitted), _ptr(num_emitted),
                                  _ptr(accepted), _stream(stream, p))
    _check("dflash_verify_sample", s)


def dflash_lm_head_ce_workspace_size(rows: int, vocab: int) -> int:
    return _lib.dflash_lm_head_ce_workspace_size(int(rows), int(vocab))


def dflash_lm_head_ce(cfg: DFlashConfig, hidden, lm_head, targets, loss_mask, decay_tau: float, row_ce, loss,
                      workspace, stream=None) -> None:
    """hidden [rows, H], lm_head [V, H] (config dtype), targets [rows] i32, loss_mask [rows] u8
    -> row_ce [rows] f32, loss [1] f64."""
    rows = hidden.shape[0]
    vocab = lm_head.shape[0]
    wp, wb = _ws(workspace)
    s = _lib.dflash_lm_head_ce(ctypes.byref(cfg), int(rows), _ptr(hidden), _ptr(lm_head), int(vocab), _ptr(targets),
                               _ptr(loss_mask), float(decay_tau), _ptr(row_ce), _ptr(loss), wp, wb,
                               _stream(stream, lm_head))
    _check("dflash_lm_head_ce", s)


def dflash_lm_head_ce_logits_size(rows: int, vocab: int) -> int:
    return _lib.dflash_lm_head_ce_logits_size(int(rows), int(vocab))


def dflash_lm_head_ce_train(cfg: DFlashConfig, hidden, lm_head, targets, loss_mask, decay_tau: float, row_ce, loss,
                            logits, workspace, stream=None) -> None:
    """dflash_lm_head_ce that also writes the fp32 logits into `logits` (a device buffer of
    dflash_lm_head_ce_logits_size(rows, vocab) bytes or more; rows of vocab rounded up to 64)."""
    rows = hidden.shape[0]
    vocab = lm_head.shape[0]
    wp, wb = _ws(workspace)
    lp, lb = _ws(logits)
    s = _lib.dflash_lm_head_ce_train(ctypes.byref(cfg), int(rows), _ptr(hidden), _ptr(lm_head), int(vocab),
                                     _ptr(targets), _ptr(loss_mask), float(decay_tau), _ptr(row_ce), _ptr(loss),
                                     lp, lb, wp, wb, _stream(stream, lm_head))
    _check("dflash_lm_head_ce_train", s)


def dflash_lm_head_ce_backward_saved(cfg: DFlashConfig, rows: int, logits, lm_head, targets, loss_mask,
                                     decay_tau: float, row_ce, d_loss: float, d_hidden, workspace,
                                     stream=None, lm_head_t=None) -> None:
    """dflash_lm_head_ce_backward from the logits dflash_lm_head_ce_train kept -> d_hidden [rows, H];
    lm_head_t: an optional kept dflash_lm_head_transpose of the head."""
    vocab = int(lm_head.shape[0])
    wp, wb = _ws(workspace)
    lp, lb = _ws(logits)
    tp, tb = _ws(lm_head_t)
    s = _lib.dflash_lm_head_ce_backward_saved(ctypes.byref(cfg), int(rows), lp, lb, _ptr(lm_head), tp, tb, vocab,
                                              _ptr(targets), _ptr(loss_mask), float(decay_tau), _ptr(row_ce),
                                              float(d_loss), _ptr(d_hidden), wp, wb, _stream(stream, lm_head))
    _check("dflash_lm_head_ce_backward_saved", s)


def dflash_lm_head_transpose_size(cfg: DFlashConfig, vocab: int) -> int:
    return _lib.dflash_lm_head_transpose_size(ctypes.byref(cfg), int(vocab))


def dflash_lm_head_transpose(cfg: DFlashConfig, lm_head, lm_head_t, stream=None) -> None:
    """lm_head [vocab, H] -> lm_head_t (a byte buffer of dflash_lm_head_transpose_size bytes): W_lm^T [H][vp]."""
    tp, tb = _ws(lm_head_t)
    s = _lib.dflash_lm_head_transpose(ctypes.byref(cfg), _ptr(lm_head), int(lm_head.shape[0]), tp, tb,
                                      _stream(stream, lm_head))
    _check("dflash_lm_head_transpose", s)


def dflash_lm_head_ce_backward_workspace_size(cfg: DFlashConfig, rows: int, vocab: int) -> int:
    return _lib.dflash_lm_head_ce_backward_workspace_size(ctypes.byref(cfg), int(rows), int(vocab))


def dflash_lm_head_ce_backward(cfg: DFlashConfig, hidden, lm_head, targets, loss_mask, decay_tau: float, row_ce,
                               d_loss: float, d_hidden, workspace, stream=None, lm_head_t=None) -> None:
    """hidden [rows, H], lm_head [vocab, H] (config dtype), targets i32 / loss_mask u8 [rows], row_ce f32 [rows]
    from dflash_lm_head_ce -> d_hidden [rows, H] (config dtype); lm_head_t: an optional kept
    dflash_lm_head_transpose of the head."""
    rows, vocab = int(hidden.shape[0]), int(lm_head.shape[0])
    wp, wb = _ws(workspace)
    tp, tb = _ws(lm_head_t)
    s = _lib.dflash_lm_head_ce_backward(ctypes.byref(cfg), rows, _ptr(hidden), _ptr(lm_head), tp, tb, vocab,
                                        _ptr(targets), _ptr(loss_mask), float(decay_tau), _ptr(row_ce),
                                        float(d_loss), _ptr(d_hidden), wp, wb, _stream(stream, hidden))
    _check("dflash_lm_head_ce_backward", s)


def dflash_block_attn_backward_workspace_size(cfg: DFlashConfig, num_blocks: int) -> int:
    return _lib.dflash_block_attn_backward_workspace_size(ctypes.byref(cfg), int(num_blocks))


def dflash_block_attn_backward(cfg: DFlashConfig, num_blocks: int, q, k_blk, v_blk, ctx_k, ctx_v,
                               ctx_total: int, block_ctx_base, block_anchor, block_valid, out, d_out,
                               d_q, d_k_blk, d_v_blk, d_ctx_k, d_ctx_v, workspace, stream=None) -> None:
    wp, wb = _ws(workspace)
    s = _lib.dflash_block_attn_backward(ctypes.byref(cfg), int(num_blocks), _ptr(q), _ptr(k_blk), _ptr(v_blk),
                                        _ptr(ctx_k), _ptr(ctx_v), int(ctx_total), _ptr(block_ctx_base),
                                        _ptr(block_anchor), _ptr(block_valid), _ptr(out), _ptr(d_out), _ptr(d_q),
                                        _ptr(d_k_blk), _ptr(d_v_blk), _ptr(d_ctx_k), _ptr(d_ctx_v), wp, wb,
                                        _stream(stream, q))
    _check("dflash_block_attn_backward", s)


def dflash_ctx_proj_backward_workspace_size(cfg: DFlashConfig, num_rows: int) -> int:
    return _lib.dflash_ctx_proj_backward_workspace_size(ctypes.byref(cfg), int(num_rows))


def dflash_ctx_proj_backward(cfg: DFlashConfig, target_states, ts_row_stride: int, ts_layer_stride: int,
                             num_rows: int, positions, layers, d_ctx_k, d_ctx_v, ctx_total: int, row_offset: int,
                             d_w_proj, d_ctx_hidden, workspace, stream=None, ctx_hidden=None, d_wk=None,
                             d_wv=None) -> None:
    """With ctx_hidden (C from dflash_ctx_proj_train), the context path's share of each layer's
    Wk / Wv gradient is added into d_wk[l] / d_wv[l] (f32 [Hkv*D, H])."""
    lw = _layers(layers)
    gk, gv = _ptr_array(d_ctx_k), _ptr_array(d_ctx_v)
    dk = _ptr_array(d_wk) if d_wk is not None else None
    dv = _ptr_array(d_wv) if d_wv is not None else None
    wp, wb = _ws(workspace)
    s = _lib.dflash_ctx_proj_backward(ctypes.byref(cfg), _ptr(target_states), int(ts_row_stride),
                                      int(ts_layer_stride), int(num_rows), _ptr(positions), lw, gk, gv,
                                      int(ctx_total), int(row_offset), _ptr(d_w_proj), _ptr(d_ctx_hidden),
                                      _ptr(ctx_hidden), dk, dv, wp, wb, _stream(stream, d_w_proj))
    _check("dflash_ctx_proj_backward", s)


def dflash_body_train_reserve_size(cfg: DFlashConfig, num_blocks: int) -> int:
    return _lib.dflash_body_train_reserve_size(ctypes.byref(cfg), int(num_blocks))


def dflash_body_forward_train(cfg: DFlashConfig, num_blocks: int, block_embeds, layers, ctx_k: List,
                              ctx_v: List, ctx_total: int, block_ctx_base, block_anchor, block_valid, out,
                              reserve, workspace, stream=None) -> None:
    """reserve: a uint8 device tensor of dflash_body_train_reserve_size bytes (kept for the backward)."""
    lw = _layers(layers)
    ck, cv = _ptr_array(ctx_k), _ptr_array(ctx_v)
    rp, rb = _ws(reserve)
    wp, wb = _ws(workspace)
    s = _lib.dflash_body_forward_train(ctypes.byref(cfg), int(num_blocks), _ptr(block_embeds), lw, ck, cv,
                                       int(ctx_total), _ptr(block_ctx_base), _ptr(block_anchor),
                                       _ptr(block_valid), _ptr(out), rp, rb, wp, wb, _stream(stream, block_embeds))
    _check("dflash_body_forward_train", s)


def train_reserve_h(reserve, num_layers: int, rows: int, hidden: int):
    """The fp32 residual streams entering each layer, [num_layers, rows, hidden]: a
    view of the start of a training reserve space (the documented part of its layout)."""
    import torch
    return reserve[: num_layers * rows * hidden * 4].view(torch.float32).view(num_layers, rows, hidden)


def _grads(grads: Sequence[Dict[str, object]]):
    arr = (DFlashLayerGrads * len(grads))()
    for i, G in enumerate(grads):
        for f in _LAYER_FIELDS:
            setattr(arr[i], f, _ptr(G.get(f)))
    return arr


def dflash_body_backward_workspace_size(cfg: DFlashConfig, num_blocks: int) -> int:
    return _lib.dflash_body_backward_workspace_size(ctypes.byref(cfg), int(num_blocks))


def dflash_body_backward(cfg: DFlashConfig, num_blocks: int, reserve, layers, ctx_k: List, ctx_v: List,
                         ctx_total: int, block_ctx_base, block_anchor, block_valid, d_out, d_block_embeds,
                         grads: Sequence[Dict[str, object]], d_ctx_k: List, d_ctx_v: List, workspace,
                         stream=None) -> None:
    """grads: one dict per layer with an fp32 tensor per weight name (as the layers' dicts)."""
    lw = _layers(layers)
    ck, cv = _ptr_array(ctx_k), _ptr_array(ctx_v)
    gk, gv = _ptr_array(d_ctx_k), _ptr_array(d_ctx_v)
    rp, rb = _ws(reserve)
    wp, wb = _ws(workspace)
    s = _lib.dflash_body_backward(ctypes.byref(cfg), int(num_blocks), rp, rb, lw, ck, cv, int(ctx_total),
                                  _ptr(block_ctx_base), _ptr(block_anchor), _ptr(block_valid), _ptr(d_out),
                                  _ptr(d_block_embeds), _grads(grads), gk, gv, wp, wb, _stream(stream, d_out))
    _check("dflash_body_backward", s)


def dflash_profile_start(kernel, max_launches: int) -> None:
    """Time the next max_launches launches of one kernel (name or dflash_kernel id)."""
    kid = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check("dflash_profile_start", _lib.dflash_profile_start(kid, int(max_launches)))


def dflash_profile_stop(max_launches: int) -> List[float]:
    """Per-launch durations in milliseconds of the launches recorded since start."""
    buf = (ctypes.c_float * int(max_launches))()
    n = ctypes.c_int32(0)
    _check("dflash_profile_stop", _lib.dflash_profile_stop(buf, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def dflash_adamw_step(dtype: int, tensors, lr: float, beta1: float, beta2: float, eps: float,
                      weight_decay: float, step: int, stream=None) -> None:
    """tensors: sequence of dicts with f32 `grad`, `master`, `exp_avg`, `exp_avg_sq` of equal numel
    and an optional `weight` (the working copy, DFLASH_BF16 or DFLASH_F32 per dtype)."""
    arr = (DFlashAdamWTensor * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i].grad = _ptr(t["grad"])
        arr[i].master = _ptr(t["master"])
        arr[i].exp_avg = _ptr(t["exp_avg"])
        arr[i].exp_avg_sq = _ptr(t["exp_avg_sq"])
        arr[i].weight = _ptr(t.get("weight"))
        arr[i].numel = int(t["master"].numel())
    first = tensors[0]["master"] if len(tensors) else None
    s = _lib.dflash_adamw_step(int(dtype), len(tensors), ctypes.addressof(arr), float(lr), float(beta1),
                               float(beta2), float(eps), float(weight_decay), int(step), _stream(stream, first))
    _check("dflash_adamw_step", s)
