"""dflash_block_attn_backward vs the oracle's attention backward (NeMo RL
"DFlash Draft Body", How It Works, step 3, and Scope: training runs the body
with an optimizer step). The oracle's backward is pinned by finite differences
of the oracle's forward.

The forward output handed to the backward is the oracle's forward output,
rounded to the config dtype (a training step stores that rounded output).

Tolerance: fp32 inputs use the forward's fp32 bar (rel-L2 1e-5, max-abs 1e-4).
With bf16 inputs the kernel rounds two operands once each: the stored forward
output o (inside rowsum(dO o)) and the rotated block keys it stages; every
other step is fp32. Each gradient element is then a sum of products with at
most two factors off by the bf16 unit 2^-9 each, so the error is a few units
relative to the gradients' scale: the forward's bf16 bar (rel-L2 1e-2,
max-abs 5e-2) holds it with room."""
import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle
from dflash_synth import WORKLOADS, Rng, random_attention_inputs, scaled
from tests.helpers import BF16_TOL, F32_TOL, compare, np64

pytestmark = pytest.mark.gpu


def _inputs(w, bases, anchors, valid, ctx_total, seed):
    dev = "cuda"
    nb, bs = len(anchors), w.block_size
    rng = Rng(seed, dev)
    q, k, v, ck, cv = random_attention_inputs(rng, nb, bs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                              ctx_total, w.torch_dtype)
    dout = rng.normal("attn.d_out", (nb * bs, w.num_q_heads * w.head_dim), dtype=w.torch_dtype)
    val = np.asarray(valid, np.uint8).reshape(-1)
    return q, k, v, ck, cv, dout, val


def _oracle_forward(w, q, k, v, ck, cv, bases, anchors, val):
    """Forward output of the oracle, block by block, rounded to the config dtype."""
    nb, bs = len(anchors), w.block_size
    out = np.zeros((nb * bs, w.num_q_heads * w.head_dim))
    ckd, cvd = np64(ck), np64(cv).transpose(0, 2, 1)
    for n in range(nb):
        rows = slice(n * bs, (n + 1) * bs)
        out[rows] = oracle.block_attn_call(np64(q[rows]), np64(k[rows]), np64(v[rows]), ckd, cvd,
                                           [bases[n]], [anchors[n]], val[rows], bs, w.num_q_heads,
                                           w.num_kv_heads, w.head_dim, w.rope_theta)
    return torch.from_numpy(out).to(w.torch_dtype).cuda()


def _gpu_backward(w, q, k, v, ck, cv, ctx_total, bases, anchors, val, out, dout):
    dev = "cuda"
    nb, bs = len(anchors), w.block_size
    cfg = d.config_from_workload(w)
    R, Hq, Hkv, D = nb * bs, w.num_q_heads, w.num_kv_heads, w.head_dim
    nan = float("nan")
    dq = torch.full((R, Hq * D), nan, dtype=torch.float32, device=dev)
    dk = torch.full((R, Hkv * D), nan, dtype=torch.float32, device=dev)
    dv = torch.full((R, Hkv * D), nan, dtype=torch.float32, device=dev)
    dck = torch.full((Hkv, ctx_total, D), nan, dtype=torch.float32, device=dev)
    dcv = torch.full((Hkv, D, ctx_total), nan, dtype=torch.float32, device=dev)
    ws = torch.empty(d.dflash_block_attn_backward_workspace_size(cfg, nb), dtype=torch.uint8, device=dev)
    base_t = torch.tensor(bases, dtype=torch.int64, device=dev)
    anc_t = torch.tensor(anchors, dtype=torch.int32, device=dev)
    val_t = torch.from_numpy(val).to(dev)
    d.dflash_block_attn_backward(cfg, nb, q, k, v, ck, cv, ctx_total, base_t, anc_t, val_t, out, dout,
                                 dq, dk, dv, dck, dcv, ws)
    torch.cuda.synchronize()
    return dq, dk, dv, dck, dcv


def _check_all(w, bases, anchors, valid, ctx_total, seed):
    q, k, v, ck, cv, dout, val = _inputs(w, bases, anchors, valid, ctx_total, seed)
    out = _oracle_forward(w, q, k, v, ck, cv, bases, anchors, val)
    got = _gpu_backward(w, q, k, v, ck, cv, ctx_total, bases, anchors, val, out, dout)
    ref = oracle.block_attn_call_backward(np64(q), np64(k), np64(v), np64(ck), np64(cv).transpose(0, 2, 1),
                                          bases, anchors, val, w.block_size, w.num_q_heads, w.num_kv_heads,
                                          w.head_dim, w.rope_theta, np64(dout))
    tol = F32_TOL if w.dtype == "f32" else BF16_TOL
    names = ["dq", "dk_blk", "dv_blk", "d_ctx_k", "d_ctx_v"]
    for name, g, r in zip(names, got[:4], ref[:4]):
        compare(g, r, tol, name)
    compare(got[4], ref[4].transpose(0, 2, 1), tol, "d_ctx_v")
    return got, ref


def test_tiny_fp32():
    w = WORKLOADS["c1"]
    valid = np.ones((5, 8), np.uint8)
    valid[3, 3:] = 0
    _check_all(w, [0] * 5, [21, 89, 0, 125, -1], valid, 128, seed=11)


def test_fp32_two_sequences_and_empty_blocks():
    w = WORKLOADS["c1"]
    S = 100
    anchors = [1, 99, -1, 50, 0, 37]
    bases = [0, 0, 0, S, S, S]
    valid = np.ones((6, 8), np.uint8)
    valid[1, 0] = 0
    valid[4, :] = 0
    got, _ = _check_all(w, bases, anchors, valid, 2 * S, seed=12)
    dq, dk, dv = got[:3]
    # The empty block (anchor -1) and the fully invalid block pass nothing back.
    for n in (2, 4):
        rows = slice(n * 8, (n + 1) * 8)
        assert (dq[rows] == 0).all()
    assert (dk[16:24] == 0).all() and (dv[16:24] == 0).all()


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 2), (8, 8)])
def test_bf16_ragged(hq, hkv):
    w = scaled(WORKLOADS["c2"], num_q_heads=hq, num_kv_heads=hkv, hidden=1024,
               block_size=16 if hq // hkv <= 4 else 8)
    S = 700
    anchors = [0, 1, 33, 128, 129, 698, -1, 511, 300]
    bases = [0, S, 0, S, 0, S, 0, S, 0]
    valid = np.ones((len(anchors), w.block_size), np.uint8)
    valid[5, 2:] = 0
    valid[2, 7] = 0
    _check_all(w, bases, anchors, valid, 2 * S + 37, seed=13)     # 37 trailing rows no block reads


@pytest.mark.parametrize("bs,hq,hkv", [(32, 4, 2), (64, 2, 2)])
def test_bf16_long_blocks(bs, hq, hkv):
    # Blocks longer than 16 rows (rotations past the tabulated rows) and than
    # 32 rows (the own keys span two key tiles).
    w = scaled(WORKLOADS["c2"], num_q_heads=hq, num_kv_heads=hkv, hidden=512, block_size=bs)
    T = 900
    anchors = [0, 5, 130, 700, -1, 836]
    valid = np.ones((len(anchors), bs), np.uint8)
    valid[2, bs // 2:] = 0
    _check_all(w, [0] * len(anchors), anchors, valid, T, seed=18 + bs)


def test_bf16_anchor_at_the_end_of_the_cache():
    # A block whose prefix ends exactly at the last cache row: its last 64-key
    # chunk reaches past the cache (element loads with clamped keys), and the
    # last context tile is ragged.
    w = scaled(WORKLOADS["c2"], num_q_heads=8, num_kv_heads=2, hidden=1024)
    T = 1000
    anchors = [1000, 999, 937, 64, 63]
    valid = np.ones((len(anchors), w.block_size), np.uint8)
    valid[0, 5:] = 0
    _check_all(w, [0] * len(anchors), anchors, valid, T, seed=17)


def test_bf16_no_blocks_zeroes_context_gradients():
    w = scaled(WORKLOADS["c2"], num_q_heads=8, num_kv_heads=2, hidden=1024)
    ctx_total = 300
    q, k, v, ck, cv, dout, val = _inputs(w, [], [], np.zeros((0,)), ctx_total, seed=14)
    got = _gpu_backward(w, q, k, v, ck, cv, ctx_total, [], [], val, q, dout)
    assert (got[3] == 0).all() and (got[4] == 0).all()


def _training_layout(w, seed):
    """Anchors as a training batch places them: anchors_per_row distinct random
    starts per sequence, each block reading the prefix of its own sequence."""
    g = np.random.default_rng(seed)
    bases, anchors = [], []
    for b in range(w.batch):
        a = np.sort(g.choice(np.arange(1, w.seq_len - w.block_size), w.anchors_per_row, replace=False))
        anchors += [int(x) for x in a]
        bases += [b * w.seq_len] * w.anchors_per_row
    return bases, anchors


def test_full_size_one_sequence_one_group_sampled():
    # The training shape (8 sequences of 4096, 32 blocks each, 32/8 heads); the
    # gradients of one sequence are checked for one KV group, whose heads are
    # independent of the others.
    w = WORKLOADS["c3"]
    bs, G, D = w.block_size, w.num_q_heads // w.num_kv_heads, w.head_dim
    bases, anchors = _training_layout(w, seed=15)
    nb, T = len(anchors), w.batch * w.seq_len
    valid = np.ones((nb, bs), np.uint8)
    valid[3, 9:] = 0
    q, k, v, ck, cv, dout, val = _inputs(w, bases, anchors, valid, T, seed=15)
    # The backward needs the forward output of every block; blocks outside the
    # checked sequence get an arbitrary stored output (their gradients are not
    # compared, and they read none of the checked sequence's rows).
    seq, g = 2, 5
    blk = list(range(seq * w.anchors_per_row, (seq + 1) * w.anchors_per_row))
    out = dout.clone()
    rows = torch.cat([torch.arange(n * bs, (n + 1) * bs) for n in blk]).cuda()
    sub = scaled(w, num_q_heads=G, num_kv_heads=1)
    qh = slice(g * G * D, (g + 1) * G * D)
    kh = slice(g * D, (g + 1) * D)
    lo, hi = seq * w.seq_len, (seq + 1) * w.seq_len
    q_s, k_s, v_s = q[rows][:, qh], k[rows][:, kh], v[rows][:, kh]
    ck_s, cv_s = ck[g:g + 1, lo:hi], cv[g:g + 1, :, lo:hi]
    a_s, b_s = [anchors[n] for n in blk], [0] * len(blk)
    val_s = val.reshape(nb, bs)[blk].reshape(-1)
    out_g = _oracle_forward(sub, q_s, k_s, v_s, ck_s, cv_s, b_s, a_s, val_s)
    out_full = out.clone()
    out_full[rows[:, None], torch.arange(qh.start, qh.stop, device="cuda")[None, :]] = out_g
    dq, dk, dv, dck, dcv = _gpu_backward(w, q, k, v, ck, cv, T, bases, anchors, val, out_full, dout)
    ref = oracle.block_attn_call_backward(np64(q_s), np64(k_s), np64(v_s), np64(ck_s),
                                          np64(cv_s).transpose(0, 2, 1), b_s, a_s, val_s, bs, G, 1, D,
                                          w.rope_theta, np64(dout[rows][:, qh]))
    compare(dq[rows][:, qh], ref[0], BF16_TOL, "dq")
    compare(dk[rows][:, kh], ref[1], BF16_TOL, "dk_blk")
    compare(dv[rows][:, kh], ref[2], BF16_TOL, "dv_blk")
    compare(dck[g, lo:hi], ref[3][0], BF16_TOL, "d_ctx_k")
    compare(dcv[g, :, lo:hi], ref[4][0].T, BF16_TOL, "d_ctx_v")
    # Rows past the last anchor of every sequence are read by no block.
    for b in range(w.batch):
        last = max(anchors[b * w.anchors_per_row:(b + 1) * w.anchors_per_row])
        assert (dck[:, b * w.seq_len + last:(b + 1) * w.seq_len] == 0).all()
    assert torch.isfinite(dq).all() and torch.isfinite(dck).all() and torch.isfinite(dcv).all()


def test_deterministic():
    w = scaled(WORKLOADS["c2"], num_q_heads=8, num_kv_heads=2, hidden=1024)
    bases, anchors = [0, 0, 0, 500], [100, 400, 499, 250]
    valid = np.ones((4, w.block_size), np.uint8)
    q, k, v, ck, cv, dout, val = _inputs(w, bases, anchors, valid, 1000, seed=16)
    out = _oracle_forward(w, q, k, v, ck, cv, bases, anchors, val)
    a = _gpu_backward(w, q, k, v, ck, cv, 1000, bases, anchors, val, out, dout)
    b = _gpu_backward(w, q, k, v, ck, cv, 1000, bases, anchors, val, out, dout)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
