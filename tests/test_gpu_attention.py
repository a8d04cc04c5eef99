"""dflash_block_attn vs the oracle's dual-source attention (NeMo RL "DFlash Draft
Body", How It Works, step 3; angelspec "DFlash", How it works, dual-source KV
context), from tiny fp32 cases to the long-context and ragged-cache shapes."""
import numpy as np
import pytest
import torch

import block_draft_model_build_amd as d
import oracle
from dflash_synth import WORKLOADS, Rng, random_attention_inputs, scaled
from tests.helpers import BF16_TOL, F32_TOL, compare, np64, workspace

pytestmark = pytest.mark.gpu


def _run(w, bases, anchors, valid, ctx_total, seed, check_blocks=None, tweak=None):
    dev = "cuda"
    nb, bs = len(anchors), w.block_size
    cfg = d.config_from_workload(w)
    rng = Rng(seed, dev)
    q, k, v, ck, cv = random_attention_inputs(rng, nb, bs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                              ctx_total, w.torch_dtype)
    if tweak is not None:
        tweak(q, k, v, ck, cv)
    base_t = torch.tensor(bases, dtype=torch.int64, device=dev)
    anc_t = torch.tensor(anchors, dtype=torch.int32, device=dev)
    val_t = torch.tensor(np.asarray(valid, np.uint8).reshape(-1), dtype=torch.uint8, device=dev)
    out = torch.full((nb * bs, w.num_q_heads * w.head_dim), float("nan"), dtype=w.torch_dtype, device=dev)
    ws = workspace(d, cfg, nb, 0, dev)
    d.dflash_block_attn(cfg, nb, q, k, v, ck, cv, ctx_total, base_t, anc_t, val_t, out, ws)
    torch.cuda.synchronize()
    blocks = list(range(nb)) if check_blocks is None else list(check_blocks)
    tol = F32_TOL if w.dtype == "f32" else BF16_TOL
    val = np.asarray(valid, np.uint8).reshape(nb, bs)
    for n in blocks:
        rows = slice(n * bs, (n + 1) * bs)
        a = int(anchors[n])
        b0 = int(bases[n])
        lo, hi = (b0, b0 + max(a, 0))
        ref = oracle.block_attn_call(np64(q[rows]), np64(k[rows]), np64(v[rows]), np64(ck[:, lo:hi]),
                                     np64(cv[:, :, lo:hi]).transpose(0, 2, 1), [0], [a], val[n], bs,
                                     w.num_q_heads,
                                     w.num_kv_heads, w.head_dim, w.rope_theta)
        got = out[rows]
        compare(got, ref, tol, f"block {n} (anchor {a})")
        zero_rows = (val[n] == 0) | (a < 0)
        if zero_rows.any():
            assert (got[torch.from_numpy(zero_rows).to(dev)].float() == 0).all()
    return out


def test_tiny_fp32():
    w = WORKLOADS["c1"]
    valid = np.ones((4, 8), np.uint8)
    valid[3, 3:] = 0
    _run(w, [0, 0, 0, 0], [21, 89, 95, 125], valid, 128, seed=1)


def test_fp32_edge_anchors():
    w = WORKLOADS["c1"]
    anchors = [0, 1, 127, -1, 64, 300]           # 300 exceeds the context: clamped to 128
    valid = np.ones((6, 8), np.uint8)
    valid[2, 1:] = 0
    _run(w, [0] * 6, anchors, valid, 128, seed=2, check_blocks=[0, 1, 2, 3, 4])


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 2), (8, 8)])
def test_bf16_ragged(hq, hkv):
    w = scaled(WORKLOADS["c2"], num_q_heads=hq, num_kv_heads=hkv, hidden=1024, block_size=16 if hq // hkv <= 4 else 8)
    S = 700
    anchors = [0, 1, 33, 128, 129, 698, -1, 511, 300]
    bases = [0, S, 0, S, 0, S, 0, S, 0]
    valid = np.ones((len(anchors), w.block_size), np.uint8)
    valid[5, 2:] = 0
    valid[2, 7] = 0
    _run(w, bases, anchors, valid, 2 * S, seed=3)


def test_bf16_split_prefixes():
    # Few blocks with long prefixes, each a group of its own: each prefix is split
    # over several work items that take interleaved 128-key tiles, merged by the
    # combine step. The last block's prefix ends 1 row before the end of the
    # caches, so one split's last tile is staged through registers.
    w = scaled(WORKLOADS["c2"], num_q_heads=8, num_kv_heads=2, hidden=1024)
    S = 6000
    _run(w, [0, S, 0, S], [5999, 3001, 700, 5999], np.ones((4, 16), np.uint8), 2 * S, seed=4)


def test_ragged_cache_requests():
    # Inference shape: 64 requests, prefixes 1024..16384 packed back to back.
    w = WORKLOADS["c5"]
    rng = np.random.default_rng(5)
    lens = rng.integers(1024, 16385, size=64)
    offs = np.concatenate([[0], np.cumsum(lens)])
    check = [0, 1, int(np.argmax(lens)), int(np.argmin(lens)), 63]
    _run(w, offs[:-1].tolist(), lens.tolist(), np.ones((64, 16), np.uint8), int(offs[-1]), seed=5,
         check_blocks=check)


def test_long_context_blocks():
    # Long-context shape: one 32768-row sequence, 512 anchors from the plan.
    w = WORKLOADS["c4"]
    S, N = 32768, 512
    anchors, _, valid, _, _ = oracle.build_plan(np.ones((1, S), np.uint8), [0], 0, 0, N, 16)
    a = anchors[0].tolist()
    check = [0, 1, 255, 510, 511]
    _run(w, [0] * N, a, valid[0], S, seed=6, check_blocks=check)


def _spikes(w, ctx_rows, own_rows, scale):
    """Every query gets +6 on the last rotary pair's first component (rotated by
    at most 0.02 rad at these positions), and the listed context keys / own keys
    become scale * e_i on that component: their scores, about
    6 * scale * log2(e) / sqrt(D) in log2 units, stand far above all others for
    every query column that can see them."""
    i = w.head_dim // 2 - 1
    D = w.head_dim

    def tweak(q, k, v, ck, cv):
        q.view(q.shape[0], -1, D)[:, :, i] += 6.0
        for t in ctx_rows:
            ck[:, t] = 0
            ck[:, t, i] = scale
        kk = k.view(k.shape[0], -1, D)
        for r in own_rows:
            kk[r] = 0
            kk[r, :, i] = scale
    return tweak


@pytest.mark.parametrize("scale", [100.0, 300.0])
def test_bf16_scores_far_above_first_keys(scale):
    # A few keys score 75 (scale 100) or 230 (scale 300) log2 units above the
    # rest, far past the first visible keys' maximum that the softmax keeps as
    # its reference; at 300, 2^(s - reference) is beyond fp32. Covers multi-block
    # groups (4 and 2 blocks), single-block groups, split prefixes, a spike
    # among a block's own keys, and blocks that never see a spike.
    w = scaled(WORKLOADS["c2"], num_q_heads=8, num_kv_heads=2, hidden=1024)
    S, bs = 6000, w.block_size
    bases = [0, 0, 0, 0, S, S, 0, S, S, S]
    anchors = [5999, 3001, 700, 130, 2999, 1000, 4000, 50, 2600, 1200]
    valid = np.ones((len(anchors), bs), np.uint8)
    valid[1, 9:] = 0
    tweak = _spikes(w, ctx_rows=[300, 2900, 5000, S + 1234, S + 2500],
                    own_rows=[3 * bs + 5, 7 * bs + 2], scale=scale)
    _run(w, bases, anchors, valid, 2 * S, seed=8, tweak=tweak)


@pytest.mark.parametrize("scale", [None, 100.0, 300.0])
def test_bf16_pipelined_tiles(scale):
    # Groups of 4 and 3 blocks of one 3000-row sequence (64 query columns per
    # block, one wave each): their prefixes are split into 256-key items, so
    # whole tiles run software-pipelined, including the first tile of later
    # splits (which sets the softmax reference), a group with an idle wave,
    # partial tiles after whole ones, and a last tile that crosses the end of
    # the caches (staged through registers after a pipelined tile). With a
    # spike at context row 1000, inside whole tiles of both groups, scores rise
    # 75 or 230 log2 units above the reference where no maximum is tracked, and
    # the row-sum guard must send those items to the second run.
    w = scaled(WORKLOADS["c2"], num_q_heads=8, num_kv_heads=2, hidden=1024)
    S, bs = 3000, w.block_size
    anchors = [2999, 2995, 2990, 2960, 1500, 1400, 1300]
    valid = np.ones((len(anchors), bs), np.uint8)
    valid[2, 11:] = 0
    tweak = None if scale is None else _spikes(w, ctx_rows=[1000], own_rows=[], scale=scale)
    _run(w, [0] * len(anchors), anchors, valid, S, seed=10, tweak=tweak)


def test_fp32_scores_far_above_first_keys():
    w = WORKLOADS["c1"]
    anchors = [100, 127, 20, 64]
    valid = np.ones((4, w.block_size), np.uint8)
    _run(w, [0] * 4, anchors, valid, 128, seed=9,
         tweak=_spikes(w, ctx_rows=[40, 90], own_rows=[2 * w.block_size + 1], scale=300.0))


@pytest.mark.parametrize("layout", ["two-block groups", "single-block groups"])
def test_deterministic_and_information_boundary(layout):
    # Two-block groups share their tiles; with the sequences alternating, every
    # block is a group of its own and its prefix is split into items that take
    # interleaved tiles.
    w = scaled(WORKLOADS["c2"], num_q_heads=8, num_kv_heads=2, hidden=1024)
    dev = "cuda"
    cfg = d.config_from_workload(w)
    S, nb, bs = 3000, 4, 16
    rng = Rng(7, dev)
    q, k, v, ck, cv = random_attention_inputs(rng, nb, bs, 8, 2, 128, 2 * S, torch.bfloat16)
    order = [0, 0, S, S] if layout == "two-block groups" else [0, S, 0, S]
    bases = torch.tensor(order, dtype=torch.int64, device=dev)
    anchors = torch.tensor([1500, 2999, 700, 2500], dtype=torch.int32, device=dev)
    valid = torch.ones(nb * bs, dtype=torch.uint8, device=dev)
    ws = workspace(d, cfg, nb, 0, dev)

    def run(q, k, v, ck, cv):
        out = torch.empty((nb * bs, 8 * 128), dtype=torch.bfloat16, device=dev)
        d.dflash_block_attn(cfg, nb, q, k, v, ck, cv, 2 * S, bases, anchors, valid, out, ws)
        torch.cuda.synchronize()
        return out

    ref = run(q, k, v, ck, cv)
    assert torch.equal(ref, run(q, k, v, ck, cv))
    ck2, cv2, k2, v2 = ck.clone(), cv.clone(), k.clone(), v.clone()
    ck2[:, 1500:S] += 3.0                # block 0 (base 0, anchor 1500) may not read these
    cv2[:, :, 1500:S] -= 2.0
    ck2[:, S:] = float("nan")            # another sequence
    cv2[:, :, S:] = float("nan")
    k2[bs:] = float("nan")               # other blocks
    v2[bs:] = float("nan")
    out = run(q, k2, v2, ck2, cv2)
    assert torch.equal(out[:bs], ref[:bs])


@pytest.mark.parametrize("bs,hq,hkv", [(1, 32, 8), (1, 8, 8), (32, 8, 4), (32, 4, 4), (4, 16, 2)])
def test_bf16_block_sizes(bs, hq, hkv):
    # The block size is a parameter (one anchor plus gamma draft positions;
    # NeMo RL "DFlash Draft Body", How It Works, step 2). Block size 1 is the
    # causal special case: each block is one query attending to its prefix and
    # itself. Block size 32 fills the 64 query columns with two query heads per
    # KV head (or one). Groups of several blocks of one sequence (shared tiles,
    # pipelined when they run whole), single-block groups whose prefixes are
    # split, anchors at 0, at tile edges and at the end of a sequence.
    w = scaled(WORKLOADS["c2"], num_q_heads=hq, num_kv_heads=hkv, hidden=hq * 128, block_size=bs)
    S = 3000
    anchors = [0, 1, 127, 128, 129, 1000, 2999, 2500, 2501, 2502, 300, 1777, 2990, 2991]
    bases = [0, 0, 0, 0, 0, 0, 0, S, S, S, 0, S, 0, 0]
    valid = np.ones((len(anchors), bs), np.uint8)
    if bs > 1:
        valid[6, bs // 2:] = 0
    _run(w, bases, anchors, valid, 2 * S, seed=11 + bs)
