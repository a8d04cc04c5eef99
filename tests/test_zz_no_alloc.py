"""dflash_ctx_append_noalloc, the allocation-free context append (for callers
that cannot allocate device memory), against dflash_ctx_append on the same
inputs. Both run the same kernels; only where the projected rows C are staged
differs (a static per-device array instead of the caller's workspace), so the
caches must agree bit for bit. Calls follow one another on the same array,
each with fewer rows than the one before, the first exactly at the array's
limit, so rows left over from a larger call must not leak into a smaller one."""
import math

import pytest
import torch

import block_draft_model_build_amd as d
from dflash_synth import WORKLOADS, Rng, layer_weights, scaled
from tests.helpers import workspace

pytestmark = pytest.mark.gpu


def _append_both(w, rows_list, cap, seed):
    dev = "cuda"
    cfg = d.config_from_workload(w)
    rng = Rng(seed, dev)
    dt = w.torch_dtype
    K = w.num_target_layers * w.target_hidden
    w_proj = rng.normal("w_proj", (w.hidden, K), std=1 / math.sqrt(K), dtype=dt)
    layers = [layer_weights(w, rng, l) for l in range(w.num_layers)]
    Hkv, D = w.num_kv_heads, w.head_dim

    def caches():
        return ([torch.full((Hkv, cap, D), 7.0, dtype=dt, device=dev) for _ in range(w.num_layers)],
                [torch.full((Hkv, D, cap), 7.0, dtype=dt, device=dev) for _ in range(w.num_layers)])

    ck_a, cv_a = caches()
    ck_b, cv_b = caches()
    gen = torch.Generator(device=dev).manual_seed(seed)
    for i, rows in enumerate(rows_list):
        X = rng.normal(f"X{i}", (rows, K), dtype=dt)
        pos = torch.randint(0, 60000, (rows,), generator=gen, device=dev, dtype=torch.int32)
        # Distinct destinations; some below 0 (padding) and some past the cache (dropped).
        dst = (torch.randperm(cap + 64, generator=gen, device=dev)[:rows] - 32).to(torch.int64)
        ws = workspace(d, cfg, 0, rows, dev)
        d.dflash_ctx_append(cfg, X, K, w.target_hidden, rows, pos, dst, w_proj, layers, ck_a, cv_a, cap, ws)
        d.dflash_ctx_append_noalloc(cfg, X, K, w.target_hidden, rows, pos, dst, w_proj, layers, ck_b, cv_b, cap)
        torch.cuda.synchronize()
        written = ((dst >= 0) & (dst < cap)).sum().item()
        for l in range(w.num_layers):
            assert torch.equal(ck_a[l], ck_b[l]), f"call {i} ({rows} rows): K cache of layer {l} differs"
            assert torch.equal(cv_a[l], cv_b[l]), f"call {i} ({rows} rows): V cache of layer {l} differs"
            assert (ck_b[l] != 7.0).any(dim=2).sum().item() >= written      # rows were really written
        del X, ws


def test_noalloc_append_matches_workspace_append_bf16():
    # The 5-layer inference dimensions: the first call fills the static array
    # exactly (4096 rows x hidden 4096 x 2 bytes = 32 MiB), then 1024 and 300.
    w = WORKLOADS["c5"]
    limit = d.DFLASH_NOALLOC_SCRATCH_BYTES // (w.hidden * 2)
    _append_both(w, [limit, 1024, 300], cap=8192, seed=301)


def test_noalloc_append_matches_workspace_append_f32():
    w = scaled(WORKLOADS["c1"], num_layers=2, seed=302)
    _append_both(w, [777, 129, 5], cap=1000, seed=303)


def test_noalloc_append_rejects_inputs_past_the_scratch():
    w = WORKLOADS["c5"]
    cfg = d.config_from_workload(w)
    K = w.num_target_layers * w.target_hidden
    rows = d.DFLASH_NOALLOC_SCRATCH_BYTES // (w.hidden * 2) + 1
    dev = "cuda"
    X = torch.zeros((8, K), dtype=torch.bfloat16, device=dev)       # never read: refused first
    pos = torch.zeros(8, dtype=torch.int32, device=dev)
    dst = torch.zeros(8, dtype=torch.int64, device=dev)
    layers = [layer_weights(w, Rng(1, dev), l) for l in range(w.num_layers)]
    ck = [torch.zeros((8, 16, 128), dtype=torch.bfloat16, device=dev) for _ in range(w.num_layers)]
    cv = [torch.zeros((8, 128, 16), dtype=torch.bfloat16, device=dev) for _ in range(w.num_layers)]
    with pytest.raises(d.DFlashError) as e:
        d.dflash_ctx_append_noalloc(cfg, X, K, w.target_hidden, rows, pos, dst, layers[0]["wq"], layers, ck, cv, 16)
    assert e.value.status == d.DFLASH_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert all((t == 0).all() for t in ck + cv)
