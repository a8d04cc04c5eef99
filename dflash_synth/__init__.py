"""Seeded synthetic workloads for the DFlash draft-body forward.

This module only draws random numbers and fixes shapes. It holds none of the
method's arithmetic, so that both the HIP path and the fp64 oracle can consume
the same inputs without sharing any computation.

Workload shapes follow the DFlash pages:
  * angelspec "DFlash" concept page, section "Configuration": hidden 4096,
    5 draft layers, 5 target layers of 4096 concatenated.
  * NeMo RL "DFlash Draft Body", section "How It Works", steps 1-2: a block is
    one anchor plus gamma draft positions (block_size = 1 + gamma, default 16),
    the caller supplies one embedding per block position.

Recipe (all tensors i.i.d.):
  * target hidden states and block embeddings: N(0, 1);
  * matrices: N(0, 1/fan_in) with the Linear layout [out, in];
  * RMSNorm weights: 1 + 0.1 * N(0, 1);
  * draws are made in fp32 and rounded to the compute dtype (bf16: round to
    nearest even), so the bytes handed to the GPU and to the oracle agree.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    batch: int                 # rows of target sequence (training) / requests (inference)
    seq_len: int               # target sequence length (training)
    num_target_layers: int
    target_hidden: int
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    intermediate: int
    num_layers: int
    block_size: int
    anchors_per_row: int
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    inference: bool = False    # precomputed context K/V cache, one block per request
    min_prefix: int = 0        # inference: prefix length ~ U{min_prefix..max_prefix}
    max_prefix: int = 0
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def num_blocks(self) -> int:
        return self.batch if self.inference else self.batch * self.anchors_per_row

    @property
    def block_rows(self) -> int:
        return self.num_blocks * self.block_size


# The five workloads. Sizes not stated for a workload take the values of the
# full 5-layer body (intermediate 12288 = 3 x hidden); the tiny fp32 case keeps
# that 3 x hidden ratio (768).
WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", "f32", batch=1, seq_len=128, num_target_layers=2, target_hidden=256,
                   hidden=256, num_q_heads=4, num_kv_heads=2, head_dim=64, intermediate=768,
                   num_layers=1, block_size=8, anchors_per_row=4, seed=1001),
    "c2": Workload("c2", "bf16", batch=4, seq_len=2048, num_target_layers=5, target_hidden=4096,
                   hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128, intermediate=12288,
                   num_layers=1, block_size=16, anchors_per_row=16, seed=1002),
    "c3": Workload("c3", "bf16", batch=8, seq_len=4096, num_target_layers=5, target_hidden=4096,
                   hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128, intermediate=12288,
                   num_layers=5, block_size=16, anchors_per_row=32, seed=1003),
    "c4": Workload("c4", "bf16", batch=1, seq_len=32768, num_target_layers=5, target_hidden=4096,
                   hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128, intermediate=12288,
                   num_layers=5, block_size=16, anchors_per_row=512, seed=1004),
    "c5": Workload("c5", "bf16", batch=64, seq_len=0, num_target_layers=5, target_hidden=4096,
                   hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128, intermediate=12288,
                   num_layers=5, block_size=16, anchors_per_row=1, inference=True,
                   min_prefix=1024, max_prefix=16384, seed=1005),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (small parity cases)."""
    return dataclasses.replace(w, **changes)


class Rng:
    """One torch generator per (workload seed, tensor tag), on a chosen device."""

    def __init__(self, seed: int, device):
        self.seed = int(seed)
        self.device = torch.device(device)

    def _gen(self, tag: str) -> torch.Generator:
        h = 0
        for ch in tag:
            h = (h * 131 + ord(ch)) % (1 << 31)
        g = torch.Generator(device=self.device)
        g.manual_seed((self.seed * 1_000_003 + h) % (1 << 62))
        return g

    def normal(self, tag: str, shape, std: float = 1.0, mean: float = 0.0,
               dtype=torch.bfloat16) -> torch.Tensor:
        t = torch.empty(shape, dtype=torch.float32, device=self.device)
        t.normal_(mean=mean, std=std, generator=self._gen(tag))
        return t.to(dtype)

    def integers(self, tag: str, low: int, high_inclusive: int, shape) -> torch.Tensor:
        return torch.randint(low, high_inclusive + 1, shape, generator=self._gen(tag),
                             device=self.device, dtype=torch.int64)


def layer_weights(w: Workload, rng: Rng, l: int) -> Dict[str, torch.Tensor]:
    H, D, I = w.hidden, w.head_dim, w.intermediate
    dt = w.torch_dtype
    return {
        "attn_norm": rng.normal(f"L{l}.attn_norm", (H,), std=0.1, mean=1.0, dtype=dt),
        "wq": rng.normal(f"L{l}.wq", (w.num_q_heads * D, H), std=1 / math.sqrt(H), dtype=dt),
        "wk": rng.normal(f"L{l}.wk", (w.num_kv_heads * D, H), std=1 / math.sqrt(H), dtype=dt),
        "wv": rng.normal(f"L{l}.wv", (w.num_kv_heads * D, H), std=1 / math.sqrt(H), dtype=dt),
        "wo": rng.normal(f"L{l}.wo", (H, w.num_q_heads * D), std=1 / math.sqrt(w.num_q_heads * D),
                         dtype=dt),
        "mlp_norm": rng.normal(f"L{l}.mlp_norm", (H,), std=0.1, mean=1.0, dtype=dt),
        "w_gate": rng.normal(f"L{l}.w_gate", (I, H), std=1 / math.sqrt(H), dtype=dt),
        "w_up": rng.normal(f"L{l}.w_up", (I, H), std=1 / math.sqrt(H), dtype=dt),
        "w_down": rng.normal(f"L{l}.w_down", (H, I), std=1 / math.sqrt(I), dtype=dt),
    }


def make_training_inputs(w: Workload, device, plan_seed: int = 0, step: int = 0,
                         mask: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """Target hidden states (stacked per target layer), W_proj, draft layers,
    block embeddings and the plan inputs (mask, sample ids, step, seed)."""
    assert not w.inference
    rng = Rng(w.seed, device)
    T = w.batch * w.seq_len
    K = w.num_target_layers * w.target_hidden
    dt = w.torch_dtype
    states = rng.normal("target_states", (w.num_target_layers, T, w.target_hidden), dtype=dt)
    w_proj = rng.normal("w_proj", (w.hidden, K), std=1 / math.sqrt(K), dtype=dt)
    layers = [layer_weights(w, rng, l) for l in range(w.num_layers)]
    emb = rng.normal("block_embeds", (w.num_blocks * w.block_size, w.hidden), dtype=dt)
    if mask is None:
        mask = torch.ones((w.batch, w.seq_len), dtype=torch.uint8, device=device)
    sample_ids = torch.arange(w.batch, dtype=torch.int64, device=device)
    return dict(states=states, w_proj=w_proj, layers=layers, emb=emb, mask=mask,
                sample_ids=sample_ids, step=step, plan_seed=plan_seed)


def make_inference_inputs(w: Workload, device) -> Dict[str, object]:
    """Ragged per-request prefixes with precomputed per-layer context K/V caches
    (K [Hkv][total][D], V transposed [Hkv][D][total], requests packed back to
    back), one block of anchor + (block_size - 1) mask-token embeddings per request."""
    assert w.inference
    rng = Rng(w.seed, device)
    dt = w.torch_dtype
    lengths = rng.integers("prefix_len", w.min_prefix, w.max_prefix, (w.batch,))
    offsets = torch.zeros(w.batch + 1, dtype=torch.int64, device=device)
    offsets[1:] = torch.cumsum(lengths, 0)
    total = int(offsets[-1].item())
    ctx_k = [rng.normal(f"L{l}.ctx_k", (w.num_kv_heads, total, w.head_dim), dtype=dt)
             for l in range(w.num_layers)]
    ctx_v = [rng.normal(f"L{l}.ctx_v", (w.num_kv_heads, w.head_dim, total), dtype=dt)
             for l in range(w.num_layers)]
    layers = [layer_weights(w, rng, l) for l in range(w.num_layers)]
    anchor_emb = rng.normal("anchor_embeds", (w.batch, w.hidden), dtype=dt)
    mask_emb = rng.normal("mask_token_embed", (w.hidden,), dtype=dt)
    emb = mask_emb.expand(w.batch, w.block_size, w.hidden).clone()
    emb[:, 0, :] = anchor_emb
    emb = emb.reshape(w.batch * w.block_size, w.hidden).contiguous()
    return dict(lengths=lengths, offsets=offsets, total=total, ctx_k=ctx_k, ctx_v=ctx_v,
                layers=layers, emb=emb,
                block_ctx_base=offsets[:-1].clone(),
                block_anchor=lengths.to(torch.int32),
                block_valid=torch.ones(w.batch * w.block_size, dtype=torch.uint8, device=device))


def random_attention_inputs(rng: Rng, num_blocks: int, block_size: int, num_q_heads: int,
                            num_kv_heads: int, head_dim: int, ctx_total: int, dtype):
    """Free-standing q / block k / block v / context caches for the attention call
    (context K [Hkv][T][D], context V transposed [Hkv][D][T])."""
    R = num_blocks * block_size
    q = rng.normal("attn.q", (R, num_q_heads * head_dim), dtype=dtype)
    k = rng.normal("attn.k", (R, num_kv_heads * head_dim), dtype=dtype)
    v = rng.normal("attn.v", (R, num_kv_heads * head_dim), dtype=dtype)
    ck = rng.normal("attn.ctx_k", (num_kv_heads, ctx_total, head_dim), dtype=dtype)
    cv = rng.normal("attn.ctx_v", (num_kv_heads, head_dim, ctx_total), dtype=dtype)
    return q, k, v, ck, cv
