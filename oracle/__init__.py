"""fp64 CPU oracle for the DFlash draft-body forward -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The HIP library never calls it and shares no code with it.

Contents:
  plan.py  -- the seeded anchor plan (integer; bit-exact spec).
  body.py  -- context projection, dual-source block attention, the draft body,
              and a brute-force dense-mask attention used to pin the gathered form.
  verify.py -- greedy and speculative-sampling verification of a drafted block.
  loss.py  -- block LM head and positionally decayed cross-entropy, and its
              gradient with respect to the hidden rows (the head is frozen).
  backward.py -- gradients of the dual-source block attention, of the
              context path (dW_proj) and of the whole body (every layer
              weight, the block embeddings and the context caches).
  optim.py -- the AdamW step that follows the backward (the reading taken
              for the optimizer the pages leave unnamed).

Parity status of each function (what pins it is listed in tests/test_oracle_*.py):
  build_plan             pinned by invariants the pages fix (determinism, equal
                         sample id -> equal anchors, anchors from valid windows,
                         loss mask excludes the anchor and invalid positions) and
                         by brute-force top-N selection; SplitMix64's increment
                         is pinned by its golden-ratio definition, its
                         finaliser's shifts and multipliers are "parity
                         unpinned" (the pages print no known-answer vector).
  rms_norm, silu, rope   pinned by closed forms and identities.
  block_attention        pinned by the brute-force dense-mask attention and by
                         closed-form special cases.
  body_forward           pinned by composition of the above plus the pages'
                         invariants; whole-body values beyond that are
                         "parity unpinned" (the pages print no worked example).
  verify_greedy          pinned by the pages' worked example and by brute force
                         over all short blocks.
  verify_sample          pinned by the speculative-sampling guarantee (emitted
                         tokens are distributed as p, chi-square over many
                         draws) and by its closed-form special cases.
  lm_head_ce             pinned by closed forms (uniform logits, two-token
                         vocabulary, shift invariance, the two-row decayed mean,
                         the undecayed limit).
  lm_head_ce_backward    pinned by central differences of lm_head_ce's loss over
                         every hidden entry (rows that do not count included),
                         and by closed forms (a one-hot head, linearity in d_loss).
  block_attn_call_backward  pinned by central finite differences of the
                         forward oracle over every input component.
  ctx_proj_backward      pinned by central differences of the forward context
                         path (ctx_proj then ctx_kv) along random directions of
                         W_proj and of C, and entry by entry on a tiny case.
  ctx_kv_weight_grads    pinned by central differences of the context path
                         (ctx_proj then ctx_kv) over every entry of Wk and Wv,
                         and, with body_backward, by central differences of a
                         whole training step's loss (tests/test_oracle_train_chain.py).
  rms_norm_backward, swiglu_backward
                         pinned by central differences of rms_norm and of
                         SiLU(g) * up, entry by entry.
  layer_forward, body_forward_layers
                         pinned to body_forward (an independent loop) to
                         rounding.
  layer_backward, body_backward
                         pinned by central differences of body_forward over
                         every weight of every layer, the block embeddings and
                         both context caches of a two-layer case with invalid
                         rows and an empty block.
  adamw_step             pinned by closed forms: the first step's normalised
                         sign step, decay alone, a constant gradient under the
                         bias correction, two steps' rate-weighted gradients,
                         decay before the step.
"""
from .plan import splitmix64, build_plan, eligible_anchors, row_key, position_key
from .verify import (
    verify_greedy_block, verify_greedy, target_choices_from_logits, verify_sample_block, verify_sample,
    inverse_cdf_draw, residual_weights, accept_proposal,
)
from .loss import lm_head_ce, lm_head_ce_rows, lm_head_ce_backward, token_ce, logsumexp_rows, position_weights
from .backward import (
    block_attention_backward, block_attn_call_backward, ctx_grad_rows, ctx_hidden_grad, ctx_proj_backward,
    ctx_kv_weight_grads,
    rms_norm_backward, swiglu_backward, layer_forward, layer_backward, body_forward_layers, body_backward,
)
from .optim import adamw_step
from .body import (
    rms_norm, silu, rope, rope_inv_freq, ctx_proj, ctx_kv, block_attention,
    dense_mask_attention, block_attn_call, body_forward, body_forward_dense,
    concat_target_states,
)

__all__ = [
    "splitmix64", "build_plan", "eligible_anchors", "row_key", "position_key",
    "rms_norm", "silu", "rope", "rope_inv_freq", "ctx_proj", "ctx_kv", "block_attention",
    "dense_mask_attention", "block_attn_call", "body_forward", "body_forward_dense",
    "concat_target_states",
    "verify_greedy_block", "verify_greedy", "target_choices_from_logits", "verify_sample_block",
    "verify_sample", "inverse_cdf_draw", "residual_weights", "accept_proposal",
    "lm_head_ce", "lm_head_ce_rows", "lm_head_ce_backward", "token_ce", "logsumexp_rows", "position_weights",
    "block_attention_backward", "block_attn_call_backward", "ctx_grad_rows", "ctx_hidden_grad", "ctx_proj_backward",
    "ctx_kv_weight_grads",
    "rms_norm_backward", "swiglu_backward", "layer_forward", "layer_backward", "body_forward_layers",
    "body_backward", "adamw_step",
]
