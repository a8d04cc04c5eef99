/*
 * libdflash -- the DFlash draft-body forward pass on AMD Instinct MI355X (gfx950),
 * with the steps around it: context-cache append, verification, the draft loss
 * and a whole training step's backward.
 *
 * What the library computes is stated on three pages:
 *   [P1] angelspec documentation, "DFlash" (sections "How it works", "Configuration");
 *   [P2] NeMo RL design docs, "DFlash Draft Body" (section "How It Works", steps 1-4, "Scope");
 *   [P3] cooking-agi deep dive, "DFlash: drafting, verification, and speed"
 *        (sections "One DFlash generation cycle", "Why can't later correct guesses
 *        simply stay?", "Sampling with temperature is not argmax matching").
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are HIP device pointers; "host" pointers are read
 *     during the call only. The library never allocates device memory and never
 *     frees caller memory; scratch space comes from the caller's workspace (size:
 *     dflash_workspace_size and the per-call *_workspace_size functions), and a
 *     training step's forward activations live in a caller-owned reserve space
 *     (dflash_body_train_reserve_size). The one exception is the static scratch
 *     array of dflash_ctx_append_noalloc, held for the life of the process.
 *   - Asynchronous calls enqueue kernels on `hip_stream` (a hipStream_t; NULL is
 *     the null stream) and return before they finish. Every argument that can be
 *     checked on the host is checked before anything is enqueued: a call that
 *     returns an error has enqueued nothing. Kernel faults surface at the
 *     caller's next synchronisation. A failed launch returns DFLASH_ERR_HIP.
 *   - Matrices are row-major. Weights use the Linear layout [out, in]: y = x W^T.
 *   - dtype DFLASH_BF16: every tensor argument (activations, weights, caches and
 *     outputs) is bfloat16; arithmetic accumulates in fp32 and the residual
 *     stream of the body is fp32. dtype DFLASH_F32: every tensor is fp32.
 *   - Shape envelope (DFLASH_ERR_UNSUPPORTED outside it; dflash_check_config tests
 *     it): one head row is 256 bytes (head_dim 128 in bf16, 64 in fp32);
 *     block_size * (num_q_heads / num_kv_heads) <= 64; hidden a multiple of 128;
 *     intermediate a multiple of 64; (num_q_heads + 2*num_kv_heads)*head_dim a
 *     multiple of 128; target_hidden a multiple of 64 (bf16) or 32 (fp32);
 *     num_layers <= 16. num_q_heads must be a multiple of num_kv_heads
 *     (DFLASH_ERR_INVALID_ARG otherwise).
 *   - Every device pointer to a tensor must be 16-byte aligned; the workspace
 *     256-byte aligned.
 *   - Calls on one stream are ordered. Apart from the measurement hook
 *     (dflash_profile_start/stop) the library keeps no state between calls and
 *     may be called from several threads on different streams with different
 *     workspaces.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dflash_status {
    DFLASH_OK = 0,
    DFLASH_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent shape */
    DFLASH_ERR_UNSUPPORTED = 2,   /* valid, but outside the shapes the kernels implement */
    DFLASH_ERR_WORKSPACE = 3,     /* workspace missing, too small or misaligned */
    DFLASH_ERR_HIP = 4,           /* a HIP launch or runtime call failed */
    DFLASH_ERR_SCRATCH_LIMIT = 5  /* input larger than an allocation-free entry point's static scratch */
} dflash_status;

typedef enum dflash_dtype { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Draft-model dimensions ([P1] "Configuration": hidden_size, num_hidden_layers,
 * num_target_layers, target_hidden_size, rope_theta; [P1] "How it works":
 * block_size; [P2] step 2: a block is one anchor plus gamma = block_size - 1
 * draft positions). rms_eps is not on the pages; 1e-6 is the usual value. */
typedef struct dflash_config {
    int32_t hidden;             /* H: draft hidden size */
    int32_t num_q_heads;        /* Hq */
    int32_t num_kv_heads;       /* Hkv; query head h reads KV head h / (Hq/Hkv) */
    int32_t head_dim;           /* D */
    int32_t intermediate;       /* I: SwiGLU width */
    int32_t num_layers;         /* draft decoder layers */
    int32_t num_target_layers;  /* L_t: target layers concatenated as context */
    int32_t target_hidden;      /* H_t */
    int32_t block_size;         /* bs = 1 + gamma */
    int32_t dtype;              /* dflash_dtype */
    double rope_theta;
    float rms_eps;
} dflash_config;

/* One draft decoder layer's weights (device pointers, dtype of the config).
 * attn_norm, mlp_norm: [H]; wq: [Hq*D, H]; wk, wv: [Hkv*D, H]; wo: [H, Hq*D];
 * w_gate, w_up: [I, H]; w_down: [H, I]. */
typedef struct dflash_layer_weights {
    const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} dflash_layer_weights;

/*
 * dflash_build_plan -- choose anchors and the per-position masks on the device.
 * [P2] step 1: an anchor is a valid position; the same mask, sample ids,
 * optimizer step and seed give the same plan; rows with equal sample ids get
 * equal anchors; a row with no valid window contributes no draft loss.
 * [P2] step 2: block n of row b covers positions anchor + k, k = 0..bs-1.
 * [P2] step 4: loss_mask leaves out the anchor and invalid positions.
 * [P1] "How it works", anchor sampling: anchors are sampled across the sequence.
 *
 * The sampler (the pages fix its properties, not its form): with SplitMix64
 * mix(), row key = mix(mix(mix(seed) ^ sample_id) ^ step) (64-bit two's
 * complement), key(a) = mix(row key ^ a). Position a is eligible when
 * mask[a] and mask[a+1] are nonzero (0 <= a <= S-2). The min(N, #eligible)
 * eligible positions with the smallest (key, a) are the anchors, stored in
 * ascending order, padded with -1.
 *
 *   mask        device u8  [batch, seq_len]          (nonzero = valid)
 *   sample_ids  device i64 [batch]
 *   anchors     device i32 [batch, N]                (out; -1 = empty slot)
 *   positions   device i32 [batch, N, block_size]    (out; anchor + k, -1 for empty slots)
 *   valid       device u8  [batch, N, block_size]    (out; anchor+k < S and mask[anchor+k])
 *   loss_mask   device u8  [batch, N, block_size]    (out; valid and k >= 1)
 *   num_anchors device i32 [batch]                   (out)
 *   block_ctx_base device i64 [batch, N] or NULL     (out; b * seq_len, the first
 *               context row of each block's sequence when the context rows of the
 *               batch are stored back to back)
 * Errors: INVALID_ARG for negative sizes, block_size < 1 or a null required
 * pointer when batch*N > 0. Deterministic: outputs are a pure function of
 * (mask, sample_ids, step, seed, N, block_size).
 */
dflash_status dflash_build_plan(const uint8_t *mask, int32_t batch, int32_t seq_len,
                                const int64_t *sample_ids, int64_t step, uint64_t seed,
                                int32_t anchors_per_row, int32_t block_size,
                                int32_t *anchors, int32_t *positions, uint8_t *valid,
                                uint8_t *loss_mask, int32_t *num_anchors,
                                int64_t *block_ctx_base, void *hip_stream);

/*
 * dflash_ctx_proj -- project target hidden states into every draft layer's
 * context K/V cache. [P1] "How it works", dual-source KV context: the target's
 * multi-layer hidden states are projected (W_proj) into the attention key/value
 * space; [P1] "Configuration": the layers in target_layer_ids, concatenated in
 * that order; [P3] "One DFlash generation cycle": target features enter every
 * draft layer's K/V.
 *
 *   C = X W_proj^T                        X [num_rows, L_t*H_t], C [num_rows, H]
 *   ctx_k[l][g][row_offset + r][:] = RoPE((C Wk_l^T)[r, g*D:(g+1)*D], positions[r])
 *   ctx_v[l][g][:][row_offset + r] = (C Wv_l^T)[r, g*D:(g+1)*D]
 *
 *   target_states  device; element (r, k) of X is at
 *                  target_states[r*ts_row_stride + (k / H_t)*ts_layer_stride + k % H_t],
 *                  so both a concatenated [rows, L_t*H_t] buffer (row stride L_t*H_t,
 *                  layer stride H_t) and per-layer slabs [L_t, rows, H_t] (row stride
 *                  H_t, layer stride rows*H_t) are read in place. Strides are in
 *                  elements and must be multiples of 8 (bf16) / 4 (fp32).
 *   positions      device i32 [num_rows]: RoPE position of each row.
 *   w_proj         device [H, L_t*H_t]
 *   layers         host array [num_layers]; only wk and wv are read.
 *   ctx_k, ctx_v   host arrays [num_layers] of device caches: K head-major
 *                  [Hkv][ctx_total][D], V transposed [Hkv][D][ctx_total] (each head's
 *                  V is stored dimension by dimension, so attention reads V^T tiles
 *                  as plain rows); rows [row_offset, row_offset + num_rows) are written.
 * RoPE pairs dimension i with i + D/2 at angle position * rope_theta^(-2i/D).
 * Errors: INVALID_ARG when row_offset + num_rows > ctx_total or a pointer is null;
 * WORKSPACE when workspace_bytes < dflash_workspace_size(cfg, 0, num_rows).
 */
dflash_status dflash_ctx_proj(const dflash_config *cfg, const void *target_states,
                              int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                              const int32_t *positions, const void *w_proj,
                              const dflash_layer_weights *layers, void *const *ctx_k,
                              void *const *ctx_v, int64_t ctx_total, int64_t row_offset,
                              void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * dflash_ctx_proj_train -- dflash_ctx_proj that also keeps C = X W_proj^T for
 * the backward (the way dflash_body_forward_train keeps the body's
 * activations): the context path's share of the Wk / Wv gradients is G^T C
 * (dflash_ctx_proj_backward). Same caches, bit for bit.
 *
 *   ctx_hidden     device [num_rows, H] in the config dtype, 16-byte aligned,
 *                  caller-owned: written with C (row r = target row r)
 *   other arguments as dflash_ctx_proj (same workspace size).
 * Errors: as dflash_ctx_proj; INVALID_ARG also for a null or misaligned
 * ctx_hidden when num_rows > 0.
 */
dflash_status dflash_ctx_proj_train(const dflash_config *cfg, const void *target_states,
                                    int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                                    const int32_t *positions, const void *w_proj,
                                    const dflash_layer_weights *layers, void *const *ctx_k,
                                    void *const *ctx_v, int64_t ctx_total, int64_t row_offset,
                                    void *ctx_hidden, void *workspace, size_t workspace_bytes,
                                    void *hip_stream);

/*
 * dflash_ctx_append -- incremental form of dflash_ctx_proj for multi-cycle
 * drafting: newly verified target hidden states are projected exactly as in
 * dflash_ctx_proj and scattered into the caches at caller-chosen rows, so
 * requests packed in one cache can each grow by a different number of rows.
 * [P2] "How It Works" (the context is the target's states before the anchor);
 * [P3] "One DFlash generation cycle", cache rollback and alignment: only the
 * verified prefix may stay in the cache, and the draft's context must stay
 * aligned with the target's.
 *
 * Row r of X (same addressing as dflash_ctx_proj) goes to cache row dst_rows[r]:
 *   ctx_k[l][g][dst_rows[r]][:] = RoPE((C Wk_l^T)[r, g*D:(g+1)*D], positions[r])
 *   ctx_v[l][g][:][dst_rows[r]] = (C Wv_l^T)[r, g*D:(g+1)*D]
 * Each row's values do not depend on the other rows of the call, so appending a
 * prefix piece by piece gives the same bytes as one dflash_ctx_proj over it.
 *
 *   positions      device i32 [num_rows]: RoPE position of each row
 *   dst_rows       device i64 [num_rows]: cache row of each row; rows whose
 *                  destination lies outside [0, ctx_total) are not written
 *                  (negative values mark padding rows). Two rows of one call
 *                  must not share a destination.
 *   other arguments as dflash_ctx_proj (workspace: dflash_workspace_size(cfg, 0, num_rows)).
 * Errors: as dflash_ctx_proj; INVALID_ARG also for a null dst_rows.
 */
dflash_status dflash_ctx_append(const dflash_config *cfg, const void *target_states,
                                int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                                const int32_t *positions, const int64_t *dst_rows, const void *w_proj,
                                const dflash_layer_weights *layers, void *const *ctx_k,
                                void *const *ctx_v, int64_t ctx_total, void *workspace,
                                size_t workspace_bytes, void *hip_stream);

/*
 * dflash_ctx_append_noalloc -- dflash_ctx_append for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, semantics and results as
 * dflash_ctx_append, minus the workspace: the projected rows C live in a static
 * device array of DFLASH_NOALLOC_SCRATCH_BYTES (32 MiB) that each GPU the
 * library runs on holds until the process ends. Nothing is allocated or freed
 * by this call.
 *
 *   Limit: num_rows * hidden * element size <= 32 MiB, i.e. up to
 *   32 MiB / (hidden * 2) rows in bf16 (4096 rows at hidden 4096) and half that
 *   in fp32; larger calls return DFLASH_ERR_SCRATCH_LIMIT before anything is
 *   enqueued.
 *   Device: the array of the current device is used, so hip_stream must belong
 *   to the current device. Its address is looked up once per device, on that
 *   device's first call.
 *   Sharing: every call on one GPU uses the same array. C is fully rewritten by
 *   each call before it is read, so nothing carries over between calls, but two
 *   calls that overlap on one GPU (different streams, or different host threads
 *   without stream order between them) race on the array and give undefined
 *   results; serialise them.
 * Errors: as dflash_ctx_append (no WORKSPACE error); SCRATCH_LIMIT as above;
 * HIP when the scratch address cannot be obtained.
 */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dflash_status dflash_ctx_append_noalloc(const dflash_config *cfg, const void *target_states,
                                        int64_t ts_row_stride, int64_t ts_layer_stride,
                                        int64_t num_rows, const int32_t *positions,
                                        const int64_t *dst_rows, const void *w_proj,
                                        const dflash_layer_weights *layers, void *const *ctx_k,
                                        void *const *ctx_v, int64_t ctx_total, void *hip_stream);

/*
 * dflash_ctx_truncate -- roll per-request context lengths back after
 * verification ([P3] "One DFlash generation cycle", cache rollback: rows of
 * rejected positions must leave the context). Attention reads only the rows
 * before a block's anchor, so rolling back is a change of length; the rows
 * past the new length stay in memory unread and are overwritten by the next
 * dflash_ctx_append.
 *
 *   lengths[i] = min(lengths[i], max(keep[i], 0))      for 0 <= i < n
 *
 *   lengths        device i64 [n], updated in place (e.g. the requests' anchors)
 *   keep           device i64 [n]
 * Errors: INVALID_ARG for n < 0 or null pointers (n > 0).
 */
dflash_status dflash_ctx_truncate(int64_t *lengths, const int64_t *keep, int32_t n, void *hip_stream);

/*
 * dflash_block_attn -- one layer's dual-source block attention.
 * [P2] step 3: a block reads the target prefix before its anchor and all
 * positions of its own block, never another block; outputs are produced for
 * block positions only. [P1] "How it works": attended together with the draft
 * tokens' own K/V. [P3] "One DFlash generation cycle": a block must not read
 * target features that contain its future.
 *
 * For block n with anchor a = block_anchor[n] and base = block_ctx_base[n], query
 * row k (position a + k) of head h attends, with softmax(q k^T / sqrt(D)), to
 *   ctx K/V row base + j of KV head g, 0 <= j < a   (prefix, strictly before the anchor)
 *   k_blk/v_blk rows n*bs + k', k' = 0..bs-1        (its whole block, both directions)
 * where g = h / (Hq/Hkv). q and k_blk arrive un-rotated and are rotated at a + k.
 *
 *   q              device [nb*bs, Hq*D]
 *   k_blk, v_blk   device [nb*bs, Hkv*D]
 *   ctx_k          device [Hkv][ctx_total][D], already rotated at its positions
 *   ctx_v          device [Hkv][D][ctx_total] (transposed, as dflash_ctx_proj writes it)
 *   block_ctx_base device i64 [nb]; block_anchor device i32 [nb] (-1: empty block)
 *   block_valid    device u8 [nb*bs]
 *   out            device [nb*bs, Hq*D]; rows with block_valid == 0 and all rows of
 *                  empty blocks are written as exact zeros.
 * Anchors and bases are clamped on the device so that base + a <= ctx_total.
 * q, k_blk, v_blk, ctx_k and ctx_v are read, and out written, with vector
 * accesses: all must be 16-byte aligned.
 * Errors: INVALID_ARG for null pointers, misaligned arrays or nb < 0; WORKSPACE when
 * workspace_bytes < dflash_workspace_size(cfg, nb, 0).
 */
dflash_status dflash_block_attn(const dflash_config *cfg, int32_t num_blocks, const void *q,
                                const void *k_blk, const void *v_blk, const void *ctx_k,
                                const void *ctx_v, int64_t ctx_total,
                                const int64_t *block_ctx_base, const int32_t *block_anchor,
                                const uint8_t *block_valid, void *out, void *workspace,
                                size_t workspace_bytes, void *hip_stream);

/*
 * dflash_body_forward -- the draft body: all num_layers draft decoder layers over
 * the blocks. [P2] step 3: the body runs the block embeddings through the draft
 * decoder layers, each block reading the prefix before its anchor and its own
 * block; step 4: one hidden state per block position, zero for invalid
 * positions; "Scope": no vocabulary logits, no loss.
 *
 * Per layer l, with h the fp32 residual stream (h = block_embeds at the start):
 *   x = RMSNorm(h) * attn_norm;  q, k, v = x Wq^T, x Wk^T, x Wv^T
 *   h += DualSourceAttention(q, k, v, ctx_k[l], ctx_v[l]) Wo^T
 *   y = RMSNorm(h) * mlp_norm;   h += (SiLU(y Wg^T) * (y Wu^T)) Wd^T
 * The attention is dflash_block_attn's, except that no row's output is zeroed
 * for block_valid == 0: inside the body invalid rows evolve like the others and
 * take part in their block's attention in every layer (rows of empty blocks
 * get a zero attention output). out = h (cast to the config dtype) on valid
 * rows, exact zero on rows with block_valid == 0 and on every row of an empty
 * block (anchor -1).
 *
 *   block_embeds   device [nb*bs, H] (caller-supplied embedding per block position)
 *   layers         host array [num_layers]
 *   ctx_k, ctx_v   host arrays [num_layers] of device caches in dflash_ctx_proj's
 *                  layouts (K [Hkv][ctx_total][D], V [Hkv][D][ctx_total])
 *   out            device [nb*bs, H]
 * block_embeds, every layer weight and the caches are read with 16-byte
 * accesses and must be 16-byte aligned.
 * Errors: INVALID_ARG for null pointers, misaligned arrays or nb < 0; WORKSPACE
 * below dflash_workspace_size(cfg, nb, 0).
 */
dflash_status dflash_body_forward(const dflash_config *cfg, int32_t num_blocks,
                                  const void *block_embeds, const dflash_layer_weights *layers,
                                  void *const *ctx_k, void *const *ctx_v, int64_t ctx_total,
                                  const int64_t *block_ctx_base, const int32_t *block_anchor,
                                  const uint8_t *block_valid, void *out, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/* Kernels that dflash_profile_start can time. */
typedef enum dflash_kernel {
    DFLASH_KERNEL_PLAN = 0,          /* anchor plan */
    DFLASH_KERNEL_CTX_PROJ = 1,      /* GEMM C = X W_proj^T */
    DFLASH_KERNEL_CTX_KV = 2,        /* GEMM of every layer's context K/V (RoPE, scatter) */
    DFLASH_KERNEL_RMSNORM = 3,
    DFLASH_KERNEL_QKV = 4,           /* GEMM x [Wq;Wk;Wv]^T */
    DFLASH_KERNEL_ATTENTION = 5,     /* dual-source block attention (per split) */
    DFLASH_KERNEL_ATTN_COMBINE = 6,  /* merge of split prefixes */
    DFLASH_KERNEL_O_PROJ = 7,        /* GEMM + residual */
    DFLASH_KERNEL_GATE_UP = 8,       /* GEMM + SiLU(gate) * up */
    DFLASH_KERNEL_DOWN = 9,          /* GEMM + residual (+ masked output on the last layer) */
    DFLASH_KERNEL_VERIFY = 10,       /* dflash_verify_greedy / dflash_verify_sample (whole call) */
    DFLASH_KERNEL_LM_HEAD = 11,      /* GEMM h W_lm^T with per-group softmax statistics */
    DFLASH_KERNEL_LM_CE = 12,        /* per-row CE and the decayed loss */
    DFLASH_KERNEL_ATTN_BWD = 13,     /* dflash_block_attn_backward (both kernels) */
    DFLASH_KERNEL_CTX_BWD_PACK = 14, /* dflash_ctx_proj_backward: gradient packing and transposes */
    DFLASH_KERNEL_CTX_BWD_DC = 15,   /* GEMM dC = G [Wk; Wv] */
    DFLASH_KERNEL_CTX_BWD_DW = 16,   /* GEMM dW_proj = dC^T X */
    DFLASH_KERNEL_BWD_PACK = 17,     /* dflash_body_backward: transposes, casts, gradient mask */
    DFLASH_KERNEL_BWD_DATA = 18,     /* GEMMs of the activation gradients (du, dy, do, dx) */
    DFLASH_KERNEL_BWD_WEIGHT = 19,   /* GEMMs of the weight gradients (contraction over rows) */
    DFLASH_KERNEL_BWD_NORM = 20,     /* RMSNorm backward and its weight-gradient column sums */
    DFLASH_KERNEL_LM_BWD_PREP = 21,  /* dflash_lm_head_ce_backward(_saved): row statistics, LM head transpose */
    DFLASH_KERNEL_LM_BWD_DZ = 22,    /* dz: GEMM of the logits with the CE gradient epilogue, or (_saved)
                                        the elementwise pass over the kept logits */
    DFLASH_KERNEL_LM_BWD_DH = 23,    /* GEMM d_hidden = dz W_lm */
    DFLASH_KERNEL_CTX_BWD_DKV = 24,  /* dflash_ctx_proj_backward: GEMM d[Wk; Wv] += G^T C */
    DFLASH_KERNEL_COUNT = 25
} dflash_kernel;

/*
 * Measurement hook (for benchmarks). dflash_profile_start makes the library
 * bracket each of the next max_launches launches of `kernel` with a pair of
 * hipEvents recorded on the launch's stream (events created here, on the
 * current device). dflash_profile_stop waits for those events, writes each
 * launch's duration in milliseconds to elapsed_ms[0 .. *launches-1] (host array
 * of max_launches floats) and uninstalls the hook. Process-wide and not
 * thread-safe: install it only around single-threaded measurement.
 * Errors: INVALID_ARG for an unknown kernel or max_launches < 1, or a stop without
 * a start; HIP when creating, recording or reading events fails.
 */
dflash_status dflash_profile_start(int32_t kernel, int32_t max_launches);
dflash_status dflash_profile_stop(float *elapsed_ms, int32_t *launches);

/*
 * dflash_verify_greedy -- greedy verification of a batch of drafted blocks.
 * [P3] "Why can't later correct guesses simply stay?": only a continuous
 * accepted prefix survives; at the first proposal that differs from the
 * target's choice the target's choice is emitted instead and the block ends;
 * if all proposals agree, the target's choice after the block (the bonus) is
 * emitted too; an accepted end-of-sequence token ends the block with nothing
 * after it. Worked example there: draft [10, 20, 99, 40] against choices
 * [10, 20, 30, 40, 50] emits [10, 20, 30] with 2 accepted.
 *
 * The target's choice at position i is the argmax over the vocabulary of
 * target_logits[b][i] (equal maxima: the smallest token id; logits must be
 * finite). Position gamma is the bonus position.
 *
 *   draft          device i32 [batch][gamma]
 *   target_logits  device [batch][gamma + 1][vocab], logits_dtype DFLASH_BF16 or DFLASH_F32
 *   eos_token      end-of-sequence id, or -1 for none
 *   emitted        device i32 [batch][gamma + 1]: emitted tokens, then -1
 *   num_emitted    device i32 [batch]; accepted: device i32 [batch] (kept proposals)
 * Errors: INVALID_ARG for negative sizes, vocab < 1, an unknown dtype or null
 * pointers; UNSUPPORTED when batch*(gamma + 1) exceeds INT32_MAX.
 */
dflash_status dflash_verify_greedy(const int32_t *draft, const void *target_logits, int32_t logits_dtype,
                                   int32_t batch, int32_t gamma, int32_t vocab, int32_t eos_token,
                                   int32_t *emitted, int32_t *num_emitted, int32_t *accepted,
                                   void *hip_stream);

/*
 * dflash_verify_sample -- speculative-sampling verification of a batch of
 * drafted blocks. [P3] "Sampling with temperature is not argmax matching": a
 * proposal y drawn from the proposal distribution q is accepted with
 * probability min(1, p(y)/q(y)) under the target distribution p; at the first
 * rejection a replacement is drawn from [p - q]_+ renormalised, and the block
 * ends. If every proposal is accepted, a bonus token is drawn from p at the
 * position after the block. An accepted end-of-sequence token ends the block.
 *
 * The random numbers are inputs. Proposal i is accepted iff
 * fp32(u_accept[b][i] * q[b][i][y]) < p[b][i][y] (a proposal outside the
 * vocabulary is rejected). The block's one draw takes the smallest token t
 * whose running fp64 sum of weights exceeds u_draw[b] times their total; if
 * [p - q]_+ sums to zero the replacement is drawn from p.
 *
 *   draft          device i32 [batch][gamma]
 *   p              device f32 [batch][gamma + 1][vocab] target probabilities
 *   q              device f32 [batch][gamma][vocab] proposal probabilities
 *   u_accept       device f32 [batch][gamma] in [0, 1); u_draw: device f32 [batch] in [0, 1)
 *   eos_token, emitted, num_emitted, accepted: as dflash_verify_greedy
 * Errors: INVALID_ARG for negative sizes, vocab < 1 or null pointers;
 * UNSUPPORTED when (gamma + 1)*vocab exceeds INT32_MAX.
 */
dflash_status dflash_verify_sample(const int32_t *draft, const float *p, const float *q,
                                   const float *u_accept, const float *u_draw, int32_t batch,
                                   int32_t gamma, int32_t vocab, int32_t eos_token, int32_t *emitted,
                                   int32_t *num_emitted, int32_t *accepted, void *hip_stream);

/*
 * dflash_lm_head_ce -- the draft's training loss over block rows: logits of
 * the (frozen, target-provided) LM head and cross-entropy against the
 * ground-truth tokens with an exponential positional decay. [P1] "How it
 * works", Loss: cross-entropy whose positional decay weights earlier
 * in-block positions more; [P1] "Configuration": embedding and lm_head come
 * from the target model; [P2] step 4: the loss mask excludes the anchor and
 * invalid positions.
 *
 *   z_r      = hidden[r] W_lm^T                 (fp32 accumulation; not stored here)
 *   CE_r     = logsumexp(z_r) - z_r[targets[r]]
 *   w_r      = exp(-(k - 1) / decay_tau),  k = r mod block_size   (k = 1: weight 1)
 *   loss     = sum(m_r w_r CE_r) / sum(m_r w_r), m_r = loss_mask[r]; 0 if no row counts
 *
 *   rows           block rows (normally num_blocks * block_size)
 *   hidden         device [rows, hidden] (e.g. dflash_body_forward's output)
 *   lm_head        device [vocab, hidden], Linear layout; any vocab >= 1
 *   targets        device i32 [rows]; a target outside [0, vocab) excludes its row
 *   loss_mask      device u8 [rows]
 *   decay_tau      > 0 (the pages give no value)
 *   row_ce         device f32 [rows]: CE_r, 0 for excluded rows
 *   loss           device f64 scalar
 *   workspace      dflash_lm_head_ce_workspace_size(rows, vocab) bytes, 256-byte aligned
 * Errors: as dflash_ctx_proj for the config; INVALID_ARG for rows < 0, vocab < 1,
 * decay_tau <= 0 or null pointers; WORKSPACE for a small or misaligned workspace.
 */
dflash_status dflash_lm_head_ce(const dflash_config *cfg, int32_t rows, const void *hidden,
                                const void *lm_head, int32_t vocab, const int32_t *targets,
                                const uint8_t *loss_mask, double decay_tau, float *row_ce,
                                double *loss, void *workspace, size_t workspace_bytes,
                                void *hip_stream);
size_t dflash_lm_head_ce_workspace_size(int32_t rows, int32_t vocab);

/*
 * dflash_lm_head_ce_train -- dflash_lm_head_ce that also keeps the fp32 logits
 * z for the backward (dflash_lm_head_ce_backward_saved), the way a training
 * forward keeps its activations, so that the gradient does not recompute the
 * product with the LM head. Same loss as dflash_lm_head_ce ([P1] "How it
 * works", Loss); row_ce and loss are bit-identical to its outputs.
 *
 *   logits        device f32 [rows][ldl], ldl = vocab rounded up to a multiple of
 *                 64; z_r[v] at logits[r * ldl + v] for v < vocab (columns past
 *                 the vocabulary are not written). 16-byte aligned, caller-owned,
 *                 logits_bytes >= dflash_lm_head_ce_logits_size(rows, vocab).
 *   other arguments as dflash_lm_head_ce (same workspace size).
 * Errors: as dflash_lm_head_ce; INVALID_ARG also for a null, small or
 * misaligned logits buffer when rows > 0.
 */
dflash_status dflash_lm_head_ce_train(const dflash_config *cfg, int32_t rows, const void *hidden,
                                      const void *lm_head, int32_t vocab, const int32_t *targets,
                                      const uint8_t *loss_mask, double decay_tau, float *row_ce, double *loss,
                                      float *logits, size_t logits_bytes, void *workspace,
                                      size_t workspace_bytes, void *hip_stream);
/* rows * ldl * 4 bytes (0 for invalid sizes). */
size_t dflash_lm_head_ce_logits_size(int32_t rows, int32_t vocab);

/*
 * dflash_lm_head_ce_backward -- gradient of dflash_lm_head_ce's loss with
 * respect to the hidden rows: the d_out that dflash_body_backward takes.
 * [P1] "Configuration": the LM head comes from the target model and stays
 * frozen, so it has no gradient here; [P1] "How it works", Loss: the decayed
 * cross-entropy being differentiated.
 *
 * With D = sum(m_r w_r) over the rows that count (loss_mask set, target inside
 * the vocabulary), c_r = d_loss m_r w_r / D (0 for the others) and
 * p_r = softmax(z_r), z_r = hidden[r] W_lm^T:
 *   dz_r        = c_r (p_r - onehot(targets[r]))
 *   d_hidden[r] = dz_r W_lm
 * The softmax uses logsumexp(z_r) = row_ce[r] + z_r[targets[r]], the second
 * term recomputed as a dot product.
 *
 *   hidden, lm_head, vocab, targets, loss_mask, decay_tau, rows
 *                  as dflash_lm_head_ce
 *   lm_head_t, lm_head_t_bytes
 *                  optional: dflash_lm_head_transpose's output for this head (the
 *                  call then skips its own transpose); NULL: the head is
 *                  transposed into the workspace. The result is the same bit for bit.
 *   row_ce         device f32 [rows]: dflash_lm_head_ce's output for the same inputs
 *   d_loss         the upstream gradient of the loss (1 for the loss itself)
 *   d_hidden       device [rows, hidden] in the config dtype, overwritten (rows
 *                  that do not count get exact zeros)
 *   workspace      dflash_lm_head_ce_backward_workspace_size(cfg, rows, vocab)
 *                  bytes, 256-byte aligned
 * dz enters the second product in the config dtype; both products accumulate
 * in fp32. Errors: as dflash_lm_head_ce (INVALID_ARG also for a null row_ce or
 * d_hidden when rows > 0, or a small or misaligned lm_head_t).
 */
dflash_status dflash_lm_head_ce_backward(const dflash_config *cfg, int32_t rows, const void *hidden,
                                         const void *lm_head, const void *lm_head_t, size_t lm_head_t_bytes,
                                         int32_t vocab, const int32_t *targets, const uint8_t *loss_mask,
                                         double decay_tau, const float *row_ce, double d_loss, void *d_hidden,
                                         void *workspace, size_t workspace_bytes, void *hip_stream);
size_t dflash_lm_head_ce_backward_workspace_size(const dflash_config *cfg, int32_t rows, int32_t vocab);

/*
 * dflash_lm_head_transpose -- W_lm^T, the head as the loss backward's second
 * product reads it. [P1] "Configuration": the LM head comes from the target
 * and stays frozen, so a training run can form its transpose once and pass it
 * to every backward call (lm_head_t) instead of having each call transpose it.
 *
 *   lm_head        device [vocab, hidden] in the config dtype
 *   lm_head_t      device [hidden][vp] in the config dtype, vp = vocab rounded
 *                  up to a multiple of 64; columns >= vocab are written as zero.
 *                  16-byte aligned, caller-owned,
 *                  lm_head_t_bytes >= dflash_lm_head_transpose_size(cfg, vocab)
 * Errors: as dflash_lm_head_ce for the config and the vocabulary; INVALID_ARG
 * for a null or misaligned lm_head, or a null, small or misaligned lm_head_t.
 */
dflash_status dflash_lm_head_transpose(const dflash_config *cfg, const void *lm_head, int32_t vocab,
                                       void *lm_head_t, size_t lm_head_t_bytes, void *hip_stream);
/* hidden * vp * element size bytes (0 for invalid sizes). */
size_t dflash_lm_head_transpose_size(const dflash_config *cfg, int32_t vocab);

/*
 * dflash_lm_head_ce_backward_saved -- dflash_lm_head_ce_backward from the
 * logits dflash_lm_head_ce_train kept for the same rows, targets and mask:
 * lse_r = row_ce[r] + logits[r][targets[r]], dz_r = c_r (softmax(z_r) -
 * onehot) in one elementwise pass over the logits, d_hidden = dz W_lm. The
 * hidden rows are not read. Same arithmetic as dflash_lm_head_ce_backward per
 * element of dz, except that the target logit in lse is the forward's own value
 * rather than a recomputed dot product; the same workspace size.
 *
 *   logits, logits_bytes   as dflash_lm_head_ce_train wrote them
 *   other arguments        as dflash_lm_head_ce_backward
 * Errors: as dflash_lm_head_ce_backward; INVALID_ARG also for a null, small or
 * misaligned logits buffer when rows > 0.
 */
dflash_status dflash_lm_head_ce_backward_saved(const dflash_config *cfg, int32_t rows, const float *logits,
                                               size_t logits_bytes, const void *lm_head, const void *lm_head_t,
                                               size_t lm_head_t_bytes, int32_t vocab, const int32_t *targets,
                                               const uint8_t *loss_mask, double decay_tau, const float *row_ce,
                                               double d_loss, void *d_hidden, void *workspace,
                                               size_t workspace_bytes, void *hip_stream);

/*
 * dflash_block_attn_backward -- gradients of dflash_block_attn. [P2] "How It
 * Works", step 3 (the dual-source visibility the forward implements) and
 * "Scope" (training runs the body with an optimizer step).
 *
 * Given the forward's inputs, its output `out` and the gradient d_out of that
 * output, writes the gradients with respect to q, k_blk, v_blk (before RoPE,
 * as dflash_block_attn takes them), the context K cache (in the rotated frame
 * it stores) and the context V cache (transposed like it). Rows whose forward
 * output is zero (block_valid == 0, empty blocks) pass no gradient back; their
 * k and v rows still receive the gradients of the other rows that read them.
 * Context rows no block reads get zero.
 *
 *   q, k_blk, v_blk, ctx_k, ctx_v, ctx_total, block_ctx_base, block_anchor,
 *   block_valid     as dflash_block_attn
 *   out, d_out      device [nb*bs, Hq*D] in the config dtype
 *   d_q             device f32 [nb*bs, Hq*D]; d_k_blk, d_v_blk: device f32 [nb*bs, Hkv*D]
 *   d_ctx_k         device f32 [Hkv][ctx_total][D]; d_ctx_v: device f32 [Hkv][D][ctx_total]
 *   workspace       dflash_block_attn_backward_workspace_size(cfg, nb) bytes, 256-byte aligned
 * Every output element is written (no accumulation into the caller's buffers);
 * results are deterministic. All arrays are 16-byte aligned. Errors: as
 * dflash_block_attn; INVALID_ARG also for a misaligned array.
 */
dflash_status dflash_block_attn_backward(const dflash_config *cfg, int32_t num_blocks, const void *q,
                                         const void *k_blk, const void *v_blk, const void *ctx_k,
                                         const void *ctx_v, int64_t ctx_total,
                                         const int64_t *block_ctx_base, const int32_t *block_anchor,
                                         const uint8_t *block_valid, const void *out, const void *d_out,
                                         float *d_q, float *d_k_blk, float *d_v_blk, float *d_ctx_k,
                                         float *d_ctx_v, void *workspace, size_t workspace_bytes,
                                         void *hip_stream);
size_t dflash_block_attn_backward_workspace_size(const dflash_config *cfg, int32_t num_blocks);

/*
 * dflash_ctx_proj_backward -- gradient of the projection W_proj through the
 * context path. [P2] "Scope": training updates the body's weights with an
 * optimizer step, W_proj among them; [P1] "How it works", dual-source KV
 * context: the target states reach every layer's K/V through W_proj.
 *
 * With the forward of dflash_ctx_proj (C = X W_proj^T, Kc_l = RoPE(C Wk_l^T),
 * Vc_l = C Wv_l^T) and the gradients of every layer's cache rows
 * [row_offset, row_offset + num_rows):
 *   Gk_l[r] = RoPE^T(d_ctx_k[l][g][row_offset + r][:], positions[r])   per head g
 *   Gv_l[r] = d_ctx_v[l][g][:][row_offset + r]                          per head g
 *   dC      = sum_l Gk_l Wk_l + Gv_l Wv_l                               [num_rows, H]
 *   d_w_proj = dC^T X                                                   [H, L_t*H_t]
 * RoPE^T is the rotation by the opposite angle.
 *
 *   target_states, ts_row_stride, ts_layer_stride, positions, layers
 *                  as dflash_ctx_proj (only wk and wv of the layers are read)
 *   d_ctx_k, d_ctx_v  host arrays [num_layers] of device f32 gradients in the
 *                  caches' layouts: K [Hkv][ctx_total][D] (rotated frame, as
 *                  dflash_block_attn_backward writes it), V [Hkv][D][ctx_total];
 *                  16-byte aligned
 *   d_w_proj       device f32 [H, L_t*H_t], overwritten (zero when num_rows == 0)
 *   d_ctx_hidden   optional device f32 [num_rows, H]: dC (NULL: not written)
 *   ctx_hidden     optional device [num_rows, H] in the config dtype: C of these rows,
 *                  as dflash_ctx_proj_train kept it. With it, the context path's share
 *                  of every layer's Wk and Wv gradient is ADDED to d_wk[l], d_wv[l]:
 *                    d_wk[l] += Gk_l^T C,   d_wv[l] += Gv_l^T C        [Hkv*D, H]
 *                  ([P1] "How it works": the projected context enters each layer's
 *                  K/V through that layer's own projections; dflash_body_backward
 *                  writes the block rows' share first). NULL: not computed.
 *   d_wk, d_wv     host arrays [num_layers] of device f32 [Hkv*D, H] (16-byte
 *                  aligned), required with ctx_hidden, else ignored; left as they
 *                  are when num_rows == 0 (the share is zero)
 *   workspace      dflash_ctx_proj_backward_workspace_size(cfg, num_rows) bytes,
 *                  256-byte aligned
 * G, dC and C enter their products in the config dtype; the products accumulate
 * in fp32. Errors: INVALID_ARG as dflash_ctx_proj, for a null d_w_proj, or, with
 * ctx_hidden, for a misaligned ctx_hidden or a null or misaligned d_wk / d_wv
 * entry; UNSUPPORTED when L_t*H_t is not a multiple of 128; WORKSPACE when the
 * workspace is missing, small or misaligned.
 */
dflash_status dflash_ctx_proj_backward(const dflash_config *cfg, const void *target_states,
                                       int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                                       const int32_t *positions, const dflash_layer_weights *layers,
                                       const float *const *d_ctx_k, const float *const *d_ctx_v,
                                       int64_t ctx_total, int64_t row_offset, float *d_w_proj,
                                       float *d_ctx_hidden, const void *ctx_hidden, float *const *d_wk,
                                       float *const *d_wv, void *workspace, size_t workspace_bytes,
                                       void *hip_stream);
size_t dflash_ctx_proj_backward_workspace_size(const dflash_config *cfg, int64_t num_rows);

/*
 * dflash_body_forward_train -- dflash_body_forward for a training step: the same
 * arithmetic and the same `out` (bit for bit), and in addition every layer's
 * input residual stream and activations, kept in a reserve space that
 * dflash_body_backward reads.
 *
 *   reserve        device, dflash_body_train_reserve_size(cfg, nb) bytes, 256-byte
 *                  aligned; owned by the caller and left untouched until the
 *                  backward. It begins with h [num_layers][nb*bs, H] fp32, h[l] the
 *                  residual stream entering layer l (h[0] = block_embeds as fp32);
 *                  the rest holds, per layer, the normalised inputs, q/k/v, the
 *                  attention output, the residual after attention, the SwiGLU
 *                  pre-activations (fp32) and SiLU(g) * up, in an internal layout.
 * Other arguments, errors and workspace as dflash_body_forward; INVALID_ARG for a
 * null reserve, WORKSPACE for a small or misaligned one.
 */
dflash_status dflash_body_forward_train(const dflash_config *cfg, int32_t num_blocks,
                                        const void *block_embeds, const dflash_layer_weights *layers,
                                        void *const *ctx_k, void *const *ctx_v, int64_t ctx_total,
                                        const int64_t *block_ctx_base, const int32_t *block_anchor,
                                        const uint8_t *block_valid, void *out, void *reserve,
                                        size_t reserve_bytes, void *workspace, size_t workspace_bytes,
                                        void *hip_stream);
/* Bytes of a training step's reserve space for num_blocks blocks (0 for an
 * invalid config). */
size_t dflash_body_train_reserve_size(const dflash_config *cfg, int32_t num_blocks);

/* Gradients of one draft layer's weights (device f32, the shapes of
 * dflash_layer_weights). */
typedef struct dflash_layer_grads {
    float *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} dflash_layer_grads;

/*
 * dflash_body_backward -- gradients of dflash_body_forward with respect to every
 * layer weight, the block embeddings and every layer's context caches. [P2]
 * "How It Works", step 1 and "Scope": the body is trained with an optimizer
 * step; step 3: the layers it differentiates; step 4: rows returned as zero
 * pass no gradient.
 *
 * d_out is the gradient of `out`. It reaches the last layer's output on the
 * rows the body returns (valid, non-empty block); then, from the last layer to
 * the first, each layer takes its forward activations from the reserve space and
 * applies
 *   d_w_down = dh^T u,  du = dh W_down,  (dg, dup) = SwiGLU backward at (g, up)
 *   d_w_gate = dg^T y,  d_w_up = dup^T y,  dy = dg W_gate + dup W_up
 *   dh1 = dh + RMSNorm backward (h1, mlp_norm) at dy           -> d_mlp_norm
 *   d_wo = dh1^T o,  do = dh1 Wo,  (dq, dk, dv, dKc, dVc) = attention backward at do
 *   d_wq|d_wk|d_wv = [dq|dk|dv]^T x,  dx = dq Wq + dk Wk + dv Wv
 *   dh_in = dh1 + RMSNorm backward (h, attn_norm) at dx         -> d_attn_norm
 * where x, y are the normalised inputs, g, up the SwiGLU pre-activations,
 * u = SiLU(g) up and o the attention output of the forward. RMSNorm backward of
 * y = x r w (r = (mean(x^2) + eps)^-1/2) at dy is r (dy w) - x r^3 sum(dy w x) / H,
 * with weight gradient sum over rows of dy x r. The attention backward is
 * dflash_block_attn_backward's, with no row's output gradient dropped (inside
 * the body invalid rows keep their attention output).
 *
 *   reserve         the reserve space dflash_body_forward_train filled for the same
 *                   blocks, weights and caches (read only)
 *   layers, ctx_k, ctx_v, ctx_total, block_ctx_base, block_anchor, block_valid
 *                   as dflash_body_forward
 *   d_out           device [nb*bs, H] in the config dtype
 *   d_block_embeds  device f32 [nb*bs, H], or NULL (not returned)
 *   grads           host array [num_layers]; every pointer device f32, 16-byte
 *                   aligned, overwritten
 *   d_ctx_k, d_ctx_v  host arrays [num_layers] of device f32 gradients in the
 *                   caches' layouts (K [Hkv][ctx_total][D] rotated frame, V
 *                   [Hkv][D][ctx_total]), overwritten; dflash_ctx_proj_backward
 *                   takes them on to W_proj
 *   workspace       dflash_body_backward_workspace_size(cfg, nb) bytes, 256-byte aligned
 * GEMM operands are in the config dtype (activation gradients are rounded to it
 * before their products); products accumulate in fp32; the residual-stream
 * gradient, the RMSNorm backward and every output are fp32. Deterministic: no
 * atomics, fixed reduction orders. With nb == 0 every output is zero.
 * Errors: as dflash_body_forward; INVALID_ARG for null required pointers or
 * misaligned arrays; UNSUPPORTED when intermediate is not a multiple of 128 or
 * hidden exceeds 8192; WORKSPACE when the workspace or the reserve is missing
 * (for nb > 0), small or misaligned.
 */
dflash_status dflash_body_backward(const dflash_config *cfg, int32_t num_blocks, const void *reserve,
                                   size_t reserve_bytes, const dflash_layer_weights *layers,
                                   void *const *ctx_k, void *const *ctx_v,
                                   int64_t ctx_total, const int64_t *block_ctx_base,
                                   const int32_t *block_anchor, const uint8_t *block_valid, const void *d_out,
                                   float *d_block_embeds, const dflash_layer_grads *grads,
                                   float *const *d_ctx_k, float *const *d_ctx_v, void *workspace,
                                   size_t workspace_bytes, void *hip_stream);
size_t dflash_body_backward_workspace_size(const dflash_config *cfg, int32_t num_blocks);

/*
 * dflash_adamw_step -- the optimizer step after the backward, over any set of
 * trainable tensors (the draft layers' weights, W_proj). [P2] "How It Works",
 * step 1, and "Scope": the draft body is trained with an optimizer step; the
 * pages name no optimizer, and this is AdamW (Adam's bias-corrected moments,
 * Kingma and Ba 2015; weight decay decoupled from the gradient, Loshchilov and
 * Hutter 2019), applied decay first, then the moments, then the step:
 *
 *   w <- w (1 - lr weight_decay)
 *   m <- beta1 m + (1 - beta1) g,    v <- beta2 v + (1 - beta2) g^2
 *   w <- w - (lr / (1 - beta1^step)) m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 *
 * elementwise in fp32; then weight = w rounded to `dtype` (the working copy the
 * next forward reads) where a weight pointer is given.
 *
 *   dtype          DFLASH_BF16 or DFLASH_F32: element type of the working copies
 *   tensors        host array of num_tensors descriptors; per tensor, device arrays
 *                  of numel elements: grad (f32, read), master weights, exp_avg and
 *                  exp_avg_sq (f32, updated in place; start the moments at zero),
 *                  weight (dtype, written; null: no working copy). All 16-byte
 *                  aligned; tensors must not overlap.
 *   step           the step number, 1 for the first update
 * Every element is independent, so results do not depend on the launch split.
 * Errors: INVALID_ARG for an unknown dtype, num_tensors < 0, step < 1, lr < 0,
 * beta outside [0, 1), eps <= 0, weight_decay < 0, negative numel, or a null or
 * misaligned array of a non-empty tensor.
 */
typedef struct dflash_adamw_tensor {
    const float *grad;
    float *master;
    float *exp_avg;
    float *exp_avg_sq;
    void *weight;
    int64_t numel;
} dflash_adamw_tensor;

dflash_status dflash_adamw_step(int32_t dtype, int32_t num_tensors, const dflash_adamw_tensor *tensors,
                                double lr, double beta1, double beta2, double eps, double weight_decay,
                                int64_t step, void *hip_stream);

/* Bytes of workspace that dflash_ctx_proj over ctx_rows rows and
 * dflash_block_attn / dflash_body_forward over num_blocks blocks need (one
 * buffer of this size serves all of them; 256-byte aligned). Returns 0 for an
 * invalid or unsupported config. */
size_t dflash_workspace_size(const dflash_config *cfg, int32_t num_blocks, int64_t ctx_rows);

/* Checks a config against the shape envelope without touching the GPU. */
dflash_status dflash_check_config(const dflash_config *cfg);

/* Static text for a status code. */
const char *dflash_status_string(dflash_status s);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
