// Host-side helpers shared by the libdflash translation units.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dflash.h"
#include "common.h"

namespace dflash {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int elem_bytes(const dflash_config& c) { return c.dtype == DFLASH_BF16 ? 2 : 4; }

// The attention scheduler sizes splits so that about kAttnItemsShared work
// items (group x split x KV head) carry the prefix work of multi-block groups
// (several blocks share each K/V tile: long items are cheapest) and about
// kAttnItemsSingle that of single-block groups (each block reads its own
// prefix: more items in flight help). Chosen by sweeps over 256..2048 items on
// the 5-layer, long-context and ragged-cache workloads.
constexpr int kAttnItemsShared = 256;
constexpr int kAttnItemsSingle = 1024;
inline int attn_target_splits(const dflash_config& c, int nb) {
    (void)nb;
    return (kAttnItemsShared + kAttnItemsSingle + c.num_kv_heads - 1) / c.num_kv_heads;
}

inline int attn_qcols(const dflash_config& c) {
    return c.block_size * (c.num_q_heads / c.num_kv_heads) <= 32 ? 32 : 64;
}

// Workspace layout (every region 256-byte aligned):
//   attention scheduler: group_start [nb+1], item_start [nb+1], sched [4] (i32),
//                        item records [splits_max][16] and block records [nb][4] (i32)
//   attention partials:  part_o [items_max][4][QC][D] f32, part_ml [items_max][4][QC][2] f32,
//                        redo [items_max][4] i32
//   body: h [R][H] f32, x [R][H], qkv [R][(Hq+2Hkv)D], att [R][Hq D], u [R][I]   (dtype)
//   ctx_proj: C [ctx_rows][H] (dtype); shares the body's space (calls are stream-ordered).
struct Workspace {
    size_t group_start, item_start, sched, meta, bmeta, part_o, part_ml, redo, h, x, qkv, att, u, c, total;
};

// Group-splits (work items per KV head) the scheduler can form for nb blocks.
inline int attn_splits_max(const dflash_config& c, int nb) {
    return nb <= 0 ? 0 : attn_target_splits(c, nb) + nb;
}

inline int attn_items_max(const dflash_config& c, int nb) {
    return c.num_kv_heads * attn_splits_max(c, nb);   // none for the context projection alone
}

inline Workspace workspace_layout(const dflash_config& c, int nb, int64_t ctx_rows) {
    Workspace w{};
    const size_t A = 256, eb = (size_t)elem_bytes(c);
    const size_t R = (size_t)nb * (size_t)c.block_size;
    const size_t H = (size_t)c.hidden, D = (size_t)c.head_dim;
    const size_t qc = (size_t)attn_qcols(c);
    const size_t parts = (size_t)attn_items_max(c, nb) * 4;
    size_t off = 0;
    w.group_start = off; off = align_up(off + sizeof(int) * ((size_t)nb + 1), A);
    w.item_start = off;  off = align_up(off + sizeof(int) * ((size_t)nb + 1), A);
    w.sched = off;       off = align_up(off + sizeof(int) * 4, A);
    w.meta = off;        off = align_up(off + sizeof(int) * 16 * (size_t)attn_splits_max(c, nb), A);
    w.bmeta = off;       off = align_up(off + sizeof(int) * 4 * (size_t)nb, A);
    w.part_o = off;      off = align_up(off + sizeof(float) * parts * qc * D, A);
    w.part_ml = off;     off = align_up(off + sizeof(float) * parts * qc * 2, A);
    w.redo = off;        off = align_up(off + sizeof(int) * parts, A);
    const size_t shared0 = off;
    w.h = off;          off = align_up(off + sizeof(float) * R * H, A);
    w.x = off;          off = align_up(off + eb * R * H, A);
    w.qkv = off;        off = align_up(off + eb * R * (size_t)(c.num_q_heads + 2 * c.num_kv_heads) * D, A);
    w.att = off;        off = align_up(off + eb * R * (size_t)c.num_q_heads * D, A);
    w.u = off;          off = align_up(off + eb * R * (size_t)c.intermediate, A);
    const size_t body_end = off;
    w.c = shared0;
    const size_t c_end = align_up(shared0 + eb * (size_t)ctx_rows * H, A);
    w.total = body_end > c_end ? body_end : c_end;
    return w;
}

// Reserve space of a training step (dflash_body_forward_train writes it,
// dflash_body_backward reads it): first every layer's fp32 input residual
// h [L][R][H] (offset 0, part of the documented interface), then one block per
// layer (offset layer0 + l * per_layer) holding that layer's activations:
//   h1 [R][H], gate [R][I], up [R][I] (fp32);  x [R][H], y [R][H], q [R][nq],
//   k [R][nk], v [R][nk], o [R][nq], u [R][I] (config dtype)
// at the offsets below, relative to the layer's block (each 256-byte aligned).
struct TrainReserve {
    size_t layer0, per_layer, h1, gate, up, x, y, q, k, v, o, u, total;
};

inline TrainReserve train_reserve_layout(const dflash_config& c, int nb) {
    TrainReserve t{};
    const size_t A = 256, eb = (size_t)elem_bytes(c);
    const size_t R = (size_t)nb * (size_t)c.block_size, H = (size_t)c.hidden, I = (size_t)c.intermediate;
    const size_t nq = (size_t)c.num_q_heads * c.head_dim, nk = (size_t)c.num_kv_heads * c.head_dim;
    t.layer0 = align_up(sizeof(float) * (size_t)c.num_layers * R * H, A);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, A);
        return o;
    };
    t.h1 = take(sizeof(float) * R * H);
    t.gate = take(sizeof(float) * R * I);
    t.up = take(sizeof(float) * R * I);
    t.x = take(eb * R * H);
    t.y = take(eb * R * H);
    t.q = take(eb * R * nq);
    t.k = take(eb * R * nk);
    t.v = take(eb * R * nk);
    t.o = take(eb * R * nq);
    t.u = take(eb * R * I);
    t.per_layer = off;
    t.total = t.layer0 + (size_t)c.num_layers * t.per_layer;
    return t;
}

inline RopeTurns make_rope_turns(const dflash_config& c) {
    RopeTurns rt{};
    const int half = c.head_dim / 2;
    for (int i = 0; i < half && i < 64; ++i)
        rt.turns[i] = pow(c.rope_theta, -2.0 * (double)i / (double)c.head_dim) / (2.0 * M_PI);
    return rt;
}

dflash_status check_config(const dflash_config* c);

// Row stride of the fp32 logits dflash_lm_head_ce_train keeps (and of the
// backward's dz): the vocabulary rounded up to 64 columns.
inline int64_t lm_logits_ld(int vocab) { return ((int64_t)vocab + 63) / 64 * 64; }

// The attention backward (attn_bwd.hip) for callers that checked the arguments:
// the kernels of dflash_block_attn_backward on `st`, with `ws` holding
// attn_backward_workspace(c, nb) bytes. A null block_valid keeps every row's
// output gradient (inside the body no row's attention output is zeroed).
hipError_t attn_backward_run(const dflash_config* cfg, int num_blocks, const void* q, const void* k_blk,
                             const void* v_blk, const void* ctx_k, const void* ctx_v, int64_t ctx_total,
                             const int64_t* block_ctx_base, const int32_t* block_anchor, const uint8_t* block_valid,
                             const void* out, const void* d_out, float* d_q, float* d_k_blk, float* d_v_blk,
                             float* d_ctx_k, float* d_ctx_v, char* ws, hipStream_t st);
size_t attn_backward_workspace(const dflash_config& c, int nb);

// Records the measurement hook's events around the launches made in its scope
// when `kernel` is the kernel being profiled (dflash_profile_start).
class ProfScope {
  public:
    ProfScope(int kernel, hipStream_t st);
    ~ProfScope();
    ProfScope(const ProfScope&) = delete;
    ProfScope& operator=(const ProfScope&) = delete;

  private:
    hipStream_t stream_;
    int slot_;
};

}  // namespace dflash
