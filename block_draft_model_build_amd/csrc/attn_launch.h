// Host-side launch sequence of the dual-source block attention: scheduler,
// per-split kernels and the combine step, shared by the body forward and the
// body backward (which recomputes each layer's attention).
#pragma once

#include "attention.h"
#include "internal.h"

namespace dflash {

template <typename T, int D, int QC>
static hipError_t attn_launch_t(const dflash_config& c, const AttnArgs<T>& a, int nb, hipStream_t st) {
    const int items_max = attn_items_max(c, nb);
    {
        ProfScope prof(DFLASH_KERNEL_ATTENTION, st);
        hipLaunchKernelGGL((block_attn_kernel<T, D, QC>), dim3(items_max), dim3(256), 0, st, a);
        hipLaunchKernelGGL((block_attn_kernel<T, D, QC, true>), dim3(items_max), dim3(256), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(DFLASH_KERNEL_ATTN_COMBINE, st);
        hipLaunchKernelGGL((attn_combine_kernel<T, D, QC>), dim3(nb, c.num_kv_heads), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t attn_launch(const dflash_config& c, const AttnArgs<T>& a, int nb, hipStream_t st) {
    constexpr int D = 256 / (int)sizeof(T);
    if (attn_qcols(c) == 32) return attn_launch_t<T, D, 32>(c, a, nb, st);
    return attn_launch_t<T, D, 64>(c, a, nb, st);
}

template <typename T>
static AttnArgs<T> attn_args(const dflash_config& c, int nb, const T* q, int64_t q_ld, const T* kb,
                             const T* vb, int64_t kv_ld, const T* ck, const T* cvt, int64_t ctx_total,
                             const int64_t* base, const int32_t* anchor, const uint8_t* valid, T* out,
                             int64_t out_ld, char* ws, const Workspace& w) {
    AttnArgs<T> a;
    a.q = q; a.q_ld = q_ld; a.kb = kb; a.vb = vb; a.kv_ld = kv_ld;
    a.ck = ck; a.cvt = cvt; a.ctx_total = ctx_total;
    a.base = base; a.anchor = anchor; a.valid = valid;
    a.out = out; a.out_ld = out_ld;
    a.nb = nb; a.bs = c.block_size; a.hq = c.num_q_heads; a.hkv = c.num_kv_heads;
    a.qscale = (float)(1.4426950408889634 / sqrt((double)c.head_dim));
    a.group_start = reinterpret_cast<const int*>(ws + w.group_start);
    a.item_start = reinterpret_cast<const int*>(ws + w.item_start);
    a.sched = reinterpret_cast<const int*>(ws + w.sched);
    a.meta = reinterpret_cast<const int*>(ws + w.meta);
    a.bmeta = reinterpret_cast<const int4*>(ws + w.bmeta);
    a.part_o = reinterpret_cast<float*>(ws + w.part_o);
    a.part_ml = reinterpret_cast<float*>(ws + w.part_ml);
    a.redo = reinterpret_cast<int*>(ws + w.redo);
    a.rt = make_rope_turns(c);
    return a;
}

static hipError_t attn_schedule(const dflash_config& c, int nb, const int64_t* base, const int32_t* anchor,
                                int64_t ctx_total, char* ws, const Workspace& w, hipStream_t st) {
    const int hkv = c.num_kv_heads;
    hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(1024), 0, st, base, anchor, nb, ctx_total,
                       (kAttnItemsShared + hkv - 1) / hkv, (kAttnItemsSingle + hkv - 1) / hkv,
                       reinterpret_cast<int*>(ws + w.group_start),
                       reinterpret_cast<int*>(ws + w.item_start), reinterpret_cast<int*>(ws + w.sched),
                       reinterpret_cast<int*>(ws + w.meta), reinterpret_cast<int4*>(ws + w.bmeta));
    return hipGetLastError();
}

}  // namespace dflash
