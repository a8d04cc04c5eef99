// Backward of the draft body (NeMo RL "DFlash Draft Body", How It Works,
// step 1 and Scope: the body is trained with an optimizer step; step 3: the
// decoder layers it runs; step 4: rows returned as zero pass no gradient).
//
// Per layer, from the last to the first, with the layer's activations from the
// training forward's reserve space (h, x, q, k, v, o, h1, y, gate, up, u):
//   d_w_down = dh^T u          du = dh W_down -> (dg, dup) in the epilogue
//   d_w_gate | d_w_up = [dg | dup]^T y          dy = [dg | dup] [W_gate; W_up]
//   dh1 = dh + RMSNorm^T(h1, mlp_norm; dy)
//   d_wo = dh1^T o             do = dh1 Wo
//   dq, dk, dv, dKc, dVc = attention backward (do)
//   d_wq | d_wk | d_wv = [dq | dk | dv]^T x     dx = [dq | dk | dv] [Wq; Wk; Wv]
//   dh_in = dh1 + RMSNorm^T(h, attn_norm; dx)
// Every product runs on the K-contiguous MFMA GEMM of gemm.h. Products that
// contract over rows (the weight gradients) take both operands transposed
// ([features][rows], zero-padded to a multiple of 64 rows); products with a
// weight on the right take that weight transposed, once per layer. Activation
// gradients enter their products in the config dtype; the residual-stream
// gradient and every output stay fp32.
#include "gemm_select.h"
#include "internal.h"
#include "norm.h"
#include "transpose.h"

namespace dflash {

namespace {

// Workspace (every region 256-byte aligned; T = config dtype, Rp = rows rounded
// up to 64):
//   attention backward scratch
//   transposes [features][Rp] T: xT, yT, oT, uT, dhT, dguT, dh1T, dqkvT
//   gradients: dh_b, dh1_b [R][H] T; dgu [R][2I] T; do_b [R][nq] T;
//     dqkv_b [R][nqkv] T; df (dy, then dx), dh1, dh [R][H] f32;
//     dq [R][nq], dk, dv [R][nk] f32; RMSNorm partial sums [R / kNormBwdRows][H] f32
//   transposed weights: W_down^T [I][H], [W_gate; W_up]^T [H][2I],
//     Wo^T [nq][H], [Wq; Wk; Wv]^T [H][nqkv]
struct BodyBwdLayout {
    size_t abw, xt, ot, yt, ut, dhb, dht, dgu, dgut, df, dh1, dh1b, dh1t, dob, dq, dk, dv, dqkv, dqkvt, dh, part,
        wdt, wgut, wot, wqkvt, total;
    int64_t rp;
};

BodyBwdLayout body_bwd_layout(const dflash_config& c, int nb) {
    BodyBwdLayout l{};
    const size_t A = 256, eb = (size_t)elem_bytes(c);
    const size_t R = (size_t)nb * c.block_size, H = c.hidden, I = c.intermediate;
    const size_t nq = (size_t)c.num_q_heads * c.head_dim, nk = (size_t)c.num_kv_heads * c.head_dim;
    const size_t nqkv = nq + 2 * nk;
    l.rp = (int64_t)((R + 63) / 64 * 64);
    const size_t Rp = (size_t)l.rp;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, A);
        return o;
    };
    l.abw = take(attn_backward_workspace(c, nb));
    l.xt = take(eb * H * Rp);
    l.ot = take(eb * nq * Rp);
    l.yt = take(eb * H * Rp);
    l.ut = take(eb * I * Rp);
    l.dhb = take(eb * R * H);
    l.dht = take(eb * H * Rp);
    l.dgu = take(eb * R * 2 * I);
    l.dgut = take(eb * 2 * I * Rp);
    l.df = take(4 * R * H);
    l.dh1 = take(4 * R * H);
    l.dh1b = take(eb * R * H);
    l.dh1t = take(eb * H * Rp);
    l.dob = take(eb * R * nq);
    l.dq = take(4 * R * nq);
    l.dk = take(4 * R * nk);
    l.dv = take(4 * R * nk);
    l.dqkv = take(eb * R * nqkv);
    l.dqkvt = take(eb * nqkv * Rp);
    l.dh = take(4 * R * H);
    l.part = take(4 * ((R + kNormBwdRows - 1) / kNormBwdRows) * H);
    l.wdt = take(eb * I * H);
    l.wgut = take(eb * H * 2 * I);
    l.wot = take(eb * nq * H);
    l.wqkvt = take(eb * H * nqkv);
    l.total = off + A;
    return l;
}

// dst[c][r] = src[r][c] for a [rows][cols] matrix of the config dtype (ld lds),
// zero for rows in [rows, rows_pad); dst has leading dimension ldd.
template <typename T>
void transpose_to(const T* src, int64_t lds, int64_t rows, int64_t rows_pad, int64_t cols, T* dst, int64_t ldd,
                  hipStream_t st) {
    hipLaunchKernelGGL((transpose_kernel<T, SrcPlain<T>>), dim3((unsigned)((rows_pad + 63) / 64), (unsigned)(cols / 64)),
                       dim3(256), 0, st, SrcPlain<T>{src, lds}, rows, rows_pad, cols, dst, ldd);
}

// fp32 [rows][cols] -> config dtype row-major (optional) and transposed [cols][rows_pad].
template <typename T>
void pack_to(const float* src, int64_t lds, int64_t rows, int64_t rows_pad, int64_t cols, T* rm, int64_t ldr, T* tr,
             int64_t ldt, hipStream_t st) {
    hipLaunchKernelGGL(pack_f32_kernel<T>, dim3((unsigned)(rows_pad / 64), (unsigned)(cols / 64)), dim3(256), 0, st,
                       src, lds, rows, rows_pad, rm, ldr, tr, ldt);
}

template <typename T>
hipError_t norm_bwd(const float* x, const T* w, const float* dy, const float* res, float* out, float* part,
                    float* dw, int R, int H, float eps, hipStream_t st) {
    ProfScope prof(DFLASH_KERNEL_BWD_NORM, st);
    const int nparts = (R + kNormBwdRows - 1) / kNormBwdRows;
    // float4 columns per thread: the fewest that cover the row
    const int nv = (H / 4 + 255) / 256;
    auto kern = nv <= 1 ? rmsnorm_bwd_kernel<T, 1>
              : nv <= 2 ? rmsnorm_bwd_kernel<T, 2>
              : nv <= 4 ? rmsnorm_bwd_kernel<T, 4> : rmsnorm_bwd_kernel<T, 8>;
    hipLaunchKernelGGL(kern, dim3(nparts), dim3(256), 0, st, x, w, dy, res, out, part, R, H, eps);
    hipLaunchKernelGGL(norm_colsum_kernel, dim3((H + 63) / 64), dim3(256), 0, st, part, nparts, H, dw);
    return hipGetLastError();
}

#define DFLASH_TRY(expr)                         \
    do {                                         \
        const hipError_t e_ = (expr);            \
        if (e_ != hipSuccess) return e_;         \
    } while (0)

// One layer: dh holds dL/d(layer output) on entry and dL/d(layer input) on exit;
// lb is the layer's block of the reserve space, hl its input residual.
template <typename T>
hipError_t layer_bwd_t(const dflash_config& c, int nb, const float* hl, const char* lb, const TrainReserve& tr,
                       const dflash_layer_weights& L, const T* ck, const T* cv, int64_t ctx_total,
                       const int64_t* base, const int32_t* anchor, float* dh, const dflash_layer_grads& G,
                       float* dck, float* dcv, char* ws, const BodyBwdLayout& lay, hipStream_t st) {
    const int R = nb * c.block_size, H = c.hidden, I = c.intermediate, D = c.head_dim;
    const int nq = c.num_q_heads * D, nk = c.num_kv_heads * D, nqkv = nq + 2 * nk;
    const int64_t Rp = lay.rp;
    auto P = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    auto SP = [&](size_t off) { return reinterpret_cast<const T*>(lb + off); };
    auto SF = [&](size_t off) { return reinterpret_cast<const float*>(lb + off); };
    const T* wq = static_cast<const T*>(L.wq);
    const T* wk = static_cast<const T*>(L.wk);
    const T* wv = static_cast<const T*>(L.wv);
    const T* wo = static_cast<const T*>(L.wo);
    const T* wg = static_cast<const T*>(L.w_gate);
    const T* wu = static_cast<const T*>(L.w_up);
    const T* wd = static_cast<const T*>(L.w_down);
    const T *x = SP(tr.x), *q = SP(tr.q), *k = SP(tr.k), *v = SP(tr.v), *o = SP(tr.o), *y = SP(tr.y), *u = SP(tr.u);
    const float *h1 = SF(tr.h1), *gate = SF(tr.gate), *up = SF(tr.up);

    // ---- transposed weights and activations
    {
        ProfScope prof(DFLASH_KERNEL_BWD_PACK, st);
        transpose_to<T>(wd, I, H, H, I, P(lay.wdt), H, st);                       // [I][H]
        transpose_to<T>(wg, H, I, I, H, P(lay.wgut), 2 * I, st);                  // [H][2I]
        transpose_to<T>(wu, H, I, I, H, P(lay.wgut) + I, 2 * I, st);
        transpose_to<T>(wo, nq, H, H, nq, P(lay.wot), H, st);                     // [nq][H]
        transpose_to<T>(wq, H, nq, nq, H, P(lay.wqkvt), nqkv, st);                // [H][nqkv]
        transpose_to<T>(wk, H, nk, nk, H, P(lay.wqkvt) + nq, nqkv, st);
        transpose_to<T>(wv, H, nk, nk, H, P(lay.wqkvt) + nq + nk, nqkv, st);
        transpose_to<T>(x, H, R, Rp, H, P(lay.xt), Rp, st);
        transpose_to<T>(y, H, R, Rp, H, P(lay.yt), Rp, st);
        transpose_to<T>(o, nq, R, Rp, nq, P(lay.ot), Rp, st);
        transpose_to<T>(u, I, R, Rp, I, P(lay.ut), Rp, st);
        pack_to<T>(dh, H, R, Rp, H, P(lay.dhb), H, P(lay.dht), Rp, st);
    }
    DFLASH_TRY(hipGetLastError());

    // ---- MLP
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_WEIGHT, H, I, (int)Rp, APlain<T>{P(lay.dht), Rp}, BPlain<T>{P(lay.ut), Rp},
                       EpStoreF32{G.w_down, I}, st));
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_DATA, R, I, H, APlain<T>{P(lay.dhb), H}, BPlain<T>{P(lay.wdt), H},
                       EpSwiGLUBwd<T>{gate, up, P(lay.dgu), I}, st));
    {
        ProfScope prof(DFLASH_KERNEL_BWD_PACK, st);
        transpose_to<T>(P(lay.dgu), 2 * I, R, Rp, 2 * I, P(lay.dgut), Rp, st);
    }
    DFLASH_TRY(hipGetLastError());
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_WEIGHT, 2 * I, H, (int)Rp, APlain<T>{P(lay.dgut), Rp},
                       BPlain<T>{P(lay.yt), Rp}, EpStoreF32Rows3{G.w_gate, G.w_up, nullptr, I, 2 * I, H}, st));
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_DATA, R, H, 2 * I, APlain<T>{P(lay.dgu), 2 * I},
                       BPlain<T>{P(lay.wgut), 2 * I}, EpStoreF32{F(lay.df), H}, st));
    DFLASH_TRY(norm_bwd<T>(h1, static_cast<const T*>(L.mlp_norm), F(lay.df), dh, F(lay.dh1), F(lay.part), G.mlp_norm,
                           R, H, c.rms_eps, st));

    // ---- attention
    {
        ProfScope prof(DFLASH_KERNEL_BWD_PACK, st);
        pack_to<T>(F(lay.dh1), H, R, Rp, H, P(lay.dh1b), H, P(lay.dh1t), Rp, st);
    }
    DFLASH_TRY(hipGetLastError());
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_WEIGHT, H, nq, (int)Rp, APlain<T>{P(lay.dh1t), Rp}, BPlain<T>{P(lay.ot), Rp},
                       EpStoreF32{G.wo, nq}, st));
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_DATA, R, nq, H, APlain<T>{P(lay.dh1b), H}, BPlain<T>{P(lay.wot), H},
                       EpStore<T>{P(lay.dob), nq}, st));
    DFLASH_TRY(attn_backward_run(&c, nb, q, k, v, ck, cv, ctx_total, base, anchor, nullptr, o, P(lay.dob),
                                 F(lay.dq), F(lay.dk), F(lay.dv), dck, dcv, ws + lay.abw, st));
    {
        ProfScope prof(DFLASH_KERNEL_BWD_PACK, st);
        T* dqkv = P(lay.dqkv);
        T* dqkvt = P(lay.dqkvt);
        pack_to<T>(F(lay.dq), nq, R, Rp, nq, dqkv, nqkv, dqkvt, Rp, st);
        pack_to<T>(F(lay.dk), nk, R, Rp, nk, dqkv + nq, nqkv, dqkvt + (int64_t)nq * Rp, Rp, st);
        pack_to<T>(F(lay.dv), nk, R, Rp, nk, dqkv + nq + nk, nqkv, dqkvt + (int64_t)(nq + nk) * Rp, Rp, st);
    }
    DFLASH_TRY(hipGetLastError());
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_WEIGHT, nqkv, H, (int)Rp, APlain<T>{P(lay.dqkvt), Rp},
                       BPlain<T>{P(lay.xt), Rp}, EpStoreF32Rows3{G.wq, G.wk, G.wv, nq, nq + nk, H}, st));
    DFLASH_TRY(gemm<T>(DFLASH_KERNEL_BWD_DATA, R, H, nqkv, APlain<T>{P(lay.dqkv), nqkv},
                       BPlain<T>{P(lay.wqkvt), nqkv}, EpStoreF32{F(lay.df), H}, st));
    return norm_bwd<T>(hl, static_cast<const T*>(L.attn_norm), F(lay.df), F(lay.dh1), dh, F(lay.part), G.attn_norm,
                       R, H, c.rms_eps, st);
}

template <typename T>
hipError_t body_bwd_t(const dflash_config& c, int nb, const char* reserve, const dflash_layer_weights* layers,
                      void* const* ck, void* const* cv, int64_t ctx_total, const int64_t* base, const int32_t* anchor,
                      const uint8_t* valid, const T* dout, float* demb, const dflash_layer_grads* grads,
                      float* const* dck, float* const* dcv, char* ws, hipStream_t st) {
    const BodyBwdLayout lay = body_bwd_layout(c, nb);
    const TrainReserve tr = train_reserve_layout(c, nb);
    const int R = nb * c.block_size, H = c.hidden;
    float* dh = demb ? demb : reinterpret_cast<float*>(ws + lay.dh);
    {
        ProfScope prof(DFLASH_KERNEL_BWD_PACK, st);
        const int64_t n4 = (int64_t)R * (H / 4);
        const unsigned grid = (unsigned)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
        hipLaunchKernelGGL(mask_grad_kernel<T>, dim3(grid), dim3(256), 0, st, dout, valid, anchor, c.block_size,
                           (int64_t)R, H, dh);
    }
    DFLASH_TRY(hipGetLastError());
    const float* hs = reinterpret_cast<const float*>(reserve);
    for (int l = c.num_layers - 1; l >= 0; --l)
        DFLASH_TRY(layer_bwd_t<T>(c, nb, hs + (int64_t)l * R * H, reserve + tr.layer0 + (size_t)l * tr.per_layer, tr,
                                  layers[l], static_cast<const T*>(ck[l]), static_cast<const T*>(cv[l]), ctx_total,
                                  base, anchor, dh, grads[l], dck ? dck[l] : nullptr, dcv ? dcv[l] : nullptr, ws,
                                  lay, st));
    return hipSuccess;
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

void zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return;
    const unsigned grid = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, st, p, n);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dflash_status body_bwd_supported(const dflash_config* cfg) {
    const dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    // (Hq * D is a multiple of 128 whenever the config is valid: (Hq + 2 Hkv) D is,
    // and D = 64 forces Hq even.)
    if (cfg->intermediate % 128 != 0 || cfg->hidden > kNormBwdMaxH)
        return DFLASH_ERR_UNSUPPORTED;
    return DFLASH_OK;
}

}  // namespace

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_body_backward_workspace_size(const dflash_config* cfg, int32_t num_blocks) {
    if (body_bwd_supported(cfg) != DFLASH_OK || num_blocks < 0 ||
        (int64_t)num_blocks * cfg->block_size > INT32_MAX / 2)
        return 0;
    return body_bwd_layout(*cfg, num_blocks).total;
}

extern "C" dflash_status dflash_body_backward(const dflash_config* cfg, int32_t num_blocks, const void* reserve,
                                              size_t reserve_bytes, const dflash_layer_weights* layers, void* const* ctx_k,
                                              void* const* ctx_v, int64_t ctx_total, const int64_t* block_ctx_base,
                                              const int32_t* block_anchor, const uint8_t* block_valid,
                                              const void* d_out, float* d_block_embeds,
                                              const dflash_layer_grads* grads, float* const* d_ctx_k,
                                              float* const* d_ctx_v, void* workspace, size_t workspace_bytes,
                                              void* hip_stream) {
    dflash_status s = body_bwd_supported(cfg);
    if (s != DFLASH_OK) return s;
    if (num_blocks < 0 || ctx_total < 0) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)num_blocks * cfg->block_size > INT32_MAX / 2 ||
        (ctx_total + 63) / 64 * cfg->num_kv_heads > INT32_MAX)
        return DFLASH_ERR_UNSUPPORTED;
    const int L = cfg->num_layers, H = cfg->hidden, I = cfg->intermediate;
    const int64_t nq = (int64_t)cfg->num_q_heads * cfg->head_dim, nk = (int64_t)cfg->num_kv_heads * cfg->head_dim;
    if (layers == nullptr || grads == nullptr || (ctx_total > 0 && (d_ctx_k == nullptr || d_ctx_v == nullptr)))
        return DFLASH_ERR_INVALID_ARG;
    for (int l = 0; l < L; ++l) {
        const dflash_layer_grads& G = grads[l];
        const float* gp[9] = {G.attn_norm, G.wq, G.wk, G.wv, G.wo, G.mlp_norm, G.w_gate, G.w_up, G.w_down};
        for (const float* p : gp)
            if (p == nullptr || !aligned16(p)) return DFLASH_ERR_INVALID_ARG;
        if (ctx_total > 0 && (d_ctx_k[l] == nullptr || d_ctx_v[l] == nullptr || !aligned16(d_ctx_k[l]) ||
                              !aligned16(d_ctx_v[l])))
            return DFLASH_ERR_INVALID_ARG;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (num_blocks == 0) {
        // No block: nothing reads the weights or the caches.
        for (int l = 0; l < L; ++l) {
            const dflash_layer_grads& G = grads[l];
            zero(G.attn_norm, H, st);
            zero(G.mlp_norm, H, st);
            zero(G.wq, nq * H, st);
            zero(G.wk, nk * H, st);
            zero(G.wv, nk * H, st);
            zero(G.wo, (int64_t)H * nq, st);
            zero(G.w_gate, (int64_t)I * H, st);
            zero(G.w_up, (int64_t)I * H, st);
            zero(G.w_down, (int64_t)H * I, st);
            if (ctx_total > 0) {
                zero(d_ctx_k[l], nk * ctx_total, st);
                zero(d_ctx_v[l], nk * ctx_total, st);
            }
        }
        return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
    }
    if (reserve == nullptr || ctx_k == nullptr || ctx_v == nullptr || block_ctx_base == nullptr ||
        block_anchor == nullptr || block_valid == nullptr || d_out == nullptr || !aligned16(d_out) ||
        !aligned16(d_block_embeds))
        return DFLASH_ERR_INVALID_ARG;
    for (int l = 0; l < L; ++l) {
        const dflash_layer_weights& W = layers[l];
        const void* ptrs[9] = {W.attn_norm, W.wq, W.wk, W.wv, W.wo, W.mlp_norm, W.w_gate, W.w_up, W.w_down};
        for (const void* p : ptrs)
            if (p == nullptr || !aligned16(p)) return DFLASH_ERR_INVALID_ARG;
        if ((ctx_total > 0 && (ctx_k[l] == nullptr || ctx_v[l] == nullptr)) || !aligned16(ctx_k[l]) ||
            !aligned16(ctx_v[l]))
            return DFLASH_ERR_INVALID_ARG;
    }
    const size_t need = body_bwd_layout(*cfg, num_blocks).total;
    if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        reserve_bytes < train_reserve_layout(*cfg, num_blocks).total || (reinterpret_cast<uintptr_t>(reserve) & 255u) != 0)
        return DFLASH_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = body_bwd_t<__bf16>(*cfg, num_blocks, static_cast<const char*>(reserve), layers, ctx_k, ctx_v, ctx_total, block_ctx_base,
                               block_anchor, block_valid, static_cast<const __bf16*>(d_out), d_block_embeds, grads,
                               d_ctx_k, d_ctx_v, ws, st);
    else
        e = body_bwd_t<float>(*cfg, num_blocks, static_cast<const char*>(reserve), layers, ctx_k, ctx_v, ctx_total, block_ctx_base,
                              block_anchor, block_valid, static_cast<const float*>(d_out), d_block_embeds, grads,
                              d_ctx_k, d_ctx_v, ws, st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
