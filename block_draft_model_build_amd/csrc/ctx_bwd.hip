// Backward of the context path (NeMo RL "DFlash Draft Body", Scope: training
// updates the projection W_proj; angelspec "DFlash", How it works: the target's
// hidden states are projected into every draft layer's K/V). The forward is
//   C = X W_proj^T,  Kc_l = RoPE(C Wk_l^T) at the rows' positions,  Vc_l = C Wv_l^T.
// Given the gradients of every layer's context K and V (as the attention
// backward writes them, in the caches' layouts), this computes
//   G = [Gk_1 .. Gk_L | Gv_1 .. Gv_L]     Gk_l = RoPE^T(dKc_l), Gv_l = dVc_l   [T, 2 L Hkv D]
//   dC = G [Wk_1; ..; Wk_L; Wv_1; ..; Wv_L]                                      [T, H]
//   dW_proj = dC^T X                                                            [H, L_t H_t]
// and, given C from the training forward, the context path's share of every
// layer's K/V projection gradient (each layer's Wk, Wv map C into its K/V):
//   d[Wk_1; ..; Wk_L; Wv_1; ..; Wv_L] += G^T C                                  [2 L Hkv D, H]
// The products run on the K-contiguous MFMA GEMM of gemm.h; the operands
// whose contraction runs down their rows (the stacked K/V weights, dC, X, G
// and C) are transposed on the way (LDS tiles; dC in the first product's
// epilogue).
#include "gemm_select.h"
#include "internal.h"
#include "transpose.h"

namespace dflash {

namespace {

struct GradPtrs {
    const float* dk[kMaxLayers];
    const float* dv[kMaxLayers];
};

// Gk: one thread per (row, 4 consecutive pairs); the pairs' rotations are
// computed once and applied to every layer and head. RoPE pairs i with
// i + D/2; its transpose is the rotation by the opposite angle.
template <typename T>
__global__ __launch_bounds__(256) void grad_pack_k_kernel(GradPtrs gp, const int32_t* positions, int64_t rows,
                                                          int64_t ctx_total, int64_t row_offset, int L, int hkv,
                                                          int D, RopeTurns rt, T* G, int64_t ldg) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    const int half = D / 2, q4 = half / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = idx / q4;
    const int i = (int)(idx - r * q4) * 4;
    if (r >= rows) return;
    float cs[4], sn[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rope_cs(rt, i + q, positions[r], cs[q], sn[q]);
    for (int l = 0; l < L; ++l)
        for (int g = 0; g < hkv; ++g) {
            const float* src = gp.dk[l] + ((int64_t)g * ctx_total + row_offset + r) * D;
            const f32x4 y1 = *reinterpret_cast<const f32x4*>(src + i);
            const f32x4 y2 = *reinterpret_cast<const f32x4*>(src + i + half);
            t4 a, b;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[q] = from_f32<T>(y1[q] * cs[q] + y2[q] * sn[q]);
                b[q] = from_f32<T>(y2[q] * cs[q] - y1[q] * sn[q]);
            }
            T* dst = G + r * ldg + (int64_t)(l * hkv + g) * D;
            *reinterpret_cast<t4*>(dst + i) = a;
            *reinterpret_cast<t4*>(dst + i + half) = b;
        }
}

// Gv: the V caches hold each head dimension by dimension ([D][ctx_total]);
// 64 rows x 64 dimensions per workgroup are transposed through LDS with
// 16-byte loads along the rows and 16-byte stores along the dimensions.
template <typename T>
__global__ __launch_bounds__(256) void grad_pack_v_kernel(GradPtrs gp, int64_t rows, int64_t ctx_total,
                                                          int64_t row_offset, int L, int hkv, int D, T* G,
                                                          int64_t ldg) {
    constexpr int VO = 16 / (int)sizeof(T);
    typedef T vout __attribute__((ext_vector_type(VO)));
    __shared__ float tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int lg = blockIdx.y, d0 = blockIdx.z * 64;
    const int l = lg / hkv, g = lg - l * hkv;
    const float* src = gp.dv[l] + (int64_t)g * D * ctx_total + row_offset;
    // Rows r0 .. r0 + 63 of each dimension row; 4 rows per load when the row
    // start is 16-byte aligned and all 4 rows exist, else one by one.
    const bool vec = ((row_offset + r0) & 3) == 0 && (ctx_total & 3) == 0;
    for (int idx = threadIdx.x; idx < 64 * 16; idx += 256) {
        const int dd = idx >> 4, t4 = (idx & 15) * 4;
        const float* srow = src + (int64_t)(d0 + dd) * ctx_total + r0 + t4;
        if (vec && r0 + t4 + 4 <= rows) {
            const f32x4 u = *reinterpret_cast<const f32x4*>(srow);
#pragma unroll
            for (int q = 0; q < 4; ++q) tile[dd][t4 + q] = u[q];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) tile[dd][t4 + q] = r0 + t4 + q < rows ? srow[q] : 0.f;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * (64 / VO); idx += 256) {
        const int tt = idx / (64 / VO), dv = (idx - tt * (64 / VO)) * VO;
        const int64_t r = r0 + tt;
        if (r >= rows) continue;
        vout o;
#pragma unroll
        for (int q = 0; q < VO; ++q) o[q] = from_f32<T>(tile[dv + q][tt]);
        *reinterpret_cast<vout*>(G + r * ldg + (int64_t)(L * hkv + lg) * D + d0 + dv) = o;
    }
}

// dC: transposed store (dC^T [H][ldt], the A operand of dW_proj) and, when
// asked for, the fp32 gradient itself [T][H].
template <typename T> struct EpDCT {
    T* dct; int64_t ldt; float* dch; int64_t ldh;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    const int col = nb + j * 32 + (lane & 31);
                    dct[(int64_t)col * ldt + row] = from_f32<T>(acc[i][j][e]);
                    if (dch) dch[(int64_t)row * ldh + col] = acc[i][j][e];
                }
            }
    }
};

// d[Wk; Wv] += acc: row r of the product is row r % (Hkv D) of layer
// (r / (Hkv D)) % L's Wk (r < L Hkv D) or Wv (after), added in fp32.
struct EpKVGradAdd {
    float* dst[2 * kMaxLayers];        // Wk of every layer, then Wv of every layer
    int kvd, H;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                const int t = row / kvd;
                float* o = dst[t] + (int64_t)(row - t * kvd) * H + nb + (lane & 31);
#pragma unroll
                for (int j = 0; j < NI; ++j) o[j * 32] += acc[i][j][e];
            }
    }
};

// Workspace (256-byte aligned regions, config dtype):
//   G [T][Kg], WkvT [H][Kg], dCT [H][Tp], XT [L_t H_t][Tp], and for the K/V weight
//   gradients GT [Kg][Tp], CT [H][Tp];  Kg = 2 L Hkv D, Tp = T rounded up to 64.
struct CtxBwdLayout {
    size_t g, wkvt, dct, xt, gt, ct, total;
    int64_t kg, tp;
};
CtxBwdLayout ctx_bwd_layout(const dflash_config& c, int64_t rows) {
    CtxBwdLayout l{};
    const size_t eb = (size_t)elem_bytes(c), A = 256;
    l.kg = (int64_t)2 * c.num_layers * c.num_kv_heads * c.head_dim;
    l.tp = (rows + 63) / 64 * 64;
    const int64_t kin = (int64_t)c.num_target_layers * c.target_hidden;
    size_t off = 0;
    l.g = off;    off = align_up(off + eb * (size_t)rows * l.kg, A);
    l.wkvt = off; off = align_up(off + eb * (size_t)c.hidden * l.kg, A);
    l.dct = off;  off = align_up(off + eb * (size_t)c.hidden * l.tp, A);
    l.xt = off;   off = align_up(off + eb * (size_t)kin * l.tp, A);
    l.gt = off;   off = align_up(off + eb * (size_t)l.kg * l.tp, A);
    l.ct = off;   off = align_up(off + eb * (size_t)c.hidden * l.tp, A);
    l.total = off + A;
    return l;
}

template <typename T>
hipError_t ctx_bwd_t(const dflash_config& c, const T* ts, int64_t rs, int64_t ls, int64_t rows,
                     const int32_t* positions, const dflash_layer_weights* layers, const GradPtrs& gp,
                     int64_t ctx_total, int64_t row_offset, float* d_w_proj, float* d_ctx_hidden, const T* C,
                     const EpKVGradAdd& dkv, char* ws, hipStream_t st) {
    const CtxBwdLayout lay = ctx_bwd_layout(c, rows);
    const int H = c.hidden, L = c.num_layers, hkv = c.num_kv_heads, D = c.head_dim;
    const int64_t kin = (int64_t)c.num_target_layers * c.target_hidden, kg = lay.kg, tp = lay.tp;
    T* G = reinterpret_cast<T*>(ws + lay.g);
    T* wkvt = reinterpret_cast<T*>(ws + lay.wkvt);
    T* dct = reinterpret_cast<T*>(ws + lay.dct);
    T* xt = reinterpret_cast<T*>(ws + lay.xt);
    {
        ProfScope prof(DFLASH_KERNEL_CTX_BWD_PACK, st);
        const int64_t quads = rows * (D / 8);
        hipLaunchKernelGGL(grad_pack_k_kernel<T>, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, gp,
                           positions, rows, ctx_total, row_offset, L, hkv, D, make_rope_turns(c), G, kg);
        hipLaunchKernelGGL(grad_pack_v_kernel<T>, dim3((unsigned)((rows + 63) / 64), L * hkv, D / 64), dim3(256), 0,
                           st, gp, rows, ctx_total, row_offset, L, hkv, D, G, kg);
        // Stacked weights, transposed: wkvt[n][(kind L + l) Hkv D + j] = W_kind,l[j][n].
        const int64_t kvd = (int64_t)hkv * D;
        for (int kind = 0; kind < 2; ++kind)
            for (int l = 0; l < L; ++l) {
                const T* w = static_cast<const T*>(kind == 0 ? layers[l].wk : layers[l].wv);
                hipLaunchKernelGGL((transpose_kernel<T, SrcPlain<T>>), dim3((unsigned)((kvd + 63) / 64), (H + 63) / 64),
                                   dim3(256), 0, st, SrcPlain<T>{w, H}, kvd, kvd, (int64_t)H,
                                   wkvt + (int64_t)(kind * L + l) * kvd, kg);
            }
        // X^T with zero columns past the last row.
        hipLaunchKernelGGL((transpose_kernel<T, SrcStacked<T>>), dim3((unsigned)(tp / 64), (unsigned)((kin + 63) / 64)),
                           dim3(256), 0, st, SrcStacked<T>{ts, rs, ls, c.target_hidden}, rows, tp, kin, xt, tp);
        if (tp > rows)
            hipLaunchKernelGGL(fill_cols_kernel<T>, dim3(64), dim3(256), 0, st, dct, tp, (int64_t)H, rows, tp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = gemm<T>(DFLASH_KERNEL_CTX_BWD_DC, (int)rows, H, (int)kg, APlain<T>{G, kg}, BPlain<T>{wkvt, kg},
                EpDCT<T>{dct, tp, d_ctx_hidden, H}, st);
    if (e != hipSuccess) return e;
    e = gemm<T>(DFLASH_KERNEL_CTX_BWD_DW, H, (int)kin, (int)tp, APlain<T>{dct, tp}, BPlain<T>{xt, tp},
                EpStoreF32{d_w_proj, kin}, st);
    if (e != hipSuccess || C == nullptr) return e;
    // d[Wk; Wv] += G^T C: both operands transposed to [features][Tp] (zero past the last row).
    T* gt = reinterpret_cast<T*>(ws + lay.gt);
    T* ct = reinterpret_cast<T*>(ws + lay.ct);
    {
        ProfScope prof(DFLASH_KERNEL_CTX_BWD_PACK, st);
        hipLaunchKernelGGL((transpose_kernel<T, SrcPlain<T>>), dim3((unsigned)(tp / 64), (unsigned)(kg / 64)),
                           dim3(256), 0, st, SrcPlain<T>{G, kg}, rows, tp, kg, gt, tp);
        hipLaunchKernelGGL((transpose_kernel<T, SrcPlain<T>>), dim3((unsigned)(tp / 64), (unsigned)(H / 64)),
                           dim3(256), 0, st, SrcPlain<T>{C, H}, rows, tp, (int64_t)H, ct, tp);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return gemm<T>(DFLASH_KERNEL_CTX_BWD_DKV, (int)kg, H, (int)tp, APlain<T>{gt, tp}, BPlain<T>{ct, tp}, dkv, st);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_ctx_proj_backward_workspace_size(const dflash_config* cfg, int64_t num_rows) {
    if (check_config(cfg) != DFLASH_OK || num_rows < 0) return 0;
    return ctx_bwd_layout(*cfg, num_rows).total;
}

extern "C" dflash_status dflash_ctx_proj_backward(const dflash_config* cfg, const void* target_states,
                                                  int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                                                  const int32_t* positions, const dflash_layer_weights* layers,
                                                  const float* const* d_ctx_k, const float* const* d_ctx_v,
                                                  int64_t ctx_total, int64_t row_offset, float* d_w_proj,
                                                  float* d_ctx_hidden, const void* ctx_hidden,
                                                  float* const* d_wk, float* const* d_wv, void* workspace,
                                                  size_t workspace_bytes, void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (num_rows < 0 || ctx_total < 0 || row_offset < 0 || row_offset + num_rows > ctx_total || d_w_proj == nullptr)
        return DFLASH_ERR_INVALID_ARG;
    const int64_t kin = (int64_t)cfg->num_target_layers * cfg->target_hidden;
    if (num_rows > INT32_MAX / 2 || kin % 128 != 0) return DFLASH_ERR_UNSUPPORTED;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (num_rows == 0) {
        // No rows: the gradient is zero.
        hipLaunchKernelGGL(fill_cols_kernel<float>, dim3(256), dim3(256), 0, st, d_w_proj, kin,
                           (int64_t)cfg->hidden, (int64_t)0, kin);
        return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
    }
    const int64_t vec = 16 / elem_bytes(*cfg);
    if (target_states == nullptr || positions == nullptr || layers == nullptr || d_ctx_k == nullptr ||
        d_ctx_v == nullptr || !aligned16(target_states) || ts_row_stride <= 0 || ts_layer_stride < 0 ||
        ts_row_stride % vec != 0 || ts_layer_stride % vec != 0)
        return DFLASH_ERR_INVALID_ARG;
    GradPtrs gp{};
    for (int l = 0; l < cfg->num_layers; ++l) {
        if (layers[l].wk == nullptr || layers[l].wv == nullptr || d_ctx_k[l] == nullptr || d_ctx_v[l] == nullptr ||
            !aligned16(layers[l].wk) || !aligned16(layers[l].wv) || !aligned16(d_ctx_k[l]) || !aligned16(d_ctx_v[l]))
            return DFLASH_ERR_INVALID_ARG;
        gp.dk[l] = d_ctx_k[l];
        gp.dv[l] = d_ctx_v[l];
    }
    EpKVGradAdd dkv{};
    if (ctx_hidden != nullptr) {
        if (!aligned16(ctx_hidden) || d_wk == nullptr || d_wv == nullptr) return DFLASH_ERR_INVALID_ARG;
        for (int l = 0; l < cfg->num_layers; ++l) {
            if (d_wk[l] == nullptr || d_wv[l] == nullptr || !aligned16(d_wk[l]) || !aligned16(d_wv[l]))
                return DFLASH_ERR_INVALID_ARG;
            dkv.dst[l] = d_wk[l];
            dkv.dst[cfg->num_layers + l] = d_wv[l];
        }
        dkv.kvd = cfg->num_kv_heads * cfg->head_dim;
        dkv.H = cfg->hidden;
    }
    const size_t need = ctx_bwd_layout(*cfg, num_rows).total;
    if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DFLASH_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = ctx_bwd_t<__bf16>(*cfg, static_cast<const __bf16*>(target_states), ts_row_stride, ts_layer_stride,
                              num_rows, positions, layers, gp, ctx_total, row_offset, d_w_proj, d_ctx_hidden,
                              static_cast<const __bf16*>(ctx_hidden), dkv, ws, st);
    else
        e = ctx_bwd_t<float>(*cfg, static_cast<const float*>(target_states), ts_row_stride, ts_layer_stride,
                             num_rows, positions, layers, gp, ctx_total, row_offset, d_w_proj, d_ctx_hidden,
                             static_cast<const float*>(ctx_hidden), dkv, ws, st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
