// Gradient of the decayed cross-entropy loss with respect to the hidden rows
// (angelspec "DFlash", How it works, Loss; Configuration: the LM head is the
// target's and frozen). With c_r the row's share of the loss and p_r the
// softmax of its logits:
//   dz_r = c_r (p_r - onehot(t_r)),   d_hidden_r = dz_r W_lm
// Row statistics first (the target logit as a dot product, then logsumexp from
// the forward's CE, and c_r from the decayed weights in a fixed order), then the
// logits' product with the gradient in its epilogue (dz stored in the config
// dtype, columns padded with zeros to a multiple of 64), then dz W_lm on the
// same K-contiguous GEMM with the head transposed through LDS tiles.
#include "gemm_select.h"
#include "internal.h"
#include "transpose.h"

namespace dflash {

namespace {

// zt[r] = hidden[r] . W_lm[targets[r]] (fp32), 0 for a target outside the vocabulary.
template <typename T>
__global__ __launch_bounds__(256) void target_logit_kernel(const T* hidden, const T* W, const int32_t* targets,
                                                           int H, int vocab, float* zt) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int t = targets[row];
    const bool ok = t >= 0 && t < vocab;
    float s = 0.f;
    if (ok) {
        const t4* hp = reinterpret_cast<const t4*>(hidden + row * H);
        const t4* wp = reinterpret_cast<const t4*>(W + (int64_t)t * H);
        for (int j = threadIdx.x; j < H / 4; j += 256) {
            const t4 a = hp[j], b = wp[j];
#pragma unroll
            for (int q = 0; q < 4; ++q) s += to_f32(a[q]) * to_f32(b[q]);
        }
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) zt[row] = (red[0] + red[1]) + (red[2] + red[3]);
}

// zt[r] = logits[r][targets[r]] from the logits the training forward kept (0
// for a target outside the vocabulary).
__global__ __launch_bounds__(256) void saved_target_logit_kernel(const float* logits, int64_t ldl,
                                                                 const int32_t* targets, int rows, int vocab,
                                                                 float* zt) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= rows) return;
    const int t = targets[r];
    zt[r] = (t >= 0 && t < vocab) ? logits[(int64_t)r * ldl + t] : 0.f;
}

// dz from the kept logits, the same arithmetic as EpCEGrad: 8 consecutive
// columns per thread (two 16-byte loads), exact zeros past the vocabulary up
// to ld and on rows whose coef is 0 (their logits are not read). Logits and dz
// (GBs, each touched once here) use non-temporal accesses: 0.65 -> 0.61 ms at
// 4096 rows x 151936.
template <typename T>
__device__ __forceinline__ void ce_grad_saved_run(const float* __restrict__ logits, int64_t ld,
                                                  const float* __restrict__ coef, const float* __restrict__ lse,
                                                  const int32_t* __restrict__ targets, int vocab,
                                                  T* __restrict__ dz, int64_t row, int64_t c0) {
    typedef T t8 __attribute__((ext_vector_type(8)));
    const float c = coef[row], L = lse[row];
    const int t = targets[row];
    float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c != 0.f) {
        const f32x4* p = reinterpret_cast<const f32x4*>(logits + row * ld + c0);
        const f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            z[q] = a[q];
            z[4 + q] = b[q];
        }
    }
    t8 o;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int64_t col = c0 + q;
        float v = 0.f;
        if (col < vocab && c != 0.f) v = c * (__expf(z[q] - L) - (col == t ? 1.f : 0.f));
        o[q] = from_f32<T>(v);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<t8*>(dz + row * ld + c0));
}

// A workgroup takes 2048 columns of one row per item, items row-major.
template <typename T>
__global__ __launch_bounds__(256) void ce_grad_saved_kernel(const float* __restrict__ logits, int64_t ld, int rows,
                                                            const float* __restrict__ coef,
                                                            const float* __restrict__ lse,
                                                            const int32_t* __restrict__ targets, int vocab,
                                                            T* __restrict__ dz) {
    const int64_t chunks = (ld + 2047) / 2048, items = (int64_t)rows * chunks;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t row = item / chunks;
        const int64_t c0 = (item - row * chunks) * 2048 + (int64_t)threadIdx.x * 8;
        if (c0 < ld) ce_grad_saved_run<T>(logits, ld, coef, lse, targets, vocab, dz, row, c0);
    }
}

// D = sum of m w over the rows that count (fp64, fixed order as the forward's
// loss), then per row coef = d_loss m w / D and lse = row_ce + zt.
__global__ __launch_bounds__(1024) void ce_grad_rows_kernel(const float* row_ce, const float* zt,
                                                            const int32_t* targets, const uint8_t* loss_mask, int rows,
                                                            int vocab, int bs, double tau, double d_loss, float* coef,
                                                            float* lse) {
    const int tid = threadIdx.x;
    __shared__ double s_d[1024];
    double den = 0.0;
    for (int r = tid; r < rows; r += 1024) {
        const int t = targets[r];
        if (loss_mask[r] == 0 || t < 0 || t >= vocab) continue;
        den += exp(-((double)(r % bs) - 1.0) / tau);
    }
    s_d[tid] = den;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (tid < o) s_d[tid] += s_d[tid + o];
        __syncthreads();
    }
    const double D = s_d[0];
    for (int r = tid; r < rows; r += 1024) {
        const int t = targets[r];
        const bool use = D > 0.0 && loss_mask[r] != 0 && t >= 0 && t < vocab;
        coef[r] = use ? (float)(d_loss * exp(-((double)(r % bs) - 1.0) / tau) / D) : 0.f;
        lse[r] = use ? row_ce[r] + zt[r] : 0.f;
    }
}

// Workspace (256-byte aligned): zt, coef, lse [rows] f32; dz [rows][Vp];
// W_lm^T [H][Vp] (config dtype), Vp = vocab rounded up to 64.
struct LmBwdLayout {
    size_t zt, coef, lse, dz, wt, total;
    int64_t vp;
};
LmBwdLayout lm_bwd_layout(const dflash_config& c, int64_t rows, int64_t vocab) {
    LmBwdLayout l{};
    const size_t A = 256, eb = (size_t)elem_bytes(c);
    l.vp = lm_logits_ld((int)vocab);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, A);
        return o;
    };
    l.zt = take(4 * (size_t)rows);
    l.coef = take(4 * (size_t)rows);
    l.lse = take(4 * (size_t)rows);
    l.dz = take(eb * (size_t)rows * (size_t)l.vp);
    l.wt = take(eb * (size_t)c.hidden * (size_t)l.vp);
    l.total = off + A;
    return l;
}

// W_lm^T [H][Vp] with zero columns for the padded vocabulary.
template <typename T>
void head_transpose(const T* W, int vocab, int H, int64_t Vp, T* wt, hipStream_t st) {
    hipLaunchKernelGGL((transpose_kernel<T, SrcPlain<T>>), dim3((unsigned)(Vp / 64), (unsigned)(H / 64)), dim3(256), 0,
                       st, SrcPlain<T>{W, H}, (int64_t)vocab, Vp, (int64_t)H, wt, Vp);
}

template <typename T>
hipError_t lm_bwd_t(const dflash_config& c, int rows, const T* hidden, const T* W, const T* W_t, int vocab,
                    const int32_t* targets, const uint8_t* loss_mask, double tau, const float* row_ce, double d_loss,
                    T* d_hidden, char* ws, hipStream_t st) {
    const LmBwdLayout lay = lm_bwd_layout(c, rows, vocab);
    const int H = c.hidden;
    const int64_t Vp = lay.vp;
    float* zt = reinterpret_cast<float*>(ws + lay.zt);
    float* coef = reinterpret_cast<float*>(ws + lay.coef);
    float* lse = reinterpret_cast<float*>(ws + lay.lse);
    T* dz = reinterpret_cast<T*>(ws + lay.dz);
    const T* wt = W_t != nullptr ? W_t : reinterpret_cast<T*>(ws + lay.wt);
    {
        ProfScope prof(DFLASH_KERNEL_LM_BWD_PREP, st);
        hipLaunchKernelGGL(target_logit_kernel<T>, dim3(rows), dim3(256), 0, st, hidden, W, targets, H, vocab, zt);
        hipLaunchKernelGGL(ce_grad_rows_kernel, dim3(1), dim3(1024), 0, st, row_ce, zt, targets, loss_mask, rows, vocab,
                           c.block_size, tau, d_loss, coef, lse);
        if (W_t == nullptr) head_transpose(W, vocab, H, Vp, reinterpret_cast<T*>(ws + lay.wt), st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(DFLASH_KERNEL_LM_BWD_DZ, st);
        const EpCEGrad<T> ep{dz, Vp, coef, lse, targets, vocab};
        const int big_tiles = ((rows + 255) / 256) * ((vocab + 255) / 256);
        if (big_tiles >= 256)
            e = launch_gemm<T, BigTile>(rows, vocab, H, APlain<T>{hidden, H}, BClamp<T>{W, H, vocab}, ep, st);
        else
            e = launch_gemm<T, MidTile>(rows, vocab, H, APlain<T>{hidden, H}, BClamp<T>{W, H, vocab}, ep, st);
    }
    if (e != hipSuccess) return e;
    return gemm<T>(DFLASH_KERNEL_LM_BWD_DH, rows, H, (int)Vp, APlain<T>{dz, Vp}, BPlain<T>{wt, Vp},
                   EpStore<T>{d_hidden, H}, st);
}

// The same gradient from the logits dflash_lm_head_ce_train kept: the row
// statistics read the target logit from them, dz is one elementwise pass, and
// only the second product remains.
template <typename T>
hipError_t lm_bwd_saved_t(const dflash_config& c, int rows, const float* logits, const T* W, const T* W_t, int vocab,
                          const int32_t* targets, const uint8_t* loss_mask, double tau, const float* row_ce,
                          double d_loss, T* d_hidden, char* ws, hipStream_t st) {
    const LmBwdLayout lay = lm_bwd_layout(c, rows, vocab);
    const int H = c.hidden;
    const int64_t Vp = lay.vp;
    float* zt = reinterpret_cast<float*>(ws + lay.zt);
    float* coef = reinterpret_cast<float*>(ws + lay.coef);
    float* lse = reinterpret_cast<float*>(ws + lay.lse);
    T* dz = reinterpret_cast<T*>(ws + lay.dz);
    const T* wt = W_t != nullptr ? W_t : reinterpret_cast<T*>(ws + lay.wt);
    {
        ProfScope prof(DFLASH_KERNEL_LM_BWD_PREP, st);
        hipLaunchKernelGGL(saved_target_logit_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, logits,
                           Vp, targets, rows, vocab, zt);
        hipLaunchKernelGGL(ce_grad_rows_kernel, dim3(1), dim3(1024), 0, st, row_ce, zt, targets, loss_mask, rows, vocab,
                           c.block_size, tau, d_loss, coef, lse);
        if (W_t == nullptr) head_transpose(W, vocab, H, Vp, reinterpret_cast<T*>(ws + lay.wt), st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(DFLASH_KERNEL_LM_BWD_DZ, st);
        const int64_t items = (int64_t)rows * ((Vp + 2047) / 2048);
        hipLaunchKernelGGL(ce_grad_saved_kernel<T>, dim3((unsigned)(items < (1 << 20) ? items : (1 << 20))), dim3(256),
                           0, st, logits, Vp, rows, coef, lse, targets, vocab, dz);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    return gemm<T>(DFLASH_KERNEL_LM_BWD_DH, rows, H, (int)Vp, APlain<T>{dz, Vp}, BPlain<T>{wt, Vp},
                   EpStore<T>{d_hidden, H}, st);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_lm_head_ce_backward_workspace_size(const dflash_config* cfg, int32_t rows, int32_t vocab) {
    if (check_config(cfg) != DFLASH_OK || rows < 0 || vocab < 1 || (int64_t)vocab + 255 > INT32_MAX) return 0;
    return lm_bwd_layout(*cfg, rows, vocab).total;
}

// A kept transposed head (dflash_lm_head_transpose): null, or 16-byte aligned and large enough.
static dflash_status head_t_check(const dflash_config* cfg, int32_t vocab, const void* lm_head_t,
                                  size_t lm_head_t_bytes) {
    if (lm_head_t == nullptr) return DFLASH_OK;
    const size_t need = (size_t)elem_bytes(*cfg) * (size_t)cfg->hidden * (size_t)lm_logits_ld(vocab);
    return aligned16(lm_head_t) && lm_head_t_bytes >= need ? DFLASH_OK : DFLASH_ERR_INVALID_ARG;
}

extern "C" size_t dflash_lm_head_transpose_size(const dflash_config* cfg, int32_t vocab) {
    if (check_config(cfg) != DFLASH_OK || vocab < 1 || (int64_t)vocab + 255 > INT32_MAX) return 0;
    return (size_t)elem_bytes(*cfg) * (size_t)cfg->hidden * (size_t)lm_logits_ld(vocab);
}

extern "C" dflash_status dflash_lm_head_transpose(const dflash_config* cfg, const void* lm_head, int32_t vocab,
                                                  void* lm_head_t, size_t lm_head_t_bytes, void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (vocab < 1) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)vocab + 255 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (lm_head == nullptr || lm_head_t == nullptr || !aligned16(lm_head) ||
        head_t_check(cfg, vocab, lm_head_t, lm_head_t_bytes) != DFLASH_OK)
        return DFLASH_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    const int64_t Vp = lm_logits_ld(vocab);
    ProfScope prof(DFLASH_KERNEL_LM_BWD_PREP, st);
    if (cfg->dtype == DFLASH_BF16)
        head_transpose(static_cast<const __bf16*>(lm_head), vocab, cfg->hidden, Vp, static_cast<__bf16*>(lm_head_t),
                       st);
    else
        head_transpose(static_cast<const float*>(lm_head), vocab, cfg->hidden, Vp, static_cast<float*>(lm_head_t), st);
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

extern "C" dflash_status dflash_lm_head_ce_backward(const dflash_config* cfg, int32_t rows, const void* hidden,
                                                    const void* lm_head, const void* lm_head_t,
                                                    size_t lm_head_t_bytes, int32_t vocab, const int32_t* targets,
                                                    const uint8_t* loss_mask, double decay_tau, const float* row_ce,
                                                    double d_loss, void* d_hidden, void* workspace,
                                                    size_t workspace_bytes, void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (rows < 0 || vocab < 1 || !(decay_tau > 0.0)) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)vocab + 255 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (rows == 0) return DFLASH_OK;
    if (hidden == nullptr || lm_head == nullptr || targets == nullptr || loss_mask == nullptr || row_ce == nullptr ||
        d_hidden == nullptr || !aligned16(hidden) || !aligned16(lm_head) || !aligned16(d_hidden) ||
        head_t_check(cfg, vocab, lm_head_t, lm_head_t_bytes) != DFLASH_OK)
        return DFLASH_ERR_INVALID_ARG;
    const size_t need = lm_bwd_layout(*cfg, rows, vocab).total;
    if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DFLASH_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = lm_bwd_t<__bf16>(*cfg, rows, static_cast<const __bf16*>(hidden), static_cast<const __bf16*>(lm_head),
                             static_cast<const __bf16*>(lm_head_t), vocab, targets, loss_mask, decay_tau, row_ce,
                             d_loss, static_cast<__bf16*>(d_hidden), ws, st);
    else
        e = lm_bwd_t<float>(*cfg, rows, static_cast<const float*>(hidden), static_cast<const float*>(lm_head),
                            static_cast<const float*>(lm_head_t), vocab, targets, loss_mask, decay_tau, row_ce, d_loss,
                            static_cast<float*>(d_hidden), ws, st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

extern "C" dflash_status dflash_lm_head_ce_backward_saved(const dflash_config* cfg, int32_t rows, const float* logits,
                                                          size_t logits_bytes, const void* lm_head,
                                                          const void* lm_head_t, size_t lm_head_t_bytes,
                                                          int32_t vocab, const int32_t* targets,
                                                          const uint8_t* loss_mask, double decay_tau,
                                                          const float* row_ce, double d_loss, void* d_hidden,
                                                          void* workspace, size_t workspace_bytes, void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (rows < 0 || vocab < 1 || !(decay_tau > 0.0)) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)vocab + 255 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (rows == 0) return DFLASH_OK;
    if (logits == nullptr || logits_bytes < (size_t)rows * (size_t)lm_logits_ld(vocab) * sizeof(float) ||
        lm_head == nullptr || targets == nullptr || loss_mask == nullptr || row_ce == nullptr || d_hidden == nullptr ||
        !aligned16(logits) || !aligned16(lm_head) || !aligned16(d_hidden) ||
        head_t_check(cfg, vocab, lm_head_t, lm_head_t_bytes) != DFLASH_OK)
        return DFLASH_ERR_INVALID_ARG;
    const size_t need = lm_bwd_layout(*cfg, rows, vocab).total;
    if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DFLASH_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = lm_bwd_saved_t<__bf16>(*cfg, rows, logits, static_cast<const __bf16*>(lm_head),
                                   static_cast<const __bf16*>(lm_head_t), vocab, targets, loss_mask, decay_tau, row_ce,
                                   d_loss, static_cast<__bf16*>(d_hidden), ws, st);
    else
        e = lm_bwd_saved_t<float>(*cfg, rows, logits, static_cast<const float*>(lm_head),
                                  static_cast<const float*>(lm_head_t), vocab, targets, loss_mask, decay_tau, row_ce,
                                  d_loss, static_cast<float*>(d_hidden), ws, st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
