// libdflash entry points: argument checks, workspace carving and launch
// sequencing for the context projection, the dual-source block attention and
// the draft body. All arithmetic happens in the kernels of gemm.h,
// attention.h and the RMSNorm kernel below.
#include <string.h>

#include <mutex>

#include "attn_launch.h"
#include "common.h"
#include "gemm.h"
#include "gemm_select.h"
#include "internal.h"
#include "norm.h"

namespace dflash {

// ------------------------------------------------------------------ typed bodies
template <typename T>
static hipError_t ctx_proj_t(const dflash_config& c, const T* ts, int64_t rs, int64_t ls, int64_t rows,
                             const int32_t* positions, const T* w_proj, const dflash_layer_weights* layers,
                             void* const* ck, void* const* cv, int64_t ctx_total, int64_t row_offset,
                             const int64_t* dst_rows, T* C, hipStream_t st) {
    const int H = c.hidden, K = c.num_target_layers * c.target_hidden;
    const int M = (int)rows;
    hipError_t e = gemm<T>(DFLASH_KERNEL_CTX_PROJ, M, H, K, AStacked<T>{ts, rs, ls, c.target_hidden}, BPlain<T>{w_proj, K},
                           EpStore<T>{C, H}, st, 4);
    if (e != hipSuccess) return e;
    BCtxKV<T> b{};
    EpCtxKV<T> ep{};
    for (int l = 0; l < c.num_layers; ++l) {
        b.wk[l] = static_cast<const T*>(layers[l].wk);
        b.wv[l] = static_cast<const T*>(layers[l].wv);
        ep.ck[l] = static_cast<T*>(ck[l]);
        ep.cv[l] = static_cast<T*>(cv[l]);
    }
    b.hkvd = c.num_kv_heads * c.head_dim;
    b.ld = H;
    ep.positions = positions;
    ep.dst_rows = dst_rows;
    ep.ctx_total = ctx_total;
    ep.row_offset = row_offset;
    ep.hkv = c.num_kv_heads;
    ep.rt = make_rope_turns(c);
    const int N = c.num_layers * 2 * c.num_kv_heads * c.head_dim;
    return gemm<T>(DFLASH_KERNEL_CTX_KV, M, N, H, APlain<T>{C, H}, b, ep, st);
}

// reserve (optional): the training reserve space (train_reserve_layout). With
// it, every layer's input residual and activations are written there and kept:
// layer l reads h_l, writes h1_l = h_l + attention and h_{l+1} = h1_l + MLP to
// new buffers, keeps the SwiGLU pre-activations, and stores q, k, v unpacked.
// The arithmetic is the same either way, so `out` is bit-identical.
template <typename T>
static hipError_t body_t(const dflash_config& c, int nb, const T* emb, const dflash_layer_weights* layers,
                         void* const* ck, void* const* cv, int64_t ctx_total, const int64_t* base,
                         const int32_t* anchor, const uint8_t* valid, T* out, char* reserve, char* ws,
                         hipStream_t st) {
    const Workspace w = workspace_layout(c, nb, 0);
    const TrainReserve tr = train_reserve_layout(c, nb);
    const int R = nb * c.block_size, H = c.hidden, D = c.head_dim;
    const int nq = c.num_q_heads * D, nk = c.num_kv_heads * D, nqkv = nq + 2 * nk, I = c.intermediate;
    float* h = reinterpret_cast<float*>(ws + w.h);
    hipError_t e = attn_schedule(c, nb, base, anchor, ctx_total, ws, w, st);
    if (e != hipSuccess) return e;
    const int64_t RH = (int64_t)R * H;
    for (int l = 0; l < c.num_layers; ++l) {
        const dflash_layer_weights& L = layers[l];
        const bool last = l + 1 == c.num_layers;
        char* lb = reserve ? reserve + tr.layer0 + (size_t)l * tr.per_layer : nullptr;
        auto at = [&](size_t off_r, size_t off_w) { return reserve ? lb + off_r : ws + off_w; };
        float* hin = reserve ? reinterpret_cast<float*>(reserve) + l * RH : h;     // residual entering layer l
        float* h1 = reserve ? reinterpret_cast<float*>(lb + tr.h1) : h;             // ... after attention
        float* hout = reserve && !last ? reinterpret_cast<float*>(reserve) + (l + 1) * RH : h;
        T* x = reinterpret_cast<T*>(at(tr.x, w.x));
        T* y = reinterpret_cast<T*>(at(tr.y, w.x));
        T* q = reinterpret_cast<T*>(at(tr.q, w.qkv));
        T* k = reserve ? reinterpret_cast<T*>(lb + tr.k) : q + nq;
        T* v = reserve ? reinterpret_cast<T*>(lb + tr.v) : q + nq + nk;
        const int q_ld = reserve ? nq : nqkv, kv_ld = reserve ? nk : nqkv;
        T* att = reinterpret_cast<T*>(at(tr.o, w.att));
        T* u = reinterpret_cast<T*>(at(tr.u, w.u));
        {
            ProfScope prof(DFLASH_KERNEL_RMSNORM, st);
            if (l == 0)
                hipLaunchKernelGGL((rmsnorm_kernel<T, T>), dim3(R), dim3(256), 0, st, emb, hin,
                                   static_cast<const T*>(L.attn_norm), x, H, c.rms_eps);
            else
                hipLaunchKernelGGL((rmsnorm_kernel<float, T>), dim3(R), dim3(256), 0, st, hin, (float*)nullptr,
                                   static_cast<const T*>(L.attn_norm), x, H, c.rms_eps);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const BQKV<T> bqkv{static_cast<const T*>(L.wq), static_cast<const T*>(L.wk), static_cast<const T*>(L.wv),
                           nq, nk, H};
        e = reserve ? gemm<T>(DFLASH_KERNEL_QKV, R, nqkv, H, APlain<T>{x, H}, bqkv, EpSplitQKV<T>{q, k, v, nq, nk}, st)
                    : gemm<T>(DFLASH_KERNEL_QKV, R, nqkv, H, APlain<T>{x, H}, bqkv, EpStore<T>{q, nqkv}, st);
        if (e != hipSuccess) return e;
        // Inside the body every row keeps its attention output (invalid rows
        // evolve like the others); only the returned rows are zeroed.
        AttnArgs<T> a = attn_args<T>(c, nb, q, q_ld, k, v, kv_ld, static_cast<const T*>(ck[l]),
                                     static_cast<const T*>(cv[l]), ctx_total, base, anchor, nullptr, att, nq, ws, w);
        if ((e = attn_launch<T>(c, a, nb, st)) != hipSuccess) return e;
        const BPlain<T> bo{static_cast<const T*>(L.wo), nq};
        e = reserve ? gemm<T>(DFLASH_KERNEL_O_PROJ, R, H, nq, APlain<T>{att, nq}, bo, EpAddF32{hin, h1, H}, st)
                    : gemm<T>(DFLASH_KERNEL_O_PROJ, R, H, nq, APlain<T>{att, nq}, bo,
                              EpResidual<T>{h, H, nullptr, nullptr, nullptr, 0}, st);
        if (e != hipSuccess) return e;
        {
            ProfScope prof(DFLASH_KERNEL_RMSNORM, st);
            hipLaunchKernelGGL((rmsnorm_kernel<float, T>), dim3(R), dim3(256), 0, st, h1, (float*)nullptr,
                               static_cast<const T*>(L.mlp_norm), y, H, c.rms_eps);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const BGateUp<T, 128> bgu{static_cast<const T*>(L.w_gate), static_cast<const T*>(L.w_up), H};
        e = reserve ? gemm<T>(DFLASH_KERNEL_GATE_UP, R, 2 * I, H, APlain<T>{y, H}, bgu,
                              EpSwiGLUSave<T>{u, reinterpret_cast<float*>(lb + tr.gate),
                                              reinterpret_cast<float*>(lb + tr.up), I},
                              st)
                    : gemm<T>(DFLASH_KERNEL_GATE_UP, R, 2 * I, H, APlain<T>{y, H}, bgu, EpSwiGLU<T>{u, I}, st);
        if (e != hipSuccess) return e;
        const BPlain<T> bd{static_cast<const T*>(L.w_down), I};
        if (last)   // out = h1 + MLP on the returned rows; h1 is only read
            e = gemm<T>(DFLASH_KERNEL_DOWN, R, H, I, APlain<T>{u, I}, bd,
                        EpResidual<T>{h1, H, out, valid, anchor, c.block_size}, st);
        else if (reserve)
            e = gemm<T>(DFLASH_KERNEL_DOWN, R, H, I, APlain<T>{u, I}, bd, EpAddF32{h1, hout, H}, st);
        else
            e = gemm<T>(DFLASH_KERNEL_DOWN, R, H, I, APlain<T>{u, I}, bd,
                        EpResidual<T>{h, H, nullptr, valid, anchor, c.block_size}, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------------------ checks
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dflash_status check_config(const dflash_config* c) {
    if (c == nullptr) return DFLASH_ERR_INVALID_ARG;
    if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return DFLASH_ERR_INVALID_ARG;
    if (c->hidden <= 0 || c->num_q_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 ||
        c->intermediate <= 0 || c->num_layers <= 0 || c->num_target_layers <= 0 || c->target_hidden <= 0 ||
        c->block_size <= 0 || !(c->rope_theta > 0.0) || !(c->rms_eps >= 0.f))
        return DFLASH_ERR_INVALID_ARG;
    if (c->num_q_heads % c->num_kv_heads != 0) return DFLASH_ERR_INVALID_ARG;
    const int eb = elem_bytes(*c), bk = 128 / eb;
    if (c->head_dim * eb != 256) return DFLASH_ERR_UNSUPPORTED;
    if (c->block_size * (c->num_q_heads / c->num_kv_heads) > 64) return DFLASH_ERR_UNSUPPORTED;
    if (c->num_layers > kMaxLayers) return DFLASH_ERR_UNSUPPORTED;
    if (c->hidden % 128 != 0 || c->intermediate % 64 != 0 || c->target_hidden % bk != 0) return DFLASH_ERR_UNSUPPORTED;
    if (((int64_t)c->num_q_heads + 2 * c->num_kv_heads) * c->head_dim % 128 != 0) return DFLASH_ERR_UNSUPPORTED;
    if ((int64_t)c->num_target_layers * c->target_hidden > INT32_MAX / 2) return DFLASH_ERR_UNSUPPORTED;
    return DFLASH_OK;
}

}  // namespace dflash

using namespace dflash;

extern "C" dflash_status dflash_check_config(const dflash_config* cfg) { return check_config(cfg); }

extern "C" const char* dflash_status_string(dflash_status s) {
    switch (s) {
        case DFLASH_OK: return "ok";
        case DFLASH_ERR_INVALID_ARG: return "invalid argument";
        case DFLASH_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case DFLASH_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case DFLASH_ERR_HIP: return "HIP launch or runtime error";
        case DFLASH_ERR_SCRATCH_LIMIT:
            return "input larger than the allocation-free entry point's static scratch (32 MiB)";
    }
    return "unknown status";
}

extern "C" size_t dflash_workspace_size(const dflash_config* cfg, int32_t num_blocks, int64_t ctx_rows) {
    if (check_config(cfg) != DFLASH_OK || num_blocks < 0 || ctx_rows < 0) return 0;
    return workspace_layout(*cfg, num_blocks, ctx_rows).total;
}

static dflash_status ws_check(const dflash_config* c, int nb, int64_t rows, void* ws, size_t bytes) {
    const size_t need = workspace_layout(*c, nb, rows).total;
    if (ws == nullptr || bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return DFLASH_ERR_WORKSPACE;
    return DFLASH_OK;
}

static dflash_status ctx_proj_entry(const dflash_config* cfg, const void* target_states, int64_t ts_row_stride,
                                    int64_t ts_layer_stride, int64_t num_rows, const int32_t* positions,
                                    const void* w_proj, const dflash_layer_weights* layers, void* const* ctx_k,
                                    void* const* ctx_v, int64_t ctx_total, int64_t row_offset, void* keep_c,
                                    void* workspace, size_t workspace_bytes, void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (num_rows < 0 || ctx_total < 0 || row_offset < 0 || row_offset + num_rows > ctx_total)
        return DFLASH_ERR_INVALID_ARG;
    if (num_rows > INT32_MAX / 2) return DFLASH_ERR_UNSUPPORTED;
    if (num_rows == 0) return DFLASH_OK;
    const int64_t vec = 16 / elem_bytes(*cfg);
    if (target_states == nullptr || positions == nullptr || w_proj == nullptr || layers == nullptr ||
        ctx_k == nullptr || ctx_v == nullptr || !aligned16(target_states) || !aligned16(w_proj) ||
        !aligned16(keep_c) || ts_row_stride <= 0 || ts_layer_stride < 0 || ts_row_stride % vec != 0 ||
        ts_layer_stride % vec != 0)
        return DFLASH_ERR_INVALID_ARG;
    for (int l = 0; l < cfg->num_layers; ++l)
        if (layers[l].wk == nullptr || layers[l].wv == nullptr || ctx_k[l] == nullptr || ctx_v[l] == nullptr ||
            !aligned16(layers[l].wk) || !aligned16(layers[l].wv))
            return DFLASH_ERR_INVALID_ARG;
    if ((s = ws_check(cfg, 0, num_rows, workspace, workspace_bytes)) != DFLASH_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    void* C = keep_c != nullptr ? keep_c : ws + workspace_layout(*cfg, 0, num_rows).c;
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = ctx_proj_t<__bf16>(*cfg, static_cast<const __bf16*>(target_states), ts_row_stride, ts_layer_stride,
                               num_rows, positions, static_cast<const __bf16*>(w_proj), layers, ctx_k, ctx_v,
                               ctx_total, row_offset, nullptr, static_cast<__bf16*>(C), st);
    else
        e = ctx_proj_t<float>(*cfg, static_cast<const float*>(target_states), ts_row_stride, ts_layer_stride,
                              num_rows, positions, static_cast<const float*>(w_proj), layers, ctx_k, ctx_v,
                              ctx_total, row_offset, nullptr, static_cast<float*>(C), st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

extern "C" dflash_status dflash_ctx_proj(const dflash_config* cfg, const void* target_states,
                                         int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                                         const int32_t* positions, const void* w_proj,
                                         const dflash_layer_weights* layers, void* const* ctx_k,
                                         void* const* ctx_v, int64_t ctx_total, int64_t row_offset,
                                         void* workspace, size_t workspace_bytes, void* hip_stream) {
    return ctx_proj_entry(cfg, target_states, ts_row_stride, ts_layer_stride, num_rows, positions, w_proj, layers,
                          ctx_k, ctx_v, ctx_total, row_offset, nullptr, workspace, workspace_bytes, hip_stream);
}

extern "C" dflash_status dflash_ctx_proj_train(const dflash_config* cfg, const void* target_states,
                                               int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                                               const int32_t* positions, const void* w_proj,
                                               const dflash_layer_weights* layers, void* const* ctx_k,
                                               void* const* ctx_v, int64_t ctx_total, int64_t row_offset,
                                               void* ctx_hidden, void* workspace, size_t workspace_bytes,
                                               void* hip_stream) {
    if (num_rows > 0 && ctx_hidden == nullptr) return DFLASH_ERR_INVALID_ARG;
    return ctx_proj_entry(cfg, target_states, ts_row_stride, ts_layer_stride, num_rows, positions, w_proj, layers,
                          ctx_k, ctx_v, ctx_total, row_offset, ctx_hidden, workspace, workspace_bytes, hip_stream);
}

// Host-side checks shared by dflash_ctx_append and its allocation-free variant.
static dflash_status ctx_append_check(const dflash_config* cfg, const void* target_states, int64_t ts_row_stride,
                                      int64_t ts_layer_stride, int64_t num_rows, const int32_t* positions,
                                      const int64_t* dst_rows, const void* w_proj,
                                      const dflash_layer_weights* layers, void* const* ctx_k, void* const* ctx_v,
                                      int64_t ctx_total) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (num_rows < 0 || ctx_total < 0) return DFLASH_ERR_INVALID_ARG;
    if (num_rows > INT32_MAX / 2) return DFLASH_ERR_UNSUPPORTED;
    if (num_rows == 0) return DFLASH_OK;
    const int64_t vec = 16 / elem_bytes(*cfg);
    if (target_states == nullptr || positions == nullptr || dst_rows == nullptr || w_proj == nullptr ||
        layers == nullptr || ctx_k == nullptr || ctx_v == nullptr || !aligned16(target_states) ||
        !aligned16(w_proj) || ts_row_stride <= 0 || ts_layer_stride < 0 || ts_row_stride % vec != 0 ||
        ts_layer_stride % vec != 0)
        return DFLASH_ERR_INVALID_ARG;
    for (int l = 0; l < cfg->num_layers; ++l)
        if (layers[l].wk == nullptr || layers[l].wv == nullptr || ctx_k[l] == nullptr || ctx_v[l] == nullptr ||
            !aligned16(layers[l].wk) || !aligned16(layers[l].wv))
            return DFLASH_ERR_INVALID_ARG;
    return DFLASH_OK;
}

static dflash_status ctx_append_run(const dflash_config* cfg, const void* target_states, int64_t ts_row_stride,
                                    int64_t ts_layer_stride, int64_t num_rows, const int32_t* positions,
                                    const int64_t* dst_rows, const void* w_proj, const dflash_layer_weights* layers,
                                    void* const* ctx_k, void* const* ctx_v, int64_t ctx_total, void* C,
                                    hipStream_t st) {
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = ctx_proj_t<__bf16>(*cfg, static_cast<const __bf16*>(target_states), ts_row_stride, ts_layer_stride,
                               num_rows, positions, static_cast<const __bf16*>(w_proj), layers, ctx_k, ctx_v,
                               ctx_total, 0, dst_rows, static_cast<__bf16*>(C), st);
    else
        e = ctx_proj_t<float>(*cfg, static_cast<const float*>(target_states), ts_row_stride, ts_layer_stride,
                              num_rows, positions, static_cast<const float*>(w_proj), layers, ctx_k, ctx_v,
                              ctx_total, 0, dst_rows, static_cast<float*>(C), st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

extern "C" dflash_status dflash_ctx_append(const dflash_config* cfg, const void* target_states,
                                           int64_t ts_row_stride, int64_t ts_layer_stride, int64_t num_rows,
                                           const int32_t* positions, const int64_t* dst_rows, const void* w_proj,
                                           const dflash_layer_weights* layers, void* const* ctx_k,
                                           void* const* ctx_v, int64_t ctx_total, void* workspace,
                                           size_t workspace_bytes, void* hip_stream) {
    dflash_status s = ctx_append_check(cfg, target_states, ts_row_stride, ts_layer_stride, num_rows, positions,
                                       dst_rows, w_proj, layers, ctx_k, ctx_v, ctx_total);
    if (s != DFLASH_OK || num_rows == 0) return s;
    if ((s = ws_check(cfg, 0, num_rows, workspace, workspace_bytes)) != DFLASH_OK) return s;
    char* C = static_cast<char*>(workspace) + workspace_layout(*cfg, 0, num_rows).c;
    return ctx_append_run(cfg, target_states, ts_row_stride, ts_layer_stride, num_rows, positions, dst_rows, w_proj,
                          layers, ctx_k, ctx_v, ctx_total, C, reinterpret_cast<hipStream_t>(hip_stream));
}

// ------------------------------------------------------------------ allocation-free context append
// The projected rows C of dflash_ctx_append_noalloc live in this array. In
// host code its name is only a host-side stand-in: the device address comes
// from hipGetSymbolAddress, looked up once per device (each GPU holds its own
// copy of the array at its own address) and kept in noalloc_scratch_ptr.
static __device__ __attribute__((aligned(256))) char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the current device's scratch array.
static dflash_status noalloc_scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DFLASH_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return DFLASH_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DFLASH_OK;
}

extern "C" dflash_status dflash_ctx_append_noalloc(const dflash_config* cfg, const void* target_states,
                                                   int64_t ts_row_stride, int64_t ts_layer_stride,
                                                   int64_t num_rows, const int32_t* positions,
                                                   const int64_t* dst_rows, const void* w_proj,
                                                   const dflash_layer_weights* layers, void* const* ctx_k,
                                                   void* const* ctx_v, int64_t ctx_total, void* hip_stream) {
    dflash_status s = ctx_append_check(cfg, target_states, ts_row_stride, ts_layer_stride, num_rows, positions,
                                       dst_rows, w_proj, layers, ctx_k, ctx_v, ctx_total);
    if (s != DFLASH_OK || num_rows == 0) return s;
    if ((uint64_t)num_rows * (uint64_t)cfg->hidden * (uint64_t)elem_bytes(*cfg) > DFLASH_NOALLOC_SCRATCH_BYTES)
        return DFLASH_ERR_SCRATCH_LIMIT;
    void* C = nullptr;
    if ((s = noalloc_scratch_ptr(&C)) != DFLASH_OK) return s;
    return ctx_append_run(cfg, target_states, ts_row_stride, ts_layer_stride, num_rows, positions, dst_rows, w_proj,
                          layers, ctx_k, ctx_v, ctx_total, C, reinterpret_cast<hipStream_t>(hip_stream));
}

// ------------------------------------------------------------------ LM head + decayed CE
// Per row: logsumexp from the per-group (max, sum) statistics in a fixed
// order (thread-strided groups, then a fixed tree), CE = lse - z[target];
// rows whose loss mask is 0 or whose target is outside the vocabulary get 0.
__global__ __launch_bounds__(256) void lm_ce_row_kernel(const float* part, int groups, const float* target_logit,
                                                        const int32_t* targets, const uint8_t* loss_mask, int vocab,
                                                        float* row_ce) {
    const int row = blockIdx.x, tid = threadIdx.x;
    __shared__ float s_m[4];
    __shared__ float s_s[4];
    const float* pr = part + (int64_t)row * groups * 2;
    float mx = -__builtin_inff();
    for (int g = tid; g < groups; g += 256) mx = fmaxf(mx, pr[2 * g]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((tid & 63) == 0) s_m[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float s = 0.f;
    for (int g = tid; g < groups; g += 256) s += pr[2 * g + 1] * __expf(pr[2 * g] - mx);
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if ((tid & 63) == 0) s_s[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
        const float tot = (s_s[0] + s_s[1]) + (s_s[2] + s_s[3]);
        const int t = targets[row];
        const bool use = loss_mask[row] != 0 && t >= 0 && t < vocab;
        row_ce[row] = use ? (mx + logf(tot)) - target_logit[row] : 0.f;
    }
}

// loss = sum(m w CE) / sum(m w), w = exp(-(k - 1) / tau), k = row % block_size,
// in fp64 with a fixed order; 0 when no row is selected.
__global__ __launch_bounds__(1024) void lm_ce_loss_kernel(const float* row_ce, const int32_t* targets,
                                                          const uint8_t* loss_mask, int rows, int vocab, int bs,
                                                          double tau, double* loss) {
    const int tid = threadIdx.x;
    __shared__ double s_n[1024], s_d[1024];
    double num = 0.0, den = 0.0;
    for (int r = tid; r < rows; r += 1024) {
        const int t = targets[r];
        if (loss_mask[r] == 0 || t < 0 || t >= vocab) continue;
        const double w = exp(-((double)(r % bs) - 1.0) / tau);
        num += w * (double)row_ce[r];
        den += w;
    }
    s_n[tid] = num;
    s_d[tid] = den;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (tid < o) {
            s_n[tid] += s_n[tid + o];
            s_d[tid] += s_d[tid + o];
        }
        __syncthreads();
    }
    if (tid == 0) *loss = s_d[0] > 0.0 ? s_n[0] / s_d[0] : 0.0;
}

static int lm_groups(int vocab) { return (vocab + 127) / 128; }   // WN = 128 in both tile shapes

extern "C" size_t dflash_lm_head_ce_workspace_size(int32_t rows, int32_t vocab) {
    if (rows < 0 || vocab < 1) return 0;
    const size_t part = align_up((size_t)rows * lm_groups(vocab) * 2 * sizeof(float), 256);
    const size_t tl = align_up((size_t)rows * sizeof(float), 256);
    return part + tl + 256;
}

extern "C" size_t dflash_lm_head_ce_logits_size(int32_t rows, int32_t vocab) {
    if (rows < 0 || vocab < 1 || (int64_t)vocab + 255 > INT32_MAX) return 0;
    return (size_t)rows * (size_t)lm_logits_ld(vocab) * sizeof(float);
}

template <typename T>
static hipError_t lm_head_ce_t(const dflash_config& c, int rows, const T* hidden, const T* lm_head, int vocab,
                               const int32_t* targets, const uint8_t* loss_mask, double tau, float* row_ce,
                               double* loss, float* logits, char* ws, hipStream_t st) {
    const int groups = lm_groups(vocab);
    float* part = reinterpret_cast<float*>(ws);
    float* tl = reinterpret_cast<float*>(ws + align_up((size_t)rows * groups * 2 * sizeof(float), 256));
    EpLseCE<T> ep{part, tl, targets, groups, vocab, logits, lm_logits_ld(vocab)};
    hipError_t e;
    {
        ProfScope prof(DFLASH_KERNEL_LM_HEAD, st);
        const int big_tiles = ((rows + 255) / 256) * ((vocab + 255) / 256);
        if (big_tiles >= 256)
            e = launch_gemm<T, BigTile>(rows, vocab, c.hidden, APlain<T>{hidden, c.hidden},
                                        BClamp<T>{lm_head, c.hidden, vocab}, ep, st);
        else
            e = launch_gemm<T, MidTile>(rows, vocab, c.hidden, APlain<T>{hidden, c.hidden},
                                        BClamp<T>{lm_head, c.hidden, vocab}, ep, st);
    }
    if (e != hipSuccess) return e;
    {
        ProfScope prof(DFLASH_KERNEL_LM_CE, st);
        hipLaunchKernelGGL(lm_ce_row_kernel, dim3(rows), dim3(256), 0, st, part, groups, tl, targets, loss_mask, vocab,
                           row_ce);
        hipLaunchKernelGGL(lm_ce_loss_kernel, dim3(1), dim3(1024), 0, st, row_ce, targets, loss_mask, rows, vocab,
                           c.block_size, tau, loss);
    }
    return hipGetLastError();
}

static dflash_status lm_head_ce_entry(const dflash_config* cfg, int32_t rows, const void* hidden,
                                      const void* lm_head, int32_t vocab, const int32_t* targets,
                                      const uint8_t* loss_mask, double decay_tau, float* row_ce, double* loss,
                                      float* logits, void* workspace, size_t workspace_bytes, void* hip_stream) {
    const size_t need = dflash_lm_head_ce_workspace_size(rows, vocab);
    if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DFLASH_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    if (rows == 0) {
        hipLaunchKernelGGL(lm_ce_loss_kernel, dim3(1), dim3(1024), 0, st, row_ce, targets, loss_mask, 0, vocab,
                           cfg->block_size, decay_tau, loss);
        return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
    }
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = lm_head_ce_t<__bf16>(*cfg, rows, static_cast<const __bf16*>(hidden), static_cast<const __bf16*>(lm_head),
                                 vocab, targets, loss_mask, decay_tau, row_ce, loss, logits, ws, st);
    else
        e = lm_head_ce_t<float>(*cfg, rows, static_cast<const float*>(hidden), static_cast<const float*>(lm_head),
                                vocab, targets, loss_mask, decay_tau, row_ce, loss, logits, ws, st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

static dflash_status lm_head_ce_check(const dflash_config* cfg, int32_t rows, const void* hidden,
                                      const void* lm_head, int32_t vocab, const int32_t* targets,
                                      const uint8_t* loss_mask, double decay_tau, const float* row_ce,
                                      const double* loss) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (rows < 0 || vocab < 1 || !(decay_tau > 0.0)) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)vocab + 255 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (hidden == nullptr && rows > 0) return DFLASH_ERR_INVALID_ARG;
    if (lm_head == nullptr || loss == nullptr || (rows > 0 && (targets == nullptr || loss_mask == nullptr ||
                                                               row_ce == nullptr)) ||
        !aligned16(hidden) || !aligned16(lm_head))
        return DFLASH_ERR_INVALID_ARG;
    return DFLASH_OK;
}

extern "C" dflash_status dflash_lm_head_ce(const dflash_config* cfg, int32_t rows, const void* hidden,
                                           const void* lm_head, int32_t vocab, const int32_t* targets,
                                           const uint8_t* loss_mask, double decay_tau, float* row_ce,
                                           double* loss, void* workspace, size_t workspace_bytes,
                                           void* hip_stream) {
    const dflash_status s = lm_head_ce_check(cfg, rows, hidden, lm_head, vocab, targets, loss_mask, decay_tau,
                                             row_ce, loss);
    if (s != DFLASH_OK) return s;
    return lm_head_ce_entry(cfg, rows, hidden, lm_head, vocab, targets, loss_mask, decay_tau, row_ce, loss, nullptr,
                            workspace, workspace_bytes, hip_stream);
}

extern "C" dflash_status dflash_lm_head_ce_train(const dflash_config* cfg, int32_t rows, const void* hidden,
                                                 const void* lm_head, int32_t vocab, const int32_t* targets,
                                                 const uint8_t* loss_mask, double decay_tau, float* row_ce,
                                                 double* loss, float* logits, size_t logits_bytes, void* workspace,
                                                 size_t workspace_bytes, void* hip_stream) {
    const dflash_status s = lm_head_ce_check(cfg, rows, hidden, lm_head, vocab, targets, loss_mask, decay_tau,
                                             row_ce, loss);
    if (s != DFLASH_OK) return s;
    if (rows > 0 && (logits == nullptr || logits_bytes < dflash_lm_head_ce_logits_size(rows, vocab) ||
                     !aligned16(logits)))
        return DFLASH_ERR_INVALID_ARG;
    return lm_head_ce_entry(cfg, rows, hidden, lm_head, vocab, targets, loss_mask, decay_tau, row_ce, loss, logits,
                            workspace, workspace_bytes, hip_stream);
}

// lengths[i] = min(lengths[i], max(keep[i], 0)).
__global__ __launch_bounds__(256) void ctx_truncate_kernel(int64_t* lengths, const int64_t* keep, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t k = keep[i] > 0 ? keep[i] : 0;
    if (k < lengths[i]) lengths[i] = k;
}

extern "C" dflash_status dflash_ctx_truncate(int64_t* lengths, const int64_t* keep, int32_t n, void* hip_stream) {
    if (n < 0) return DFLASH_ERR_INVALID_ARG;
    if (n == 0) return DFLASH_OK;
    if (lengths == nullptr || keep == nullptr) return DFLASH_ERR_INVALID_ARG;
    hipLaunchKernelGGL(ctx_truncate_kernel, dim3((n + 255) / 256), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), lengths, keep, (int)n);
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

extern "C" dflash_status dflash_block_attn(const dflash_config* cfg, int32_t num_blocks, const void* q,
                                           const void* k_blk, const void* v_blk, const void* ctx_k,
                                           const void* ctx_v, int64_t ctx_total, const int64_t* block_ctx_base,
                                           const int32_t* block_anchor, const uint8_t* block_valid, void* out,
                                           void* workspace, size_t workspace_bytes, void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (num_blocks < 0 || ctx_total < 0) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)num_blocks * cfg->block_size > INT32_MAX / 2) return DFLASH_ERR_UNSUPPORTED;
    if (num_blocks == 0) return DFLASH_OK;
    if (q == nullptr || k_blk == nullptr || v_blk == nullptr || block_ctx_base == nullptr ||
        block_anchor == nullptr || block_valid == nullptr || out == nullptr ||
        (ctx_total > 0 && (ctx_k == nullptr || ctx_v == nullptr)) || !aligned16(ctx_k) || !aligned16(ctx_v) ||
        !aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(out))
        return DFLASH_ERR_INVALID_ARG;
    if ((s = ws_check(cfg, num_blocks, 0, workspace, workspace_bytes)) != DFLASH_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    const Workspace w = workspace_layout(*cfg, num_blocks, 0);
    const int64_t nq = (int64_t)cfg->num_q_heads * cfg->head_dim, nk = (int64_t)cfg->num_kv_heads * cfg->head_dim;
    hipError_t e = attn_schedule(*cfg, num_blocks, block_ctx_base, block_anchor, ctx_total, ws, w, st);
    if (e == hipSuccess) {
        if (cfg->dtype == DFLASH_BF16) {
            using T = __bf16;
            e = attn_launch<T>(*cfg,
                               attn_args<T>(*cfg, num_blocks, static_cast<const T*>(q), nq, static_cast<const T*>(k_blk),
                                            static_cast<const T*>(v_blk), nk, static_cast<const T*>(ctx_k),
                                            static_cast<const T*>(ctx_v), ctx_total, block_ctx_base, block_anchor,
                                            block_valid, static_cast<T*>(out), nq, ws, w),
                               num_blocks, st);
        } else {
            using T = float;
            e = attn_launch<T>(*cfg,
                               attn_args<T>(*cfg, num_blocks, static_cast<const T*>(q), nq, static_cast<const T*>(k_blk),
                                            static_cast<const T*>(v_blk), nk, static_cast<const T*>(ctx_k),
                                            static_cast<const T*>(ctx_v), ctx_total, block_ctx_base, block_anchor,
                                            block_valid, static_cast<T*>(out), nq, ws, w),
                               num_blocks, st);
        }
    }
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

static dflash_status body_entry(const dflash_config* cfg, int32_t num_blocks, const void* block_embeds,
                                const dflash_layer_weights* layers, void* const* ctx_k, void* const* ctx_v,
                                int64_t ctx_total, const int64_t* block_ctx_base, const int32_t* block_anchor,
                                const uint8_t* block_valid, void* out, void* reserve, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (num_blocks < 0 || ctx_total < 0) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)num_blocks * cfg->block_size > INT32_MAX / 2) return DFLASH_ERR_UNSUPPORTED;
    if (num_blocks == 0) return DFLASH_OK;
    if (block_embeds == nullptr || layers == nullptr || ctx_k == nullptr || ctx_v == nullptr ||
        block_ctx_base == nullptr || block_anchor == nullptr || block_valid == nullptr || out == nullptr ||
        !aligned16(block_embeds))
        return DFLASH_ERR_INVALID_ARG;
    for (int l = 0; l < cfg->num_layers; ++l) {
        const dflash_layer_weights& L = layers[l];
        const void* ptrs[9] = {L.attn_norm, L.wq, L.wk, L.wv, L.wo, L.mlp_norm, L.w_gate, L.w_up, L.w_down};
        for (const void* p : ptrs)
            if (p == nullptr || !aligned16(p)) return DFLASH_ERR_INVALID_ARG;
        if ((ctx_total > 0 && (ctx_k[l] == nullptr || ctx_v[l] == nullptr)) || !aligned16(ctx_k[l]) ||
            !aligned16(ctx_v[l]))
            return DFLASH_ERR_INVALID_ARG;
    }
    if ((s = ws_check(cfg, num_blocks, 0, workspace, workspace_bytes)) != DFLASH_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    hipError_t e;
    if (cfg->dtype == DFLASH_BF16)
        e = body_t<__bf16>(*cfg, num_blocks, static_cast<const __bf16*>(block_embeds), layers, ctx_k, ctx_v,
                           ctx_total, block_ctx_base, block_anchor, block_valid, static_cast<__bf16*>(out),
                           static_cast<char*>(reserve), ws, st);
    else
        e = body_t<float>(*cfg, num_blocks, static_cast<const float*>(block_embeds), layers, ctx_k, ctx_v,
                          ctx_total, block_ctx_base, block_anchor, block_valid, static_cast<float*>(out),
                          static_cast<char*>(reserve), ws, st);
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

extern "C" dflash_status dflash_body_forward(const dflash_config* cfg, int32_t num_blocks, const void* block_embeds,
                                             const dflash_layer_weights* layers, void* const* ctx_k,
                                             void* const* ctx_v, int64_t ctx_total, const int64_t* block_ctx_base,
                                             const int32_t* block_anchor, const uint8_t* block_valid, void* out,
                                             void* workspace, size_t workspace_bytes, void* hip_stream) {
    return body_entry(cfg, num_blocks, block_embeds, layers, ctx_k, ctx_v, ctx_total, block_ctx_base, block_anchor,
                      block_valid, out, nullptr, workspace, workspace_bytes, hip_stream);
}

extern "C" size_t dflash_body_train_reserve_size(const dflash_config* cfg, int32_t num_blocks) {
    if (check_config(cfg) != DFLASH_OK || num_blocks < 0 || (int64_t)num_blocks * cfg->block_size > INT32_MAX / 2)
        return 0;
    return train_reserve_layout(*cfg, num_blocks).total;
}

extern "C" dflash_status dflash_body_forward_train(const dflash_config* cfg, int32_t num_blocks,
                                                   const void* block_embeds, const dflash_layer_weights* layers,
                                                   void* const* ctx_k, void* const* ctx_v, int64_t ctx_total,
                                                   const int64_t* block_ctx_base, const int32_t* block_anchor,
                                                   const uint8_t* block_valid, void* out, void* reserve,
                                                   size_t reserve_bytes, void* workspace, size_t workspace_bytes,
                                                   void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (num_blocks > 0 && (int64_t)num_blocks * cfg->block_size <= INT32_MAX / 2) {
        if (reserve == nullptr) return DFLASH_ERR_INVALID_ARG;
        if (reserve_bytes < train_reserve_layout(*cfg, num_blocks).total ||
            (reinterpret_cast<uintptr_t>(reserve) & 255u) != 0)
            return DFLASH_ERR_WORKSPACE;
    }
    return body_entry(cfg, num_blocks, block_embeds, layers, ctx_k, ctx_v, ctx_total, block_ctx_base, block_anchor,
                      block_valid, out, reserve, workspace, workspace_bytes, hip_stream);
}
