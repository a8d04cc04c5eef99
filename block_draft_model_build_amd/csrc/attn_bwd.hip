// Backward of the dual-source block attention (NeMo RL "DFlash Draft Body",
// How It Works, step 3, and Scope: training runs the body with an optimizer
// step). For one block, KV head g and query column c (head g*G + c/bs, row
// c % bs, rotated at anchor + row and scaled by 1/sqrt(D)):
//   s = q~ K~^T, p = softmax(s), o = p V,
//   dV = p^T dO, dp = dO V^T, ds = p (dp - rowsum(dO o)),
//   dq~ = ds K~, dK~ = ds^T q~,
// with dO zero on rows whose output the forward zeroes (invalid positions,
// empty blocks). dq and the block's own dk are rotated back (RoPE^T is the
// rotation by the opposite angle); context dK stays in the rotated frame the
// cache holds.
//
// First version, fp32 arithmetic on the vector units (no MFMA), deterministic:
//  * attn_bwd_query_kernel, one workgroup per (block, KV head): softmax
//    statistics (pass 1), then per 64-key chunk ds and p into LDS and the dq
//    sums over the chunk (pass 2); the block's own keys get their dk and dv
//    there (only their own queries read them). Writes q~, lse and
//    rowsum(dO o) for the second kernel.
//  * attn_bwd_ctx_kernel, one workgroup per (64-row context tile, KV head):
//    walks every block that reads the tile, in block order, and accumulates
//    the tile's dK and dV in registers: no atomics, fixed summation order.
#include "internal.h"
#include "attention.h"

namespace dflash {

namespace {

constexpr int kBwKeys = 64;     // keys per chunk (query kernel) and rows per tile (context kernel)

__global__ __launch_bounds__(256) void zero_fill_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}
constexpr int kBwThreads = 256;

template <typename T> struct BwArgs {
    const T *q, *kb, *vb;        // [nb*bs, Hq*D], [nb*bs, Hkv*D] x2 (un-rotated q, kb)
    int64_t q_ld, kv_ld;
    const T *ck, *cvt;           // [Hkv][ctx_total][D] rotated, [Hkv][D][ctx_total]
    int64_t ctx_total;
    const int64_t* base;
    const int32_t* anchor;
    const uint8_t* valid;
    const T *out, *dout;         // forward output and its gradient [nb*bs, Hq*D]
    float *dq, *dkb, *dvb;       // [nb*bs, Hq*D], [nb*bs, Hkv*D] x2
    float *dck, *dcv;            // [Hkv][ctx_total][D], [Hkv][D][ctx_total]
    float *qt, *lse, *delta;     // workspace: [nb][Hkv][64][D], [nb][Hkv][64] x2
    int nb, bs, hq, hkv;
    RopeTurns rt;
};

// LDS of both kernels: q~ and masked dO of one block (fp32), ds and p of a
// chunk (fp32, padded rows), K~ and V of a chunk (T, padded rows).
template <typename T, int D> struct BwLds {
    static constexpr int KP = D + (sizeof(T) == 2 ? 2 : 1);   // padded K/V row (elements)
    float q[64][D];
    float dout[64][D];
    float ds[kBwKeys][65];
    float p[kBwKeys][65];
    T k[kBwKeys][KP];
    T v[kBwKeys][KP];
    float red[4][64][2];
};

template <typename T, int D>
__device__ __forceinline__ void load_block_q(const BwArgs<T>& a, int n, int g, int amax, BwLds<T, D>& L, int C, int G,
                                             float scale) {
    // q~ = RoPE(q, anchor + row) * scale; columns past C are zero.
    for (int idx = threadIdx.x; idx < 64 * (D / 2); idx += kBwThreads) {
        const int c = idx / (D / 2), i = idx - c * (D / 2);
        float y1 = 0.f, y2 = 0.f;
        if (c < C && amax >= 0) {
            const int k = c % a.bs, hh = c / a.bs;
            const T* qr = a.q + (int64_t)(n * a.bs + k) * a.q_ld + (int64_t)(g * G + hh) * D;
            const float x1 = to_f32(qr[i]), x2 = to_f32(qr[i + D / 2]);
            float cs, sn;
            rope_cs(a.rt, i, amax + k, cs, sn);
            y1 = (x1 * cs - x2 * sn) * scale;
            y2 = (x2 * cs + x1 * sn) * scale;
        }
        L.q[c][i] = y1;
        L.q[c][i + D / 2] = y2;
    }
}

template <typename T, int D>
__device__ __forceinline__ void load_block_dout(const BwArgs<T>& a, int n, int g, bool live, BwLds<T, D>& L, int C,
                                                int G) {
    for (int idx = threadIdx.x; idx < 64 * D; idx += kBwThreads) {
        const int c = idx / D, d = idx - c * D;
        float v = 0.f;
        if (c < C && live) {
            const int k = c % a.bs, hh = c / a.bs, row = n * a.bs + k;
            if (a.valid[row] != 0) v = to_f32(a.dout[(int64_t)row * a.q_ld + (int64_t)(g * G + hh) * D + d]);
        }
        L.dout[c][d] = v;
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void attn_bwd_query_kernel(BwArgs<T> a) {
    __shared__ BwLds<T, D> L;
    const int n = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int G = a.hq / a.hkv, bs = a.bs, C = bs * G;
    const float scale = 1.f / sqrtf((float)D);
    const int64_t base = clamp_base(a.base[n], a.ctx_total);
    const int an = anchor_eff(a.anchor[n], base, a.ctx_total);
    const bool live = an >= 0;
    const int nkeys = live ? an + bs : 0;
    const T* ckg = a.ck + ((int64_t)g * a.ctx_total + base) * D;
    const T* cvg = a.cvt + (int64_t)g * D * a.ctx_total + base;

    load_block_q<T, D>(a, n, g, an, L, C, G, scale);
    load_block_dout<T, D>(a, n, g, live, L, C, G);
    __syncthreads();
    // rowsum(dO o) per column, and q~ for the context kernel.
    float* qt = a.qt + ((int64_t)n * a.hkv + g) * 64 * D;
    for (int idx = tid; idx < 64 * D; idx += kBwThreads) qt[idx] = (&L.q[0][0])[idx];
    if (tid < 64) {
        float s = 0.f;
        const int c = tid;
        if (c < C && live) {
            const int k = c % bs, hh = c / bs, row = n * bs + k;
            const T* orow = a.out + (int64_t)row * a.q_ld + (int64_t)(g * G + hh) * D;
            for (int d = 0; d < D; ++d) s += L.dout[c][d] * to_f32(orow[d]);
        }
        L.red[0][c][1] = s;
        a.delta[((int64_t)n * a.hkv + g) * 64 + c] = s;
    }

    // Stage keys [j0, j0 + 64): context rows before the anchor, then the
    // block's own rows rotated at anchor + row; zero past the block's keys.
    auto stage = [&](int j0) {
        for (int idx = tid; idx < kBwKeys * (D / 2); idx += kBwThreads) {
            const int kk = idx / (D / 2), i = idx - kk * (D / 2);
            const int j = j0 + kk;
            float k1 = 0.f, k2 = 0.f;
            if (j < an) {
                k1 = to_f32(ckg[(int64_t)j * D + i]);
                k2 = to_f32(ckg[(int64_t)j * D + i + D / 2]);
            } else if (j < nkeys) {
                const T* kr = a.kb + (int64_t)(n * bs + (j - an)) * a.kv_ld + (int64_t)g * D;
                const float x1 = to_f32(kr[i]), x2 = to_f32(kr[i + D / 2]);
                float cs, sn;
                rope_cs(a.rt, i, j, cs, sn);                 // own row j - an sits at position an + (j - an)
                k1 = x1 * cs - x2 * sn;
                k2 = x2 * cs + x1 * sn;
            }
            L.k[kk][i] = from_f32<T>(k1);
            L.k[kk][i + D / 2] = from_f32<T>(k2);
        }
        for (int idx = tid; idx < kBwKeys * D; idx += kBwThreads) {
            const int d = idx / kBwKeys, kk = idx - d * kBwKeys;   // consecutive threads: consecutive keys
            const int j = j0 + kk;
            T v = from_f32<T>(0.f);
            if (j < an) v = cvg[(int64_t)d * a.ctx_total + j];
            else if (j < nkeys) v = a.vb[(int64_t)(n * bs + (j - an)) * a.kv_ld + (int64_t)g * D + d];
            L.v[kk][d] = v;
        }
    };
    // Scores of the 16 columns cq*16.. of key slot kk.
    const int kk = tid % kBwKeys, cq = tid / kBwKeys;
    auto scores = [&](float (&s)[16]) {
#pragma unroll
        for (int c = 0; c < 16; ++c) s[c] = 0.f;
        for (int d = 0; d < D; ++d) {
            const float kv = to_f32(L.k[kk][d]);
#pragma unroll
            for (int c = 0; c < 16; ++c) s[c] += L.q[cq * 16 + c][d] * kv;
        }
    };

    // Pass 1: per-column max and sum of exp over all keys.
    float m[16], l[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        m[c] = -__builtin_inff();
        l[c] = 0.f;
    }
    for (int j0 = 0; j0 < nkeys; j0 += kBwKeys) {
        __syncthreads();
        stage(j0);
        __syncthreads();
        if (j0 + kk < nkeys) {
            float s[16];
            scores(s);
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float mn = fmaxf(m[c], s[c]);
                l[c] = l[c] * __expf(m[c] - mn) + __expf(s[c] - mn);
                m[c] = mn;
            }
        }
    }
    // Merge the 64 key slots of every column in a fixed order (the chunk
    // buffers ds / p hold the per-slot maxima and sums meanwhile).
    auto& s_m = L.ds;
    auto& s_l = L.p;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        s_m[kk][cq * 16 + c] = m[c];
        s_l[kk][cq * 16 + c] = l[c];
    }
    __syncthreads();
    if (tid < 64) {
        float mx = -__builtin_inff();
        for (int k = 0; k < kBwKeys; ++k) mx = fmaxf(mx, s_m[k][tid]);
        float sum = 0.f;
        for (int k = 0; k < kBwKeys; ++k)
            if (s_m[k][tid] != -__builtin_inff()) sum += s_l[k][tid] * __expf(s_m[k][tid] - mx);
        const float lse = sum > 0.f ? mx + logf(sum) : 0.f;
        L.red[0][tid][0] = lse;
        a.lse[((int64_t)n * a.hkv + g) * 64 + tid] = lse;
    }
    __syncthreads();

    // Pass 2: ds and p per chunk; dq~ sums; the block's own keys' dk~ and dv.
    const int dc = tid / 4, dqq = tid % 4;          // dq~ owner: column dc, d quarter dqq
    float dqa[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) dqa[i] = 0.f;
    for (int j0 = 0; j0 < nkeys; j0 += kBwKeys) {
        __syncthreads();
        stage(j0);
        __syncthreads();
        {
            float s[16], dp[16];
            scores(s);
#pragma unroll
            for (int c = 0; c < 16; ++c) dp[c] = 0.f;
            for (int d = 0; d < D; ++d) {
                const float vv = to_f32(L.v[kk][d]);
#pragma unroll
                for (int c = 0; c < 16; ++c) dp[c] += L.dout[cq * 16 + c][d] * vv;
            }
            const bool key_ok = j0 + kk < nkeys;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const int col = cq * 16 + c;
                const float pc = key_ok && col < C ? __expf(s[c] - L.red[0][col][0]) : 0.f;
                L.p[kk][col] = pc;
                L.ds[kk][col] = pc * (dp[c] - L.red[0][col][1]);
            }
        }
        __syncthreads();
        for (int k = 0; k < kBwKeys; ++k) {
            const float w = L.ds[k][dc];
#pragma unroll
            for (int i = 0; i < D / 4; ++i) dqa[i] += w * to_f32(L.k[k][dqq * (D / 4) + i]);
        }
        // Own keys of this chunk: j in [an, an + bs).
        const int lo = max(j0, an), hi = min(j0 + kBwKeys, nkeys);
        for (int idx = tid; idx < (hi > lo ? hi - lo : 0) * D; idx += kBwThreads) {
            const int r = idx / D, d = idx - r * D;
            const int slot = lo + r - j0;
            float dk = 0.f, dv = 0.f;
            for (int c = 0; c < C; ++c) {
                dk += L.ds[slot][c] * L.q[c][d];
                dv += L.p[slot][c] * L.dout[c][d];
            }
            const int row = n * bs + (lo + r - an);
            // dk~ is rotated back after the chunk; park it in dkb and fix below.
            a.dkb[(int64_t)row * (a.hkv * D) + (int64_t)g * D + d] = dk;
            a.dvb[(int64_t)row * (a.hkv * D) + (int64_t)g * D + d] = dv;
        }
    }
    __syncthreads();
    // dq = RoPE^T(dq~) * scale: pairs (i, i + D/2) live in quarters dqq and dqq + 2
    // (staged through the dO buffer, no longer needed).
    auto& s_dq = L.dout;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) s_dq[dc][dqq * (D / 4) + i] = dqa[i];
    __syncthreads();
    for (int idx = tid; idx < C * (D / 2); idx += kBwThreads) {
        const int c = idx / (D / 2), i = idx - c * (D / 2);
        const int k = c % bs, hh = c / bs, row = n * bs + k;
        float x1 = 0.f, x2 = 0.f;
        if (live) {
            float cs, sn;
            rope_cs(a.rt, i, an + k, cs, sn);
            const float y1 = s_dq[c][i], y2 = s_dq[c][i + D / 2];
            x1 = (y1 * cs + y2 * sn) * scale;
            x2 = (y2 * cs - y1 * sn) * scale;
        }
        float* o = a.dq + (int64_t)row * (a.hq * D) + (int64_t)(g * G + hh) * D;
        o[i] = x1;
        o[i + D / 2] = x2;
    }
    // Own keys: rotate dk~ back at anchor + row; empty blocks write zeros.
    __syncthreads();
    for (int idx = tid; idx < bs * (D / 2); idx += kBwThreads) {
        const int k = idx / (D / 2), i = idx - k * (D / 2);
        const int row = n * bs + k;
        float* dk = a.dkb + (int64_t)row * (a.hkv * D) + (int64_t)g * D;
        float x1 = 0.f, x2 = 0.f;
        if (live) {
            float cs, sn;
            rope_cs(a.rt, i, an + k, cs, sn);
            const float y1 = dk[i], y2 = dk[i + D / 2];
            x1 = y1 * cs + y2 * sn;
            x2 = y2 * cs - y1 * sn;
        } else {
            float* dv = a.dvb + (int64_t)row * (a.hkv * D) + (int64_t)g * D;
            dv[i] = 0.f;
            dv[i + D / 2] = 0.f;
        }
        dk[i] = x1;
        dk[i + D / 2] = x2;
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void attn_bwd_ctx_kernel(BwArgs<T> a) {
    __shared__ BwLds<T, D> L;
    const int t0 = blockIdx.x * kBwKeys, g = blockIdx.y, tid = threadIdx.x;
    const int G = a.hq / a.hkv, bs = a.bs, C = bs * G;
    const int kk = tid % kBwKeys, part = tid / kBwKeys;   // key slot; column quarter (A) / d quarter (B)
    // Stage the tile's K~ and V once.
    const T* ckg = a.ck + (int64_t)g * a.ctx_total * D;
    const T* cvg = a.cvt + (int64_t)g * D * a.ctx_total;
    for (int idx = tid; idx < kBwKeys * D; idx += kBwThreads) {
        const int r = idx / D, d = idx - r * D;
        const int64_t j = t0 + r;
        L.k[r][d] = j < a.ctx_total ? ckg[j * D + d] : from_f32<T>(0.f);
    }
    for (int idx = tid; idx < kBwKeys * D; idx += kBwThreads) {
        const int d = idx / kBwKeys, r = idx - d * kBwKeys;
        const int64_t j = t0 + r;
        L.v[r][d] = j < a.ctx_total ? cvg[(int64_t)d * a.ctx_total + j] : from_f32<T>(0.f);
    }
    float dk[D / 4], dv[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        dk[i] = 0.f;
        dv[i] = 0.f;
    }
    const int64_t key = t0 + kk;                            // this thread's context row (A and B)
    for (int n = 0; n < a.nb; ++n) {
        const int64_t base = clamp_base(a.base[n], a.ctx_total);
        const int an = anchor_eff(a.anchor[n], base, a.ctx_total);
        if (an <= 0 || base >= t0 + kBwKeys || base + an <= t0) continue;   // block n reads none of the tile
        __syncthreads();
        const float* qt = a.qt + ((int64_t)n * a.hkv + g) * 64 * D;
        for (int idx = tid; idx < 64 * D; idx += kBwThreads) (&L.q[0][0])[idx] = qt[idx];
        load_block_dout<T, D>(a, n, g, true, L, C, G);
        if (tid < 64) {
            L.red[0][tid][0] = a.lse[((int64_t)n * a.hkv + g) * 64 + tid];
            L.red[0][tid][1] = a.delta[((int64_t)n * a.hkv + g) * 64 + tid];
        }
        __syncthreads();
        const bool seen = key >= base && key < base + an;
        {
            float s[16], dp[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                s[c] = 0.f;
                dp[c] = 0.f;
            }
            for (int d = 0; d < D; ++d) {
                const float kv = to_f32(L.k[kk][d]), vv = to_f32(L.v[kk][d]);
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    s[c] += L.q[part * 16 + c][d] * kv;
                    dp[c] += L.dout[part * 16 + c][d] * vv;
                }
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const int col = part * 16 + c;
                const float pc = seen && col < C ? __expf(s[c] - L.red[0][col][0]) : 0.f;
                L.p[kk][col] = pc;
                L.ds[kk][col] = pc * (dp[c] - L.red[0][col][1]);
            }
        }
        __syncthreads();
        for (int c = 0; c < C; ++c) {
            const float w = L.ds[kk][c], pc = L.p[kk][c];
#pragma unroll
            for (int i = 0; i < D / 4; ++i) {
                dk[i] += w * L.q[c][part * (D / 4) + i];
                dv[i] += pc * L.dout[c][part * (D / 4) + i];
            }
        }
    }
    if (key < a.ctx_total) {
        float* ok = a.dck + ((int64_t)g * a.ctx_total + key) * D + part * (D / 4);
#pragma unroll
        for (int i = 0; i < D / 4; ++i) ok[i] = dk[i];
#pragma unroll
        for (int i = 0; i < D / 4; ++i) a.dcv[((int64_t)g * D + part * (D / 4) + i) * a.ctx_total + key] = dv[i];
    }
}

template <typename T, int D>
hipError_t attn_bwd_t(const BwArgs<T>& a, hipStream_t st) {
    {
        ProfScope prof(DFLASH_KERNEL_ATTN_BWD, st);
        hipLaunchKernelGGL((attn_bwd_query_kernel<T, D>), dim3(a.nb, a.hkv), dim3(kBwThreads), 0, st, a);
        if (a.ctx_total > 0)
            hipLaunchKernelGGL((attn_bwd_ctx_kernel<T, D>), dim3((unsigned)((a.ctx_total + kBwKeys - 1) / kBwKeys),
                                                               a.hkv),
                               dim3(kBwThreads), 0, st, a);
    }
    return hipGetLastError();
}

size_t bw_workspace(const dflash_config& c, int nb) {
    const size_t per = (size_t)nb * c.num_kv_heads * 64;
    return align_up(per * c.head_dim * sizeof(float), 256) + 2 * align_up(per * sizeof(float), 256) + 256;
}

}  // namespace

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_block_attn_backward_workspace_size(const dflash_config* cfg, int32_t num_blocks) {
    if (check_config(cfg) != DFLASH_OK || num_blocks < 0) return 0;
    return bw_workspace(*cfg, num_blocks);
}

extern "C" dflash_status dflash_block_attn_backward(
    const dflash_config* cfg, int32_t num_blocks, const void* q, const void* k_blk, const void* v_blk,
    const void* ctx_k, const void* ctx_v, int64_t ctx_total, const int64_t* block_ctx_base,
    const int32_t* block_anchor, const uint8_t* block_valid, const void* out, const void* d_out, float* d_q,
    float* d_k_blk, float* d_v_blk, float* d_ctx_k, float* d_ctx_v, void* workspace, size_t workspace_bytes,
    void* hip_stream) {
    dflash_status s = check_config(cfg);
    if (s != DFLASH_OK) return s;
    if (num_blocks < 0 || ctx_total < 0) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)num_blocks * cfg->block_size > INT32_MAX / 2 || ctx_total > (int64_t)INT32_MAX * 64)
        return DFLASH_ERR_UNSUPPORTED;
    if (num_blocks == 0 && ctx_total == 0) return DFLASH_OK;
    if ((num_blocks > 0 && (q == nullptr || k_blk == nullptr || v_blk == nullptr || block_ctx_base == nullptr ||
                            block_anchor == nullptr || block_valid == nullptr || out == nullptr || d_out == nullptr ||
                            d_q == nullptr || d_k_blk == nullptr || d_v_blk == nullptr)) ||
        (ctx_total > 0 && (ctx_k == nullptr || ctx_v == nullptr || d_ctx_k == nullptr || d_ctx_v == nullptr)))
        return DFLASH_ERR_INVALID_ARG;
    const size_t need = bw_workspace(*cfg, num_blocks);
    if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DFLASH_ERR_WORKSPACE;
    const size_t per = (size_t)num_blocks * cfg->num_kv_heads * 64;
    char* ws = static_cast<char*>(workspace);
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t e;
    auto fill = [&](auto tag) -> hipError_t {
        using T = decltype(tag);
        BwArgs<T> a{};
        a.q = static_cast<const T*>(q);
        a.kb = static_cast<const T*>(k_blk);
        a.vb = static_cast<const T*>(v_blk);
        a.q_ld = (int64_t)cfg->num_q_heads * cfg->head_dim;
        a.kv_ld = (int64_t)cfg->num_kv_heads * cfg->head_dim;
        a.ck = static_cast<const T*>(ctx_k);
        a.cvt = static_cast<const T*>(ctx_v);
        a.ctx_total = ctx_total;
        a.base = block_ctx_base;
        a.anchor = block_anchor;
        a.valid = block_valid;
        a.out = static_cast<const T*>(out);
        a.dout = static_cast<const T*>(d_out);
        a.dq = d_q;
        a.dkb = d_k_blk;
        a.dvb = d_v_blk;
        a.dck = d_ctx_k;
        a.dcv = d_ctx_v;
        a.qt = reinterpret_cast<float*>(ws);
        a.lse = reinterpret_cast<float*>(ws + align_up(per * cfg->head_dim * sizeof(float), 256));
        a.delta = a.lse + align_up(per * sizeof(float), 256) / sizeof(float);
        a.nb = num_blocks;
        a.bs = cfg->block_size;
        a.hq = cfg->num_q_heads;
        a.hkv = cfg->num_kv_heads;
        a.rt = make_rope_turns(*cfg);
        if (num_blocks == 0) {
            // No block reads the context: its gradient is zero.
            const int64_t cnt = (int64_t)cfg->num_kv_heads * ctx_total * cfg->head_dim;
            const unsigned grid = (unsigned)((cnt + 1023) / 1024 < 65535 ? (cnt + 1023) / 1024 : 65535);
            hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, st, d_ctx_k, cnt);
            hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, st, d_ctx_v, cnt);
            return hipGetLastError();
        }
        if constexpr (sizeof(T) == 2) return attn_bwd_t<T, 128>(a, st);
        else return attn_bwd_t<T, 64>(a, st);
    };
    e = cfg->dtype == DFLASH_BF16 ? fill(__bf16{}) : fill(float{});
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
