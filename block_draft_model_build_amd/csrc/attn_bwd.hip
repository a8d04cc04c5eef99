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
// Two kernels, deterministic (no atomics, fixed summation orders), in two
// implementations:
//  * a query-major kernel, one workgroup per (block, KV head): the softmax
//    statistics of the block's query columns, dq over all the keys the block
//    reads, and the block's own keys' dk and dv (only its own queries read
//    them); it leaves q~, masked dO, the logsumexp and rowsum(dO o) per
//    column in the workspace for the second kernel;
//  * a key-major kernel, one workgroup per (64-row context tile, KV head):
//    visits every block that reads the tile, in block order, and accumulates
//    the tile's dK and dV.
// fp32 configs (D = 64) run both on the vector units (attn_bwd_*_kernel, two
// passes over the keys); bf16 configs (D = 128) on the matrix cores (namespace
// mfb below: one pass with an online softmax, transposed LDS reads).
#include "internal.h"
#include "attention.h"

namespace dflash {

namespace {

constexpr int kBwKeys = 64;     // keys per chunk (query kernel) and rows per tile (context kernel)
constexpr int kBwThreads = 256;

__global__ __launch_bounds__(256) void zero_fill_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

template <typename T> struct BwArgs {
    const T *q, *kb, *vb;        // [nb*bs, Hq*D], [nb*bs, Hkv*D] x2 (un-rotated q, kb)
    int64_t q_ld, kv_ld;
    const T *ck, *cvt;           // [Hkv][ctx_total][D] rotated, [Hkv][D][ctx_total]
    int64_t ctx_total;
    const int64_t* base;
    const int32_t* anchor;
    const uint8_t* valid;        // rows whose forward output is zero where 0; null: none
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
            if (a.valid == nullptr || a.valid[row] != 0)
                v = to_f32(a.dout[(int64_t)row * a.q_ld + (int64_t)(g * G + hh) * D + d]);
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

// ---------------------------------------------------------------------------
// bf16 path on the matrix cores (D = 128). Four waves per workgroup; wave w
// owns column half wm = w / 2 and key half wn = w % 2 of a 64 x 64 tile.
// Operand fragments follow the MFMA 32x32x16 layout of Mfma<__bf16>: lane l
// holds 8 consecutive contraction indices 8 (l / 32) + 0..7 of row / column
// l % 32. Fragments whose contraction index runs down the rows of a row-major
// LDS tile come from the gfx950 transposed LDS read (lds_tr below). Products
// whose contraction runs over keys or columns take their left operand
// straight from a previous product's accumulator: a row permutation of that
// product (key_perm) makes each lane hold 8 consecutive keys / columns.
namespace mfb {

constexpr int D = 128;
constexpr int KT = 64;                // keys per chunk / tile, columns per block

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Row-major tiles of 64 rows x 128 bf16 (K~, Q~, dO): 16-byte chunk c of row r
// is stored at chunk position c ^ (r & 15).
__device__ __forceinline__ int koff(int r, int d) { return r * 256 + ((((d >> 3) ^ (r & 15))) << 4) + ((d & 7) << 1); }
// V^T tiles of 128 rows (d) x 64 keys: chunk c of row d at c ^ (d & 7).
__device__ __forceinline__ int voff(int d, int j) { return d * 128 + ((((j >> 3) ^ (d & 7))) << 4) + ((j & 7) << 1); }

// Transposed LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane j supplies the address of 4 consecutive 16-bit elements; lane i gets
// element i % 4 of lane 4 e + i / 4 as its element e. So if lane j of the
// group points at row r0 + j / 4, column c0 + 4 (j % 4) of a row-major tile,
// lane i receives column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ s16x4 lds_tr(const char* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 a, s16x4 b) {
    s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 lds_frag(const char* base, int off) { return *(const bf16x8*)(base + off); }
// Group-relative column offset that makes output lane i of a transposed read
// hold column key_perm(i) (bits 2 and 3 of i swapped).
__device__ __forceinline__ int perm_col(int r) { return ((r & 1) << 3) | ((r & 2) << 1); }

// Fragment of a 32x32x16 operand whose contraction index k runs down the rows
// of a row-major tile: rows k0 + 8 (l / 32) + 0..7, column n0 + l % 32.
__device__ __forceinline__ bf16x8 tr_frag_k(const char* base, int k0, int n0, int lane) {
    const int i = lane & 15, G = lane >> 4;
    const int r = k0 + 8 * (G >> 1) + (i >> 2), col = n0 + 16 * (G & 1) + 4 * (i & 3);
    return join(lds_tr(base + koff(r, col)), lds_tr(base + koff(r + 4, col)));
}

// The same fragment from a plain (unswizzled) row-major tile with rows of
// row_bytes bytes.
__device__ __forceinline__ bf16x8 tr_frag_plain(const char* base, int row_bytes, int k0, int n0, int lane) {
    const int i = lane & 15, G = lane >> 4;
    const int r = k0 + 8 * (G >> 1) + (i >> 2), col = n0 + 16 * (G & 1) + 4 * (i & 3);
    return join(lds_tr(base + r * row_bytes + col * 2), lds_tr(base + (r + 4) * row_bytes + col * 2));
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int half) {
    bf16x8 f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = static_cast<__bf16>(v[8 * half + i]);
    return f;
}

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
// Renumber a 1-D grid of `total` items so that every XCD gets a contiguous run
// of items (blocks of one sequence share their context; tiles of one sequence
// share their blocks); the items past the last multiple of 8 keep their index.
__device__ __forceinline__ int xcd_item(int id, int total) {
    const int t8 = total / 8 * 8;
    return id < t8 ? (id % 8) * (total / 8) + id / 8 : id;
}

__device__ __forceinline__ void dma16(const void* src, char* lds_base) {
    __builtin_amdgcn_global_load_lds(DFLASH_GPTR(src), DFLASH_LPTR(lds_base), 16, 0, 0);
}

// 64 rows of a row-major [rows][128] bf16 array into a swizzled tile; row r of
// the tile reads source row rowmap(r). Each wave issues 4 loads (1 KB each).
template <typename RowPtr>
__device__ __forceinline__ void dma_rows(char* tile, RowPtr rowptr, int wave, int lane) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int u0 = (it * 4 + wave) * 64, u = u0 + lane;
        const int r = u >> 4, ch = u & 15;
        dma16(rowptr(r) + ((ch ^ (r & 15)) << 3), tile + u0 * 16);
    }
}

constexpr int kRopeRows = 16;   // block rows whose rotations the query kernel tabulates

struct QueryLds {
    char k[2][KT * 256];     // K~ chunk (swizzled rows), two stages
    char vt[2][D * 128];     // V^T chunk, two stages
    float m[2][KT], l[2][KT];
    float rc[kRopeRows][D / 2], rs[kRopeRows][D / 2];   // cos / sin of block row k, pair i
};

struct CtxLds {
    char k[KT * 256];        // K~ tile
    char vt[D * 128];        // V^T tile
    char q[KT * 256];        // Q~ of the current block
    char dout[KT * 256];     // masked dO of the current block
    float lse[KT], delta[KT];
    int list[256], list_an[256];
    int64_t list_base[256];
    int cnt[4];
};

struct MfArgs {
    BwArgs<__bf16> a;
    __bf16 *qt, *dot;        // workspace [nb][Hkv][64][128]: Q~ and masked dO per block
};

// Query-major kernel: one workgroup per (block, KV head). Scores are kept in
// log2 units (Q~ carries log2(e) / sqrt(D)), so every probability is one exp2.
// Small enough (registers, 64 KB of LDS) for two workgroups per compute unit.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_query_kernel(MfArgs m) {
    const BwArgs<__bf16>& a = m.a;
    __shared__ QueryLds L;
    const int item = xcd_item(blockIdx.x, a.nb * a.hkv);
    const int n = item % a.nb, g = item / a.nb, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1, h = lane >> 5, l32 = lane & 31;
    const int G = a.hq / a.hkv, bs = a.bs, C = bs * G;
    const float scale = 1.f / sqrtf((float)D);
    const float qscale = 1.4426950408889634f * scale;     // log2(e) / sqrt(D)
    const int64_t base = clamp_base(a.base[n], a.ctx_total);
    const int an = anchor_eff(a.anchor[n], base, a.ctx_total);
    const int64_t slot = (int64_t)n * a.hkv + g;
    if (an < 0) {
        // Empty block: nothing is read, nothing passes back.
        for (int idx = tid; idx < C * D; idx += 256) {
            const int c = idx / D, d = idx - c * D;
            a.dq[(int64_t)(n * bs + c % bs) * a.q_ld + (int64_t)(g * G + c / bs) * D + d] = 0.f;
        }
        for (int idx = tid; idx < bs * D; idx += 256) {
            const int r = idx / D, d = idx - r * D;
            a.dkb[(int64_t)(n * bs + r) * a.kv_ld + (int64_t)g * D + d] = 0.f;
            a.dvb[(int64_t)(n * bs + r) * a.kv_ld + (int64_t)g * D + d] = 0.f;
        }
        return;
    }
    const __bf16* ckg = a.ck + ((int64_t)g * a.ctx_total + base) * D;
    const __bf16* cvg = a.cvt + (int64_t)g * D * a.ctx_total + base;
    const int64_t lim = a.ctx_total - base;          // cache rows addressable from this base

    // Rotations of the block rows (position an + k), computed once: rows below
    // kRopeRows from the table, longer blocks' further rows directly.
    for (int idx = tid; idx < min(bs, kRopeRows) * (D / 2); idx += 256) {
        const int k = idx / (D / 2), i = idx - k * (D / 2);
        rope_cs(a.rt, i, an + k, L.rc[k][i], L.rs[k][i]);
    }
    __syncthreads();
    auto rot = [&](int k, int i, float& cs, float& sn) {
        if (k < kRopeRows) {
            cs = L.rc[k][i];
            sn = L.rs[k][i];
        } else {
            rope_cs(a.rt, i, an + k, cs, sn);
        }
    };

    // This lane's column (B operand n index) and its Q~ / dO fragments.
    const int c = 32 * wm + l32;
    const bool col_ok = c < C;
    const int kq = c % bs, hq = c / bs, qrow = n * bs + kq;
    bf16x8 qf[8], df[8];
    float delta = 0.f;
    {
        const __bf16* qr = a.q + (int64_t)qrow * a.q_ld + (int64_t)(g * G + hq) * D;
        const __bf16* orow = a.out + (int64_t)qrow * a.q_ld + (int64_t)(g * G + hq) * D;
        const __bf16* dr = a.dout + (int64_t)qrow * a.q_ld + (int64_t)(g * G + hq) * D;
        const bool live_row = col_ok && (a.valid == nullptr || a.valid[qrow] != 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 lo = {}, hi = {}, dlo = {}, dhi = {};
            if (col_ok) {
                lo = *(const bf16x8*)(qr + 16 * ks + 8 * h);
                hi = *(const bf16x8*)(qr + 64 + 16 * ks + 8 * h);
            }
            if (live_row) {
                dlo = *(const bf16x8*)(dr + 16 * ks + 8 * h);
                dhi = *(const bf16x8*)(dr + 64 + 16 * ks + 8 * h);
                const bf16x8 olo = *(const bf16x8*)(orow + 16 * ks + 8 * h);
                const bf16x8 ohi = *(const bf16x8*)(orow + 64 + 16 * ks + 8 * h);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    delta += (float)dlo[i] * (float)olo[i] + (float)dhi[i] * (float)ohi[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float cs, sn;
                rot(kq, 16 * ks + 8 * h + i, cs, sn);
                const float x1 = (float)lo[i], x2 = (float)hi[i];
                qf[ks][i] = static_cast<__bf16>((x1 * cs - x2 * sn) * qscale);
                qf[ks + 4][i] = static_cast<__bf16>((x2 * cs + x1 * sn) * qscale);
            }
            df[ks] = dlo;
            df[ks + 4] = dhi;
        }
        delta += __shfl_xor(delta, 32, 64);
        if (!col_ok) delta = 0.f;
    }
    if (wn == 0) {
        // Q~ and masked dO for the context kernel and the own keys (workspace).
        __bf16* qt = m.qt + slot * KT * D + (int64_t)c * D;
        __bf16* dt = m.dot + slot * KT * D + (int64_t)c * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int d0 = 16 * ks + 8 * h;
            *(bf16x8*)(qt + d0) = qf[ks];
            *(bf16x8*)(dt + d0) = df[ks];
        }
        if (h == 0) a.delta[slot * KT + c] = delta;
    }

    // Context keys [0, an) in 64-key chunks (DMA, K rows clamped to the last
    // visible one), then the block's own keys (rotated here).
    const int nctx = (an + KT - 1) / KT;
    auto stage_ctx = [&](int ch, int buf) {
        char* Lk = L.k[buf];
        char* Lvt = L.vt[buf];
        const int j0 = ch * KT;
        dma_rows(Lk, [&](int r) { return ckg + (int64_t)min(j0 + r, an - 1) * D; }, w, lane);
        if ((int64_t)j0 + KT <= lim) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int u0 = (it * 4 + w) * 64, u = u0 + lane;
                const int d = u >> 3, cc = u & 7;
                dma16(cvg + (int64_t)d * a.ctx_total + j0 + ((cc ^ (d & 7)) << 3), Lvt + u0 * 16);
            }
        } else {
            // Chunk reaching the end of the cache: element loads, keys clamped.
            for (int idx = tid; idx < D * KT; idx += 256) {
                const int d = idx / KT, j = idx - d * KT;
                const int64_t jj = min((int64_t)(j0 + j), lim - 1);
                *(__bf16*)(Lvt + voff(d, j)) = cvg[(int64_t)d * a.ctx_total + jj];
            }
        }
    };
    auto stage_own = [&](int buf) {
        char* Lk = L.k[buf];
        char* Lvt = L.vt[buf];
        for (int idx = tid; idx < KT * (D / 2); idx += 256) {
            const int r = idx / (D / 2), i = idx - r * (D / 2);
            float y1 = 0.f, y2 = 0.f;
            if (r < bs) {
                const __bf16* kr = a.kb + (int64_t)(n * bs + r) * a.kv_ld + (int64_t)g * D;
                const float x1 = (float)kr[i], x2 = (float)kr[i + D / 2];
                float cs, sn;
                rot(r, i, cs, sn);
                y1 = x1 * cs - x2 * sn;
                y2 = x2 * cs + x1 * sn;
            }
            *(__bf16*)(Lk + koff(r, i)) = static_cast<__bf16>(y1);
            *(__bf16*)(Lk + koff(r, i + D / 2)) = static_cast<__bf16>(y2);
        }
        for (int idx = tid; idx < KT * D; idx += 256) {
            const int r = idx / D, d = idx - r * D;
            __bf16 v = static_cast<__bf16>(0.f);
            if (r < bs) v = a.vb[(int64_t)(n * bs + r) * a.kv_ld + (int64_t)g * D + d];
            *(__bf16*)(Lvt + voff(d, r)) = v;
        }
    };

    // One pass with a running maximum m per column (online softmax):
    // p~ = 2^(s - m), l = sum p~, dQ~ accumulates dS~ K~ with dS~ = p~ (dP - delta),
    // rescaled when m moves; at the end P = p~ / l and dQ~ = (sum dS~ K~) / l.
    // m only moves when a chunk's maximum exceeds it by more than 8 (p~ stays
    // below 2^8), so rescales are rare after the first chunk.
    float mrun = -__builtin_inff(), lrun = 0.f;
    f32x16 dq[4] = {};
    const int i16 = lane & 15, G16 = lane >> 4;
    const int kcol = 32 * wn + 16 * (G16 & 1) + perm_col(i16 & 3);   // V^T column (key) of this lane's A rows
    const int krow = 32 * wn + key_perm(l32);                         // K~ row of this lane's A rows
    // nv: keys of the chunk that are visible; p and ds come back in p / ds.
    auto chunk = [&](const char* Lk, const char* Lvt, int nv, f32x16& p, f32x16& ds) {
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            s = Mfma<__bf16>::mma(lds_frag(Lk, koff(krow, 16 * ks + 8 * h)), qf[ks], s);
            const int d0 = 16 * ks + 8 * h + (i16 >> 2);
            const bf16x8 va = join(lds_tr(Lvt + voff(d0, kcol)), lds_tr(Lvt + voff(d0 + 4, kcol)));
            dp = Mfma<__bf16>::mma(va, df[ks], dp);
        }
        if (nv < KT) {
            const int nvl = nv - 32 * wn - 8 * h;       // keys acc_key(e) < nvl are visible
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (acc_key(e) >= nvl) s[e] = -__builtin_inff();
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));            // both key halves of the column
        const bool move = mx > mrun + 8.f;
        if (__any(move)) {
            const float mnew = move ? mx : mrun;
            const float f = mrun == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mrun - mnew);
            mrun = mnew;
            lrun *= f;
            // dQ~ accumulator rows are columns: fetch each row's factor from its lane.
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float fe = __shfl(f, acc_row(e, lane), 64);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) dq[dt][e] *= fe;
            }
        }
        const float muse = mrun == -__builtin_inff() ? 0.f : mrun;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            p[e] = __builtin_amdgcn_exp2f(s[e] - muse);
            ps += p[e];
            ds[e] = p[e] * (dp[e] - delta);
        }
        lrun += ps;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 af = pack8(ds, kk);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                dq[dt] = Mfma<__bf16>::mma(af, tr_frag_k(Lk, 32 * wn + 16 * kk, 32 * dt, lane), dq[dt]);
        }
    };

    __syncthreads();
    if (nctx > 0) stage_ctx(0, 0);
    else stage_own(0);
    for (int ch = 0; ch < nctx; ++ch) {
        wait_vmcnt<0>();
        __syncthreads();
        if (ch + 1 < nctx) stage_ctx(ch + 1, (ch + 1) & 1);
        else stage_own((ch + 1) & 1);
        f32x16 p, ds;
        chunk(L.k[ch & 1], L.vt[ch & 1], min(KT, an - ch * KT), p, ds);
    }
    wait_vmcnt<0>();
    __syncthreads();
    const int so = nctx & 1;                          // stage holding the own keys
    f32x16 p_own, ds_own;
    chunk(L.k[so], L.vt[so], bs, p_own, ds_own);

    // Column statistics: add the lane halves, then merge the two key halves.
    lrun += __shfl_xor(lrun, 32, 64);
    if (h == 0) {
        L.m[wn][c] = mrun;
        L.l[wn][c] = lrun;
    }
    __syncthreads();
    if (tid < KT) {
        const int cc = tid;
        const float m0 = L.m[0][cc], m1 = L.m[1][cc];
        const float mm = fmaxf(m0, m1);
        const float f0 = m0 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
        const float f1 = m1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        const float ll = L.l[0][cc] * f0 + L.l[1][cc] * f1;
        // lse in log2 units; unused columns get +inf (their probabilities are exactly zero).
        const bool used = cc < C && ll > 0.f;
        const float lse = used ? mm + __log2f(ll) : __builtin_inff();
        a.lse[slot * KT + cc] = lse;
        // Factor that turns each key half's p~ into P.
        L.m[0][cc] = used ? f0 / ll : 0.f;
        L.m[1][cc] = used ? f1 / ll : 0.f;
    }
    __syncthreads();
    // The own chunk's P and dS ([key][column], 16 KB each) go to the free stage;
    // Q~ and dO (plain [column][d] rows) go over the own keys' stage.
    float* Pown = reinterpret_cast<float*>(L.k[so ^ 1]);
    float* Down = reinterpret_cast<float*>(L.vt[so ^ 1]);
    __bf16* Qs = reinterpret_cast<__bf16*>(L.k[so]);
    __bf16* Ds = reinterpret_cast<__bf16*>(L.vt[so]);
    {
        const float f = L.m[wn][c];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 32 * wn + acc_key(e) + 8 * h;
            Pown[key * KT + c] = p_own[e] * f;
            Down[key * KT + c] = ds_own[e] * f;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float fe = L.m[wn][32 * wm + acc_row(e, lane)];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) dq[dt][e] *= fe;
        }
        if (wn == 0) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                *(bf16x8*)(Qs + c * D + 16 * ks + 8 * h) = qf[ks];
                *(bf16x8*)(Ds + c * D + 16 * ks + 8 * h) = df[ks];
            }
        }
    }
    __syncthreads();

    // Own keys: dK~ = dS^T Q~ and dV = P^T dO on the matrix cores (keys x d,
    // contracting over the block's columns); wave w takes d tile w. dK~ goes
    // through LDS to be rotated back pairwise (and out of log2 units: Q~
    // carries log2(e)).
    constexpr float kLn2 = 0.6931471805599453f;
    {
        const int ntk = bs > 32 ? 2 : 1;
        f32x16 ak[2] = {}, av[2] = {};
        for (int mt = 0; mt < ntk; ++mt) {
            const int key = 32 * mt + l32;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const float* dsr = Down + key * KT + 16 * ks + 8 * h;
                const float* pr = Pown + key * KT + 16 * ks + 8 * h;
                bf16x8 a_ds, a_p;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    a_ds[i] = static_cast<__bf16>(dsr[i]);
                    a_p[i] = static_cast<__bf16>(pr[i]);
                }
                const bf16x8 bq = tr_frag_plain(reinterpret_cast<const char*>(Qs), D * 2, 16 * ks, 32 * w, lane);
                const bf16x8 bd = tr_frag_plain(reinterpret_cast<const char*>(Ds), D * 2, 16 * ks, 32 * w, lane);
                ak[mt] = Mfma<__bf16>::mma(a_ds, bq, ak[mt]);
                av[mt] = Mfma<__bf16>::mma(a_p, bd, av[mt]);
            }
        }
        __syncthreads();                               // P and dS are read: their space takes dK~
        float* dkst = Pown;   // [key][D] fp32: bs x 512 bytes, past 16 KB over the dead Q~ / dO tiles
        const int d = 32 * w + l32;
        for (int mt = 0; mt < ntk; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = 32 * mt + acc_row(e, lane);
                if (key < bs) {
                    dkst[key * D + d] = ak[mt][e] * kLn2;
                    a.dvb[(int64_t)(n * bs + key) * a.kv_ld + (int64_t)g * D + d] = av[mt][e];
                }
            }
    }
    __syncthreads();
    {
        const float* dkst = Pown;
        for (int idx = tid; idx < bs * (D / 2); idx += 256) {
            const int r = idx / (D / 2), i = idx - r * (D / 2);
            const float k1 = dkst[r * D + i], k2 = dkst[r * D + i + D / 2];
            float cs, sn;
            rot(r, i, cs, sn);
            float* dk = a.dkb + (int64_t)(n * bs + r) * a.kv_ld + (int64_t)g * D;
            dk[i] = k1 * cs + k2 * sn;
            dk[i + D / 2] = k2 * cs - k1 * sn;
        }
    }
    __syncthreads();

    // dQ~: add the two key halves, rotate back, scale.
    float* red = reinterpret_cast<float*>(L.k[0]);  // both K~ stages: 32 KB
    if (wn == 1) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[((wm * 4 + dt) * 16 + e) * 64 + lane] = dq[dt][e];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) dq[dt][e] += red[((wm * 4 + dt) * 16 + e) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int cc = 32 * wm + acc_row(e, lane);
            if (cc >= C) continue;
            const int k = cc % bs, hh = cc / bs;
            float* o = a.dq + (int64_t)(n * bs + k) * a.q_ld + (int64_t)(g * G + hh) * D;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const int i = 32 * dt + l32;
                float cs, sn;
                rot(k, i, cs, sn);
                const float y1 = dq[dt][e], y2 = dq[dt + 2][e];
                o[i] = (y1 * cs + y2 * sn) * scale;
                o[i + D / 2] = (y2 * cs - y1 * sn) * scale;
            }
        }
    }
}

// Key-major kernel over the context: one workgroup per (64-row tile, KV head);
// the blocks that read the tile are visited in index order, so every dK / dV
// sum has a fixed order. Sized (registers, 67 KB of LDS) for two workgroups
// per compute unit: one loads a block's Q~ / dO while the other computes.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_ctx_kernel(MfArgs m) {
    const BwArgs<__bf16>& a = m.a;
    __shared__ CtxLds L;
    const int tiles = (int)((a.ctx_total + KT - 1) / KT);
    const int item = xcd_item(blockIdx.x, tiles * a.hkv);
    const int g = item / tiles, tid = threadIdx.x;
    const int64_t t0 = (int64_t)(item % tiles) * KT;
    const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1, h = lane >> 5, l32 = lane & 31;
    const int64_t T = a.ctx_total;
    const __bf16* ckg = a.ck + (int64_t)g * T * D;
    const __bf16* cvg = a.cvt + (int64_t)g * D * T;
    // The tile's K~ and V^T (rows past the cache clamped to its last row),
    // staged once the first block that reads the tile is found.
    bool staged = false;
    auto stage_tile = [&]() {
        dma_rows(L.k, [&](int r) { return ckg + min(t0 + r, T - 1) * D; }, w, lane);
        if (t0 + KT <= T) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int u0 = (it * 4 + w) * 64, u = u0 + lane;
                const int d = u >> 3, cc = u & 7;
                dma16(cvg + (int64_t)d * T + t0 + ((cc ^ (d & 7)) << 3), L.vt + u0 * 16);
            }
        } else {
            for (int idx = tid; idx < D * KT; idx += 256) {
                const int d = idx / KT, j = idx - d * KT;
                *(__bf16*)(L.vt + voff(d, j)) = cvg[(int64_t)d * T + min(t0 + j, T - 1)];
            }
        }
    };
    const int64_t key = t0 + 32 * wn + l32;            // key column of this lane in S and dP
    const int i16 = lane & 15, G16 = lane >> 4;
    const int vcol = 32 * wn + 16 * (G16 & 1) + 4 * (i16 & 3);
    const int cr = 32 * wm + key_perm(l32);            // Q~ / dO row of this lane's A operands
    f32x16 dk[4] = {}, dv[4] = {};
    for (int b0 = 0; b0 < a.nb; b0 += 256) {
        // The blocks of [b0, b0 + 256) that read this tile, in index order.
        const int nn = b0 + tid;
        bool reads = false;
        int64_t bb = 0;
        int ba = -1;
        if (nn < a.nb) {
            bb = clamp_base(a.base[nn], T);
            ba = anchor_eff(a.anchor[nn], bb, T);
            reads = ba > 0 && bb < t0 + KT && bb + ba > t0;
        }
        const uint64_t mask = __ballot(reads);
        if (lane == 0) L.cnt[w] = __popcll(mask);
        __syncthreads();
        int off = 0, total = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            off += i < w ? L.cnt[i] : 0;
            total += L.cnt[i];
        }
        if (reads) {
            const int at = off + __popcll(mask & ((1ull << lane) - 1));
            L.list[at] = nn;
            L.list_base[at] = bb;
            L.list_an[at] = ba;
        }
        if (total > 0 && !staged) {
            stage_tile();                             // completes with the first block's loads below
            staged = true;
        }
        for (int it = 0; it < total; ++it) {
            __syncthreads();                           // the list, and the previous block's reads
            const int64_t slot = (int64_t)L.list[it] * a.hkv + g;
            dma_rows(L.q, [&](int r) { return m.qt + (slot * KT + r) * D; }, w, lane);
            dma_rows(L.dout, [&](int r) { return m.dot + (slot * KT + r) * D; }, w, lane);
            if (w == 0 && lane < 16) dma16(a.lse + slot * KT + 4 * lane, (char*)L.lse);
            if (w == 1 && lane < 16) dma16(a.delta + slot * KT + 4 * lane, (char*)L.delta);
            const int64_t base = L.list_base[it];
            const int an = L.list_an[it];
            wait_vmcnt<0>();
            __syncthreads();
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 kf = lds_frag(L.k, koff(32 * wn + l32, 16 * ks + 8 * h));
                s = Mfma<__bf16>::mma(lds_frag(L.q, koff(cr, 16 * ks + 8 * h)), kf, s);
                const int d0 = 16 * ks + 8 * h + (i16 >> 2);
                const bf16x8 vf = join(lds_tr(L.vt + voff(d0, vcol)), lds_tr(L.vt + voff(d0 + 4, vcol)));
                dp = Mfma<__bf16>::mma(lds_frag(L.dout, koff(cr, 16 * ks + 8 * h)), vf, dp);
            }
            // Scores are in log2 units (Q~ carries log2(e)): P = 2^(s - lse).
            // Keys outside [base, base + an) get 2^-inf = 0 (no branch per element).
            const float hide = key >= base && key < base + an ? 0.f : -__builtin_inff();
            f32x16 p, ds;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int cc = 32 * wm + acc_key(e) + 8 * h;
                p[e] = __builtin_amdgcn_exp2f(s[e] - L.lse[cc] + hide);
                ds[e] = p[e] * (dp[e] - L.delta[cc]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 pa = pack8(p, kk), da = pack8(ds, kk);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    dv[dt] = Mfma<__bf16>::mma(pa, tr_frag_k(L.dout, 32 * wm + 16 * kk, 32 * dt, lane), dv[dt]);
                    dk[dt] = Mfma<__bf16>::mma(da, tr_frag_k(L.q, 32 * wm + 16 * kk, 32 * dt, lane), dk[dt]);
                }
            }
        }
        __syncthreads();
    }
    // Add the two column halves and write the tile's gradients.
    __syncthreads();
    float* red = reinterpret_cast<float*>(L.k);     // 64 KB: the K~, V^T, Q~ and dO tiles
    if (wm == 1) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                red[((wn * 8 + dt) * 16 + e) * 64 + lane] = dk[dt][e];
                red[((wn * 8 + 4 + dt) * 16 + e) * 64 + lane] = dv[dt][e];
            }
    }
    __syncthreads();
    if (wm == 0) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                dk[dt][e] += red[((wn * 8 + dt) * 16 + e) * 64 + lane];
                dv[dt][e] += red[((wn * 8 + 4 + dt) * 16 + e) * 64 + lane];
            }
    }
    __syncthreads();
    // dK rows go out directly (lanes cover consecutive dimensions); dV goes
    // through LDS as [d][key] so that each dimension's 64 keys leave as one
    // contiguous 256-byte run of the transposed gradient.
    constexpr int VP = KT + 4;                        // padded row (floats), 16-byte aligned
    float* dvt = red;                                 // [D][VP] fp32 = 34 KB of the 64 KB
    if (wm == 0) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int d = 32 * dt + l32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int jj = 32 * wn + acc_row(e, lane);
                const int64_t j = t0 + jj;
                if (j < T) a.dck[((int64_t)g * T + j) * D + d] = dk[dt][e] * 0.6931471805599453f;   // Q~ carries log2(e)
                dvt[d * VP + jj] = dv[dt][e];
            }
        }
    }
    __syncthreads();
    const bool vec = (T & 3) == 0 && t0 + KT <= T;
    for (int idx = tid; idx < D * (KT / 4); idx += 256) {
        const int d = idx / (KT / 4), j4 = (idx - d * (KT / 4)) * 4;
        float* o = a.dcv + ((int64_t)g * D + d) * T + t0 + j4;
        const float* src = dvt + d * VP + j4;
        if (vec) {
            *(f32x4*)o = *(const f32x4*)src;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (t0 + j4 + q < T) o[q] = src[q];
        }
    }
}

}  // namespace mfb

// fp32 (D = 64): the vector-unit kernels.
hipError_t attn_bwd_f32(const BwArgs<float>& a, hipStream_t st) {
    {
        ProfScope prof(DFLASH_KERNEL_ATTN_BWD, st);
        hipLaunchKernelGGL((attn_bwd_query_kernel<float, 64>), dim3(a.nb, a.hkv), dim3(kBwThreads), 0, st, a);
        if (a.ctx_total > 0)
            hipLaunchKernelGGL((attn_bwd_ctx_kernel<float, 64>),
                               dim3((unsigned)((a.ctx_total + kBwKeys - 1) / kBwKeys), a.hkv), dim3(kBwThreads), 0,
                               st, a);
    }
    return hipGetLastError();
}

// bf16 (D = 128): the matrix-core kernels.
hipError_t attn_bwd_bf16(const mfb::MfArgs& m, hipStream_t st) {
    {
        ProfScope prof(DFLASH_KERNEL_ATTN_BWD, st);
        hipLaunchKernelGGL(mfb::bwd_query_kernel, dim3(m.a.nb * m.a.hkv), dim3(256), 0, st, m);
        if (m.a.ctx_total > 0)
            hipLaunchKernelGGL(mfb::bwd_ctx_kernel,
                               dim3((unsigned)((m.a.ctx_total + mfb::KT - 1) / mfb::KT * m.a.hkv)), dim3(256), 0, st,
                               m);
    }
    return hipGetLastError();
}

// Workspace: per (block, KV head) the block's 64 query columns; bf16 keeps
// Q~ and masked dO (bf16), fp32 keeps Q~ (fp32); both keep lse and
// rowsum(dO o) per column.
struct BwLayout {
    size_t qt, dot, lse, delta, total;
};
BwLayout bw_layout(const dflash_config& c, int nb) {
    const size_t per = (size_t)nb * c.num_kv_heads * 64;
    BwLayout l{};
    size_t off = 0;
    l.qt = off;
    if (c.dtype == DFLASH_BF16) {
        off = align_up(off + per * c.head_dim * 2, 256);
        l.dot = off;
        off = align_up(off + per * c.head_dim * 2, 256);
    } else {
        off = align_up(off + per * c.head_dim * 4, 256);
        l.dot = off;
    }
    l.lse = off;
    off = align_up(off + per * 4, 256);
    l.delta = off;
    off = align_up(off + per * 4, 256);
    l.total = off + 256;
    return l;
}
size_t bw_workspace(const dflash_config& c, int nb) { return bw_layout(c, nb).total; }

}  // namespace

// The whole attention backward on the stream, arguments checked by the caller.
hipError_t attn_backward_run(const dflash_config* cfg, int num_blocks, const void* q, const void* k_blk,
                             const void* v_blk, const void* ctx_k, const void* ctx_v, int64_t ctx_total,
                             const int64_t* block_ctx_base, const int32_t* block_anchor, const uint8_t* block_valid,
                             const void* out, const void* d_out, float* d_q, float* d_k_blk, float* d_v_blk,
                             float* d_ctx_k, float* d_ctx_v, char* ws, hipStream_t st) {
    const BwLayout lay = bw_layout(*cfg, num_blocks);
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
        a.qt = reinterpret_cast<float*>(ws + lay.qt);
        a.lse = reinterpret_cast<float*>(ws + lay.lse);
        a.delta = reinterpret_cast<float*>(ws + lay.delta);
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
        if constexpr (sizeof(T) == 2) {
            mfb::MfArgs m{a, reinterpret_cast<__bf16*>(ws + lay.qt), reinterpret_cast<__bf16*>(ws + lay.dot)};
            return attn_bwd_bf16(m, st);
        } else {
            return attn_bwd_f32(a, st);
        }
    };
    return cfg->dtype == DFLASH_BF16 ? fill(__bf16{}) : fill(float{});
}

size_t attn_backward_workspace(const dflash_config& c, int nb) { return bw_layout(c, nb).total; }

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
    if ((int64_t)num_blocks * cfg->block_size > INT32_MAX / 2 || (int64_t)num_blocks * cfg->num_kv_heads > INT32_MAX ||
        (ctx_total + 63) / 64 * cfg->num_kv_heads > INT32_MAX)
        return DFLASH_ERR_UNSUPPORTED;
    if (num_blocks == 0 && ctx_total == 0) return DFLASH_OK;
    if ((num_blocks > 0 && (q == nullptr || k_blk == nullptr || v_blk == nullptr || block_ctx_base == nullptr ||
                            block_anchor == nullptr || block_valid == nullptr || out == nullptr || d_out == nullptr ||
                            d_q == nullptr || d_k_blk == nullptr || d_v_blk == nullptr)) ||
        (ctx_total > 0 && (ctx_k == nullptr || ctx_v == nullptr || d_ctx_k == nullptr || d_ctx_v == nullptr)))
        return DFLASH_ERR_INVALID_ARG;
    // 16-byte vector loads of the inputs and stores of the gradients.
    for (const void* p : {q, k_blk, v_blk, ctx_k, ctx_v, out, d_out, (const void*)d_q, (const void*)d_k_blk,
                          (const void*)d_v_blk, (const void*)d_ctx_k, (const void*)d_ctx_v})
        if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return DFLASH_ERR_INVALID_ARG;
    const size_t need = bw_workspace(*cfg, num_blocks);
    if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DFLASH_ERR_WORKSPACE;
    hipError_t e = attn_backward_run(cfg, num_blocks, q, k_blk, v_blk, ctx_k, ctx_v, ctx_total, block_ctx_base,
                                     block_anchor, block_valid, out, d_out, d_q, d_k_blk, d_v_blk, d_ctx_k, d_ctx_v,
                                     static_cast<char*>(workspace), reinterpret_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
