// Dual-source block attention for gfx950.
//
// Work unit ("item"): one block n, one KV head g and one split s of the block's
// prefix. Its 64 (or 32) query columns are the block's bs positions times the
// G = Hq/Hkv query heads that share KV head g, so every K/V byte fetched serves
// all G heads. Keys are the prefix rows [s*chunk, min(a, (s+1)*chunk)) of the
// projected context plus, for split 0, the block's own bs rows.
//
// Layout of the math (keys on MFMA rows, queries on MFMA columns):
//   S^T[key, q] = K[key, :] . Q[q, :]        A = K tile from LDS, B = Q in registers
//   O^T[d, q]  += V^T[d, key] . P^T[key, q]  A = V^T tile from LDS, B = P in registers
// Each lane owns one query column, so the row max / row sum of the online
// softmax are in-lane reductions plus one exchange between the two lane halves,
// and P goes from the S^T accumulators straight into the B operand of the P.V
// product without any shuffle: the 8 (bf16) keys a lane holds for one 16-deep
// MFMA step are matched by reading the same 8 keys of V^T.
//
// A workgroup is 4 waves. Per 128-key super-tile, the K rows and the
// transposed V rows are staged in LDS (next super-tile prefetched into
// registers meanwhile); wave w consumes keys [32w, 32w+32). The 4 waves' partial
// softmax states are merged through LDS at the end. When a block's prefix is
// split over several items, each item writes its partial (max, sum, O) and a
// combine kernel merges the splits in split order, so results do not depend on
// timing.
#pragma once

#include "common.h"

namespace dflash {

template <typename T> struct AttnArgs {
    const T* q; int64_t q_ld;          // [nb*bs, *] rows; head h at column h*D
    const T* kb; const T* vb; int64_t kv_ld;
    const T* ck; const T* cv; int64_t ctx_total;
    const int64_t* base; const int32_t* anchor; const uint8_t* valid;
    T* out; int64_t out_ld;
    int nb, bs, hq, hkv;
    float qscale;                      // log2(e) / sqrt(D)
    const int* item_start;             // [nb + 1] prefix sums of splits per block
    const int* chunk;                  // keys per split
    float* part_o;                     // [items][QC][D]
    float* part_ml;                    // [items][QC][2]
    RopeTurns rt;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float v) {
    return __shfl_xor(v, 32, 64);
}

template <typename T, int D, int QC>
struct AttnTile {
    static constexpr int EB = (int)sizeof(T);
    static constexpr int KSTEP = Mfma<T>::KSTEP, E = Mfma<T>::E;
    static constexpr int QS = QC / 32, DS = D / 32, DK = D / KSTEP, PK = 32 / KSTEP;
    static constexpr int KROW = D * EB + 16;          // bytes per K row in LDS
    static constexpr int SUPER = 128;                 // keys per super-tile
    static constexpr int VROW = SUPER * EB + 16;      // bytes per V^T row (prefix)
    static constexpr int BVROW = 32 * EB + 16;        // bytes per V^T row (block keys)
    static constexpr int KS_BYTES = SUPER * KROW;
    static constexpr int VT_BYTES = D * VROW;
    static constexpr int KB_BYTES = 32 * KROW;
    static constexpr int VB_BYTES = D * BVROW;
    static constexpr int MERGE_BYTES = 2 * (DS * QS * 16 * 64 * 4) + 4 * 2 * QS * 64 * 4;
    static constexpr int MAIN_BYTES = KS_BYTES + VT_BYTES;
    static constexpr int LDS_BYTES = (MAIN_BYTES > MERGE_BYTES ? MAIN_BYTES : MERGE_BYTES) + KB_BYTES + VB_BYTES;
    static constexpr int ROW_CHUNKS = D * EB / 16;    // 16-byte chunks per K/V row (16)
    static_assert(ROW_CHUNKS == 16, "a K/V row is 256 bytes");
    static constexpr int EC = 16 / EB;                // elements per 16-byte chunk
};

// One wave: fold a 32-key slice (K rows at ks, V^T at vt with row pitch vrow)
// with `nvalid` visible keys into the running softmax state.
template <typename T, int D, int QC>
__device__ __forceinline__ void attn_slice(const char* ks, const char* vt, int vrow, int nvalid,
                                           const typename Mfma<T>::frag (&qf)[QC / 32][D / Mfma<T>::KSTEP],
                                           f32x16 (&o)[D / 32][QC / 32], float (&m)[QC / 32],
                                           float (&l)[QC / 32], int lane) {
    using TT = AttnTile<T, D, QC>;
    typedef typename Mfma<T>::frag frag;
    constexpr int QS = TT::QS, DS = TT::DS, DK = TT::DK, PK = TT::PK, E = TT::E, EB = TT::EB;
    const int h = lane >> 5;
    f32x16 s[QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[qs][e] = 0.f;
    const char* krow = ks + (lane & 31) * TT::KROW + h * E * EB;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        frag a = *reinterpret_cast<const frag*>(krow + kk * TT::KSTEP * EB);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[qs] = Mfma<T>::mma(a, qf[qs][kk], s[qs]);
    }
    const float NEG_INF = -__builtin_inff();
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        float mx = NEG_INF;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (acc_row(e, lane) >= nvalid) s[qs][e] = NEG_INF;
            mx = fmaxf(mx, s[qs][e]);
        }
        mx = fmaxf(mx, xor32(mx));
        const float mnew = fmaxf(m[qs], mx);
        const float muse = (mnew == NEG_INF) ? 0.f : mnew;
        const float alpha = fast_exp2(m[qs] - muse);
        m[qs] = mnew;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s[qs][e] = fast_exp2(s[qs][e] - muse);
            ps += s[qs][e];
        }
        l[qs] = l[qs] * alpha + ps;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[ds][qs][e] *= alpha;
    }
    const char* vbase = vt + (lane & 31) * vrow;
#pragma unroll
    for (int st = 0; st < PK; ++st) {
        frag pf[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            if constexpr (E == 8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) pf[qs][i] = from_f32<T>(s[qs][st * 8 + i]);
            } else {
                pf[qs] = s[qs][st];
            }
        }
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            frag a;
            const char* vr = vbase + ds * 32 * vrow;
            if constexpr (E == 8) {
                u32x2 lo = *reinterpret_cast<const u32x2*>(vr + (16 * st + 4 * h) * EB);
                u32x2 hi = *reinterpret_cast<const u32x2*>(vr + (16 * st + 8 + 4 * h) * EB);
                u32x4 both = {lo[0], lo[1], hi[0], hi[1]};
                a = __builtin_bit_cast(frag, both);
            } else {
                a = *reinterpret_cast<const T*>(vr + acc_row(st, lane) * EB);
            }
#pragma unroll
            for (int qs = 0; qs < QS; ++qs) o[ds][qs] = Mfma<T>::mma(a, pf[qs], o[ds][qs]);
        }
    }
}

template <typename T, int D, int QC>
__global__ __launch_bounds__(256) void block_attn_kernel(AttnArgs<T> p) {
    using TT = AttnTile<T, D, QC>;
    typedef typename Mfma<T>::frag frag;
    constexpr int QS = TT::QS, DS = TT::DS, DK = TT::DK, E = TT::E, EB = TT::EB, EC = TT::EC;
    constexpr int KSTEP = TT::KSTEP, SUPER = TT::SUPER;
    __shared__ __attribute__((aligned(16))) char smem[TT::LDS_BYTES];
    char* Ks = smem;
    char* Vt = smem + TT::KS_BYTES;
    char* Kb = smem + (TT::LDS_BYTES - TT::KB_BYTES - TT::VB_BYTES);
    char* Vbt = Kb + TT::KB_BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int hkv = p.hkv, bs = p.bs, G = p.hq / p.hkv;
    const int total = p.item_start[p.nb] * hkv;
    const int item = blockIdx.x;
    if (item >= total) return;
    const int sg = item / hkv, g = item - sg * hkv;
    int lo = 0, hi = p.nb;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (p.item_start[mid] <= sg) lo = mid; else hi = mid;
    }
    const int n = lo;
    const int s = sg - p.item_start[n];
    const int nsplit = p.item_start[n + 1] - p.item_start[n];
    const int qcols = bs * G;

    int64_t base = p.base[n];
    base = base < 0 ? 0 : (base > p.ctx_total ? p.ctx_total : base);
    int a = p.anchor[n];
    if (a < 0) {                                   // empty block: zero rows
        if (s == 0) {
            for (int idx = tid; idx < bs * G * D; idx += 256) {
                int k = idx / (G * D), r = idx - k * G * D;
                p.out[(int64_t)(n * bs + k) * p.out_ld + (int64_t)g * G * D + r] = from_f32<T>(0.f);
            }
        }
        return;
    }
    if ((int64_t)a > p.ctx_total - base) a = (int)(p.ctx_total - base);
    const int chunk = *p.chunk;
    const int kbeg = s * chunk;
    const int kend = min(a, kbeg + chunk);

    // ---- queries: rotate at a + k, scale by log2(e)/sqrt(D), keep as B fragments
    frag qf[QS][DK];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        const int c = qs * 32 + (lane & 31);
        const bool live = c < qcols;
        const int k = live ? c % bs : 0, hh = live ? c / bs : 0;
        const T* qrow = p.q + (int64_t)(n * bs + k) * p.q_ld + (int64_t)(g * G + hh) * D;
        const int pos = a + k;
#pragma unroll
        for (int kk = 0; kk < DK / 2; ++kk) {
            float x1[E], x2[E];
            const int d0 = kk * KSTEP + h * E;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                x1[e] = live ? to_f32(qrow[d0 + e]) : 0.f;
                x2[e] = live ? to_f32(qrow[d0 + D / 2 + e]) : 0.f;
            }
            float y1[E], y2[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float cs, sn;
                rope_cs(p.rt, d0 + e, pos, cs, sn);
                y1[e] = (x1[e] * cs - x2[e] * sn) * p.qscale;
                y2[e] = (x2[e] * cs + x1[e] * sn) * p.qscale;
            }
            if constexpr (E == 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qf[qs][kk][e] = from_f32<T>(y1[e]);
                    qf[qs][kk + DK / 2][e] = from_f32<T>(y2[e]);
                }
            } else {
                qf[qs][kk] = y1[0];
                qf[qs][kk + DK / 2] = y2[0];
            }
        }
    }

    f32x16 o[DS][QS];
    float m[QS], l[QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        m[qs] = -__builtin_inff();
        l[qs] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[ds][qs][e] = 0.f;
    }

    // ---- the block's own keys (split 0 only): rotate K at a + k', stage K and V^T
    if (s == 0) {
        // K: 32 rows x D (rows >= bs are zero and masked)
        for (int idx = tid; idx < 32 * (D / 2); idx += 256) {
            const int k = idx / (D / 2), i = idx - k * (D / 2);
            float y1 = 0.f, y2 = 0.f;
            if (k < bs) {
                const T* kr = p.kb + (int64_t)(n * bs + k) * p.kv_ld + (int64_t)g * D;
                float x1 = to_f32(kr[i]), x2 = to_f32(kr[i + D / 2]);
                float cs, sn;
                rope_cs(p.rt, i, a + k, cs, sn);
                y1 = x1 * cs - x2 * sn;
                y2 = x2 * cs + x1 * sn;
            }
            *reinterpret_cast<T*>(Kb + k * TT::KROW + i * EB) = from_f32<T>(y1);
            *reinterpret_cast<T*>(Kb + k * TT::KROW + (i + D / 2) * EB) = from_f32<T>(y2);
        }
        for (int idx = tid; idx < 32 * D; idx += 256) {
            const int k = idx / D, d = idx - k * D;
            T v = from_f32<T>(0.f);
            if (k < bs) v = p.vb[(int64_t)(n * bs + k) * p.kv_ld + (int64_t)g * D + d];
            *reinterpret_cast<T*>(Vbt + d * TT::BVROW + k * EB) = v;
        }
        __syncthreads();
        if (wave == 0) attn_slice<T, D, QC>(Kb, Vbt, TT::BVROW, bs, qf, o, m, l, lane);
    }

    // ---- prefix: 128-key super-tiles, K rows and transposed V staged in LDS
    const int ntile = kend > kbeg ? (kend - kbeg + SUPER - 1) / SUPER : 0;
    const T* ckg = p.ck + (int64_t)g * p.ctx_total * D;
    const T* cvg = p.cv + (int64_t)g * p.ctx_total * D;
    u32x4 rk[8], rv[8];
    auto gload = [&](int t0) {
        // K: chunk c = tid + 256 i -> key c/16, column chunk c%16
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int key = t0 + (tid >> 4) + 16 * i;
            key = key < kend ? key : kend - 1;
            rk[i] = *reinterpret_cast<const u32x4*>(ckg + (base + key) * D + (tid & 15) * EC);
        }
        // V: two passes of 64 keys; thread owns keys 4*(tid/16)..+3 of a pass, chunk tid%16
#pragma unroll
        for (int ps = 0; ps < 2; ++ps)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int key = t0 + ps * 64 + 4 * (tid >> 4) + j;
                key = key < kend ? key : kend - 1;
                rv[ps * 4 + j] = *reinterpret_cast<const u32x4*>(cvg + (base + key) * D + (tid & 15) * EC);
            }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4*>(Ks + ((tid >> 4) + 16 * i) * TT::KROW + (tid & 15) * 16) = rk[i];
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const int key0 = ps * 64 + 4 * (tid >> 4);
            const T* v0 = reinterpret_cast<const T*>(&rv[ps * 4 + 0]);
            const T* v1 = reinterpret_cast<const T*>(&rv[ps * 4 + 1]);
            const T* v2 = reinterpret_cast<const T*>(&rv[ps * 4 + 2]);
            const T* v3 = reinterpret_cast<const T*>(&rv[ps * 4 + 3]);
#pragma unroll
            for (int e = 0; e < EC; ++e) {
                const int d = (tid & 15) * EC + e;
                T* dst = reinterpret_cast<T*>(Vt + d * TT::VROW + key0 * EB);
                dst[0] = v0[e]; dst[1] = v1[e]; dst[2] = v2[e]; dst[3] = v3[e];
            }
        }
    };

    if (ntile > 0) gload(kbeg);
    for (int t = 0; t < ntile; ++t) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (t + 1 < ntile) gload(kbeg + (t + 1) * SUPER);
        const int nvalid = kend - (kbeg + t * SUPER + wave * 32);
        if (nvalid > 0)
            attn_slice<T, D, QC>(Ks + wave * 32 * TT::KROW, Vt + wave * 32 * EB, TT::VROW,
                                 nvalid < 32 ? nvalid : 32, qf, o, m, l, lane);
    }

    // ---- merge the 4 waves: (3 -> 1, 2 -> 0), then (1 -> 0)
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) l[qs] += xor32(l[qs]);
    float* mo = reinterpret_cast<float*>(smem);                    // [2][DS][QS][16][64]
    float* mml = mo + 2 * DS * QS * 16 * 64;                       // [2][2][QS][64]
    auto put = [&](int slot) {
        float* dst = mo + slot * DS * QS * 16 * 64;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int qs = 0; qs < QS; ++qs)
#pragma unroll
                for (int e = 0; e < 16; ++e) dst[((ds * QS + qs) * 16 + e) * 64 + lane] = o[ds][qs][e];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            mml[((slot * 2 + 0) * QS + qs) * 64 + lane] = m[qs];
            mml[((slot * 2 + 1) * QS + qs) * 64 + lane] = l[qs];
        }
    };
    auto take = [&](int slot) {
        const float* src = mo + slot * DS * QS * 16 * 64;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const float m2 = mml[((slot * 2 + 0) * QS + qs) * 64 + lane];
            const float l2 = mml[((slot * 2 + 1) * QS + qs) * 64 + lane];
            const float mx = fmaxf(m[qs], m2);
            const float mu = (mx == -__builtin_inff()) ? 0.f : mx;
            const float f1 = fast_exp2(m[qs] - mu), f2 = fast_exp2(m2 - mu);
            m[qs] = mx;
            l[qs] = l[qs] * f1 + l2 * f2;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    o[ds][qs][e] = o[ds][qs][e] * f1 + src[((ds * QS + qs) * 16 + e) * 64 + lane] * f2;
        }
    };
    __syncthreads();
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) take(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    take(0);

    // ---- write: final rows, or this split's partial state
    if (nsplit == 1) {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int c = qs * 32 + (lane & 31);
            if (c >= qcols) continue;
            const int k = c % bs, hh = c / bs;
            const int row = n * bs + k;
            const bool keep = p.valid[row] != 0;
            const float inv = 1.f / l[qs];
            T* orow = p.out + (int64_t)row * p.out_ld + (int64_t)(g * G + hh) * D;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    orow[ds * 32 + acc_row(e, lane)] = from_f32<T>(keep ? o[ds][qs][e] * inv : 0.f);
        }
    } else {
        const int64_t pi = (int64_t)(p.item_start[n] + s) * hkv + g;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int c = qs * 32 + (lane & 31);
            float* po = p.part_o + (pi * QC + c) * D;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int e = 0; e < 16; ++e) po[ds * 32 + acc_row(e, lane)] = o[ds][qs][e];
            if (h == 0) {
                p.part_ml[(pi * QC + c) * 2 + 0] = m[qs];
                p.part_ml[(pi * QC + c) * 2 + 1] = l[qs];
            }
        }
    }
}

// Merge the splits of every block whose prefix was split, in split order.
template <typename T, int D, int QC>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs<T> p) {
    const int n = blockIdx.x, g = blockIdx.y;
    const int nsplit = p.item_start[n + 1] - p.item_start[n];
    if (nsplit <= 1 || p.anchor[n] < 0) return;
    const int G = p.hq / p.hkv, bs = p.bs, qcols = bs * G;
    for (int idx = threadIdx.x; idx < qcols * D; idx += blockDim.x) {
        const int c = idx / D, d = idx - c * D;
        float mx = -__builtin_inff();
        for (int s = 0; s < nsplit; ++s) {
            const int64_t pi = (int64_t)(p.item_start[n] + s) * p.hkv + g;
            mx = fmaxf(mx, p.part_ml[(pi * QC + c) * 2]);
        }
        float L = 0.f, acc = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const int64_t pi = (int64_t)(p.item_start[n] + s) * p.hkv + g;
            const float f = fast_exp2(p.part_ml[(pi * QC + c) * 2] - mx);
            L += p.part_ml[(pi * QC + c) * 2 + 1] * f;
            acc += p.part_o[(pi * QC + c) * D + d] * f;
        }
        const int k = c % bs, hh = c / bs, row = n * bs + k;
        p.out[(int64_t)row * p.out_ld + (int64_t)(g * G + hh) * D + d] =
            from_f32<T>(p.valid[row] != 0 ? acc / L : 0.f);
    }
}

// Splits per block: chunk = max(512, ceil(sum of prefixes / target) rounded up
// to a multiple of 128); block n gets max(1, ceil(a_n / chunk)) splits.
__global__ __launch_bounds__(1024) void attn_schedule_kernel(const int64_t* base, const int32_t* anchor,
                                                             int nb, int64_t ctx_total, int target,
                                                             int* item_start, int* chunk_out) {
    __shared__ long long red[1024];
    __shared__ int scan[1024];
    __shared__ int chunk_s;
    const int tid = threadIdx.x;
    auto a_eff = [&](int n) -> int64_t {
        int64_t b = base[n];
        b = b < 0 ? 0 : (b > ctx_total ? ctx_total : b);
        int64_t a = anchor[n];
        if (a < 0) return -1;
        return a > ctx_total - b ? ctx_total - b : a;
    };
    long long sum = 0;
    for (int n = tid; n < nb; n += 1024) {
        int64_t a = a_eff(n);
        sum += a > 0 ? a : 0;
    }
    red[tid] = sum;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) {
        long long per = (red[0] + target - 1) / target;
        per = (per + 127) / 128 * 128;
        if (per < 512) per = 512;
        if (per > (1 << 30)) per = 1 << 30;
        chunk_s = (int)per;
        *chunk_out = (int)per;
    }
    __syncthreads();
    const int chunk = chunk_s;
    const int per_t = (nb + 1023) / 1024;
    const int n0 = tid * per_t;
    int local = 0;
    for (int i = 0; i < per_t; ++i) {
        const int n = n0 + i;
        if (n < nb) {
            int64_t a = a_eff(n);
            local += a <= 0 ? 1 : (int)((a + chunk - 1) / chunk);
        }
    }
    scan[tid] = local;
    __syncthreads();
    for (int w = 1; w < 1024; w <<= 1) {
        int v = tid >= w ? scan[tid - w] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    int run = scan[tid] - local;
    for (int i = 0; i < per_t; ++i) {
        const int n = n0 + i;
        if (n < nb) {
            item_start[n] = run;
            int64_t a = a_eff(n);
            run += a <= 0 ? 1 : (int)((a + chunk - 1) / chunk);
        }
    }
    if (tid == 1023) item_start[nb] = scan[1023];
}

}  // namespace dflash
