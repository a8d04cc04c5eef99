// Dual-source block attention for gfx950.
//
// Work unit ("item"): a group of up to 4 consecutive blocks that read the same
// sequence (equal context base), one KV head g, and one split s of the group's
// prefix range. The 4 waves of the workgroup share every K/V tile: with 4
// blocks in the group each wave serves one block; with fewer, several waves
// serve one block and divide its keys. A block's query columns are its bs
// positions times the G = Hq/Hkv query heads of KV head g (<= 64 columns), so a
// K/V byte fetched once serves every query head of the group.
//
// Keys are the prefix rows [s*chunk, min(a, (s+1)*chunk)) of the projected
// context plus, for split 0, the block's own bs rows. A single-block group (bf16)
// split nsplit ways gives split s the 128-key tiles s, s + nsplit, ... of its
// prefix instead: its items run side by side and read neighbouring 256-byte
// pieces of each V^T row at about the same time (the transposed cache's rows are
// a whole context apart).
//
// Math layout (keys on MFMA rows, queries on MFMA columns):
//   S^T[key, q] = K[key, :] . Q[q, :]        A = K rows from LDS, B = Q in registers
//   O^T[d, q]  += V^T[d, key] . P^T[key, q]  A = V^T rows from LDS, B = P in registers
// Each lane owns one query column: the online-softmax max and sum are in-lane
// reductions plus one exchange between the two lane halves, and P goes from the
// S^T accumulators straight into the B operand of the P.V product. The K rows
// are fed to the S^T product in a permuted order (bits 2 and 3 of the row
// index swapped inside each 16-row group) so that the 8 P values a lane holds
// for one 16-key MFMA step belong to 8 consecutive keys; the matching V^T
// operand is then one 16-byte LDS read. The context V cache is stored
// transposed ([Hkv][D][T]) so V^T tiles are staged into LDS by plain copies.
//
// Per 128-key super-tile the K rows and V^T columns go into one of two LDS
// stages (bf16: direct-to-LDS loads, through registers only for a tile that
// crosses the end of the caches; fp32: through registers), one barrier per
// tile, the next tile in flight while this one is computed. A wave that owns
// its block and sees a tile whole runs the tile's slices software-pipelined
// (attn_tile_pipelined); partial tiles, and blocks shared by several waves (a
// group of one or two blocks), run slice by slice. Waves serving the same
// block merge their softmax states through LDS at the end. When a group's
// prefix is split over several items, each item writes per-block partial
// (max, sum, O) and a combine kernel merges the splits in split order, so
// results do not depend on timing.
#pragma once

#include <type_traits>

#include "common.h"
#include "dma_limits.h"

namespace dflash {

constexpr int kMaxGroup = 4;

template <typename T> struct AttnArgs {
    const T* q; int64_t q_ld;          // [nb*bs, *] rows; head h at column h*D
    const T* kb; const T* vb; int64_t kv_ld;
    const T* ck;                       // [Hkv][ctx_total][D], rotated
    const T* cvt;                      // [Hkv][D][ctx_total]
    int64_t ctx_total;
    const int64_t* base; const int32_t* anchor;
    const uint8_t* valid;              // rows written as zero where 0; null: every row kept
    T* out; int64_t out_ld;
    int nb, bs, hq, hkv;
    float qscale;                      // log2(e) / sqrt(D)
    const int* group_start;            // [groups + 1]
    const int* item_start;             // [groups + 1] prefix sums of splits per group
    const int* sched;                  // [0] keys per split of multi-block groups,
                                       // [1] number of groups, [2] of single-block groups,
                                       // [3] number of group-splits
    const int* meta;                   // [group-splits][16] item records in dispatch order (AttnMeta)
    const int4* bmeta;                 // [nb] block records (AttnBlockMeta)
    float* part_o;                     // [items][kMaxGroup][QC][D]
    float* part_ml;                    // [items][kMaxGroup][QC][2]
    int* redo;                         // [items][4]: a wave's scores outran its reference
    RopeTurns rt;
};

// Item record (16 int32 per group-split), written by the scheduler in
// dispatch order so that a workgroup fetches everything it needs to start in
// one scalar load instead of a chain of dependent ones.
enum AttnMeta {
    kMetaN0 = 0,        // first block of the group
    kMetaNg = 1,        // blocks in the group (1..4)
    kMetaS = 2,         // split index
    kMetaNsplit = 3,    // splits of the group
    kMetaChunk = 4,     // keys per split
    kMetaSg = 5,        // group-split index (item_start[group] + s)
    kMetaBaseLo = 6,    // clamped context base, low and high words
    kMetaBaseHi = 7,
    kMetaAnchor = 8,    // 8..11: effective anchors of the group's blocks (-1: absent or empty)
    kMetaAmax = 12,     // largest of them
};
// Block record: {first group-split of its group, splits, position in its group, effective anchor}.
enum AttnBlockMeta { kBmSg0 = 0, kBmNsplit = 1, kBmJ = 2, kBmAnchor = 3 };

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }
// Key fed to MFMA row r of a 32-key slice.
__device__ __forceinline__ int key_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// Key held by accumulator element e of a lane in half h of the wave:
// key_perm(acc_row(e, lane)) = (e & 7) + 16 (e >> 3) + 8 h. The e-dependent
// part is a compile-time constant, so masks compare against nvalid - 8 h.
__device__ __forceinline__ constexpr int acc_key(int e) { return (e & 7) + 16 * (e >> 3); }

__device__ __forceinline__ int64_t clamp_base(int64_t b, int64_t total) { return b < 0 ? 0 : (b > total ? total : b); }
__device__ __forceinline__ int anchor_eff(int a, int64_t base, int64_t total) {
    if (a < 0) return -1;
    return (int64_t)a > total - base ? (int)(total - base) : a;
}

template <typename T, int D, int QC>
struct AttnTile {
    static constexpr int EB = (int)sizeof(T);
    static constexpr int KSTEP = Mfma<T>::KSTEP, E = Mfma<T>::E;
    static constexpr int QS = QC / 32, DS = D / 32, DK = D / KSTEP, PK = 32 / KSTEP;
    static constexpr int SUPER = 128;                 // keys per super-tile
    // bf16: unpadded 256-byte K and V^T rows whose 16-byte chunks are XOR-
    // swizzled by (row & 15), which reads both fragment patterns without LDS
    // bank conflicts and lets whole rows arrive by direct-to-LDS loads. fp32:
    // rows padded by 16 bytes.
    static constexpr bool SWZ = EB == 2;
    static constexpr int KROW = SWZ ? D * EB : D * EB + 16;          // bytes per K row in LDS
    static constexpr int VROW = SWZ ? SUPER * EB : SUPER * EB + 16;  // bytes per V^T row in LDS
    static_assert(!SWZ || (D * EB == 256 && SUPER * EB == 256 && D == SUPER), "swizzled rows are 256 bytes");
    // Byte offset of byte b of K row r, and of key `key` in V^T row d.
    __device__ static __forceinline__ int koff(int r, int b) {
        return r * KROW + (SWZ ? ((((b >> 4) ^ (r & 15)) << 4) | (b & 15)) : b);
    }
    __device__ static __forceinline__ int voff(int d, int key) {
        const int b = key * EB;
        return d * VROW + (SWZ ? ((((b >> 4) ^ (d & 15)) << 4) | (b & 15)) : b);
    }
    static constexpr int KS_BYTES = SUPER * KROW;
    static constexpr int VT_BYTES = D * VROW;
    static constexpr int STAGE = KS_BYTES + VT_BYTES;
    // LDS layout: K stage 0, K stage 1, V^T stage 0, V^T stage 1 (bf16: 32 KB
    // each), so that with the stage known at compile time every fragment read
    // of a tile is a base register plus an immediate offset below 64 KB.
    __device__ static __forceinline__ char* kstage(char* smem, int stage) { return smem + stage * KS_BYTES; }
    __device__ static __forceinline__ char* vstage(char* smem, int stage) {
        return smem + 2 * KS_BYTES + stage * VT_BYTES;
    }
    static constexpr int SLOT_FLOATS = DS * QS * 16 * 64;
    static constexpr int MERGE_BYTES = 2 * SLOT_FLOATS * 4 + 2 * 2 * QS * 64 * 4;
    static constexpr int LDS_BYTES = 2 * STAGE > MERGE_BYTES ? 2 * STAGE : MERGE_BYTES;
    static constexpr int EC = 16 / EB;                // elements per 16-byte chunk
    static constexpr int KCH = D * EB / 16;           // 16-byte chunks per K row
    static constexpr int VCH = SUPER * EB / 16;       // 16-byte chunks per V^T row
    static_assert(KCH == 16, "a K row is 256 bytes");
    static_assert((SUPER * KCH) % 256 == 0 && (D * VCH) % 256 == 0, "whole chunks per thread");
    static constexpr int KLD = SUPER * KCH / 256;     // K chunks per thread per super-tile
    static constexpr int VLD = D * VCH / 256;         // V^T chunks per thread per super-tile
};

// One wave folds a 32-key slice into its running softmax state, given the
// slice's K fragments (kf[kk]: row key_perm(lane % 32), d-slice kk) and V^T
// fragments (vf[st][ds]: row d = 32 ds + lane % 32, keys 16 st + 8 (lane / 32)
// .. + 7 for bf16) of which the first `nvalid` keys are visible.
// S^T of a 32-key slice; getk(kk) returns the K fragment of d-step kk.
template <typename T, int D, int QC, class GetK>
__device__ __forceinline__ void attn_scores(const GetK& getk,
                                            const typename Mfma<T>::frag (&qf)[QC / 32][D / Mfma<T>::KSTEP],
                                            f32x16 (&s)[QC / 32]) {
    using TT = AttnTile<T, D, QC>;
    constexpr int QS = TT::QS, DK = TT::DK;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[qs][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        const typename Mfma<T>::frag a = getk(kk);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[qs] = Mfma<T>::mma(a, qf[qs][kk], s[qs]);
    }
}

// Two ways to keep P = 2^(s - m) in range (O and l always share the reference m,
// so both give the same softmax):
// - fixed (LAZY false): m is the maximum of the first visible keys of each query
//   column and never moves, so O is never rescaled inside the key loop; mt
//   tracks the true maximum, and the kernel flags its item for a second,
//   LAZY run when some column's scores rose more than kFixedRange above m;
// - lazy (LAZY true): m moves when some column's scores pass it by more than
//   kLazy, and O and l are rescaled then.
constexpr float kFixedRange = 32.f;
// Range guard of the pipelined tiles, which track no maximum: a column whose
// row sum l (relative to m) passes this is flagged for the LAZY run. Every P
// of the column is then at most l, and |O| at most l * max |V|.
constexpr float kFixedSum = 1099511627776.f;   // 2^40

// Softmax half of a slice: masks keys at or past `nvalid`, updates the running
// state (m, l, mt; O is rescaled only in the lazy form) and returns P = 2^(s - m)
// as the B operand of the P.V product (pf[st][qs]: keys 16 st .. 16 st + 15).
template <typename T, int D, int QC, bool LAZY>
__device__ __forceinline__ void attn_softmax(f32x16 (&s)[QC / 32], int nvalid, f32x16 (&o)[D / 32][QC / 32],
                                             float (&m)[QC / 32], float (&l)[QC / 32], float (&mt)[QC / 32],
                                             typename Mfma<T>::frag (&pf)[32 / Mfma<T>::KSTEP][QC / 32], int lane) {
    using TT = AttnTile<T, D, QC>;
    constexpr int QS = TT::QS, DS = TT::DS, PK = TT::PK, E = TT::E;
    const int h = lane >> 5;
    constexpr float kLazy = 8.f;
    const float NEG_INF = -__builtin_inff();
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        float mx = NEG_INF;
        if (nvalid < 32) {
            const int nv = nvalid - 8 * h;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (acc_key(e) >= nv) s[qs][e] = NEG_INF;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qs][e]);
        mx = fmaxf(mx, xor32(mx));
        if constexpr (LAZY) {
            const bool grow = mx > m[qs] + kLazy;    // also true on the first visible keys
            if (__any(grow)) {
                const float mnew = grow ? mx : m[qs];
                const float alpha = (m[qs] == NEG_INF) ? 0.f : fast_exp2(m[qs] - mnew);
                m[qs] = mnew;
                l[qs] *= alpha;
#pragma unroll
                for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[ds][qs][e] *= alpha;
            }
        } else {
            if (m[qs] == NEG_INF) m[qs] = mx;
            mt[qs] = fmaxf(mt[qs], mx);
        }
        const float muse = (m[qs] == NEG_INF) ? 0.f : m[qs];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s[qs][e] = fast_exp2(s[qs][e] - muse);
            ps += s[qs][e];
        }
        l[qs] += ps;
    }
#pragma unroll
    for (int st = 0; st < PK; ++st)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            if constexpr (E == 8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) pf[st][qs][i] = from_f32<T>(s[qs][st * 8 + i]);
            } else {
                pf[st][qs] = s[qs][st];
            }
        }
}

// P.V half of a slice: O^T += V^T P^T; getv(st, ds) returns the V^T fragment of
// MFMA step st, d-tile ds. Keys at or past `nvalid` enter as exact zeros of V,
// even where V is not finite.
template <typename T, int D, int QC, class GetV>
__device__ __forceinline__ void attn_pv(const typename Mfma<T>::frag (&pf)[32 / Mfma<T>::KSTEP][QC / 32],
                                        const GetV& getv, int nvalid, f32x16 (&o)[D / 32][QC / 32], int lane) {
    using TT = AttnTile<T, D, QC>;
    typedef typename Mfma<T>::frag frag;
    constexpr int QS = TT::QS, DS = TT::DS, PK = TT::PK, E = TT::E;
    const int h = lane >> 5;
#pragma unroll
    for (int st = 0; st < PK; ++st)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            frag a = getv(st, ds);
            if (nvalid < 32) {
                const int nv = nvalid - 8 * h;
                if constexpr (E == 8) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (16 * st + i >= nv) a[i] = from_f32<T>(0.f);
                } else {
                    if (acc_key(st) >= nv) a = 0.f;
                }
            }
#pragma unroll
            for (int qs = 0; qs < QS; ++qs) o[ds][qs] = Mfma<T>::mma(a, pf[st][qs], o[ds][qs]);
        }
}

template <typename T, int D, int QC, bool LAZY, class GetV>
__device__ __forceinline__ void attn_update(f32x16 (&s)[QC / 32], const GetV& getv, int nvalid,
                                            f32x16 (&o)[D / 32][QC / 32], float (&m)[QC / 32],
                                            float (&l)[QC / 32], float (&mt)[QC / 32], int lane) {
    typename Mfma<T>::frag pf[32 / Mfma<T>::KSTEP][QC / 32];
    attn_softmax<T, D, QC, LAZY>(s, nvalid, o, m, l, mt, pf, lane);
    attn_pv<T, D, QC>(pf, getv, nvalid, o, lane);
}

// One wave folds the 32-key slice starting at key0 of a tile staged in LDS
// (K rows at ks, V^T rows at vt; `nvalid` visible keys) into its running
// softmax state.
template <typename T, int D, int QC, bool LAZY>
__device__ __forceinline__ void attn_slice(const char* ks, const char* vt, int key0, int nvalid,
                                           const typename Mfma<T>::frag (&qf)[QC / 32][D / Mfma<T>::KSTEP],
                                           f32x16 (&o)[D / 32][QC / 32], float (&m)[QC / 32],
                                           float (&l)[QC / 32], float (&mt)[QC / 32], int lane) {
    using TT = AttnTile<T, D, QC>;
    typedef typename Mfma<T>::frag frag;
    constexpr int E = TT::E, EB = TT::EB;
    const int h = lane >> 5;
    const int kr = key0 + key_perm(lane & 31);
    f32x16 sc[QC / 32];
    attn_scores<T, D, QC>(
        [&](int kk) { return *reinterpret_cast<const frag*>(ks + TT::koff(kr, (kk * TT::KSTEP + h * E) * EB)); },
        qf, sc);
    auto getv = [&](int st, int ds) -> frag {
        const int d = ds * 32 + (lane & 31);
        if constexpr (E == 8)
            return *reinterpret_cast<const frag*>(vt + TT::voff(d, key0 + 16 * st + 8 * h));
        else
            return *reinterpret_cast<const T*>(vt + TT::voff(d, key0 + acc_key(st) + 8 * h));
    };
    attn_update<T, D, QC, LAZY>(sc, getv, nvalid, o, m, l, mt, lane);
}

// Softmax of one query half qs of a slice with every key visible, fixed
// reference. With SET the scores are raw: their maximum sets the reference m
// of columns that have none yet (and feeds the true maximum mt). Otherwise
// the score product started from -m, so P = 2^s directly; mt is not tracked
// there, and the row sum l guards the range instead (block_attn_kernel flags
// an item whose l passes kFixedSum).
template <typename T, int D, int QC, bool SET>
__device__ __forceinline__ void attn_softmax_half(f32x16& s, int qs, float (&m)[QC / 32], float (&l)[QC / 32],
                                                  float (&mt)[QC / 32], typename Mfma<T>::frag (&pf)[32 / Mfma<T>::KSTEP]) {
    constexpr int PK = 32 / Mfma<T>::KSTEP;
    if constexpr (SET) {
        const float NEG_INF = -__builtin_inff();
        float mx = NEG_INF;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = fmaxf(mx, xor32(mx));
        if (m[qs] == NEG_INF) m[qs] = mx;
        mt[qs] = fmaxf(mt[qs], mx);
        const float muse = (m[qs] == NEG_INF) ? 0.f : m[qs];
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] -= muse;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = fast_exp2(s[e]);
#pragma unroll
    for (int st = 0; st < PK; ++st)
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[st][i] = from_f32<T>(s[st * 8 + i]);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += s[e];
    l[qs] += ps;
}

// One wave folds all four 32-key slices of a 128-key bf16 tile staged in LDS,
// every key visible, with the fixed softmax reference. Work is split into
// units u = 2 * slice + qs (a slice's scores for one half of the query
// columns), which are independent in the softmax and in the P.V product. The
// units are software-pipelined: stage u runs the score MFMAs of unit u + 1
// and the P.V MFMAs of unit u - 1 on the matrix cores while the vector units
// run the softmax of unit u (none of the three depends on another, and with
// the fixed reference the softmax never touches O). FIRST: the columns have
// no reference yet, and units 0 and 1 set it.
template <typename T, int D, int QC, bool FIRST>
__device__ __forceinline__ void attn_tile_pipelined(const char* ks, const char* vt,
                                                    const typename Mfma<T>::frag (&qf)[QC / 32][D / Mfma<T>::KSTEP],
                                                    f32x16 (&o)[D / 32][QC / 32], float (&m)[QC / 32],
                                                    float (&l)[QC / 32], float (&mt)[QC / 32], int lane) {
    using TT = AttnTile<T, D, QC>;
    typedef typename Mfma<T>::frag frag;
    constexpr int QS = TT::QS, PK = TT::PK, E = TT::E, EB = TT::EB, DK = TT::DK, DS = TT::DS;
    static_assert(E == 8 && TT::SWZ && QS == 2, "bf16 tiles, two query halves");
    const int h = lane >> 5;
    const int kr = key_perm(lane & 31);
    frag kf[DK], vf[PK][DS];
    f32x16 sc[QS];
    frag pf[QS][PK];
    auto load_k = [&](int sl) {
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            kf[kk] = *reinterpret_cast<const frag*>(ks + TT::koff(sl * 32 + kr, (kk * TT::KSTEP + h * E) * EB));
    };
    auto load_v = [&](int sl) {
#pragma unroll
        for (int st = 0; st < PK; ++st)
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
                vf[st][ds] = *reinterpret_cast<const frag*>(vt + TT::voff(ds * 32 + (lane & 31), sl * 32 + 16 * st + 8 * h));
    };
    // Unit u's scores start from -m (0 for the units that set m).
    auto scores = [&](int u) {
        const int qs = u & 1;
        const float init = (FIRST && u < 2) ? 0.f : -m[qs];
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[qs][e] = init;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) sc[qs] = Mfma<T>::mma(kf[kk], qf[qs][kk], sc[qs]);
    };
    auto pv = [&](int qs) {
#pragma unroll
        for (int st = 0; st < PK; ++st)
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) o[ds][qs] = Mfma<T>::mma(vf[st][ds], pf[qs][st], o[ds][qs]);
    };
    load_k(0);
    scores(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        // unit u + 1 needs the K fragments of slice (u + 1) / 2, unit u - 1 the
        // V fragments of slice (u - 1) / 2: both are new on odd u.
        if (u & 1) {
            if (u + 1 < 8) load_k((u + 1) >> 1);
            load_v((u - 1) >> 1);
        }
        if (u + 1 < 8) scores(u + 1);
        if (u >= 1) pv((u - 1) & 1);
        if (FIRST && u < 2)
            attn_softmax_half<T, D, QC, true>(sc[u & 1], u & 1, m, l, mt, pf[u & 1]);
        else
            attn_softmax_half<T, D, QC, false>(sc[u & 1], u & 1, m, l, mt, pf[u & 1]);

        __builtin_amdgcn_sched_barrier(0);
    }
    pv(1);
}

// The main instantiation runs every item with the fixed softmax reference
// and records per wave whether its scores outran it. The REDO instantiation,
// launched after it, runs only the items so recorded, with the lazily moved
// reference, and overwrites their results.
template <typename T, int D, int QC, bool REDO = false>
__global__ __launch_bounds__(256) void block_attn_kernel(AttnArgs<T> p) {
    using TT = AttnTile<T, D, QC>;
    typedef typename Mfma<T>::frag frag;
    constexpr int QS = TT::QS, DS = TT::DS, DK = TT::DK, E = TT::E, EB = TT::EB, EC = TT::EC;
    constexpr int KSTEP = TT::KSTEP, SUPER = TT::SUPER;
    __shared__ __attribute__((aligned(16))) char smem[TT::LDS_BYTES];

    // The wave index is uniform across the wave: scalar registers for everything derived from it.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5;
    const int hkv = p.hkv, bs = p.bs, G = p.hq / p.hkv;
    // Item records are stored in dispatch order (longest work first):
    // workgroup b runs record b / hkv for KV head hkv - 1 - b % hkv.
    const int slot = (int)blockIdx.x / hkv;
    if (slot >= p.sched[3]) return;
    const int g = hkv - 1 - ((int)blockIdx.x - slot * hkv);
    const int* rec = p.meta + 16 * (int64_t)slot;
    const int n0 = rec[kMetaN0], ng = rec[kMetaNg], s = rec[kMetaS], nsplit = rec[kMetaNsplit];
    const int chunk = rec[kMetaChunk], sg = rec[kMetaSg], amax = rec[kMetaAmax];
    const int64_t base = (int64_t)(uint32_t)rec[kMetaBaseLo] | ((int64_t)rec[kMetaBaseHi] << 32);
    const int anc[kMaxGroup] = {rec[kMetaAnchor], rec[kMetaAnchor + 1], rec[kMetaAnchor + 2], rec[kMetaAnchor + 3]};
    auto anchor_of = [&](int jj) {                    // jj < ng
        return jj == 0 ? anc[0] : (jj == 1 ? anc[1] : (jj == 2 ? anc[2] : anc[3]));
    };
    const int item = sg * hkv + g;                    // index of this item's partials and redo flags
    if constexpr (REDO) {
        const int4 f = *reinterpret_cast<const int4*>(p.redo + 4 * (int64_t)item);
        if ((f.x | f.y | f.z | f.w) == 0) return;
    }
    const int wpb = ng == 1 ? 4 : (ng == 2 ? 2 : 1);   // waves per block
    const int j = wave / wpb;                          // this wave's block in the group
    const int phase = wave - j * wpb;                  // this wave's share of the block's keys
    const bool active = j < ng;
    const int qcols = bs * G;
    const int kbeg = s * chunk;

    const int n = n0 + (active ? j : 0);
    const int a = active ? anchor_of(j) : -1;
    const int kend_g = min(amax, kbeg + chunk);
    const int kend = min(a, kbeg + chunk);
    // Single-block groups split over several items take interleaved tiles
    // (split s of nsplit: tiles s, s + nsplit, ...), so the items of one group,
    // dispatched together, read neighbouring pieces of the V^T rows together.
    const bool ilv = TT::SWZ && ng == 1 && nsplit > 1;
    const int tfirst = ilv ? s * SUPER : kbeg, tstep = ilv ? nsplit * SUPER : SUPER;
    const int kclamp = ilv ? amax : kend_g;       // end of the keys this item may read
    const int kvalid = ilv ? a : kend;            // end of this wave's block's visible keys

    // ---- queries of this wave's block, rotated at a + k and scaled by
    // log2(e)/sqrt(D). Their loads are issued here, with the own keys' loads,
    // before the first context tile's DMA; the rotation comes after it, so the
    // tile streams in while both are processed (loads complete in issue order).
    frag qf[QS][DK];
    u32x4 qraw[QS][DK / 2][2];
    float qraw1[QS][DK / 2][2];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        const int c = qs * 32 + (lane & 31);
        const bool live = a >= 0 && c < qcols;
        const int k = live ? c % bs : 0, hh = live ? c / bs : 0;
        const T* qrow = p.q + (int64_t)(n * bs + k) * p.q_ld + (int64_t)(g * G + hh) * D;
#pragma unroll
        for (int kk = 0; kk < DK / 2; ++kk) {
            const int d0 = kk * KSTEP + h * E;
            if constexpr (E == 8) {
                qraw[qs][kk][0] = qraw[qs][kk][1] = u32x4{0, 0, 0, 0};
                if (live) {
                    qraw[qs][kk][0] = *reinterpret_cast<const u32x4*>(qrow + d0);
                    qraw[qs][kk][1] = *reinterpret_cast<const u32x4*>(qrow + d0 + D / 2);
                }
            } else {
                qraw1[qs][kk][0] = live ? to_f32(qrow[d0]) : 0.f;
                qraw1[qs][kk][1] = live ? to_f32(qrow[d0 + D / 2]) : 0.f;
            }
        }
    }
    auto rotate_q = [&]() {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int c = qs * 32 + (lane & 31);
            const bool live = a >= 0 && c < qcols;
            const int k = live ? c % bs : 0;
            const int pos = (a >= 0 ? a : 0) + k;
#pragma unroll
            for (int kk = 0; kk < DK / 2; ++kk) {
                const int d0 = kk * KSTEP + h * E;
                float x1[E], x2[E];
                if constexpr (E == 8) {
                    bf16x8 v1 = __builtin_bit_cast(bf16x8, qraw[qs][kk][0]);
                    bf16x8 v2 = __builtin_bit_cast(bf16x8, qraw[qs][kk][1]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) { x1[e] = to_f32(v1[e]); x2[e] = to_f32(v2[e]); }
                } else {
                    x1[0] = qraw1[qs][kk][0];
                    x2[0] = qraw1[qs][kk][1];
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float cs, sn;
                    rope_cs(p.rt, d0 + e, pos, cs, sn);
                    const float y1 = (x1[e] * cs - x2[e] * sn) * p.qscale;
                    const float y2 = (x2[e] * cs + x1[e] * sn) * p.qscale;
                    if constexpr (E == 8) {
                        qf[qs][kk][e] = from_f32<T>(y1);
                        qf[qs][kk + DK / 2][e] = from_f32<T>(y2);
                    } else {
                        qf[qs][kk] = y1;
                        qf[qs][kk + DK / 2] = y2;
                    }
                }
            }
        }
        // Q is only ever an MFMA operand, which may sit in AGPRs (gfx950): keep
        // it there and leave the VGPRs to the softmax and the K/V fragments.
        if constexpr (E == 8) {
#pragma unroll
            for (int qs = 0; qs < QS; ++qs)
#pragma unroll
                for (int kk = 0; kk < DK; ++kk) asm volatile("" : "+a"(qf[qs][kk]));
        }
    };

    f32x16 o[DS][QS];
    float m[QS], l[QS], mt[QS];          // reference, sum, true maximum (attn_update)
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        m[qs] = mt[qs] = -__builtin_inff();
        l[qs] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[ds][qs][e] = 0.f;
    }

    // ---- context rows of the group: K rows and V^T columns [kbeg, kend_g) of the
    // sequence's range of the caches, in 128-key super-tiles through 2 LDS stages.
    const int ntile = ilv ? (amax > tfirst ? (amax - tfirst + tstep - 1) / tstep : 0)
                          : (kend_g > kbeg ? (kend_g - kbeg + SUPER - 1) / SUPER : 0);
    const T* ckg = p.ck + ((int64_t)g * p.ctx_total + base) * D;
    const T* cvg = p.cvt + (int64_t)g * D * p.ctx_total + base;
    const int64_t lim = p.ctx_total - base;          // keys of this range present in the caches
    u32x4 rk[TT::KLD], rv[TT::VLD];
    // Register path: K rows past the group's end repeat its last row, V^T keys
    // past it are zero, so nothing outside [0, kclamp) is read.
    auto gload = [&](int t0) {
        // K: chunk c = tid + 256 i -> key c / 16, 16-byte column c % 16
#pragma unroll
        for (int i = 0; i < TT::KLD; ++i) {
            const int c = tid + 256 * i;
            int key = t0 + c / TT::KCH;
            key = key < kclamp ? key : kclamp - 1;
            rk[i] = *reinterpret_cast<const u32x4*>(ckg + (int64_t)key * D + (c % TT::KCH) * EC);
        }
        // V^T: chunk c -> row d = c / VCH, keys t0 + (c % VCH) * EC ..
#pragma unroll
        for (int i = 0; i < TT::VLD; ++i) {
            const int c = tid + 256 * i;
            const int d = c / TT::VCH;
            const int key = t0 + (c % TT::VCH) * EC;
            const T* src = cvg + (int64_t)d * p.ctx_total + key;
            if (key + EC <= kclamp) {
                rv[i] = *reinterpret_cast<const u32x4*>(src);
            } else {
                T tmp[EC];
#pragma unroll
                for (int e = 0; e < EC; ++e) tmp[e] = key + e < kclamp ? src[e] : from_f32<T>(0.f);
                rv[i] = *reinterpret_cast<const u32x4*>(tmp);
            }
        }
    };
    auto lstore = [&](int stage) {
        char* Ks = TT::kstage(smem, stage);
        char* Vt = TT::vstage(smem, stage);
#pragma unroll
        for (int i = 0; i < TT::KLD; ++i) {
            const int c = tid + 256 * i;
            *reinterpret_cast<u32x4*>(Ks + TT::koff(c / TT::KCH, (c % TT::KCH) * 16)) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < TT::VLD; ++i) {
            const int c = tid + 256 * i;
            *reinterpret_cast<u32x4*>(Vt + TT::voff(c / TT::VCH, (c % TT::VCH) * EC)) = rv[i];
        }
    };
    // Direct-to-LDS path (bf16, tiles inside the cache range): each wave moves
    // 32 K rows and 32 V^T rows, 4 rows of 256 bytes per instruction; lane i
    // lands at physical chunk i % 16 of row i / 16, so it fetches the logical
    // chunk (i % 16) ^ (row & 15). Keys past the group's end are read as they
    // are: scores there are masked and V there is zeroed before use.
    auto tile_dma_ok = [&](int t0) {
        return TT::SWZ && (int64_t)t0 + SUPER <= lim && p.ctx_total <= vt_dma_max_ctx(EB, TT::EC);
    };
    // Sources are a wave-uniform base plus a 32-bit lane offset; the swizzle
    // (row & 15) repeats every 4 instructions, so 4 lane offsets serve all 8
    // rows of each cache. The largest V^T lane offset, (15 * ctx_total +
    // 15 * EC) * EB bytes, fits in 32 bits only up to vt_dma_max_ctx rows
    // (143,165,568 for bf16); tile_dma_ok sends longer caches down the
    // register-staged path, so no offset below wraps.
    const int rsub = lane >> 4, pc = lane & 15;
    uint32_t koff_l[4], voff_l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = i * 4 + rsub;                   // row within a 16-row swizzle period
        koff_l[i] = (uint32_t)(r * D + (pc ^ r) * EC) * EB;
        voff_l[i] = (uint32_t)((int64_t)r * p.ctx_total + (pc ^ r) * EC) * EB;
    }
    auto issue_dma = [&](int t0, int stage) {
        if constexpr (TT::SWZ) {
            char* Ks = TT::kstage(smem, stage);
            char* Vt = TT::vstage(smem, stage);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int R = wave * 32 + i * 4;      // first row of this instruction
                const char* kb = reinterpret_cast<const char*>(ckg + (int64_t)(t0 + R - (i & 3) * 4) * D);
                __builtin_amdgcn_global_load_lds(DFLASH_GPTR(kb + koff_l[i & 3]), DFLASH_LPTR(Ks + R * TT::KROW), 16,
                                                 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int R = wave * 32 + i * 4;
                const char* vb = reinterpret_cast<const char*>(cvg + (int64_t)(R - (i & 3) * 4) * p.ctx_total + t0);
                __builtin_amdgcn_global_load_lds(DFLASH_GPTR(vb + voff_l[i & 3]), DFLASH_LPTR(Vt + R * TT::VROW), 16,
                                                 0, 0);
            }
        }
    };

    constexpr int OWN = TT::SWZ ? 1 : 0;

    // ---- split 0: the blocks' own keys. Block jj's rows go to slot jj (32 rows)
    // of stage OWN: K rotated at its anchor + k', V^T transposed; rows >= bs zero.
    // Every 16-byte chunk of the group's K and V rows is requested before any
    // is used (one round trip to memory, not one per element), and before the
    // first context tile's DMA. K row chunks c and c + KCH/2 hold the rotation
    // partners (i, i + D/2).
    constexpr int HC = TT::KCH / 2;
    constexpr int KIT = (kMaxGroup * 32 * HC + 255) / 256;
    constexpr int VIT = (kMaxGroup * 32 * TT::KCH + 255) / 256;
    const int nrows = ng * bs;
    u32x4 k1[KIT], k2[KIT], vv[VIT];
    if (s == 0) {
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int w = tid + 256 * it, row = w / HC, c = w - row * HC;
            k1[it] = k2[it] = u32x4{0, 0, 0, 0};
            if (row < nrows) {
                const int jj = row / bs, k = row - jj * bs;
                const T* kr = p.kb + (int64_t)((n0 + jj) * bs + k) * p.kv_ld + (int64_t)g * D;
                k1[it] = *reinterpret_cast<const u32x4*>(kr + c * EC);
                k2[it] = *reinterpret_cast<const u32x4*>(kr + (c + HC) * EC);
            }
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int w = tid + 256 * it, row = w / TT::KCH, c = w - row * TT::KCH;
            vv[it] = u32x4{0, 0, 0, 0};
            if (row < nrows) {
                const int jj = row / bs, k = row - jj * bs;
                vv[it] = *reinterpret_cast<const u32x4*>(p.vb + (int64_t)((n0 + jj) * bs + k) * p.kv_ld +
                                                         (int64_t)g * D + c * EC);
            }
        }
    }
    // bf16 stages the first tile while the queries and the blocks' own keys are
    // processed (they use stage 1); fp32 stages its tiles from registers below.
    if constexpr (TT::SWZ) {
        if (ntile > 0 && tile_dma_ok(tfirst)) issue_dma(tfirst, 0);
    }
    rotate_q();
    if (s == 0) {
        char* Ks = TT::kstage(smem, OWN);
        char* Vt = TT::vstage(smem, OWN);
        // Block jj's rows go to slot jj (32 rows) of stage OWN: K rotated at its
        // anchor + k, V^T transposed. Rows bs..31 of a slot are never read
        // unmasked (the own-key slice masks keys past bs), nor are empty blocks'.
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int w = tid + 256 * it, row = w / HC, c = w - row * HC;
            if (row < nrows) {
                const int jj = row / bs, k = row - jj * bs;
                const int aj = anchor_of(jj);
                T x1[EC], x2[EC], y1[EC], y2[EC];
                *reinterpret_cast<u32x4*>(x1) = k1[it];
                *reinterpret_cast<u32x4*>(x2) = k2[it];
#pragma unroll
                for (int e = 0; e < EC; ++e) {
                    float cs, sn;
                    rope_cs(p.rt, c * EC + e, (aj >= 0 ? aj : 0) + k, cs, sn);
                    const float f1 = to_f32(x1[e]), f2 = to_f32(x2[e]);
                    y1[e] = from_f32<T>(f1 * cs - f2 * sn);
                    y2[e] = from_f32<T>(f2 * cs + f1 * sn);
                }
                *reinterpret_cast<u32x4*>(Ks + TT::koff(jj * 32 + k, c * 16)) = *reinterpret_cast<u32x4*>(y1);
                *reinterpret_cast<u32x4*>(Ks + TT::koff(jj * 32 + k, (c + HC) * 16)) = *reinterpret_cast<u32x4*>(y2);
            }
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int w = tid + 256 * it, row = w / TT::KCH, c = w - row * TT::KCH;
            if (row < nrows) {
                const int jj = row / bs, k = row - jj * bs;
                T v[EC];
                *reinterpret_cast<u32x4*>(v) = vv[it];
#pragma unroll
                for (int e = 0; e < EC; ++e) *reinterpret_cast<T*>(Vt + TT::voff(c * EC + e, jj * 32 + k)) = v[e];
            }
        }
        __syncthreads();
        if (active && phase == 0 && a >= 0) attn_slice<T, D, QC, REDO>(Ks, Vt, j * 32, bs, qf, o, m, l, mt, lane);
        __syncthreads();
    }

    // One tile of this wave's block: its slices phase, phase + wpb, ...
    auto tile_compute = [&](int t) {
        if (active && a >= 0) {
            const char* Ks = TT::kstage(smem, t & 1);
            const char* Vt = TT::vstage(smem, t & 1);
            for (int sl = phase; sl < SUPER / 32; sl += wpb) {
                const int nvalid = kvalid - (tfirst + t * tstep + sl * 32);
                if (nvalid > 0)
                    attn_slice<T, D, QC, REDO>(Ks, Vt, sl * 32, nvalid < 32 ? nvalid : 32, qf, o, m, l, mt, lane);
            }
        }
    };
    if constexpr (TT::SWZ) {
        // Tile t + 1 is staged into the other stage while tile t is computed:
        // by DMA when it lies inside the cache range, else (a tile crossing the
        // end of the caches) through registers after this tile's work.
        if (ntile > 0 && !tile_dma_ok(tfirst)) {
            gload(tfirst);
            lstore(0);
        }
        wait_vmcnt<0>();
        __syncthreads();
        // Leading tiles that this wave's block sees whole, with one wave per
        // block: pipelined slices (attn_tile_pipelined); the tiles after them
        // slice by slice. The count is per wave (uniform within it): both
        // loops stage each tile the same way and meet the workgroup at one
        // barrier per tile, so the waves of a group whose anchors lie in
        // different tiles switch loops at different tiles.
        int nfull = 0;
        if constexpr (!REDO && QS == 2) {
            if (wpb == 1 && active && a >= 0) {
                const int kv = min(a, kbeg + chunk);
                nfull = kv > kbeg ? min(ntile, (kv - kbeg) / SUPER) : 0;
            }
        }
        auto stage_next = [&](int t, auto&& compute) {
            const int t1 = tfirst + (t + 1) * tstep;
            const bool next = t + 1 < ntile;
            const bool dma = next && tile_dma_ok(t1);
            if (dma) issue_dma(t1, (t + 1) & 1);
            compute(t);
            if (next && !dma) {
                gload(t1);
                lstore((t + 1) & 1);
            }
            wait_vmcnt<0>();
            __syncthreads();
        };
        int t = 0;
        if constexpr (!REDO && QS == 2) {
            // The stage of each tile is a compile-time constant (tile t sits
            // in stage t & 1): pairs of tiles per iteration.
            auto piped = [&](int tt, auto first, auto stage) {
                stage_next(tt, [&](int) {
                    if (active)
                        attn_tile_pipelined<T, D, QC, decltype(first)::value>(
                            TT::kstage(smem, decltype(stage)::value), TT::vstage(smem, decltype(stage)::value), qf, o,
                            m, l, mt, lane);
                });
            };
            using S0 = std::integral_constant<int, 0>;
            using S1 = std::integral_constant<int, 1>;
            using F0 = std::integral_constant<bool, false>;
            // Splits after the first have no own keys: their first tile sets
            // the reference.
            if (s > 0 && nfull > 0) {
                piped(0, std::integral_constant<bool, true>(), S0());
                t = 1;
            }
            if (t < nfull && (t & 1)) piped(t++, F0(), S1());
            for (; t + 1 < nfull; t += 2) {
                piped(t, F0(), S0());
                piped(t + 1, F0(), S1());
            }
            if (t < nfull) piped(t++, F0(), S0());
        }
        for (; t < ntile; ++t) stage_next(t, tile_compute);
    }
    if constexpr (!TT::SWZ) {
        if (ntile > 0) {
            gload(kbeg);
            lstore(0);
            if (ntile > 1) gload(kbeg + SUPER);
        }
        for (int t = 0; t < ntile; ++t) {
            __syncthreads();
            if (t + 1 < ntile) lstore((t + 1) & 1);
            if (t + 2 < ntile) gload(kbeg + (t + 2) * SUPER);
            tile_compute(t);
        }
    }

    if constexpr (!REDO) {
        bool over = false;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) over |= mt[qs] > m[qs] + kFixedRange || !(l[qs] <= kFixedSum);
        over = __any(over);
        if (lane == 0) p.redo[4 * (int64_t)item + wave] = over ? 1 : 0;
    }

    // ---- merge the waves serving one block (tree over phases), via LDS
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) l[qs] += xor32(l[qs]);
    float* mo = reinterpret_cast<float*>(smem);                  // [2 slots][DS][QS][16][64]
    float* mml = mo + 2 * TT::SLOT_FLOATS;                       // [2 slots][2][QS][64]
    for (int step = 1; step < 4; step <<= 1) {
        __syncthreads();
        if (step < wpb && active && (phase % (2 * step)) == step) {
            const int slot = wave >> 1;
            float* dst = mo + slot * TT::SLOT_FLOATS;
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
        }
        __syncthreads();
        if (step < wpb && active && (phase % (2 * step)) == 0) {
            const int slot = (wave + step) >> 1;
            const float* src = mo + slot * TT::SLOT_FLOATS;
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
        }
    }
    // The merge's last LDS reads are done: the LDS now stages the outputs.
    __syncthreads();
    if (!active || phase != 0) return;

    // ---- write: final rows of this block, or this split's partial state.
    // A lane holds 4 consecutive d of one column (32 qs + lane % 32), so
    // direct stores scatter 8-byte pieces over 32 rows per instruction. The
    // final rows go through this wave's LDS region instead (16-byte chunks
    // XOR-swizzled by the row), then out as 16-byte lanes, 256 contiguous
    // bytes per row (writes then reads by the same wave: a wave-level fence
    // between them). The fp32 partial state keeps its direct 16-byte stores:
    // staged the same way it measured no faster.
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    if (a < 0) {
        if (s == 0)
            for (int idx = lane; idx < bs * G * D; idx += 64) {
                const int k = idx / (G * D), r = idx - k * G * D;
                p.out[(int64_t)(n * bs + k) * p.out_ld + (int64_t)g * G * D + r] = from_f32<T>(0.f);
            }
        return;
    }
    if (nsplit == 1) {
        constexpr int RB = D * EB, NCH = RB / 16;      // bytes and 16-byte chunks per row
        static_assert(4 * QC * RB <= TT::LDS_BYTES, "four waves' rows fit in the LDS");
        char* st = smem + wave * QC * RB;
        typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int c = qs * 32 + (lane & 31);
            const int row = n * bs + (c < qcols ? c % bs : 0);
            const bool keep = c < qcols && (p.valid == nullptr || p.valid[row] != 0);
            const float inv = keep ? 1.f / l[qs] : 0.f;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int eg = 0; eg < 4; ++eg) {
                    T4 v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = from_f32<T>(o[ds][qs][4 * eg + t] * inv);
                    const int b = (ds * 32 + acc_row(4 * eg, lane)) * EB;
                    *reinterpret_cast<T4*>(st + c * RB + ((((b >> 4) ^ (c & (NCH - 1)))) << 4) + (b & 15)) = v;
                }
        }
        wave_sync();
#pragma unroll
        for (int i = 0; i < QC * NCH / 64; ++i) {
            const int idx = i * 64 + lane, c = idx / NCH, ch = idx % NCH;
            if (c >= qcols) continue;
            const int k = c % bs, hh = c / bs;
            const u32x4 v = *reinterpret_cast<const u32x4*>(st + c * RB + ((ch ^ (c & (NCH - 1))) << 4));
            *reinterpret_cast<u32x4*>(p.out + (int64_t)(n * bs + k) * p.out_ld + (int64_t)(g * G + hh) * D + ch * EC) = v;
        }
    } else {
        const int64_t pi = ((int64_t)sg * hkv + g) * kMaxGroup + j;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int c = qs * 32 + (lane & 31);
            float* po = p.part_o + (pi * QC + c) * D;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int eg = 0; eg < 4; ++eg) {
                    f32x4 v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = o[ds][qs][4 * eg + t];
                    *reinterpret_cast<f32x4*>(po + ds * 32 + acc_row(4 * eg, lane)) = v;
                }
            if (h == 0) {
                p.part_ml[(pi * QC + c) * 2 + 0] = m[qs];
                p.part_ml[(pi * QC + c) * 2 + 1] = l[qs];
            }
        }
    }
}

// Merge the splits of a block whose group's prefix was split, in split order:
// per query column the global max and 1/sum first, then every output element
// as one weighted sum over the splits. One workgroup per (block, KV head).
template <typename T, int D, int QC>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs<T> p) {
    constexpr int MAXF = 32;                       // splits whose weights are kept in LDS
    __shared__ float s_mu[QC], s_inv[QC];
    __shared__ float s_f[MAXF][QC];
    // One workgroup per (block, KV head); the block's record says where its
    // group's splits are.
    const int n = blockIdx.x, g = blockIdx.y;
    const int4 bm = p.bmeta[n];
    const int nsplit = bm[kBmNsplit];
    if (nsplit <= 1 || bm[kBmAnchor] < 0) return;
    const int j = bm[kBmJ], sg0 = bm[kBmSg0];
    const int G = p.hq / p.hkv, bs = p.bs, qcols = bs * G;
    const int tid = threadIdx.x;
    auto part = [&](int s) -> int64_t { return ((int64_t)(sg0 + s) * p.hkv + g) * kMaxGroup + j; };
    for (int c = tid; c < qcols; c += 256) {
        float mx = -__builtin_inff();
        for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, p.part_ml[(part(s) * QC + c) * 2]);
        const float mu = (mx == -__builtin_inff()) ? 0.f : mx;
        float L = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float f = fast_exp2(p.part_ml[(part(s) * QC + c) * 2] - mu);
            if (s < MAXF) s_f[s][c] = f;
            L += p.part_ml[(part(s) * QC + c) * 2 + 1] * f;
        }
        s_mu[c] = mu;
        s_inv[c] = 1.f / L;
    }
    __syncthreads();
    for (int idx = tid; idx < qcols * (D / 4); idx += 256) {
        const int c = idx / (D / 4), d = (idx - c * (D / 4)) * 4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < nsplit; ++s) {
            const float f = s < MAXF ? s_f[s][c] : fast_exp2(p.part_ml[(part(s) * QC + c) * 2] - s_mu[c]);
            const f32x4 v = *reinterpret_cast<const f32x4*>(p.part_o + (part(s) * QC + c) * D + d);
            acc += v * f;
        }
        const int k = c % bs, hh = c / bs, row = n * bs + k;
        const bool keep = p.valid == nullptr || p.valid[row] != 0;
        T* o = p.out + (int64_t)row * p.out_ld + (int64_t)(g * G + hh) * D + d;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(keep ? acc[e] * s_inv[c] : 0.f);
    }
}

// Groups and splits. A group starts at every block whose index is a multiple
// of 4 or whose (clamped) context base differs from the previous block's. A
// group's stream length is its largest (clamped) anchor. Single-block and
// multi-block groups get separate split sizes: chunk = max(256, ceil(sum of
// their lengths / target) rounded up to 128), target_single (single) or
// target_shared (multi) splits in total; a group gets max(1, ceil(length /
// chunk)) splits. The multi-block chunk then grows in 128-key steps until its
// groups' splits (each rounded up) fit the target. The item records are
// written longest work first.
//
// One workgroup of 1024 threads. Up to kSchedCache groups, every group's
// start, length and first item sit in LDS once computed (each later phase
// would otherwise wait on dependent global loads again), and sums and scans
// go through wave shuffles with one barrier per step.
constexpr int kSchedCache = 4096;
static __global__ __launch_bounds__(1024) void attn_schedule_kernel(const int64_t* base, const int32_t* anchor, int nb,
                                                             int64_t ctx_total, int target_shared, int target_single,
                                                             int* group_start, int* item_start, int* sched, int* meta,
                                                             int4* bmeta) {
    __shared__ int gs_s[kSchedCache + 1], gl_s[kSchedCache], is_s[kSchedCache + 1];
    __shared__ int wscan[16];
    __shared__ long long wred[2][16];
    __shared__ int chunk_s[2];
    __shared__ long long sum_s[2];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per_t = (nb + 1023) / 1024;
    const int b0 = tid * per_t;
    auto starts = [&](int n) {
        return n == 0 || (n & 3) == 0 || clamp_base(base[n], ctx_total) != clamp_base(base[n - 1], ctx_total);
    };
    auto block_run = [&](int n) {
        int64_t b = clamp_base(base[n], ctx_total);
        return anchor_eff(anchor[n], b, ctx_total);
    };
    // Exclusive prefix of v over the threads in index order; *total = the sum.
    auto exclusive_scan = [&](int v, int* total) {
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o, 64);
            if (lane >= o) incl += u;
        }
        if (lane == 63) wscan[wv] = incl;
        __syncthreads();
        int before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int x = wscan[w];
            before += w < wv ? x : 0;
            all += x;
        }
        __syncthreads();
        *total = all;
        return before + incl - v;
    };
    // Sums of a and b over all threads (integers: any order gives the same).
    auto block_sum2 = [&](long long a, long long b, long long* sa, long long* sb) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            a += __shfl_xor(a, o, 64);
            b += __shfl_xor(b, o, 64);
        }
        if (lane == 0) {
            wred[0][wv] = a;
            wred[1][wv] = b;
        }
        __syncthreads();
        long long ta = 0, tb = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            ta += wred[0][w];
            tb += wred[1][w];
        }
        __syncthreads();
        *sa = ta;
        *sb = tb;
    };
    // 1. group starts
    int cnt = 0;
    for (int i = 0; i < per_t; ++i) if (b0 + i < nb && starts(b0 + i)) ++cnt;
    int ng;
    int gidx = exclusive_scan(cnt, &ng);
    for (int i = 0; i < per_t; ++i)
        if (b0 + i < nb && starts(b0 + i)) {
            if (gidx <= kSchedCache) gs_s[gidx] = b0 + i;
            group_start[gidx++] = b0 + i;
        }
    if (tid == 0) {
        group_start[ng] = nb;
        if (ng <= kSchedCache) gs_s[ng] = nb;
    }
    __threadfence_block();
    __syncthreads();
    const bool cached = ng <= kSchedCache;
    auto gstart = [&](int gi) { return cached ? gs_s[gi] : group_start[gi]; };
    auto group_len_of = [&](int gi) {
        int mx = -1;
        for (int n = gstart(gi), e = gstart(gi + 1); n < e; ++n) mx = max(mx, block_run(n));
        return mx;
    };
    // 2. group lengths -> the two split sizes
    const int gper = (ng + 1023) / 1024;
    const int g0 = tid * gper;
    if (cached) {
        for (int i = 0; i < gper; ++i)
            if (g0 + i < ng) gl_s[g0 + i] = group_len_of(g0 + i);
        __syncthreads();
    }
    auto group_len = [&](int gi) { return cached ? gl_s[gi] : group_len_of(gi); };
    auto single = [&](int gi) { return gstart(gi + 1) - gstart(gi) == 1; };
    {
        long long sum[2] = {0, 0};
        for (int i = 0; i < gper; ++i)
            if (g0 + i < ng) sum[single(g0 + i) ? 1 : 0] += max(group_len(g0 + i), 0);
        long long t0, t1;
        block_sum2(sum[0], sum[1], &t0, &t1);
        if (tid < 2) {
            const long long tot = tid == 0 ? t0 : t1;
            const int target = tid == 0 ? target_shared : target_single;
            sum_s[tid] = tot;
            long long c = (tot + target - 1) / target;
            c = (c + 127) / 128 * 128;
            if (c < 256) c = 256;
            if (c > (1 << 30)) c = 1 << 30;
            chunk_s[tid] = (int)c;
        }
        __syncthreads();
    }
    // Multi-block groups: rounding each group's split count up can exceed the
    // target. When there are fewer such groups than the target, binary-search
    // (in 128-key steps) the smallest chunk whose total split count fits,
    // between the chunk above and sum / (target - groups), which always fits;
    // their items then fill one round of workgroups as evenly as it allows.
    auto count_multi = [&](long long c) {            // called by every thread
        long long local_cnt = 0;
        for (int i = 0; i < gper; ++i)
            if (g0 + i < ng && !single(g0 + i)) {
                const int len = group_len(g0 + i);
                local_cnt += len <= 0 ? 1 : (len + c - 1) / c;
            }
        long long tot, unused;
        block_sum2(local_cnt, 0, &tot, &unused);
        return tot;
    };
    {
        const long long n_multi = count_multi(1LL << 30);
        long long lo = chunk_s[0];
        if (n_multi > 0 && n_multi < target_shared && count_multi(lo) > target_shared) {
            long long hi = (sum_s[0] + (target_shared - n_multi) - 1) / (target_shared - n_multi);
            hi = (hi + 127) / 128 * 128;
            if (hi > (1 << 30)) hi = 1 << 30;
            while (hi - lo > 128) {                   // count(lo) > target >= count(hi)
                long long mid = (lo + hi) / 2 / 128 * 128;
                if (mid <= lo) mid = lo + 128;
                if (count_multi(mid) <= target_shared) hi = mid; else lo = mid;
            }
            if (tid == 0) chunk_s[0] = (int)hi;
        }
        __syncthreads();
    }
    if (tid < 2) sched[tid == 0 ? 0 : 2] = chunk_s[tid];
    if (tid == 0) sched[1] = ng;
    // 3. splits per group -> item_start
    auto splits = [&](int gi) {
        const int len = group_len(gi);
        const int chunk = chunk_s[single(gi) ? 1 : 0];
        return len <= 0 ? 1 : (len + chunk - 1) / chunk;
    };
    int local = 0;
    for (int i = 0; i < gper; ++i)
        if (g0 + i < ng) local += splits(g0 + i);
    int nsg;
    int run = exclusive_scan(local, &nsg);
    for (int i = 0; i < gper; ++i)
        if (g0 + i < ng) {
            if (cached) is_s[g0 + i] = run;
            item_start[g0 + i] = run;
            run += splits(g0 + i);
        }
    if (tid == 0) {
        item_start[ng] = nsg;
        if (cached) is_s[ng] = nsg;
        sched[3] = nsg;
    }
    __syncthreads();
    auto first_item = [&](int gi) { return cached ? is_s[gi] : item_start[gi]; };
    // 4. dispatch order: longest work first (each item's visible keys plus a
    //    fixed cost for its start), ties by group-split index, so the longest
    //    items start together and the short ones fill the tail. Ranks are
    //    counted by comparison (deterministic). Beyond kSortMax group-splits
    //    the reverse of block order is used (blocks come in ascending anchor
    //    order within a sequence).
    constexpr int kSortMax = 4096;
    __shared__ int key_s[kSortMax], rank_s[kSortMax];
    const bool sorted = nsg <= kSortMax;
    if (sorted) {
        for (int i = 0; i < gper; ++i) {
            const int gi = g0 + i;
            if (gi >= ng) continue;
            const int len = max(group_len(gi), 0), ns = splits(gi);
            const int chunk = chunk_s[single(gi) ? 1 : 0];
            const bool ilv = single(gi) && ns > 1;
            for (int sp = 0; sp < ns; ++sp) {
                const int keys = ilv ? (len + ns - 1) / ns : max(0, min(len, (sp + 1) * chunk) - sp * chunk);
                key_s[first_item(gi) + sp] = keys + (sp == 0 ? 384 : 256);
            }
        }
        __syncthreads();
        for (int x = tid; x < nsg; x += 1024) {
            const int kx = key_s[x];
            int r = 0;
            for (int y = 0; y < nsg; ++y) {
                const int ky = key_s[y];
                r += ky > kx || (ky == kx && y < x);
            }
            rank_s[x] = r;
        }
        __syncthreads();
    }
    for (int i = 0; i < gper; ++i) {
        const int gi = g0 + i;
        if (gi >= ng) continue;
        const int n0 = gstart(gi), cnt_g = gstart(gi + 1) - n0;
        const int ns = splits(gi), sg0 = first_item(gi);
        const int chunk = chunk_s[single(gi) ? 1 : 0];
        const int64_t b = clamp_base(base[n0], ctx_total);
        int a[kMaxGroup], amax = -1;
        for (int jj = 0; jj < kMaxGroup; ++jj) {
            a[jj] = jj < cnt_g ? block_run(n0 + jj) : -1;
            amax = max(amax, a[jj]);
        }
        for (int jj = 0; jj < cnt_g; ++jj) bmeta[n0 + jj] = make_int4(sg0, ns, jj, a[jj]);
        for (int s = 0; s < ns; ++s) {
            int* m = meta + 16 * (int64_t)(sorted ? rank_s[sg0 + s] : nsg - 1 - (sg0 + s));
            m[kMetaN0] = n0;
            m[kMetaNg] = cnt_g;
            m[kMetaS] = s;
            m[kMetaNsplit] = ns;
            m[kMetaChunk] = chunk;
            m[kMetaSg] = sg0 + s;
            m[kMetaBaseLo] = (int)(uint32_t)(uint64_t)b;
            m[kMetaBaseHi] = (int)((uint64_t)b >> 32);
            for (int jj = 0; jj < kMaxGroup; ++jj) m[kMetaAnchor + jj] = a[jj];
            m[kMetaAmax] = amax;
            m[13] = m[14] = m[15] = 0;
        }
    }
}

}  // namespace dflash
