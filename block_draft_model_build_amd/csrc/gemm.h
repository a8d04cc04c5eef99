// Tiled MFMA GEMM  C[M, N] = A[M, K] * B[N, K]^T  with fused epilogues.
//
// Both operands are K-contiguous (activations [rows, in], Linear weights
// [out, in]), so every 16-byte global load and every MFMA operand fragment is a
// contiguous K slice. One workgroup = 4 waves (256 threads) computes a BM x BN
// tile; each wave owns a WM x WN sub-tile made of 32x32 MFMA tiles. The K loop
// streams 64-byte-deep slabs of A and B straight into a 4-stage LDS ring (see
// gemm_nt_kernel).
//
// Operand "loaders" resolve row pointers, which lets a single GEMM read
// several weight matrices as one virtual B (Q|K|V, interleaved gate/up, every
// layer's K|V) and read stacked per-layer target states as one virtual A,
// without copying anything.
#pragma once

#include "common.h"

namespace dflash {

// BM x BN tile, WAVES_M x WAVES_N waves, K slabs of ROWB bytes per row, NST
// LDS stages.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int ROWB_ = 64, int NST_ = 4>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int ROWB = ROWB_, NST = NST_;
    static_assert(ROWB == 64 || ROWB == 128, "64- or 128-byte slabs");
    static_assert(NST >= 2 && NST <= 4, "2 to 4 stages");
    static constexpr int NW = WAVES_M * WAVES_N, THREADS = 64 * NW;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MI = WM / 32, NI = WN / 32;
    static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
    static constexpr int RUN = 1024 / ROWB;            // rows one 1 KB DMA instruction fills
    static_assert(BM % (RUN * NW) == 0 && BN % (RUN * NW) == 0, "whole DMA runs per wave");
};

// ---------------------------------------------------------------- A loaders
template <typename T> struct APlain {
    const T* a; int64_t ld;
    __device__ const T* row(int r) const { return a + (int64_t)r * ld; }
    __device__ const T* at(const T* p, int k0) const { return p + k0; }
};

// X[r, k] = a[r*rs + (k / ht)*ls + k % ht]; a K slab never straddles two layers.
template <typename T> struct AStacked {
    const T* a; int64_t rs, ls; int ht;
    __device__ const T* row(int r) const { return a + (int64_t)r * rs; }
    __device__ const T* at(const T* p, int k0) const {
        int layer = k0 / ht;
        return p + (int64_t)layer * ls + (k0 - layer * ht);
    }
};

// ---------------------------------------------------------------- B loaders
template <typename T> struct BPlain {
    const T* w; int64_t ld;
    __device__ const T* row(int n) const { return w + (int64_t)n * ld; }
};

// Rows past n_rows repeat the last row (a ragged N; the epilogue ignores them).
template <typename T> struct BClamp {
    const T* w; int64_t ld; int n_rows;
    __device__ const T* row(int n) const { return w + (int64_t)(n < n_rows ? n : n_rows - 1) * ld; }
};

// Rows [0, nq) of Wq, then Wk, then Wv.
template <typename T> struct BQKV {
    const T *wq, *wk, *wv; int nq, nk; int64_t ld;
    __device__ const T* row(int n) const {
        if (n < nq) return wq + (int64_t)n * ld;
        n -= nq;
        if (n < nk) return wk + (int64_t)n * ld;
        return wv + (int64_t)(n - nk) * ld;
    }
};

// Each WN-wide wave column holds WN/2 gate rows followed by the same WN/2 up
// rows, so SiLU(gate) * up pairs sit in one lane.
template <typename T, int WN> struct BGateUp {
    const T *wg, *wu; int64_t ld;
    __device__ const T* row(int n) const {
        int w = n / WN, r = n - w * WN;
        int o = w * (WN / 2) + (r < WN / 2 ? r : r - WN / 2);
        return (r < WN / 2 ? wg : wu) + (int64_t)o * ld;
    }
};

// Every layer's [Wk; Wv] stacked: row n -> layer n / (2*Hkv*D).
template <typename T> struct BCtxKV {
    const T* wk[kMaxLayers];
    const T* wv[kMaxLayers];
    int hkvd; int64_t ld;
    __device__ const T* row(int n) const {
        int l = n / (2 * hkvd), r = n - l * 2 * hkvd;
        return r < hkvd ? wk[l] + (int64_t)r * ld : wv[l] + (int64_t)(r - hkvd) * ld;
    }
};

// ---------------------------------------------------------------- epilogues
// Each epilogue receives one wave's accumulators: MI x NI tiles of 32x32 whose
// top-left element is (mb, nb) in the GEMM's (virtual) output.

template <typename T> struct EpStore {          // out[row, col] = acc
    T* out; int64_t ldo;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                T* o = out + (int64_t)row * ldo + nb + (lane & 31);
#pragma unroll
                for (int j = 0; j < NI; ++j) o[j * 32] = from_f32<T>(acc[i][j][e]);
            }
    }
};

// h[row, col] += acc (fp32 residual stream). With `out` set (last layer) the
// sum is not written back; instead out[row, col] = sum on rows that are valid
// and belong to a non-empty block (anchor >= 0), exact zero elsewhere.
template <typename T> struct EpResidual {
    float* h; int64_t ldh; T* out; const uint8_t* valid; const int32_t* anchor; int bs;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                float* hp = h + (int64_t)row * ldh + nb + (lane & 31);
                if (out == nullptr) {
#pragma unroll
                    for (int j = 0; j < NI; ++j) hp[j * 32] += acc[i][j][e];
                } else {
                    T* op = out + (int64_t)row * ldh + nb + (lane & 31);
                    bool keep = valid[row] != 0 && anchor[row / bs] >= 0;
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        op[j * 32] = keep ? from_f32<T>(hp[j * 32] + acc[i][j][e]) : from_f32<T>(0.f);
                }
            }
    }
};

// u[row, c] = SiLU(gate) * up with the BGateUp column order.
template <typename T> struct EpSwiGLU {
    T* u; int64_t ldu;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
        static_assert(NI % 2 == 0, "gate and up halves");
        const int c0 = (nb / WN) * (WN / 2) + (lane & 31);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                T* o = u + (int64_t)row * ldu + c0;
#pragma unroll
                for (int j = 0; j < NI / 2; ++j) {
                    float g = acc[i][j][e], up = acc[i][j + NI / 2][e];
                    o[j * 32] = from_f32<T>(g / (1.f + __expf(-g)) * up);
                }
            }
    }
};

// dst[row, col] = src[row, col] + acc (fp32 residual stream written to a new
// buffer: the layer's input stays intact for the backward).
struct EpAddF32 {
    const float* src; float* dst; int64_t ld;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                const int64_t o = (int64_t)row * ld + nb + (lane & 31);
#pragma unroll
                for (int j = 0; j < NI; ++j) dst[o + j * 32] = src[o + j * 32] + acc[i][j][e];
            }
    }
};

// The Q|K|V product (BQKV column order) stored as three packed matrices
// q [rows][nq], k [rows][nk], v [rows][nk]. nq and nk are multiples of 32, so a
// 32-column tile lies in one of them.
template <typename T> struct EpSplitQKV {
    T *q, *k, *v; int nq, nk;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int c = nb + j * 32;
            T* base;
            int64_t ld;
            if (c < nq) { base = q + c; ld = nq; }
            else if (c < nq + nk) { base = k + (c - nq); ld = nk; }
            else { base = v + (c - nq - nk); ld = nk; }
            base += lane & 31;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = mb + i * 32 + acc_row(e, lane);
                    if (row < M) base[(int64_t)row * ld] = from_f32<T>(acc[i][j][e]);
                }
        }
    }
};

// EpSwiGLU that also keeps the fp32 pre-activations gate[row, c] and
// up[row, c] (ld ldu) for the backward.
template <typename T> struct EpSwiGLUSave {
    T* u; float* gate; float* up; int64_t ldu;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
        static_assert(NI % 2 == 0, "gate and up halves");
        const int c0 = (nb / WN) * (WN / 2) + (lane & 31);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                const int64_t o = (int64_t)row * ldu + c0;
#pragma unroll
                for (int j = 0; j < NI / 2; ++j) {
                    float g = acc[i][j][e], p = acc[i][j + NI / 2][e];
                    u[o + j * 32] = from_f32<T>(g / (1.f + __expf(-g)) * p);
                    gate[o + j * 32] = g;
                    up[o + j * 32] = p;
                }
            }
    }
};

// Backward of u = SiLU(g) * up through the product du = dh W_down (acc = du at
// [row, c], c < I): with s = sigmoid(g),
//   dg = du * up * s * (1 + g (1 - s)),  dup = du * g * s,
// stored side by side, dgu[row, c] = dg and dgu[row, I + c] = dup (ld 2I).
template <typename T> struct EpSwiGLUBwd {
    const float* gate; const float* up; T* dgu; int I;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                const int c = nb + (lane & 31);
                const float* gp = gate + (int64_t)row * I + c;
                const float* up_ = up + (int64_t)row * I + c;
                T* o = dgu + (int64_t)row * 2 * I + c;
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    const float g = gp[j * 32], p = up_[j * 32], du = acc[i][j][e];
                    const float s = 1.f / (1.f + __expf(-g));
                    o[j * 32] = from_f32<T>(du * p * s * (1.f + g * (1.f - s)));
                    o[I + j * 32] = from_f32<T>(du * g * s);
                }
            }
    }
};

// fp32 rows split over up to three outputs: rows [0, s1) -> out0, [s1, s2) ->
// out1, [s2, M) -> out2, each [rows][ld] (stacked weight gradients).
struct EpStoreF32Rows3 {
    float* out0; float* out1; float* out2; int s1, s2; int64_t ld;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                float* o = row < s1 ? out0 + (int64_t)row * ld
                                    : row < s2 ? out1 + (int64_t)(row - s1) * ld : out2 + (int64_t)(row - s2) * ld;
                o += nb + (lane & 31);
#pragma unroll
                for (int j = 0; j < NI; ++j) o[j * 32] = acc[i][j][e];
            }
    }
};

// out[row, col] = acc in fp32.
struct EpStoreF32 {
    float* out; int64_t ldo;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                float* o = out + (int64_t)row * ldo + nb + (lane & 31);
#pragma unroll
                for (int j = 0; j < NI; ++j) o[j * 32] = acc[i][j][e];
            }
    }
};

// Block LM head with a fused softmax statistic: for every row, the maximum
// and sum of exp(z - max) over each WN-column group of logits z (columns past
// n_cols excluded), written to part[row][group], and the logit of the row's
// target token. The 32 lanes of a wave half hold 32 consecutive columns of a
// row, so each statistic is an in-lane pass over the NI column tiles plus a
// 5-step exchange within the half. With `logits` set the fp32 logits are kept
// too (logits[row * ldl + col], col < n_cols).
template <typename T> struct EpLseCE {
    float* part;                  // [M][groups][2]
    float* target_logit;          // [M]
    const int32_t* targets;       // [M]
    int groups, n_cols;
    float* logits = nullptr;      // optional [M][ldl]
    int64_t ldl = 0;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
        const int grp = nb / WN;
        if (grp >= groups) return;                  // a whole group past the vocabulary
        const int col = nb + (lane & 31);
        const float NEG_INF = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                float mx = NEG_INF;
#pragma unroll
                for (int j = 0; j < NI; ++j) mx = fmaxf(mx, col + j * 32 < n_cols ? acc[i][j][e] : NEG_INF);
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < NI; ++j) s += col + j * 32 < n_cols ? __expf(acc[i][j][e] - mx) : 0.f;
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
                if (row >= M) continue;
                if ((lane & 31) == 0) {
                    part[((int64_t)row * groups + grp) * 2 + 0] = mx;
                    part[((int64_t)row * groups + grp) * 2 + 1] = s;
                }
                const int t = targets[row];
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    if (col + j * 32 == t) target_logit[row] = acc[i][j][e];
                if (logits != nullptr) {
                    float* lr = logits + (int64_t)row * ldl;
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        if (col + j * 32 < n_cols) lr[col + j * 32] = acc[i][j][e];
                }
            }
    }
};

// Gradient of the decayed CE with respect to the logits z = acc:
// dz[row, col] = coef[row] * (exp(z - lse[row]) - [col == targets[row]]) for
// col < vocab, exact zero for vocab <= col < ldz (the padding the next product
// contracts over) and on rows whose coef is 0 (rows that do not count).
template <typename T> struct EpCEGrad {
    T* dz; int64_t ldz; const float* coef; const float* lse; const int32_t* targets; int vocab;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = mb + i * 32 + acc_row(e, lane);
                if (row >= M) continue;
                const float c = coef[row], L = lse[row];
                const int t = targets[row];
                T* o = dz + (int64_t)row * ldz;
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    const int col = nb + j * 32 + (lane & 31);
                    if (col >= ldz) continue;
                    float v = 0.f;
                    if (col < vocab && c != 0.f) v = c * (__expf(acc[i][j][e] - L) - (col == t ? 1.f : 0.f));
                    o[col] = from_f32<T>(v);
                }
            }
    }
};

// Context K/V: virtual column n = l*(2*Hkv*D) + [K heads | V heads]. K columns
// are rotated (pair d with d + D/2; both live in this wave because WN is a
// multiple of D and heads start at multiples of D) and written to the
// head-major cache [Hkv][ctx_total][D]; V columns go to the transposed cache
// [Hkv][D][ctx_total] (4 consecutive rows per lane -> one vector store).
template <typename T> struct EpCtxKV {
    T* ck[kMaxLayers];
    T* cv[kMaxLayers];
    const int* positions;
    const int64_t* dst_rows;      // cache row per GEMM row (scatter), or null: row_offset + row
    int64_t ctx_total, row_offset;
    int hkv;
    RopeTurns rt;
    // Cache row of GEMM row `row`, or -1 when it is not to be written.
    __device__ int64_t dst(int row) const {
        if (dst_rows == nullptr) return row_offset + row;
        const int64_t d = dst_rows[row];
        return d >= 0 && d < ctx_total ? d : -1;
    }
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
        constexpr int D = 256 / (int)sizeof(T);   // head rows are 256 bytes
        constexpr int half = D / 2;
        constexpr int pj = half / 32;             // partner tile distance
        static_assert(NI % (2 * pj) == 0, "a wave covers whole heads");
        typedef T T4 __attribute__((ext_vector_type(4)));
        const int hkvd = hkv * D;
        const bool vec_ok = dst_rows == nullptr && (row_offset & 3) == 0 && (ctx_total & 3) == 0;
#pragma unroll
        for (int q = 0; q < NI / 2; ++q) {
            const int j = (q / pj) * 2 * pj + q % pj;   // first tile of a (d, d + D/2) pair
            const int jp = j + pj;
            const int n = nb + j * 32;
            const int l = n / (2 * hkvd);
            const int r = n - l * 2 * hkvd;
            const bool is_v = r >= hkvd;
            const int rr = is_v ? r - hkvd : r;
            const int g = rr / D;
            const int dd = rr - g * D + (lane & 31);      // in [0, D/2)
            if (is_v) {
                T* v1 = cv[l] + ((int64_t)g * D + dd) * ctx_total;
                T* v2 = v1 + (int64_t)half * ctx_total;
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int eg = 0; eg < 4; ++eg) {
                        const int r0 = mb + i * 32 + acc_row(4 * eg, lane);   // 4 consecutive rows
                        if (vec_ok && r0 + 3 < M) {
                            T4 a1, a2;
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                a1[t] = from_f32<T>(acc[i][j][4 * eg + t]);
                                a2[t] = from_f32<T>(acc[i][jp][4 * eg + t]);
                            }
                            *reinterpret_cast<T4*>(v1 + row_offset + r0) = a1;
                            *reinterpret_cast<T4*>(v2 + row_offset + r0) = a2;
                        } else {
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                const int64_t crow = r0 + t < M ? dst(r0 + t) : -1;
                                if (crow >= 0) {
                                    v1[crow] = from_f32<T>(acc[i][j][4 * eg + t]);
                                    v2[crow] = from_f32<T>(acc[i][jp][4 * eg + t]);
                                }
                            }
                        }
                    }
            } else {
                T* kbase = ck[l] + (int64_t)g * ctx_total * D;
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = mb + i * 32 + acc_row(e, lane);
                        if (row >= M) continue;
                        const int64_t crow = dst(row);
                        if (crow < 0) continue;
                        T* o = kbase + crow * D;
                        const float x1 = acc[i][j][e], x2 = acc[i][jp][e];
                        float c, s;
                        rope_cs(rt, dd, positions[row], c, s);
                        o[dd] = from_f32<T>(x1 * c - x2 * s);
                        o[dd + half] = from_f32<T>(x2 * c + x1 * s);
                    }
            }
        }
    }
};

// ---------------------------------------------------------------- kernel


// 16-byte chunk swizzle of the LDS rows: row r keeps logical chunk c at
// physical chunk c ^ swz(r). Chosen by measuring LDS bank conflicts of the
// fragment read pattern (32 rows x one chunk per half-wave) on gfx950: these
// read conflict-free for 64- and 128-byte rows. swz(r + 32) == swz(r).
template <int ROWB> __device__ __forceinline__ int swz(int r) {
    return ROWB == 64 ? (r >> 2) & 3 : (r >> 1) & 7;
}

// Main loop: 64-byte-deep K slabs (32 bf16 / 16 fp32) of A and B move from
// global memory straight into LDS (global_load_lds_dwordx4: lane i of a wave
// writes LDS bytes [16i, 16i + 16) of a 1 KB run, i.e. 16 rows x 64 bytes), in
// a ring of 4 stages with 3 slabs in flight. One barrier per slab; MFMA
// fragments of the next k-step are read while the current one multiplies.
template <typename T, class Cfg, class AL, class BL, class EP>
__global__ __launch_bounds__(Cfg::THREADS) void gemm_nt_kernel(int M, int N, int K, AL al, BL bl, EP ep,
                                                                int group) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, MI = Cfg::MI, NI = Cfg::NI;
    constexpr int EB = (int)sizeof(T);
    constexpr int ROWB = Cfg::ROWB;                // bytes per LDS row (one K slab)
    constexpr int BK = ROWB / EB;
    constexpr int NST = Cfg::NST;                  // LDS stages
    constexpr int A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
    constexpr int NW = Cfg::NW, RUN = Cfg::RUN, CPR = ROWB / 16;
    constexpr int A_INST = BM / (RUN * NW), B_INST = BN / (RUN * NW);   // DMA runs per wave per slab
    constexpr int LPS = A_INST + B_INST;                // DMA instructions per wave per slab
    constexpr int KSTEP = Mfma<T>::KSTEP, E = Mfma<T>::E, KK = BK / KSTEP;
    typedef typename Mfma<T>::frag frag;

    __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

    // Tile order: consecutive tiles walk down M inside groups of `group` row
    // tiles so the B slab they share stays hot in L2 (chosen per call site).
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;   // B loaders clamp a ragged N
    int tm, tn;
    {
        // Workgroups are dealt round-robin to the 8 XCDs (each with its own
        // L2); renumber so that each XCD gets a contiguous run of tiles.
        int id = blockIdx.x;
        {
            const int G = tiles_m * tiles_n, G8 = G / 8 * 8;
            if (id < G8) id = (id % 8) * (G / 8) + id / 8;
        }
        const int per_group = group * tiles_n;
        const int gi = id / per_group;
        const int first_m = gi * group;
        const int gm = min(tiles_m - first_m, group);
        const int local = id - gi * per_group;
        tm = first_m + local % gm;
        tn = local / gm;
    }
    const int m0 = tm * BM, n0 = tn * BN;

    // DMA sources: wave w fills A rows [w*BM/NW, (w+1)*BM/NW) and B rows
    // [w*BN/NW, ...) in runs of RUN rows; lane -> (row lane/CPR, physical chunk lane%CPR).
    const T* ap[A_INST];
    const T* bp[B_INST];
    const int rr = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < A_INST; ++i) {
        const int r = wave * (BM / NW) + i * RUN + rr;
        const int gr = m0 + r < M ? m0 + r : M - 1;
        ap[i] = al.row(gr) + ((pc ^ swz<ROWB>(r)) * (16 / EB));
    }
#pragma unroll
    for (int i = 0; i < B_INST; ++i) {
        const int r = wave * (BN / NW) + i * RUN + rr;
        bp[i] = bl.row(n0 + r) + ((pc ^ swz<ROWB>(r)) * (16 / EB));
    }
    auto issue = [&](int kt) {
        char* st = smem + (kt % NST) * STAGE;
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < A_INST; ++i)
            __builtin_amdgcn_global_load_lds(DFLASH_GPTR(al.at(ap[i], k0)),
                                             DFLASH_LPTR(st + (wave * (BM / NW) + i * RUN) * ROWB), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < B_INST; ++i)
            __builtin_amdgcn_global_load_lds(DFLASH_GPTR(bp[i] + k0),
                                             DFLASH_LPTR(st + A_BYTES + (wave * (BN / NW) + i * RUN) * ROWB), 16,
                                             0, 0);
    };

    // Fragment addresses: lane reads row (lane % 32) of each 32-row sub-tile at
    // byte offset (kk*KSTEP + h*E)*EB of the row, through the swizzle.
    int foff[KK];
    {
        const int r = lane & 31;                  // swz(r + 32j) == swz(r)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int fb = (kk * KSTEP + h * E) * EB;
            foff[kk] = r * ROWB + (((fb >> 4) ^ swz<ROWB>(r)) << 4) + (fb & 15);
        }
    }

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = K / BK;
#pragma unroll
    for (int t = 0; t < NST - 1; ++t)
        if (t < KT) issue(t);

    // Slab t is complete (for every wave) once this wave has at most the
    // later slabs' DMAs outstanding and all waves have met at the barrier.
    auto wait_slab = [&](int t) {
        const int later = min(NST - 2, KT - 1 - t);
        if constexpr (NST >= 4) {
            if (later >= 2) wait_vmcnt<2 * LPS>();
            else if (later == 1) wait_vmcnt<LPS>();
            else wait_vmcnt<0>();
        } else if constexpr (NST == 3) {
            if (later >= 1) wait_vmcnt<LPS>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    frag af[2][MI], bf[2][NI];
    auto read_frags = [&](int t, int kk, int buf) {
        const char* st = smem + (t % NST) * STAGE;
        const char* a_base = st + (wm * Cfg::WM) * ROWB + foff[kk];
        const char* b_base = st + A_BYTES + (wn * Cfg::WN) * ROWB + foff[kk];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[buf][i] = *reinterpret_cast<const frag*>(a_base + i * 32 * ROWB);
#pragma unroll
        for (int j = 0; j < NI; ++j) bf[buf][j] = *reinterpret_cast<const frag*>(b_base + j * 32 * ROWB);
    };

    wait_slab(0);
    read_frags(0, 0, 0);
    for (int t = 0; t < KT; ++t) {
        // The stage slab t + NST - 1 lands in was last read in iteration t - 1,
        // whose reads all completed before this wave's previous barrier.
        if (t + NST - 1 < KT) issue(t + NST - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < KK) read_frags(t, kk + 1, cur ^ 1);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] = Mfma<T>::mma(af[cur][i], bf[cur][j], acc[i][j]);
            // Interleave the next k-step's fragment reads with these MFMAs.
            if (kk + 1 < KK) {
#pragma unroll
                for (int q = 0; q < MI + NI; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, MI * NI - (MI + NI), 0);
            }
        }
        // The last k-step's MFMAs are in flight: meet the other waves on the
        // next slab and start reading it meanwhile.
        if (t + 1 < KT) {
            __builtin_amdgcn_sched_barrier(0);
            wait_slab(t + 1);
            read_frags(t + 1, 0, KK & 1);
        }
    }
    static_assert(KK % 2 == 0, "fragment buffers alternate within a slab");

    ep.template apply<MI, NI, Cfg::WN>(m0 + wm * Cfg::WM, n0 + wn * Cfg::WN, acc, lane, M);
}

template <typename T, class Cfg, class AL, class BL, class EP>
hipError_t launch_gemm(int M, int N, int K, const AL& al, const BL& bl, const EP& ep,
                       hipStream_t stream, int group = 8) {
    if (M <= 0) return hipSuccess;
    const int tiles = ((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
    hipLaunchKernelGGL((gemm_nt_kernel<T, Cfg, AL, BL, EP>), dim3(tiles), dim3(Cfg::THREADS), 0, stream, M, N,
                       K, al, bl, ep, group);
    return hipGetLastError();
}

}  // namespace dflash
