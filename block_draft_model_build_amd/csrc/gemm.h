// Tiled MFMA GEMM  C[M, N] = A[M, K] * B[N, K]^T  with fused epilogues.
//
// Both operands are K-contiguous (activations [rows, in], Linear weights
// [out, in]), so every 16-byte global load and every MFMA operand fragment is a
// contiguous K slice. One workgroup = 4 waves (256 threads) computes a BM x BN
// tile; each wave owns a WM x WN sub-tile made of 32x32 MFMA tiles. The K loop
// moves 128-byte-deep slabs (64 bf16 / 32 fp32) of A and B through LDS, double
// buffered, with the next slab prefetched into registers while the current one
// feeds the matrix cores. LDS rows are padded by 16 bytes so the 32 rows one
// fragment load touches fall on distinct banks.
//
// Operand "loaders" resolve row pointers, which lets a single GEMM read
// several weight matrices as one virtual B (Q|K|V, interleaved gate/up, every
// layer's K|V) and read stacked per-layer target states as one virtual A,
// without copying anything.
#pragma once

#include "common.h"

namespace dflash {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MI = WM / 32, NI = WN / 32;
    static_assert(WAVES_M * WAVES_N == 4, "4 waves per workgroup");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
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

// Context K/V: virtual column n = l*(2*Hkv*D) + [K heads | V heads]. K columns
// are rotated (pair d with d + D/2; both live in this wave because WN is a
// multiple of D and heads start at multiples of D) and written to the
// head-major cache [Hkv][ctx_total][D]; V columns go to the transposed cache
// [Hkv][D][ctx_total] (4 consecutive rows per lane -> one vector store).
template <typename T> struct EpCtxKV {
    T* ck[kMaxLayers];
    T* cv[kMaxLayers];
    const int* positions;
    int64_t ctx_total, row_offset;
    int hkv;
    RopeTurns rt;
    template <int MI, int NI, int WN>
    __device__ void apply(int mb, int nb, f32x16 (&acc)[MI][NI], int lane, int M) const {
        constexpr int D = 256 / (int)sizeof(T);   // head rows are 256 bytes
        constexpr int half = D / 2;
        constexpr int pj = half / 32;             // partner tile distance
        static_assert(NI % (2 * pj) == 0, "a wave covers whole heads");
        typedef T T4 __attribute__((ext_vector_type(4)));
        const int hkvd = hkv * D;
        const bool vec_ok = (row_offset & 3) == 0 && (ctx_total & 3) == 0;
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
                T* v1 = cv[l] + ((int64_t)g * D + dd) * ctx_total + row_offset;
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
                            *reinterpret_cast<T4*>(v1 + r0) = a1;
                            *reinterpret_cast<T4*>(v2 + r0) = a2;
                        } else {
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                if (r0 + t < M) {
                                    v1[r0 + t] = from_f32<T>(acc[i][j][4 * eg + t]);
                                    v2[r0 + t] = from_f32<T>(acc[i][jp][4 * eg + t]);
                                }
                        }
                    }
            } else {
                T* kbase = ck[l] + ((int64_t)g * ctx_total + row_offset) * D;
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = mb + i * 32 + acc_row(e, lane);
                        if (row >= M) continue;
                        T* o = kbase + (int64_t)row * D;
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
template <typename T, class Cfg, class AL, class BL, class EP>
__global__ __launch_bounds__(256) void gemm_nt_kernel(int M, int N, int K, AL al, BL bl, EP ep) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, MI = Cfg::MI, NI = Cfg::NI;
    constexpr int ROWB = 128 + 16;                 // bytes per padded LDS row
    constexpr int EB = (int)sizeof(T);
    constexpr int BK = 128 / EB;
    constexpr int ACH = BM / 32, BCH = BN / 32;    // 16-byte chunks per thread per slab
    constexpr int KSTEP = Mfma<T>::KSTEP, E = Mfma<T>::E;
    typedef typename Mfma<T>::frag frag;

    __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * ROWB];
    auto sA = [&](int buf) { return smem + buf * (BM + BN) * ROWB; };
    auto sB = [&](int buf) { return smem + buf * (BM + BN) * ROWB + BM * ROWB; };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

    // Tile order: consecutive workgroups walk down M inside groups of 8 row
    // tiles so the B slab they share stays hot in L2.
    const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
    int tm, tn;
    {
        const int id = blockIdx.x;
        const int group = 8;
        const int per_group = group * tiles_n;
        const int gi = id / per_group;
        const int first_m = gi * group;
        const int gm = min(tiles_m - first_m, group);
        const int local = id - gi * per_group;
        tm = first_m + local % gm;
        tn = local / gm;
    }
    const int m0 = tm * BM, n0 = tn * BN;

    const T* ap[ACH];
    const T* bp[BCH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        int r = m0 + (tid >> 3) + 32 * i;
        ap[i] = al.row(r < M ? r : M - 1);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) bp[i] = bl.row(n0 + (tid >> 3) + 32 * i);
    const int kofs = (tid & 7) * (16 / EB);
    const int lds_w = (tid >> 3) * ROWB + (tid & 7) * 16;

    u32x4 ra[ACH], rb[BCH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) ra[i] = *reinterpret_cast<const u32x4*>(al.at(ap[i], k0) + kofs);
#pragma unroll
        for (int i = 0; i < BCH; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + k0 + kofs);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4*>(sA(buf) + lds_w + 32 * i * ROWB) = ra[i];
#pragma unroll
        for (int i = 0; i < BCH; ++i) *reinterpret_cast<u32x4*>(sB(buf) + lds_w + 32 * i * ROWB) = rb[i];
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = K / BK;
    gload(0);
    lstore(0);
    __syncthreads();

    const int frag_off = (lane & 31) * ROWB + (lane >> 5) * E * EB;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * BK);
        const char* a_base = sA(cur) + (wm * Cfg::WM) * ROWB + frag_off;
        const char* b_base = sB(cur) + (wn * Cfg::WN) * ROWB + frag_off;
#pragma unroll
        for (int kk = 0; kk < BK / KSTEP; ++kk) {
            frag af[MI], bf[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                af[i] = *reinterpret_cast<const frag*>(a_base + i * 32 * ROWB + kk * KSTEP * EB);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                bf[j] = *reinterpret_cast<const frag*>(b_base + j * 32 * ROWB + kk * KSTEP * EB);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] = Mfma<T>::mma(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

    ep.template apply<MI, NI, Cfg::WN>(m0 + wm * Cfg::WM, n0 + wn * Cfg::WN, acc, lane, M);
}

template <typename T, class Cfg, class AL, class BL, class EP>
hipError_t launch_gemm(int M, int N, int K, const AL& al, const BL& bl, const EP& ep,
                       hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    const int tiles = ((M + Cfg::BM - 1) / Cfg::BM) * (N / Cfg::BN);
    hipLaunchKernelGGL((gemm_nt_kernel<T, Cfg, AL, BL, EP>), dim3(tiles), dim3(256), 0, stream, M, N,
                       K, al, bl, ep);
    return hipGetLastError();
}

}  // namespace dflash
