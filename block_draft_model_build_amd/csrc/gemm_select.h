// Tile-shape choice shared by every libdflash GEMM call site.
#pragma once

#include "gemm.h"
#include "internal.h"

#include <type_traits>

namespace dflash {

// 256x256 tiles with 8 waves (two per SIMD, 64x128 each) and 128-byte K slabs
// double buffered in LDS (the best of a measured sweep over tile shapes, wave
// counts, slab depths and stage counts on the context-projection, gate/up and
// down shapes); 128x128 tiles with 4 waves (one 32-row MFMA strip each) when
// the big tiles would leave compute units idle. When even the 128x128 grid is
// at most one tile per compute unit (1024-row o_proj and down), a CU holds one
// workgroup anyway, so its LDS goes to 128-byte slabs in 4 stages: twice the
// bytes in flight (inference body 5.56 -> 5.40 ms per step).
using BigTile = TileCfg<256, 256, 4, 2, 128, 2>;
using MidTile = TileCfg<128, 128, 4, 1>;
using MidDeep = TileCfg<128, 128, 4, 1, 128, 4>;
// 256x192 tiles (waves of 64x96) for products whose 256x256 grid would leave
// its last round of tiles part-empty, when the 192-wide grid fills its rounds
// with less total time (3/4 of the work per tile). Only for epilogues that do
// not depend on 128-column waves. 4096-row QKV product (6144 columns): 384 big
// tiles in 1.5 rounds -> 512 tiles in 2 rounds, 1.06 -> 0.92 ms per step.
using WideTile = TileCfg<256, 192, 4, 2, 128, 2>;
// The same deep 128x128 tiles with 8 waves (32x64 each: two waves per SIMD hide
// each other's fragment-read latency) for plain-store and residual epilogues
// (1024-row o_proj and down: 1.02 -> 0.94 ms per inference step).
using MidDeep8 = TileCfg<128, 128, 4, 2, 128, 4>;
// 128x192 tiles with 128-byte slabs in 4 stages (160 KB of LDS) when they make
// at most one tile per compute unit where the 128x128 grid makes more (1024-row
// QKV product: 384 -> 256 tiles, 0.43 -> 0.31 ms per inference step).
using MidWideDeep = TileCfg<128, 192, 4, 1, 128, 4>;
template <class EP> struct AnyWaveWidth : std::false_type {};
template <typename T> struct AnyWaveWidth<EpStore<T>> : std::true_type {};
template <typename T> struct AnyWaveWidth<EpResidual<T>> : std::true_type {};
template <> struct AnyWaveWidth<EpAddF32> : std::true_type {};
template <typename T> struct AnyWaveWidth<EpSplitQKV<T>> : std::true_type {};
template <typename T> struct AnyWaveWidth<EpSwiGLUBwd<T>> : std::true_type {};
static_assert(BigTile::WN == 128 && MidTile::WN == 128 && MidDeep::WN == 128, "gate/up interleave and RoPE pairing assume WN = 128");

// `group`: row tiles walked together in the tile order (gemm_nt_kernel). 8 by
// default; the context projection (K = 20480, A of stacked target states) is
// 4-5% faster with 4, while the context-path backward's dC product (a
// transposed-store epilogue) is 25% slower with 4 (measured on the 5-layer shapes).
template <typename T, class AL, class BL, class EP>
static hipError_t gemm(int kid, int M, int N, int K, const AL& al, const BL& bl, const EP& ep, hipStream_t st,
                       int group = 8) {
    ProfScope prof(kid, st);
    const int big_tiles = ((M + 255) / 256) * (N / 256);
    if constexpr (AnyWaveWidth<EP>::value) {
        const int r256 = (big_tiles + 255) / 256, t192 = ((M + 255) / 256) * (N / 192);
        if (N % 192 == 0 && big_tiles >= 256 && 3 * ((t192 + 255) / 256) < 4 * r256)
            return launch_gemm<T, WideTile>(M, N, K, al, bl, ep, st, group);
    }
    // From half a round of big tiles up: 128x128 tiles move about half the flops per compute unit
    // and would need at least two rounds (1024-row context K/V product of five layers:
    // 640 tiles in 2.5 rounds against 160 big ones).
    if (N % 256 == 0 && big_tiles >= 128) return launch_gemm<T, BigTile>(M, N, K, al, bl, ep, st, group);
    const int mid_tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if constexpr (AnyWaveWidth<EP>::value) {
        const int t192 = ((M + 127) / 128) * (N / 192);
        if (N % 192 == 0 && mid_tiles > 256 && t192 <= 256)
            return launch_gemm<T, MidWideDeep>(M, N, K, al, bl, ep, st, group);
    }
    if constexpr (AnyWaveWidth<EP>::value) {
        if (mid_tiles <= 256) return launch_gemm<T, MidDeep8>(M, N, K, al, bl, ep, st, group);
    }
    if (mid_tiles <= 256) return launch_gemm<T, MidDeep>(M, N, K, al, bl, ep, st, group);
    return launch_gemm<T, MidTile>(M, N, K, al, bl, ep, st, group);
}

}  // namespace dflash
