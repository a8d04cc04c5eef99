// Shared device helpers for libdflash (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Address-space casts for the direct-to-LDS loads (global_load_lds_dwordx4:
// lane i of the wave writes its 16 bytes to LDS at M0 base + 16 i).
#define DFLASH_GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define DFLASH_LPTR(p) ((void __attribute__((address_space(3)))*)(p))

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (LDS and export counters left unconstrained).
template <int n> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
constexpr int kMaxLayers = 16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (gfx950 converts in hardware).
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return static_cast<__bf16>(x); }

// One MFMA shape per element type, both 32x32 output tiles with the same
// accumulator layout: lane l, accumulator element e holds
//   row = 8*(e/4) + 4*(l/32) + (e%4),  col = l%32.
// The A and B operands each carry E consecutive k values per lane; lane half
// l/32 selects which E-wide slice of the KSTEP-deep contraction it holds. Both
// operands are always loaded with the same k slicing, so the result does not
// depend on how the hardware orders k inside one instruction.
template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
    static constexpr int KSTEP = 16;
    static constexpr int E = 8;
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    static constexpr int KSTEP = 2;
    static constexpr int E = 1;
    typedef float frag;
    __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// Fraction-of-a-turn rotary frequencies, computed on the host in fp64:
// turns[i] = rope_theta^(-2i/D) / (2*pi). The angle of pair i at position p is
// 2*pi*frac(p * turns[i]); taking the fractional part in fp64 keeps the angle
// exact to ~1e-12 rad at any position. The hardware sine and cosine
// (v_sin_f32, v_cos_f32) take their argument in turns, so the reduced
// fraction goes to them directly.
struct RopeTurns {
    double turns[64];
};

__device__ __forceinline__ void rope_cs(const RopeTurns& rt, int i, int pos, float& c, float& s) {
    double t = (double)pos * rt.turns[i];
    t -= floor(t);
    const float f = (float)t;            // turns, in [0, 1]
    s = __builtin_amdgcn_sinf(f);
    c = __builtin_amdgcn_cosf(f);
}

}  // namespace dflash
