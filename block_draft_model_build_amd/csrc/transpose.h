// LDS-tiled transposes and fills feeding the backward GEMMs, whose operands
// must be contiguous along the contraction.
#pragma once

#include "common.h"

namespace dflash {

template <typename T> struct SrcPlain {
    const T* p; int64_t ld;
    __device__ const T* at(int64_t r, int64_t c) const { return p + r * ld + c; }
};
// Element (r, k) of the concatenated target states, as dflash_ctx_proj reads them.
template <typename T> struct SrcStacked {
    const T* p; int64_t rs, ls; int ht;
    __device__ const T* at(int64_t r, int64_t c) const {
        const int64_t layer = c / ht;
        return p + r * rs + layer * ls + (c - layer * ht);
    }
};

// dst[c * ldd + r] = src(r, c) for r < rows_pad (zero past rows), c < cols, in
// 64 x 64 tiles through LDS with 16-byte loads along c and 16-byte stores
// along r, non-temporal: each source byte is read once and the transposes are
// too large to stay cached for the product that reads them (the backward's
// transposes and casts 2.27 -> 2.09 ms per step). cols is a multiple of 64; src rows hold 16-byte aligned runs of
// V = 16 / sizeof(T) elements (a run never straddles two target layers);
// ldd and the column offset of dst keep 16-byte alignment.
template <typename T, class Src>
__global__ __launch_bounds__(256) void transpose_kernel(Src src, int64_t rows, int64_t rows_pad, int64_t cols, T* dst,
                                                        int64_t ldd) {
    constexpr int V = 16 / (int)sizeof(T);
    typedef T vec __attribute__((ext_vector_type(V)));
    __shared__ float tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
    for (int idx = threadIdx.x; idx < 64 * (64 / V); idx += 256) {
        const int rr = idx / (64 / V), cv = (idx - rr * (64 / V)) * V;
        const int64_t r = r0 + rr;
        vec v = {};
        if (r < rows) v = __builtin_nontemporal_load(reinterpret_cast<const vec*>(src.at(r, c0 + cv)));
#pragma unroll
        for (int q = 0; q < V; ++q) tile[rr][cv + q] = to_f32(v[q]);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * (64 / V); idx += 256) {
        const int cc = idx / (64 / V), rv = (idx - cc * (64 / V)) * V;
        const int64_t r = r0 + rv;
        if (r >= rows_pad) continue;
        vec v;
#pragma unroll
        for (int q = 0; q < V; ++q) v[q] = from_f32<T>(tile[rv + q][cc]);
        __builtin_nontemporal_store(v, reinterpret_cast<vec*>(dst + (c0 + cc) * ldd + r));
    }
}

template <typename T>
__global__ __launch_bounds__(256) void fill_cols_kernel(T* p, int64_t ld, int64_t nrows, int64_t c0, int64_t c1) {
    const int64_t w = c1 - c0, n = nrows * w;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / w;
        p[r * ld + c0 + (i - r * w)] = from_f32<T>(0.f);
    }
}


// fp32 src [rows][cols] (ld lds) -> config dtype, written row-major to rm (ld
// ldr; optional) and transposed to tr [cols][ldt] with zero columns for rows
// in [rows, rows_pad). 64 x 64 tiles through LDS: 16-byte loads along the
// columns, 16-byte stores along the rows of the transpose. cols, lds, ldr and
// ldt are multiples of 4, 4, 4 and 16 / sizeof(T); rows_pad of 64.
template <typename T>
__global__ __launch_bounds__(256) void pack_f32_kernel(const float* __restrict__ src, int64_t lds, int64_t rows,
                                                       int64_t rows_pad, T* __restrict__ rm, int64_t ldr,
                                                       T* __restrict__ tr, int64_t ldt) {
    constexpr int V = 16 / (int)sizeof(T);
    typedef T vec __attribute__((ext_vector_type(V)));
    typedef T vec4 __attribute__((ext_vector_type(4)));
    __shared__ float tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
    for (int idx = threadIdx.x; idx < 64 * 16; idx += 256) {
        const int rr = idx >> 4, cv = (idx & 15) * 4;
        const int64_t r = r0 + rr;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (r < rows) v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + r * lds + c0 + cv));
#pragma unroll
        for (int q = 0; q < 4; ++q) tile[rr][cv + q] = v[q];
        if (rm != nullptr && r < rows) {
            vec4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = from_f32<T>(v[q]);
            *reinterpret_cast<vec4*>(rm + r * ldr + c0 + cv) = o;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * (64 / V); idx += 256) {
        const int cc = idx / (64 / V), rv = (idx - cc * (64 / V)) * V;
        const int64_t r = r0 + rv;
        if (r >= rows_pad) continue;
        vec o;
#pragma unroll
        for (int q = 0; q < V; ++q) o[q] = from_f32<T>(tile[rv + q][cc]);
        __builtin_nontemporal_store(o, reinterpret_cast<vec*>(tr + (c0 + cc) * ldt + r));
    }
}

// dh[row] = d_out[row] (as fp32) on rows the body returns (valid, in a block
// with an anchor), zero elsewhere: the gradient reaching the last layer's
// output. Four elements per thread; H is a multiple of 4.
template <typename T>
__global__ __launch_bounds__(256) void mask_grad_kernel(const T* __restrict__ dout, const uint8_t* __restrict__ valid,
                                                        const int32_t* __restrict__ anchor, int bs, int64_t rows,
                                                        int H, float* __restrict__ dh) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    const int64_t q4 = H / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * q4; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / q4;
        const bool keep = valid[row] != 0 && anchor[row / bs] >= 0;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (keep) {
            const t4 u = reinterpret_cast<const t4*>(dout)[i];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = to_f32(u[q]);
        }
        reinterpret_cast<f32x4*>(dh)[i] = v;
    }
}

}  // namespace dflash
