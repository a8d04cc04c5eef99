// Row normalisation kernels of the draft layers (RMSNorm forward and backward).
#pragma once

#include "common.h"

namespace dflash {

// out[row] = x / sqrt(mean(x^2) + eps) * w, x read as fp32; optionally copies
// x into the fp32 residual stream (first layer: embeddings -> h). 16-byte
// loads; rows of up to 256 * 4 vectors stay in registers between the sum and
// the scaling (H = 4096 in fp32), together with their weights, which are read
// before the reduction so that a row costs one memory round trip; longer rows
// are read twice.
template <typename TIN, typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const TIN* __restrict__ in, float* __restrict__ hcopy,
                                                      const T* __restrict__ w, T* __restrict__ out, int H,
                                                      float eps) {
    constexpr int VI = 16 / (int)sizeof(TIN);     // elements per 16-byte load
    constexpr int NV = 4;                         // vectors per thread kept in registers
    typedef TIN vin __attribute__((ext_vector_type(VI)));
    typedef T vout __attribute__((ext_vector_type(VI)));
    typedef float vf32 __attribute__((ext_vector_type(VI)));
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const TIN* x = in + row * H;
    const int nvec = H / VI;
    const bool cached = nvec <= 256 * NV;
    vin v[NV];
    vout wv[NV];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int j = threadIdx.x + 256 * k;
        if (j < nvec) {
            v[k] = reinterpret_cast<const vin*>(x)[j];
            wv[k] = reinterpret_cast<const vout*>(w)[j];
        }
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int j = threadIdx.x + 256 * k;
        if (j < nvec) {
#pragma unroll
            for (int q = 0; q < VI; ++q) ss += to_f32(v[k][q]) * to_f32(v[k][q]);
        }
    }
    if (!cached)
        for (int j = threadIdx.x + 256 * NV; j < nvec; j += 256) {
            const vin u = reinterpret_cast<const vin*>(x)[j];
#pragma unroll
            for (int q = 0; q < VI; ++q) ss += to_f32(u[q]) * to_f32(u[q]);
        }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    auto emit = [&](int j, const vin& u, const vout& ww) {
        vout o;
        vf32 hc;
#pragma unroll
        for (int q = 0; q < VI; ++q) {
            const float f = to_f32(u[q]);
            o[q] = from_f32<T>(f * r * to_f32(ww[q]));
            hc[q] = f;
        }
        if (hcopy) reinterpret_cast<vf32*>(hcopy + row * H)[j] = hc;
        reinterpret_cast<vout*>(out + row * H)[j] = o;
    };
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int j = threadIdx.x + 256 * k;
        if (j < nvec) emit(j, v[k], wv[k]);
    }
    if (!cached)
        for (int j = threadIdx.x + 256 * NV; j < nvec; j += 256)
            emit(j, reinterpret_cast<const vin*>(x)[j], reinterpret_cast<const vout*>(w)[j]);
}


// Backward of y = x r w, r = (mean(x^2) + eps)^(-1/2) per row, given dy:
//   out = res + r (dy w) - x r^3 (sum_j dy_j w_j x_j) / H
// (res: the residual path's gradient, added here), and per workgroup the
// partial column sums of dy x r over its kNormBwdRows rows; dw is their sum
// over workgroups (norm_colsum_kernel, fixed order). A thread keeps NV float4
// columns of a row (H <= 1024 NV) and its accumulators in registers. Few rows
// per workgroup and few registers per thread let several workgroups share a
// compute unit, so several rows are in flight there while one waits at its
// row reduction: with one 16-row workgroup per compute unit the kernel moved
// 3.1 TB/s. The three row inputs are read once: non-temporal loads.
constexpr int kNormBwdRows = 4;
constexpr int kNormBwdMaxH = 8192;

template <typename T, int NV>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float* __restrict__ x, const T* __restrict__ w,
                                                          const float* __restrict__ dy,
                                                          const float* __restrict__ res, float* __restrict__ out,
                                                          float* __restrict__ part, int rows, int H, float eps) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    __shared__ float red[2][2][4];
    const int nvec = H / 4, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    f32x4 wv[NV], acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int j = tid + 256 * k;
        acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        wv[k] = acc[k];
        if (j < nvec) {
            const t4 u = reinterpret_cast<const t4*>(w)[j];
#pragma unroll
            for (int q = 0; q < 4; ++q) wv[k][q] = to_f32(u[q]);
        }
    }
    const int r0 = blockIdx.x * kNormBwdRows;
    for (int rr = 0; rr < kNormBwdRows; ++rr) {
        const int64_t row = r0 + rr;
        if (row >= rows) break;                       // the same for the whole workgroup
        const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * H);
        const f32x4* gr = reinterpret_cast<const f32x4*>(dy + row * H);
        const f32x4* rs = reinterpret_cast<const f32x4*>(res + row * H);
        f32x4 xv[NV], gv[NV], rv[NV];
        float ss = 0.f, dot = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int j = tid + 256 * k;
            xv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            gv[k] = rv[k] = xv[k];
            if (j < nvec) {
                xv[k] = __builtin_nontemporal_load(&xr[j]);
                gv[k] = __builtin_nontemporal_load(&gr[j]);
                rv[k] = __builtin_nontemporal_load(&rs[j]);
            }
        }
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ss += xv[k][q] * xv[k][q];
                dot += gv[k][q] * wv[k][q] * xv[k][q];
            }
        for (int o = 32; o > 0; o >>= 1) {
            ss += __shfl_xor(ss, o, 64);
            dot += __shfl_xor(dot, o, 64);
        }
        // Two copies of the reduction slots (by row parity): a wave can only
        // rewrite a copy after every wave has read it, one barrier later.
        if (lane == 0) {
            red[rr & 1][0][wave] = ss;
            red[rr & 1][1][wave] = dot;
        }
        __syncthreads();
        const float tss = red[rr & 1][0][0] + red[rr & 1][0][1] + red[rr & 1][0][2] + red[rr & 1][0][3];
        const float tdot = red[rr & 1][1][0] + red[rr & 1][1][1] + red[rr & 1][1][2] + red[rr & 1][1][3];
        const float r = 1.0f / sqrtf(tss / (float)H + eps);
        const float coef = r * r * r * tdot / (float)H;
        f32x4* orow = reinterpret_cast<f32x4*>(out + row * H);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int j = tid + 256 * k;
            if (j < nvec) {
                orow[j] = rv[k] + r * gv[k] * wv[k] - xv[k] * coef;
                acc[k] += gv[k] * xv[k] * r;
            }
        }
    }
    f32x4* pr = reinterpret_cast<f32x4*>(part + (int64_t)blockIdx.x * H);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int j = tid + 256 * k;
        if (j < nvec) pr[j] = acc[k];
    }
}

// dw[j] = sum over p < nparts of part[p][j]. A workgroup takes 64 columns as
// 16 float4 lanes x 16 slices; slice s sums the parts p = s (mod 16), then
// slice 0 adds the 16 slice sums in order. H is a multiple of 4.
static __global__ __launch_bounds__(256) void norm_colsum_kernel(const float* __restrict__ part, int nparts, int H,
                                                                 float* __restrict__ dw) {
    __shared__ f32x4 sl[16][16];
    const int c4 = threadIdx.x & 15, s = threadIdx.x >> 4;
    const int j = blockIdx.x * 64 + c4 * 4;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (j < H) {
#pragma unroll 8
        for (int p = s; p < nparts; p += 16) a += *reinterpret_cast<const f32x4*>(part + (int64_t)p * H + j);
    }
    sl[s][c4] = a;
    __syncthreads();
    if (s == 0 && j < H) {
        f32x4 t = sl[0][c4];
#pragma unroll
        for (int q = 1; q < 16; ++q) t += sl[q][c4];
#pragma unroll
        for (int q = 0; q < 4; ++q) dw[j + q] = t[q];   // dw: caller's buffer, 4-byte aligned
    }
}

}  // namespace dflash
