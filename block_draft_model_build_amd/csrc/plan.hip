// dflash_build_plan: seeded anchor selection on the device.
//
// NeMo RL "DFlash Draft Body", How It Works, steps 1, 2 and 4, and the angelspec
// "DFlash" page, How it works (anchor sampling): anchors are valid positions
// sampled across the sequence; the plan is a pure function of the mask, sample
// ids, optimizer step and seed; equal sample ids give equal anchors; a block is
// the anchor plus gamma draft positions; the loss mask leaves out the anchor
// and invalid positions.
//
// One workgroup (1024 threads) per batch row. Every eligible position gets a
// 64-bit SplitMix64 key; the N smallest keys are found with an 8-pass radix
// select (8-bit digits, histogram in LDS), the keys being recomputed in every
// pass instead of stored, so nothing but a 256-bin histogram lives in LDS at
// any sequence length. Equal keys are broken by position. A block-wide scan
// over contiguous position ranges then writes the chosen anchors in ascending
// order.
#include "common.h"
#include "internal.h"

namespace dflash {

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr int kPlanThreads = 1024;

// Inclusive block scan of one int per thread.
__device__ int block_inclusive_scan(int v, int* buf) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int w = 1; w < kPlanThreads; w <<= 1) {
        int add = tid >= w ? buf[tid - w] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    int r = buf[tid];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const uint8_t* __restrict__ mask, int S, const int64_t* __restrict__ sample_ids, uint64_t step,
    uint64_t seed, int N, int bs, int32_t* anchors, int32_t* positions, uint8_t* valid,
    uint8_t* loss_mask, int32_t* num_anchors, int64_t* block_ctx_base) {
    __shared__ unsigned hist[256];
    __shared__ int scanbuf[kPlanThreads];
    __shared__ uint64_t sel_prefix;
    __shared__ int sel_need;

    const int b = blockIdx.x, tid = threadIdx.x;
    const uint8_t* m = mask + (int64_t)b * S;
    const uint64_t rk = splitmix64(splitmix64(splitmix64(seed) ^ (uint64_t)sample_ids[b]) ^ step);
    const int P = S > 1 ? S - 1 : 0;                     // candidate positions 0..S-2
    const int per = (P + kPlanThreads - 1) / kPlanThreads;
    const int p0 = tid * per, p1 = min(P, p0 + per);
    auto eligible = [&](int a) { return m[a] != 0 && m[a + 1] != 0; };

    int cnt = 0;
    for (int a = p0; a < p1; ++a) cnt += eligible(a) ? 1 : 0;
    const int total = block_inclusive_scan(cnt, scanbuf);
    int elig_count;
    {
        if (tid == kPlanThreads - 1) sel_need = total;
        __syncthreads();
        elig_count = sel_need;
        __syncthreads();
    }
    const int n = min(N, elig_count);

    // Radix select: the n-th smallest key (when n < #eligible).
    uint64_t prefix = 0, pmask = 0;
    int need = n;
    const bool take_all = (n == elig_count);
    if (!take_all && n > 0) {
        for (int digit = 7; digit >= 0; --digit) {
            for (int i = tid; i < 256; i += kPlanThreads) hist[i] = 0;
            __syncthreads();
            const int sh = digit * 8;
            for (int a = p0; a < p1; ++a) {
                if (!eligible(a)) continue;
                const uint64_t key = splitmix64(rk ^ (uint64_t)a);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                int before = 0, bk = 0;
                for (bk = 0; bk < 256; ++bk) {
                    if (before + (int)hist[bk] >= need) break;
                    before += hist[bk];
                }
                sel_need = need - before;
                sel_prefix = prefix | ((uint64_t)bk << sh);
            }
            __syncthreads();
            need = sel_need;
            prefix = sel_prefix;
            pmask |= (uint64_t)255 << sh;
            __syncthreads();
        }
    }
    // prefix = threshold key T; `need` keys equal to T are taken, lowest positions first.
    auto chosen_strict = [&](int a, uint64_t key) { return take_all || key < prefix; };

    int eq_local = 0;
    if (!take_all && n > 0)
        for (int a = p0; a < p1; ++a)
            if (eligible(a) && splitmix64(rk ^ (uint64_t)a) == prefix) ++eq_local;
    const int eq_incl = block_inclusive_scan(eq_local, scanbuf);
    int eq_rank = eq_incl - eq_local;

    int sel_local = 0;
    if (n > 0)
        for (int a = p0; a < p1; ++a) {
            if (!eligible(a)) continue;
            const uint64_t key = take_all ? 0 : splitmix64(rk ^ (uint64_t)a);
            if (chosen_strict(a, key)) ++sel_local;
            else if (key == prefix) { if (eq_rank < need) ++sel_local; ++eq_rank; }
        }
    const int sel_incl = block_inclusive_scan(sel_local, scanbuf);
    int out_i = sel_incl - sel_local;
    eq_rank = eq_incl - eq_local;
    int32_t* arow = anchors + (int64_t)b * N;
    if (n > 0)
        for (int a = p0; a < p1; ++a) {
            if (!eligible(a)) continue;
            const uint64_t key = take_all ? 0 : splitmix64(rk ^ (uint64_t)a);
            bool take = false;
            if (chosen_strict(a, key)) take = true;
            else if (key == prefix) { take = eq_rank < need; ++eq_rank; }
            if (take) arow[out_i++] = a;
        }
    for (int i = n + tid; i < N; i += kPlanThreads) arow[i] = -1;
    if (tid == 0) num_anchors[b] = n;
    if (block_ctx_base != nullptr)
        for (int i = tid; i < N; i += kPlanThreads) block_ctx_base[(int64_t)b * N + i] = (int64_t)b * S;
    __threadfence_block();
    __syncthreads();

    for (int idx = tid; idx < N * bs; idx += kPlanThreads) {
        const int i = idx / bs, k = idx - i * bs;
        const int a = arow[i];
        const int64_t o = (int64_t)b * N * bs + idx;
        if (a < 0) {
            positions[o] = -1; valid[o] = 0; loss_mask[o] = 0;
        } else {
            const int64_t pos = (int64_t)a + k;
            const bool ok = pos < S && m[pos] != 0;
            positions[o] = (int32_t)pos;
            valid[o] = ok ? 1 : 0;
            loss_mask[o] = (ok && k >= 1) ? 1 : 0;
        }
    }
}

}  // namespace dflash

using namespace dflash;

extern "C" dflash_status dflash_build_plan(const uint8_t* mask, int32_t batch, int32_t seq_len,
                                           const int64_t* sample_ids, int64_t step, uint64_t seed,
                                           int32_t anchors_per_row, int32_t block_size,
                                           int32_t* anchors, int32_t* positions, uint8_t* valid,
                                           uint8_t* loss_mask, int32_t* num_anchors,
                                           int64_t* block_ctx_base, void* hip_stream) {
    if (batch < 0 || seq_len < 0 || anchors_per_row < 0 || block_size < 1) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)seq_len + block_size > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (batch == 0) return DFLASH_OK;
    if (sample_ids == nullptr || num_anchors == nullptr || (seq_len > 0 && mask == nullptr))
        return DFLASH_ERR_INVALID_ARG;
    if (anchors_per_row > 0 &&
        (anchors == nullptr || positions == nullptr || valid == nullptr || loss_mask == nullptr))
        return DFLASH_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    ProfScope prof(DFLASH_KERNEL_PLAN, st);
    hipLaunchKernelGGL(plan_kernel, dim3(batch), dim3(kPlanThreads), 0, st, mask, seq_len, sample_ids,
                       (uint64_t)step, seed, anchors_per_row, block_size, anchors, positions, valid,
                       loss_mask, num_anchors, block_ctx_base);
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
