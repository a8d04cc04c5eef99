// dflash_build_plan: seeded anchor selection on the device.
//
// NeMo RL "DFlash Draft Body", How It Works, steps 1, 2 and 4, and the angelspec
// "DFlash" page, How it works (anchor sampling): anchors are valid positions
// sampled across the sequence; the plan is a pure function of the mask, sample
// ids, optimizer step and seed; equal sample ids give equal anchors; a block is
// the anchor plus gamma draft positions; the loss mask leaves out the anchor
// and invalid positions.
//
// One workgroup (1024 threads) per batch row; the row's eligibility bitmask
// lives in LDS (rows up to 524288 positions). Every eligible position gets a
// 64-bit SplitMix64 key, recomputed where needed instead of stored; see
// plan_kernel for the selection.
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
constexpr int kPlanMaxWords = 16384;      // rows up to 32 * 16384 positions keep their bitmask in LDS
constexpr int kPlanBins = 4096;           // 12-bit digits
constexpr int kPlanMaxCand = 2048;        // keys of the threshold bin ranked exactly

__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Inclusive block scan of one int per thread: lane shuffles inside each wave,
// then a shuffle scan of the 16 wave totals. buf holds >= 32 ints.
__device__ int block_inclusive_scan(int v, int* buf) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = wave_inclusive_scan(v);
    if (lane == 63) buf[w] = incl;
    __syncthreads();
    if (w == 0) {
        int t = lane < kPlanThreads / 64 ? buf[lane] : 0;
        t = wave_inclusive_scan(t);
        if (lane < kPlanThreads / 64) buf[kPlanThreads / 64 + lane] = t;
    }
    __syncthreads();
    if (w > 0) incl += buf[kPlanThreads / 64 + w - 1];
    __syncthreads();
    return incl;
}

// Selection: keys of one row are distinct (the SplitMix64 finaliser is a
// bijection and row_key ^ a differs for every a), so the anchors are exactly
// the eligible positions whose key is <= the n-th smallest key. That key's
// leading bits are found with 12-bit-digit histograms (one sweep when the row
// is not huge), the keys sharing its bin are ranked exactly, and the chosen
// positions are compacted in ascending order from a bitmask in LDS.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const uint8_t* __restrict__ mask, int S, const int64_t* __restrict__ sample_ids, uint64_t step,
    uint64_t seed, int N, int bs, int32_t* anchors, int32_t* positions, uint8_t* valid,
    uint8_t* loss_mask, int32_t* num_anchors, int64_t* block_ctx_base) {
    __shared__ uint32_t bits[kPlanMaxWords];          // eligible, then chosen
    __shared__ unsigned hist[kPlanBins];
    __shared__ unsigned long long cand_key[kPlanMaxCand];
    __shared__ int cand_pos[kPlanMaxCand];
    __shared__ int scanbuf[2 * kPlanThreads / 64];
    __shared__ int s_int[4];                          // [0] count, [1] need, [2] threshold bin, [3] candidates

    const int b = blockIdx.x, tid = threadIdx.x;
    const uint8_t* m = mask + (int64_t)b * S;
    const uint64_t rk = splitmix64(splitmix64(splitmix64(seed) ^ (uint64_t)sample_ids[b]) ^ step);
    const int P = S > 1 ? S - 1 : 0;                  // candidate anchors 0..S-2
    const int words = (P + 31) / 32;

    // 1. Eligibility bits: a is eligible when mask[a] and mask[a + 1] are set.
    int cnt = 0;
    for (int w = tid; w < words; w += kPlanThreads) {
        const int a0 = w * 32;
        uint8_t v[33];
#pragma unroll
        for (int i = 0; i < 33; ++i) v[i] = a0 + i < S ? m[a0 + i] : 0;
        uint32_t x = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) x |= (uint32_t)((v[i] != 0) & (v[i + 1] != 0) & (a0 + i < P)) << i;
        bits[w] = x;
        cnt += __popc(x);
    }
    if (tid == 0) s_int[0] = 0;
    __syncthreads();
    atomicAdd(&s_int[0], cnt);
    __syncthreads();
    const int n = min(N, s_int[0]);
    const bool take_all = n == s_int[0];

    // 2. Leading bits of the n-th smallest key (skipped when every eligible
    //    position is taken or none is asked for).
    unsigned long long prefix = 0, pmask = 0;
    int need = n;
    if (!take_all && n > 0) {
        const int shifts[6] = {52, 40, 28, 16, 4, 0};
        const int widths[6] = {12, 12, 12, 12, 12, 4};
        for (int lvl = 0; lvl < 6; ++lvl) {
            const int sh = shifts[lvl];
            const unsigned dm = (1u << widths[lvl]) - 1u;
            for (int i = tid; i < kPlanBins; i += kPlanThreads) hist[i] = 0;
            __syncthreads();
            for (int w = tid; w < words; w += kPlanThreads) {
                const uint32_t x = bits[w];
#pragma unroll 8
                for (int i = 0; i < 32; ++i) {
                    const unsigned long long key = splitmix64(rk ^ (uint64_t)(w * 32 + i));
                    if (((x >> i) & 1u) && (key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dm], 1u);
                }
            }
            __syncthreads();
            // Scan of the bins: thread t owns bins [4t, 4t + 4).
            unsigned hb[4];
            int own = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) { hb[j] = hist[4 * tid + j]; own += (int)hb[j]; }
            const int incl = block_inclusive_scan(own, scanbuf);
            int run = incl - own;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < need && run + (int)hb[j] >= need) {
                    s_int[1] = need - run;
                    s_int[2] = 4 * tid + j;
                    s_int[3] = (int)hb[j];
                }
                run += (int)hb[j];
            }
            __syncthreads();
            need = s_int[1];
            prefix |= (unsigned long long)s_int[2] << sh;
            pmask |= (unsigned long long)dm << sh;
            const int in_bin = s_int[3];
            __syncthreads();
            if (in_bin <= kPlanMaxCand) break;
        }
        // 3. Keep keys below the bin; collect the bin's keys and rank them exactly.
        if (tid == 0) s_int[3] = 0;
        __syncthreads();
        for (int w = tid; w < words; w += kPlanThreads) {
            const uint32_t x = bits[w];
            uint32_t keep = 0;
#pragma unroll 8
            for (int i = 0; i < 32; ++i) {
                if (!((x >> i) & 1u)) continue;
                const unsigned long long key = splitmix64(rk ^ (uint64_t)(w * 32 + i));
                const unsigned long long top = key & pmask;
                if (top < prefix) {
                    keep |= 1u << i;
                } else if (top == prefix) {
                    const int c = atomicAdd(&s_int[3], 1);
                    if (c < kPlanMaxCand) { cand_key[c] = key; cand_pos[c] = w * 32 + i; }
                }
            }
            bits[w] = keep;
        }
        __syncthreads();
        const int nc = min(s_int[3], kPlanMaxCand);
        for (int i = tid; i < nc; i += kPlanThreads) {
            int rank = 0;
            for (int j = 0; j < nc; ++j)
                rank += (cand_key[j] < cand_key[i] || (cand_key[j] == cand_key[i] && cand_pos[j] < cand_pos[i])) ? 1 : 0;
            if (rank < need) atomicOr(&bits[cand_pos[i] >> 5], 1u << (cand_pos[i] & 31));
        }
        __syncthreads();
    } else if (n == 0) {
        for (int w = tid; w < words; w += kPlanThreads) bits[w] = 0;
        __syncthreads();
    }

    // 4. Compaction in ascending position order: thread t owns a contiguous
    //    run of words.
    const int wper = (words + kPlanThreads - 1) / kPlanThreads;
    const int w0 = min(words, tid * wper), w1 = min(words, w0 + wper);
    int mine = 0;
    for (int w = w0; w < w1; ++w) mine += __popc(bits[w]);
    int out_i = block_inclusive_scan(mine, scanbuf) - mine;
    int32_t* arow = anchors + (int64_t)b * N;
    for (int w = w0; w < w1; ++w) {
        uint32_t x = bits[w];
        while (x) {
            const int i = __ffs(x) - 1;
            x &= x - 1;
            if (out_i < N) arow[out_i] = w * 32 + i;
            ++out_i;
        }
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
    if (seq_len > 32 * kPlanMaxWords) return DFLASH_ERR_UNSUPPORTED;
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
