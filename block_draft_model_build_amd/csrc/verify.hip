// Batched verification of drafted blocks (cooking-agi deep dive "DFlash:
// drafting, verification, and speed": greedy verification and its worked
// example; speculative sampling's acceptance test and [p - q]_+ redraw).
//
// Greedy: one workgroup per (request, position) takes the argmax of the
// target's logits (ties to the smallest token id) straight into emitted[b][i];
// a second kernel, one thread per request, keeps the longest agreeing prefix
// of the draft. Because kept proposals equal the target's choices, the
// emitted tokens are the first n + 1 choices and no other buffer is needed.
//
// Sampling: one workgroup per request. Each proposal's acceptance is decided
// in parallel (fp32(u * q(y)) < p(y)); the first rejection (or the end of the
// block) fixes the one distribution a draw is taken from: [p - q]_+ at that
// position (p itself when that sums to zero), or p after the block for the
// bonus token. The draw is the inverse CDF at u_draw * total in fp64: each of
// the 16 waves sums a contiguous sixteenth of the vocabulary with coalesced
// loads, and the wave whose part holds the crossing walks it again in
// 256-token steps (a wave sum per step, a lane scan in the step that crosses).
// Ties at a boundary within fp64 rounding may go to either neighbour.
#include "internal.h"

namespace dflash {

namespace {

constexpr int kVerifyThreads = 256;
constexpr int kSampleThreads = 1024;        // 16 waves per request: more loads in flight

template <typename T> __device__ __forceinline__ float logit_f32(const T* row, int v) { return to_f32(row[v]); }

// argmax of one row: larger value wins, equal values go to the smaller index.
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

template <typename T>
__global__ __launch_bounds__(kVerifyThreads) void verify_argmax_kernel(const T* logits, int vocab, int rows,
                                                                       int32_t* choice) {
    const int row = blockIdx.x;
    if (row >= rows) return;
    const T* x = logits + (int64_t)row * vocab;
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    constexpr int VEC = 16 / (int)sizeof(T);
    const bool vec_ok = (vocab % VEC) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
    if (vec_ok) {
        // Batches of 8 independent 16-byte loads per thread keep enough bytes
        // in flight to stream the row near HBM speed (non-temporal: each logit
        // is read once); the scan order (and so the tie rule) is unchanged:
        // each thread still visits its indices in increasing order.
        typedef T TV __attribute__((ext_vector_type(VEC)));
        constexpr int NB = 8, STRIDE = kVerifyThreads * VEC;
        for (int base = threadIdx.x * VEC; base < vocab; base += NB * STRIDE) {
            TV t[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (base + b * STRIDE < vocab) t[b] = __builtin_nontemporal_load(reinterpret_cast<const TV*>(x + base + b * STRIDE));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int v0 = base + b * STRIDE;
                if (v0 < vocab) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) better(bv, bi, to_f32(t[b][e]), v0 + e);
                }
            }
        }
    } else {
        for (int v = threadIdx.x; v < vocab; v += kVerifyThreads) better(bv, bi, logit_f32(x, v), v);
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        better(bv, bi, ov, oi);
    }
    __shared__ float s_v[kVerifyThreads / 64];
    __shared__ int s_i[kVerifyThreads / 64];
    if ((threadIdx.x & 63) == 0) {
        s_v[threadIdx.x >> 6] = bv;
        s_i[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kVerifyThreads / 64; ++w) better(bv, bi, s_v[w], s_i[w]);
        choice[row] = bi < vocab ? bi : 0;     // all -inf / NaN rows: token 0
    }
}

// emitted[b] holds the target's choices on entry.
__global__ __launch_bounds__(256) void verify_greedy_finish_kernel(const int32_t* draft, int batch, int gamma,
                                                                   int eos, int32_t* emitted, int32_t* num_emitted,
                                                                   int32_t* accepted) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= batch) return;
    const int32_t* d = draft + (int64_t)b * gamma;
    int32_t* e = emitted + (int64_t)b * (gamma + 1);
    int n = 0;
    while (n < gamma && d[n] == e[n]) ++n;
    int keep = n + 1, acc = n;                 // the kept prefix plus the target's next choice
    if (eos >= 0)
        for (int i = 0; i < n; ++i)
            if (d[i] == eos) {
                keep = acc = i + 1;            // accepted end of sequence: no further token
                break;
            }
    for (int i = keep; i <= gamma; ++i) e[i] = -1;
    num_emitted[b] = keep;
    accepted[b] = acc;
}

// Weight of token v in the distribution a draw is taken from.
struct DrawWeights {
    const float* p;
    const float* q;      // null: weights are p itself
    __device__ double operator()(int v) const {
        if (q == nullptr) return (double)p[v];
        const double w = (double)p[v] - (double)q[v];
        return w > 0.0 ? w : 0.0;
    }
};

__global__ __launch_bounds__(kSampleThreads) void verify_sample_kernel(
    const int32_t* draft, const float* p, const float* q, const float* u_accept, const float* u_draw, int gamma,
    int vocab, int eos, int32_t* emitted, int32_t* num_emitted, int32_t* accepted) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    __shared__ int s_first;                    // first rejected position (gamma: none)
    __shared__ int s_eos;                      // first accepted end-of-sequence position (gamma: none)
    __shared__ int s_tok;
    if (tid == 0) {
        s_first = gamma;
        s_eos = gamma;
        s_tok = -1;
    }
    __syncthreads();
    const int32_t* d = draft + (int64_t)b * gamma;
    const float* pb = p + (int64_t)b * (gamma + 1) * vocab;
    const float* qb = q + (int64_t)b * gamma * vocab;
    for (int i = tid; i < gamma; i += kSampleThreads) {
        const int y = d[i];
        bool ok = false;
        if (y >= 0 && y < vocab) {
            const float prod = u_accept[(int64_t)b * gamma + i] * qb[(int64_t)i * vocab + y];
            ok = prod < pb[(int64_t)i * vocab + y];
        }
        if (!ok) atomicMin(&s_first, i);
        else if (y == eos) atomicMin(&s_eos, i);
    }
    __syncthreads();
    const int first = s_first;
    int32_t* e = emitted + (int64_t)b * (gamma + 1);
    if (s_eos < first) {                       // an accepted end-of-sequence ends the block
        const int keep = s_eos + 1;
        for (int i = tid; i <= gamma; i += kSampleThreads) e[i] = i < keep ? d[i] : -1;
        if (tid == 0) {
            num_emitted[b] = keep;
            accepted[b] = keep;
        }
        return;
    }
    // The draw: residual at the first rejection, or p after the block.
    DrawWeights w{pb + (int64_t)first * vocab, first < gamma ? qb + (int64_t)first * vocab : nullptr};
    // Each wave owns a contiguous quarter of the vocabulary, read in steps of
    // 64 lanes x 4 tokens (lane l takes tokens 4l..4l+3 of a step).
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int NWAVE = kSampleThreads / 64;
    const int steps = (vocab + 255) / 256;
    const int per_wave = (steps + NWAVE - 1) / NWAVE;
    const int s0 = wave * per_wave, s1 = min(steps, s0 + per_wave);
    const bool vec = (vocab & 3) == 0 && ((reinterpret_cast<uintptr_t>(w.p) | reinterpret_cast<uintptr_t>(w.q)) & 15) == 0;
    auto lane_weights = [&](int s, double (&x)[4]) {
        const int v = s * 256 + lane * 4;
        if (vec && v < vocab) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(w.p + v);
            f32x4 qv = {0.f, 0.f, 0.f, 0.f};
            if (w.q != nullptr) qv = *reinterpret_cast<const f32x4*>(w.q + v);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const double y = (double)pv[e4] - (w.q != nullptr ? (double)qv[e4] : 0.0);
                x[e4] = y > 0.0 ? y : 0.0;
            }
        } else {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) x[e4] = v + e4 < vocab ? w(v + e4) : 0.0;
        }
    };
    auto wave_sum = [&](double x) {            // fixed butterfly order: same result in every lane
        for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
        return x;
    };
    __shared__ double s_seg[NWAVE];
    for (int pass = 0; pass < 2; ++pass) {
        double acc = 0.0;
#pragma unroll 4
        for (int s = s0; s < s1; ++s) {
            double x[4];
            lane_weights(s, x);
            acc += ((x[0] + x[1]) + x[2]) + x[3];
        }
        acc = wave_sum(acc);
        if (lane == 0) s_seg[wave] = acc;
        __syncthreads();
        double total = 0.0;
        for (int k = 0; k < NWAVE; ++k) total += s_seg[k];
        if (total > 0.0 || w.q == nullptr) break;
        w.q = nullptr;                         // [p - q]_+ is zero: draw from p
        __syncthreads();
    }
    double total = 0.0, before = 0.0;
    for (int k = 0; k < NWAVE; ++k) {
        if (k == wave) before = total;
        total += s_seg[k];
    }
    const double target = (double)u_draw[b] * total;
    if (before <= target && before + s_seg[wave] > target) {
        // This wave's quarter holds the crossing: walk it step by step.
        double run = before;
        for (int s = s0; s < s1; ++s) {
            double x[4];
            lane_weights(s, x);
            const double mine = ((x[0] + x[1]) + x[2]) + x[3];
            const double step_total = wave_sum(mine);
            if (run + step_total > target) {
                double incl = mine;            // inclusive scan of the lanes' sums
                for (int o = 1; o < 64; o <<= 1) {
                    const double y = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += y;
                }
                double excl = __shfl_up(incl, 1, 64);   // the previous lane's bound: lanes partition
                if (lane == 0) excl = 0.0;
                const bool here = run + excl <= target && run + incl > target;
                if (here) {
                    double r = run + excl;
                    int t = -1, last = -1;
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        r += x[e4];
                        if (x[e4] > 0.0) last = s * 256 + lane * 4 + e4;
                        if (t < 0 && x[e4] > 0.0 && r > target) t = s * 256 + lane * 4 + e4;
                    }
                    s_tok = t >= 0 ? t : last;         // rounding inside the lane: its last positive token
                }
                if (!__any(here) && lane == 0) s_tok = -2;   // rounding left no lane: fallback below
                break;
            }
            run += step_total;
        }
    }
    __syncthreads();
    if (s_tok < 0) {
        // Rounding put the target past the end of the running sums: take the
        // last token of positive weight.
        __shared__ int s_last;
        if (tid == 0) s_last = -1;
        __syncthreads();
        for (int v = vocab - 1 - tid; v >= 0; v -= kSampleThreads)
            if (w(v) > 0.0) {
                atomicMax(&s_last, v);
                break;
            }
        __syncthreads();
        if (tid == 0) s_tok = s_last >= 0 ? s_last : 0;
        __syncthreads();
    }
    const int keep = first + 1;
    for (int i = tid; i <= gamma; i += kSampleThreads) e[i] = i < first ? d[i] : (i == first ? s_tok : -1);
    if (tid == 0) {
        num_emitted[b] = keep;
        accepted[b] = first;
    }
}

}  // namespace

}  // namespace dflash

using namespace dflash;

extern "C" dflash_status dflash_verify_greedy(const int32_t* draft, const void* target_logits, int32_t logits_dtype,
                                              int32_t batch, int32_t gamma, int32_t vocab, int32_t eos_token,
                                              int32_t* emitted, int32_t* num_emitted, int32_t* accepted,
                                              void* hip_stream) {
    if (batch < 0 || gamma < 0 || vocab < 1 || (logits_dtype != DFLASH_BF16 && logits_dtype != DFLASH_F32))
        return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)batch * (gamma + 1) > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (batch == 0) return DFLASH_OK;
    if (target_logits == nullptr || emitted == nullptr || num_emitted == nullptr || accepted == nullptr ||
        (gamma > 0 && draft == nullptr))
        return DFLASH_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    const int rows = batch * (gamma + 1);
    {
        ProfScope prof(DFLASH_KERNEL_VERIFY, st);
        if (logits_dtype == DFLASH_BF16)
            hipLaunchKernelGGL(verify_argmax_kernel<__bf16>, dim3(rows), dim3(kVerifyThreads), 0, st,
                               static_cast<const __bf16*>(target_logits), vocab, rows, emitted);
        else
            hipLaunchKernelGGL(verify_argmax_kernel<float>, dim3(rows), dim3(kVerifyThreads), 0, st,
                               static_cast<const float*>(target_logits), vocab, rows, emitted);
        hipLaunchKernelGGL(verify_greedy_finish_kernel, dim3((batch + 255) / 256), dim3(256), 0, st, draft, batch,
                           gamma, eos_token, emitted, num_emitted, accepted);
    }
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

extern "C" dflash_status dflash_verify_sample(const int32_t* draft, const float* p, const float* q,
                                              const float* u_accept, const float* u_draw, int32_t batch,
                                              int32_t gamma, int32_t vocab, int32_t eos_token, int32_t* emitted,
                                              int32_t* num_emitted, int32_t* accepted, void* hip_stream) {
    if (batch < 0 || gamma < 0 || vocab < 1) return DFLASH_ERR_INVALID_ARG;
    if ((int64_t)(gamma + 1) * vocab > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (batch == 0) return DFLASH_OK;
    if (p == nullptr || u_draw == nullptr || emitted == nullptr || num_emitted == nullptr || accepted == nullptr ||
        (gamma > 0 && (draft == nullptr || q == nullptr || u_accept == nullptr)))
        return DFLASH_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    {
        ProfScope prof(DFLASH_KERNEL_VERIFY, st);
        hipLaunchKernelGGL(verify_sample_kernel, dim3(batch), dim3(kSampleThreads), 0, st, draft, p, q, u_accept,
                           u_draw, gamma, vocab, eos_token, emitted, num_emitted, accepted);
    }
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}
