// Block-wide primitives of the 1024-thread selection kernels (coverage budgets,
// capped eviction): deterministic sums (fixed reduction tree, so equal inputs
// give equal bits and, rounding being monotone, sums of masked non-negative
// terms never grow when the mask shrinks), ballot-based ranks in element order,
// and the exact "best n by key, ties to the lowest index" threshold.
#pragma once

#include "dk_common.h"

namespace dk {
namespace blk {

constexpr int kBlkThreads = 1024;
constexpr int kBlkWaves = kBlkThreads / kWave;

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
    return v;
}

// Block sums of N values; every thread gets the same results (fixed order).
// buf: [N][kBlkWaves]; the caller alternates two buffers between calls, so one
// barrier per call suffices.
template <int N>
__device__ __forceinline__ void block_sums_f(float (&v)[N], float (*buf)[kBlkWaves]) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_sum_f(v[i]);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) buf[i][wave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kBlkWaves; ++w) s += buf[i][w];
        v[i] = s;
    }
}
template <int N>
__device__ __forceinline__ void block_sums_i(int (&v)[N], int (*buf)[kBlkWaves]) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_sum_i(v[i]);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) buf[i][wave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < kBlkWaves; ++w) s += buf[i][w];
        v[i] = s;
    }
}

// Exclusive ranks, in chunk-id order, of the flagged elements of R rows, and
// each row's total.  cnt: [R][EPT * kBlkWaves] ints, tot: [R].
template <int R, int EPT>
__device__ __forceinline__ void block_ranks(const bool (&flag)[R][EPT], int (&rank)[R][EPT], int (&total)[R],
                                            int* cnt, int* tot) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint64_t below = (1ull << lane) - 1ull;
    uint64_t bal[R][EPT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            bal[r][e] = __ballot(flag[r][e]);
            if (lane == 0) cnt[(r * EPT + e) * kBlkWaves + wave] = __popcll(bal[r][e]);
        }
    __syncthreads();
    if (wave < R) {
        // the counts of row `wave` in id order (e, then wave), scanned by one wave
        constexpr int N = EPT * kBlkWaves;
        constexpr int P = (N + kWave - 1) / kWave;
        int* c = cnt + wave * N;
        int loc[P];
        int s = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = lane * P + p;
            loc[p] = i < N ? c[i] : 0;
            s += loc[p];
        }
        const int inc = wave_inclusive_scan(s);
        int run = inc - s;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = lane * P + p;
            if (i < N) c[i] = run;
            run += loc[p];
        }
        if (lane == kWave - 1) tot[wave] = inc;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            rank[r][e] = cnt[(r * EPT + e) * kBlkWaves + wave] + __popcll(bal[r][e] & below);
        total[r] = tot[r];
    }
    __syncthreads();   // cnt and tot are free again
}

// The best n (1 <= n <= flagged count) of the flagged elements by key
// (larger first), ties to the lower element index (thread + kBlkThreads e).
// key: [EPT], flag: [EPT]; out: take[EPT].  Uses ibuf[2] alternately from *par.
template <int EPT>
__device__ __forceinline__ void block_best(const uint32_t (&key)[EPT], const bool (&flag)[EPT], int n,
                                           bool (&take)[EPT], int (*ibuf)[1][kBlkWaves], int& par, int* cnt,
                                           int* tot) {
    // the largest v with at least n flagged keys >= v
    uint32_t v = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = v | (1u << bit);
        int part[1] = {0};
#pragma unroll
        for (int e = 0; e < EPT; ++e) part[0] += flag[e] && key[e] >= cand ? 1 : 0;
        block_sums_i<1>(part, ibuf[par]);
        par ^= 1;
        if (part[0] >= n) v = cand;
    }
    int gt[1] = {0};
#pragma unroll
    for (int e = 0; e < EPT; ++e) gt[0] += flag[e] && key[e] > v ? 1 : 0;
    block_sums_i<1>(gt, ibuf[par]);
    par ^= 1;
    bool tie[1][EPT];
    int rank[1][EPT], total[1];
#pragma unroll
    for (int e = 0; e < EPT; ++e) tie[0][e] = flag[e] && key[e] == v;
    block_ranks<1, EPT>(tie, rank, total, cnt, tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e) take[e] = flag[e] && (key[e] > v || (tie[0][e] && rank[0][e] < n - gt[0]));
}

}  // namespace blk

// Wave-level versions: one wave owns a whole row (element j = lane + 64 e), so no
// barrier is needed.  Sums are a fixed tree (lane-serial, DPP sums of 16-lane
// rows, then the four rows read from lanes 0, 16, 32, 48 and added in order):
// deterministic, identical in every lane, and monotone in every term.
namespace wv {

__device__ __forceinline__ float sum_f(float v) {
    v = dpp_group_sum<16>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}
// integer sums below 2^24 are exact in fp32
__device__ __forceinline__ int sum_i(int v) { return (int)sum_f((float)v); }
__device__ __forceinline__ uint32_t max_u(uint32_t v) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ uint64_t lanes_below() { return (1ull << (threadIdx.x & (kWave - 1))) - 1ull; }

// The best n (1 <= n <= flagged count) of the flagged elements by key (larger
// first), ties to the lower element index (lane + 64 e).
template <int EPL>
__device__ __forceinline__ void best(const uint32_t (&key)[EPL], const bool (&flag)[EPL], int n, bool (&take)[EPL]) {
    uint32_t v = 0u;   // the largest v with at least n flagged keys >= v
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = v | (1u << bit);
        int part = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part += flag[e] && key[e] >= cand ? 1 : 0;
        if (sum_i(part) >= n) v = cand;
    }
    int gt = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) gt += flag[e] && key[e] > v ? 1 : 0;
    const int room = n - sum_i(gt);
    const uint64_t below = lanes_below();
    int pre = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const bool tie = flag[e] && key[e] == v;
        const uint64_t tb = __ballot(tie);
        take[e] = flag[e] && (key[e] > v || (tie && pre + __popcll(tb & below) < room));
        pre += __popcll(tb);
    }
}

}  // namespace wv
}  // namespace dk
