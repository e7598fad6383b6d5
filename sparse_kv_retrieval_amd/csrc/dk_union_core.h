// Block-wide union of two ascending chunk lists with membership bits.
//
// Adaptive DHiSparse, Figure 3 (2): the selections of several queries are
// resolved together so every distinct chunk moves once while each query keeps
// its own selection.  DualDecoder "6.3": the overlap of the real and the
// speculative sets is the prediction accuracy.
//
// Both inputs are strictly ascending, so the union is a merge: S0[i] lands at
// i + |{S1 < S0[i]}| - |{S0 & S1 below it}| and a chunk of S1 that S0 lacks
// lands at |{S0 < y}| + j - |{S0 & S1 below it}|.  The shared-chunk counts
// come from one block scan over S0's "also in S1" flags.
#pragma once

#include "dk_common.h"

namespace dk {

// |{a[i] < x}| for an ascending a of n <= 64 entries: fixed steps, no branches
// on the data, so two searches of one lane interleave their LDS reads.
__device__ __forceinline__ int lower_bound_64(const int32_t* a, int n, int32_t x) {
    int lo = 0;
#pragma unroll
    for (int s = 64; s >= 1; s >>= 1)
        if (lo + s <= n && a[lo + s - 1] < x) lo += s;
    return lo;
}

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int32_t x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Every thread of the block calls it.  s0, s1: the T (1 or 2) ascending lists
// of length k in LDS (s1 unused when T == 1); dup_pre: LDS scratch of k + 1
// ints; scratch: LDS scratch for block_exclusive_scan.  Writes the N = T * k
// union entries (ascending, -1 / 0 padded) to uo / mo and, when u_ids is not
// null, the union ids to u_ids (LDS).  Returns the union size; *nshared gets
// |S0 & S1| (k when T == 1).  Rows that are not ascending produce a union that
// stays inside [0, N) but is otherwise unspecified.
__device__ __forceinline__ int block_union_two(const int32_t* s0, const int32_t* s1, int T, int k,
                                               int32_t* uo, uint8_t* mo, int32_t* dup_pre,
                                               int* scratch, int32_t* u_ids, int* nshared) {
    const int N = T * k;
    const int tid = threadIdx.x, nthr = blockDim.x;
    int count;
    if (T == 1) {
        for (int i = tid; i < k; i += nthr) {
            uo[i] = s0[i];
            mo[i] = 1;
            if (u_ids) u_ids[i] = s0[i];
        }
        count = k;
        *nshared = k;
    } else if (k <= kWave) {
        // One wave: lane l searches S0[l] in S1 and S1[l] in S0; the shared
        // chunks below a position come from one ballot, not a block scan.
        if (tid < kWave) {
            const bool h = tid < k;
            const int32_t x = h ? s0[tid] : 0, y = h ? s1[tid] : 0;
            const int j = h ? lower_bound_64(s1, k, x) : k;
            const int i = h ? lower_bound_64(s0, k, y) : k;
            const bool both = h && j < k && s1[j] == x;
            const bool iny = h && i < k && s0[i] == y;
            const uint64_t dm = __builtin_amdgcn_ballot_w64(both);
            const auto below = [](int n) { return n <= 0 ? 0ull : (n >= 64 ? ~0ull : (~0ull >> (64 - n))); };
            if (h) {
                const int pos = tid + j - __builtin_popcountll(dm & below(tid));
                if (pos >= 0 && pos < N) {
                    uo[pos] = x;
                    mo[pos] = both ? 3 : 1;
                    if (u_ids) u_ids[pos] = x;
                }
            }
            if (h && !iny) {
                const int pos = i + tid - __builtin_popcountll(dm & below(i));
                if (pos >= 0 && pos < N) {
                    uo[pos] = y;
                    mo[pos] = 2;
                    if (u_ids) u_ids[pos] = y;
                }
            }
            if (tid == 0) scratch[0] = __builtin_popcountll(dm);
        }
        __syncthreads();
        const int total = scratch[0];
        *nshared = total;
        count = 2 * k - total;
    } else {
        // flags of S0 entries that S1 also holds, scanned in S0 order
        const int per = (k + nthr - 1) / nthr;
        const int lo = min(k, tid * per), hi = min(k, lo + per);
        int mine = 0;
        for (int i = lo; i < hi; ++i) {
            const int j = lower_bound_i32(s1, k, s0[i]);
            mine += (j < k && s1[j] == s0[i]);
        }
        int total;
        int run = block_exclusive_scan(mine, scratch, &total);
        for (int i = lo; i < hi; ++i) {
            dup_pre[i] = run;
            const int j = lower_bound_i32(s1, k, s0[i]);
            run += (j < k && s1[j] == s0[i]);
        }
        if (tid == 0) dup_pre[k] = total;
        __syncthreads();
        *nshared = total;
        count = 2 * k - total;
        for (int i = tid; i < k; i += nthr) {
            const int32_t x = s0[i];
            const int j = lower_bound_i32(s1, k, x);
            const bool both = j < k && s1[j] == x;
            const int pos = i + j - dup_pre[i];
            if (pos < 0 || pos >= N) continue;   // only for rows that are not ascending
            uo[pos] = x;
            mo[pos] = both ? 3 : 1;
            if (u_ids) u_ids[pos] = x;
        }
        for (int j = tid; j < k; j += nthr) {
            const int32_t y = s1[j];
            const int i = lower_bound_i32(s0, k, y);
            if (i < k && s0[i] == y) continue;
            const int pos = i + j - dup_pre[i];
            if (pos < 0 || pos >= N) continue;
            uo[pos] = y;
            mo[pos] = 2;
            if (u_ids) u_ids[pos] = y;
        }
    }
    for (int i = count + tid; i < N; i += nthr) {
        uo[i] = -1;
        mo[i] = 0;
    }
    return count;
}

}  // namespace dk
