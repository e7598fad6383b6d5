// Delta selection with capped eviction over a bounded working set.
//
// OasisKV, "Delta Selection and Capped Eviction": blocks of the predicted set
// that are already resident cost no traffic; the resident blocks outside the set
// are ranked by the step at which they were last selected; each admitted
// non-resident block is paired with one eviction target, least recently
// selected first; at most `cap` pairs are admitted per step and KV head, which
// bounds the step's transfers to cap * Hkv blocks per request whatever the
// prediction does.
//
// Readings: hits keep their slot and are stamped with the step; targets are the
// slots whose chunk is not predicted, empty slots first, then the oldest stamp,
// then the lower slot; the admitted misses are the best min(cap, misses,
// targets) by (score descending, id ascending); they are paired in ascending
// chunk order with the chosen targets in ascending slot order.  Misses not
// admitted have no slot this step.
//
// One block of 1024 threads per (b, g); predicted entries and slots are held
// EPT per thread (index = thread + 1024 e).  A hit is found by a binary search of
// each occupied slot's chunk among the ascending predicted ids in LDS.  Admitted
// misses and the targets past the empty slots are the exact best n by a 32-bit
// key (score; inverted stamp) with ties to the lower index, by count bisection;
// both are then ranked in index order by ballots and paired rank to rank.
// resident and stamp are read whole before any of them is written, so the plan
// updates them in place.  Up to 512 entries and slots one wave does the same work
// alone (index = lane + 64 e), with wave reductions instead of block barriers.
#include "dk_block.h"

namespace dk {
namespace {

using namespace blk;

template <int EPT>
__global__ __launch_bounds__(kBlkThreads) void k_capped_plan(
    const int32_t* __restrict__ sel_ids, const float* __restrict__ sel_score, const int32_t* __restrict__ sel_count,
    int N, int64_t sel_stride, int64_t count_stride, int32_t* __restrict__ resident, int32_t* __restrict__ stamp,
    int S, int cap, int32_t step, int32_t* __restrict__ sel_slot, int32_t* __restrict__ admit_chunk,
    int32_t* __restrict__ admit_slot, int32_t* __restrict__ admit_count, int32_t* __restrict__ hit_count) {
    extern __shared__ int sm_cp[];
    int* pid = sm_cp;          // [N] predicted ids (INT_MAX past the count)
    int* hitslot = pid + N;    // [N] slot holding each predicted id, or -1
    int* tslot = hitslot + N;  // [min(N, S)] the chosen targets in slot order
    __shared__ int s_i3[2][3][kBlkWaves];
    __shared__ int s_i1[2][1][kBlkWaves];
    __shared__ int s_cnt[2 * EPT * kBlkWaves];
    __shared__ int s_tot[2];
    const int64_t bg = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t* ids = sel_ids + bg * sel_stride;
    const float* scr = sel_score ? sel_score + bg * sel_stride : nullptr;
    const int n = sel_count ? min(max(sel_count[bg * count_stride], 0), N) : N;
    int32_t* res = resident + bg * S;
    int32_t* st = stamp + bg * S;

    int my_id[EPT], my_res[EPT], my_st[EPT];
    uint32_t my_key[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * kBlkThreads;
        my_id[e] = i < n ? ids[i] : -1;
        my_key[e] = i < n && scr ? score_key(scr[i]) : 1u;   // no scores: all tied, lower id first
        if (i < N) {
            pid[i] = i < n ? my_id[e] : INT32_MAX;
            hitslot[i] = -1;
        }
        my_res[e] = i < S ? res[i] : -1;
        my_st[e] = i < S ? st[i] : 0;
    }
    __syncthreads();
    bool hit[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int s = tid + e * kBlkThreads;
        hit[e] = false;
        if (s < S && my_res[e] >= 0) {
            int lo = 0, hi = n;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (pid[mid] < my_res[e]) lo = mid + 1;
                else hi = mid;
            }
            if (lo < n && pid[lo] == my_res[e]) {
                hitslot[lo] = s;
                hit[e] = true;
            }
        }
    }
    __syncthreads();
    bool miss[EPT], emp[EPT], occ[EPT];
    int hs[EPT];
    int c3[3] = {0, 0, 0};
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * kBlkThreads;   // entry and slot index
        hs[e] = i < n ? hitslot[i] : -1;
        miss[e] = i < n && hs[e] < 0;
        emp[e] = i < S && my_res[e] < 0;
        occ[e] = i < S && my_res[e] >= 0 && !hit[e];
        c3[0] += miss[e] ? 1 : 0;
        c3[1] += emp[e] ? 1 : 0;
        c3[2] += occ[e] ? 1 : 0;
    }
    block_sums_i<3>(c3, s_i3[0]);
    int par = 0;
    const int n_miss = c3[0], n_empty = c3[1], n_occ = c3[2];
    const int a = min(min(cap, n_miss), n_empty + n_occ);

    bool adm[EPT], tgt[EPT];
    if (a == n_miss) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) adm[e] = miss[e];
    } else if (a == 0) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) adm[e] = false;
    } else {
        block_best<EPT>(my_key, miss, a, adm, s_i1, par, s_cnt, s_tot);
    }
    if (a == 0) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) tgt[e] = false;
    } else if (a <= n_empty) {
        bool f[1][EPT];
        int rk[1][EPT], tt[1];
#pragma unroll
        for (int e = 0; e < EPT; ++e) f[0][e] = emp[e];
        block_ranks<1, EPT>(f, rk, tt, s_cnt, s_tot);
#pragma unroll
        for (int e = 0; e < EPT; ++e) tgt[e] = emp[e] && rk[0][e] < a;
    } else if (a - n_empty == n_occ) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) tgt[e] = emp[e] || occ[e];
    } else {
        uint32_t old[EPT];   // larger = selected longer ago
        bool take[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) old[e] = ~((uint32_t)my_st[e] ^ 0x80000000u);
        block_best<EPT>(old, occ, a - n_empty, take, s_i1, par, s_cnt, s_tot);
#pragma unroll
        for (int e = 0; e < EPT; ++e) tgt[e] = emp[e] || take[e];
    }

    // pair the admitted misses (id order) with the targets (slot order)
    bool f2[2][EPT];
    int rk2[2][EPT], tt2[2];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        f2[0][e] = adm[e];
        f2[1][e] = tgt[e];
    }
    block_ranks<2, EPT>(f2, rk2, tt2, s_cnt, s_tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        if (tgt[e] && rk2[1][e] < a) tslot[rk2[1][e]] = tid + e * kBlkThreads;
    __syncthreads();

    int32_t* oslot = sel_slot + bg * N;
    int32_t* ac = admit_chunk ? admit_chunk + bg * cap : nullptr;
    int32_t* as = admit_slot ? admit_slot + bg * cap : nullptr;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * kBlkThreads;
        if (i < S && hit[e]) st[i] = step;
        if (i < N) {
            int slot = -1;
            if (hs[e] >= 0) {
                slot = hs[e];
            } else if (adm[e] && rk2[0][e] < a) {
                const int r = rk2[0][e];
                slot = tslot[r];
                res[slot] = my_id[e];
                st[slot] = step;
                ac[r] = my_id[e];
                as[r] = slot;
            }
            oslot[i] = slot;
        }
    }
    for (int r = a + tid; r < cap; r += kBlkThreads) {
        ac[r] = -1;
        as[r] = -1;
    }
    if (tid == 0) {
        admit_count[bg] = a;
        if (hit_count) hit_count[bg] = n - n_miss;
    }
}

template <int EPL>
__global__ __launch_bounds__(kWave) void k_capped_wave(
    const int32_t* __restrict__ sel_ids, const float* __restrict__ sel_score, const int32_t* __restrict__ sel_count,
    int N, int64_t sel_stride, int64_t count_stride, int32_t* __restrict__ resident, int32_t* __restrict__ stamp,
    int S, int cap, int32_t step, int32_t* __restrict__ sel_slot, int32_t* __restrict__ admit_chunk,
    int32_t* __restrict__ admit_slot, int32_t* __restrict__ admit_count, int32_t* __restrict__ hit_count) {
    extern __shared__ int sm_cw[];
    int* pid = sm_cw;          // [N] predicted ids (INT_MAX past the count)
    int* hitslot = pid + N;    // [N] slot holding each predicted id, or -1
    int* tslot = hitslot + N;  // [min(N, S)] the chosen targets in slot order
    const int64_t bg = blockIdx.x;
    const int lane = threadIdx.x;
    const uint64_t below = wv::lanes_below();
    const int32_t* ids = sel_ids + bg * sel_stride;
    const float* scr = sel_score ? sel_score + bg * sel_stride : nullptr;
    const int n = sel_count ? min(max(sel_count[bg * count_stride], 0), N) : N;
    int32_t* res = resident + bg * S;
    int32_t* st = stamp + bg * S;

    int my_id[EPL], my_res[EPL], my_st[EPL];
    uint32_t my_key[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int i = lane + e * kWave;
        my_id[e] = i < n ? ids[i] : -1;
        my_key[e] = i < n && scr ? score_key(scr[i]) : 1u;   // no scores: all tied, lower id first
        if (i < N) {
            pid[i] = i < n ? my_id[e] : INT32_MAX;
            hitslot[i] = -1;
        }
        my_res[e] = i < S ? res[i] : -1;
        my_st[e] = i < S ? st[i] : 0;
    }
    __syncthreads();
    bool hit[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int s = lane + e * kWave;
        hit[e] = false;
        if (s < S && my_res[e] >= 0) {
            int lo = 0, hi = n;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (pid[mid] < my_res[e]) lo = mid + 1;
                else hi = mid;
            }
            if (lo < n && pid[lo] == my_res[e]) {
                hitslot[lo] = s;
                hit[e] = true;
            }
        }
    }
    __syncthreads();
    bool miss[EPL], emp[EPL], occ[EPL];
    int hs[EPL];
    int c0 = 0, c1 = 0, c2 = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int i = lane + e * kWave;
        hs[e] = i < n ? hitslot[i] : -1;
        miss[e] = i < n && hs[e] < 0;
        emp[e] = i < S && my_res[e] < 0;
        occ[e] = i < S && my_res[e] >= 0 && !hit[e];
        c0 += miss[e] ? 1 : 0;
        c1 += emp[e] ? 1 : 0;
        c2 += occ[e] ? 1 : 0;
    }
    const int n_miss = wv::sum_i(c0), n_empty = wv::sum_i(c1), n_occ = wv::sum_i(c2);
    const int a = min(min(cap, n_miss), n_empty + n_occ);

    bool adm[EPL], tgt[EPL];
    if (a == n_miss) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) adm[e] = miss[e];
    } else if (a == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) adm[e] = false;
    } else {
        wv::best<EPL>(my_key, miss, a, adm);
    }
    if (a == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) tgt[e] = false;
    } else if (a <= n_empty) {
        int pre = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint64_t b = __ballot(emp[e]);
            tgt[e] = emp[e] && pre + __popcll(b & below) < a;
            pre += __popcll(b);
        }
    } else if (a - n_empty == n_occ) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) tgt[e] = emp[e] || occ[e];
    } else {
        uint32_t old[EPL];   // larger = selected longer ago
        bool take[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) old[e] = ~((uint32_t)my_st[e] ^ 0x80000000u);
        wv::best<EPL>(old, occ, a - n_empty, take);
#pragma unroll
        for (int e = 0; e < EPL; ++e) tgt[e] = emp[e] || take[e];
    }

    // pair the admitted misses (id order) with the targets (slot order)
    int ra[EPL];
    int tpre = 0, apre = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const uint64_t tb = __ballot(tgt[e]);
        const int rt = tpre + __popcll(tb & below);
        if (tgt[e] && rt < a) tslot[rt] = lane + e * kWave;
        tpre += __popcll(tb);
        const uint64_t ab = __ballot(adm[e]);
        ra[e] = apre + __popcll(ab & below);
        apre += __popcll(ab);
    }
    __syncthreads();

    int32_t* oslot = sel_slot + bg * N;
    int32_t* ac = admit_chunk ? admit_chunk + bg * cap : nullptr;
    int32_t* as = admit_slot ? admit_slot + bg * cap : nullptr;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int i = lane + e * kWave;
        if (i < S && hit[e]) st[i] = step;
        if (i < N) {
            int slot = -1;
            if (hs[e] >= 0) {
                slot = hs[e];
            } else if (adm[e] && ra[e] < a) {
                slot = tslot[ra[e]];
                res[slot] = my_id[e];
                st[slot] = step;
                ac[ra[e]] = my_id[e];
                as[ra[e]] = slot;
            }
            oslot[i] = slot;
        }
    }
    for (int r = a + lane; r < cap; r += kWave) {
        ac[r] = -1;
        as[r] = -1;
    }
    if (lane == 0) {
        admit_count[bg] = a;
        if (hit_count) hit_count[bg] = n - n_miss;
    }
}

}  // namespace

hipError_t launch_capped_plan(const int32_t* sel_ids, const float* sel_score, const int32_t* sel_count, int B,
                              int Hkv, int N, int64_t sel_stride, int64_t count_stride, int32_t* resident,
                              int32_t* stamp, int S, int cap, int32_t step, int32_t* sel_slot, int32_t* admit_chunk,
                              int32_t* admit_slot, int32_t* admit_count, int32_t* hit_count, hipStream_t st) {
    const int m = N > S ? N : S;
    const size_t lds = (2 * (size_t)N + (size_t)(N < S ? N : S)) * 4;
    const dim3 grid((unsigned)((int64_t)B * Hkv));
#define DK_CP(E_)                                                                                                   \
    hipLaunchKernelGGL(k_capped_plan<E_>, grid, dim3(kBlkThreads), lds, st, sel_ids, sel_score, sel_count, N,    \
                       sel_stride, count_stride, resident, stamp, S, cap, step, sel_slot, admit_chunk, admit_slot, \
                       admit_count, hit_count)
#define DK_CW(E_)                                                                                                   \
    hipLaunchKernelGGL(k_capped_wave<E_>, grid, dim3(kWave), lds, st, sel_ids, sel_score, sel_count, N, sel_stride, \
                       count_stride, resident, stamp, S, cap, step, sel_slot, admit_chunk, admit_slot, admit_count,  \
                       hit_count)
    static_assert(kCappedMaxN <= 4 * kBlkThreads, "four entries per thread at most");
    if (m <= 2 * kWave) DK_CW(2);
    else if (m <= 4 * kWave) DK_CW(4);
    else if (m <= 8 * kWave) DK_CW(8);
    else if (m <= kBlkThreads) DK_CP(1);
    else if (m <= 2 * kBlkThreads) DK_CP(2);
    else if (m <= kCappedMaxN) DK_CP(4);
    else return hipErrorInvalidValue;
#undef DK_CP
#undef DK_CW
    return hipGetLastError();
}

}  // namespace dk
