// Union of the two queries' chunk sets, with per-query membership bits, and the
// optional hot-cache transfer plan of the host-pool path.
//
// Adaptive DHiSparse, Figure 3 (2): the selections of several queries are
// resolved together so every distinct chunk moves once while each query keeps
// its own selection.  DualDecoder "6.3": the overlap of the real and the
// speculative sets is the prediction accuracy.  Adaptive DHiSparse Figure 2 and
// the OasisKV summary's "KV selection" stage: compare the new set with the
// resident set and plan the copies of the missing chunks.
//
// One block per (b, g); the merge itself is block_union_two (dk_union_core.h).
#include "dk_common.h"
#include "dk_union_core.h"

namespace dk {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_union(
    const int32_t* __restrict__ topk_idx, int T, int k, int32_t* __restrict__ union_ids,
    uint8_t* __restrict__ member, int32_t* __restrict__ union_count, int32_t* __restrict__ overlap,
    int32_t* __restrict__ resident, int slots, int32_t* __restrict__ slot_of_union,
    int32_t* __restrict__ miss_chunk, int32_t* __restrict__ miss_slot,
    int32_t* __restrict__ miss_count, int32_t* __restrict__ hit_count) {
    extern __shared__ int32_t sm[];
    const int N = T * k;
    int32_t* s0 = sm;               // [k]
    int32_t* s1 = s0 + k;           // [k]
    int32_t* dup_pre = s1 + k;      // [k + 1]: shared chunks among S0[0..i)
    int32_t* u_ids = dup_pre + k + 1;   // [N] union ids (plan only)
    int32_t* scratch = u_ids + N;   // [8]
    const int tid = threadIdx.x;
    const int64_t bg = blockIdx.x;
    const int32_t* src = topk_idx + bg * T * k;
    int32_t* uo = union_ids + bg * N;
    uint8_t* mo = member + bg * N;

    for (int i = tid; i < k; i += kThreads) {
        s0[i] = src[i];
        s1[i] = T == 2 ? src[k + i] : 0;
    }
    __syncthreads();

    int nshared;
    const int count = block_union_two(s0, s1, T, k, uo, mo, dup_pre, scratch, u_ids, &nshared);
    if (tid == 0) {
        union_count[bg] = count;
        if (overlap) overlap[bg] = nshared;
    }
    if (resident == nullptr) return;

    // ---- hot-cache plan -------------------------------------------------------
    // Hits keep their slot; misses (ascending chunk order) take the free slots
    // (chunk not in the new union, or empty) in ascending slot order.
    __syncthreads();
    int32_t* res = scratch + 8;              // [slots] current resident table
    int32_t* free_list = res + slots;        // [slots] free slots in ascending order
    int32_t* u_slot = free_list + slots;     // [N] slot of each union entry (-1 = miss)
    int32_t* rs = resident + bg * slots;
    for (int s = tid; s < slots; s += kThreads) res[s] = rs[s];
    __syncthreads();

    // free slots, ranked by slot index
    int nfree;
    {
        const int per = (slots + kThreads - 1) / kThreads;
        const int lo = min(slots, tid * per), hi = min(slots, lo + per);
        int mine = 0;
        for (int s = lo; s < hi; ++s) {
            const int32_t c = res[s];
            const int p = c >= 0 ? lower_bound_i32(u_ids, count, c) : count;
            mine += !(p < count && u_ids[p] == c);
        }
        int total;
        int r = block_exclusive_scan(mine, scratch, &total);
        nfree = total;
        for (int s = lo; s < hi; ++s) {
            const int32_t c = res[s];
            const int p = c >= 0 ? lower_bound_i32(u_ids, count, c) : count;
            if (!(p < count && u_ids[p] == c)) free_list[r++] = s;
        }
    }
    // slot of each union entry that is already resident
    for (int i = tid; i < count; i += kThreads) u_slot[i] = -1;
    __syncthreads();
    for (int s = tid; s < slots; s += kThreads) {
        const int32_t c = res[s];
        if (c < 0) continue;
        const int p = lower_bound_i32(u_ids, count, c);
        if (p < count && u_ids[p] == c) u_slot[p] = s;
    }
    __syncthreads();
    // misses, ranked in union order
    {
        const int per = (count + kThreads - 1) / kThreads;
        const int lo = min(count, tid * per), hi = min(count, lo + per);
        int mine = 0;
        for (int i = lo; i < hi; ++i) mine += u_slot[i] < 0;
        int total;
        int r = block_exclusive_scan(mine, scratch, &total);
        int32_t* so = slot_of_union + bg * N;
        int32_t* mc = miss_chunk + bg * N;
        int32_t* ms = miss_slot + bg * N;
        for (int i = lo; i < hi; ++i) {
            int s = u_slot[i];
            if (s < 0) {
                // a resident table holding one chunk twice leaves too few free
                // slots; such entries get no slot rather than a stray one
                s = r < nfree ? free_list[r] : -1;
                mc[r] = u_ids[i];
                ms[r] = s;
                ++r;
                u_slot[i] = s;
            }
            so[i] = s;
        }
        for (int i = count + tid; i < N; i += kThreads) so[i] = -1;
        for (int i = total + tid; i < N; i += kThreads) { mc[i] = -1; ms[i] = -1; }
        if (tid == 0) {
            miss_count[bg] = total;
            hit_count[bg] = count - total;
        }
    }
    __syncthreads();
    // the cache now holds exactly the union
    for (int s = tid; s < slots; s += kThreads) rs[s] = -1;
    __syncthreads();
    for (int i = tid; i < count; i += kThreads)
        if (u_slot[i] >= 0 && u_slot[i] < slots) rs[u_slot[i]] = u_ids[i];
}

}  // namespace

hipError_t launch_union(const int32_t* topk_idx, int B, int Hkv, int T, int k, int C,
                        int32_t* union_ids, uint8_t* member, int32_t* union_count, int32_t* overlap,
                        const dk_cache_plan* plan, hipStream_t st) {
    (void)C;
    const int N = T * k;
    const int slots = plan ? plan->slots : 0;
    const size_t lds = (size_t)(2 * k + k + 1 + N + 8 + (plan ? 2 * slots + N : 0)) * 4;
    hipLaunchKernelGGL(k_union, dim3((unsigned)((int64_t)B * Hkv)), dim3(kThreads), lds, st,
                       topk_idx, T, k, union_ids, member, union_count, overlap,
                       plan ? plan->resident : nullptr, slots,
                       plan ? plan->slot_of_union : nullptr, plan ? plan->miss_chunk : nullptr,
                       plan ? plan->miss_slot : nullptr, plan ? plan->miss_count : nullptr,
                       plan ? plan->hit_count : nullptr);
    return hipGetLastError();
}

}  // namespace dk
