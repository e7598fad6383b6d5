// Token-level indexer: exact top-k token positions from bf16 indexer keys.
//
// Adaptive DHiSparse, Figure 2: an indexer turns its index state into the
// top-k positions a decode step reads; Table 3: 2,048 positions per selecting
// layer.  Every token of a (request, KV head) has one indexer key, so the keys
// are their own landmarks (chunk = 1) and a token's score is the mean over the
// query heads of the group of the scaled dot products, as for chunk scores.
// The set is the k best tokens, ties to the lower position, in ascending order.
//
// Two kernels:
//   k_idx_score  : streams the bf16 keys once (non-temporal 16-byte loads, D/8
//                  lanes per row), writes fp32 scores of every token for each
//                  query of the request to the workspace, and each block's
//                  score range.
//   k_idx_select : one block per (b, g, t).  Finds the threshold pair
//                  (tau, id_tau), the k-th element in (score descending,
//                  position ascending) order, then writes every position with
//                  score > tau, or score == tau and position <= id_tau, in
//                  ascending order.  The k-th element's bin comes from a
//                  histogram over 2048 bins linear in the score between the
//                  row's minimum and maximum (one row's scores cluster; linear
//                  bins spread them, where the float's exponent bits would not).
//                  That bin's elements are gathered into LDS and ranked exactly.
//                  A bin too large to gather falls back to an 11/11/10-bit radix
//                  select over order-preserving keys inside it, followed by a
//                  count of the equal keys in position order.  Every pass keeps
//                  eight 16-byte loads per lane in flight.  With union outputs,
//                  the last of the T blocks of a (b, g) merges its T sets
//                  (Adaptive DHiSparse, Figure 3 (2)).
#include "dk_common.h"
#include "dk_union_core.h"

namespace dk {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreRows = 1024;   // tokens per scoring block (the workspace's per-block ranges)
// Scoring blocks are made longer (doubling up to 8192 rows, at most the row
// rounded up) as long as at least kScoreMinBlocks blocks remain, two per CU:
// fewer block starts and epilogues, one resident round.  Measured on 32 rows of
// 131072 tokens (512 blocks of 8192): the scoring call 230-231 us against
// 251-252 us with 1024-row blocks; 16384 rows (one block per CU) took 280 us.
constexpr int kScoreRowsLong = 8192;
constexpr int kScoreMinBlocks = 512;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBins = 2048;        // = 2 * kSelThreads
constexpr int kCap = 2048;         // candidates ranked in LDS

// ---------------------------------------------------------------------------
// Scores: s[b, g, t, n] = scale * <mean over the group's heads of q[b, t, h], key[b, g, n]>
// (the mean of the scaled per-head dots, up to fp32 rounding).
// ---------------------------------------------------------------------------
template <int D, int T, int RPB>
__global__ __launch_bounds__(kScoreThreads) void k_idx_score(const float* __restrict__ q, int Hq,
                                                            const uint16_t* __restrict__ keys, dk_strides ks,
                                                            int Hkv, int C, float scale, int blocks_per_bg,
                                                            float* __restrict__ scores, float* __restrict__ bmin,
                                                            float* __restrict__ bmax, uint32_t* __restrict__ arrivals) {
    constexpr int LPR = D / 8, RPW = kWave / LPR, U = 8, ROWS_PER_ITER = 4 * RPW * U;
    __shared__ float sres[T][RPB];
    __shared__ __align__(16) float qs[T][D];
    __shared__ float red[2][T][kScoreThreads / kWave];
    const int blk = blockIdx.x % blocks_per_bg;
    const int bg = blockIdx.x / blocks_per_bg;
    const int b = bg / Hkv, g = bg - b * Hkv;
    const int row0 = blk * RPB;
    const int nrows = min(RPB, C - row0);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int rp = lane / LPR, part = lane % LPR;
    const int G = Hq / Hkv;
    // the selection kernel that follows counts its (b, g, t) blocks from zero
    if (arrivals && blk == 0 && threadIdx.x == 0) arrivals[bg] = 0u;

    // the first rows are requested before the query staging
    const uint16_t* base = keys + (int64_t)b * ks.b + (int64_t)g * ks.h + (int64_t)row0 * ks.t + part * 8;
    u32x4_t x[U];
    auto load_rows = [&](int it) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = it + (u * 4 + wave) * RPW + rp;
            x[u] = r < nrows ? nt_load_u4(base + (int64_t)r * ks.t) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    load_rows(0);
    for (int i = threadIdx.x; i < T * D; i += kScoreThreads) {
        const int t = i / D, e = i - t * D;
        float acc = 0.f;
        for (int h = 0; h < G; ++h) acc += q[(((int64_t)b * T + t) * Hq + g * G + h) * D + e];
        qs[t][e] = acc / (float)G;
    }
    __syncthreads();
    float qr[T][8];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[t][e] = qs[t][part * 8 + e];

    for (int it = 0; it < nrows; it += ROWS_PER_ITER) {
        if (it) load_rows(it);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = it + (u * 4 + wave) * RPW + rp;
            const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
            float sc[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    a = fmaf(qr[t][2 * j], bf16_lo(w[j]), a);
                    a = fmaf(qr[t][2 * j + 1], bf16_hi(w[j]), a);
                }
                sc[t] = scale * dpp_group_sum<LPR>(a);
            }
            if (part < T && r < nrows) sres[part][r] = part == 0 ? sc[0] : sc[T - 1];
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float* dst = scores + ((int64_t)bg * T + t) * C + row0;
        float lo = INFINITY, hi = -INFINITY;
        for (int i = threadIdx.x; i < nrows; i += kScoreThreads) {
            const float v = sres[t][i];
            dst[i] = v;
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
        }
        for (int off = 1; off < kWave; off <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, off, kWave));
            hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
        }
        if (lane == 0) {
            red[0][t][wave] = lo;
            red[1][t][wave] = hi;
        }
    }
    __syncthreads();
    if (threadIdx.x < T) {
        const int t = threadIdx.x;
        float lo = red[0][t][0], hi = red[1][t][0];
        for (int w2 = 1; w2 < kScoreThreads / kWave; ++w2) {
            lo = fminf(lo, red[0][t][w2]);
            hi = fmaxf(hi, red[1][t][w2]);
        }
        bmin[((int64_t)bg * T + t) * blocks_per_bg + blk] = lo;
        bmax[((int64_t)bg * T + t) * blocks_per_bg + blk] = hi;
    }
}

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------
// linear bin of a score: non-decreasing in v, 0 for every v when inv == 0
__device__ __forceinline__ int bin_of(float v, float lo, float inv) {
    const float x = (v - lo) * inv;
    if (!(x > 0.f)) return 0;
    if (x >= (float)(kBins - 1)) return kBins - 1;
    return (int)x;
}

// exclusive scan over the lanes of a wave; *total gets the wave's sum
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
    const int inc = wave_inclusive_scan(v);
    *total = __shfl(inc, kWave - 1, kWave);
    return inc - v;
}

__device__ __forceinline__ int wave_sum(int v) {
    for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Of the bins hist[0 .. nb) (nb <= 2 * blockDim.x), the one that holds the need-th
// largest element, counting from the top bin.  Every thread gets the bin, the
// elements in the bins above it (*above) and in it (*in).
__device__ __forceinline__ int pick_bin(const int* hist, int nb, int need, int* scratch, int* ish,
                                        int* above, int* in) {
    const int tid = threadIdx.x;
    const int b_hi = nb - 1 - 2 * tid, b_lo = b_hi - 1;
    const int c_hi = b_hi >= 0 ? hist[b_hi] : 0, c_lo = b_lo >= 0 ? hist[b_lo] : 0;
    int tot;
    const int before = block_exclusive_scan(c_hi + c_lo, scratch, &tot);
    if (before < need && need <= before + c_hi + c_lo) {
        const bool top = before + c_hi >= need;
        ish[0] = top ? b_hi : b_lo;
        ish[1] = top ? before : before + c_hi;
        ish[2] = top ? c_hi : c_lo;
    }
    __syncthreads();
    *above = ish[1];
    *in = ish[2];
    const int r = ish[0];
    __syncthreads();
    return r;
}

// Eight 256-position chunks of a wave's segment per step, every load issued
// before the first is used; f(i0, v) gets each chunk's first position and values.
#ifndef DK_SEL_SEGMENT_UNROLL
#define DK_SEL_SEGMENT_UNROLL 8   // 16-byte score loads in flight per lane while a wave scans its segment
#endif
template <typename F>
__device__ __forceinline__ void for_segment(const float* s, int s0, int s1, F f) {
    constexpr int U = DK_SEL_SEGMENT_UNROLL;
    const int lane = threadIdx.x & (kWave - 1);
    for (int c0 = s0; c0 < s1; c0 += 256 * U) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i0 = c0 + 256 * u + 4 * lane;
            v[u] = i0 < s1 ? *reinterpret_cast<const float4*>(s + i0) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i0 = c0 + 256 * u + 4 * lane;
            if (c0 + 256 * u < s1) f(i0, v[u]);       // wave-uniform: the chunk is (partly) in range
        }
    }
}

constexpr int kSelPool = 4 * 4096 + 16;   // ints: hist + candidates (+ the ordered lists), or the union merge
constexpr int kMaxSplitK = 4096;          // the split selection keeps at most this many positions per row
constexpr int kMaxSlices = 8;             // slices per row of the split selection
constexpr int kSplitMinC = 32768;         // rows at least this long are split

// LDS of one selection block
struct SelLds {
    int* pool;        // [kSelPool]
    int* scratch;     // [kSelWaves + 1]
    int* wsel;        // [kSelWaves]: positions each wave's segment contributes
    int* weq;         // [kSelWaves]
    int* ish;         // [8]
    float* fsh;       // [2]
    uint32_t* ush;    // [1]
};
#define DK_SEL_LDS                                     \
    __shared__ int pool_[kSelPool];                    \
    __shared__ int scratch_[kSelWaves + 1];            \
    __shared__ int wsel_[kSelWaves];                   \
    __shared__ int weq_[kSelWaves];                    \
    __shared__ int ish_[8];                            \
    __shared__ float fsh_[2];                          \
    __shared__ uint32_t ush_[1];                       \
    SelLds L;                                          \
    L.pool = pool_;                                    \
    L.scratch = scratch_;                              \
    L.wsel = wsel_;                                    \
    L.weq = weq_;                                      \
    L.ish = ish_;                                      \
    L.fsh = fsh_;                                      \
    L.ush = ush_

// The row's score range from the scoring blocks' ranges: every thread gets the
// same lo and bins-per-unit (one wave reduces in a fixed order; a barrier follows).
__device__ __forceinline__ void row_range(const float* bmin, const float* bmax, int row, int blocks_per_row,
                                          float* fsh, float* lo_out, float* inv_out) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    if (tid < kWave) {
        float lo = INFINITY, hi = -INFINITY;
        for (int i = lane; i < blocks_per_row; i += kWave) {
            lo = fminf(lo, bmin[(int64_t)row * blocks_per_row + i]);
            hi = fmaxf(hi, bmax[(int64_t)row * blocks_per_row + i]);
        }
        for (int off = 1; off < kWave; off <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, off, kWave));
            hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
        }
        if (lane == 0) {
            fsh[0] = lo;
            fsh[1] = hi;
        }
    }
    __syncthreads();
    const float lo = fsh[0];
    const float span = fsh[1] - lo;
    *lo_out = lo;
    *inv_out = span > 0.f ? (float)kBins / span : 0.f;
}

// The k best positions of one row (ties to the lower position), written in
// ascending order by one block.
__device__ __forceinline__ void select_row(const float* __restrict__ scores, const float* __restrict__ bmin,
                           const float* __restrict__ bmax, int blocks_per_row, int row, int C, int k,
                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_score, const SelLds& L) {
    int* pool = L.pool;
    int* scratch = L.scratch;
    int* wsel = L.wsel;
    int* weq = L.weq;
    int* ish = L.ish;
    float* fsh = L.fsh;
    uint32_t* ush = L.ush;
    int* hist = pool;                                   // [kBins]
    float* cval = reinterpret_cast<float*>(pool + kBins);   // [kCap]
    int* cid = pool + kBins + kCap;                     // [kCap]

    const float* s = scores + (int64_t)row * C;
    int32_t* out = topk_idx + (int64_t)row * k;
    float* outs = topk_score ? topk_score + (int64_t)row * k : nullptr;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    // wave w owns positions [w * seg, (w + 1) * seg)
    const int seg = ((C + kSelWaves - 1) / kSelWaves + 255) & ~255;
    const int s0 = wave * seg, s1 = min(C, s0 + seg);

    if (k >= C) {
        for (int i = tid; i < C; i += kSelThreads) {
            store_agent(out + i, i);
            if (outs) outs[i] = s[i];
        }
    } else {
        // the row's range, from the scoring blocks
        for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
        float lo, inv;
        row_range(bmin, bmax, row, blocks_per_row, fsh, &lo, &inv);

        // ---- linear-bin histogram of the row
        for_segment(s, s0, s1, [&](int i0, const float4& v4) {
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i0 + j < s1) atomicAdd(&hist[bin_of(vv[j], lo, inv)], 1);
        });
        __syncthreads();
        int above, inside;
        const int p0 = pick_bin(hist, kBins, k, scratch, ish, &above, &inside);
        int need = k - above;     // elements to take from inside bin p0 (1 <= need <= inside)

        uint32_t tau_key;
        int id_tau;
        if (inside <= kCap) {
            // ---- gather bin p0; count per wave the elements of higher bins
            if (tid == 0) ish[3] = 0;
            if (tid < kSelWaves) wsel[tid] = 0;
            __syncthreads();
            int n_above = 0;
            for_segment(s, s0, s1, [&](int i0, const float4& v4) {
                const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (i0 + j >= s1) continue;
                    const int bn = bin_of(vv[j], lo, inv);
                    if (bn > p0) {
                        ++n_above;
                    } else if (bn == p0) {
                        const int slot = atomicAdd(&ish[3], 1);
                        cval[slot] = vv[j];
                        cid[slot] = i0 + j;
                    }
                }
            });
            n_above = wave_sum(n_above);
            if (lane == 0) atomicAdd(&wsel[wave], n_above);
            __syncthreads();
            // exact rank of each candidate in (score descending, position ascending) order
            const int n = ish[3];
            for (int i = tid; i < n; i += kSelThreads) {
                const float v = cval[i];
                const int id = cid[i];
                int rank = 0;
                for (int j = 0; j < n; ++j) {
                    const float u = cval[j];
                    rank += (u > v) || (u == v && cid[j] < id);
                }
                if (rank < need) atomicAdd(&wsel[id / seg], 1);
                if (rank == need - 1) {
                    ush[0] = score_key(v);
                    ish[2] = id;
                }
            }
            __syncthreads();
            tau_key = ush[0];
            id_tau = ish[2];
        } else {
            // ---- radix select over the keys inside bin p0: 11, 11 and 10 bits
            uint32_t prefix = 0;
            const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
            for (int pz = 0; pz < 3; ++pz) {
                const int sh = shifts[pz], nb = 1 << widths[pz];
                const uint32_t hmask = pz == 0 ? 0u : ~((1u << (sh + widths[pz])) - 1u);
                for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
                __syncthreads();
                for_segment(s, s0, s1, [&](int i0, const float4& v4) {
                    const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (i0 + j >= s1 || bin_of(vv[j], lo, inv) != p0) continue;
                        const uint32_t kv = score_key(vv[j]);
                        if ((kv & hmask) == prefix) atomicAdd(&hist[(kv >> sh) & (uint32_t)(nb - 1)], 1);
                    }
                });
                __syncthreads();
                int ab, in;
                const int d = pick_bin(hist, nb, need, scratch, ish, &ab, &in);
                need -= ab;
                prefix |= (uint32_t)d << sh;
            }
            tau_key = prefix;
            // need of the elements with key tau_key (all inside bin p0) are taken, the
            // lowest positions first; per wave: elements above tau_key and equal to it
            int n_gt = 0, n_eq = 0;
            for_segment(s, s0, s1, [&](int i0, const float4& v4) {
                const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (i0 + j >= s1) continue;
                    const uint32_t kv = score_key(vv[j]);
                    n_gt += kv > tau_key;
                    n_eq += kv == tau_key;
                }
            });
            n_gt = wave_sum(n_gt);
            n_eq = wave_sum(n_eq);
            if (lane == 0) {
                wsel[wave] = n_gt;
                weq[wave] = n_eq;
            }
            __syncthreads();
            if (tid == 0) {
                int run = 0;
                for (int w2 = 0; w2 < kSelWaves; ++w2) {
                    const int e = weq[w2];
                    const int take = min(e, max(0, need - run));
                    wsel[w2] += take;
                    weq[w2] = run;          // equal keys before wave w2's segment
                    run += e;
                }
            }
            __syncthreads();
            // the wave whose segment holds the need-th equal key finds its position
            const int before = weq[wave];
            const int mine = (wave + 1 < kSelWaves ? weq[wave + 1] : 0x7fffffff) - before;
            if (before < need && need - before <= mine) {
                int run = before;
                for (int c0 = s0; c0 < s1 && run < need; c0 += 256) {
                    const int i0 = c0 + lane * 4;
                    int f[4] = {0, 0, 0, 0};
                    if (i0 < s1) {
                        const float4 v4 = *reinterpret_cast<const float4*>(s + i0);
                        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) f[j] = i0 + j < s1 && score_key(vv[j]) == tau_key;
                    }
                    int tot;
                    const int ex = wave_excl_scan(f[0] + f[1] + f[2] + f[3], &tot);
                    int r = run + ex;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (f[j]) {
                            if (r == need - 1) ish[2] = i0 + j;
                            ++r;
                        }
                    }
                    run += tot;
                }
            }
            __syncthreads();
            id_tau = ish[2];
        }

        // ---- per-wave output offsets, then the positions in ascending order
        if (tid == 0) {
            int run = 0;
            for (int w2 = 0; w2 < kSelWaves; ++w2) {
                const int c = wsel[w2];
                wsel[w2] = run;
                run += c;
            }
        }
        __syncthreads();
        // positions in ascending order are (lane, j) within a group of four: one
        // ballot per j gives every flagged element its rank without a scan, and a
        // group with nothing selected (most of them) costs four compares
        int run = wsel[wave];
        const uint64_t below = (1ull << lane) - 1ull;
        for_segment(s, s0, s1, [&](int i0, const float4& v4) {
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
            bool f[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t kv = score_key(vv[j]);
                f[j] = i0 + j < s1 && (kv > tau_key || (kv == tau_key && i0 + j <= id_tau));
            }
            const uint64_t m0 = __ballot(f[0]), m1 = __ballot(f[1]), m2 = __ballot(f[2]), m3 = __ballot(f[3]);
            if ((m0 | m1 | m2 | m3) == 0ull) return;
            int pos = run + __popcll(m0 & below) + __popcll(m1 & below) + __popcll(m2 & below) +
                      __popcll(m3 & below);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (f[j]) {
                    if (pos < k) {
                        store_agent(out + pos, i0 + j);
                        if (outs) outs[pos] = vv[j];
                    }
                    ++pos;
                }
            }
            run += __popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3);
        });
    }
}

// Union of the (b, g)'s T sets, by the last of its T blocks to finish.  The
// positions were stored at agent scope; once every lane's stores have completed
// the block counts itself in, and the last block reads all T sets back at agent
// scope.  The scoring kernel of the same call zeroed the counter.
__device__ __forceinline__ void union_last(int bg, int T, int k, const int32_t* __restrict__ topk_idx, const UnionOut& un,
                           uint32_t* __restrict__ arrivals, const SelLds& L) {
    const int tid = threadIdx.x;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        L.ish[7] = __hip_atomic_fetch_add(&arrivals[bg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned)(T - 1);
    __syncthreads();
    if (!L.ish[7]) return;
    int32_t* u0s = L.pool;               // the selection's LDS is free now
    int32_t* u1s = u0s + k;
    int32_t* dup_pre = u1s + k;
    const int32_t* src = topk_idx + (int64_t)bg * T * k;
    for (int i = tid; i < k; i += kSelThreads) {
        u0s[i] = load_agent(src + i);
        u1s[i] = T == 2 ? load_agent(src + k + i) : 0;
    }
    __syncthreads();
    const int N = T * k;
    int nshared;
    const int count = block_union_two(u0s, u1s, T, k, un.ids + (int64_t)bg * N, un.member + (int64_t)bg * N,
                                      dup_pre, L.scratch, nullptr, &nshared);
    if (tid == 0) {
        un.count[bg] = count;
        if (un.overlap) un.overlap[bg] = nshared;
    }
}

__global__ __launch_bounds__(kSelThreads) void k_idx_select(const float* __restrict__ scores,
                                                           const float* __restrict__ bmin,
                                                           const float* __restrict__ bmax, int blocks_per_row,
                                                           int T, int C, int k, int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_score, UnionOut un,
                                                           uint32_t* __restrict__ arrivals) {
    DK_SEL_LDS;
    const int row = blockIdx.x;
    select_row(scores, bmin, bmax, blocks_per_row, row, C, k, topk_idx, topk_score, L);
    if (un.ids == nullptr) return;
    union_last(row / T, T, k, topk_idx, un, arrivals, L);
}

// ---------------------------------------------------------------------------
// Split selection for long rows: a row streams through one CU at a fraction of
// the chip's bandwidth, so rows of 32768 scores or more are cut into P slices
// of Ls positions (a multiple of 16 * 256) and three kernels share the work.
//   k_sel_hist   (P blocks per row): the slice's histogram over the row's
//                linear bins, to the workspace.
//   k_sel_gather (P blocks per row): the P histograms summed (the same sums in
//                every block), the threshold bin p0 as select_row picks it; the
//                slice's positions of higher bins in ascending order (a count
//                pass, then a write pass with ballot ranks) and its positions
//                inside p0, to the workspace.  A row whose bin p0 holds more
//                than kCap positions is flagged.
//   k_sel_final  (one block per row): flagged rows run select_row.  Otherwise
//                the candidates of p0 are ranked (score descending, position
//                ascending) and the best (k - above) kept; every kept position
//                goes to its rank in the ascending merge of the two lists.
// The result equals select_row's.  The blocks of a row share an XCD.
// ---------------------------------------------------------------------------
struct SplitArgs {
    const float* scores;
    const float* bmin;
    const float* bmax;
    int blocks_per_row, C, k, P, Ls, acap;
    int* hist;          // [rows][P][kBins]
    int32_t* a_id;      // [rows][P][acap]: positions of higher bins, ascending
    float* a_val;
    int32_t* c_id;      // [rows][P][kCap]: positions inside p0
    float* c_val;
    int* cnt;           // [rows][P][2]: higher-bin and p0 counts
    int* flag;          // [rows]: 1 when bin p0 overflows the candidate space
};

__global__ __launch_bounds__(kSelThreads) void k_sel_hist(SplitArgs a) {
    __shared__ int hist[kBins];
    __shared__ float fsh[2];
    int row, p;
    xcd_unit(blockIdx.x, a.P, gridDim.x / a.P, row, p);
    const int tid = threadIdx.x, wave = tid / kWave;
    for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
    float lo, inv;
    row_range(a.bmin, a.bmax, row, a.blocks_per_row, fsh, &lo, &inv);
    const float* s = a.scores + (int64_t)row * a.C;
    const int seg = a.Ls / kSelWaves;
    const int a0 = p * a.Ls, a1 = min(a.C, a0 + a.Ls);
    const int s0 = min(a1, a0 + wave * seg), s1 = min(a1, s0 + seg);
    for_segment(s, s0, s1, [&](int i0, const float4& v4) {
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i0 + j < s1) atomicAdd(&hist[bin_of(vv[j], lo, inv)], 1);
    });
    __syncthreads();
    int* dst = a.hist + ((int64_t)row * a.P + p) * kBins;
    for (int i = tid; i < kBins; i += kSelThreads) dst[i] = hist[i];
}

__global__ __launch_bounds__(kSelThreads) void k_sel_gather(SplitArgs a) {
    __shared__ int hist[kBins];
    __shared__ int scratch[kSelWaves + 1];
    __shared__ int ish[8];
    __shared__ float fsh[2];
    __shared__ int wa[kSelWaves], wc[kSelWaves];
    int row, p;
    xcd_unit(blockIdx.x, a.P, gridDim.x / a.P, row, p);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    for (int i = tid; i < kBins; i += kSelThreads) {
        // every slice's count in flight at once, then the sum in slice order
        int hv[kMaxSlices];
#pragma unroll
        for (int q2 = 0; q2 < kMaxSlices; ++q2)
            hv[q2] = q2 < a.P ? a.hist[((int64_t)row * a.P + q2) * kBins + i] : 0;
        int h = 0;
#pragma unroll
        for (int q2 = 0; q2 < kMaxSlices; ++q2) h += hv[q2];
        hist[i] = h;
    }
    float lo, inv;
    row_range(a.bmin, a.bmax, row, a.blocks_per_row, fsh, &lo, &inv);   // its barrier covers hist[]
    int above, inside;
    const int p0 = pick_bin(hist, kBins, a.k, scratch, ish, &above, &inside);
    if (inside > kCap) {
        if (p == 0 && tid == 0) a.flag[row] = 1;
        return;
    }
    if (p == 0 && tid == 0) a.flag[row] = 0;
    const float* s = a.scores + (int64_t)row * a.C;
    const int seg = a.Ls / kSelWaves;
    const int a0 = p * a.Ls, a1 = min(a.C, a0 + a.Ls);
    const int s0 = min(a1, a0 + wave * seg), s1 = min(a1, s0 + seg);
    // count pass: per wave, positions of higher bins and of bin p0
    int na = 0, nc = 0;
    for_segment(s, s0, s1, [&](int i0, const float4& v4) {
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i0 + j >= s1) continue;
            const int bn = bin_of(vv[j], lo, inv);
            na += bn > p0;
            nc += bn == p0;
        }
    });
    na = wave_sum(na);
    nc = wave_sum(nc);
    if (lane == 0) {
        wa[wave] = na;
        wc[wave] = nc;
    }
    __syncthreads();
    if (tid == 0) {
        int ra = 0, rc = 0;
        for (int w2 = 0; w2 < kSelWaves; ++w2) {
            const int x = wa[w2], y = wc[w2];
            wa[w2] = ra;
            wc[w2] = rc;
            ra += x;
            rc += y;
        }
        a.cnt[((int64_t)row * a.P + p) * 2] = ra;
        a.cnt[((int64_t)row * a.P + p) * 2 + 1] = rc;
    }
    __syncthreads();
    // write pass: ballot ranks keep each wave's positions in ascending order
    const int64_t lbase = ((int64_t)row * a.P + p);
    int32_t* aid = a.a_id + lbase * a.acap;
    float* aval = a.a_val + lbase * a.acap;
    int32_t* cid = a.c_id + lbase * kCap;
    float* cval = a.c_val + lbase * kCap;
    int runa = wa[wave], runc = wc[wave];
    const uint64_t below = (1ull << lane) - 1ull;
    for_segment(s, s0, s1, [&](int i0, const float4& v4) {
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
        bool fa[4], fc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bn = i0 + j < s1 ? bin_of(vv[j], lo, inv) : -1;
            fa[j] = bn > p0;
            fc[j] = bn == p0;
        }
        const uint64_t a0m = __ballot(fa[0]), a1m = __ballot(fa[1]), a2m = __ballot(fa[2]), a3m = __ballot(fa[3]);
        const uint64_t c0m = __ballot(fc[0]), c1m = __ballot(fc[1]), c2m = __ballot(fc[2]), c3m = __ballot(fc[3]);
        if ((a0m | a1m | a2m | a3m | c0m | c1m | c2m | c3m) == 0ull) return;
        int pa = runa + __popcll(a0m & below) + __popcll(a1m & below) + __popcll(a2m & below) +
                 __popcll(a3m & below);
        int pc = runc + __popcll(c0m & below) + __popcll(c1m & below) + __popcll(c2m & below) +
                 __popcll(c3m & below);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (fa[j]) {
                if (pa < a.acap) {
                    aid[pa] = i0 + j;
                    aval[pa] = vv[j];
                }
                ++pa;
            } else if (fc[j]) {
                if (pc < kCap) {
                    cid[pc] = i0 + j;
                    cval[pc] = vv[j];
                }
                ++pc;
            }
        }
        runa += __popcll(a0m) + __popcll(a1m) + __popcll(a2m) + __popcll(a3m);
        runc += __popcll(c0m) + __popcll(c1m) + __popcll(c2m) + __popcll(c3m);
    });
}

// the number of entries of the ascending list x[0 .. n) below v
__device__ __forceinline__ int count_below(const int* x, int n, int v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (x[mid] < v) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kSelThreads) void k_sel_final(SplitArgs a, int T, int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_score, UnionOut un,
                                                          uint32_t* __restrict__ arrivals) {
    DK_SEL_LDS;
    __shared__ int la[kMaxSlices + 1], lc[kMaxSlices + 1];
    const int row = blockIdx.x;   // one block per row: XCD row % 8, as the row's other blocks
    const int tid = threadIdx.x;
    const int k = a.k;
    if (a.flag[row]) {
        select_row(a.scores, a.bmin, a.bmax, a.blocks_per_row, row, a.C, k, topk_idx, topk_score, L);
    } else {
        // LDS: win flags [kCap] | cval [kCap] | cid [kCap] | kept ids [kCap] | higher-bin ids [kMaxSplitK]
        int* win = L.pool;
        float* cval = reinterpret_cast<float*>(L.pool + kCap);
        int* cid = L.pool + 2 * kCap;
        int* wid = L.pool + 3 * kCap;
        int* ids = L.pool + 4 * kCap;
        // the slices' counts, read in parallel, then their prefix sums
        if (tid < a.P) {
            la[tid + 1] = a.cnt[((int64_t)row * a.P + tid) * 2];
            lc[tid + 1] = a.cnt[((int64_t)row * a.P + tid) * 2 + 1];
        }
        __syncthreads();
        if (tid == 0) {
            la[0] = lc[0] = 0;
            for (int q2 = 1; q2 <= a.P; ++q2) {
                la[q2] += la[q2 - 1];
                lc[q2] += lc[q2 - 1];
            }
        }
        __syncthreads();
        const int A = la[a.P], n = lc[a.P];
        const int need = k - A;   // 1 <= need <= n
        // the lists of all slices concatenated (slice order keeps positions ascending)
        for (int j = tid; j < A; j += kSelThreads) {
            int q2 = 0;
            while (la[q2 + 1] <= j) ++q2;
            ids[j] = a.a_id[((int64_t)row * a.P + q2) * a.acap + (j - la[q2])];
        }
        for (int j = tid; j < n; j += kSelThreads) {
            int q2 = 0;
            while (lc[q2 + 1] <= j) ++q2;
            const int64_t at = ((int64_t)row * a.P + q2) * kCap + (j - lc[q2]);
            cid[j] = a.c_id[at];
            cval[j] = a.c_val[at];
        }
        __syncthreads();
        // exact rank of each candidate in (score descending, position ascending) order
        for (int i = tid; i < n; i += kSelThreads) {
            const float v = cval[i];
            const int id = cid[i];
            int rank = 0;
            for (int j = 0; j < n; ++j) {
                const float u = cval[j];
                rank += (u > v) || (u == v && cid[j] < id);
            }
            win[i] = rank < need;
        }
        __syncthreads();
        // the kept candidates in ascending position order
        for (int i = tid; i < n; i += kSelThreads) {
            if (!win[i]) continue;
            const int id = cid[i];
            int r = 0;
            for (int j = 0; j < n; ++j) r += win[j] && cid[j] < id;
            wid[r] = i;
        }
        __syncthreads();
        int32_t* out = topk_idx + (int64_t)row * k;
        float* outs = topk_score ? topk_score + (int64_t)row * k : nullptr;
        for (int j = tid; j < A; j += kSelThreads) {
            int q2 = 0;
            while (la[q2 + 1] <= j) ++q2;
            const int x = ids[j];
            int lo2 = 0, hi2 = need;   // kept candidates below x
            while (lo2 < hi2) {
                const int mid = (lo2 + hi2) >> 1;
                if (cid[wid[mid]] < x) lo2 = mid + 1;
                else hi2 = mid;
            }
            const int pos = j + lo2;
            store_agent(out + pos, x);
            if (outs) outs[pos] = a.a_val[((int64_t)row * a.P + q2) * a.acap + (j - la[q2])];
        }
        for (int r = tid; r < need; r += kSelThreads) {
            const int i = wid[r];
            const int pos = r + count_below(ids, A, cid[i]);
            store_agent(out + pos, cid[i]);
            if (outs) outs[pos] = cval[i];
        }
    }
    if (un.ids == nullptr) return;
    union_last(row / T, T, k, topk_idx, un, arrivals, L);
}

}  // namespace

IndexPlan plan_index_topk(int B, int Hkv, int T, int C) {
    IndexPlan p{};
    p.rows_per_block = kScoreRows;
    const int64_t rows = (int64_t)B * Hkv * T;
    p.blocks_per_bg = (C + kScoreRows - 1) / kScoreRows;
    int cap = kScoreRows;
    while (cap < kScoreRowsLong && cap < C) cap *= 2;
    p.score_rows = kScoreRows;
    while (p.score_rows < cap &&
           (int64_t)B * Hkv * ((C + 2 * p.score_rows - 1) / (2 * p.score_rows)) >= kScoreMinBlocks)
        p.score_rows *= 2;
    p.score_blocks_per_bg = (C + p.score_rows - 1) / p.score_rows;
    const size_t sbytes = (((size_t)rows * C * 4) + 255) & ~(size_t)255;
    const size_t mbytes = (((size_t)rows * p.blocks_per_bg * 4) + 255) & ~(size_t)255;
    const size_t abytes = (((size_t)B * Hkv * 4) + 255) & ~(size_t)255;
    p.off_min = sbytes;
    p.off_max = sbytes + mbytes;
    p.off_arrive = sbytes + 2 * mbytes;
    size_t off = sbytes + 2 * mbytes + abytes;
    p.slices = 0;
    p.slice_len = 0;
    if (C >= kSplitMinC) {
        int P = C / 16384;
        if (P > kMaxSlices) P = kMaxSlices;
        const int per = (C + P - 1) / P;
        p.slice_len = (per + 4095) & ~4095;
        p.slices = (C + p.slice_len - 1) / p.slice_len;
        auto take = [&](size_t bytes) {
            const size_t at = off;
            off += (bytes + 255) & ~(size_t)255;
            return at;
        };
        const size_t rp = (size_t)rows * p.slices;
        p.off_hist = take(rp * kBins * 4);
        p.off_aid = take(rp * kMaxSplitK * 4);
        p.off_aval = take(rp * kMaxSplitK * 4);
        p.off_cid = take(rp * kCap * 4);
        p.off_cval = take(rp * kCap * 4);
        p.off_cnt = take(rp * 2 * 4);
        p.off_flag = take((size_t)rows * 4);
    }
    p.ws_bytes = off;
    return p;
}

hipError_t launch_index_topk(const float* q, int B, int T, int Hq, const uint16_t* keys, dk_strides ks, int Hkv,
                             int C, int d, int k, float scale, int32_t* topk_idx, float* topk_score, void* ws,
                             const IndexPlan& plan, const UnionOut* un, hipStream_t st) {
    float* scores = (float*)ws;
    float* bmin = (float*)((char*)ws + plan.off_min);
    float* bmax = (float*)((char*)ws + plan.off_max);
    uint32_t* arrivals = un ? (uint32_t*)((char*)ws + plan.off_arrive) : nullptr;
    const int64_t bg = (int64_t)B * Hkv;
    // the scoring kernel's own blocks; its per-block ranges fit the workspace's,
    // which is sized for the shorter blocks
    const dim3 sg((unsigned)(bg * plan.score_blocks_per_bg));
#define DK_IDX_SCORE_R(D_, T_, R_)                                                                           \
    hipLaunchKernelGGL((k_idx_score<D_, T_, R_>), sg, dim3(kScoreThreads), 0, st, q, Hq, keys, ks, Hkv, C, scale, \
                       plan.score_blocks_per_bg, scores, bmin, bmax, arrivals)
#define DK_IDX_SCORE(D_, T_)                                                   \
    do {                                                                       \
        if (plan.score_rows == 8192) DK_IDX_SCORE_R(D_, T_, 8192);             \
        else if (plan.score_rows == 4096) DK_IDX_SCORE_R(D_, T_, 4096);        \
        else if (plan.score_rows == 2048) DK_IDX_SCORE_R(D_, T_, 2048);        \
        else DK_IDX_SCORE_R(D_, T_, 1024);                                     \
    } while (0)
    if (d == 128) {
        if (T == 2) DK_IDX_SCORE(128, 2); else DK_IDX_SCORE(128, 1);
    } else {
        if (T == 2) DK_IDX_SCORE(64, 2); else DK_IDX_SCORE(64, 1);
    }
#undef DK_IDX_SCORE
#undef DK_IDX_SCORE_R
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_select_rows(scores, bmin, bmax, plan.score_blocks_per_bg, B, Hkv, T, C, k, topk_idx, topk_score,
                              un, arrivals, plan, ws, st);
}

hipError_t launch_select_rows(const float* scores, const float* bmin, const float* bmax, int blocks_per_row, int B,
                              int Hkv, int T, int C, int k, int32_t* topk_idx, float* topk_score, const UnionOut* un,
                              uint32_t* arrivals, const IndexPlan& plan, void* ws, hipStream_t st) {
    const UnionOut uo = un ? *un : UnionOut{nullptr, nullptr, nullptr, nullptr};
    const int64_t rows = (int64_t)B * Hkv * T;
    if (plan.slices == 0 || k >= C || k > kMaxSplitK) {
        hipLaunchKernelGGL(k_idx_select, dim3((unsigned)rows), dim3(kSelThreads), 0, st, scores, bmin, bmax,
                           blocks_per_row, T, C, k, topk_idx, topk_score, uo, arrivals);
        return hipGetLastError();
    }
    char* w = (char*)ws;
    SplitArgs a{scores, bmin, bmax, blocks_per_row, C, k, plan.slices, plan.slice_len, kMaxSplitK,
                (int*)(w + plan.off_hist), (int32_t*)(w + plan.off_aid), (float*)(w + plan.off_aval),
                (int32_t*)(w + plan.off_cid), (float*)(w + plan.off_cval), (int*)(w + plan.off_cnt),
                (int*)(w + plan.off_flag)};
    const dim3 grid((unsigned)(rows * plan.slices));
    hipLaunchKernelGGL(k_sel_hist, grid, dim3(kSelThreads), 0, st, a);
    hipLaunchKernelGGL(k_sel_gather, grid, dim3(kSelThreads), 0, st, a);
    hipLaunchKernelGGL(k_sel_final, dim3((unsigned)rows), dim3(kSelThreads), 0, st, a, T, topk_idx, topk_score, uo,
                       arrivals);
    return hipGetLastError();
}

}  // namespace dk
