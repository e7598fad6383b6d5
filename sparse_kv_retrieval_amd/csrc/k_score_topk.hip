// Chunk scores of both queries and each query's k best chunks.
//
// DualDecoder (arXiv 2607.26475), "4.1 KV Retrieval Predictability": the
// retrieval index comes from the current query and the fixed landmarks, and the
// speculative token predicts the next step's index from the same landmarks.
// Blocks are ranked per KV head (OasisKV summary, "Look-ahead Attention").
//
//   s[b, g, t, c] = reduce_{h in group g} scale * <q[b, t, h], lm[b, g, c]>
//
// Kernel 1 (k_score_split) streams one range of a (b, g)'s landmark rows: the
// wave reads whole 128-byte lines of consecutive rows (LPR lanes per row, each
// lane 16-byte pieces spaced 128 bytes apart), keeps the query vectors in
// registers, and leaves order-preserving uint32 score keys in LDS.  A radix
// select over those keys finds each query's k-th key; a block scan then emits
// the winners in ascending chunk order.  With one range per (b, g) this is the
// final answer; otherwise every range writes its k candidates and kernel 2
// (k_topk_merge) repeats the selection over the candidates.  Candidates of
// range s all have lower ids than those of range s + 1, so candidate position
// order equals chunk id order and the tie rule (lower id first) carries over.
//
// With the mean reduction the G query heads are averaged first (mean of dot
// products = dot product with the mean query), so each landmark row costs
// T dot products; the max reduction keeps all G*T vectors.
#include "dk_common.h"

namespace dk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 4096;       // landmark rows per range (LDS: T * 16 KiB)
constexpr int kMaxCand = 8192;       // candidates per (b, g, t) in the merge

// Select the k largest keys of keys[0..n) (k <= n), ties to the lower position,
// and call emit(j, position, key) for j = 0..k-1 in ascending position order.
// Uses `hist` (256 uint), `scratch` (>= 5 int) and `bc` (2 int) of LDS.  Every
// thread of the block must call it.
template <typename Emit>
__device__ void block_topk(const uint32_t* keys, int n, int k, uint32_t* hist, int* scratch,
                           int* bc, Emit emit) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            uint32_t key = keys[i];
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            const int c0 = (int)hist[4 * tid], c1 = (int)hist[4 * tid + 1];
            const int c2 = (int)hist[4 * tid + 2], c3 = (int)hist[4 * tid + 3];
            const int s = c0 + c1 + c2 + c3;
            int v = s;  // inclusive suffix sum over lanes >= tid
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                int t = __shfl_down(v, off, kWave);
                if (tid + off < kWave) v += t;
            }
            int above = v - s;
            const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
            for (int bb = 3; bb >= 0; --bb) {
                if (above < need && need <= above + cs[bb]) {
                    bc[0] = 4 * tid + bb;
                    bc[1] = need - above;
                }
                above += cs[bb];
            }
        }
        __syncthreads();
        prefix |= (uint32_t)bc[0] << shift;
        pmask |= 0xffu << shift;
        need = bc[1];
    }
    const uint32_t thr = prefix;
    // keys > thr are all taken; of the keys == thr, the `need` lowest positions.
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int eq = 0;
    for (int i = lo; i < hi; ++i) eq += keys[i] == thr;
    int tot;
    const int eq_before = block_exclusive_scan(eq, scratch, &tot);
    int sel = 0, er = eq_before;
    for (int i = lo; i < hi; ++i) {
        const uint32_t key = keys[i];
        const bool take = key > thr || (key == thr && er < need);
        er += key == thr;
        sel += take;
    }
    int pos = block_exclusive_scan(sel, scratch, &tot);
    er = eq_before;
    for (int i = lo; i < hi; ++i) {
        const uint32_t key = keys[i];
        const bool take = key > thr || (key == thr && er < need);
        er += key == thr;
        if (take && pos < k) emit(pos++, i, key);
    }
}

// DPL dims per lane, LPR lanes per landmark row, RPW rows per wave pass.
template <int D, int NQ>
struct ScoreShape {
    static constexpr int DPL = NQ <= 2 ? 16 : (NQ <= 8 ? 8 : 4);
    static constexpr int LPR = D / DPL;
    static constexpr int RPW = kWave / LPR;
    static constexpr int NLD = DPL / 4;   // 16-byte loads per lane per row
    static_assert(D % DPL == 0 && LPR <= kWave, "shape");
};

template <int D, int NQ, int T, bool MAXRED, int UNROLL>
__global__ __launch_bounds__(kThreads) void k_score_split(
    const float* __restrict__ q, int Hq, const float* __restrict__ lm, dk_strides ls, int Hkv,
    int C, int k, float scale, int rows_per_split, int splits, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_idx, int32_t* __restrict__ topk_idx, float* __restrict__ topk_score) {
    using S = ScoreShape<D, NQ>;
    constexpr int G = MAXRED ? NQ / T : 0;   // heads per group in max mode
    extern __shared__ uint32_t smem[];
    uint32_t* keys = smem;                          // [T][rows_per_split]
    uint32_t* hist = smem + T * rows_per_split;     // [256]
    int* scratch = (int*)(hist + 256);              // [8]
    int* bc = scratch + 8;                          // [2]

    const int split = blockIdx.x % splits;
    const int bg = blockIdx.x / splits;
    const int b = bg / Hkv, g = bg - b * Hkv;
    const int row0 = split * rows_per_split;
    const int nrows = min(rows_per_split, C - row0);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int rp = lane / S::LPR;          // row inside the wave pass
    const int part = lane % S::LPR;        // this lane's 16-byte pieces: part*16 + 64*LPR*i

    // Query vectors for this lane's dims.
    const int Gq = Hq / Hkv;
    float qv[NQ][S::DPL];
#pragma unroll
    for (int i = 0; i < S::NLD; ++i) {
        const int dim = part * 4 + i * 4 * S::LPR;
#pragma unroll
        for (int v = 0; v < NQ; ++v) {
            if constexpr (MAXRED) {
                const int t = v / G, h = v % G;
                const float4 x = *reinterpret_cast<const float4*>(
                    q + (((int64_t)b * T + t) * Hq + g * Gq + h) * D + dim);
                qv[v][4 * i] = x.x; qv[v][4 * i + 1] = x.y;
                qv[v][4 * i + 2] = x.z; qv[v][4 * i + 3] = x.w;
            } else {
                float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int h = 0; h < Gq; ++h) {
                    const float4 x = *reinterpret_cast<const float4*>(
                        q + (((int64_t)b * T + v) * Hq + g * Gq + h) * D + dim);
                    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
                }
                const float gd = (float)Gq;
                qv[v][4 * i] = acc.x / gd; qv[v][4 * i + 1] = acc.y / gd;
                qv[v][4 * i + 2] = acc.z / gd; qv[v][4 * i + 3] = acc.w / gd;
            }
        }
    }

    const float* base = lm + (int64_t)b * ls.b + (int64_t)g * ls.h + (int64_t)row0 * ls.t + part * 4;
    constexpr int ROWS_PER_ITER = 4 * S::RPW * UNROLL;
    for (int it = 0; it < nrows; it += ROWS_PER_ITER) {
        float4 x[UNROLL][S::NLD];
        int rr[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            rr[u] = it + (u * 4 + wave) * S::RPW + rp;
            const bool ok = rr[u] < nrows;
            const float* p = base + (int64_t)(ok ? rr[u] : 0) * ls.t;
#pragma unroll
            for (int i = 0; i < S::NLD; ++i)
                x[u][i] = ok ? *reinterpret_cast<const float4*>(p + i * 4 * S::LPR)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float dot[NQ];
#pragma unroll
            for (int v = 0; v < NQ; ++v) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < S::NLD; ++i) {
                    a = fmaf(qv[v][4 * i], x[u][i].x, a);
                    a = fmaf(qv[v][4 * i + 1], x[u][i].y, a);
                    a = fmaf(qv[v][4 * i + 2], x[u][i].z, a);
                    a = fmaf(qv[v][4 * i + 3], x[u][i].w, a);
                }
                dot[v] = a;
            }
#pragma unroll
            for (int off = 1; off < S::LPR; off <<= 1)
#pragma unroll
                for (int v = 0; v < NQ; ++v) dot[v] += __shfl_xor(dot[v], off, kWave);
            if (part == 0 && rr[u] < nrows) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    float s;
                    if constexpr (MAXRED) {
                        s = scale * dot[t * G];
#pragma unroll
                        for (int h = 1; h < G; ++h) s = fmaxf(s, scale * dot[t * G + h]);
                    } else {
                        s = scale * dot[t];
                    }
                    keys[t * rows_per_split + rr[u]] = score_key(s);
                }
            }
        }
    }
    __syncthreads();

    const int kk = min(k, nrows);
    for (int t = 0; t < T; ++t) {
        const uint32_t* kt = keys + t * rows_per_split;
        if (splits == 1) {
            int32_t* oi = topk_idx + ((int64_t)bg * T + t) * k;
            float* os = topk_score ? topk_score + ((int64_t)bg * T + t) * k : nullptr;
            block_topk(kt, nrows, kk, hist, scratch, bc, [&](int j, int i, uint32_t key) {
                oi[j] = row0 + i;
                if (os) os[j] = key_score(key);
            });
        } else {
            const int64_t off = (((int64_t)bg * T + t) * splits + split) * k;
            uint32_t* ck = cand_key + off;
            int32_t* ci = cand_idx + off;
            block_topk(kt, nrows, kk, hist, scratch, bc, [&](int j, int i, uint32_t key) {
                ck[j] = key;
                ci[j] = row0 + i;
            });
            for (int j = kk + threadIdx.x; j < k; j += kThreads) {
                ck[j] = 0u;      // below every real key: never selected
                ci[j] = -1;
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void k_topk_merge(const uint32_t* __restrict__ cand_key,
                                                         const int32_t* __restrict__ cand_idx,
                                                         int T, int k, int splits,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_score) {
    extern __shared__ uint32_t smem[];
    const int n = splits * k;
    uint32_t* keys = smem;
    uint32_t* hist = smem + n;
    int* scratch = (int*)(hist + 256);
    int* bc = scratch + 8;
    const int bg = blockIdx.x;
    for (int t = 0; t < T; ++t) {
        const int64_t off = ((int64_t)bg * T + t) * n;
        for (int i = threadIdx.x; i < n; i += kThreads) keys[i] = cand_key[off + i];
        __syncthreads();
        int32_t* oi = topk_idx + ((int64_t)bg * T + t) * k;
        float* os = topk_score ? topk_score + ((int64_t)bg * T + t) * k : nullptr;
        const int32_t* ci = cand_idx + off;
        block_topk(keys, n, k, hist, scratch, bc, [&](int j, int i, uint32_t key) {
            oi[j] = ci[i];
            if (os) os[j] = key_score(key);
        });
        __syncthreads();
    }
}

template <int D, int NQ, int T, bool MAXRED>
hipError_t launch_split(const float* q, int B, int Hq, const float* lm, dk_strides ls, int Hkv,
                        int C, int k, float scale, const TopkPlan& p, uint32_t* ck, int32_t* ci,
                        int32_t* oi, float* os, hipStream_t st) {
    const size_t lds = (size_t)(T * p.rows + 256 + 10) * 4;
    const unsigned grid = (unsigned)((int64_t)B * Hkv * p.splits);
    constexpr int UNROLL = NQ <= 2 ? 4 : 2;
    hipLaunchKernelGGL((k_score_split<D, NQ, T, MAXRED, UNROLL>), dim3(grid), dim3(kThreads), lds,
                       st, q, Hq, lm, ls, Hkv, C, k, scale, p.rows, p.splits, ck, ci, oi, os);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_split(int nq, int T, bool maxred, const float* q, int B, int Hq,
                          const float* lm, dk_strides ls, int Hkv, int C, int k, float scale,
                          const TopkPlan& p, uint32_t* ck, int32_t* ci, int32_t* oi, float* os,
                          hipStream_t st) {
#define DK_SPLIT(NQ_, T_, MX_)                                                                   \
    if (nq == NQ_ && T == T_ && maxred == MX_)                                                   \
        return launch_split<D, NQ_, T_, MX_>(q, B, Hq, lm, ls, Hkv, C, k, scale, p, ck, ci, oi, \
                                             os, st);
    DK_SPLIT(1, 1, false)
    DK_SPLIT(2, 2, false)
    DK_SPLIT(1, 1, true)
    DK_SPLIT(2, 1, true)
    DK_SPLIT(4, 1, true)
    DK_SPLIT(8, 1, true)
    DK_SPLIT(16, 1, true)
    DK_SPLIT(2, 2, true)
    DK_SPLIT(4, 2, true)
    DK_SPLIT(8, 2, true)
    DK_SPLIT(16, 2, true)
#undef DK_SPLIT
    return hipErrorInvalidValue;
}

}  // namespace

TopkPlan plan_topk(int B, int Hkv, int T, int C, int k) {
    (void)T;
    TopkPlan p{0, 0, 0};
    const int64_t bg = (int64_t)B * Hkv;
    int64_t want = (2048 + bg - 1) / bg;
    int64_t by_rows = C / (2 * (int64_t)k);
    if (by_rows < 1) by_rows = 1;
    int64_t s = want < by_rows ? want : by_rows;
    if (s < 1) s = 1;
    const int64_t min_s = (C + kMaxRows - 1) / kMaxRows;
    if (s < min_s) s = min_s;
    if (s > 1 && s * k > kMaxCand) {
        s = kMaxCand / k;
        if (s < min_s) return p;   // unsupported: the merge could not hold the candidates
    }
    if (s < 1) return p;
    p.splits = (int)s;
    p.rows = (int)((C + s - 1) / s);
    // Every range must be non-empty.
    while (p.splits > 1 && (int64_t)(p.splits - 1) * p.rows >= C) {
        p.splits -= 1;
        p.rows = (C + p.splits - 1) / p.splits;
    }
    if (p.rows > kMaxRows) { p.splits = 0; return p; }
    p.ws_bytes = p.splits > 1 ? (size_t)bg * T * p.splits * k * 8 : 0;
    return p;
}

hipError_t launch_score_topk(const float* q, int B, int T, int Hq, const float* lm, dk_strides ls,
                             int Hkv, int C, int d, int k, float scale, dk_group_reduce reduce,
                             int32_t* topk_idx, float* topk_score, void* ws, const TopkPlan& p,
                             hipStream_t st) {
    const bool maxred = reduce == DK_REDUCE_MAX;
    const int G = Hq / Hkv;
    const int nq = maxred ? G * T : T;
    const int64_t ncand = (int64_t)B * Hkv * T * p.splits * k;
    uint32_t* ck = p.splits > 1 ? (uint32_t*)ws : nullptr;
    int32_t* ci = p.splits > 1 ? (int32_t*)((char*)ws + ncand * 4) : nullptr;
    hipError_t e = d == 128
        ? dispatch_split<128>(nq, T, maxred, q, B, Hq, lm, ls, Hkv, C, k, scale, p, ck, ci, topk_idx,
                              topk_score, st)
        : dispatch_split<64>(nq, T, maxred, q, B, Hq, lm, ls, Hkv, C, k, scale, p, ck, ci, topk_idx,
                             topk_score, st);
    if (e != hipSuccess || p.splits == 1) return e;
    const size_t lds = (size_t)(p.splits * k + 256 + 10) * 4;
    hipLaunchKernelGGL(k_topk_merge, dim3((unsigned)((int64_t)B * Hkv)), dim3(kThreads), lds, st,
                       ck, ci, T, k, p.splits, topk_idx, topk_score);
    return hipGetLastError();
}

}  // namespace dk
