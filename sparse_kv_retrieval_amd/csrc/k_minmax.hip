// Min/max chunk summaries and upper-bound chunk scores.
//
// OasisKV summary, "Look-ahead Attention": the draft query ranks every block of
// a KV head from compressed key summaries, two vectors per block (coordinate-
// wise minimum and maximum), at 1/16 of the key bytes for 32-row chunks.  The
// score of chunk c for query head h is the largest dot product any key inside
// the box [kmin, kmax] can reach,
//   U(q, c) = sum_d max(q_d kmin_d, q_d kmax_d) = sum_d (q_d m_d + |q_d| r_d),
// with centre m = (kmin + kmax) / 2 and radius r = (kmax - kmin) / 2, combined
// over the group's heads like chunk scores (mean or max) and scaled.  For the
// mean the heads fold into two vectors per query token, the mean query and the
// mean |query|, so the bound costs two FMAs per dimension.
//
// k_build_minmax writes the summaries (exact: minima and maxima of the keys,
// in the keys' dtype).  k_row_score streams them and writes fp32 score rows
// and block ranges in the format of the exact selection kernel, which then
// returns the k best chunks (ties to the lower id, ascending) and, optionally,
// the union of the T sets.  Without the box (BOX = false) the same kernel
// streams one landmark per chunk and writes the plain chunk scores, the rows the
// coverage selection reads.
#include "dk_common.h"

namespace dk {
namespace {

constexpr int kMmThreads = 256;

template <typename T>
struct MmElems;
template <>
struct MmElems<uint16_t> {
    static constexpr int kPer16B = 8;
    __device__ static void unpack(const uint4& v, float* f) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
    // the values are bf16 already: the upper halves are the exact bits
    __device__ static uint4 pack(const float* f) {
        auto h = [](float x) { return __float_as_uint(x) >> 16; };
        return make_uint4(h(f[0]) | (h(f[1]) << 16), h(f[2]) | (h(f[3]) << 16), h(f[4]) | (h(f[5]) << 16),
                          h(f[6]) | (h(f[7]) << 16));
    }
};
template <>
struct MmElems<float> {
    static constexpr int kPer16B = 4;
    __device__ static void unpack(const uint4& v, float* f) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ static uint4 pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};

// One thread owns 16 bytes of a key row of one chunk and walks the chunk's rows.
template <typename T>
__global__ __launch_bounds__(kMmThreads) void k_build_minmax(const T* __restrict__ K, dk_strides ks, int Hkv, int C,
                                                            int d, int chunk, T* __restrict__ kmin,
                                                            T* __restrict__ kmax, int tpr, int cpb, int64_t total) {
    constexpr int EPT = MmElems<T>::kPer16B;
    const int lc = threadIdx.x / tpr;
    const int part = threadIdx.x - lc * tpr;
    if (lc >= cpb) return;
    const int64_t cid = (int64_t)blockIdx.x * cpb + lc;   // flattened (b, g, c)
    if (cid >= total) return;
    const int64_t bg = cid / C;
    const int c = (int)(cid - bg * C);
    const int b = (int)(bg / Hkv);
    const int g = (int)(bg - (int64_t)b * Hkv);
    const T* src = K + (int64_t)b * ks.b + (int64_t)g * ks.h + (int64_t)c * chunk * ks.t + part * EPT;
    float lo[EPT], hi[EPT];
    MmElems<T>::unpack(ld16(src), lo);
#pragma unroll
    for (int e = 0; e < EPT; ++e) hi[e] = lo[e];
    int n = 1;
    for (; n + 8 <= chunk; n += 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld16(src + (int64_t)(n + u) * ks.t);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float f[EPT];
            MmElems<T>::unpack(v[u], f);
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                lo[e] = fminf(lo[e], f[e]);
                hi[e] = fmaxf(hi[e], f[e]);
            }
        }
    }
    for (; n < chunk; ++n) {
        float f[EPT];
        MmElems<T>::unpack(ld16(src + (int64_t)n * ks.t), f);
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            lo[e] = fminf(lo[e], f[e]);
            hi[e] = fmaxf(hi[e], f[e]);
        }
    }
    st16(kmin + cid * d + part * EPT, MmElems<T>::pack(lo));
    st16(kmax + cid * d + part * EPT, MmElems<T>::pack(hi));
}

// Scores of one block of chunk rows for the T queries of (b, g): D/8 lanes per
// row, 8 dimensions per lane, row sums in DPP.  NQ query vectors: T (mean: the
// heads folded) or G*T (max: one per head).  BOX: upper bounds over [kmin, kmax];
// otherwise plain scores of the landmarks in kmin (kmax unused).
template <typename ET, int D, int NQ, int T, bool MAXRED, bool BOX>
__global__ __launch_bounds__(kMmThreads) void k_row_score(const float* __restrict__ q, int Hq,
                                                            const ET* __restrict__ kmin, const ET* __restrict__ kmax,
                                                            dk_strides ss, int Hkv, int C, float scale,
                                                            int rows_per_block, int blocks_per_bg,
                                                            float* __restrict__ scores, float* __restrict__ bmin,
                                                            float* __restrict__ bmax, uint32_t* __restrict__ arrivals) {
    constexpr int LPR = D / 8, RPW = kWave / LPR, EPT = MmElems<ET>::kPer16B, NV = 8 / EPT;
    constexpr int G = MAXRED ? NQ / T : 1;
    extern __shared__ float sm_mm[];   // [T][rows_per_block], then [BOX ? 2 : 1][NQ][D] query vectors
    const int blk = blockIdx.x % blocks_per_bg;
    const int bg = blockIdx.x / blocks_per_bg;
    const int b = bg / Hkv, g = bg - b * Hkv;
    const int row0 = blk * rows_per_block;
    const int nrows = min(rows_per_block, C - row0);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int rp = lane / LPR, part = lane % LPR;
    const int Gq = Hq / Hkv;
    if (arrivals && blk == 0 && threadIdx.x == 0) arrivals[bg] = 0u;

    // query vectors: per head (max), or the head mean and the mean |q| (mean)
    float* qv = sm_mm + T * rows_per_block;   // [NQ][D] values, then [NQ][D] magnitudes
    for (int i = threadIdx.x; i < NQ * D; i += kMmThreads) {
        const int v = i / D, e = i - v * D;
        if constexpr (MAXRED) {
            const float x = q[(((int64_t)b * T + v / G) * Hq + g * Gq + v % G) * D + e];
            qv[i] = x;
            if constexpr (BOX) qv[NQ * D + i] = fabsf(x);
        } else {
            float s = 0.f, a = 0.f;
            for (int h = 0; h < Gq; ++h) {
                const float x = q[(((int64_t)b * T + v) * Hq + g * Gq + h) * D + e];
                s += x;
                a += fabsf(x);
            }
            qv[i] = s / (float)Gq;
            if constexpr (BOX) qv[NQ * D + i] = a / (float)Gq;
        }
    }
    __syncthreads();
    float qm[NQ][8], qa[NQ][8];
#pragma unroll
    for (int v = 0; v < NQ; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qm[v][e] = qv[v * D + part * 8 + e];
            qa[v][e] = BOX ? qv[NQ * D + v * D + part * 8 + e] : 0.f;
        }

    const ET* lb = kmin + (int64_t)b * ss.b + (int64_t)g * ss.h + (int64_t)row0 * ss.t + part * 8;
    const ET* hb = BOX ? kmax + (int64_t)b * ss.b + (int64_t)g * ss.h + (int64_t)row0 * ss.t + part * 8 : nullptr;
    constexpr int U = 4;
    for (int it = 0; it < nrows; it += 4 * RPW * U) {
        uint4 xl[U][NV], xh[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = it + (u * 4 + wave) * RPW + rp;
#pragma unroll
            for (int x = 0; x < NV; ++x) {
                xl[u][x] = r < nrows ? ld16(lb + (int64_t)r * ss.t + x * EPT) : make_uint4(0, 0, 0, 0);
                if constexpr (BOX)
                    xh[u][x] = r < nrows ? ld16(hb + (int64_t)r * ss.t + x * EPT) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = it + (u * 4 + wave) * RPW + rp;
            float mid[8], rad[8];
#pragma unroll
            for (int x = 0; x < NV; ++x) {
                float fl[EPT], fh[EPT];
                MmElems<ET>::unpack(xl[u][x], fl);
                if constexpr (BOX) {
                    MmElems<ET>::unpack(xh[u][x], fh);
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        mid[x * EPT + e] = 0.5f * (fl[e] + fh[e]);
                        rad[x * EPT + e] = 0.5f * (fh[e] - fl[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPT; ++e) mid[x * EPT + e] = fl[e];
                }
            }
            float sc[T];
#pragma unroll
            for (int t = 0; t < T; ++t) sc[t] = -INFINITY;
#pragma unroll
            for (int v = 0; v < NQ; ++v) {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (BOX) a = fmaf(qa[v][e], rad[e], fmaf(qm[v][e], mid[e], a));
                    else a = fmaf(qm[v][e], mid[e], a);
                }
                const float sv = scale * dpp_group_sum<LPR>(a);
                const int t = MAXRED ? v / G : v;
                sc[t] = MAXRED ? fmaxf(sc[t], sv) : sv;
            }
            if (part < T && r < nrows) sm_mm[part * rows_per_block + r] = part == 0 ? sc[0] : sc[T - 1];
        }
    }
    __syncthreads();
    __shared__ float red[2][T][kMmThreads / kWave];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float* dst = scores + ((int64_t)bg * T + t) * C + row0;
        float lo = INFINITY, hi = -INFINITY;
        for (int i = threadIdx.x; i < nrows; i += kMmThreads) {
            const float v = sm_mm[t * rows_per_block + i];
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
        for (int w2 = 1; w2 < kMmThreads / kWave; ++w2) {
            lo = fminf(lo, red[0][t][w2]);
            hi = fmaxf(hi, red[1][t][w2]);
        }
        bmin[((int64_t)bg * T + t) * blocks_per_bg + blk] = lo;
        bmax[((int64_t)bg * T + t) * blocks_per_bg + blk] = hi;
    }
}

// Rows per block of k_row_score: the plan's scoring-block length, at most 4096
// so that its dynamic LDS (T rows of scores plus the query vectors) stays within
// 64 KiB; the per-block ranges it writes fit the workspace, sized for 1024.
struct RowBlocks {
    int rows, per_bg;
};
inline RowBlocks row_blocks(const IndexPlan& p, int C) {
    const int rows = p.score_rows < 4096 ? p.score_rows : 4096;
    return {rows, (C + rows - 1) / rows};
}

template <typename ET, int D, int NQ, int T, bool MAXRED, bool BOX>
void launch_row_score(dim3 grid, size_t lds, hipStream_t st, const float* q, int Hq, const void* kmin,
                      const void* kmax, dk_strides ss, int Hkv, int C, float scale, const IndexPlan& p,
                      float* scores, float* bmin, float* bmax, uint32_t* arrivals) {
    hipLaunchKernelGGL((k_row_score<ET, D, NQ, T, MAXRED, BOX>), grid, dim3(kMmThreads), lds, st, q, Hq,
                       (const ET*)kmin, (const ET*)kmax, ss, Hkv, C, scale, row_blocks(p, C).rows, row_blocks(p, C).per_bg,
                       scores, bmin, bmax, arrivals);
}

template <typename ET, int D, bool BOX>
hipError_t dispatch_rows(int nq, int T, bool maxred, dim3 grid, size_t lds, hipStream_t st, const float* q, int Hq,
                       const void* kmin, const void* kmax, dk_strides ss, int Hkv, int C, float scale,
                       const IndexPlan& p, float* scores, float* bmin, float* bmax, uint32_t* arrivals) {
#define DK_MM(NQ_, T_, MX_) \
    launch_row_score<ET, D, NQ_, T_, MX_, BOX>(grid, lds, st, q, Hq, kmin, kmax, ss, Hkv, C, scale, p, scores, bmin, bmax, arrivals)
    if (!maxred) {
        if (T == 2) DK_MM(2, 2, false); else DK_MM(1, 1, false);
    } else if (T == 2) {
        if (nq == 2) DK_MM(2, 2, true); else if (nq == 4) DK_MM(4, 2, true); else DK_MM(8, 2, true);
    } else {
        if (nq == 1) DK_MM(1, 1, true); else if (nq == 2) DK_MM(2, 1, true); else if (nq == 4) DK_MM(4, 1, true);
        else DK_MM(8, 1, true);
    }
#undef DK_MM
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build_minmax(const void* K, dk_dtype dt, dk_strides ks, int B, int Hkv, int L, int d, int chunk,
                               void* kmin, void* kmax, hipStream_t st) {
    const int C = L / chunk;
    const int esz = dt == DK_BF16 ? 2 : 4;
    const int tpr = d * esz / 16;
    const int cpb = kMmThreads / tpr;
    const int64_t total = (int64_t)B * Hkv * C;
    const dim3 grid((unsigned)((total + cpb - 1) / cpb));
    if (dt == DK_BF16)
        hipLaunchKernelGGL(k_build_minmax<uint16_t>, grid, dim3(kMmThreads), 0, st, (const uint16_t*)K, ks, Hkv, C,
                           d, chunk, (uint16_t*)kmin, (uint16_t*)kmax, tpr, cpb, total);
    else
        hipLaunchKernelGGL(k_build_minmax<float>, grid, dim3(kMmThreads), 0, st, (const float*)K, ks, Hkv, C, d,
                           chunk, (float*)kmin, (float*)kmax, tpr, cpb, total);
    return hipGetLastError();
}

hipError_t launch_score_rows(const float* q, int B, int T, int Hq, const void* a, const void* b, dk_dtype dt,
                             dk_strides ss, int Hkv, int C, int d, float scale, dk_group_reduce reduce, void* ws,
                             const IndexPlan& plan, uint32_t* arrivals, hipStream_t st) {
    float* scores = (float*)ws;
    float* bmin = (float*)((char*)ws + plan.off_min);
    float* bmax = (float*)((char*)ws + plan.off_max);
    const int G = Hq / Hkv;
    const bool maxred = reduce == DK_REDUCE_MAX;
    const int nq = maxred ? G * T : T;
    const RowBlocks rb = row_blocks(plan, C);
    const dim3 grid((unsigned)((int64_t)B * Hkv * rb.per_bg));
    const size_t lds = ((size_t)T * rb.rows + (b ? 2 : 1) * (size_t)nq * d) * 4;
#define DK_ROWS(ET_, D_, BOX_)                                                                                  \
    return dispatch_rows<ET_, D_, BOX_>(nq, T, maxred, grid, lds, st, q, Hq, a, b, ss, Hkv, C, scale, plan,    \
                                        scores, bmin, bmax, arrivals)
    if (dt == DK_BF16) {
        if (d == 128) { if (b) DK_ROWS(uint16_t, 128, true); else DK_ROWS(uint16_t, 128, false); }
        else { if (b) DK_ROWS(uint16_t, 64, true); else DK_ROWS(uint16_t, 64, false); }
    } else {
        if (d == 128) { if (b) DK_ROWS(float, 128, true); else DK_ROWS(float, 128, false); }
        else { if (b) DK_ROWS(float, 64, true); else DK_ROWS(float, 64, false); }
    }
#undef DK_ROWS
}

hipError_t launch_minmax_topk(const float* q, int B, int T, int Hq, const void* kmin, const void* kmax, dk_dtype dt,
                              dk_strides ss, int Hkv, int C, int d, int k, float scale, dk_group_reduce reduce,
                              int32_t* topk_idx, float* topk_score, void* ws, const IndexPlan& plan,
                              const UnionOut* un, hipStream_t st) {
    uint32_t* arrivals = un ? (uint32_t*)((char*)ws + plan.off_arrive) : nullptr;
    hipError_t e = launch_score_rows(q, B, T, Hq, kmin, kmax, dt, ss, Hkv, C, d, scale, reduce, ws, plan, arrivals,
                                     st);
    if (e != hipSuccess) return e;
    return launch_select_rows((const float*)ws, (const float*)((char*)ws + plan.off_min),
                              (const float*)((char*)ws + plan.off_max), row_blocks(plan, C).per_bg, B, Hkv, T, C, k, topk_idx,
                              topk_score, un, arrivals, plan, ws, st);
}

}  // namespace dk
