// Coverage budgets over chunk score rows.
//
// MOIRA (abstract): per request, KV head and step the selection keeps the
// smallest set of chunks whose estimated attention mass reaches a fraction gamma
// of the total.  The estimate is the softmax of the row's chunk scores; the kept
// set is the shortest prefix of the chunks in (score descending, id ascending)
// order whose mass reaches gamma, at least one chunk and at most k_max.  It is
// written as ascending ids with its size, and optionally merged with the other
// query's set into the union of the two ragged sets.
//
// One block of 1024 threads owns the T rows of one (b, g) and keeps every score
// of a row in registers (EPT per thread; chunk id = thread + 1024 e).  The
// masses are w = exp(s - max s), their total Z.  A 32-step bisection on the
// order-preserving key of the scores finds the largest key v whose mass
// E(v) = sum of w over the chunks with key >= v still reaches gamma * Z.  Every
// E is summed by one fixed tree (each thread's EPT terms in order, a wave
// butterfly, then the 16 wave sums in order): the sums are deterministic and,
// rounding being monotone, never increase with v, so the bisection is exact for
// them.  The chunks above v are kept; of those tied at v (one score, one mass)
// the lowest ids are kept until the mass reaches gamma * Z.  A set larger than
// k_max is replaced by the top k_max, found by a second bisection on counts.
// Tie ranks and output positions come from ballots and one wave's scan of the
// per-wave counts.
//
// Rows of up to 4096 chunks take the wave form instead: one wave per row with
// its 64 * EPL scores and masses in registers (chunk id = lane + 64 e), every
// sum a wave reduction (DPP row sums, then four lanes in order), so the
// bisections need no barrier; the T waves of a (b, g) exchange their 64-bit
// selection masks through LDS once for the union.
#include "dk_block.h"

namespace dk {
namespace {

using namespace blk;
constexpr int kCovThreads = kBlkThreads;
constexpr int kCovWaves = kBlkWaves;

template <int EPT, int T>
__global__ __launch_bounds__(kCovThreads) void k_cov_select(const float* __restrict__ scores, int C, float gamma,
                                                           int k_max, int32_t* __restrict__ sel_idx,
                                                           int32_t* __restrict__ sel_count,
                                                           float* __restrict__ sel_score, UnionOut un) {
    __shared__ float s_f[2][T][kCovWaves];
    __shared__ int s_i[2][2 * T][kCovWaves];
    __shared__ int s_cnt[T * EPT * kCovWaves];
    __shared__ int s_tot[T];
    const int64_t bg = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;

    uint32_t key[T][EPT];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float* row = scores + (bg * T + t) * C;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int j = tid + e * kCovThreads;
            key[t][e] = j < C ? score_key(row[j]) : 0u;   // a real (non-NaN) score's key is > 0
        }
    }
    // row maxima (s_i[0]); the reductions below start on buffer 1
    float smax[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        uint32_t m = 0u;
#pragma unroll
        for (int e = 0; e < EPT; ++e) m = max(m, key[t][e]);
        m = wave_max_u(m);
        if (lane == 0) s_i[0][t][wave] = (int)m;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; ++t) {
        uint32_t m = 0u;
#pragma unroll
        for (int w2 = 0; w2 < kCovWaves; ++w2) m = max(m, (uint32_t)s_i[0][t][w2]);
        smax[t] = key_score(m);
    }
    // masses; a tied chunk's mass is recomputed from the key with this expression
    float w[T][EPT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int e = 0; e < EPT; ++e) w[t][e] = key[t][e] ? expf(key_score(key[t][e]) - smax[t]) : 0.f;
    int par = 1;
    float target[T];
    {
        float z[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            z[t] = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e) z[t] += w[t][e];
        }
        block_sums_f<T>(z, s_f[par]);
        par ^= 1;
#pragma unroll
        for (int t = 0; t < T; ++t) target[t] = gamma * z[t];
    }

    uint32_t v[T];     // threshold key
    int n[T];          // chunks kept
    int rtie[T];       // chunks kept among those tied at v (lowest ids)
    bool over[T];
    const bool all = gamma >= 1.0f;   // every chunk, so the top k_max
#pragma unroll
    for (int t = 0; t < T; ++t) { v[t] = 0u; n[t] = 0; rtie[t] = 0; over[t] = all; }
    if (!all) {
        // the largest key v with E(v) >= gamma * Z
        for (int bit = 31; bit >= 0; --bit) {
            float part[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t cand = v[t] | (1u << bit);
                part[t] = 0.f;
#pragma unroll
                for (int e = 0; e < EPT; ++e) part[t] += key[t][e] >= cand ? w[t][e] : 0.f;
            }
            block_sums_f<T>(part, s_f[par]);
            par ^= 1;
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (part[t] >= target[t]) v[t] |= 1u << bit;
        }
        // mass above v (= E(v + 1) by the same tree, so below the target), counts above and at v
        float above[T];
        int cnt[2 * T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            above[t] = 0.f;
            cnt[2 * t] = cnt[2 * t + 1] = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                above[t] += key[t][e] > v[t] ? w[t][e] : 0.f;
                cnt[2 * t] += key[t][e] > v[t] ? 1 : 0;
                cnt[2 * t + 1] += key[t][e] == v[t] ? 1 : 0;
            }
        }
        block_sums_f<T>(above, s_f[par]);
        block_sums_i<2 * T>(cnt, s_i[par]);
        par ^= 1;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float wt = expf(key_score(v[t]) - smax[t]);
            const float need = (target[t] - above[t]) / wt;   // > 0
            int r = cnt[2 * t + 1];
            if (wt > 0.f && need < (float)r) r = max(1, (int)ceilf(need));
            rtie[t] = r;
            n[t] = cnt[2 * t] + r;
            over[t] = n[t] > k_max;
        }
    }
    bool any_over = false;
#pragma unroll
    for (int t = 0; t < T; ++t) any_over |= over[t];
    if (any_over) {
        // the largest key vc with at least k_max chunks at or above it
        uint32_t vc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) vc[t] = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            int part[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t cand = vc[t] | (1u << bit);
                part[t] = 0;
#pragma unroll
                for (int e = 0; e < EPT; ++e) part[t] += key[t][e] >= cand ? 1 : 0;
            }
            block_sums_i<T>(part, s_i[par]);
            par ^= 1;
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (part[t] >= k_max) vc[t] |= 1u << bit;
        }
        int gt[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            gt[t] = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) gt[t] += key[t][e] > vc[t] ? 1 : 0;
        }
        block_sums_i<T>(gt, s_i[par]);
        par ^= 1;
#pragma unroll
        for (int t = 0; t < T; ++t)
            if (over[t]) {
                v[t] = vc[t];
                rtie[t] = k_max - gt[t];
                n[t] = k_max;
            }
    }

    // kept: above v, or tied at v with one of the rtie lowest ids
    bool flag[T][EPT];
    int rank[T][EPT], tot[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int e = 0; e < EPT; ++e) flag[t][e] = key[t][e] == v[t];
    block_ranks<T, EPT>(flag, rank, tot, s_cnt, s_tot);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int e = 0; e < EPT; ++e) flag[t][e] = key[t][e] > v[t] || (flag[t][e] && rank[t][e] < rtie[t]);
    block_ranks<T, EPT>(flag, rank, tot, s_cnt, s_tot);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        int32_t* oi = sel_idx + (bg * T + t) * k_max;
        float* os = sel_score ? sel_score + (bg * T + t) * k_max : nullptr;
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if (flag[t][e] && rank[t][e] < k_max) {   // at most k_max flags: the guard never fires
                oi[rank[t][e]] = tid + e * kCovThreads;
                if (os) os[rank[t][e]] = key_score(key[t][e]);
            }
        for (int i = n[t] + tid; i < k_max; i += kCovThreads) {
            oi[i] = -1;
            if (os) os[i] = -INFINITY;
        }
        if (tid == 0) sel_count[bg * T + t] = n[t];
    }

    if (un.ids) {
        const int slots = T * k_max;
        bool uf[1][EPT];
        int upos[1][EPT], utot[1];
#pragma unroll
        for (int e = 0; e < EPT; ++e) uf[0][e] = flag[0][e] || flag[T - 1][e];
        block_ranks<1, EPT>(uf, upos, utot, s_cnt, s_tot);
        int32_t* ui = un.ids + bg * slots;
        uint8_t* um = un.member + bg * slots;
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if (uf[0][e] && upos[0][e] < slots) {
                ui[upos[0][e]] = tid + e * kCovThreads;
                um[upos[0][e]] = (uint8_t)((flag[0][e] ? 1 : 0) | (T == 2 && flag[T - 1][e] ? 2 : 0));
            }
        for (int i = utot[0] + tid; i < slots; i += kCovThreads) {
            ui[i] = -1;
            um[i] = 0;
        }
        if (tid == 0) {
            un.count[bg] = utot[0];
            if (un.overlap) un.overlap[bg] = T == 2 ? n[0] + n[1] - utot[0] : n[0];
        }
    }
}

template <int EPL, int T>
__global__ __launch_bounds__(kWave * T) void k_cov_wave(const float* __restrict__ scores, int C, float gamma,
                                                       int k_max, int32_t* __restrict__ sel_idx,
                                                       int32_t* __restrict__ sel_count, float* __restrict__ sel_score,
                                                       UnionOut un) {
    __shared__ uint64_t s_mask[T][EPL];
    __shared__ int s_n[T];
    const int64_t bg = blockIdx.x;
    const int t = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const uint64_t below = wv::lanes_below();
    const float* row = scores + (bg * T + t) * C;
    uint32_t key[EPL];
    float w[EPL];
    uint32_t m = 0u;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int j = lane + e * kWave;
        key[e] = j < C ? score_key(row[j]) : 0u;   // a real (non-NaN) score's key is > 0
        m = max(m, key[e]);
    }
    const float smax = key_score(wv::max_u(m));
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        w[e] = key[e] ? expf(key_score(key[e]) - smax) : 0.f;   // tied chunks: recomputed below alike
        z += w[e];
    }
    const float target = gamma * wv::sum_f(z);

    uint32_t v = 0u;   // threshold key
    int n = 0, rtie = 0;
    bool over = gamma >= 1.0f;   // every chunk, so the top k_max
    if (!over) {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = v | (1u << bit);
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) part += key[e] >= cand ? w[e] : 0.f;
            if (wv::sum_f(part) >= target) v = cand;
        }
        float above = 0.f;
        int gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            above += key[e] > v ? w[e] : 0.f;
            gt += key[e] > v ? 1 : 0;
            eq += key[e] == v ? 1 : 0;
        }
        above = wv::sum_f(above);
        gt = wv::sum_i(gt);
        eq = wv::sum_i(eq);
        const float wt = expf(key_score(v) - smax);
        const float need = (target - above) / wt;   // > 0: the mass above v is below the target
        int r = eq;
        if (wt > 0.f && need < (float)r) r = max(1, (int)ceilf(need));
        rtie = r;
        n = gt + r;
        over = n > k_max;
    }
    if (over) {
        uint32_t vc = 0u;   // the largest key with at least k_max chunks at or above it
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = vc | (1u << bit);
            int part = 0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) part += key[e] >= cand ? 1 : 0;
            if (wv::sum_i(part) >= k_max) vc = cand;
        }
        int gt = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) gt += key[e] > vc ? 1 : 0;
        v = vc;
        rtie = k_max - wv::sum_i(gt);
        n = k_max;
    }

    // kept: above v, or tied at v with one of the rtie lowest ids; written in id order
    int32_t* oi = sel_idx + (bg * T + t) * k_max;
    float* os = sel_score ? sel_score + (bg * T + t) * k_max : nullptr;
    int tpre = 0, spre = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const bool tie = key[e] == v;
        const uint64_t tb = __ballot(tie);
        const bool sel = key[e] > v || (tie && tpre + __popcll(tb & below) < rtie);
        tpre += __popcll(tb);
        const uint64_t sb = __ballot(sel);
        const int pos = spre + __popcll(sb & below);
        spre += __popcll(sb);
        if (sel && pos < k_max) {   // at most k_max are kept: the guard never fires
            oi[pos] = lane + e * kWave;
            if (os) os[pos] = key_score(key[e]);
        }
        if (lane == 0) s_mask[t][e] = sb;
    }
    for (int i = n + lane; i < k_max; i += kWave) {
        oi[i] = -1;
        if (os) os[i] = -INFINITY;
    }
    if (lane == 0) {
        sel_count[bg * T + t] = n;
        s_n[t] = n;
    }
    if (!un.ids) return;
    __syncthreads();
    if (t != 0) return;
    // lane e merges mask word e: chunks 64 e + bit, in ascending order
    const int slots = T * k_max;
    uint64_t m0 = 0ull, m1 = 0ull;
    if (lane < EPL) {
        m0 = s_mask[0][lane];
        m1 = s_mask[T - 1][lane];
    }
    uint64_t um = m0 | m1;
    const int c = __popcll(um);
    const int inc = wave_inclusive_scan(c);
    int pos = inc - c;
    const int total = __builtin_amdgcn_readlane(inc, kWave - 1);
    int32_t* ui = un.ids + bg * slots;
    uint8_t* mb = un.member + bg * slots;
    while (um) {
        const int bit = __builtin_ctzll(um);
        um &= um - 1ull;
        if (pos < slots) {
            ui[pos] = lane * kWave + bit;
            mb[pos] = (uint8_t)(((m0 >> bit) & 1ull) | (T == 2 ? ((m1 >> bit) & 1ull) << 1 : 0ull));
        }
        ++pos;
    }
    for (int i = total + lane; i < slots; i += kWave) {
        ui[i] = -1;
        mb[i] = 0;
    }
    if (lane == 0) {
        un.count[bg] = total;
        if (un.overlap) un.overlap[bg] = T == 2 ? s_n[0] + s_n[1] - total : s_n[0];
    }
}

template <int EPL>
hipError_t launch_cov_wave(int T, unsigned grid, hipStream_t st, const float* scores, int C, float gamma, int k_max,
                           int32_t* sel_idx, int32_t* sel_count, float* sel_score, const UnionOut& un) {
    if (T == 2)
        hipLaunchKernelGGL((k_cov_wave<EPL, 2>), dim3(grid), dim3(2 * kWave), 0, st, scores, C, gamma, k_max, sel_idx,
                           sel_count, sel_score, un);
    else
        hipLaunchKernelGGL((k_cov_wave<EPL, 1>), dim3(grid), dim3(kWave), 0, st, scores, C, gamma, k_max, sel_idx,
                           sel_count, sel_score, un);
    return hipGetLastError();
}

template <int EPT>
hipError_t launch_cov(int T, unsigned grid, hipStream_t st, const float* scores, int C, float gamma, int k_max,
                      int32_t* sel_idx, int32_t* sel_count, float* sel_score, const UnionOut& un) {
    if (T == 2)
        hipLaunchKernelGGL((k_cov_select<EPT, 2>), dim3(grid), dim3(kCovThreads), 0, st, scores, C, gamma, k_max,
                           sel_idx, sel_count, sel_score, un);
    else
        hipLaunchKernelGGL((k_cov_select<EPT, 1>), dim3(grid), dim3(kCovThreads), 0, st, scores, C, gamma, k_max,
                           sel_idx, sel_count, sel_score, un);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_coverage(const float* q, int B, int T, int Hq, const void* lm, dk_dtype dt, dk_strides ls, int Hkv,
                           int C, int d, float scale, dk_group_reduce reduce, float gamma, int k_max,
                           int32_t* sel_idx, int32_t* sel_count, float* sel_score, const UnionOut* un, void* ws,
                           const IndexPlan& plan, hipStream_t st) {
    hipError_t e = launch_score_rows(q, B, T, Hq, lm, nullptr, dt, ls, Hkv, C, d, scale, reduce, ws, plan, nullptr,
                                     st);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((int64_t)B * Hkv);
    const UnionOut none{nullptr, nullptr, nullptr, nullptr};
    const UnionOut& u = un ? *un : none;
    const float* scores = (const float*)ws;
    if (C <= 4 * kWave) return launch_cov_wave<4>(T, grid, st, scores, C, gamma, k_max, sel_idx, sel_count, sel_score, u);
    if (C <= 16 * kWave) return launch_cov_wave<16>(T, grid, st, scores, C, gamma, k_max, sel_idx, sel_count, sel_score, u);
    if (C <= 64 * kWave) return launch_cov_wave<64>(T, grid, st, scores, C, gamma, k_max, sel_idx, sel_count, sel_score, u);
    if (C <= 8 * kCovThreads) return launch_cov<8>(T, grid, st, scores, C, gamma, k_max, sel_idx, sel_count, sel_score, u);
    if (C <= kCoverageMaxC) return launch_cov<16>(T, grid, st, scores, C, gamma, k_max, sel_idx, sel_count, sel_score, u);
    return hipErrorInvalidValue;
}

}  // namespace dk
