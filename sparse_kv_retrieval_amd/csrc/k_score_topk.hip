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
#include <type_traits>

#include "dk_attn_fast.h"
#include "dk_common.h"
#include "dk_union_core.h"

namespace dk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 4096;       // landmark rows per range (LDS: T * 16 KiB)
constexpr int kMaxCand = 8192;       // candidates per (b, g, t) in the merge
constexpr int kShadowMaxC = 6144;    // chunks per (b, g) with a shadow (pass-2 LDS <= 64 KiB)

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// streamed once: non-temporal 16-byte loads
__device__ __forceinline__ float4 nt_load_f4(const float* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t f16_bits(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
// a.lo*b.lo + a.hi*b.hi + c in fp32 (v_dot2_f32_f16; fp16 products are exact in fp32)
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                  false);
}

// Exclusive prefix sum within a group of kThreads threads (group g holds
// threads g * kThreads .. + kThreads - 1 of the block; a kThreads block is one
// group).  scratch: 4 ints of the group's own LDS.  Every thread of the block
// must call it: it holds two block barriers.
__device__ __forceinline__ int group_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & (kWave - 1), gw = (threadIdx.x / kWave) & 3;
    const int inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[gw] = inc;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int c = scratch[w];
        pre += w < gw ? c : 0;
        tot += c;
    }
    *total = tot;
    __syncthreads();   // scratch is rewritten by the next call
    return pre + inc - v;
}

// The k-th largest of keys[0..n) (1 <= k <= n) by an 8-bit radix select; also
// returns how many of the keys equal to it belong to the k largest (*need).
// Uses `hist` (256 uint) and `bc` (2 int) of LDS.  Works within a group of
// kThreads threads (its keys and LDS its own); every thread of the block must
// call it, the same number of times.
__device__ uint32_t block_kth_key(const uint32_t* keys, int n, int k, uint32_t* hist, int* bc,
                                  int* need_out) {
    const int tid = threadIdx.x & (kThreads - 1);
    uint32_t prefix = 0, pmask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
        __syncthreads();
        if (shift == 24) {
            // The top byte (sign and high exponent bits) takes few distinct values
            // within a wave: add one count per distinct digit instead of one LDS
            // atomic per key on the same few bins.
            const int lane = tid & (kWave - 1);
            for (int i0 = 0; i0 < n; i0 += kThreads) {
                const int i = i0 + tid;
                bool active = i < n;
                const uint32_t digit = active ? keys[i] >> 24 : 0u;
                uint64_t act = __builtin_amdgcn_ballot_w64(active);
                while (act) {
                    const int leader = (int)__builtin_ctzll(act);
                    const uint32_t ld = (uint32_t)__builtin_amdgcn_readlane((int)digit, leader);
                    const uint64_t same = __builtin_amdgcn_ballot_w64(active && digit == ld);
                    if (lane == leader) atomicAdd(&hist[ld], (uint32_t)__builtin_popcountll(same));
                    act &= ~same;
                    active = active && digit != ld;
                }
            }
        } else {
            for (int i = tid; i < n; i += kThreads) {
                uint32_t key = keys[i];
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
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
    *need_out = need;
    return prefix;
}

// ---------------------------------------------------------------------------
// Wave-level selection over at most 256 keys held 4 per lane (value v of lane l
// is position l + 64 v).  No block barriers: one wave owns the work and a
// 256-bin histogram in LDS.
// ---------------------------------------------------------------------------
// inclusive prefix sum over the wave (DPP row shifts, then row broadcasts)
__device__ __forceinline__ int wave_prefix_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// The k-th largest of up to 256 keys held 4 per lane (1 <= k <= number of keys;
// unused slots hold 0, below every real key) by a bitwise search over the key
// space with wave-wide ballot counts; also how many keys equal to it are among
// the k largest.  No LDS, no barriers.
// With LOW_BIT > 0 only the key bits above it are settled: r is then the
// largest key with those low bits zero that still has k keys at or above it, a
// lower bound of the k-th largest (need_out is then not meaningful).
template <int LOW_BIT = 0>
__device__ uint32_t wave_kth_key_bisect(const uint32_t (&x)[4], int k, int* need_out) {
    uint32_t r = 0;
    for (int bit = 31; bit >= LOW_BIT; --bit) {
        const uint32_t c = r | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(x[v] >= c));
        if (cnt >= k) r = c;
    }
    int greater = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) greater += __builtin_popcountll(__builtin_amdgcn_ballot_w64(x[v] > r));
    *need_out = k - greater;
    return r;
}

// The k-th largest of the keys (1 <= k <= number of non-zero keys; empty slots
// hold 0) and how many keys equal to it belong to the k largest.
__device__ uint32_t wave_kth_key(const uint32_t (&x)[4], int k, uint32_t* hist, int* need_out) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t prefix = 0, pmask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if ((x[v] & pmask) == prefix) atomicAdd(&hist[(x[v] >> shift) & 255u], 1u);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane l owns digits 255 - 4l - j, j = 0..3 (descending), so the count of
        // keys above its digits is the exclusive prefix over lanes below it
        const uint4 h4 = reinterpret_cast<const uint4*>(hist)[63 - lane];
        const int c[4] = {(int)h4.w, (int)h4.z, (int)h4.y, (int)h4.x};
        const int tot = c[0] + c[1] + c[2] + c[3];
        int above = wave_prefix_sum(tot) - tot;
        int digit = -1, nneed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (above < need && need <= above + c[j]) {
                digit = 255 - 4 * lane - j;
                nneed = need - above;
            }
            above += c[j];
        }
        const uint64_t found = __builtin_amdgcn_ballot_w64(digit >= 0);
        const int src = (int)__builtin_ctzll(found);
        digit = __builtin_amdgcn_readlane(digit, src);
        need = __builtin_amdgcn_readlane(nneed, src);
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xffu << shift;
        __builtin_amdgcn_wave_barrier();
    }
    *need_out = need;
    return prefix;
}

// Select the k largest keys of keys[0..n) (k <= n), ties to the lower position,
// and call emit(j, position, key) for j = 0..k-1 in ascending position order.
// Uses `hist` (256 uint), `scratch` (>= 4 int) and `bc` (2 int) of LDS.  Works
// within a group of kThreads threads, like block_kth_key; every thread of the
// block must call it.
template <typename Emit>
__device__ void block_topk(const uint32_t* keys, int n, int k, uint32_t* hist, int* scratch,
                           int* bc, Emit emit) {
    const int tid = threadIdx.x & (kThreads - 1);
    int need;
    const uint32_t thr = block_kth_key(keys, n, k, hist, bc, &need);
    // keys > thr are all taken; of the keys == thr, the `need` lowest positions.
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int eq = 0;
    for (int i = lo; i < hi; ++i) eq += keys[i] == thr;
    int tot;
    const int eq_before = group_exclusive_scan(eq, scratch, &tot);
    int sel = 0, er = eq_before;
    for (int i = lo; i < hi; ++i) {
        const uint32_t key = keys[i];
        const bool take = key > thr || (key == thr && er < need);
        er += key == thr;
        sel += take;
    }
    int pos = group_exclusive_scan(sel, scratch, &tot);
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
                x[u][i] = ok ? nt_load_f4(p + i * 4 * S::LPR) : make_float4(0.f, 0.f, 0.f, 0.f);
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

// ---------------------------------------------------------------------------
// Landmark shadow: 8-bit codes with one scale per chunk.  For row c,
//   s_c = max_i |lm[c, i]| / 127,  m_i = rint(lm[c, i] / s_c)  (|m_i| <= 127),
// stored as the byte m_i + 128, so |lm[c, i] - s_c m_i| <= s_c (1/2 + 127 u).
// scale_max[b, g] = max_c s_c, or +inf when a landmark of (b, g) is not finite
// (the selection then re-scores every chunk of that (b, g) exactly).  One
// block per (b, g); TPR threads per row, four dimensions each.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void k_build_shadow(const float* __restrict__ lm, dk_strides ls,
                                                          int Hkv, int C, uint8_t* __restrict__ lm8,
                                                          float* __restrict__ chunk_scale,
                                                          float* __restrict__ scale_max) {
    constexpr int TPR = D / 4;                 // threads per row, one float4 each
    constexpr int RPB = kThreads / TPR;        // rows per block pass
    __shared__ float smax[kThreads / kWave];
    __shared__ int sbad;
    const int bg = blockIdx.x;
    const int b = bg / Hkv, g = bg - b * Hkv;
    const int tr = threadIdx.x / TPR, part = threadIdx.x % TPR;
    if (threadIdx.x == 0) sbad = 0;
    __syncthreads();
    float vmax = 0.f;
    bool bad = false;
    const float* base = lm + (int64_t)b * ls.b + (int64_t)g * ls.h + part * 4;
    uint8_t* obase = lm8 + (int64_t)bg * C * D + part * 4;
    for (int r0 = 0; r0 < C; r0 += RPB) {
        const int r = r0 + tr;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < C) x = *reinterpret_cast<const float4*>(base + (int64_t)r * ls.t);
        // largest magnitude of the row: its TPR threads are an aligned lane group
        // inf or NaN anywhere (fmaxf would drop a NaN)
        bad |= !(fabsf(x.x) <= 3.0e38f && fabsf(x.y) <= 3.0e38f && fabsf(x.z) <= 3.0e38f &&
                 fabsf(x.w) <= 3.0e38f);
        float a = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
        for (int off = 1; off < TPR; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, kWave));
        if (r < C) {
            const float sc = __fdiv_rn(a, 127.0f);
            auto code = [sc](float v) -> uint32_t {
                const float m = sc > 0.f ? rintf(__fdiv_rn(v, sc)) : 0.f;
                return (uint32_t)((int)fminf(fmaxf(m, -127.f), 127.f) + 128);
            };
            *reinterpret_cast<uint32_t*>(obase + (int64_t)r * D) =
                code(x.x) | (code(x.y) << 8) | (code(x.z) << 16) | (code(x.w) << 24);
            if (part == 0) chunk_scale[(int64_t)bg * C + r] = sc;
            vmax = fmaxf(vmax, sc);
        }
    }
    if (bad) sbad = 1;
    for (int off = 1; off < kWave; off <<= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) smax[threadIdx.x / kWave] = vmax;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = 0.f;
        for (int w = 0; w < kThreads / kWave; ++w) m = fmaxf(m, smax[w]);
        scale_max[bg] = sbad ? INFINITY : m;
    }
}

// ---------------------------------------------------------------------------
// Shadow scoring and exact selection in one kernel: one block per (b, g) with
// T groups of kThreads threads; the scores never leave LDS.
//
// Pass 1 (every wave): the shadow score of every chunk from the 8-bit codes,
// streamed with non-temporal 16-byte loads; LPR = D / 16 lanes per row, 16
// codes per lane.  A byte pair becomes two exact fp16 values with one v_perm
// against the fp16 exponent byte 0x64 (0x64XX is 1024 + XX = code + 1152),
// multiplied into the fp16 query with v_dot2_f32_f16; each lane then takes 1152
// times its share of the query sum off once, the row sums use DPP only, and
// the chunk's scale multiplies the sum.  Two load batches alternate, so one is
// in flight while the other is decoded.
//
// Pass 2 (group t selects for query t).  Every chunk's fp32 score s (as this
// kernel computes it) lies in [s_lo - d_c, s_lo + d_c] with d_c = K * s_c, K
// from the query's 1-norm (the derivation is at the bound below).  L, at most
// the k-th largest per-thread maximum of s_lo - d_c, is a lower bound of the
// k-th largest s; the candidates {c : s_lo[c] + d_c >= L} hold every chunk of
// the top k, ties included.  Their fp32 re-scores give the exact top-k (ties
// to the lower id), written in ascending order.  With a union output the block
// then merges the T lists, which it still holds in LDS.
// ---------------------------------------------------------------------------
#ifndef DK_SCORE_LO_UNROLL
#define DK_SCORE_LO_UNROLL 2   // 16-byte code loads per lane per batch
#endif

// bytes 0, 1 (sel 0x04010400) or 2, 3 (sel 0x04030402) of w as two fp16 values byte + 1024
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t sel) {
    return __builtin_amdgcn_perm(0x64646464u, w, sel);
}

// 32-bit words of one group's LDS: keys [Cp] | cand [max(Cp, 256)] | qv [nvec][D]
// | hist [256] | scratch [8] | bc [2] | misc [6], Cp = C rounded up to 4 so that
// every array starts on 16 bytes.  Pass 1 keeps its scores [T][C] over group
// 0's keys and cand.
__host__ __device__ inline size_t select_group_words(int C, int D, int nvec) {
    const int Cp = (C + 3) & ~3;
    return (size_t)Cp + (size_t)(Cp > 256 ? Cp : 256) + (size_t)nvec * D + 256 + 16;
}

// The work of one (b, g): the block's threads in LDS smem2 (T groups of
// select_group_words).  KPT: shadow scores each pass-2 thread holds in registers
// (at least C / 256).
template <int D, int NQ, int T, bool MAXRED, int F, int KPT>
__device__ __forceinline__ void score_select_block(
    uint32_t* smem2, int bg, const float* __restrict__ q, int Hq, const uint8_t* __restrict__ lm8,
    const float* __restrict__ chunk_scale, const float* __restrict__ scale_max, const float* __restrict__ lm,
    dk_strides ls, int Hkv, int C, int k, float scale, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_score, const UnionOut& un) {
    constexpr int NVEC = MAXRED ? NQ / T : 1;          // query vectors per group
    constexpr int NW = T * F * kThreads / kWave;       // waves of the block (pass 1 uses all)
    const int Cp = (C + 3) & ~3;
    const int cand_words = Cp > kThreads ? Cp : kThreads;
    const size_t gw = select_group_words(C, D, NVEC);
    auto qv_of = [&](int u) { return (float*)(smem2 + (size_t)u * gw + Cp + cand_words); };
    auto misc_of = [&](int u) { return (int*)(smem2 + (size_t)u * gw + gw - 6); };

    const int b = bg / Hkv, g = bg - b * Hkv;
    const int Gq = Hq / Hkv;
    const float SM = scale_max[bg];   // for pass 2, loaded early

    // ================= pass 1: shadow scores of every chunk =================
    {
        constexpr int LPR = D / 16, RPW = kWave / LPR, U = DK_SCORE_LO_UNROLL;
        constexpr int G = MAXRED ? NQ / T : 0;
        float* sres = (float*)smem2;                   // [T][C]
        const int lane = threadIdx.x & (kWave - 1), bw = threadIdx.x / kWave;
        const int rp = lane / LPR, part = lane % LPR;

        const uint8_t* base = lm8 + (int64_t)bg * C * D + part * 16;
        const float* sbase = chunk_scale + (int64_t)bg * C;
        u32x4_t xa[U], xb[U];
        float ra[U], rb[U];
        // Rows go in batches of BR consecutive rows, one wave per batch: each
        // wave takes its first two batches statically and every later one from
        // a counter in LDS, so waves that meet slower memory take fewer batches
        // and the waves end pass 1 together.
        constexpr int BR = RPW * U;
        const int nbatch = (C + BR - 1) / BR;
        int* batch_ctr = misc_of(0) + 2;
        auto grab = [&]() {
            int j = 0;
            if (lane == 0) j = atomicAdd(batch_ctr, 1);
            return __builtin_amdgcn_readfirstlane(j);
        };
        auto load_rows = [&](int jb, u32x4_t (&xx)[U], float (&rr)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = jb * BR + u * RPW + rp;
                xx[u] = r < C ? nt_load_u4(base + (int64_t)r * D)
                              : u32x4_t{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
                rr[u] = part < T && r < C ? sbase[r] : 0.f;
            }
        };
        // the first two batches of rows are requested before anything else
        int ja = bw, jb = NW + bw;
        if (ja < nbatch) load_rows(ja, xa, ra);
        if (jb < nbatch) load_rows(jb, xb, rb);
        if (threadIdx.x == 0) *batch_ctr = 2 * NW;   // read only after the staging barrier below
        // The query elements this thread stages: their loads go out right
        // after the first two batches of rows, so both arrive within about one
        // memory latency (a wait for the queries is also a wait for the rows
        // issued before them).
        constexpr int QI = (NQ * D + NW * kWave - 1) / (NW * kWave);   // query elements per thread
        float xqv[QI];
#pragma unroll
        for (int j = 0; j < QI; ++j) {
            const int i = threadIdx.x + j * NW * kWave;
            const int v = i / D, e = i - v * D;
            float xq = 0.f;
            if (i < NQ * D) {
                if constexpr (MAXRED) {
                    xq = q[(((int64_t)b * T + v / G) * Hq + g * Gq + v % G) * D + e];
                } else {
                    // heads four at a time, their loads issued together
                    const float* qh0 = q + (((int64_t)b * T + v) * Hq + g * Gq) * D + e;
                    for (int h0 = 0; h0 < Gq; h0 += 4) {
                        float x4[4];
#pragma unroll
                        for (int hh = 0; hh < 4; ++hh) x4[hh] = h0 + hh < Gq ? qh0[(int64_t)(h0 + hh) * D] : 0.f;
#pragma unroll
                        for (int hh = 0; hh < 4; ++hh) xq += x4[hh];
                    }
                    xq = xq / (float)Gq;
                }
            }
            xqv[j] = xq;
        }
        // the chunk scales also go to LDS for pass 2: over group 1's keys (group
        // 0's cand with T = 1), which pass 2 writes only after reading them
        float* scl = (float*)smem2 + (T == 2 ? gw : (size_t)C);

        // The query vectors go through LDS once per block, into the groups'
        // qv[] (vector v is vector v % NVEC of group v / NVEC), which pass 2
        // re-scores with.
#pragma unroll
        for (int j = 0; j < QI; ++j) {
            const int i = threadIdx.x + j * NW * kWave;
            if (i < NQ * D) qv_of(i / D / NVEC)[(i / D % NVEC) * D + i % D] = xqv[j];
        }
        __syncthreads();
        uint32_t qh[NQ][8];
        float qbias[NQ];   // 1152 times this lane's share of the fp16 query sum
#pragma unroll
        for (int v = 0; v < NQ; ++v) {
            const float* qp = qv_of(v / NVEC) + (v % NVEC) * D;
            float sq = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const _Float16 h0 = (_Float16)qp[part * 16 + 2 * j];
                const _Float16 h1 = (_Float16)qp[part * 16 + 2 * j + 1];
                qh[v][j] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                sq += (float)h0 + (float)h1;
            }
            qbias[v] = 1152.f * sq;
        }

        auto process = [&](int jbt, const u32x4_t (&x)[U], const float (&rs)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int rr = jbt * BR + u * RPW + rp;
                uint32_t h[8];
                h[0] = code_pair(x[u].x, 0x04010400u); h[1] = code_pair(x[u].x, 0x04030402u);
                h[2] = code_pair(x[u].y, 0x04010400u); h[3] = code_pair(x[u].y, 0x04030402u);
                h[4] = code_pair(x[u].z, 0x04010400u); h[5] = code_pair(x[u].z, 0x04030402u);
                h[6] = code_pair(x[u].w, 0x04010400u); h[7] = code_pair(x[u].w, 0x04030402u);
                float dot[NQ];
#pragma unroll
                for (int v = 0; v < NQ; ++v) {
                    float a = dot2_f16(qh[v][0], h[0], 0.f);
#pragma unroll
                    for (int jj = 1; jj < 8; ++jj) a = dot2_f16(qh[v][jj], h[jj], a);
                    dot[v] = dpp_group_sum<LPR>(a - qbias[v]);
                }
                // per-query scores with compile-time register indices
                const float sc = scale * rs[u];
                float sct[T];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    if constexpr (MAXRED) {
                        sct[t] = sc * dot[t * G];
#pragma unroll
                        for (int hh = 1; hh < G; ++hh) sct[t] = fmaxf(sct[t], sc * dot[t * G + hh]);
                    } else {
                        sct[t] = sc * dot[t];
                    }
                }
                if (part < T && rr < C) sres[part * C + rr] = (part == 0) ? sct[0] : sct[T - 1];
                if (part == 0 && rr < C) scl[rr] = rs[u];
            }
        };
        // two batches in flight: a batch's registers are refilled once it is
        // scored.  Batches come from the counter in increasing order, so once jb
        // is past the end the batch taken into ja is too.
        for (;;) {
            if (ja >= nbatch) break;
            process(ja, xa, ra);
            ja = grab();
            if (ja < nbatch) load_rows(ja, xa, ra);
            if (jb >= nbatch) break;
            process(jb, xb, rb);
            jb = grab();
            if (jb < nbatch) load_rows(jb, xb, rb);
        }
        {
            // The error bound's query factor for pass 2.  With m_i the codes,
            // s_c the chunk scale, q^ = fp16(q) and u16 = 2^-11:
            //   |sum q_i l_i - s_c sum q^_i m_i| <= s_c (1/2 + 127 u32) |q|_1            (the codes)
            //                                     + s_c 127 (u16 |q|_1 + D 2^-25)   (q in fp16, subnormals too),
            // the fp32 sums here and of the fp32 re-score add at most (D + 40)
            // roundings of terms up to 127 s_c |q_i|; the lanes sum q^_i (code_i + 1152)
            // and take off 1152 times their fp32 sum of q^: at most 48000 u32 s_c |q|_1
            // more; the scale products add a few relative roundings: |s - s_lo| <= kq * s_c.  A query value beyond fp16
            // voids the bound (kq = inf: every chunk becomes a candidate).
            float* pq = qv_of(0) + NVEC * D;   // group 0's hist[]: free until pass 2
            for (int v = bw; v < NQ; v += NW) {
                const float* qp = qv_of(v / NVEC) + (v % NVEC) * D;
                float a1 = 0.f, am = 0.f;
                for (int e = lane; e < D; e += kWave) {
                    a1 += fabsf(qp[e]);
                    am = fmaxf(am, fabsf(qp[e]));
                }
                for (int off = 1; off < kWave; off <<= 1) {
                    a1 += __shfl_xor(a1, off, kWave);
                    am = fmaxf(am, __shfl_xor(am, off, kWave));
                }
                if (lane == 0) {
                    pq[2 * v] = a1;
                    pq[2 * v + 1] = am;
                }
            }
            __syncthreads();   // (the end of pass 1)
            if (threadIdx.x < T) {
                const int t = threadIdx.x;
                float l1 = 0.f, amax = 0.f;
                for (int v = (MAXRED ? t * G : t); v < (MAXRED ? (t + 1) * G : t + 1); ++v) {
                    l1 = fmaxf(l1, pq[2 * v]);
                    amax = fmaxf(amax, pq[2 * v + 1]);
                }
                l1 *= 1.0f + (float)(D + 8) * 5.9604645e-8f;   // round the sum up
                const float u16 = 4.8828125e-4f, u32 = 5.9604645e-8f;
                float k_ = fabsf(scale) *
                           (l1 * (0.5f + 127.f * u32 + 127.f * u16 + ((float)(D + 40) * 127.f + 48000.f) * u32) +
                            127.f * (float)D * 2.9802322e-8f) * 1.01f;
                if (!(amax <= 65000.f) || !(k_ <= 3.0e38f)) k_ = INFINITY;
                misc_of(t)[1] = __float_as_int(k_);
            }
        }
    }
    // Pass 2 runs T groups of kThreads threads; the waves beyond them (F = 2)
    // end here, and the block barriers below wait only for the waves left.
    if (threadIdx.x >= T * kThreads) return;

    // ================= pass 2: exact top-k of group t's query ================
    constexpr int LPR = D / 8;                 // lanes per fp32 row, 8 floats each
    constexpr int RPW = kWave / LPR;
    const int t = threadIdx.x / kThreads;
    uint32_t* keys = smem2 + (size_t)t * gw;
    int32_t* cand = (int32_t*)(keys + Cp);
    uint32_t* cand_u = (uint32_t*)cand;
    float* qv = qv_of(t);
    uint32_t* hist = (uint32_t*)(qv + NVEC * D);     // [256]
    int* scratch = (int*)(hist + 256);               // [8]
    int* bc = scratch + 8;                           // [2]
    int* misc = misc_of(t);                          // [0] candidates, [1] bound factor (bits)
    const int tid = threadIdx.x & (kThreads - 1), lane = tid & (kWave - 1), wave = tid / kWave;

    // this thread's contiguous range of shadow scores and chunk scales (both
    // in LDS), kept in registers
    static_assert(KPT % 4 == 0 && KPT <= kShadowMaxC / kThreads, "KPT: a multiple of 4, at most 24");
    const int per = (C + kThreads - 1) / kThreads;
    const int lo = min(C, tid * per), hi = min(C, lo + per);
    const float* sl = (const float*)smem2 + t * C;
    const float* cs = (const float*)smem2 + (T == 2 ? gw : (size_t)C);
    float sv[KPT], sc[KPT];
    if ((per & 3) == 0 && (C & 3) == 0) {
#pragma unroll
        for (int i = 0; i < KPT / 4; ++i) {
            if (lo + 4 * i < hi) {
                const float4 x = *reinterpret_cast<const float4*>(sl + lo + 4 * i);
                const float4 y = *reinterpret_cast<const float4*>(cs + lo + 4 * i);
                sv[4 * i] = x.x; sv[4 * i + 1] = x.y; sv[4 * i + 2] = x.z; sv[4 * i + 3] = x.w;
                sc[4 * i] = y.x; sc[4 * i + 1] = y.y; sc[4 * i + 2] = y.z; sc[4 * i + 3] = y.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) sv[4 * i + j] = sc[4 * i + j] = 0.f;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            sv[i] = lo + i < hi ? sl[lo + i] : 0.f;
            sc[i] = lo + i < hi ? cs[lo + i] : 0.f;
        }
    }
    __syncthreads();   // every score is in registers: the scores' LDS is reused from here on
    const float Kq = __int_as_float(misc[1]);

    // the bound |s - s_lo| <= Kq * s_c (Kq from pass 1); a landmark the codes
    // cannot hold, or Kq = inf, voids it: every chunk is then a candidate
    const bool valid = SM <= 3.0e38f && Kq <= 3.0e38f;
    // the key order is the float order: the maximum of the lower bounds takes one key
    uint32_t kr[KPT];
    float flo = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const float d = Kq * sc[i];
        const float slo = sv[i] - d, shi = sv[i] + d;
        const float pad = (fabsf(sv[i]) + d) * 2.4e-7f + 1e-37f;   // round the bounds outwards
        kr[i] = lo + i < hi ? score_key(shi + pad) : 0u;
        if (lo + i < hi) flo = fmaxf(flo, slo - pad);
    }
    uint32_t* tmaxs = cand_u;                     // [256] scratch (cand[] is not used yet)
    tmaxs[tid] = hi > lo ? score_key(flo) : 0u;
    __syncthreads();
    if (wave == 0) {
        // a lower bound of the k-th largest of the per-thread maxima (its top 20
        // key bits, a relative 2^-11 of the score below it at most): at least k
        // chunks score at least this much.  For k > 256 the bound is 0, i.e.
        // every chunk is a candidate.
        uint32_t kb = 0u;
        if (k <= kThreads) {
            uint32_t x[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) x[v] = tmaxs[lane + 64 * v];
            int nd;
            kb = wave_kth_key_bisect<12>(x, k, &nd);
        }
        if (lane == 0) bc[0] = (int)kb;
    }
    __syncthreads();
    const uint32_t thr_key = valid ? (uint32_t)bc[0] : 0u;

    // candidates in ascending chunk order
    int mine = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) mine += (lo + i < hi) && kr[i] >= thr_key;
    int ncand;
    int pos = group_exclusive_scan(mine, scratch, &ncand);
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if ((lo + i < hi) && kr[i] >= thr_key) cand[pos++] = lo + i;
    if (tid == 0) misc[0] = ncand;
    __syncthreads();
    // the wave selection below needs at most 256 candidates in every group (a
    // block-uniform choice: the block selection holds block barriers)
    bool wide = false;
    for (int u = 0; u < T; ++u) wide = wide || misc_of(u)[0] > kThreads;

    // exact fp32 scores of the candidates (keys[] is reused for them); UG rows
    // per lane group are loaded before any is used, so the gathers overlap
    constexpr int UG = 8;
    const int rp = lane / LPR, part = lane % LPR;
    const float* lb = lm + (int64_t)b * ls.b + (int64_t)g * ls.h + part * 8;
    float qm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qm[e] = qv[part * 8 + e];
    for (int j0 = 0; j0 < ncand; j0 += 4 * RPW * UG) {
        float x[UG][8];
        int jj[UG];
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            jj[u] = j0 + (u * 4 + wave) * RPW + rp;
            if (jj[u] < ncand) {
                const float* src = lb + (int64_t)cand[jj[u]] * ls.t;
                const float4 x0 = *reinterpret_cast<const float4*>(src);
                const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
                x[u][0] = x0.x; x[u][1] = x0.y; x[u][2] = x0.z; x[u][3] = x0.w;
                x[u][4] = x1.x; x[u][5] = x1.y; x[u][6] = x1.z; x[u][7] = x1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            float best;
            if (MAXRED) {
                best = -INFINITY;
                for (int v = 0; v < NVEC; ++v) {
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) a = fmaf(qv[v * D + part * 8 + e], x[u][e], a);
                    a = dpp_group_sum<LPR>(a);
                    best = fmaxf(best, scale * a);
                }
            } else {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) a = fmaf(qm[e], x[u][e], a);
                best = scale * dpp_group_sum<LPR>(a);
            }
            if (jj[u] < ncand && part == 0) keys[jj[u]] = score_key(best);
        }
    }
    __syncthreads();
    int32_t* oi = topk_idx + ((int64_t)bg * T + t) * k;
    float* os = topk_score ? topk_score + ((int64_t)bg * T + t) * k : nullptr;
    // the group's k ids in ascending order also go to sel[] (over keys[], once
    // the selection has read them) for the union below
    int32_t* sel = (int32_t*)keys;
    if (!wide) {
        // one wave: exact k-th key, then the winners in ascending position order
        if (wave == 0) {
            uint32_t x[4];
            int32_t cid[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool in = lane + 64 * v < ncand;
                x[v] = in ? keys[lane + 64 * v] : 0u;
                cid[v] = in ? cand[lane + 64 * v] : 0;
            }
            int need;
            const uint32_t thr2 = wave_kth_key_bisect(x, k, &need);
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            int base = 0, eq_base = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool eq = x[v] == thr2 && lane + 64 * v < ncand;
                const uint64_t eqm = __builtin_amdgcn_ballot_w64(eq);
                const int eq_rank = eq_base + __builtin_popcountll(eqm & below);
                const bool take = (x[v] > thr2 && lane + 64 * v < ncand) || (eq && eq_rank < need);
                const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
                if (take) {
                    const int jpos = base + __builtin_popcountll(tm & below);
                    if (jpos < k) {
                        oi[jpos] = cid[v];
                        sel[jpos] = cid[v];
                        if (os) os[jpos] = key_score(x[v]);
                    }
                }
                base += __builtin_popcountll(tm);
                eq_base += __builtin_popcountll(eqm);
            }
        }
    } else {
        // the ids also go to sel[] through global memory, as emit runs while
        // the selection still reads keys[]
        block_topk(keys, ncand, k, hist, scratch, bc, [&](int jpos, int i, uint32_t key) {
            oi[jpos] = cand[i];
            if (os) os[jpos] = key_score(key);
        });
        __syncthreads();
        for (int i = tid; i < k; i += kThreads) sel[i] = oi[i];
    }
    if (un.ids == nullptr) return;

    // Union of the (b, g)'s T sets (block-wide; sel[] of group 1 is s1).
    __syncthreads();
    int32_t* s0 = (int32_t*)smem2;
    int32_t* s1 = (int32_t*)(smem2 + gw);
    int32_t* dup_pre = (int32_t*)smem2 + Cp;              // group 0's cand[] (k + 1 ints)
    int* uscratch = (int*)(qv_of(0) + NVEC * D);          // group 0's hist[]
    const int N = T * k;
    int nshared;
    const int count = block_union_two(s0, s1, T, k, un.ids + (int64_t)bg * N, un.member + (int64_t)bg * N,
                                      dup_pre, uscratch, nullptr, &nshared);
    if (threadIdx.x == 0) {
        un.count[bg] = count;
        if (un.overlap) un.overlap[bg] = nshared;
    }
}

// One decode step of one layer for one (b, g) per block: the shadow scoring,
// exact selection and union above, then the attention fast path over the union
// the block has just written.  A block needs no other block's result, so the
// blocks that finish their selection early stream their attention while the
// others still score: the selection phase of one block overlaps the gathers of
// another, and the attention launch and its start-up latency go away.
struct StepArgs {
    const float* q;
    int Hq, Hkv, C, k;
    float scale;
    const uint8_t* lm8;
    const float* chunk_scale;
    const float* scale_max;
    const float* lm;
    dk_strides ls;
    int32_t* topk_idx;
    float* topk_score;
    UnionOut un;
    attn::AttnArgs a;   // block_ids / member / count are the union outputs
};

template <int KPT>
__global__ __launch_bounds__(2 * kThreads) void k_step_fused(StepArgs s) {
    extern __shared__ uint32_t smem2[];
    int bg, unused;
    xcd_unit(blockIdx.x, 1, gridDim.x, bg, unused);
    score_select_block<128, 2, 2, false, 1, KPT>(smem2, bg, s.q, s.Hq, s.lm8, s.chunk_scale, s.scale_max, s.lm,
                                                 s.ls, s.Hkv, s.C, s.k, s.scale, s.topk_idx, s.topk_score, s.un);
    __syncthreads();   // the union this block wrote is visible to all its threads; LDS is free
    if (threadIdx.x >= attn::kFastThreads) return;
    // The CU's other block may still be selecting: its ALU work yields to these
    // waves' loads and DMA issues, which keep HBM busy (measured: 4.71 -> 4.67 ms
    // per 32-layer step at B = 64, L = 128K; the reverse order gains nothing).
    __builtin_amdgcn_s_setprio(2);
    attn::attn_fast_block<false>(s.a, *reinterpret_cast<attn::FastSmem*>(smem2), bg, 0);
}

template <int D, int NQ, int T, bool MAXRED, int F, int KPT>
__global__ __launch_bounds__(T * kThreads * F) void k_score_select(
    const float* __restrict__ q, int Hq, const uint8_t* __restrict__ lm8, const float* __restrict__ chunk_scale,
    const float* __restrict__ scale_max, const float* __restrict__ lm, dk_strides ls, int Hkv, int C, int k,
    float scale, int32_t* __restrict__ topk_idx, float* __restrict__ topk_score, UnionOut un) {
    extern __shared__ uint32_t smem2[];
    int bg, unused;
    xcd_unit(blockIdx.x, 1, gridDim.x, bg, unused);
    score_select_block<D, NQ, T, MAXRED, F, KPT>(smem2, bg, q, Hq, lm8, chunk_scale, scale_max, lm, ls, Hkv, C, k,
                                                 scale, topk_idx, topk_score, un);
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

template <int D, int NQ, int T, bool MAXRED>
hipError_t launch_score_select(const float* q, int B, int Hq, const dk_landmark_shadow* sh, const float* lm,
                               dk_strides ls, int Hkv, int C, int k, float scale, int32_t* topk_idx,
                               float* topk_score, const UnionOut& un, hipStream_t st) {
    constexpr int NVEC = MAXRED ? NQ / T : 1;
    const size_t lds = (size_t)T * select_group_words(C, D, NVEC) * 4;
    const int64_t bg = (int64_t)B * Hkv;
    // With at most one block per CU (256 CUs) the score pass streams with twice
    // the waves (rows enough to stream: C >= 512; a short row is latency-bound
    // and pays for the extra waves); with more blocks two resident blocks per
    // CU give the same.
    auto go = [&](auto kpt) {
        constexpr int KPT = decltype(kpt)::value;
        if (bg <= 256 && C >= 512)
            hipLaunchKernelGGL((k_score_select<D, NQ, T, MAXRED, 2, KPT>), dim3((unsigned)bg), dim3(2 * T * kThreads),
                               lds, st, q, Hq, sh->lm8, sh->chunk_scale, sh->scale_max, lm, ls, Hkv, C, k, scale,
                               topk_idx, topk_score, un);
        else
            hipLaunchKernelGGL((k_score_select<D, NQ, T, MAXRED, 1, KPT>), dim3((unsigned)bg), dim3(T * kThreads),
                               lds, st, q, Hq, sh->lm8, sh->chunk_scale, sh->scale_max, lm, ls, Hkv, C, k, scale,
                               topk_idx, topk_score, un);
    };
    // pass 2 keeps ceil(C / 256) scores per thread in registers: the mean-reduced
    // selections (the decode step's) get a register count fitted to C, so no
    // masked slots run; the others keep the largest
    constexpr int kMax = kShadowMaxC / kThreads;
    const int per = (C + kThreads - 1) / kThreads;
    if constexpr (!MAXRED) {
        if (per <= 4)
            go(std::integral_constant<int, 4>{});
        else if (per <= 16)
            go(std::integral_constant<int, 16>{});
        else
            go(std::integral_constant<int, kMax>{});
    } else {
        go(std::integral_constant<int, kMax>{});
    }
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_score_select(int nq, int T, bool maxred, const float* q, int B, int Hq,
                                 const dk_landmark_shadow* sh, const float* lm, dk_strides ls, int Hkv, int C,
                                 int k, float scale, int32_t* topk_idx, float* topk_score, const UnionOut& un,
                                 hipStream_t st) {
#define DK_SS(NQ_, T_, MX_) \
    if (nq == NQ_ && T == T_ && maxred == MX_) \
        return launch_score_select<D, NQ_, T_, MX_>(q, B, Hq, sh, lm, ls, Hkv, C, k, scale, topk_idx, topk_score, \
                                                    un, st);
    DK_SS(1, 1, false)
    DK_SS(2, 2, false)
    DK_SS(1, 1, true)
    DK_SS(2, 1, true)
    DK_SS(4, 1, true)
    DK_SS(8, 1, true)
    DK_SS(16, 1, true)
    DK_SS(2, 2, true)
    DK_SS(4, 2, true)
    DK_SS(8, 2, true)
    DK_SS(16, 2, true)
#undef DK_SS
    return hipErrorInvalidValue;
}

}  // namespace

TopkPlan plan_topk(int B, int Hkv, int T, int C, int k, bool shadow) {
    TopkPlan p{0, 0, 0};
    const int64_t bg = (int64_t)B * Hkv;
    if (shadow) {
        // one block per (b, g) scores and selects; everything stays in LDS
        if (C > kShadowMaxC) return p;
        p.splits = 1;
        p.rows = C;
        return p;
    }
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

hipError_t launch_build_shadow(const float* lm, dk_strides ls, int B, int Hkv, int C, int d,
                               uint8_t* lm8, float* chunk_scale, float* scale_max, hipStream_t st) {
    const unsigned grid = (unsigned)((int64_t)B * Hkv);
    if (d == 128)
        hipLaunchKernelGGL(k_build_shadow<128>, dim3(grid), dim3(kThreads), 0, st, lm, ls, Hkv, C, lm8, chunk_scale,
                           scale_max);
    else
        hipLaunchKernelGGL(k_build_shadow<64>, dim3(grid), dim3(kThreads), 0, st, lm, ls, Hkv, C, lm8, chunk_scale,
                           scale_max);
    return hipGetLastError();
}

hipError_t launch_score_topk(const float* q, int B, int T, int Hq, const float* lm, dk_strides ls,
                             int Hkv, int C, int d, int k, float scale, dk_group_reduce reduce,
                             const dk_landmark_shadow* shadow, int32_t* topk_idx, float* topk_score,
                             void* ws, const TopkPlan& p, const UnionOut* un, hipStream_t st) {
    const bool maxred = reduce == DK_REDUCE_MAX;
    const int G = Hq / Hkv;
    const int nq = maxred ? G * T : T;
    const int64_t bg = (int64_t)B * Hkv;
    if (shadow) {
        // the kernel merges the union itself when the merge's scan prefix
        // (k + 1 ints) fits where its first group's candidates were
        const int Cp = (C + 3) & ~3;
        const bool fuse = un && (int64_t)k + 1 <= (int64_t)(Cp > kThreads ? Cp : kThreads);
        const UnionOut none{nullptr, nullptr, nullptr, nullptr};
        const UnionOut uo = fuse ? *un : none;
        hipError_t e = d == 128
            ? dispatch_score_select<128>(nq, T, maxred, q, B, Hq, shadow, lm, ls, Hkv, C, k, scale, topk_idx,
                                         topk_score, uo, st)
            : dispatch_score_select<64>(nq, T, maxred, q, B, Hq, shadow, lm, ls, Hkv, C, k, scale, topk_idx,
                                        topk_score, uo, st);
        if (e != hipSuccess || !un || fuse) return e;
        return launch_union(topk_idx, B, Hkv, T, k, C, un->ids, un->member, un->count, un->overlap,
                            nullptr, st);
    }
    const int64_t ncand = bg * T * p.splits * k;
    uint32_t* ck = p.splits > 1 ? (uint32_t*)ws : nullptr;
    int32_t* ci = p.splits > 1 ? (int32_t*)((char*)ws + ncand * 4) : nullptr;
    hipError_t e = d == 128
        ? dispatch_split<128>(nq, T, maxred, q, B, Hq, lm, ls, Hkv, C, k, scale, p, ck, ci, topk_idx,
                              topk_score, st)
        : dispatch_split<64>(nq, T, maxred, q, B, Hq, lm, ls, Hkv, C, k, scale, p, ck, ci, topk_idx,
                             topk_score, st);
    if (e != hipSuccess) return e;
    if (p.splits > 1) {
        const size_t lds = (size_t)(p.splits * k + 256 + 10) * 4;
        hipLaunchKernelGGL(k_topk_merge, dim3((unsigned)bg), dim3(kThreads), lds, st, ck, ci, T, k,
                           p.splits, topk_idx, topk_score);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!un) return hipSuccess;
    return launch_union(topk_idx, B, Hkv, T, k, C, un->ids, un->member, un->count, un->overlap, nullptr,
                        st);
}


hipError_t launch_step_fused(const float* q, int B, int Hq, int Hkv, int C, int k, float scale,
                             const dk_landmark_shadow* sh, const float* lm, dk_strides ls, const void* K,
                             const void* V, dk_strides ks, dk_strides vs, int chunk, int32_t* topk_idx,
                             float* topk_score, const UnionOut& un, float* out, float* lse, hipStream_t st) {
    constexpr int T = 2;
    StepArgs s{};
    s.q = q; s.Hq = Hq; s.Hkv = Hkv; s.C = C; s.k = k; s.scale = scale;
    s.lm8 = sh->lm8; s.chunk_scale = sh->chunk_scale; s.scale_max = sh->scale_max;
    s.lm = lm; s.ls = ls; s.topk_idx = topk_idx; s.topk_score = topk_score; s.un = un;
    attn::AttnArgs& a = s.a;
    a.q = q; a.Hq = Hq; a.Hkv = Hkv; a.T = T; a.G = Hq / Hkv;
    a.K = K; a.V = V; a.ks = ks; a.vs = vs; a.chunk = chunk;
    a.block_ids = un.ids; a.member = un.member; a.count = un.count;
    a.N = T * k; a.pool_blocks = C;
    a.scale_log2 = scale * attn::kLog2e;
    a.splits = 1; a.nparts = 1;
    a.out = out; a.lse = lse;
    const size_t lds_sel = (size_t)T * select_group_words(C, 128, 1) * 4;
    const size_t lds = lds_sel > sizeof(attn::FastSmem) ? lds_sel : sizeof(attn::FastSmem);
    const unsigned grid = (unsigned)((int64_t)B * Hkv);
    const int per = (C + kThreads - 1) / kThreads;
    if (per <= 4)
        hipLaunchKernelGGL(k_step_fused<4>, dim3(grid), dim3(2 * kThreads), lds, st, s);
    else if (per <= 16)
        hipLaunchKernelGGL(k_step_fused<16>, dim3(grid), dim3(2 * kThreads), lds, st, s);
    else
        hipLaunchKernelGGL(k_step_fused<kShadowMaxC / kThreads>, dim3(grid), dim3(2 * kThreads), lds, st, s);
    return hipGetLastError();
}

}  // namespace dk
