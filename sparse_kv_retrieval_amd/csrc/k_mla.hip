// Attention over a latent KV head with token-level selection, on the matrix cores.
//
// Adaptive DHiSparse, Figure 2: attention reads the rows the indexer selected;
// Figure 3 (2): the selections of the step's queries are resolved together and
// each query attends over its own.  One latent row per token holds the key
// (all dk = 576 columns: 512 content + 64 position) and, in its first dv = 512
// columns, the value; every query head of the group reads the same rows.
//
//   out[b, t, h] = softmax_j(scale * <q[b, t, h], lat[j]>) lat[j, :512] over the
//                  tokens j of query t's own set, lse = log of the softmax sum.
//
// With 128 heads and two tokens per request, 256 query rows share every
// latent row: the product is a dense GEMM (about 480 flop per byte of latent
// row), so it runs on v_mfma_f32_16x16x32_bf16.
//
// Block (512 threads, 8 waves): 64 query rows = HB heads x T tokens (HB = 64/T)
// of one (b, g), over one contiguous range of its union entries, 32 tokens per
// tile.
//   * the range's union entries are staged in LDS first, then tiles of 32
//     latent rows (36 KiB) go global -> LDS by DMA into a three-stage ring (two
//     tiles in flight while one is used); each LDS row is padded by 16 bytes
//     (1168-byte stride: eight consecutive rows start on distinct bank groups)
//     and its 16-byte pieces are XOR-permuted by 2 * ((row / 8) mod 4), so the
//     key reads (16 bytes per lane, eight consecutive rows) and the value reads
//     (2 bytes per lane, four groups of rows eight apart) hit distinct banks, and
//     every read is a per-lane base plus immediate offsets;
//   * S = Q K^T: wave w owns row tile w % 4 (16 rows of one query token) and
//     token half w / 4, Q in registers as bf16 A operands, K pieces from LDS as
//     B operands, 18 k-steps;
//   * online softmax in log2 units per row (mask: the token is in the row's own
//     set), the row maximum shared between the two token halves through LDS,
//     weights rounded to bf16 into LDS;
//   * O += P V: wave w owns value columns 64w..64w+63 for all 64 rows, P rows
//     from LDS as A operands, value columns gathered from the same LDS tile.
// Ranges of one (b, g) are combined by k_mla_merge.  The four row groups of a
// (b, g, range) share an XCD (block id mod 8) so that the other three find the
// tiles in L2.
#include "dk_common.h"

namespace dk {
namespace {

constexpr int kMlaThreads = 512;
constexpr int kMlaWaves = kMlaThreads / 64;
constexpr int kMlaRows = 64;              // query rows per block
constexpr int kMlaDk = 576, kMlaDv = 512;
constexpr int kMlaTok = 32;               // tokens per tile
constexpr int kMlaPieces = kMlaDk / 8;    // 16-byte pieces per latent row (72)
constexpr int kMlaRowPieces = kMlaPieces + 1;   // LDS row: 72 pieces + one pad (1168 bytes)
constexpr int kMlaRowBytes = kMlaRowPieces * 16;
constexpr int kMlaDmaTotal = (kMlaTok * kMlaRowPieces + 63) / 64;       // 37 per tile
constexpr int kMlaTilePieces = kMlaDmaTotal * 64;                       // ring stage, DMA overrun included
constexpr int kMlaDmaMax = (kMlaDmaTotal + kMlaWaves - 1) / kMlaWaves;   // 5 (waves 0-4), else 4
constexpr int kMlaStages = 3;             // LDS ring: two tiles in flight while one is used
constexpr int kMlaMaxRange = 2048;        // union entries per block (ids staged in LDS)
constexpr int kPRow = 40;                 // bf16 per row of the P tile (80 bytes)
constexpr float kMlaSlack = 8.f;          // log2 headroom of the lazy running maximum

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct __align__(16) MlaSmem {
    uint4 tile[kMlaStages][kMlaTilePieces];   // latent rows, 73 pieces each (the last a pad)
    int32_t ids[kMlaMaxRange];             // the range's token ids (0 when invalid)
    uint8_t mem[kMlaMaxRange];             // and their member bits (0 when invalid)
    uint16_t p[kMlaRows * kPRow];          // bf16 weights [row][token]
    float alpha[kMlaRows];                 // per-row rescale of this tile
    float hmax[2][kMlaRows];               // tile maximum of each token half
    float row_m[kMlaRows];
    float row_l[2][kMlaRows];
    int flag[kMlaWaves];
};

// LDS DMA that keeps the lines in L2 (the other row groups read the same tile)
__device__ __forceinline__ void lds_dma16_keep(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
// piece permutation of LDS row j: global piece p sits at position p ^ mla_swz(j)
__device__ __forceinline__ int mla_swz(int j) { return 2 * ((j >> 3) & 3); }

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();
}

__device__ __forceinline__ float dpp_group_max16(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
    return v;
}

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct MlaArgs {
    const float* q;            // [B, T, Hq, 576]
    const uint16_t* lat;       // latent rows, strides ks (elements)
    dk_strides ks;
    const int32_t* ids;        // [B * Hkv, N] token ids of the union, ascending
    const uint8_t* member;     // [B * Hkv, N] bit t: in query t's set (NULL: every bit)
    const int32_t* count;      // [B * Hkv]
    int B, T, Hq, Hkv, N, L, splits, rgroups, work;   // work = B * Hkv * splits
    float scale_log2;
    float* out;                // [B, T, Hq, 512]
    float* lse;                // [B, T, Hq] or NULL
    float* part_o;             // [work][rgroups][64][512] when splits > 1
    float* part_ml;            // [work][rgroups][64][2]
};

__global__ __launch_bounds__(kMlaThreads) void k_mla_attn(MlaArgs a) {
    __shared__ MlaSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // S phase: wave w owns row tile mw (rows 16mw .. 16mw+15) and token half nw;
    // O phase: value columns 64w .. 64w+63 of all 64 rows
    const int mw = w & 3, nw = w >> 2;
    // block -> (work item f, row group rg); the row groups of f share blockIdx mod 8
    const int blk = blockIdx.x;
    const int f = (blk / (8 * a.rgroups)) * 8 + (blk % 8);
    const int rg = (blk / 8) % a.rgroups;
    if (f >= a.work) return;
    const int split = f % a.splits;
    const int bg = f / a.splits;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int T = a.T, HB = kMlaRows / T, G = a.Hq / a.Hkv;
    const int t_w = (16 * mw) / HB;                           // query token of row tile mw
    const int h_lane = g * G + rg * HB + (16 * mw) % HB + (lane & 15);   // head of row lane%16

    // entries of this range
    const int cnt = max(0, min(a.count[bg], a.N));
    const int per = (cnt + a.splits - 1) / a.splits;
    const int u0 = min(cnt, split * per);
    const int u1 = min(min(cnt, u0 + per), u0 + kMlaMaxRange);   // the plan keeps per <= kMlaMaxRange
    const int ntiles = (u1 - u0 + kMlaTok - 1) / kMlaTok;
    const int32_t* ids = a.ids + (int64_t)bg * a.N;
    const uint8_t* mem = a.member ? a.member + (int64_t)bg * a.N : nullptr;
    const char* lat_bg = (const char*)(a.lat + (int64_t)b * a.ks.b + (int64_t)g * a.ks.h);
    const int64_t row_bytes = a.ks.t * 2;

    // the tile's 37 DMA instructions: wave w issues i = w, w + 8, ... (< 37); the
    // (row, global piece) of each of this lane's slots is the same for every tile
    const int n_ent = u1 - u0;
    int slot[kMlaDmaMax];                            // row << 16 | byte offset in the row, or -1
#pragma unroll
    for (int c = 0; c < kMlaDmaMax; ++c) {
        const int pos = 64 * (w + kMlaWaves * c) + lane;
        const int j = pos / kMlaRowPieces, qp = pos - j * kMlaRowPieces;
        slot[c] = (qp < kMlaPieces && j < kMlaTok) ? (j << 16) | (16 * (qp ^ mla_swz(j))) : -1;
    }
    // source of slot c of a tile (pad slot, past the tile or past the range: row 0)
    auto dma_src = [&](int tile, int c) {
        int id = 0, off = 0;
        if (slot[c] >= 0) {
            const int e = tile * kMlaTok + (slot[c] >> 16);
            if (e < n_ent) {
                id = sm.ids[e];
                off = slot[c] & 0xffff;
            }
        }
        return lat_bg + (int64_t)id * row_bytes + off;
    };
    auto issue_slot = [&](int tile, int stage, int c) {
        const int i = w + kMlaWaves * c;             // DMA instruction (wave-uniform)
        if (i < kMlaDmaTotal) lds_dma16_keep(dma_src(tile, c), lds_addr(&sm.tile[stage][0]) + 1024u * (uint32_t)i);
    };
    auto issue_tile = [&](int tile, int stage) {
#pragma unroll
        for (int c = 0; c < kMlaDmaMax; ++c) issue_slot(tile, stage, c);
    };
    // DMAs per tile of this wave (the wait counts below)
    const bool dma5 = w < kMlaDmaTotal - kMlaWaves * (kMlaDmaMax - 1);

    // ---- prologue: the range's entries into LDS, the queries, tiles 0 and 1
    for (int x = tid; x < n_ent; x += kMlaThreads) {
        int v = ids[u0 + x];
        int m = mem ? (int)mem[u0 + x] : 0xff;
        if (v < 0 || v >= a.L) {
            v = 0;
            m = 0;
        }
        sm.ids[x] = v;
        sm.mem[x] = (uint8_t)m;
    }
    uint4 qa[18];
    {
        const float* qrow = a.q + (((int64_t)b * T + t_w) * a.Hq + h_lane) * kMlaDk + 8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * s);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * s + 4);
            qa[s] = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                               pack_bf16x2(x1.z, x1.w));
        }
    }
    __syncthreads();                                  // entries staged, every earlier load complete
    if (ntiles > 0) issue_tile(0, 0);
    if (ntiles > 1) issue_tile(1, 1);

    float m_run[4], l_half[4];
    f32x4_t acc[4][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        m_run[e] = -INFINITY;
        l_half[e] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int jt = 16 * nw + (lane & 15);        // this lane's token in the S phase

    // The loop issues no vector-memory operation but the tile DMAs, so the wait
    // counts are exact: at the top of iteration it the DMAs of tiles it and it + 1
    // may be outstanding, and tile it is complete once only tile it + 1's remain.
    // Tile it + 2 is issued during this iteration's S phase into the stage tile
    // it - 1 used; the barrier below is the last point any wave read it, and it
    // also orders this tile's P, flags and maxima after the previous tile's reads.
    for (int it = 0; it < ntiles; ++it) {
        const int stage = it % kMlaStages;
        if (it + 1 < ntiles) {
            if (dma5) vm_wait<kMlaDmaMax>();
            else vm_wait<kMlaDmaMax - 1>();
        } else {
            vm_wait<0>();
        }
        lds_barrier();
        const bool prefetch = it + 2 < ntiles;
        const int nstage = (it + 2) % kMlaStages;
        const uint4* tl = sm.tile[stage];

        // ---- S = Q K^T for row tile mw and the 16 tokens of half nw
        f32x4_t sacc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        // key operands in groups of three k-steps, the next group loaded before
        // the current one's products (at most six operands live)
        // global piece 4s + lane/16 of row jt sits at (4s + lane/16) ^ x, x = mla_swz(jt):
        // 4 (s ^ x/4) + (lane/16 ^ x%4), i.e. +4 pieces for even s and -4 for odd s when x >= 4
        const int xs = mla_swz(jt);
        const uint4* krow = tl + jt * kMlaRowPieces + ((lane >> 4) ^ (xs & 3));
        const uint4* kev = krow + 4 * (xs >> 2);
        const uint4* kod = krow - 4 * (xs >> 2);
        uint4 kb[2][3];
#pragma unroll
        for (int u = 0; u < 3; ++u) kb[0][u] = ((u & 1) ? kod : kev)[4 * u];
#pragma unroll
        for (int gi = 0; gi < 6; ++gi) {
            if (gi + 1 < 6) {
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const int st = 3 * (gi + 1) + u;
                    kb[(gi + 1) & 1][u] = ((st & 1) ? kod : kev)[4 * st];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int st = 3 * gi + u;
                sacc[st & 3] = mfma16(qa[st], kb[gi & 1][u], sacc[st & 3]);
            }
            // one DMA of tile it + 2 per group, under the products
            if (gi < kMlaDmaMax && prefetch) issue_slot(it + 2, nstage, gi);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- mask and online softmax (log2 units) with a lazy running maximum:
        // the weights use m_run as long as no logit of the row exceeds it by more
        // than kMlaSlack (the result does not depend on the reference, and the
        // weights stay below 2^kMlaSlack); otherwise the exact maximum over both
        // token halves is exchanged and the row rescaled.  Each lane keeps its own
        // token's share of the row sum, summed over the lanes once at the end.
        const int et = it * kMlaTok + jt;
        const bool valid = et < n_ent && ((sm.mem[et] >> t_w) & 1);
        float z[4];
        bool over = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = valid ? ((sacc[0][e] + sacc[1][e]) + (sacc[2][e] + sacc[3][e])) * a.scale_log2 : -INFINITY;
            over |= z[e] > m_run[e] + kMlaSlack;     // also any finite z while m_run is -inf
        }
        float l_prev[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * mw + 4 * (lane >> 4) + e;
            l_prev[e] = l_half[e];
            const float p = m_run[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[e] - m_run[e]);
            const __bf16 pb = (__bf16)p;
            l_half[e] += (float)pb;
            sm.p[r * kPRow + jt] = __builtin_bit_cast(uint16_t, pb);
        }
        const uint64_t anyover = __ballot(over);
        if (lane == 0) sm.flag[w] = anyover != 0;
        lds_barrier();
        bool rescale = false;
#pragma unroll
        for (int x = 0; x < kMlaWaves; ++x) rescale |= sm.flag[x] != 0;
        if (rescale) {
            // exact maximum of each row over both halves, then the weights again
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float hm = dpp_group_max16(z[e]);
                if ((lane & 15) == 0) sm.hmax[nw][16 * mw + 4 * (lane >> 4) + e] = hm;
            }
            lds_barrier();
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mw + 4 * (lane >> 4) + e;
                const float mx = fmaxf(sm.hmax[0][r], sm.hmax[1][r]);
                const float mn = fmaxf(m_run[e], mx);
                float alpha = 1.f, p = 0.f;
                if (mn != -INFINITY) {
                    alpha = __builtin_amdgcn_exp2f(m_run[e] - mn);
                    p = __builtin_amdgcn_exp2f(z[e] - mn);
                }
                const __bf16 pb = (__bf16)p;
                l_half[e] = l_prev[e] * alpha + (float)pb;
                m_run[e] = mn;
                sm.p[r * kPRow + jt] = __builtin_bit_cast(uint16_t, pb);
                if (nw == 0 && (lane & 15) == 0) sm.alpha[r] = alpha;
            }
            lds_barrier();
        }

        // ---- O += P V for value columns 64w .. 64w+63 of all 64 rows
        if (rescale) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[16 * m + 4 * (lane >> 4)]);
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    acc[m][n][0] *= al.x;
                    acc[m][n][1] *= al.y;
                    acc[m][n][2] *= al.z;
                    acc[m][n][3] *= al.w;
                }
            }
        }
        uint4 pa[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            pa[m] = *reinterpret_cast<const uint4*>(&sm.p[(16 * m + (lane & 15)) * kPRow + 8 * (lane >> 4)]);
        // value column c = 64w + 16n + lane%16 of token j = 8g + e (g = lane/16) sits in
        // piece (c / 8) ^ 2g = 8w + 2 (n ^ g) + (lane%16) / 8 of LDS row j
        const int gq = lane >> 4;
        const uint16_t* vcol = reinterpret_cast<const uint16_t*>(tl) + 8 * gq * (kMlaRowBytes / 2) +
                               8 * (8 * w + ((lane & 15) >> 3)) + (lane & 7);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const uint16_t* vn = vcol + 16 * (n ^ gq);
            uint16_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = vn[e * (kMlaRowBytes / 2)];
            const uint4 vb = make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                                        v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16));
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m][n] = mfma16(pa[m], vb, acc[m][n]);
        }
    }

    // ---- row statistics to every wave, then this wave's columns of all rows
#pragma unroll
    for (int e = 0; e < 4; ++e) l_half[e] = dpp_group_sum<16>(l_half[e]);
    if ((lane & 15) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * mw + 4 * (lane >> 4) + e;
            if (nw == 0) sm.row_m[r] = m_run[e];
            sm.row_l[nw][r] = l_half[e];
        }
    }
    lds_barrier();
    constexpr float kLn2 = 0.69314718055994531f;
    if (a.splits == 1) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * m + 4 * (lane >> 4) + e;
                const int t = r / HB, h = g * G + rg * HB + r % HB;
                const float l = sm.row_l[0][r] + sm.row_l[1][r];
                const float inv = l > 0.f ? 1.f / l : 0.f;
                float* orow = a.out + (((int64_t)b * T + t) * a.Hq + h) * kMlaDv + 64 * w + (lane & 15);
#pragma unroll
                for (int n = 0; n < 4; ++n) orow[16 * n] = acc[m][n][e] * inv;
                if (a.lse && w == 0 && (lane & 15) == 0)
                    a.lse[((int64_t)b * T + t) * a.Hq + h] = l > 0.f ? sm.row_m[r] * kLn2 + logf(l) : -INFINITY;
            }
        }
    } else {
        const int64_t slot = (int64_t)f * a.rgroups + rg;
        float* po = a.part_o + slot * kMlaRows * kMlaDv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * m + 4 * (lane >> 4) + e;
                float* prow = po + (int64_t)r * kMlaDv + 64 * w + (lane & 15);
#pragma unroll
                for (int n = 0; n < 4; ++n) prow[16 * n] = acc[m][n][e];
            }
        }
        if (w == 0) {
            float* pml = a.part_ml + slot * kMlaRows * 2;
            pml[2 * lane] = sm.row_m[lane];
            pml[2 * lane + 1] = sm.row_l[0][lane] + sm.row_l[1][lane];
        }
    }
}

// One wave per query row: combine the ranges' (m, l, O) by the online-softmax rule.
__global__ __launch_bounds__(256) void k_mla_merge(MlaArgs a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // over B * Hkv * rgroups * 64
    const int total = a.B * a.Hkv * a.rgroups * kMlaRows;
    if (row >= total) return;
    const int r = row % kMlaRows;
    const int rg = (row / kMlaRows) % a.rgroups;
    const int bg = row / (kMlaRows * a.rgroups);
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int T = a.T, HB = kMlaRows / T, G = a.Hq / a.Hkv;
    const int t = r / HB, h = g * G + rg * HB + r % HB;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) {
        const int64_t slot = ((int64_t)bg * a.splits + s) * a.rgroups + rg;
        M = fmaxf(M, a.part_ml[(slot * kMlaRows + r) * 2]);
    }
    float Lsum = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int s = 0; s < a.splits; ++s) {
            const int64_t slot = ((int64_t)bg * a.splits + s) * a.rgroups + rg;
            const float ms = a.part_ml[(slot * kMlaRows + r) * 2];
            if (ms == -INFINITY) continue;
            const float c = exp2f(ms - M);
            Lsum += c * a.part_ml[(slot * kMlaRows + r) * 2 + 1];
            const float4* po = reinterpret_cast<const float4*>(a.part_o + (slot * kMlaRows + r) * kMlaDv) + 2 * lane;
            const float4 x0 = po[0], x1 = po[1];
            o[0] += c * x0.x; o[1] += c * x0.y; o[2] += c * x0.z; o[3] += c * x0.w;
            o[4] += c * x1.x; o[5] += c * x1.y; o[6] += c * x1.z; o[7] += c * x1.w;
        }
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    float4* orow = reinterpret_cast<float4*>(a.out + (((int64_t)b * T + t) * a.Hq + h) * kMlaDv) + 2 * lane;
    orow[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    orow[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
    if (a.lse && lane == 0)
        a.lse[((int64_t)b * T + t) * a.Hq + h] = Lsum > 0.f ? M * 0.69314718055994531f + logf(Lsum) : -INFINITY;
}

}  // namespace

MlaPlan plan_mla(int B, int Hkv, int T, int Hq, int N) {
    MlaPlan p{};
    const int HB = kMlaRows / T;
    p.rgroups = (Hq / Hkv) / HB;
    const int64_t bg = (int64_t)B * Hkv;
    // one block per CU (the accumulators and the bf16 queries take the register
    // file), at least two tiles per range
    int64_t s = (256 + bg * p.rgroups - 1) / (bg * p.rgroups);
    const int64_t max_s = (N + 2 * kMlaTok - 1) / (2 * kMlaTok);
    if (s > max_s) s = max_s;
    // a range's entries must fit the LDS staging
    const int64_t min_s = (N + kMlaMaxRange - 1) / kMlaMaxRange;
    if (s < min_s) s = min_s;
    if (s < 1) s = 1;
    p.splits = (int)s;
    if (p.splits > 1) {
        const size_t slots = (size_t)bg * p.splits * p.rgroups;
        p.ws_bytes = slots * kMlaRows * (kMlaDv + 2) * 4;
    }
    return p;
}

hipError_t launch_mla_attention(const float* q, int B, int T, int Hq, int Hkv, const void* lat, dk_strides ks,
                                const int32_t* ids, const uint8_t* member, const int32_t* count, int N, int L,
                                float scale, float* out, float* lse, void* ws, const MlaPlan& plan,
                                hipStream_t st) {
    MlaArgs a{};
    a.q = q;
    a.lat = (const uint16_t*)lat;
    a.ks = ks;
    a.ids = ids;
    a.member = member;
    a.count = count;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.L = L;
    a.splits = plan.splits;
    a.rgroups = plan.rgroups;
    a.work = B * Hkv * plan.splits;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = out;
    a.lse = lse;
    if (plan.splits > 1) {
        const size_t slots = (size_t)a.work * plan.rgroups;
        a.part_o = (float*)ws;
        a.part_ml = (float*)ws + slots * kMlaRows * kMlaDv;
    }
    const unsigned grid = (unsigned)(((a.work + 7) / 8) * 8 * plan.rgroups);
    hipLaunchKernelGGL(k_mla_attn, dim3(grid), dim3(kMlaThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const int rows = B * Hkv * plan.rgroups * kMlaRows;
    hipLaunchKernelGGL(k_mla_merge, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace dk
