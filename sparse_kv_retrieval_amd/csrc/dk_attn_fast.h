// The attention fast path as a block-level device function, shared by the
// attention kernel (k_attention.hip) and the fused decode-step kernel
// (k_score_topk.hip): bf16 K/V, d = 128, G = 4, T = 2, chunk a multiple of 32.
//
// DualDecoder (arXiv 2607.26475), "4.2" and "5.3": the result equals attention
// over the true retrieval index; "5.2" and "6.4": the real and the speculative
// token share one pass.  Adaptive DHiSparse Figure 3 (2): each query attends
// over its own selection.
#pragma once

#include "dk_common.h"

namespace dk {
namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNoLogit = -1e30f;   // running-max floor of the fast path (log2 units)

struct AttnArgs {
    const float* q;
    int Hq, Hkv, T, G;
    const void* K;
    const void* V;
    dk_strides ks, vs;
    int chunk;
    const int32_t* block_ids;
    const uint8_t* member;
    const int32_t* count;
    int N, pool_blocks;
    float scale_log2;
    int splits;
    float* out;
    float* lse;
    float* part_acc;   // [bg][part][R][D]
    float* part_ml;    // [bg][part][R][2]
    int nparts;        // partial slots per (b, g): the ranges, plus one for the tail rows
    // rows every query attends besides its chunks (k_attn_tail)
    const void* Kt;
    const void* Vt;
    dk_strides kts, vts;
    const int32_t* tail_len;
    int tail_max;
    const void* Kn;    // [B, T, Hkv, D]: the step's own tokens
    const void* Vn;
};

__device__ __forceinline__ void entry_range(const AttnArgs& a, int bg, int split, int& u0, int& u1) {
    int n = a.count ? a.count[bg] : a.N;
    n = n < 0 ? 0 : (n > a.N ? a.N : n);
    u0 = (int)((int64_t)split * n / a.splits);
    u1 = (int)((int64_t)(split + 1) * n / a.splits);
}

// ---------------------------------------------------------------------------
// Fast path: bf16, D = 128, G = 4, T = 2, chunk % 32 == 0.
//
// Each of the block's four waves streams its own 16-key tiles (tiles w, w + 4,
// ... of the block's range) through a private two-stage LDS ring filled by
// direct global-to-LDS loads, so no block barrier sits inside the tile loop and
// a wave waits only for its own loads.  Per tile a wave computes S^T = K Q^T for
// all eight query rows (four 16x16x32 products) and O^T += V^T P^T over all 128
// value dims (eight 16x16x16 products), keeping its own running maximum, row sum
// and output; the four partial results are merged through LDS at the end.
// ---------------------------------------------------------------------------
constexpr int kFastWaves = 4;
constexpr int kFastThreads = kFastWaves * 64;
constexpr int kFastStages = 2;     // per-wave LDS ring: one tile computed, one in flight
constexpr int kFastMaxEntries = 256;
constexpr float kFastSlack = 8.f;  // log2 headroom of the lazy running maximum

struct __align__(16) FastSmem {
    uint4 kv[kFastWaves][kFastStages][2][16 * 16];  // [wave][stage][K|V][row * 16 + 16-byte piece]
    int32_t erow[kFastMaxEntries];                  // first pool row of each entry's chunk
    uint32_t ebits[kFastMaxEntries];                // membership bits (0: skip the entry)
};

typedef __bf16 bf16x4k_t __attribute__((ext_vector_type(4)));
// D (16x16 fp32) += A (16x16) B (16x16), bf16 operands of four elements per lane
__device__ __forceinline__ f32x4_t mfma16k16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4k_t, a), __builtin_bit_cast(bf16x4k_t, b),
                                                     c, 0, 0, 0);
}

// kTail: the (b, g)'s last range also attends the request's tail rows and the
// step's own rows (masked per key row)
template <bool kTail>
__device__ __forceinline__ void attn_fast_block(const AttnArgs& a, FastSmem& sm, int bg, int split) {
    constexpr int D = 128, G = 4, T = 2, R = G * T, KT = 16, NS = kFastStages;
    constexpr int kRowBytes = D * 2;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;   // matrix-core lane coordinates
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    int u0, u1;
    entry_range(a, bg, split, u0, u1);
    const int tpc = a.chunk / KT;
    const int ntiles = a.pool_blocks > 0 ? (u1 - u0) * tpc : 0;
    // Rows besides the chunks, attended by the (b, g)'s last range: nt rows of
    // the request's tail, then the step's T own rows
    int nt = 0, nx = 0;
    if (kTail && split == a.splits - 1) {
        if (a.Kt) {
            nt = a.tail_len ? a.tail_len[b] : a.tail_max;
            nt = nt < 0 ? 0 : (nt > a.tail_max ? a.tail_max : nt);
        }
        nx = nt + (a.Kn ? T : 0);
    }
    const int ttot = ntiles + (nx + KT - 1) / KT;

    // Query operand of S^T = K Q^T (B of the 16x16x32 product): lane (lr, lg)
    // holds query row lr (token lr / 4, head g * 4 + lr % 4) at dims
    // 32 ks + 8 lg .. + 7; columns 8..15 stay zero.
    const bool qrow = lr < R;
    float4 qf[4][2];
    {
        const int r = qrow ? lr : 0;
        const float* qp = a.q + (((int64_t)b * T + r / G) * a.Hq + g * G + r % G) * D + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qf[ks][0] = qrow ? *reinterpret_cast<const float4*>(qp + 32 * ks) : make_float4(0.f, 0.f, 0.f, 0.f);
            qf[ks][1] = qrow ? *reinterpret_cast<const float4*>(qp + 32 * ks + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    const int32_t* ids = a.block_ids + (int64_t)bg * a.N;
    const uint8_t* mem = a.member + (int64_t)bg * a.N;
    // This block's entries go to LDS, so the tile loop issues no vector loads of
    // its own besides the DMA (keeps the explicit vmcnt accounting exact).
    for (int e = tid; e < u1 - u0; e += kFastThreads) {
        const int c = ids[u0 + e];
        uint32_t m = mem[u0 + e];
        if (c < 0 || c >= a.pool_blocks) m = 0;
        sm.erow[e] = (m ? c : 0) * a.chunk;
        sm.ebits[e] = m;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint4 qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qb[ks] = make_uint4(pack_bf16x2(qf[ks][0].x, qf[ks][0].y), pack_bf16x2(qf[ks][0].z, qf[ks][0].w),
                            pack_bf16x2(qf[ks][1].x, qf[ks][1].y), pack_bf16x2(qf[ks][1].z, qf[ks][1].w));

    // DMA geometry: a wave fills its 16-row K and V tiles with four 1 KiB
    // wave-loads each.  Row r's 16-byte pieces are XOR-swizzled, K by r & 15 and
    // V by 2 (r & 7), so that the matrix-core operand reads below (16 key rows at
    // one K piece; 4 key rows at two adjacent V pieces) hit distinct LDS banks.
    const uint16_t* Kb = (const uint16_t*)a.K + (int64_t)b * a.ks.b + (int64_t)g * a.ks.h;
    const uint16_t* Vb = (const uint16_t*)a.V + (int64_t)b * a.vs.b + (int64_t)g * a.vs.h;
    int koff[4], voff[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int p = jj * 64 + lane;
        const int row = p >> 4, phys = p & 15;
        koff[jj] = row * (int)a.ks.t + (phys ^ (row & 15)) * 8;
        voff[jj] = row * (int)a.vs.t + (phys ^ (2 * (row & 7))) * 8;
    }
    // the wave index as a scalar: the DMA's LDS bases (M0) are then plain SALU math
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const uint16_t* Ktb = (const uint16_t*)a.Kt + (int64_t)b * a.kts.b + (int64_t)g * a.kts.h;
    const uint16_t* Vtb = (const uint16_t*)a.Vt + (int64_t)b * a.vts.b + (int64_t)g * a.vts.h;
    auto issue = [&](int it, int slot) {
        if (!kTail || it < ntiles) {
            const int e = it / tpc;
            const int row0 = sm.erow[e] + (it - e * tpc) * KT;
            const uint16_t* kp = Kb + (int64_t)row0 * a.ks.t;
            const uint16_t* vp = Vb + (int64_t)row0 * a.vs.t;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) lds_dma16(kp + koff[jj], lds_addr(&sm.kv[wu][slot][0][jj * 64]));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) lds_dma16(vp + voff[jj], lds_addr(&sm.kv[wu][slot][1][jj * 64]));
        } else {
            // tail / own rows: each lane addresses its row; rows past nx read
            // row 0 (masked below)
            const int r0 = (it - ntiles) * KT;
            const uint16_t* kp[4];
            const uint16_t* vp[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int p = jj * 64 + lane;
                const int row = p >> 4, phys = p & 15;
                const int xr = r0 + row < nx ? r0 + row : 0;
                const uint16_t* krow;
                const uint16_t* vrow;
                if (xr < nt) {
                    krow = Ktb + (int64_t)xr * a.kts.t;
                    vrow = Vtb + (int64_t)xr * a.vts.t;
                } else {
                    const int64_t off = (((int64_t)b * T + (xr - nt)) * a.Hkv + g) * D;
                    krow = (const uint16_t*)a.Kn + off;
                    vrow = (const uint16_t*)a.Vn + off;
                }
                kp[jj] = krow + (phys ^ (row & 15)) * 8;
                vp[jj] = vrow + (phys ^ (2 * (row & 7))) * 8;
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) lds_dma16(kp[jj], lds_addr(&sm.kv[wu][slot][0][jj * 64]));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) lds_dma16(vp[jj], lds_addr(&sm.kv[wu][slot][1][jj * 64]));
        }
    };
    // Operand reads within a tile (bytes).  K (A of S^T): key lr, logical piece
    // lg + 4 ks.  V (A of O^T = V^T P^T, transposed reads): value dims 16 j + lr,
    // keys 4 lg .. + 3, so that the k-th element of the operand is the key whose
    // weight S^T leaves in element k of the same lane.
    int kro[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kro[ks] = lr * kRowBytes + ((lg + 4 * ks) ^ lr) * 16;
    int vro[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int key = 4 * lg + (lr >> 2);
        const int lp = 2 * j + ((lr & 3) >> 1);
        vro[j] = key * kRowBytes + (lp ^ (2 * (key & 7))) * 16 + 8 * (lr & 1);
    }

    // Running max in log2 units, moved only when a logit exceeds it by more than
    // the slack (weights stay below 2^slack).  It starts at a finite floor far
    // below every logit, so exp2 of (masked logit = -inf) - max is 0 without a
    // guard, and a wave (or range) with no valid key ends with l = 0 (a range
    // reports out 0, lse -inf).
    float m_run = kNoLogit, l_part = 0.f;     // l_part: this lane's share of row lr's sum
    f32x4_t acc[8];                           // O^T: value dims 16 j + 4 lg + i of row lr
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    static_assert(NS == 2, "the waits below count one tile (8 loads) in flight");
    if (w < ttot) issue(w, 0);
    for (int it = w, slot = 0; it < ttot; it += kFastWaves, slot ^= 1) {
        // the other slot was computed in the previous iteration: its reads have
        // returned, so the next tile may overwrite it
        const bool more = it + kFastWaves < ttot;
        if (more) issue(it + kFastWaves, slot ^ 1);
        // tile `it` has landed when at most the 8 loads of the next one are pending
        if (more) lds_dma_wait<8>();
        else lds_dma_wait<0>();
        const bool xtile = kTail && it >= ntiles; // tail / own rows: every query, masked by row
        const uint32_t m_cur = xtile ? 3u : sm.ebits[it / tpc];
        if (m_cur == 0) continue;
        const char* kb = reinterpret_cast<const char*>(sm.kv[wu][slot][0]);
        const char* vb = reinterpret_cast<const char*>(sm.kv[wu][slot][1]);
        uint4 kr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kr[ks] = *reinterpret_cast<const uint4*>(kb + kro[ks]);
        uint2 vr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[j] = lds_read_tr(vb + vro[j]);

        // ---- S^T for all eight query rows: element i of s is key 4 lg + i ----
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s = mfma16(kr[ks], qb[ks], s);

        // ---- online softmax of row lr ----
        const bool on = qrow && ((m_cur >> (lr >> 2)) & 1u);
        float z[4];
        float hm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bool key = true;
            if (xtile) {
                // a tail row is seen by every query, the own row of token t' by
                // the queries of tokens t >= t' (row lr is token lr / 4)
                const int xr = (it - ntiles) * KT + 4 * lg + i;
                key = xr < nt || (xr < nx && xr - nt <= (lr >> 2));
            }
            z[i] = on && key ? s[i] * a.scale_log2 : -INFINITY;
            hm = fmaxf(hm, z[i]);
        }
        hm = group4_max(hm);
        const bool over = hm > m_run + kFastSlack;
        float alpha = 1.f;
        if (over) {
            alpha = __builtin_amdgcn_exp2f(m_run - hm);
            m_run = hm;
        }
        // weights rounded to bf16 (to nearest even); the row sum adds the rounded
        // values the value product uses, so each output stays an exact convex
        // combination of its values
        uint32_t pk[2];
        float ls = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x2_t v = {(__bf16)__builtin_amdgcn_exp2f(z[2 * h] - m_run),
                                (__bf16)__builtin_amdgcn_exp2f(z[2 * h + 1] - m_run)};
            pk[h] = __builtin_bit_cast(uint32_t, v);
            ls += bf16_lo(pk[h]) + bf16_hi(pk[h]);
        }
        l_part = l_part * alpha + ls;
        if (__builtin_amdgcn_ballot_w64(over) != 0ull) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] *= alpha;
        }

        // ---- O^T += V^T P^T over all 128 value dims ----
        const uint2 pb = make_uint2(pk[0], pk[1]);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma16k16(vr[j], pb, acc[j]);
    }
    lds_dma_wait<0>();

    // ---- merge the four waves' (m, l, O) through LDS (the rings, free once
    // every wave is past its last tile); the rows then leave as whole lines, one
    // 16-byte store per thread.  Scattered 4-byte stores of partial lines cost
    // several microseconds per launch at full size.
    const float l_row = group4_sum(l_part);
    __syncthreads();
    float* os = reinterpret_cast<float*>(&sm.kv[0][0][0][0]);   // [wave][R][D]
    float* ml = os + kFastWaves * R * D;                         // [wave][R][2]
    if (qrow) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<float4*>(os + (w * R + lr) * D + 16 * j + 4 * lg) =
                make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
        if (lg == 0) {
            ml[(w * R + lr) * 2] = m_run;
            ml[(w * R + lr) * 2 + 1] = l_row;
        }
    }
    __syncthreads();
    for (int q4 = tid; q4 < R * 32; q4 += kFastThreads) {
        const bool single = a.nparts == 1;
        const int r = q4 >> 5, c4 = q4 & 31;      // 8 rows x 32 float4 (one pass at 256 threads)
        float M = kNoLogit;
#pragma unroll
        for (int ww = 0; ww < kFastWaves; ++ww) M = fmaxf(M, ml[(ww * R + r) * 2]);
        float L = 0.f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ww = 0; ww < kFastWaves; ++ww) {
            const float f = __builtin_amdgcn_exp2f(ml[(ww * R + r) * 2] - M);
            L += ml[(ww * R + r) * 2 + 1] * f;
            const float4 x = *reinterpret_cast<const float4*>(os + (ww * R + r) * D + 4 * c4);
            o.x += x.x * f; o.y += x.y * f; o.z += x.z * f; o.w += x.w * f;
        }
        const int t = r / G, h = g * G + r % G;
        if (single) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
            *reinterpret_cast<float4*>(a.out + (((int64_t)b * T + t) * a.Hq + h) * D + 4 * c4) = o;
            if (c4 == 0 && a.lse)
                a.lse[((int64_t)b * T + t) * a.Hq + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
        } else {
            const int64_t slot = ((int64_t)bg * a.nparts + split) * R + r;
            *reinterpret_cast<float4*>(a.part_acc + slot * D + 4 * c4) = o;
            if (c4 == 0) {
                a.part_ml[slot * 2] = M;
                a.part_ml[slot * 2 + 1] = L;
            }
        }
    }
}

}  // namespace attn
}  // namespace dk
