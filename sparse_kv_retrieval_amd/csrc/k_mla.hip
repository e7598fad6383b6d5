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
// Block (512 threads, 8 waves, two per SIMD): 64 query rows = HB heads x T
// tokens (HB = 64/T) of one (b, g), over one contiguous range of its union
// entries, 32 tokens per tile.  Each SIMD runs one wave of each role, so one
// wave's LDS and DMA waits are covered by the other's matrix work:
//   * S waves (0..3), 16 query rows of one token each: S^T = K Q^T for all 32
//     tokens of the tile (K pieces from LDS as A operands, Q in registers as B
//     operands, 18 k-steps, two token tiles), then the online softmax per row
//     in log2 units inside the wave (a row's 32 weights sit in its 4 lanes) with
//     a lazy running maximum; the weights, rounded to bf16, already have the
//     layout of the B operand of the value product and go to LDS with the
//     per-row rescale factor;
//   * O waves (4..7), value columns 128(w-4) .. +127 of all 64 rows:
//     O^T += V^T P^T with V^T operands from ds_read_b64_tr_b16 (4 tokens x 1
//     column per lane and read, in the weights' token order); they also issue
//     the tile DMAs and the ids DMA.
//   * S of tile i + 1 and O of tile i run in one barrier interval.
// Tiles of 32 latent rows go global -> LDS by DMA into a four-stage ring; an LDS
// row is 1184 bytes (72 pieces + 2 pad), which keeps the key reads (16 lanes =
// 16 rows, one piece) at the full ds_read_b128 rate.  The tile's token ids
// arrive by a dword DMA a tile ahead of its rows, so the only vector-memory
// operations in the loop are DMAs and the wait counts are exact.
// Ranges of one (b, g) are combined by k_mla_merge.  The four row groups of a
// (b, g, range) share an XCD (block id mod 8) so that the other three find the
// tiles in L2.
#include "dk_common.h"

namespace dk {
namespace {

constexpr int kMlaThreads = 512;
constexpr int kMlaRows = 64;              // query rows per block: 16 per S wave
constexpr int kMlaDk = 576, kMlaDv = 512;
constexpr int kMlaTok = 32;               // tokens per tile
constexpr int kMlaPieces = kMlaDk / 8;    // 16-byte pieces per latent row (72)
constexpr int kMlaRowPieces = kMlaPieces + 2;                            // LDS row with its pad (74)
constexpr int kMlaRowBytes = 16 * kMlaRowPieces;                         // 1184
constexpr int kMlaTileBytes = kMlaTok * kMlaRowBytes;                    // 37,888
constexpr int kMlaDmaTotal = kMlaTok * kMlaRowPieces / 64;               // 37 per tile
constexpr int kMlaDmaMax = (kMlaDmaTotal + 3) / 4;                       // O wave 0: 10, others 9
constexpr int kMlaStages = 4;             // tile i in O, i + 1 in S, i + 2 and i + 3 in flight
constexpr int kMlaMaxRange = 2048;        // union entries per block (member bits staged in LDS)
constexpr int kMlaIdSlots = 8;            // ring of tile ids (a tile's ids land 5 tiles before its rows)
constexpr int kMlaColTiles = kMlaDv / 16 / 4;                            // 8 value column tiles per O wave
constexpr float kMlaSlack = 8.f;          // log2 headroom of the lazy running maximum

static_assert(kMlaDmaTotal * 64 == kMlaTok * kMlaRowPieces, "a tile is a whole number of DMAs");

struct __align__(16) MlaSmem {
    uint4 tile[kMlaStages][kMlaTileBytes / 16];
    uint4 p[2][4][4][16];                  // [buffer][row tile][lane group][row]: 8 bf16 weights
    float alpha[2][kMlaRows];              // per-row rescale of the tile's weights
    int flag[2][4];                        // some row of the row tile rescaled
    union {
        int32_t idr[kMlaIdSlots][kMlaTok]; // token ids of a tile, five tiles ahead of its rows
        struct {
            float row_m[kMlaRows];         // after the loop: row statistics
            float row_l[kMlaRows];
        } st;
    } u;
    uint8_t mem[kMlaMaxRange];             // member bits of the range (0: invalid entry)
};

// LDS DMA that keeps the lines in L2 (the other row groups read the same tile)
__device__ __forceinline__ void lds_dma16_keep(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
// the same from a scalar base plus a 32-bit per-lane offset
__device__ __forceinline__ void lds_dma16_keep_off(const void* base, uint32_t off, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_keep(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();
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

// kWide: the latent rows of one (b, g) span 4 GiB or more (64-bit row addresses)
template <bool kWide>
__global__ __launch_bounds__(kMlaThreads) void k_mla_attn(MlaArgs a) {
    __shared__ MlaSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool s_wave = w < 4;
    const int wr = w & 3;                     // row tile (S wave) or column quarter (O wave)
    const int lr = lane & 15, lg = lane >> 4;
    // block -> (b, g), range, row group: every block of one (b, g) has the same
    // blockIdx mod 8, i.e. the same XCD, so the row groups find the tiles and the
    // ranges find the queries in that XCD's L2
    const int blk = blockIdx.x;
    const int n_per = a.splits * a.rgroups;
    const int bg = (blk / (8 * n_per)) * 8 + (blk % 8);
    const int kq = (blk / 8) % n_per;
    const int split = kq / a.rgroups, rg = kq - split * a.rgroups;
    if (bg >= a.B * a.Hkv) return;
    const int f = bg * a.splits + split;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int T = a.T, HB = kMlaRows / T, G = a.Hq / a.Hkv;

    // entries of this range
    const int cnt = __builtin_amdgcn_readfirstlane(max(0, min(a.count[bg], a.N)));
    const int per = (cnt + a.splits - 1) / a.splits;
    const int u0 = min(cnt, split * per);
    const int u1 = min(min(cnt, u0 + per), u0 + kMlaMaxRange);   // the plan keeps per <= kMlaMaxRange
    const int n_ent = u1 - u0;
    const int ntiles = (n_ent + kMlaTok - 1) / kMlaTok;
    const int32_t* ids = a.ids + (int64_t)bg * a.N + u0;
    const uint8_t* mem = a.member ? a.member + (int64_t)bg * a.N + u0 : nullptr;
    const char* lat_bg = (const char*)(a.lat + (int64_t)b * a.ks.b + (int64_t)g * a.ks.h);
    const int64_t row_bytes = a.ks.t * 2;
    const int L = a.L;

    // ---- O waves: tile DMAs.  DMA i of a tile lands LDS pieces 64i .. 64i + 63:
    // row pos / 74, piece pos % 74 (72, 73: the pad, loaded from the row start);
    // O wave wr issues i = wr, wr + 4, ...
    int dsel[kMlaDmaMax];                     // row << 16 | byte offset in the row
#pragma unroll
    for (int c = 0; c < kMlaDmaMax; ++c) {
        const int pos = 64 * (wr + 4 * c) + lane;
        const int j = pos / kMlaRowPieces, qp = pos - j * kMlaRowPieces;
        dsel[c] = (min(j, kMlaTok - 1) << 16) | (qp < kMlaPieces ? 16 * qp : 0);
    }
    // the token ids of tile x into u.idr[x % 8] (lanes 0..31 of one O wave;
    // entries past the range repeat the last one, and the rows' member bits
    // mask them out)
    auto issue_ids = [&](int x) {
        if (lane < kMlaTok)
            lds_dma4_keep(ids + min(x * kMlaTok + lane, n_ent - 1), lds_addr(&sm.u.idr[x % kMlaIdSlots][0]));
    };
    // rows of a tile: the ids of this lane's rows from LDS, then DMA c (invalid
    // ids read row 0, masked out by their bits)
    auto read_ids = [&](int x, int (&id)[kMlaDmaMax]) {
#pragma unroll
        for (int c = 0; c < kMlaDmaMax; ++c) id[c] = sm.u.idr[x % kMlaIdSlots][dsel[c] >> 16];
    };
    const uint32_t row_bytes32 = (uint32_t)row_bytes;
    auto issue_one = [&](int c, int stage, const int (&id)[kMlaDmaMax]) {
        const int i = wr + 4 * c;
        if (i < kMlaDmaTotal) {
            const int v = (id[c] < 0 || id[c] >= L) ? 0 : id[c];
            const uint32_t lds = lds_addr(&sm.tile[stage][0]) + 1024u * (uint32_t)i;
            if (kWide)
                lds_dma16_keep(lat_bg + (int64_t)v * row_bytes + (dsel[c] & 0xffff), lds);
            else
                lds_dma16_keep_off(lat_bg, __umul24((uint32_t)v, row_bytes32) + (uint32_t)(dsel[c] & 0xffff), lds);
        }
    };
    auto issue_tile = [&](int x, int stage) {
        int id[kMlaDmaMax];
        read_ids(x, id);
#pragma unroll
        for (int c = 0; c < kMlaDmaMax; ++c) issue_one(c, stage, id);
    };
    // ---- prologue.  O waves: each fetches the ids of tiles 0..4 itself (the
    // four write the same values) and issues tiles 0..2 as soon as its own have
    // landed.  S waves: the member bits and the queries meanwhile.
    if (!s_wave) {
#pragma unroll
        for (int x = 0; x < 5; ++x)
            if (x < ntiles) issue_ids(x);
    }
    constexpr int kStage = kMlaMaxRange / (kMlaThreads / 2);   // entries per S-wave thread
    int sv[kStage], sb[kStage];
    if (s_wave) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int x = min(tid + (kMlaThreads / 2) * i, max(n_ent - 1, 0));
            sv[i] = n_ent > 0 ? ids[x] : 0;
            sb[i] = mem && n_ent > 0 ? (int)mem[x] : 0xff;
        }
    }
    constexpr float kLn2 = 0.69314718055994531f;

    // The two roles run separate loops with the same sequence of barriers:
    // (1) bits staged and tile 0 landed, one per iteration, (2) row statistics
    // published.
    if (s_wave) {
        // ---- S wave: rows 16wr .. 16wr + 15 (one query token)
        const int t_w = (16 * wr) / HB;
        const int h_lane = g * G + rg * HB + (16 * wr) % HB + lr;   // head of row lane%16
        // the queries: issued after the bits, converted as the first tile's
        // k-steps need them (S waves issue no DMAs, so the compiler's own wait
        // counts are exact here)
        uint4 qa[18];
        {
            const float* qrow = a.q + (((int64_t)b * T + t_w) * a.Hq + h_lane) * kMlaDk + 8 * lg;
#pragma unroll
            for (int s = 0; s < 18; ++s) {
                const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * s);
                const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * s + 4);
                qa[s] = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                                   pack_bf16x2(x1.z, x1.w));
            }
        }
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int x = tid + (kMlaThreads / 2) * i;
            if (x < n_ent) sm.mem[x] = (uint8_t)((sv[i] < 0 || sv[i] >= L) ? 0 : sb[i]);
        }
        // key piece 4s + lg of row 16tt + lr
        const int koff = lr * kMlaRowBytes + 16 * lg;
        float m_run = -INFINITY, l_part = 0.f;
        // S^T of tile x, mask, lazy-maximum softmax, weights to LDS
        auto s_tile = [&](int x) {
            const char* st = reinterpret_cast<const char*>(&sm.tile[x % kMlaStages][0]) + koff;
            uint32_t mb[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                mb[tt] = *reinterpret_cast<const uint32_t*>(&sm.mem[x * kMlaTok + 16 * tt + 4 * lg]);
            f32x4_t sacc[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}},
                                  {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
            // groups of two k-steps x two token tiles; operands read kAhead groups
            // ahead (the schedule barriers keep the compiler from sinking them).

            constexpr int kAhead = 3;
            uint4 kb[kAhead + 1][4];
#pragma unroll
            for (int gq = 0; gq < kAhead; ++gq)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    kb[gq][u] = *reinterpret_cast<const uint4*>(st + 64 * (2 * gq + (u >> 1)) +
                                                                (u & 1) * 16 * kMlaRowBytes);
#pragma unroll
            for (int gq = 0; gq < 9; ++gq) {
                if (gq + kAhead < 9) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        kb[(gq + kAhead) % (kAhead + 1)][u] = *reinterpret_cast<const uint4*>(
                            st + 64 * (2 * (gq + kAhead) + (u >> 1)) + (u & 1) * 16 * kMlaRowBytes);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s = 2 * gq + (u >> 1), tt = u & 1;
                    sacc[tt][s & 1] = mfma16(kb[gq % (kAhead + 1)][u], qa[s], sacc[tt][s & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            const int buf = x & 1;
            float z[2][4];
            float hm = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int e0 = x * kMlaTok + 16 * tt + 4 * lg;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t valid = (uint32_t)(e0 + e < n_ent) & (mb[tt] >> (8 * e + t_w));
                    const float zs = (sacc[tt][0][e] + sacc[tt][1][e]) * a.scale_log2;
                    z[tt][e] = (valid & 1u) ? zs : -INFINITY;
                    hm = fmaxf(hm, z[tt][e]);
                }
            }
            hm = group4_max(hm);
            // the reference moves only when a logit exceeds it by more than the
            // slack (the result does not depend on it; weights stay below 2^slack)
            const bool over = hm > m_run + kMlaSlack;     // also any finite logit while m_run is -inf
            float alpha = 1.f;
            if (over) {
                alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - hm);
                m_run = hm;
            }
            // weights rounded to bf16 (v_cvt_pk_bf16_f32, to nearest even); the row
            // sum adds the rounded values the value product uses
            uint32_t pk[4];
            float ls = 0.f;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float z0 = z[h >> 1][2 * (h & 1)], z1 = z[h >> 1][2 * (h & 1) + 1];
                const float p0 = z0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z0 - m_run);
                const float p1 = z1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z1 - m_run);
                const bf16x2_t v = {(__bf16)p0, (__bf16)p1};
                pk[h] = __builtin_bit_cast(uint32_t, v);
                ls += __uint_as_float(pk[h] << 16) + __uint_as_float(pk[h] & 0xffff0000u);
            }
            l_part = l_part * alpha + ls;
            sm.p[buf][wr][lg][lr] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            if (lg == 0) sm.alpha[buf][16 * wr + lr] = alpha;
            const uint64_t anyover = __ballot(over);
            if (lane == 0) sm.flag[buf][wr] = anyover != 0;
        };

        lds_barrier();                                // (1)
        if (ntiles > 0) s_tile(0);
        for (int it = 0; it < ntiles; ++it) {
            lds_barrier();
            if (it + 1 < ntiles) s_tile(it + 1);
        }
        const float l_row = group4_sum(l_part);
        if (lg == 0) {
            const int r = 16 * wr + lr;
            sm.u.st.row_m[r] = m_run;
            sm.u.st.row_l[r] = l_row;
            const int t = r / HB, h = g * G + rg * HB + r % HB;
            if (a.splits == 1) {
                if (a.lse)
                    a.lse[((int64_t)b * T + t) * a.Hq + h] = l_row > 0.f ? m_run * kLn2 + logf(l_row) : -INFINITY;
            } else {
                float* pml = a.part_ml + ((int64_t)f * a.rgroups + rg) * kMlaRows * 2;
                pml[2 * r] = m_run;
                pml[2 * r + 1] = l_row;
            }
        }
        lds_barrier();                                // (2)
    } else {
        // ---- O wave: value columns 128wr .. 128wr + 127 of all 64 rows
        // transposed value reads: lane i of group lg addresses row 4lg + i/4 (and
        // 16 more), columns 128wr + 16ct + 4(i%4) .. +3
        const int voff = (4 * lg + (lr >> 2)) * kMlaRowBytes + 256 * wr + 8 * (lr & 3);
        const bool dma10 = wr == 0;           // O wave 0 issues 10 DMAs per tile, the others 9
        f32x4_t acc[4][kMlaColTiles];         // rows 16rt + lr, columns 128wr + 16ct + 4lg + e
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < kMlaColTiles; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // O^T of tile y; with dma, tile y + 3's rows are issued first: the DMA
        // queue drains while the S wave of this SIMD holds the matrix core, and
        // the products here then run beside that wave's softmax
        auto o_tile = [&](int y, bool dma, const int (&id)[kMlaDmaMax]) {
            const int dstage = (y + 3) % kMlaStages;
            const int buf = y & 1;
            const char* st = reinterpret_cast<const char*>(&sm.tile[y % kMlaStages][0]) + voff;
            const int4 fl = *reinterpret_cast<const int4*>(&sm.flag[buf][0]);
            uint4 pb[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) pb[rt] = sm.p[buf][rt][lg][lr];
            uint2 vb[3][2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                vb[ct][0] = lds_read_tr(st + 32 * ct);
                vb[ct][1] = lds_read_tr(st + 32 * ct + 16 * kMlaRowBytes);
            }
            if (dma) {
#pragma unroll
                for (int c = 0; c < kMlaDmaMax; ++c) issue_one(c, dstage, id);
            }
            if ((fl.x | fl.y | fl.z | fl.w) != 0) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const float al = sm.alpha[buf][16 * rt + lr];
#pragma unroll
                    for (int ct = 0; ct < kMlaColTiles; ++ct) acc[rt][ct] *= al;
                }
            }
#pragma unroll
            for (int ct = 0; ct < kMlaColTiles; ++ct) {
                if (ct + 2 < kMlaColTiles) {
                    vb[(ct + 2) % 3][0] = lds_read_tr(st + 32 * (ct + 2));
                    vb[(ct + 2) % 3][1] = lds_read_tr(st + 32 * (ct + 2) + 16 * kMlaRowBytes);
                }
                const uint4 va = make_uint4(vb[ct % 3][0].x, vb[ct % 3][0].y, vb[ct % 3][1].x, vb[ct % 3][1].y);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) acc[rt][ct] = mfma16(va, pb[rt], acc[rt][ct]);
            }
        };

        vm_wait<0>();                                 // this wave's ids of tiles 0..4 landed
#pragma unroll
        for (int x = 0; x < 3; ++x)
            if (x < ntiles) issue_tile(x, x);
        int id[kMlaDmaMax];                           // ids of the rows of tile it + 3
        if (3 < ntiles) read_ids(3, id);
        if (ntiles > 2) {
            if (dma10) vm_wait<2 * kMlaDmaMax>(); else vm_wait<2 * (kMlaDmaMax - 1)>();
        } else if (ntiles > 1) {
            if (dma10) vm_wait<kMlaDmaMax>(); else vm_wait<kMlaDmaMax - 1>();
        } else {
            vm_wait<0>();
        }
        lds_barrier();                                // (1)
        // O of tile it runs beside S of tile it + 1.  At the top of iteration it
        // the DMAs of tiles it + 1 and it + 2 may be outstanding (and, issued
        // before tile it + 2's rows, tile it + 4's ids); tile it + 1 and those ids
        // are complete once only tile it + 2's rows remain.  The barrier also
        // publishes tile it's weights and frees the stage of tile it - 1, which
        // receives tile it + 3; tile it + 5's ids go to the slot of tile it - 3.
        // Tile it + 4's ids are read at the end of the iteration, for the next.
        for (int it = 0; it < ntiles; ++it) {
            if (it + 2 < ntiles) {
                if (dma10) vm_wait<kMlaDmaMax>(); else vm_wait<kMlaDmaMax - 1>();
            } else {
                vm_wait<0>();
            }
            lds_barrier();
            if (it + 5 < ntiles && wr == 0) issue_ids(it + 5);
            o_tile(it, it + 3 < ntiles, id);
            if (it + 4 < ntiles) read_ids(it + 4, id);
        }
        lds_barrier();                                // (2)
        if (a.splits == 1) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r = 16 * rt + lr;
                const int t = r / HB, h = g * G + rg * HB + r % HB;
                const float l = sm.u.st.row_l[r];
                const float inv = l > 0.f ? 1.f / l : 0.f;
                float* orow = a.out + (((int64_t)b * T + t) * a.Hq + h) * kMlaDv + 128 * wr + 4 * lg;
#pragma unroll
                for (int ct = 0; ct < kMlaColTiles; ++ct)
                    *reinterpret_cast<float4*>(orow + 16 * ct) =
                        make_float4(acc[rt][ct][0] * inv, acc[rt][ct][1] * inv, acc[rt][ct][2] * inv,
                                    acc[rt][ct][3] * inv);
            }
        } else {
            float* po = a.part_o + ((int64_t)f * a.rgroups + rg) * kMlaRows * kMlaDv;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                float* prow = po + (int64_t)(16 * rt + lr) * kMlaDv + 128 * wr + 4 * lg;
#pragma unroll
                for (int ct = 0; ct < kMlaColTiles; ++ct)
                    *reinterpret_cast<float4*>(prow + 16 * ct) =
                        make_float4(acc[rt][ct][0], acc[rt][ct][1], acc[rt][ct][2], acc[rt][ct][3]);
            }
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
    // one block per CU (the LDS ring takes the CU's LDS), at least two tiles per range
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
    const unsigned grid = (unsigned)(((B * Hkv + 7) / 8) * 8 * plan.splits * plan.rgroups);
    // row offsets fit 32 bits unless one (b, g)'s rows span 4 GiB
    const bool wide = (int64_t)L * ks.t * 2 >= (int64_t(1) << 32);
    if (wide)
        hipLaunchKernelGGL(k_mla_attn<true>, dim3(grid), dim3(kMlaThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_mla_attn<false>, dim3(grid), dim3(kMlaThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const int rows = B * Hkv * plan.rgroups * kMlaRows;
    hipLaunchKernelGGL(k_mla_merge, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace dk
