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
// Block (256 threads, 4 waves): 64 query rows = HB heads x T tokens (HB = 64/T)
// of one (b, g), over one contiguous range of its union entries, 32 tokens per
// tile.
//   * tiles of 32 latent rows (36 KiB) go global -> LDS by DMA into a two-stage
//     ring; 16-byte pieces are XOR-swizzled by token so that both the key reads
//     (16 bytes per lane) and the value reads (2 bytes per lane) spread over the
//     banks;
//   * S = Q K^T: wave w owns rows 16w..16w+15 (one query token), Q in registers
//     as bf16 A operands, K pieces from LDS as B operands, 18 k-steps x 2 token
//     groups;
//   * online softmax in log2 units per row (mask: the token is in the row's own
//     set), weights rounded to bf16 into LDS;
//   * O += P V: wave w owns value columns 128w..128w+127 for all 64 rows, P rows
//     from LDS as A operands, value columns gathered from the same LDS tile.
// Ranges of one (b, g) are combined by k_mla_merge.  The four row groups of a
// (b, g, range) share an XCD (block id mod 8) so that the other three find the
// tiles in L2.
#include "dk_common.h"

namespace dk {
namespace {

constexpr int kMlaThreads = 256;
constexpr int kMlaRows = 64;              // query rows per block
constexpr int kMlaDk = 576, kMlaDv = 512;
constexpr int kMlaTok = 32;               // tokens per tile
constexpr int kMlaPieces = kMlaDk / 8;    // 16-byte pieces per latent row (72)
constexpr int kMlaTileBytes = kMlaTok * kMlaPieces * 16;   // 36864
constexpr int kMlaDmaPerWave = kMlaTok * kMlaPieces / 64 / 4;   // 9
constexpr int kPRow = 40;                 // bf16 per row of the P tile (80 bytes)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct __align__(16) MlaSmem {
    uint4 tile[2][kMlaTok * kMlaPieces];   // latent rows, swizzled pieces
    uint16_t p[kMlaRows * kPRow];          // bf16 weights [row][token]
    float alpha[kMlaRows];                 // per-row rescale of this tile
    float row_m[kMlaRows];
    float row_l[kMlaRows];
    int flag[4];
};

__device__ __forceinline__ int mla_swz(int j) { return (j ^ (j >> 3)) & 7; }

// LDS DMA that keeps the lines in L2 (the other row groups read the same tile)
__device__ __forceinline__ void lds_dma16_keep(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
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
    // block -> (work item f, row group rg); the row groups of f share blockIdx mod 8
    const int blk = blockIdx.x;
    const int f = (blk / (8 * a.rgroups)) * 8 + (blk % 8);
    const int rg = (blk / 8) % a.rgroups;
    if (f >= a.work) return;
    const int split = f % a.splits;
    const int bg = f / a.splits;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int T = a.T, HB = kMlaRows / T, G = a.Hq / a.Hkv;
    const int t_w = (16 * w) / HB;                           // this wave's query token
    const int h_lane = g * G + rg * HB + (16 * w) % HB + (lane & 15);   // head of row lane%16

    // entries of this range
    const int cnt = max(0, min(a.count[bg], a.N));
    const int per = (cnt + a.splits - 1) / a.splits;
    const int u0 = min(cnt, split * per), u1 = min(cnt, u0 + per);
    const int ntiles = (u1 - u0 + kMlaTok - 1) / kMlaTok;
    const int32_t* ids = a.ids + (int64_t)bg * a.N;
    const uint8_t* mem = a.member ? a.member + (int64_t)bg * a.N : nullptr;
    const char* lat_bg = (const char*)(a.lat + (int64_t)b * a.ks.b + (int64_t)g * a.ks.h);
    const int64_t row_bytes = a.ks.t * 2;

    // per-lane token of a tile: lane < 32 holds token `lane`
    auto load_tok = [&](int tile, int& id, int& mb) {
        const int e = u0 + tile * kMlaTok + (lane & 31);
        const int ec = e < u1 ? e : u0;          // a valid entry, or the first one
        int v = (u1 > u0) ? ids[ec] : 0;
        int m = (u1 > u0) ? (mem ? (int)mem[ec] : 0xff) : 0;
        if (e >= u1 || lane >= 32 || v < 0 || v >= a.L) {
            v = 0;
            m = 0;
        }
        id = v;
        mb = m;
    };
    auto issue_tile = [&](int tile_id_reg, int buf) {
        const uint32_t base = lds_addr(&sm.tile[buf][0]);
#pragma unroll
        for (int c = 0; c < kMlaDmaPerWave; ++c) {
            const int i = w + 4 * c;                 // DMA instruction (wave-uniform)
            const int pos = 64 * i + lane;           // piece position in the tile
            const int j = pos / kMlaPieces, qp = pos - j * kMlaPieces;
            const int piece = qp ^ mla_swz(j);
            const int id = __shfl(tile_id_reg, j, kWave);
            lds_dma16_keep(lat_bg + (int64_t)id * row_bytes + piece * 16, base + 1024u * (uint32_t)i);
        }
    };

    // ---- prologue: union entries of tiles 0 and 1, the queries, tile 0
    int id_c, mem_c, id_n1, mem_n1;
    load_tok(0, id_c, mem_c);
    load_tok(1, id_n1, mem_n1);
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
    if (ntiles > 0) issue_tile(id_c, 0);

    float m_run[4], l_run[4];
    f32x4_t acc[4][8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        m_run[e] = -INFINITY;
        l_run[e] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Ordering of the vector-memory queue: the entries of tile it + 1 are loaded
    // at the end of iteration it - 1, so using them for the DMA of tile it + 1
    // makes the compiler wait for every earlier load, tile it's DMA included;
    // the DMA of tile it + 1 then runs under the compute of tile it.
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntiles) {
            issue_tile(id_n1, buf ^ 1);
            vm_wait<kMlaDmaPerWave>();               // all but tile it + 1: tile it has landed
        } else {
            vm_wait<0>();
        }
        lds_barrier();

        // ---- S = Q K^T for this wave's 16 rows and the tile's 32 tokens
        const uint4* tl = sm.tile[buf];
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        const int j0 = lane & 15, j1 = 16 + (lane & 15);
        const int sw0 = mla_swz(j0), sw1 = mla_swz(j1);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
            const int piece = 4 * s + (lane >> 4);
            const uint4 k0 = tl[j0 * kMlaPieces + (piece ^ sw0)];
            const uint4 k1 = tl[j1 * kMlaPieces + (piece ^ sw1)];
            s0 = mfma16(qa[s], k0, s0);
            s1 = mfma16(qa[s], k1, s1);
        }
        // ---- mask, online softmax (log2 units), bf16 weights to LDS
        const int mb0 = __shfl(mem_c, j0, kWave), mb1 = __shfl(mem_c, j1, kWave);
        const bool v0 = (mb0 >> t_w) & 1, v1 = (mb1 >> t_w) & 1;
        bool moved = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float z0 = v0 ? s0[e] * a.scale_log2 : -INFINITY;
            const float z1 = v1 ? s1[e] * a.scale_log2 : -INFINITY;
            const float mx = dpp_group_max16(fmaxf(z0, z1));
            const float mn = fmaxf(m_run[e], mx);
            float alpha = 1.f, p0 = 0.f, p1 = 0.f;
            if (mn != -INFINITY) {
                alpha = exp2f(m_run[e] - mn);
                p0 = exp2f(z0 - mn);
                p1 = exp2f(z1 - mn);
            }
            const uint32_t pb0 = f32_to_bf16_rne(p0), pb1 = f32_to_bf16_rne(p1);
            const float ps = __uint_as_float(pb0 << 16) + __uint_as_float(pb1 << 16);
            l_run[e] = l_run[e] * alpha + dpp_group_sum<16>(ps);
            m_run[e] = mn;
            moved |= alpha != 1.f;
            const int r = 16 * w + 4 * (lane >> 4) + e;
            sm.p[r * kPRow + j0] = (uint16_t)pb0;
            sm.p[r * kPRow + j1] = (uint16_t)pb1;
            if ((lane & 15) == 0) sm.alpha[r] = alpha;
        }
        const uint64_t anymove = __ballot(moved);
        if (lane == 0) sm.flag[w] = anymove != 0;
        lds_barrier();

        // ---- O += P V for value columns 128w .. 128w+127 of all 64 rows
        if (sm.flag[0] | sm.flag[1] | sm.flag[2] | sm.flag[3]) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[16 * m + 4 * (lane >> 4)]);
#pragma unroll
                for (int n = 0; n < 8; ++n) {
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
        const uint16_t* tb = reinterpret_cast<const uint16_t*>(tl);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int col = 128 * w + 16 * n + (lane & 15);
            const int cp = col >> 3, ce = col & 7;
            uint16_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 8 * (lane >> 4) + e;
                v[e] = tb[(j * kMlaPieces + (cp ^ mla_swz(j))) * 8 + ce];
            }
            const uint4 vb = make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                                        v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16));
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m][n] = mfma16(pa[m], vb, acc[m][n]);
        }
        int id_n2, mem_n2;
        load_tok(it + 2, id_n2, mem_n2);
        lds_barrier();
        id_n1 = id_n2;
        mem_c = mem_n1;
        mem_n1 = mem_n2;
    }

    // ---- row statistics to every wave, then this wave's columns of all rows
    if ((lane & 15) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * w + 4 * (lane >> 4) + e;
            sm.row_m[r] = m_run[e];
            sm.row_l[r] = l_run[e];
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    constexpr float kLn2 = 0.69314718055994531f;
    if (a.splits == 1) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * m + 4 * (lane >> 4) + e;
                const int t = r / HB, h = g * G + rg * HB + r % HB;
                const float l = sm.row_l[r];
                const float inv = l > 0.f ? 1.f / l : 0.f;
                float* orow = a.out + (((int64_t)b * T + t) * a.Hq + h) * kMlaDv + 128 * w + (lane & 15);
#pragma unroll
                for (int n = 0; n < 8; ++n) orow[16 * n] = acc[m][n][e] * inv;
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
                float* prow = po + (int64_t)r * kMlaDv + 128 * w + (lane & 15);
#pragma unroll
                for (int n = 0; n < 8; ++n) prow[16 * n] = acc[m][n][e];
            }
        }
        if (w == 0) {
            float* pml = a.part_ml + slot * kMlaRows * 2;
            pml[2 * lane] = sm.row_m[lane];
            pml[2 * lane + 1] = sm.row_l[lane];
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
