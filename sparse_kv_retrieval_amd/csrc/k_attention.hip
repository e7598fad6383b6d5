// Sparse decode attention of both queries in one pass over the union.
//
// DualDecoder (arXiv 2607.26475), "4.2" and "5.3": the result must equal
// attention over the true retrieval index; "5.2" and "6.4": the real and the
// speculative token share one attention launch.  Adaptive DHiSparse Figure 3
// (2): each query attends over its own selection, so a union chunk is masked out
// for a query whose membership bit is clear.
//
// Split-K flash decoding: a block owns one (b, g) and one contiguous range of
// its union entries (the ranges split the entry count evenly, so the work
// follows the ragged union sizes), keeps a running max m, sum l and weighted
// value sum per query row, and either writes the normalised result (one range)
// or its (m, l, acc) partial for k_attn_merge, which combines the ranges with
// the online-softmax rule.  Logits are kept in log2 units (scale * log2 e).
//
// Fast path (bf16 K/V, d = 128, G = 4, T = 2, chunk a multiple of 32): four
// independent waves per block, each over its own 16-row tiles of K and V
// (every fourth tile of the block's range) that stream from HBM straight into a
// private two-stage LDS ring with global_load_lds_dwordx4 (non-temporal; no
// register staging), so no block barrier sits in the tile loop and each tile is
// read from HBM once for all eight query rows.  Both products run on the matrix
// cores with the keys along M: S^T = K Q^T (v_mfma_f32_16x16x32_bf16) gives
// every lane one query row's logits of four keys; after the online-softmax step
// those weights, rounded to bf16, are already the B operand of O^T = V^T P^T
// (v_mfma_f32_16x16x16_bf16), whose A operand comes from transposed LDS reads of
// V (ds_read_b64_tr_b16).  Each wave keeps its own running max, sums and all 128
// value dims; the four partial results are merged through LDS at the end.  K
// and V pieces are XOR-swizzled by row in LDS so that the operand reads hit
// distinct banks.  The running max moves only when a logit exceeds it by a
// slack, so most tiles need no rescale; the row sums use the rounded weights,
// so each output stays an exact convex combination of its values.
//
// Rows besides the chunks (dk_sparse_decode_attn_tail: a request's tail rows
// and the step's own rows, causally masked): on the fast path the last range of
// each (b, g) streams them as extra tiles of the same loop, masked per key row,
// so they need no partial of their own; elsewhere k_attn_tail writes them as
// one more partial for the merge.
#include "dk_attn_fast.h"

namespace dk {
using namespace attn;
namespace {

constexpr int kThreads = 256;

// Write one query row's result: normalised output (single range) or its partial.
template <int D>
__device__ __forceinline__ void emit_row(const AttnArgs& a, int b, int bg, int split, int t, int h,
                                         int r, int R, float m, float l, const float* acc,
                                         int dim0, int ndim, bool lead) {
    if (a.nparts == 1) {
        float* o = a.out + (((int64_t)b * a.T + t) * a.Hq + h) * D + dim0;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        for (int e = 0; e < ndim; ++e) o[e] = acc[e] * inv;
        if (lead && a.lse)
            a.lse[((int64_t)b * a.T + t) * a.Hq + h] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    } else {
        const int64_t slot = ((int64_t)bg * a.nparts + split) * R + r;
        float* p = a.part_acc + slot * D + dim0;
        for (int e = 0; e < ndim; ++e) p[e] = acc[e];
        if (lead) {
            a.part_ml[slot * 2] = m;
            a.part_ml[slot * 2 + 1] = l;
        }
    }
}

// The fast path's kernel: one (b, g) range per block (the body lives in
// dk_attn_fast.h, shared with the fused decode-step kernel).
template <bool kTail>
__global__ __launch_bounds__(kFastThreads) void k_attn_bf16_d128_g4t2(AttnArgs a) {
    __shared__ FastSmem sm;
    int bg, split;
    xcd_unit(blockIdx.x, a.splits, gridDim.x / a.splits, bg, split);
    attn_fast_block<kTail>(a, sm, bg, split);
}

// ---------------------------------------------------------------------------
// Generic path: fp32 or bf16 K/V, D in {64, 128}, any G*T <= 16, any chunk.
// Correct and simple; used off the fast path's shapes.
// ---------------------------------------------------------------------------
// One tile of up to TR K and V rows staged through registers: every thread
// issues all of its 16-byte loads before any is waited on, so a tile costs one
// memory latency; the values are widened to fp32 when written to LDS.  K rows
// in LDS are padded to D + 4 floats (16-byte aligned rows, float4 reads spread
// over the banks).
template <typename KVT, int D, int TR>
struct TileRegs {
    static constexpr int kEpv = 16 / (int)sizeof(KVT);          // elements per 16-byte vector
    static constexpr int kVpr = D / kEpv;                        // vectors per row
    static constexpr int kPer = (TR * kVpr + kThreads - 1) / kThreads;
    uint4 k[kPer], v[kPer];
};

struct RowPair {
    const void* k;
    const void* v;
};

// rows(rr) gives the addresses of K and V row rr of the tile (16-byte aligned)
template <typename KVT, int D, int TR, typename Rows>
__device__ __forceinline__ void tile_load(TileRegs<KVT, D, TR>& t, int nr, Rows rows) {
    using TT = TileRegs<KVT, D, TR>;
#pragma unroll
    for (int p = 0; p < TT::kPer; ++p) {
        const int i = threadIdx.x + p * kThreads;
        const int rr = i / TT::kVpr, x = i - rr * TT::kVpr;
        if (rr < nr) {
            const RowPair rp = rows(rr);
            t.k[p] = ((const uint4*)rp.k)[x];
            t.v[p] = ((const uint4*)rp.v)[x];
        }
    }
}

__device__ __forceinline__ void widen(const uint4& u, float* f, uint16_t) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(w[j] << 16);
        f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen(const uint4& u, float* f, float) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
}

template <typename KVT, int D, int TR>
__device__ __forceinline__ void tile_store(const TileRegs<KVT, D, TR>& t, int nr, float (*kt)[D + 4],
                                           float (*vt)[D]) {
    using TT = TileRegs<KVT, D, TR>;
    constexpr int E = TT::kEpv;
#pragma unroll
    for (int p = 0; p < TT::kPer; ++p) {
        const int i = threadIdx.x + p * kThreads;
        const int rr = i / TT::kVpr, x = i - rr * TT::kVpr;
        if (rr < nr) {
            float f[E];
            widen(t.k[p], f, KVT{});
#pragma unroll
            for (int e = 0; e < E; e += 4) *(float4*)&kt[rr][x * E + e] = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
            widen(t.v[p], f, KVT{});
#pragma unroll
            for (int e = 0; e < E; e += 4) *(float4*)&vt[rr][x * E + e] = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
        }
    }
}

// One tile of nr (<= TR) key rows already in kt / vt.  Wave w owns query rows
// r = w + 4x (x < XR): it computes their logits with one lane per key row, so a
// K row is read from LDS once for all of the wave's rows, updates (m, l, acc)
// by online softmax, and forms the weighted value sum, reading each V row once
// for all of its rows.  The probabilities pass through the wave's own zs rows,
// four per LDS read.  vis(r, jj) says whether query row r may use key row jj.
// Only the wave's own LDS rows are written: no block barrier inside.
template <int D, int TR, int XR, typename Vis>
__device__ __forceinline__ void attend_tile(const AttnArgs& a, int nr, const float (*qs)[D],
                                            const float (*kt)[D + 4], const float (*vt)[D], float (*zs)[TR],
                                            Vis vis, float* m_run, float* l_run, float (*acc)[D / kWave]) {
    static_assert(TR == 32 || TR == 64, "tile rows");
    constexpr int DPL = D / kWave;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float s[XR][4];
#pragma unroll
    for (int x = 0; x < XR; ++x)
#pragma unroll
        for (int c = 0; c < 4; ++c) s[x][c] = 0.f;
    const int jr = lane < nr ? lane : 0;       // lanes past the tile are masked below
#pragma unroll 4
    for (int dd = 0; dd < D; dd += 4) {
        const float4 kv = *(const float4*)&kt[jr][dd];
#pragma unroll
        for (int x = 0; x < XR; ++x) {
            const float4 qv = *(const float4*)&qs[w + 4 * x][dd];
            s[x][0] = fmaf(qv.x, kv.x, s[x][0]);
            s[x][1] = fmaf(qv.y, kv.y, s[x][1]);
            s[x][2] = fmaf(qv.z, kv.z, s[x][2]);
            s[x][3] = fmaf(qv.w, kv.w, s[x][3]);
        }
    }
#pragma unroll
    for (int x = 0; x < XR; ++x) {
        const int r = w + 4 * x;
        float z = ((s[x][0] + s[x][1]) + (s[x][2] + s[x][3])) * a.scale_log2;
        if (!(lane < nr && vis(r, lane))) z = -INFINITY;
        float cm = z;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off, kWave));
        const float mn = fmaxf(m_run[x], cm);
        const float alpha = mn == -INFINITY ? 1.f : exp2f(m_run[x] - mn);
        const float p = mn == -INFINITY ? 0.f : exp2f(z - mn);
        float ps = p;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) ps += __shfl_xor(ps, off, kWave);
        l_run[x] = l_run[x] * alpha + ps;
        m_run[x] = mn;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[x][e] *= alpha;
        if (lane < TR) zs[r][lane] = p;
    }
    __builtin_amdgcn_wave_barrier();
    for (int j4 = 0; j4 < nr; j4 += 4) {
        float pj[XR][4];
#pragma unroll
        for (int x = 0; x < XR; ++x) {
            const float4 p4 = *(const float4*)&zs[w + 4 * x][j4];
            pj[x][0] = p4.x;
            pj[x][1] = p4.y;
            pj[x][2] = p4.z;
            pj[x][3] = p4.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (j4 + q < nr) {
                float v[DPL];
#pragma unroll
                for (int e = 0; e < DPL; ++e) v[e] = vt[j4 + q][lane * DPL + e];
#pragma unroll
                for (int x = 0; x < XR; ++x)
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[x][e] = fmaf(pj[x][q], v[e], acc[x][e]);
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// The block's query rows r = t * G + hh of (b, g) into qs, all loads issued
// before the first is used; with bf16 K/V the query is read as bf16 (RNE).
// Rows R .. 4 * XR - 1 are zero: they are computed and dropped.
template <typename KVT, int D, int XR>
__device__ __forceinline__ void stage_q(const AttnArgs& a, int b, int g, float (*qs)[D]) {
    constexpr int VPR = D / 4, NV = 4 * XR * VPR, PER = (NV + kThreads - 1) / kThreads;
    const int G = a.G, R = G * a.T;
    float4 v[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int i = threadIdx.x + p * kThreads;
        const int r = i / VPR, x = i - r * VPR;
        v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < NV && r < R) {
            const int t = r / G, hh = r - t * G;
            v[p] = *(const float4*)&a.q[(((int64_t)b * a.T + t) * a.Hq + g * G + hh) * D + 4 * x];
        }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int i = threadIdx.x + p * kThreads;
        const int r = i / VPR, x = i - r * VPR;
        if (i < NV) {
            float4 u = v[p];
            if (sizeof(KVT) == 2) {
                u.x = __uint_as_float(f32_to_bf16_rne(u.x) << 16);
                u.y = __uint_as_float(f32_to_bf16_rne(u.y) << 16);
                u.z = __uint_as_float(f32_to_bf16_rne(u.z) << 16);
                u.w = __uint_as_float(f32_to_bf16_rne(u.w) << 16);
            }
            *(float4*)&qs[r][4 * x] = u;
        }
    }
}

template <typename KVT, int D, int XR>
__global__ __launch_bounds__(kThreads) void k_attn_generic(AttnArgs a) {
    constexpr int TR = 32, RMAX = 16, DPL = D / kWave;
    __shared__ __align__(16) float qs[RMAX][D];
    __shared__ __align__(16) float kt[TR][D + 4];
    __shared__ __align__(16) float vt[TR][D];
    __shared__ __align__(16) float zs[RMAX][TR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int bg, split;
    xcd_unit(blockIdx.x, a.splits, gridDim.x / a.splits, bg, split);
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int G = a.G, T = a.T, R = G * T;
    int u0, u1;
    entry_range(a, bg, split, u0, u1);

    stage_q<KVT, D, XR>(a, b, g, qs);
    const KVT* Kb = (const KVT*)a.K + (int64_t)b * a.ks.b + (int64_t)g * a.ks.h;
    const KVT* Vb = (const KVT*)a.V + (int64_t)b * a.vs.b + (int64_t)g * a.vs.h;

    float m_run[XR], l_run[XR], acc[XR][DPL];
#pragma unroll
    for (int x = 0; x < XR; ++x) {
        m_run[x] = -INFINITY;
        l_run[x] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[x][e] = 0.f;
    }
    const int tiles_per_chunk = (a.chunk + TR - 1) / TR;
    for (int u = u0; u < u1; ++u) {
        const int c = a.block_ids[(int64_t)bg * a.N + u];
        uint32_t m = a.member ? a.member[(int64_t)bg * a.N + u] : 0xffu;
        if (c < 0 || c >= a.pool_blocks) m = 0;
        if (m == 0) continue;
        for (int st = 0; st < tiles_per_chunk; ++st) {
            const int r0 = st * TR;
            const int nr = min(TR, a.chunk - r0);
            TileRegs<KVT, D, TR> tr;
            tile_load(tr, nr, [&](int rr) {
                const int64_t row = (int64_t)c * a.chunk + r0 + rr;
                return RowPair{Kb + row * a.ks.t, Vb + row * a.vs.t};
            });
            __syncthreads();
            tile_store(tr, nr, kt, vt);
            __syncthreads();
            attend_tile<D, TR, XR>(a, nr, qs, kt, vt, zs, [&](int r, int) { return ((m >> (r / G)) & 1u) != 0; },
                                   m_run, l_run, acc);
        }
    }
#pragma unroll
    for (int x = 0; x < XR; ++x) {
        const int r = w + 4 * x;
        if (r >= R) break;
        const int t = r / G, hh = r - t * G;
        emit_row<D>(a, b, bg, split, t, g * G + hh, r, R, m_run[x], l_run[x], acc[x], lane * DPL,
                    DPL, lane == 0);
    }
}

// ---------------------------------------------------------------------------
// Tail rows and the step's own rows off the fast path, one block per (b, g),
// written as the last partial of the (b, g) (DualDecoder "5.2": the real token is masked from the
// speculative token's row, the speculative token sees the real one; Adaptive
// DHiSparse Figure 2: the request's tail rows are resolved for every lookup).
// Rows 0 .. nt-1 are the tail, rows nt .. nt+T-1 the step's tokens; 64-row
// tiles go through LDS as in the generic kernel, so a tail shorter than a
// 32-row chunk and the step's two rows take one tile.
// ---------------------------------------------------------------------------
template <typename KVT, int D, int XR>
__global__ __launch_bounds__(kThreads) void k_attn_tail(AttnArgs a) {
    constexpr int TR = 64, RMAX = 16, DPL = D / kWave;
    __shared__ __align__(16) float qs[RMAX][D];
    __shared__ __align__(16) float kt[TR][D + 4];
    __shared__ __align__(16) float vt[TR][D];
    __shared__ __align__(16) float zs[RMAX][TR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int G = a.G, T = a.T, R = G * T;
    int nt = 0;
    if (a.Kt) {
        nt = a.tail_len ? a.tail_len[b] : a.tail_max;
        nt = nt < 0 ? 0 : (nt > a.tail_max ? a.tail_max : nt);
    }
    const int nrows = nt + (a.Kn ? T : 0);
    const KVT* Ktb = (const KVT*)a.Kt + (int64_t)b * a.kts.b + (int64_t)g * a.kts.h;
    const KVT* Vtb = (const KVT*)a.Vt + (int64_t)b * a.vts.b + (int64_t)g * a.vts.h;
    auto rows_at = [&](int base) {
        return [=](int rr) {
            const int row = base + rr;
            if (row < nt) return RowPair{Ktb + (int64_t)row * a.kts.t, Vtb + (int64_t)row * a.vts.t};
            const int64_t off = (((int64_t)b * T + (row - nt)) * a.Hkv + g) * D;
            return RowPair{(const KVT*)a.Kn + off, (const KVT*)a.Vn + off};
        };
    };
    // the first tile is on its way while the queries are staged; later, the
    // next tile's loads are in flight while the current one is used
    TileRegs<KVT, D, TR> tr;
    if (nrows > 0) tile_load(tr, min(TR, nrows), rows_at(0));
    stage_q<KVT, D, XR>(a, b, g, qs);
    float m_run[XR], l_run[XR], acc[XR][DPL];
#pragma unroll
    for (int x = 0; x < XR; ++x) {
        m_run[x] = -INFINITY;
        l_run[x] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[x][e] = 0.f;
    }
    for (int base = 0; base < nrows; base += TR) {
        const int nr = min(TR, nrows - base);
        __syncthreads();
        tile_store(tr, nr, kt, vt);
        __syncthreads();
        if (base + TR < nrows) tile_load(tr, min(TR, nrows - base - TR), rows_at(base + TR));
        // a tail row is seen by every query; the fresh row of token t' only by
        // queries t >= t'
        attend_tile<D, TR, XR>(a, nr, qs, kt, vt, zs,
                               [&](int r, int jj) { return base + jj < nt || base + jj - nt <= r / G; },
                               m_run, l_run, acc);
    }
#pragma unroll
    for (int x = 0; x < XR; ++x) {
        const int r = w + 4 * x;
        if (r >= R) break;
        const int t = r / G, hh = r - t * G;
        emit_row<D>(a, b, bg, a.nparts - 1, t, g * G + hh, r, R, m_run[x], l_run[x], acc[x], lane * DPL, DPL,
                    lane == 0);
    }
}

// ---------------------------------------------------------------------------
// Merge of the split partials (online-softmax combination), one block per (b, g).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_merge(AttnArgs a) {
    constexpr int P = 8;   // partials read per batch: their loads are in flight together
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int R = a.G * a.T;
    constexpr int D4 = D / 4;
    for (int i = threadIdx.x; i < R * D4; i += kThreads) {
        const int r = i / D4, d4 = i - r * D4;
        const int64_t slot0 = (int64_t)bg * a.nparts * R + r;   // partial s of row r: slot0 + s * R
        float M = -INFINITY;
        for (int s0 = 0; s0 < a.nparts; s0 += P) {
            float m[P];
#pragma unroll
            for (int j = 0; j < P; ++j)
                m[j] = s0 + j < a.nparts ? a.part_ml[(slot0 + (int64_t)(s0 + j) * R) * 2] : -INFINITY;
#pragma unroll
            for (int j = 0; j < P; ++j) M = fmaxf(M, m[j]);
        }
        float L = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (M != -INFINITY) {
            for (int s0 = 0; s0 < a.nparts; s0 += P) {
                float2 ml[P];
                float4 x[P];
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const int64_t slot = slot0 + (int64_t)(s0 + j) * R;
                    const bool in = s0 + j < a.nparts;
                    ml[j] = in ? *reinterpret_cast<const float2*>(a.part_ml + slot * 2) : make_float2(-INFINITY, 0.f);
                    x[j] = in ? *reinterpret_cast<const float4*>(a.part_acc + slot * D + d4 * 4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    if (ml[j].x == -INFINITY) continue;
                    const float f = exp2f(ml[j].x - M);
                    L += ml[j].y * f;
                    acc.x += x[j].x * f; acc.y += x[j].y * f; acc.z += x[j].z * f; acc.w += x[j].w * f;
                }
            }
        }
        const int t = r / a.G, hh = r - t * a.G;
        const int h = g * a.G + hh;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float* o = a.out + (((int64_t)b * a.T + t) * a.Hq + h) * D + d4 * 4;
        *reinterpret_cast<float4*>(o) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        if (d4 == 0 && a.lse)
            a.lse[((int64_t)b * a.T + t) * a.Hq + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
}

}  // namespace

bool use_fast_path(dk_dtype dt, int D, int G, int T, int chunk, dk_strides ks, dk_strides vs) {
    return dt == DK_BF16 && D == 128 && G == 4 && T == 2 && chunk % 32 == 0 &&
           ks.t < (1 << 26) && vs.t < (1 << 26);
}

AttnPlan plan_attn(int B, int Hkv, int T, int Hq, int dv, int N, int chunk, bool tail) {
    AttnPlan p{1, 1, 0};
    const int64_t bg = (int64_t)B * Hkv;
    const int R = (Hq / Hkv) * T;
    const int64_t tiles = (int64_t)N * ((chunk + 31) / 32);
    // at least about 256 blocks, one per CU: fewer, longer ranges write fewer
    // partials (at B * Hkv >= 256 none at all, and no merge), and the partial
    // writes cost far more than their bytes suggest while the ranges' gathers
    // stream (measured: at B * Hkv = 128 two ranges beat four, at 256 one range
    // beats two).  For long unions at least ~20 tiles of a full union per range
    // (about 11 at the usual half-full union), for short ones (latency-bound) at
    // least ~6; never more entries per range than the fast path stages in LDS
    int64_t want = (256 + bg - 1) / bg;
    int64_t by_work = tiles >= 120 ? tiles / 20 : tiles / 6;
    if (by_work < 1) by_work = 1;
    int64_t s = want < by_work ? want : by_work;
    // and at most ~128 tiles of a full union per range: with ragged unions (a
    // coverage budget's sets) the longest (b, g) then spreads over ranges
    const int64_t cap_s = (tiles + 127) / 128;
    if (s < cap_s) s = cap_s;
    const int64_t min_s = (N + kFastMaxEntries - 1) / kFastMaxEntries;
    if (s < min_s) s = min_s;
    if (s > 64 && min_s <= 64) s = 64;
    if (s < 1) s = 1;
    p.splits = (int)s;
    p.nparts = (int)s + (tail ? 1 : 0);
    p.ws_bytes = p.nparts > 1 ? (size_t)(bg * p.nparts * R) * (size_t)(dv + 2) * 4 : 0;
    return p;
}

// kernel selection by K/V type, head size and query rows per wave (R <= 16)
struct GenericKernel {
    template <typename KVT, int D, int XR>
    static void launch(dim3 grid, hipStream_t st, const AttnArgs& a) {
        hipLaunchKernelGGL((k_attn_generic<KVT, D, XR>), grid, dim3(kThreads), 0, st, a);
    }
};
struct TailKernel {
    template <typename KVT, int D, int XR>
    static void launch(dim3 grid, hipStream_t st, const AttnArgs& a) {
        hipLaunchKernelGGL((k_attn_tail<KVT, D, XR>), grid, dim3(kThreads), 0, st, a);
    }
};
template <typename K, typename KVT, int D>
void launch_xr(int R, dim3 grid, hipStream_t st, const AttnArgs& a) {
    switch ((R + 3) / 4) {
        case 1: K::template launch<KVT, D, 1>(grid, st, a); break;
        case 2: K::template launch<KVT, D, 2>(grid, st, a); break;
        case 3: K::template launch<KVT, D, 3>(grid, st, a); break;
        default: K::template launch<KVT, D, 4>(grid, st, a); break;
    }
}
template <typename K>
void launch_rows(dk_dtype dt, int D, int R, dim3 grid, hipStream_t st, const AttnArgs& a) {
    if (dt == DK_BF16) {
        if (D == 128) launch_xr<K, uint16_t, 128>(R, grid, st, a);
        else launch_xr<K, uint16_t, 64>(R, grid, st, a);
    } else {
        if (D == 128) launch_xr<K, float, 128>(R, grid, st, a);
        else launch_xr<K, float, 64>(R, grid, st, a);
    }
}

hipError_t launch_attention(const float* q, int B, int T, int Hq, int Hkv, const void* K,
                            const void* V, dk_dtype dt, dk_strides ks, dk_strides vs, int D,
                            int chunk, const int32_t* block_ids, const uint8_t* member,
                            const int32_t* count, int N, int pool_blocks, float scale, float* out,
                            float* lse, void* ws, const AttnPlan& plan, const AttnTail* tail,
                            hipStream_t st) {
    AttnArgs a{};
    a.q = q; a.Hq = Hq; a.Hkv = Hkv; a.T = T; a.G = Hq / Hkv;
    a.K = K; a.V = V; a.ks = ks; a.vs = vs; a.chunk = chunk;
    a.block_ids = block_ids; a.member = member; a.count = count;
    a.N = N; a.pool_blocks = pool_blocks;
    a.scale_log2 = scale * kLog2e;
    a.splits = plan.splits;
    a.nparts = plan.nparts;
    a.out = out; a.lse = lse;
    const int64_t bg = (int64_t)B * Hkv;
    const int R = a.G * T;
    a.part_acc = plan.nparts > 1 ? (float*)ws : nullptr;
    a.part_ml = plan.nparts > 1 ? (float*)ws + bg * plan.nparts * R * D : nullptr;
    if (tail) {
        a.Kt = tail->K_tail; a.Vt = tail->V_tail; a.kts = tail->kts; a.vts = tail->vts;
        a.tail_len = tail->tail_len; a.tail_max = tail->tail_max;
        a.Kn = tail->K_new; a.Vn = tail->V_new;
    }
    const unsigned grid = (unsigned)(bg * plan.splits);
    const bool fast = use_fast_path(dt, D, a.G, T, chunk, ks, vs);
    if (fast) {
        // the fast kernel's last range of each (b, g) attends the tail and own
        // rows itself: no tail partial, and with one range no merge either
        if (tail) {
            a.nparts = plan.splits;
            hipLaunchKernelGGL(k_attn_bf16_d128_g4t2<true>, dim3(grid), dim3(kFastThreads), 0, st, a);
        } else {
            hipLaunchKernelGGL(k_attn_bf16_d128_g4t2<false>, dim3(grid), dim3(kFastThreads), 0, st, a);
        }
    } else {
        launch_rows<GenericKernel>(dt, D, R, dim3(grid), st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (tail && !fast) {
        launch_rows<TailKernel>(dt, D, R, dim3((unsigned)bg), st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.nparts == 1) return hipSuccess;
    if (D == 128) hipLaunchKernelGGL(k_attn_merge<128>, dim3((unsigned)bg), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(k_attn_merge<64>, dim3((unsigned)bg), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dk
