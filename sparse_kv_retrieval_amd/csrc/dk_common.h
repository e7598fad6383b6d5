// Internal helpers shared by the libdualkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dualkv.h"

namespace dk {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 words: a dword holds two bf16 values, the lower element in bits 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// Order-preserving uint32 key of an fp32 score: a > b  <=>  key(a) > key(b).
// -0 is folded onto +0 so equal scores give equal keys.  Finite inputs; every
// finite score (and -inf) maps to a key above 0, so 0 marks an empty slot.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
    if (f == 0.0f) f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// Block-wide exclusive prefix sum of one int per thread.  `scratch` holds at
// least blockDim.x / 64 + 1 ints of LDS.  Returns the exclusive prefix and
// writes the block total to *total.  Every thread of the block must call it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    return v;
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = (blockDim.x + kWave - 1) / kWave;
    int inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nwaves; ++w) {
            int t = scratch[w];
            scratch[w] = run;
            run += t;
        }
        scratch[nwaves] = run;
    }
    __syncthreads();
    int excl = scratch[wave] + inc - v;
    *total = scratch[nwaves];
    __syncthreads();
    return excl;
}

// ---------------------------------------------------------------------------
// Cross-lane helpers.
// ---------------------------------------------------------------------------
// sum over the aligned group of LPR (4, 8 or 16) lanes, every lane gets the total
template <int LPR>
__device__ __forceinline__ float dpp_group_sum(float v) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "groups of 4, 8 or 16 lanes");
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    if constexpr (LPR == 4) {
        return v;
    } else if constexpr (LPR == 8) {
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    } else {
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    }
    return v;
}

// Workgroups go to the 8 XCDs (each with its own L2) round-robin by block id.
// Block id -> (unit, sub) with `per` blocks per unit and n_units units: when
// n_units is a multiple of 8 every block of a unit runs on XCD unit % 8, so the
// kernels of one step that map their blocks this way find a (b, g)'s
// intermediate rows in the L2 that wrote them; otherwise the plain order.
__device__ __forceinline__ void xcd_unit(int bid, int per, int n_units, int& unit, int& sub) {
    if ((n_units & 7) == 0) {
        const int slot = bid >> 3;
        sub = slot % per;
        unit = (slot / per) * 8 + (bid & 7);
    } else {
        sub = bid % per;
        unit = bid / per;
    }
}

// value of lane i ^ 1 (DPP quad_perm [1,0,3,2]; a VALU op, no LDS round trip)
__device__ __forceinline__ float dpp_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// ---------------------------------------------------------------------------
// Agent-scope relaxed store / load: written through to, and read from, the
// device-coherent level, so another block (on any XCD) that reads the value
// after a device-scope atomic sees it without a whole-cache fence.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_agent(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_agent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Streamed once: non-temporal 16-byte loads.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t nt_load_u4(const void* p) {
#ifdef DK_SCORE_PLAIN_LOADS
    return *reinterpret_cast<const u32x4_t*>(p);
#else
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#endif
}

// ---------------------------------------------------------------------------
// Global -> LDS DMA (gfx950 global_load_lds_dwordx4).  Lane i's 16 bytes land
// at lds_base + 16 * i; lds_base must be wave-uniform.  The load is issued from
// inline asm so that the compiler does not insert its own (conservative)
// vmcnt waits; callers wait with lds_dma_wait<N>() (N = loads that may still be
// in flight) and must issue no other vector-memory loads between a DMA and its
// wait.  Non-temporal: the streamed KV is not reused.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((lds_char_t*)(p));
}
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void lds_dma_wait() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
}
// s_barrier without the compiler's release fence (which would wait for every
// outstanding DMA); ordering of LDS accesses is kept by the asm memory clobbers.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Matrix-core operands (v_mfma_f32_16x16x32_bf16: A is 16 x 32, B is 32 x 16;
// lane l holds A[l % 16][8 (l / 16) .. + 7] and B[8 (l / 16) .. + 7][l % 16];
// the fp32 result has D[4 (l / 16) + i][l % 16] in element i of lane l).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (v_permlane16/32_swap:
// with both operands equal, the two results hold the values of the lane pair)
__device__ __forceinline__ float group4_max(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// ds_read_b64_tr_b16: within each 16-lane group, lane i addresses 8 bytes (row
// i / 4, columns 4 (i % 4) .. + 3 of a 4 x 16 bf16 block); lane j receives
// column j of that block, its four rows in ascending order.
__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p)));
}

// ---------------------------------------------------------------------------
// 16-byte global loads/stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace dk

// ---------------------------------------------------------------------------
// Launchers (one per kernel family).  Arguments are already validated.
// ---------------------------------------------------------------------------
namespace dk {

hipError_t launch_landmarks(const void* K, dk_dtype dt, dk_strides ks, int B, int Hkv, int L,
                            int d, int chunk, float* lm, hipStream_t st);

struct TopkPlan {
    int splits;        // chunk-range splits per (b, g)
    int rows;          // chunks per split (last split may have fewer)
    size_t ws_bytes;   // candidate buffer bytes (0 when splits == 1)
};
TopkPlan plan_topk(int B, int Hkv, int T, int C, int k, bool shadow);
// Union outputs computed in the same call as the top-k (dk_score_topk_union).
struct UnionOut {
    int32_t* ids;        // [B, Hkv, T*k]
    uint8_t* member;     // [B, Hkv, T*k]
    int32_t* count;      // [B, Hkv]
    int32_t* overlap;    // [B, Hkv] or null
};
// One fused kernel for dk_decode_step (shadow scores, selection, union and the
// attention fast path per (b, g)); T = 2, G = 4, d = 128, bf16 K/V, mean reduce.
hipError_t launch_step_fused(const float* q, int B, int Hq, int Hkv, int C, int k, float scale,
                             const dk_landmark_shadow* sh, const float* lm, dk_strides ls, const void* K,
                             const void* V, dk_strides ks, dk_strides vs, int chunk, int32_t* topk_idx,
                             float* topk_score, const UnionOut& un, float* out, float* lse, hipStream_t st);
hipError_t launch_score_topk(const float* q, int B, int T, int Hq, const float* lm, dk_strides ls,
                             int Hkv, int C, int d, int k, float scale, dk_group_reduce reduce,
                             const dk_landmark_shadow* shadow, int32_t* topk_idx, float* topk_score,
                             void* ws, const TopkPlan& plan, const UnionOut* un, hipStream_t st);
// Token-level indexer on bf16 keys (k_indexer.hip): fp32 scores of every token in
// the workspace, then an exact threshold select per (b, g, t).
struct IndexPlan {
    int rows_per_block;  // score rows (tokens or chunks) per scoring block
    int blocks_per_bg;   // scoring blocks per (b, g); the per-block ranges are sized for these
    // the token-level bf16 scoring kernel's own blocks (longer for long rows with
    // many (b, g)); its per-block ranges use score_blocks_per_bg <= blocks_per_bg
    int score_rows, score_blocks_per_bg;
    size_t off_min;      // byte offsets of the per-block score minima / maxima
    size_t off_max;
    size_t off_arrive;   // one arrival counter per (b, g) for the fused union
    // split selection of long rows (slices == 0: one block per row)
    int slices;          // blocks per row
    int slice_len;       // positions per slice (a multiple of 4096)
    size_t off_hist, off_aid, off_aval, off_cid, off_cval, off_cnt, off_flag;
    size_t ws_bytes;
};
IndexPlan plan_index_topk(int B, int Hkv, int T, int C);
// The exact selection over fp32 score rows [B*Hkv*T][C] with per-block ranges
// (the plan's layout), optionally with the union of each (b, g)'s T sets.
hipError_t launch_select_rows(const float* scores, const float* bmin, const float* bmax, int blocks_per_row, int B,
                              int Hkv, int T, int C, int k, int32_t* topk_idx, float* topk_score, const UnionOut* un,
                              uint32_t* arrivals, const IndexPlan& plan, void* ws, hipStream_t st);
// Min/max chunk summaries and the top-k by their upper-bound scores (k_minmax.hip).
hipError_t launch_build_minmax(const void* K, dk_dtype dt, dk_strides ks, int B, int Hkv, int L, int d, int chunk,
                               void* kmin, void* kmax, hipStream_t st);
hipError_t launch_minmax_topk(const float* q, int B, int T, int Hq, const void* kmin, const void* kmax, dk_dtype dt,
                              dk_strides ss, int Hkv, int C, int d, int k, float scale, dk_group_reduce reduce,
                              int32_t* topk_idx, float* topk_score, void* ws, const IndexPlan& plan,
                              const UnionOut* un, hipStream_t st);
// Plain (box == null) or upper-bound (kmin = a, kmax = b) chunk score rows and their
// block ranges into the IndexPlan workspace.
hipError_t launch_score_rows(const float* q, int B, int T, int Hq, const void* a, const void* b, dk_dtype dt,
                             dk_strides ss, int Hkv, int C, int d, float scale, dk_group_reduce reduce, void* ws,
                             const IndexPlan& plan, uint32_t* arrivals, hipStream_t st);
constexpr int kCoverageMaxC = 16384;   // chunks per row of the coverage selection (registers of one block)
hipError_t launch_coverage(const float* q, int B, int T, int Hq, const void* lm, dk_dtype dt, dk_strides ls, int Hkv,
                           int C, int d, float scale, dk_group_reduce reduce, float gamma, int k_max,
                           int32_t* sel_idx, int32_t* sel_count, float* sel_score, const UnionOut* un, void* ws,
                           const IndexPlan& plan, hipStream_t st);
constexpr int kCappedMaxN = 4096;   // predicted entries and slots per (b, g) of the capped plan (LDS <= 48 KB)
hipError_t launch_capped_plan(const int32_t* sel_ids, const float* sel_score, const int32_t* sel_count, int B,
                              int Hkv, int N, int64_t sel_stride, int64_t count_stride, int32_t* resident,
                              int32_t* stamp, int S, int cap, int32_t step, int32_t* sel_slot, int32_t* admit_chunk,
                              int32_t* admit_slot, int32_t* admit_count, int32_t* hit_count, hipStream_t st);
hipError_t launch_index_topk(const float* q, int B, int T, int Hq, const uint16_t* keys, dk_strides ks, int Hkv,
                             int C, int d, int k, float scale, int32_t* topk_idx, float* topk_score, void* ws,
                             const IndexPlan& plan, const UnionOut* un, hipStream_t st);
// Latent attention with token-level selection on the matrix cores (k_mla.hip):
// dk = 576, dv = 512, bf16, value = the first 512 columns of the key rows.
struct MlaPlan {
    int splits;       // union ranges per (b, g)
    int rgroups;      // 64-row query groups per (b, g)
    size_t ws_bytes;  // range partials (0 when splits == 1)
};
MlaPlan plan_mla(int B, int Hkv, int T, int Hq, int N);
hipError_t launch_mla_attention(const float* q, int B, int T, int Hq, int Hkv, const void* lat, dk_strides ks,
                                const int32_t* ids, const uint8_t* member, const int32_t* count, int N, int L,
                                float scale, float* out, float* lse, void* ws, const MlaPlan& plan,
                                hipStream_t st);
hipError_t launch_build_shadow(const float* lm, dk_strides ls, int B, int Hkv, int C, int d,
                               uint8_t* lm8, float* chunk_scale, float* scale_max, hipStream_t st);

hipError_t launch_union(const int32_t* topk_idx, int B, int Hkv, int T, int k, int C,
                        int32_t* union_ids, uint8_t* member, int32_t* union_count, int32_t* overlap,
                        const dk_cache_plan* plan, hipStream_t st);

hipError_t launch_gather(const void* K_src, const void* V_src, dk_dtype dt, dk_strides ss, int B,
                         int Hkv, int chunk, int d, const int32_t* src_chunk, const int32_t* dst_slot,
                         const int32_t* count, int N, int src_blocks, void* K_dst, void* V_dst,
                         dk_strides ds, int dst_blocks, hipStream_t st);
hipError_t launch_gather_stream(const void* K_src, const void* V_src, dk_dtype dt, dk_strides ss, int B,
                         int Hkv, int chunk, int d, const int32_t* src_chunk, const int32_t* dst_slot,
                         const int32_t* count, int N, int src_blocks, void* K_dst, void* V_dst,
                         dk_strides ds, int dst_blocks, hipStream_t st);

struct AttnPlan {
    int splits;        // union-range splits per (b, g)
    int nparts;        // partial slots per (b, g): splits, plus one for tail rows
    size_t ws_bytes;   // partial results (0 when nparts == 1)
};
// Rows every query attends besides its chunks (dk_sparse_decode_attn_tail).
struct AttnTail {
    const void* K_tail;       // [B, Hkv, tail_max, D] with strides kts / vts, or null
    const void* V_tail;
    dk_strides kts, vts;
    const int32_t* tail_len;  // [B] or null (tail_max rows each)
    int tail_max;
    const void* K_new;        // [B, T, Hkv, D] contiguous, or null
    const void* V_new;
};
AttnPlan plan_attn(int B, int Hkv, int T, int Hq, int dv, int N, int chunk, bool tail = false);
// the attention fast path's shapes: bf16, d = 128, G = 4, T = 2, chunk a multiple of 32
bool use_fast_path(dk_dtype dt, int D, int G, int T, int chunk, dk_strides ks, dk_strides vs);
hipError_t launch_attention(const float* q, int B, int T, int Hq, int Hkv, const void* K,
                            const void* V, dk_dtype dt, dk_strides ks, dk_strides vs, int D,
                            int chunk, const int32_t* block_ids, const uint8_t* member,
                            const int32_t* count, int N, int pool_blocks, float scale, float* out,
                            float* lse, void* ws, const AttnPlan& plan, const AttnTail* tail,
                            hipStream_t st);

}  // namespace dk
