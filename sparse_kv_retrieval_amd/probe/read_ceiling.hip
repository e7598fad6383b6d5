// Read-rate ceilings of the card, for the measurement in bench.py --ceiling.
// Not part of libdualkv: a separate library (libdkprobe.so) that bench.py loads
// only for that measurement.
//
// Both kernels read tiles of 16 KiB (8 KiB from each of two arrays, the K and V
// halves of one 32-row chunk pair of a bf16 d = 128 pool), 256 threads per
// block, a fixed number of tiles per block, either contiguous (tile i is chunk
// i) or gathered (tile i is chunk ids[i]):
//   * dkp_reg:  16-byte loads into registers, two tiles in flight per block;
//   * dkp_ring: global_load_lds_dwordx4 into a three-stage LDS ring, two tiles
//               in flight while one is read, the attention kernel's data path.
// Each thread folds what it reads into one word, so the loads are not removed;
// nothing else is computed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256, kStages = 3, kChunkBytes = 8192;

typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)((lds_char_t*)(p)); }
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory"); }
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16 bytes of piece i (0..15: 1 KiB each, 8 from K then 8 from V) of tile chunk c, lane l
__device__ __forceinline__ const char* piece(const char* K, const char* V, long long c, int i, int l) {
    return (i < 8 ? K : V) + c * kChunkBytes + (i & 7) * 1024 + l * 16;
}

__global__ __launch_bounds__(kThreads) void k_ring(const char* K, const char* V, const long long* ids, int tpb,
                                                   unsigned* sink) {
    __shared__ uint4 ring[kStages][1024];
    __shared__ long long sid[256];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long t0 = (long long)blockIdx.x * tpb;
    for (int i = threadIdx.x; i < tpb; i += kThreads) sid[i] = ids ? ids[t0 + i] : t0 + i;
    __syncthreads();
    auto issue = [&](int it) {
        const int s = it % kStages;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * w + q;
            dma16(piece(K, V, sid[it], i, lane), lds_addr(&ring[s][i * 64]));
        }
    };
    unsigned acc = 0;
    if (tpb > 0) issue(0);
    if (tpb > 1) issue(1);
    for (int it = 0; it < tpb; ++it) {
        if (it + 1 < tpb) dma_wait<4>();
        else dma_wait<0>();
        raw_barrier();
        if (it + 2 < tpb) issue(it + 2);
        acc ^= ring[it % kStages][threadIdx.x].x;
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void k_reg(const char* K, const char* V, const long long* ids, int tpb,
                                                  unsigned* sink) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long long t0 = (long long)blockIdx.x * tpb;
    auto chunk = [&](int it) { return ids ? ids[t0 + it] : t0 + it; };
    unsigned acc = 0;
    uint4 a[4], b[4];
    auto load = [&](uint4* r, int it) {
        const long long c = chunk(it);
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = *reinterpret_cast<const uint4*>(piece(K, V, c, 4 * w + q, lane));
    };
    if (tpb > 0) load(a, 0);
    for (int it = 0; it < tpb; ++it) {
        if (it + 1 < tpb) load(b, it + 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc ^= a[q].x ^ a[q].y ^ a[q].z ^ a[q].w;
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = b[q];
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Launch one read pass on `stream`: blocks x tiles_per_block tiles of 16 KiB.
// K, V: device arrays of at least (largest chunk read + 1) * 8 KiB each; ids:
// device int64 [blocks * tiles_per_block] chunk ids, or NULL for contiguous
// tiles; sink: device uint32 [blocks] (written only in the impossible case of
// a checksum match).  mode 0: register loads, 1: LDS-DMA ring.  Returns a
// hipError_t value (0 on success).
int dkp_read_pass(int mode, const void* K, const void* V, const long long* ids, int blocks, int tiles_per_block,
                  unsigned* sink, void* stream) {
    if (blocks < 1 || tiles_per_block < 1 || tiles_per_block > 256 || !K || !V || !sink) return (int)hipErrorInvalidValue;
    if (mode == 0)
        hipLaunchKernelGGL(k_reg, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, (const char*)K, (const char*)V,
                           ids, tiles_per_block, sink);
    else
        hipLaunchKernelGGL(k_ring, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, (const char*)K,
                           (const char*)V, ids, tiles_per_block, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
