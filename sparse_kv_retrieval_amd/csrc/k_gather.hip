// Device-side gather of selected KV chunks into destination slots.
//
// DualDecoder (arXiv 2607.26475), "5.4 Layer-Scoped KV Memory Management",
// GPU-side sparse KV assembly: a GPU kernel places selected KV blocks into the
// attention layout in HBM.  Ids outside the source or destination range are
// skipped, never dereferenced.
//
// Two kernels:
//  k_gather        one block per (b, g, entry); for a source in HBM, where many
//                  short-lived blocks keep the memory system busy.
//  k_gather_stream a small persistent grid for a source in pinned host memory
//                  read over PCIe (Adaptive DHiSparse, Figure 2: the resolver
//                  copies missed rows into the hot cache).  Each load waits
//                  microseconds on the link, so a block-per-entry grid would
//                  hold CU slots that the concurrently running scoring and
//                  attention kernels need; one thin wave per CU saturates the
//                  link instead.
#include "dk_common.h"

namespace dk {
namespace {

__global__ __launch_bounds__(256) void k_gather(const char* __restrict__ Ks,
                                                const char* __restrict__ Vs, dk_strides ss,
                                                int Hkv, int chunk, int row_bytes, int esz,
                                                const int32_t* __restrict__ src_chunk,
                                                const int32_t* __restrict__ dst_slot,
                                                const int32_t* __restrict__ count, int N,
                                                int src_blocks, char* __restrict__ Kd,
                                                char* __restrict__ Vd, dk_strides ds,
                                                int dst_blocks) {
    const int64_t e = blockIdx.x;
    const int64_t bg = e / N;
    const int j = (int)(e - bg * N);
    const int n = count ? count[bg] : N;
    if (j >= n) return;
    const int c = src_chunk[bg * N + j];
    const int s = dst_slot ? dst_slot[bg * N + j] : j;
    if (c < 0 || c >= src_blocks || s < 0 || s >= dst_blocks) return;
    const int b = (int)(bg / Hkv), g = (int)(bg - (int64_t)b * Hkv);
    const int upr = row_bytes / 16;   // 16-byte units per row
    const int units = chunk * upr;
    const int64_t sb = ((int64_t)b * ss.b + (int64_t)g * ss.h + (int64_t)c * chunk * ss.t) * esz;
    const int64_t db = ((int64_t)b * ds.b + (int64_t)g * ds.h + (int64_t)s * chunk * ds.t) * esz;
    for (int i = threadIdx.x; i < units; i += 256) {
        const int r = i / upr, x = i - r * upr;
        const int64_t so = sb + (int64_t)r * ss.t * esz + x * 16;
        const int64_t dof = db + (int64_t)r * ds.t * esz + x * 16;
        st16(Kd + dof, ld16(Ks + so));
        st16(Vd + dof, ld16(Vs + so));
    }
}

// Few blocks, many loads in flight: 32 blocks of 256 threads (one per CU on 32
// of the 256 CUs), four K and four V 16-byte loads in flight per lane (1 MiB in
// all; the link needs a few hundred KB).  Every lane that waits on PCIe holds
// part of its CU's memory pipeline, and HBM kernels running on that CU at the
// same time wait behind it, so the gather is kept off most CUs.  Measured on
// the host-pool step (per-layer hot caches, B=32, L=128K, 32 layers): one
// wave on every CU gave 16.4 ms per step (hot-cache attention about 480 us per
// layer under the gather, the gather at 49.9 GB/s); this form 15.4 ms
// (attention about 210-235 us, the gather at 53.7 GB/s).  16, 24 and 48 blocks,
// two or eight loads per lane, 128 or 512 threads, 8 blocks of 1024 threads
// were all between 15.4 and 16.0 ms.
constexpr int kStreamThreads = 256;
constexpr int kStreamBlocks = 32;
constexpr int kStreamUnroll = 4;     // K and V loads in flight per lane: 2 x kStreamUnroll

__global__ __launch_bounds__(kStreamThreads) void k_gather_stream(
    const char* __restrict__ Ks, const char* __restrict__ Vs, dk_strides ss, int Hkv, int chunk,
    int row_bytes, int esz, const int32_t* __restrict__ src_chunk, const int32_t* __restrict__ dst_slot,
    const int32_t* __restrict__ count, int N, int src_blocks, char* __restrict__ Kd,
    char* __restrict__ Vd, dk_strides ds, int dst_blocks, int64_t BG) {
    constexpr int NT = kStreamThreads;
    __shared__ int e_c[NT];
    __shared__ int e_s[NT];
    const int tid = threadIdx.x;
    const int upr = row_bytes / 16;   // 16-byte units per row
    const int upc = chunk * upr;      // 16-byte units per chunk and tensor
    for (int64_t bg = blockIdx.x; bg < BG; bg += gridDim.x) {
        int n = count ? count[bg] : N;
        n = n < 0 ? 0 : (n > N ? N : n);
        const int b = (int)(bg / Hkv), g = (int)(bg - (int64_t)b * Hkv);
        const int64_t sbase = (int64_t)b * ss.b + (int64_t)g * ss.h;
        const int64_t dbase = (int64_t)b * ds.b + (int64_t)g * ds.h;
        for (int jb = 0; jb < n; jb += NT) {
            const int m = n - jb < NT ? n - jb : NT;
            __syncthreads();   // the previous batch's entries are no longer read
            if (tid < m) {
                const int c = src_chunk[bg * N + jb + tid];
                const int s = dst_slot ? dst_slot[bg * N + jb + tid] : jb + tid;
                const bool ok = c >= 0 && c < src_blocks && s >= 0 && s < dst_blocks;
                e_c[tid] = ok ? c : -1;
                e_s[tid] = s;
            }
            __syncthreads();
            const int total = m * upc;
            for (int i0 = 0; i0 < total; i0 += NT * kStreamUnroll) {
                uint4 kv[kStreamUnroll], vv[kStreamUnroll];
                int64_t dof[kStreamUnroll];
#pragma unroll
                for (int u = 0; u < kStreamUnroll; ++u) {
                    const int i = i0 + u * NT + tid;
                    dof[u] = -1;
                    if (i < total) {
                        const int j = i / upc;
                        const int rem = i - j * upc;
                        const int r = rem / upr, x = rem - r * upr;
                        const int c = e_c[j];
                        if (c >= 0) {
                            const int64_t so = (sbase + ((int64_t)c * chunk + r) * ss.t) * esz + x * 16;
                            dof[u] = (dbase + ((int64_t)e_s[j] * chunk + r) * ds.t) * esz + x * 16;
                            kv[u] = ld16(Ks + so);
                            vv[u] = ld16(Vs + so);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < kStreamUnroll; ++u) {
                    if (dof[u] >= 0) {
                        st16(Kd + dof[u], kv[u]);
                        st16(Vd + dof[u], vv[u]);
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gather_stream(const void* K_src, const void* V_src, dk_dtype dt, dk_strides ss,
                                int B, int Hkv, int chunk, int d, const int32_t* src_chunk,
                                const int32_t* dst_slot, const int32_t* count, int N, int src_blocks,
                                void* K_dst, void* V_dst, dk_strides ds, int dst_blocks,
                                hipStream_t st) {
    const int esz = dt == DK_BF16 ? 2 : 4;
    const int64_t BG = (int64_t)B * Hkv;
    if (BG == 0 || N == 0) return hipSuccess;
    // indices within one batch of entries stay well inside int
    if ((int64_t)chunk * (d * esz / 16) * kStreamThreads > 0x7fffffff - 4096) return hipErrorInvalidValue;
    const int grid = BG < kStreamBlocks ? (int)BG : kStreamBlocks;
    hipLaunchKernelGGL(k_gather_stream, dim3(grid), dim3(kStreamThreads), 0, st, (const char*)K_src,
                       (const char*)V_src, ss, Hkv, chunk, d * esz, esz, src_chunk, dst_slot, count,
                       N, src_blocks, (char*)K_dst, (char*)V_dst, ds, dst_blocks, BG);
    return hipGetLastError();
}

hipError_t launch_gather(const void* K_src, const void* V_src, dk_dtype dt, dk_strides ss, int B,
                         int Hkv, int chunk, int d, const int32_t* src_chunk,
                         const int32_t* dst_slot, const int32_t* count, int N, int src_blocks,
                         void* K_dst, void* V_dst, dk_strides ds, int dst_blocks, hipStream_t st) {
    const int esz = dt == DK_BF16 ? 2 : 4;
    const int64_t blocks = (int64_t)B * Hkv * N;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gather, dim3((unsigned)blocks), dim3(256), 0, st, (const char*)K_src,
                       (const char*)V_src, ss, Hkv, chunk, d * esz, esz, src_chunk, dst_slot, count,
                       N, src_blocks, (char*)K_dst, (char*)V_dst, ds, dst_blocks);
    return hipGetLastError();
}

}  // namespace dk
