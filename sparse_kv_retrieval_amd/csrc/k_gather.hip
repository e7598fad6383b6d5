// Device-side gather of selected KV chunks into destination slots.
//
// DualDecoder (arXiv 2607.26475), "5.4 Layer-Scoped KV Memory Management",
// GPU-side sparse KV assembly: a GPU kernel places selected KV blocks into the
// attention layout in HBM.  One block per (b, g, entry) copies the entry's K and
// V rows with 16-byte loads and stores; ids outside the source or destination
// range are skipped, never dereferenced.
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

}  // namespace

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
