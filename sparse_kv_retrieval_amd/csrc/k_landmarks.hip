// Chunk landmarks: the mean key of every fixed-size chunk of a KV pool.
//
// DualDecoder (arXiv 2607.26475), "2.2 Dynamic Sparse KV Cache" and "4.1 KV
// Retrieval Predictability": adjacent KV entries form chunks summarised by
// landmarks that are built once before decoding.
//
// Pure streaming kernel: every key byte is read once, every landmark written
// once.  A thread owns 16 bytes of a key row (8 bf16 or 4 fp32 dims) of one
// chunk and walks the chunk's rows, keeping fp32 sums; d/EPT threads cover a
// row, so one wave-wide load covers whole 128-byte lines of consecutive rows.
#include "dk_common.h"

namespace dk {
namespace {

template <typename T>
struct Elems;
template <>
struct Elems<uint16_t> {
    static constexpr int kPer16B = 8;
    __device__ static void add(float* acc, uint4 v) {
        acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
        acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
        acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
        acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
    }
};
template <>
struct Elems<float> {
    static constexpr int kPer16B = 4;
    __device__ static void add(float* acc, uint4 v) {
        acc[0] += __uint_as_float(v.x); acc[1] += __uint_as_float(v.y);
        acc[2] += __uint_as_float(v.z); acc[3] += __uint_as_float(v.w);
    }
};

template <typename T>
__global__ __launch_bounds__(256) void k_landmarks(const T* __restrict__ K, dk_strides ks, int Hkv,
                                                   int C, int d, int chunk, float* __restrict__ lm,
                                                   int tpr, int cpb, int64_t total) {
    constexpr int EPT = Elems<T>::kPer16B;
    const int lc = threadIdx.x / tpr;
    const int part = threadIdx.x - lc * tpr;
    if (lc >= cpb) return;
    const int64_t cid = (int64_t)blockIdx.x * cpb + lc;   // flattened (b, g, c)
    if (cid >= total) return;
    const int64_t bg = cid / C;
    const int c = (int)(cid - bg * C);
    const int b = (int)(bg / Hkv);
    const int g = (int)(bg - (int64_t)b * Hkv);
    const T* src = K + (int64_t)b * ks.b + (int64_t)g * ks.h + (int64_t)c * chunk * ks.t + part * EPT;

    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
    int n = 0;
    for (; n + 8 <= chunk; n += 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld16(src + (int64_t)(n + u) * ks.t);
#pragma unroll
        for (int u = 0; u < 8; ++u) Elems<T>::add(acc, v[u]);
    }
    for (; n < chunk; ++n) Elems<T>::add(acc, ld16(src + (int64_t)n * ks.t));

    const float div = (float)chunk;
    float* dst = lm + cid * d + part * EPT;
    if constexpr (EPT == 8) {
        float4 lo = make_float4(acc[0] / div, acc[1] / div, acc[2] / div, acc[3] / div);
        float4 hi = make_float4(acc[4] / div, acc[5] / div, acc[6] / div, acc[7] / div);
        reinterpret_cast<float4*>(dst)[0] = lo;
        reinterpret_cast<float4*>(dst)[1] = hi;
    } else {
        reinterpret_cast<float4*>(dst)[0] =
            make_float4(acc[0] / div, acc[1] / div, acc[2] / div, acc[3] / div);
    }
}

}  // namespace

hipError_t launch_landmarks(const void* K, dk_dtype dt, dk_strides ks, int B, int Hkv, int L,
                            int d, int chunk, float* lm, hipStream_t st) {
    const int C = L / chunk;
    const int64_t total = (int64_t)B * Hkv * C;
    const int ept = dt == DK_BF16 ? 8 : 4;
    const int tpr = d / ept;
    const int cpb = 256 / tpr;
    const int64_t blocks = (total + cpb - 1) / cpb;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (dt == DK_BF16)
        hipLaunchKernelGGL(k_landmarks<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const uint16_t*)K, ks, Hkv, C, d, chunk, lm, tpr, cpb, total);
    else
        hipLaunchKernelGGL(k_landmarks<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const float*)K, ks, Hkv, C, d, chunk, lm, tpr, cpb, total);
    return hipGetLastError();
}

}  // namespace dk
