// libdualkv C ABI: argument checks, workspace sizing, launches, error text.
// Every check runs before anything is enqueued; a failing call enqueues nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "dk_common.h"

namespace {

thread_local std::string g_err;

dk_status fail(dk_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

dk_status hip_fail(hipError_t e, const char* what) {
    return fail(DK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int dtype_size(dk_dtype dt) { return dt == DK_BF16 ? 2 : (dt == DK_F32 ? 4 : 0); }

bool strides_ok(dk_strides s, int esz) {
    if (s.b < 0 || s.h < 0 || s.t < 0) return false;
    return (s.b * esz) % 16 == 0 && (s.h * esz) % 16 == 0 && (s.t * esz) % 16 == 0;
}

// Device address of pinned host memory, or nullptr when `p` is not host memory
// that HIP has pinned (pageable memory, device memory, unknown pointers).
void* mapped_host_ptr(const void* p) {
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();   // the query's failure is an answer, not a sticky error
        return nullptr;
    }
    return a.type == hipMemoryTypeHost ? a.devicePointer : nullptr;
}

#define DK_REQUIRE(cond, status, ...) \
    do {                              \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

}  // namespace

extern "C" {

int dk_abi_version(void) { return DK_ABI_VERSION; }

const char* dk_last_error(void) { return g_err.c_str(); }

dk_status dk_build_landmarks(const void* K, dk_dtype k_dtype, dk_strides ks, int B, int Hkv, int L,
                             int d, int chunk, float* lm, void* stream) {
    g_err.clear();
    const int esz = dtype_size(k_dtype);
    DK_REQUIRE(K && lm, DK_ERR_INVALID_ARG, "dk_build_landmarks: K and lm must be non-NULL");
    DK_REQUIRE(esz != 0, DK_ERR_INVALID_ARG, "dk_build_landmarks: unknown k_dtype %d", (int)k_dtype);
    DK_REQUIRE(B >= 1 && Hkv >= 1 && L >= 1 && d >= 1 && chunk >= 1, DK_ERR_INVALID_ARG,
               "dk_build_landmarks: B, Hkv, L, d, chunk must be >= 1");
    DK_REQUIRE(L % chunk == 0, DK_ERR_INVALID_ARG, "dk_build_landmarks: L (%d) %% chunk (%d) != 0", L,
               chunk);
    DK_REQUIRE(d % 8 == 0 && d <= 512, DK_ERR_UNSUPPORTED,
               "dk_build_landmarks: d must be a multiple of 8 and <= 512 (got %d)", d);
    DK_REQUIRE(aligned16(K) && aligned16(lm) && strides_ok(ks, esz), DK_ERR_UNSUPPORTED,
               "dk_build_landmarks: K, lm and K's strides must be 16-byte aligned");
    DK_REQUIRE((int64_t)B * Hkv * (L / chunk) < (int64_t)1 << 40, DK_ERR_INVALID_ARG,
               "dk_build_landmarks: too many chunks");
    hipError_t e = dk::launch_landmarks(K, k_dtype, ks, B, Hkv, L, d, chunk, lm, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, "dk_build_landmarks");
}

dk_status dk_build_minmax(const void* K, dk_dtype k_dtype, dk_strides ks, int B, int Hkv, int L, int d, int chunk,
                          void* kmin, void* kmax, void* stream) {
    g_err.clear();
    const char* fn = "dk_build_minmax";
    const int esz = dtype_size(k_dtype);
    DK_REQUIRE(K && kmin && kmax, DK_ERR_INVALID_ARG, "%s: K, kmin and kmax must be non-NULL", fn);
    DK_REQUIRE(esz != 0, DK_ERR_INVALID_ARG, "%s: unknown k_dtype %d", fn, (int)k_dtype);
    DK_REQUIRE(B >= 1 && Hkv >= 1 && L >= 1 && d >= 1 && chunk >= 1, DK_ERR_INVALID_ARG,
               "%s: B, Hkv, L, d, chunk must be >= 1", fn);
    DK_REQUIRE(L % chunk == 0, DK_ERR_INVALID_ARG, "%s: L (%d) %% chunk (%d) != 0", fn, L, chunk);
    DK_REQUIRE(d == 64 || d == 128, DK_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
    DK_REQUIRE(aligned16(K) && aligned16(kmin) && aligned16(kmax) && strides_ok(ks, esz), DK_ERR_UNSUPPORTED,
               "%s: K, kmin, kmax and K's strides must be 16-byte aligned", fn);
    DK_REQUIRE((int64_t)B * Hkv * (L / chunk) < (int64_t)1 << 40, DK_ERR_INVALID_ARG, "%s: too many chunks", fn);
    hipError_t e = dk::launch_build_minmax(K, k_dtype, ks, B, Hkv, L, d, chunk, kmin, kmax, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

dk_status dk_build_landmark_shadow(const float* lm, dk_strides ls, int B, int Hkv, int C, int d, uint8_t* lm8,
                                   float* chunk_scale, float* scale_max, void* stream) {
    g_err.clear();
    DK_REQUIRE(lm && lm8 && chunk_scale && scale_max, DK_ERR_INVALID_ARG,
               "dk_build_landmark_shadow: lm, lm8, chunk_scale, scale_max must be non-NULL");
    DK_REQUIRE(B >= 1 && Hkv >= 1 && C >= 1 && d >= 1, DK_ERR_INVALID_ARG,
               "dk_build_landmark_shadow: B, Hkv, C, d must be >= 1");
    DK_REQUIRE(d == 64 || d == 128, DK_ERR_UNSUPPORTED, "dk_build_landmark_shadow: d must be 64 or 128");
    DK_REQUIRE(aligned16(lm) && aligned16(lm8) && strides_ok(ls, 4), DK_ERR_UNSUPPORTED,
               "dk_build_landmark_shadow: lm, lm8 and lm's strides must be 16-byte aligned");
    hipError_t e = dk::launch_build_shadow(lm, ls, B, Hkv, C, d, lm8, chunk_scale, scale_max, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, "dk_build_landmark_shadow");
}

size_t dk_score_topk_workspace_size(int B, int Hkv, int T, int C, int k, int with_shadow) {
    if (B < 1 || Hkv < 1 || T < 1 || T > 2 || k < 1 || C < k) return 0;
    return dk::plan_topk(B, Hkv, T, C, k, with_shadow != 0).ws_bytes;
}

size_t dk_index_topk_workspace_size(int B, int Hkv, int T, int C) {
    if (B < 1 || Hkv < 1 || T < 1 || T > 2 || C < 1) return 0;
    return dk::plan_index_topk(B, Hkv, T, C).ws_bytes;
}

}  // extern "C"

namespace {

// Argument checks shared by dk_score_topk and dk_score_topk_union; `fn` names
// the entry point in the messages.
dk_status check_score_topk(const char* fn, const float* q, int B, int T, int Hq, const void* lm,
                           dk_dtype lm_dtype, dk_strides ls, int Hkv, int C, int d, int k, float scale,
                           dk_group_reduce reduce, const dk_landmark_shadow* shadow, int32_t* topk_idx,
                           void* ws, size_t ws_bytes, dk::TopkPlan* plan_out) {
    DK_REQUIRE(q && lm && topk_idx, DK_ERR_INVALID_ARG, "%s: q, lm, topk_idx must be non-NULL", fn);
    DK_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && C >= 1 && d >= 1, DK_ERR_INVALID_ARG,
               "%s: B, Hq, Hkv, C, d must be >= 1", fn);
    DK_REQUIRE(T == 1 || T == 2, DK_ERR_INVALID_ARG, "%s: T must be 1 or 2 (got %d)", fn, T);
    DK_REQUIRE(Hq % Hkv == 0, DK_ERR_INVALID_ARG, "%s: Hq (%d) %% Hkv (%d) != 0", fn, Hq, Hkv);
    DK_REQUIRE(k >= 1 && k <= C, DK_ERR_INVALID_ARG, "%s: need 1 <= k (%d) <= C (%d)", fn, k, C);
    DK_REQUIRE(reduce == DK_REDUCE_MEAN || reduce == DK_REDUCE_MAX, DK_ERR_INVALID_ARG,
               "%s: unknown reduce %d", fn, (int)reduce);
    DK_REQUIRE(std::isfinite(scale), DK_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    DK_REQUIRE(!shadow || (shadow->lm8 && shadow->chunk_scale && shadow->scale_max), DK_ERR_INVALID_ARG,
               "%s: shadow->lm8, chunk_scale and scale_max must be non-NULL", fn);
    DK_REQUIRE(lm_dtype == DK_F32, DK_ERR_UNSUPPORTED, "%s: landmarks must be DK_F32", fn);
    DK_REQUIRE(d == 64 || d == 128, DK_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
    DK_REQUIRE(C <= 65536, DK_ERR_UNSUPPORTED, "%s: C must be <= 65536 (got %d)", fn, C);
    const int G = Hq / Hkv;
    if (reduce == DK_REDUCE_MAX) {
        const int nq = G * T;
        DK_REQUIRE(nq <= 16 && (nq & (nq - 1)) == 0, DK_ERR_UNSUPPORTED,
                   "%s: max reduction needs G*T a power of two <= 16 (got %d)", fn, nq);
    }
    DK_REQUIRE(aligned16(q) && aligned16(lm) && strides_ok(ls, 4) && (!shadow || (aligned16(shadow->lm8) && aligned16(shadow->chunk_scale))),
               DK_ERR_UNSUPPORTED, "%s: q, lm, lm's strides, lm8 and chunk_scale must be 16-byte aligned", fn);
    const dk::TopkPlan plan = dk::plan_topk(B, Hkv, T, C, k, shadow != nullptr);
    DK_REQUIRE(plan.splits > 0, DK_ERR_UNSUPPORTED, "%s: no plan for C=%d k=%d%s", fn, C, k,
               shadow ? " with a shadow (C <= 6144)" : "");
    DK_REQUIRE(ws_bytes >= plan.ws_bytes && (plan.ws_bytes == 0 || ws), DK_ERR_INVALID_ARG,
               "%s: workspace needs %zu bytes (got %zu)", fn, plan.ws_bytes, ws_bytes);
    *plan_out = plan;
    return DK_OK;
}

// Argument checks of the token-level path (DK_BF16 indexer keys).
dk_status check_index_topk(const char* fn, const float* q, int B, int T, int Hq, const void* lm, dk_strides ls,
                           int Hkv, int C, int d, int k, float scale, dk_group_reduce reduce,
                           const dk_landmark_shadow* shadow, int32_t* topk_idx, void* ws, size_t ws_bytes,
                           dk::IndexPlan* plan_out) {
    DK_REQUIRE(q && lm && topk_idx, DK_ERR_INVALID_ARG, "%s: q, lm, topk_idx must be non-NULL", fn);
    DK_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && C >= 1 && d >= 1, DK_ERR_INVALID_ARG,
               "%s: B, Hq, Hkv, C, d must be >= 1", fn);
    DK_REQUIRE(T == 1 || T == 2, DK_ERR_INVALID_ARG, "%s: T must be 1 or 2 (got %d)", fn, T);
    DK_REQUIRE(Hq % Hkv == 0, DK_ERR_INVALID_ARG, "%s: Hq (%d) %% Hkv (%d) != 0", fn, Hq, Hkv);
    DK_REQUIRE(k >= 1 && k <= C, DK_ERR_INVALID_ARG, "%s: need 1 <= k (%d) <= C (%d)", fn, k, C);
    DK_REQUIRE(std::isfinite(scale), DK_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    DK_REQUIRE(reduce == DK_REDUCE_MEAN, DK_ERR_UNSUPPORTED, "%s: bf16 indexer keys need DK_REDUCE_MEAN", fn);
    DK_REQUIRE(!shadow, DK_ERR_UNSUPPORTED, "%s: bf16 indexer keys take no shadow", fn);
    DK_REQUIRE(d == 64 || d == 128, DK_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
    DK_REQUIRE(C % 4 == 0 && C <= (1 << 28), DK_ERR_UNSUPPORTED,
               "%s: bf16 indexer keys need C %% 4 == 0 and C <= 2^28 (got %d)", fn, C);
    DK_REQUIRE(aligned16(q) && aligned16(lm) && strides_ok(ls, 2), DK_ERR_UNSUPPORTED,
               "%s: q, the keys and their strides must be 16-byte aligned", fn);
    const dk::IndexPlan plan = dk::plan_index_topk(B, Hkv, T, C);
    DK_REQUIRE(ws && ws_bytes >= plan.ws_bytes, DK_ERR_INVALID_ARG, "%s: workspace needs %zu bytes (got %zu)",
               fn, plan.ws_bytes, ws_bytes);
    *plan_out = plan;
    return DK_OK;
}

// Limits of the union stage (one block per (b, g), everything in LDS).
dk_status check_union(const char* fn, int T, int k, int slots, bool with_plan) {
    const int N = T * k;
    DK_REQUIRE(N <= 8192 && slots <= 8192, DK_ERR_UNSUPPORTED, "%s: T*k and slots must be <= 8192", fn);
    const int64_t lds = (int64_t)(3 * k + 1 + N + 8 + (with_plan ? 2 * slots + N : 0)) * 4;
    DK_REQUIRE(lds <= 65536, DK_ERR_UNSUPPORTED, "%s: k and slots too large for one block", fn);
    return DK_OK;
}

// Attention call shared by dk_sparse_decode_attn and dk_sparse_decode_attn_noalloc:
// the kernel family that runs and the scratch bytes it needs.
struct AttnCall {
    bool latent;          // dk 576 / dv 512 rows on the matrix cores
    dk::AttnPlan plan;
    dk::MlaPlan mla;
    size_t ws_bytes;
};

dk_status check_attn(const char* fn, const float* q, int B, int T, int Hq, int Hkv, const void* K, const void* V,
                     dk_dtype kv_dtype, dk_strides ks, dk_strides vs, int dk, int dv, int chunk,
                     const int32_t* block_ids, const uint8_t* member, const float* out, int pool_blocks, int N,
                     float scale, AttnCall* c) {
    const int esz = dtype_size(kv_dtype);
    DK_REQUIRE(q && K && V && block_ids && out, DK_ERR_INVALID_ARG, "%s: q, K, V, block_ids, out must be non-NULL",
               fn);
    DK_REQUIRE(esz != 0, DK_ERR_INVALID_ARG, "%s: unknown kv_dtype %d", fn, (int)kv_dtype);
    DK_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && dk >= 1 && dv >= 1 && chunk >= 1 && N >= 1 && pool_blocks >= 0,
               DK_ERR_INVALID_ARG, "%s: sizes out of range", fn);
    DK_REQUIRE(T == 1 || T == 2, DK_ERR_INVALID_ARG, "%s: T must be 1 or 2 (got %d)", fn, T);
    DK_REQUIRE(Hq % Hkv == 0, DK_ERR_INVALID_ARG, "%s: Hq (%d) %% Hkv (%d) != 0", fn, Hq, Hkv);
    DK_REQUIRE(member || T == 1, DK_ERR_INVALID_ARG, "%s: member is required when T == 2", fn);
    DK_REQUIRE(std::isfinite(scale), DK_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    if (dk == 576 && dv == 512) {
        // latent rows: the value is the first 512 columns of the key rows
        DK_REQUIRE(kv_dtype == DK_BF16 && chunk == 1, DK_ERR_UNSUPPORTED,
                   "%s: latent attention (dk 576, dv 512) needs bf16 rows and chunk == 1", fn);
        DK_REQUIRE(K == V && ks.b == vs.b && ks.h == vs.h && ks.t == vs.t, DK_ERR_UNSUPPORTED,
                   "%s: latent attention reads the value from the key rows: V must equal K, vs must equal ks", fn);
        DK_REQUIRE(ks.t >= 576 && ks.b >= 0 && ks.h >= 0, DK_ERR_INVALID_ARG,
                   "%s: latent rows need a row stride >= 576", fn);
        const int HB = 64 / T;
        DK_REQUIRE((Hq / Hkv) % HB == 0, DK_ERR_UNSUPPORTED,
                   "%s: latent attention needs Hq/Hkv a multiple of %d (got %d)", fn, HB, Hq / Hkv);
        DK_REQUIRE(aligned16(q) && aligned16(out) && aligned16(K) && strides_ok(ks, 2), DK_ERR_UNSUPPORTED,
                   "%s: q, out, the latent rows and their strides must be 16-byte aligned", fn);
        c->latent = true;
        c->mla = dk::plan_mla(B, Hkv, T, Hq, N);
        c->ws_bytes = c->mla.ws_bytes;
        return DK_OK;
    }
    DK_REQUIRE(dk == dv && (dk == 64 || dk == 128), DK_ERR_UNSUPPORTED,
               "%s: needs dk == dv in {64, 128}, or dk 576 / dv 512 (got %d, %d)", fn, dk, dv);
    DK_REQUIRE((Hq / Hkv) * T <= 16, DK_ERR_UNSUPPORTED, "%s: G*T must be <= 16", fn);
    DK_REQUIRE(aligned16(q) && aligned16(out) && aligned16(K) && aligned16(V) && strides_ok(ks, esz) &&
                   strides_ok(vs, esz),
               DK_ERR_UNSUPPORTED, "%s: q, out, K, V and strides must be 16-byte aligned", fn);
    c->latent = false;
    c->plan = dk::plan_attn(B, Hkv, T, Hq, dv, N, chunk);
    c->ws_bytes = c->plan.ws_bytes;
    return DK_OK;
}

hipError_t run_attn(const AttnCall& c, const float* q, int B, int T, int Hq, int Hkv, const void* K, const void* V,
                    dk_dtype kv_dtype, dk_strides ks, dk_strides vs, int dk, int chunk, const int32_t* block_ids,
                    const uint8_t* member, const int32_t* count, int N, int pool_blocks, float scale, float* out,
                    float* lse, void* ws, hipStream_t st) {
    if (c.latent)
        return dk::launch_mla_attention(q, B, T, Hq, Hkv, K, ks, block_ids, member, count, N, pool_blocks, scale, out,
                                        lse, ws, c.mla, st);
    return dk::launch_attention(q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, dk, chunk, block_ids, member, count, N,
                                pool_blocks, scale, out, lse, ws, c.plan, nullptr, st);
}

}  // namespace

// Scratch of dk_sparse_decode_attn_noalloc, for callers that cannot allocate:
// the attention partials live in this fixed device array instead of a caller
// workspace.  Each device the library runs on holds its own copy until the
// process ends.  In host code `scratch` is only a handle, not a device address:
// the address comes from hipGetSymbolAddress, once per device (static_scratch).
static __device__ __align__(256) unsigned char scratch[64u << 20];

namespace {

constexpr size_t kStaticScratchBytes = sizeof(scratch);
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device that `st` belongs to (the current
// device for the null stream), looked up with that device current on the first
// call for the device and kept.
hipError_t static_scratch(hipStream_t st, void** out) {
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Argument checks of the attention with tail and own rows (dk_sparse_decode_attn_tail,
// dk_decode_step with an extra); `fn` names the entry point in the messages.
dk_status check_attn_tail(const char* fn, const float* q, int B, int T, int Hq, int Hkv, const void* K,
                          const void* V, dk_dtype kv_dtype, dk_strides ks, dk_strides vs, int dk, int dv,
                          int chunk, const int32_t* block_ids, const uint8_t* member, int N, int pool_blocks,
                          const dk_attn_extra* extra, float scale, const float* out, const void* ws,
                          size_t ws_bytes, dk::AttnPlan* plan_out) {
    const int esz = dtype_size(kv_dtype);
    DK_REQUIRE(q && K && V && block_ids && out && extra, DK_ERR_INVALID_ARG,
               "%s: q, K, V, block_ids, out, extra must be non-NULL", fn);
    DK_REQUIRE(esz != 0, DK_ERR_INVALID_ARG, "%s: unknown kv_dtype %d", fn, (int)kv_dtype);
    DK_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && dk >= 1 && dv >= 1 && chunk >= 1 && N >= 1 &&
                   pool_blocks >= 0,
               DK_ERR_INVALID_ARG, "%s: sizes out of range", fn);
    DK_REQUIRE(T == 1 || T == 2, DK_ERR_INVALID_ARG, "%s: T must be 1 or 2 (got %d)", fn, T);
    DK_REQUIRE(Hq % Hkv == 0, DK_ERR_INVALID_ARG, "%s: Hq (%d) %% Hkv (%d) != 0", fn, Hq, Hkv);
    DK_REQUIRE(member || T == 1, DK_ERR_INVALID_ARG, "%s: member is required when T == 2", fn);
    DK_REQUIRE(std::isfinite(scale), DK_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    DK_REQUIRE(!extra->K_tail == !extra->V_tail, DK_ERR_INVALID_ARG,
               "%s: K_tail and V_tail must both be given or both be NULL", fn);
    DK_REQUIRE(!extra->K_new == !extra->V_new, DK_ERR_INVALID_ARG,
               "%s: K_new and V_new must both be given or both be NULL", fn);
    DK_REQUIRE(!extra->K_tail || (extra->tail_max >= 0 && extra->tail_k_s.b >= 0 && extra->tail_k_s.h >= 0 &&
                                  extra->tail_k_s.t >= 0 && extra->tail_v_s.b >= 0 && extra->tail_v_s.h >= 0 &&
                                  extra->tail_v_s.t >= 0),
               DK_ERR_INVALID_ARG, "%s: tail_max and the tail strides must be >= 0", fn);
    DK_REQUIRE(dk == dv && (dk == 64 || dk == 128), DK_ERR_UNSUPPORTED,
               "%s: needs dk == dv in {64, 128} (got %d, %d)", fn, dk, dv);
    DK_REQUIRE((Hq / Hkv) * T <= 16, DK_ERR_UNSUPPORTED, "%s: G*T must be <= 16", fn);
    DK_REQUIRE(aligned16(q) && aligned16(out) && aligned16(K) && aligned16(V) && strides_ok(ks, esz) &&
                   strides_ok(vs, esz) &&
                   (!extra->K_tail || (aligned16(extra->K_tail) && aligned16(extra->V_tail) &&
                                       strides_ok(extra->tail_k_s, esz) && strides_ok(extra->tail_v_s, esz))) &&
                   (!extra->K_new || (aligned16(extra->K_new) && aligned16(extra->V_new))),
               DK_ERR_UNSUPPORTED, "%s: q, out, K, V, the tail and new rows and their strides must be 16-byte aligned",
               fn);
    const dk::AttnPlan plan = dk::plan_attn(B, Hkv, T, Hq, dv, N, chunk, true);
    DK_REQUIRE(ws_bytes >= plan.ws_bytes && (plan.ws_bytes == 0 || ws), DK_ERR_INVALID_ARG,
               "%s: workspace needs %zu bytes (got %zu)", fn, plan.ws_bytes, ws_bytes);
    *plan_out = plan;
    return DK_OK;
}

}  // namespace

extern "C" {

dk_status dk_score_topk(const float* q, int B, int T, int Hq, const void* lm, dk_dtype lm_dtype,
                        dk_strides ls, int Hkv, int C, int d, int k, float scale,
                        dk_group_reduce reduce, const dk_landmark_shadow* shadow, int32_t* topk_idx,
                        float* topk_score, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (lm_dtype == DK_BF16) {
        dk::IndexPlan ip{};
        const dk_status s = check_index_topk("dk_score_topk", q, B, T, Hq, lm, ls, Hkv, C, d, k, scale, reduce,
                                             shadow, topk_idx, ws, ws_bytes, &ip);
        if (s != DK_OK) return s;
        hipError_t e = dk::launch_index_topk(q, B, T, Hq, (const uint16_t*)lm, ls, Hkv, C, d, k, scale, topk_idx,
                                             topk_score, ws, ip, nullptr, (hipStream_t)stream);
        return e == hipSuccess ? DK_OK : hip_fail(e, "dk_score_topk");
    }
    dk::TopkPlan plan{};
    const dk_status s = check_score_topk("dk_score_topk", q, B, T, Hq, lm, lm_dtype, ls, Hkv, C, d, k, scale,
                                         reduce, shadow, topk_idx, ws, ws_bytes, &plan);
    if (s != DK_OK) return s;
    hipError_t e = dk::launch_score_topk(q, B, T, Hq, (const float*)lm, ls, Hkv, C, d, k, scale, reduce,
                                         shadow, topk_idx, topk_score, ws, plan, nullptr, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, "dk_score_topk");
}

dk_status dk_score_topk_union(const float* q, int B, int T, int Hq, const void* lm, dk_dtype lm_dtype,
                              dk_strides ls, int Hkv, int C, int d, int k, float scale,
                              dk_group_reduce reduce, const dk_landmark_shadow* shadow,
                              int32_t* topk_idx, float* topk_score, int32_t* union_ids, uint8_t* member,
                              int32_t* union_count, int32_t* overlap, void* ws, size_t ws_bytes,
                              void* stream) {
    g_err.clear();
    const char* fn = "dk_score_topk_union";
    if (lm_dtype == DK_BF16) {
        dk::IndexPlan ip{};
        dk_status s = check_index_topk(fn, q, B, T, Hq, lm, ls, Hkv, C, d, k, scale, reduce, shadow, topk_idx, ws,
                                       ws_bytes, &ip);
        if (s != DK_OK) return s;
        DK_REQUIRE(union_ids && member && union_count, DK_ERR_INVALID_ARG,
                   "%s: union_ids, member, union_count must be non-NULL", fn);
        s = check_union(fn, T, k, 0, false);
        if (s != DK_OK) return s;
        const dk::UnionOut un{union_ids, member, union_count, overlap};
        hipError_t e = dk::launch_index_topk(q, B, T, Hq, (const uint16_t*)lm, ls, Hkv, C, d, k, scale, topk_idx,
                                             topk_score, ws, ip, &un, (hipStream_t)stream);
        return e == hipSuccess ? DK_OK : hip_fail(e, fn);
    }
    dk::TopkPlan plan{};
    dk_status s = check_score_topk(fn, q, B, T, Hq, lm, lm_dtype, ls, Hkv, C, d, k, scale, reduce, shadow,
                                   topk_idx, ws, ws_bytes, &plan);
    if (s != DK_OK) return s;
    DK_REQUIRE(union_ids && member && union_count, DK_ERR_INVALID_ARG,
               "%s: union_ids, member, union_count must be non-NULL", fn);
    s = check_union(fn, T, k, 0, false);
    if (s != DK_OK) return s;
    const dk::UnionOut un{union_ids, member, union_count, overlap};
    hipError_t e = dk::launch_score_topk(q, B, T, Hq, (const float*)lm, ls, Hkv, C, d, k, scale, reduce,
                                         shadow, topk_idx, topk_score, ws, plan, &un, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

dk_status dk_score_topk_minmax(const float* q, int B, int T, int Hq, const void* kmin, const void* kmax,
                               dk_dtype dtype, dk_strides ss, int Hkv, int C, int d, int k, float scale,
                               dk_group_reduce reduce, int32_t* topk_idx, float* topk_score, int32_t* union_ids,
                               uint8_t* member, int32_t* union_count, int32_t* overlap, void* ws, size_t ws_bytes,
                               void* stream) {
    g_err.clear();
    const char* fn = "dk_score_topk_minmax";
    const int esz = dtype_size(dtype);
    DK_REQUIRE(q && kmin && kmax && topk_idx, DK_ERR_INVALID_ARG, "%s: q, kmin, kmax, topk_idx must be non-NULL", fn);
    DK_REQUIRE(esz != 0, DK_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    DK_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && C >= 1 && d >= 1, DK_ERR_INVALID_ARG,
               "%s: B, Hq, Hkv, C, d must be >= 1", fn);
    DK_REQUIRE(T == 1 || T == 2, DK_ERR_INVALID_ARG, "%s: T must be 1 or 2 (got %d)", fn, T);
    DK_REQUIRE(Hq % Hkv == 0, DK_ERR_INVALID_ARG, "%s: Hq (%d) %% Hkv (%d) != 0", fn, Hq, Hkv);
    DK_REQUIRE(k >= 1 && k <= C, DK_ERR_INVALID_ARG, "%s: need 1 <= k (%d) <= C (%d)", fn, k, C);
    DK_REQUIRE(reduce == DK_REDUCE_MEAN || reduce == DK_REDUCE_MAX, DK_ERR_INVALID_ARG, "%s: unknown reduce %d", fn,
               (int)reduce);
    DK_REQUIRE(std::isfinite(scale), DK_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    DK_REQUIRE(!union_ids || (member && union_count), DK_ERR_INVALID_ARG,
               "%s: with union_ids, member and union_count must be non-NULL", fn);
    DK_REQUIRE(d == 64 || d == 128, DK_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
    DK_REQUIRE(C % 4 == 0 && C <= (1 << 28), DK_ERR_UNSUPPORTED, "%s: needs C %% 4 == 0 and C <= 2^28 (got %d)",
               fn, C);
    const int G = Hq / Hkv;
    if (reduce == DK_REDUCE_MAX) {
        const int nq = G * T;
        DK_REQUIRE(nq <= 8 && (nq & (nq - 1)) == 0, DK_ERR_UNSUPPORTED,
                   "%s: max reduction needs G*T a power of two <= 8 (got %d)", fn, nq);
    }
    DK_REQUIRE(aligned16(q) && aligned16(kmin) && aligned16(kmax) && strides_ok(ss, esz), DK_ERR_UNSUPPORTED,
               "%s: q, kmin, kmax and the summaries' strides must be 16-byte aligned", fn);
    const dk::IndexPlan plan = dk::plan_index_topk(B, Hkv, T, C);
    DK_REQUIRE(ws && ws_bytes >= plan.ws_bytes, DK_ERR_INVALID_ARG, "%s: workspace needs %zu bytes (got %zu)", fn,
               plan.ws_bytes, ws_bytes);
    if (union_ids) {
        const dk_status s = check_union(fn, T, k, 0, false);
        if (s != DK_OK) return s;
    }
    const dk::UnionOut un{union_ids, member, union_count, overlap};
    hipError_t e = dk::launch_minmax_topk(q, B, T, Hq, kmin, kmax, dtype, ss, Hkv, C, d, k, scale, reduce, topk_idx,
                                          topk_score, ws, plan, union_ids ? &un : nullptr, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

size_t dk_coverage_workspace_size(int B, int Hkv, int T, int C) {
    if (B < 1 || Hkv < 1 || T < 1 || T > 2 || C < 1) return 0;
    return dk::plan_index_topk(B, Hkv, T, C).ws_bytes;
}

dk_status dk_score_coverage(const float* q, int B, int T, int Hq, const void* lm, dk_dtype lm_dtype,
                            dk_strides ls, int Hkv, int C, int d, float scale, dk_group_reduce reduce,
                            float gamma, int k_max, int32_t* sel_idx, int32_t* sel_count, float* sel_score,
                            int32_t* union_ids, uint8_t* member, int32_t* union_count, int32_t* overlap,
                            void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    const char* fn = "dk_score_coverage";
    const int esz = dtype_size(lm_dtype);
    DK_REQUIRE(q && lm && sel_idx && sel_count, DK_ERR_INVALID_ARG,
               "%s: q, lm, sel_idx, sel_count must be non-NULL", fn);
    DK_REQUIRE(esz != 0, DK_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)lm_dtype);
    DK_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && C >= 1 && d >= 1, DK_ERR_INVALID_ARG,
               "%s: B, Hq, Hkv, C, d must be >= 1", fn);
    DK_REQUIRE(T == 1 || T == 2, DK_ERR_INVALID_ARG, "%s: T must be 1 or 2 (got %d)", fn, T);
    DK_REQUIRE(Hq % Hkv == 0, DK_ERR_INVALID_ARG, "%s: Hq (%d) %% Hkv (%d) != 0", fn, Hq, Hkv);
    DK_REQUIRE(k_max >= 1 && k_max <= C, DK_ERR_INVALID_ARG, "%s: need 1 <= k_max (%d) <= C (%d)", fn, k_max, C);
    DK_REQUIRE(gamma > 0.0f && gamma <= 1.0f, DK_ERR_INVALID_ARG, "%s: need 0 < gamma <= 1 (got %g)", fn,
               (double)gamma);
    DK_REQUIRE(reduce == DK_REDUCE_MEAN || reduce == DK_REDUCE_MAX, DK_ERR_INVALID_ARG, "%s: unknown reduce %d", fn,
               (int)reduce);
    DK_REQUIRE(std::isfinite(scale), DK_ERR_INVALID_ARG, "%s: scale must be finite", fn);
    DK_REQUIRE(!union_ids || (member && union_count), DK_ERR_INVALID_ARG,
               "%s: with union_ids, member and union_count must be non-NULL", fn);
    DK_REQUIRE(d == 64 || d == 128, DK_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
    DK_REQUIRE(C <= dk::kCoverageMaxC, DK_ERR_UNSUPPORTED, "%s: C must be <= %d (got %d)", fn, dk::kCoverageMaxC,
               C);
    if (reduce == DK_REDUCE_MAX) {
        const int nq = (Hq / Hkv) * T;
        DK_REQUIRE(nq <= 8 && (nq & (nq - 1)) == 0, DK_ERR_UNSUPPORTED,
                   "%s: max reduction needs G*T a power of two <= 8 (got %d)", fn, nq);
    }
    DK_REQUIRE(aligned16(q) && aligned16(lm) && strides_ok(ls, esz), DK_ERR_UNSUPPORTED,
               "%s: q, lm and lm's strides must be 16-byte aligned", fn);
    const dk::IndexPlan plan = dk::plan_index_topk(B, Hkv, T, C);
    DK_REQUIRE(ws && ws_bytes >= plan.ws_bytes, DK_ERR_INVALID_ARG, "%s: workspace needs %zu bytes (got %zu)", fn,
               plan.ws_bytes, ws_bytes);
    const dk::UnionOut un{union_ids, member, union_count, overlap};
    hipError_t e = dk::launch_coverage(q, B, T, Hq, lm, lm_dtype, ls, Hkv, C, d, scale, reduce, gamma, k_max, sel_idx,
                                       sel_count, sel_score, union_ids ? &un : nullptr, ws, plan, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

dk_status dk_capped_plan(const int32_t* sel_ids, const float* sel_score, const int32_t* sel_count, int B, int Hkv,
                         int N, int sel_stride, int count_stride, int32_t* resident, int32_t* stamp, int slots,
                         int cap, int32_t step, int32_t* sel_slot, int32_t* admit_chunk, int32_t* admit_slot,
                         int32_t* admit_count, int32_t* hit_count, void* stream) {
    g_err.clear();
    const char* fn = "dk_capped_plan";
    DK_REQUIRE(sel_ids && resident && stamp && sel_slot && admit_count, DK_ERR_INVALID_ARG,
               "%s: sel_ids, resident, stamp, sel_slot, admit_count must be non-NULL", fn);
    DK_REQUIRE(B >= 1 && Hkv >= 1 && N >= 1 && slots >= 1, DK_ERR_INVALID_ARG, "%s: B, Hkv, N, slots must be >= 1",
               fn);
    DK_REQUIRE(sel_stride >= N, DK_ERR_INVALID_ARG, "%s: sel_stride (%d) must be >= N (%d)", fn, sel_stride, N);
    DK_REQUIRE(!sel_count || count_stride >= 1, DK_ERR_INVALID_ARG, "%s: count_stride must be >= 1", fn);
    DK_REQUIRE(cap >= 0 && cap <= (1 << 20), DK_ERR_INVALID_ARG, "%s: need 0 <= cap <= 2^20 (got %d)", fn, cap);
    DK_REQUIRE(cap == 0 || (admit_chunk && admit_slot), DK_ERR_INVALID_ARG,
               "%s: admit_chunk and admit_slot must be non-NULL when cap > 0", fn);
    DK_REQUIRE(N <= dk::kCappedMaxN && slots <= dk::kCappedMaxN, DK_ERR_UNSUPPORTED,
               "%s: N and slots must be <= %d (got %d, %d)", fn, dk::kCappedMaxN, N, slots);
    hipError_t e = dk::launch_capped_plan(sel_ids, sel_score, sel_count, B, Hkv, N, sel_stride, count_stride, resident,
                                          stamp, slots, cap, step, sel_slot, admit_chunk, admit_slot, admit_count,
                                          hit_count, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

dk_status dk_union_select(const int32_t* topk_idx, int B, int Hkv, int T, int k, int C,
                          int32_t* union_ids, uint8_t* member, int32_t* union_count,
                          int32_t* overlap, const dk_cache_plan* plan, void* stream) {
    g_err.clear();
    DK_REQUIRE(topk_idx && union_ids && member && union_count, DK_ERR_INVALID_ARG,
               "dk_union_select: topk_idx, union_ids, member, union_count must be non-NULL");
    DK_REQUIRE(B >= 1 && Hkv >= 1, DK_ERR_INVALID_ARG, "dk_union_select: B, Hkv must be >= 1");
    DK_REQUIRE(T == 1 || T == 2, DK_ERR_INVALID_ARG, "dk_union_select: T must be 1 or 2 (got %d)", T);
    DK_REQUIRE(k >= 1 && k <= C && C <= (1 << 30), DK_ERR_INVALID_ARG,
               "dk_union_select: need 1 <= k (%d) <= C (%d) <= 2^30", k, C);
    const int N = T * k;
    int slots = 0;
    if (plan) {
        DK_REQUIRE(plan->resident && plan->slot_of_union && plan->miss_chunk && plan->miss_slot &&
                       plan->miss_count && plan->hit_count,
                   DK_ERR_INVALID_ARG, "dk_union_select: every cache-plan array must be non-NULL");
        DK_REQUIRE(plan->slots >= N, DK_ERR_INVALID_ARG,
                   "dk_union_select: cache slots (%d) must be >= T*k (%d)", plan->slots, N);
        slots = plan->slots;
    }
    const dk_status s = check_union("dk_union_select", T, k, slots, plan != nullptr);
    if (s != DK_OK) return s;
    hipError_t e = dk::launch_union(topk_idx, B, Hkv, T, k, C, union_ids, member, union_count, overlap,
                                    plan, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, "dk_union_select");
}

dk_status dk_gather_kv(const void* K_src, const void* V_src, dk_dtype dt, dk_strides src_s, int B,
                       int Hkv, int chunk, int d, const int32_t* src_chunk, const int32_t* dst_slot,
                       const int32_t* count, int N, int src_blocks, void* K_dst, void* V_dst,
                       dk_strides dst_s, int dst_blocks, int src_kind, void* stream) {
    g_err.clear();
    const int esz = dtype_size(dt);
    DK_REQUIRE(K_src && V_src && K_dst && V_dst && src_chunk, DK_ERR_INVALID_ARG,
               "dk_gather_kv: K_src, V_src, K_dst, V_dst, src_chunk must be non-NULL");
    DK_REQUIRE(esz != 0, DK_ERR_INVALID_ARG, "dk_gather_kv: unknown dtype %d", (int)dt);
    DK_REQUIRE(B >= 1 && Hkv >= 1 && chunk >= 1 && d >= 1 && N >= 0 && src_blocks >= 0 && dst_blocks >= 0,
               DK_ERR_INVALID_ARG, "dk_gather_kv: sizes out of range");
    DK_REQUIRE(src_kind == DK_SRC_DEVICE || src_kind == DK_SRC_HOST_COPY || src_kind == DK_SRC_HOST_MAPPED,
               DK_ERR_INVALID_ARG, "dk_gather_kv: src_kind must be 0, 1 or 2 (got %d)", src_kind);
    DK_REQUIRE(src_s.b >= 0 && src_s.h >= 0 && src_s.t >= 0 && dst_s.b >= 0 && dst_s.h >= 0 && dst_s.t >= 0,
               DK_ERR_INVALID_ARG, "dk_gather_kv: strides must be >= 0");
    DK_REQUIRE(aligned16(K_src) && aligned16(V_src) && aligned16(K_dst) && aligned16(V_dst) &&
                   strides_ok(src_s, esz) && strides_ok(dst_s, esz) && (d * esz) % 16 == 0,
               DK_ERR_UNSUPPORTED, "dk_gather_kv: pools, strides and rows must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    if (N == 0) return DK_OK;
    const void* Ks = K_src;
    const void* Vs = V_src;
    if (src_kind != DK_SRC_DEVICE) {
        void* km = mapped_host_ptr(K_src);
        void* vm = mapped_host_ptr(V_src);
        DK_REQUIRE(km && vm, DK_ERR_INVALID_ARG,
                   "dk_gather_kv: a host source pool must be pinned host memory (hipHostMalloc)");
        Ks = km;
        Vs = vm;
    }
    if (src_kind == DK_SRC_DEVICE) {
        hipError_t e = dk::launch_gather(Ks, Vs, dt, src_s, B, Hkv, chunk, d, src_chunk, dst_slot,
                                         count, N, src_blocks, K_dst, V_dst, dst_s, dst_blocks, st);
        return e == hipSuccess ? DK_OK : hip_fail(e, "dk_gather_kv");
    }
    if (src_kind == DK_SRC_HOST_MAPPED) {
        hipError_t e = dk::launch_gather_stream(Ks, Vs, dt, src_s, B, Hkv, chunk, d, src_chunk, dst_slot,
                                                count, N, src_blocks, K_dst, V_dst, dst_s, dst_blocks, st);
        return e == hipSuccess ? DK_OK : hip_fail(e, "dk_gather_kv");
    }
    // Host pool: one copy per run of consecutive source chunks going to
    // consecutive slots (rows of consecutive chunks are adjacent when the row
    // stride equals the row width; otherwise every chunk is its own 2-D copy).
    const size_t row_bytes = (size_t)d * esz;
    const size_t spitch = (size_t)src_s.t * esz, dpitch = (size_t)dst_s.t * esz;
    const bool merge_runs = spitch == row_bytes && dpitch == row_bytes;
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            const int64_t bg = (int64_t)b * Hkv + g;
            int n = count ? count[bg] : N;
            n = n < 0 ? 0 : (n > N ? N : n);
            int j = 0;
            while (j < n) {
                const int c = src_chunk[bg * N + j];
                const int s = dst_slot ? dst_slot[bg * N + j] : j;
                if (c < 0 || c >= src_blocks || s < 0 || s >= dst_blocks) { ++j; continue; }
                int run = 1;
                if (merge_runs) {
                    while (j + run < n) {
                        const int c2 = src_chunk[bg * N + j + run];
                        const int s2 = dst_slot ? dst_slot[bg * N + j + run] : j + run;
                        if (c2 != c + run || s2 != s + run || c2 >= src_blocks || s2 >= dst_blocks) break;
                        ++run;
                    }
                }
                const int64_t so = ((int64_t)b * src_s.b + (int64_t)g * src_s.h + (int64_t)c * chunk * src_s.t) * esz;
                const int64_t dof = ((int64_t)b * dst_s.b + (int64_t)g * dst_s.h + (int64_t)s * chunk * dst_s.t) * esz;
                const size_t rows = (size_t)run * chunk;
                hipError_t e;
                if (merge_runs) {
                    e = hipMemcpyAsync((char*)K_dst + dof, (const char*)K_src + so, rows * row_bytes,
                                       hipMemcpyHostToDevice, st);
                    if (e == hipSuccess)
                        e = hipMemcpyAsync((char*)V_dst + dof, (const char*)V_src + so, rows * row_bytes,
                                           hipMemcpyHostToDevice, st);
                } else {
                    e = hipMemcpy2DAsync((char*)K_dst + dof, dpitch, (const char*)K_src + so, spitch,
                                         row_bytes, rows, hipMemcpyHostToDevice, st);
                    if (e == hipSuccess)
                        e = hipMemcpy2DAsync((char*)V_dst + dof, dpitch, (const char*)V_src + so, spitch,
                                             row_bytes, rows, hipMemcpyHostToDevice, st);
                }
                if (e != hipSuccess) return hip_fail(e, "dk_gather_kv (host)");
                j += run;
            }
        }
    }
    return DK_OK;
}

size_t dk_attn_workspace_size(int B, int Hkv, int T, int Hq, int dv, int N, int chunk) {
    if (B < 1 || Hkv < 1 || T < 1 || T > 2 || Hq < 1 || Hq % Hkv || dv < 1 || N < 1 || chunk < 1)
        return 0;
    if (dv == 512 && chunk == 1) return dk::plan_mla(B, Hkv, T, Hq, N).ws_bytes;
    return dk::plan_attn(B, Hkv, T, Hq, dv, N, chunk).ws_bytes;
}

dk_status dk_sparse_decode_attn(const float* q, int B, int T, int Hq, int Hkv, const void* K,
                                const void* V, dk_dtype kv_dtype, dk_strides ks, dk_strides vs, int dk,
                                int dv, int chunk, const int32_t* block_ids, const uint8_t* member,
                                const int32_t* count, int N, int pool_blocks, float scale, float* out,
                                float* lse, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    const char* fn = "dk_sparse_decode_attn";
    AttnCall c{};
    dk_status s = check_attn(fn, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, dk, dv, chunk, block_ids, member,
                             out, pool_blocks, N, scale, &c);
    if (s != DK_OK) return s;
    DK_REQUIRE(ws_bytes >= c.ws_bytes && (c.ws_bytes == 0 || ws), DK_ERR_INVALID_ARG,
               "%s: workspace needs %zu bytes (got %zu)", fn, c.ws_bytes, ws_bytes);
    hipError_t e = run_attn(c, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, dk, chunk, block_ids, member, count, N,
                            pool_blocks, scale, out, lse, ws, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

size_t dk_decode_step_workspace_size(int B, int Hkv, int T, int Hq, int C, int d, int k, int chunk,
                                     int with_shadow, int with_tail) {
    if (B < 1 || Hkv < 1 || T < 1 || Hq < 1 || C < 1 || d < 1 || k < 1 || chunk < 1) return 0;
    const size_t a = dk_score_topk_workspace_size(B, Hkv, T, C, k, with_shadow);
    const size_t b = with_tail ? dk_attn_tail_workspace_size(B, Hkv, T, Hq, d, T * k, chunk)
                               : dk_attn_workspace_size(B, Hkv, T, Hq, d, T * k, chunk);
    return a > b ? a : b;
}

dk_status dk_decode_step(const float* q, int B, int T, int Hq, int Hkv, const void* lm, dk_dtype lm_dtype,
                         dk_strides ls, int C, int d, int k, float scale, dk_group_reduce reduce,
                         const dk_landmark_shadow* shadow, const void* K, const void* V, dk_dtype kv_dtype,
                         dk_strides ks, dk_strides vs, int chunk, const dk_attn_extra* extra,
                         int32_t* topk_idx, float* topk_score,
                         int32_t* union_ids, uint8_t* member, int32_t* union_count, int32_t* overlap, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    const char* fn = "dk_decode_step";
    DK_REQUIRE(lm_dtype == DK_F32, DK_ERR_UNSUPPORTED, "%s: landmarks must be DK_F32", fn);
    dk::TopkPlan tplan{};
    // the two calls' checks, before anything is enqueued (the workspace serves them in turn)
    dk_status s = check_score_topk(fn, q, B, T, Hq, lm, lm_dtype, ls, Hkv, C, d, k, scale, reduce, shadow, topk_idx,
                                   ws, ws_bytes, &tplan);
    if (s != DK_OK) return s;
    DK_REQUIRE(union_ids && member && union_count, DK_ERR_INVALID_ARG,
               "%s: union_ids, member, union_count must be non-NULL", fn);
    s = check_union(fn, T, k, 0, false);
    if (s != DK_OK) return s;
    AttnCall c{};
    dk::AttnPlan tail_plan{};
    if (extra) {
        s = check_attn_tail(fn, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, d, d, chunk, union_ids, member, T * k, C,
                            extra, scale, out, ws, ws_bytes, &tail_plan);
        if (s != DK_OK) return s;
        c.plan = tail_plan;
    } else {
        s = check_attn(fn, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, d, d, chunk, union_ids, member, out, C, T * k,
                       scale, &c);
        if (s != DK_OK) return s;
        DK_REQUIRE(ws_bytes >= c.ws_bytes && (c.ws_bytes == 0 || ws), DK_ERR_INVALID_ARG,
                   "%s: workspace needs %zu bytes (got %zu)", fn,
                   c.ws_bytes > tplan.ws_bytes ? c.ws_bytes : tplan.ws_bytes, ws_bytes);
    }
    const dk::UnionOut un{union_ids, member, union_count, overlap};
    const hipStream_t st = (hipStream_t)stream;
    const dk::AttnTail tail = extra ? dk::AttnTail{extra->K_tail, extra->V_tail, extra->tail_k_s, extra->tail_v_s,
                                                   extra->tail_len, extra->K_tail ? extra->tail_max : 0,
                                                   extra->K_new, extra->V_new}
                                    : dk::AttnTail{};
    // One kernel when every (b, g) is one block of each call: the shadow selection
    // with its union in the block (k + 1 <= 256), the attention fast path with one
    // range per (b, g) and no partials, and 512 threads per selection block.  Not
    // with tail rows: their addressing takes the fused kernel past 128 registers, one
    // block per CU instead of two (measured slower than the two calls' kernels).
    const bool fused = shadow && reduce == DK_REDUCE_MEAN && T == 2 && Hq == 4 * Hkv && d == 128 && !c.latent &&
                       dk::use_fast_path(kv_dtype, d, Hq / Hkv, T, chunk, ks, vs) && c.plan.splits == 1 &&
                       c.plan.nparts == 1 && !extra && k + 1 <= 256 && (int64_t)B * Hkv > 256;
    hipError_t e;
    if (fused) {
        e = dk::launch_step_fused(q, B, Hq, Hkv, C, k, scale, shadow, (const float*)lm, ls, K, V, ks, vs, chunk,
                                  topk_idx, topk_score, un, out, lse, st);
    } else {
        e = dk::launch_score_topk(q, B, T, Hq, (const float*)lm, ls, Hkv, C, d, k, scale, reduce, shadow, topk_idx,
                                  topk_score, ws, tplan, &un, st);
        if (e == hipSuccess && extra)
            e = dk::launch_attention(q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, d, chunk, union_ids, member,
                                     union_count, T * k, C, scale, out, lse, ws, tail_plan, &tail, st);
        else if (e == hipSuccess)
            e = run_attn(c, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, d, chunk, union_ids, member, union_count,
                         T * k, C, scale, out, lse, ws, st);
    }
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

dk_status dk_sparse_decode_attn_noalloc(const float* q, int B, int T, int Hq, int Hkv, const void* K,
                                        const void* V, dk_dtype kv_dtype, dk_strides ks, dk_strides vs, int dk,
                                        int dv, int chunk, const int32_t* block_ids, const uint8_t* member,
                                        const int32_t* count, int N, int pool_blocks, float scale, float* out,
                                        float* lse, void* stream) {
    g_err.clear();
    const char* fn = "dk_sparse_decode_attn_noalloc";
    AttnCall c{};
    dk_status s = check_attn(fn, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, dk, dv, chunk, block_ids, member,
                             out, pool_blocks, N, scale, &c);
    if (s != DK_OK) return s;
    DK_REQUIRE(c.ws_bytes <= kStaticScratchBytes, DK_ERR_UNSUPPORTED,
               "%s: this shape needs %zu bytes of scratch, more than the library's fixed %zu; use "
               "dk_sparse_decode_attn with a workspace", fn, c.ws_bytes, kStaticScratchBytes);
    void* ws = nullptr;
    hipError_t e = hipSuccess;
    if (c.ws_bytes > 0) {
        e = static_scratch((hipStream_t)stream, &ws);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    e = run_attn(c, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, dk, chunk, block_ids, member, count, N, pool_blocks,
                 scale, out, lse, ws, (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

size_t dk_attn_tail_workspace_size(int B, int Hkv, int T, int Hq, int dv, int N, int chunk) {
    if (B < 1 || Hkv < 1 || T < 1 || T > 2 || Hq < 1 || Hq % Hkv || dv < 1 || N < 1 || chunk < 1)
        return 0;
    return dk::plan_attn(B, Hkv, T, Hq, dv, N, chunk, true).ws_bytes;
}

dk_status dk_sparse_decode_attn_tail(const float* q, int B, int T, int Hq, int Hkv, const void* K,
                                     const void* V, dk_dtype kv_dtype, dk_strides ks, dk_strides vs,
                                     int dk, int dv, int chunk, const int32_t* block_ids,
                                     const uint8_t* member, const int32_t* count, int N, int pool_blocks,
                                     const dk_attn_extra* extra, float scale, float* out, float* lse,
                                     void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    const char* fn = "dk_sparse_decode_attn_tail";
    dk::AttnPlan plan{};
    dk_status s = check_attn_tail(fn, q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, dk, dv, chunk, block_ids, member, N,
                                  pool_blocks, extra, scale, out, ws, ws_bytes, &plan);
    if (s != DK_OK) return s;
    const dk::AttnTail tail{extra->K_tail, extra->V_tail, extra->tail_k_s, extra->tail_v_s, extra->tail_len,
                            extra->K_tail ? extra->tail_max : 0, extra->K_new, extra->V_new};
    hipError_t e = dk::launch_attention(q, B, T, Hq, Hkv, K, V, kv_dtype, ks, vs, dk, chunk, block_ids,
                                        member, count, N, pool_blocks, scale, out, lse, ws, plan, &tail,
                                        (hipStream_t)stream);
    return e == hipSuccess ? DK_OK : hip_fail(e, fn);
}

}  // extern "C"
