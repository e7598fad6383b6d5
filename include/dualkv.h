/*
 * dualkv.h - C ABI of libdualkv: one decode step of dual-query sparse KV-cache
 * retrieval attention on MI355X (gfx950).
 *
 * The step, per request b, KV head g and query t (t = 0 the real token, t = 1
 * the speculative look-ahead token), is:
 *   landmarks  -> dk_build_landmarks     (once per prefilled pool)
 *   scores     -> dk_score_topk          (chunk scores and the k best chunks)
 *   union      -> dk_union_select        (one list of distinct chunks, plus an
 *                                         optional hot-cache transfer plan)
 *   gather     -> dk_gather_kv           (chunk copies; fused into attention on
 *                                         the HBM-pool path)
 *   attention  -> dk_sparse_decode_attn  (each query over its own chunks)
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers are owned by the caller.  The library never allocates or frees
 *   memory; calls that need scratch space take a workspace pointer whose size
 *   comes from the matching *_workspace_size function.
 * - `stream` is a hipStream_t passed as void*; NULL is the null stream.  Every
 *   call only enqueues work on `stream` and returns, except dk_gather_kv in
 *   host mode, which reads its host-side lists while it enqueues copies.
 * - Arguments are checked before anything is enqueued.  A call that returns
 *   anything other than DK_OK has enqueued nothing and written nothing; the
 *   reason is in dk_last_error().  HIP failures return DK_ERR_HIP with the HIP
 *   error string.  One exception: dk_gather_kv with DK_SRC_HOST_COPY issues one
 *   copy per run of chunks, and when the HIP runtime fails partway (DK_ERR_HIP)
 *   the copies issued before the failure stay enqueued; the destination slots
 *   are then undefined.
 * - Tensors are dense in their last dimension.  KV pools are described by a
 *   base pointer and dk_strides {b, h, t}: the element offset of row n of
 *   (request b, head g) is b*s.b + g*s.h + n*s.t.  Pool and landmark rows must
 *   start on 16-byte boundaries (base pointer and every stride, in bytes, are
 *   multiples of 16).
 * - Chunk ids, slot ids and counts are int32.  Ids that fall outside the range
 *   a call is told about (pool_blocks, C, slots) are skipped on the device,
 *   never dereferenced.
 * - The library keeps no global state besides the thread-local error string;
 *   calls on different streams may run concurrently.
 */
#ifndef DUALKV_H
#define DUALKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DK_ABI_VERSION 14

typedef enum {
    DK_OK = 0,
    DK_ERR_INVALID_ARG = 1,   /* a size, pointer or stride is out of range       */
    DK_ERR_UNSUPPORTED = 2,   /* valid, but a shape or alignment v1 does not run */
    DK_ERR_HIP = 3            /* the HIP runtime reported an error               */
} dk_status;

typedef enum { DK_F32 = 0, DK_BF16 = 1 } dk_dtype;

/* How the G query heads of one KV head combine into one chunk score. */
typedef enum { DK_REDUCE_MEAN = 0, DK_REDUCE_MAX = 1 } dk_group_reduce;

/* Where dk_gather_kv reads its source pool from. */
typedef enum {
    DK_SRC_DEVICE = 0,       /* device memory; one kernel                                  */
    DK_SRC_HOST_COPY = 1,    /* pinned host memory; one hipMemcpyAsync per run of chunks   */
    DK_SRC_HOST_MAPPED = 2   /* pinned host memory read by the gather kernel through its
                                device mapping (zero-copy over PCIe); one kernel            */
} dk_src_kind;

typedef struct { int64_t b, h, t; } dk_strides;   /* element strides of dims 0, 1, 2 */

/* ABI version of the loaded library (DK_ABI_VERSION it was built with). */
int dk_abi_version(void);

/* Text of the last failure on the calling thread; valid until its next dk_* call. */
const char* dk_last_error(void);

/*
 * dk_build_landmarks - the mean key of every chunk.
 *
 * DualDecoder (arXiv 2607.26475), "2.2 Dynamic Sparse KV Cache": adjacent KV
 * entries are grouped into chunks, each summarised by a GPU-resident landmark;
 * "4.1 KV Retrieval Predictability": landmarks are built before decoding and
 * stay fixed.  The landmark is the arithmetic mean of the chunk's keys.
 *
 *   lm[b, g, c, :] = (1 / chunk) * sum_{n = c*chunk}^{c*chunk + chunk - 1} K[b, g, n, :]
 *
 * K       : keys, k_dtype (DK_F32 or DK_BF16), rows [B, Hkv, L] of d elements,
 *           strides ks.  Read only.
 * lm      : out, fp32 [B, Hkv, C, d] contiguous, C = L / chunk.  Sums are kept in fp32.
 * Errors  : DK_ERR_INVALID_ARG unless B, Hkv, L, d, chunk >= 1, L % chunk == 0 and
 *           K, lm non-NULL; DK_ERR_UNSUPPORTED unless d % 8 == 0, d <= 512 and
 *           the 16-byte alignment rule holds.
 */
dk_status dk_build_landmarks(const void* K, dk_dtype k_dtype, dk_strides ks,
                             int B, int Hkv, int L, int d, int chunk,
                             float* lm, void* stream);

/*
 * Landmark shadow: 8-bit codes of the landmarks with one scale per chunk.  It
 * lets dk_score_topk stream a quarter of the fp32 landmark bytes and still
 * return exactly the k chunks that scoring with the fp32 landmarks returns:
 * every chunk whose shadow score is within a proven error bound of the k-th
 * score is re-scored from the fp32 landmarks before the final selection.  For
 * chunk c, s_c = max_i |lm[c, i]| / 127, and byte i is rint(lm[c, i] / s_c) + 128
 * (|code - 128| <= 127), so |lm[c, i] - s_c (byte - 128)| <= s_c (1/2 + 127 u).
 * Made once per pool by dk_build_landmark_shadow.
 */
typedef struct {
    const uint8_t* lm8;         /* codes [B, Hkv, C, d], contiguous                        */
    const float*   chunk_scale; /* [B, Hkv, C]: s_c                                        */
    const float*   scale_max;   /* [B, Hkv]: max_c s_c, or +inf when a landmark is not finite */
} dk_landmark_shadow;

/*
 * dk_build_landmark_shadow - 8-bit codes and per-chunk scales of fp32 landmarks.
 *
 * lm          : fp32 landmarks, rows [B, Hkv, C] of d, strides ls (as written by
 *               dk_build_landmarks).
 * lm8         : out, uint8 [B, Hkv, C, d] contiguous (the codes above).
 * chunk_scale : out, fp32 [B, Hkv, C] contiguous.
 * scale_max   : out, fp32 [B, Hkv]; +inf when a landmark of (b, g) is inf or NaN
 *               (the scoring then re-scores every chunk of that (b, g) exactly).
 * Errors      : DK_ERR_INVALID_ARG unless sizes >= 1 and pointers non-NULL;
 *               DK_ERR_UNSUPPORTED unless d is 64 or 128 and the 16-byte alignment
 *               rule holds.
 */
dk_status dk_build_landmark_shadow(const float* lm, dk_strides ls, int B, int Hkv, int C, int d,
                                   uint8_t* lm8, float* chunk_scale, float* scale_max, void* stream);

/*
 * dk_score_topk - chunk scores of both queries and each query's k best chunks.
 *
 * DualDecoder "4.1": the retrieval index of a step comes from the current query
 * and the landmarks, and the speculative token with the same landmarks predicts
 * the next step's index; the sparse budget is a fixed number of chunks per KV
 * head (OasisKV summary, "Look-ahead Attention": blocks are ranked per KV head).
 *
 *   s[b, g, t, c] = reduce_{h in group g} scale * <q[b, t, h, :], lm[b, g, c, :]>
 *   topk_idx[b, g, t, :] = the k chunk ids with the largest s, ties to the lower
 *                          id, written in ascending id order.
 *
 * Token-level selection (Adaptive DHiSparse, Figure 2: an indexer emits the
 * top-k token positions of the step; Table 3: 2,048 per selecting layer) is
 * the same call with lm_dtype = DK_BF16: lm then holds one bf16 indexer key
 * per token, "chunk" means token (C = tokens), q holds the indexer queries
 * (Hq indexer heads over Hkv key heads) and the scores are exact fp32 dot
 * products with the keys.
 *
 * q          : fp32 [B, T, Hq, d] contiguous; query head h belongs to KV head h / (Hq/Hkv).
 * lm         : DK_F32 landmarks, or DK_BF16 per-token indexer keys; rows [B, Hkv, C]
 *              of d, strides ls (elements).
 * reduce     : DK_REDUCE_MEAN (mean over the group's heads) or DK_REDUCE_MAX.
 * shadow     : the landmarks' shadow (see above) or NULL.  With a shadow the
 *              result is the same; the call reads about a quarter of the bytes.
 * topk_idx   : out, int32 [B, Hkv, T, k].
 * topk_score : out, fp32 [B, Hkv, T, k] (the selected scores, same order) or NULL.
 * ws         : workspace of dk_score_topk_workspace_size(B, Hkv, T, C, k,
 *              shadow != NULL) bytes for DK_F32 landmarks (0 with a shadow: one
 *              block per (b, g) then scores and selects in LDS), of
 *              dk_index_topk_workspace_size(B, Hkv, T, C) bytes for DK_BF16 keys
 *              (may be NULL when that size is 0).  Contents on entry are ignored.
 * Errors     : DK_ERR_INVALID_ARG unless 1 <= T <= 2, Hq % Hkv == 0, 1 <= k <= C,
 *              pointers non-NULL and ws_bytes large enough; DK_ERR_UNSUPPORTED
 *              unless d is 64 or 128 and the 16-byte alignment rule holds, and,
 *              for DK_F32, C <= 65536 (C <= 6144 with a shadow) and the number
 *              of query vectors (T for mean, G*T for max) is at most 16; for
 *              DK_BF16, reduce is DK_REDUCE_MEAN, shadow is NULL, C % 4 == 0 and
 *              C <= 2^28.
 */
size_t dk_score_topk_workspace_size(int B, int Hkv, int T, int C, int k, int with_shadow);
/* Workspace bytes of dk_score_topk / dk_score_topk_union with DK_BF16 indexer
 * keys: the fp32 scores of every token (B*Hkv*T*C*4) plus per-block ranges. */
size_t dk_index_topk_workspace_size(int B, int Hkv, int T, int C);
dk_status dk_score_topk(const float* q, int B, int T, int Hq,
                        const void* lm, dk_dtype lm_dtype, dk_strides ls, int Hkv, int C, int d,
                        int k, float scale, dk_group_reduce reduce,
                        const dk_landmark_shadow* shadow,
                        int32_t* topk_idx, float* topk_score,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * dk_build_minmax - coordinate-wise minimum and maximum key of every chunk.
 *
 * OasisKV summary, "Look-ahead Attention": a draft query ranks every block of a
 * KV head from compressed key summaries, two vectors per block (coordinate-wise
 * min and max), 1/16 of the key bytes for 32-row chunks.
 *
 * K          : keys (k_dtype, DK_BF16 or DK_F32) with strides ks, rows [B, Hkv, L] of d.
 * kmin, kmax : out, k_dtype [B, Hkv, L/chunk, d] contiguous; the exact minima and
 *              maxima of the chunk's keys.
 * Errors     : DK_ERR_INVALID_ARG unless sizes >= 1, L % chunk == 0 and pointers
 *              non-NULL; DK_ERR_UNSUPPORTED unless d is 64 or 128 and the 16-byte
 *              alignment rule holds.
 */
dk_status dk_build_minmax(const void* K, dk_dtype k_dtype, dk_strides ks, int B, int Hkv, int L, int d,
                          int chunk, void* kmin, void* kmax, void* stream);

/*
 * dk_score_topk_minmax - each query's k best chunks by upper-bound scores from
 * min/max summaries, optionally with the union of the T sets.
 *
 * For query head h and chunk c the score bounds every key of the chunk:
 *   U = scale * sum_d max(q[b,t,h,d] * kmin[b,g,c,d], q[b,t,h,d] * kmax[b,g,c,d]),
 * combined over the group's heads by `reduce` (mean or max) like chunk scores;
 * topk_idx as in dk_score_topk (ties to the lower id, ascending).  With
 * union_ids non-NULL the union outputs of dk_union_select are written too.
 *
 * kmin, kmax : summaries (dtype) with strides ss, rows [B, Hkv, C] of d.
 * ws         : dk_index_topk_workspace_size(B, Hkv, T, C) bytes; contents ignored.
 * Errors     : those of dk_score_topk; DK_ERR_UNSUPPORTED unless d is 64 or 128,
 *              C % 4 == 0, C <= 2^28, G*T is a power of two <= 8 for max, and the
 *              16-byte alignment rule holds; union limits as dk_union_select.
 */
dk_status dk_score_topk_minmax(const float* q, int B, int T, int Hq, const void* kmin, const void* kmax,
                               dk_dtype dtype, dk_strides ss, int Hkv, int C, int d, int k, float scale,
                               dk_group_reduce reduce, int32_t* topk_idx, float* topk_score,
                               int32_t* union_ids, uint8_t* member, int32_t* union_count, int32_t* overlap,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * dk_score_coverage - for each query, the smallest set of chunks whose estimated
 * attention mass reaches a fraction gamma, optionally with the union of the T
 * sets.
 *
 * MOIRA (abstract): per request, layer, KV head and step a coverage rule keeps
 * the smallest set of pages whose estimated attention mass reaches gamma.  The
 * estimate here is the softmax over the row of the chunk scores of
 * dk_score_topk (landmark dot products combined over the group's heads by
 * `reduce`, times scale); the set is the shortest prefix of the chunks in
 * (score descending, id ascending) order whose mass reaches gamma * total, at
 * least 1 and at most k_max chunks (gamma = 1: the k_max best).
 *
 * q          : fp32 [B, T, Hq, d] contiguous.
 * lm         : landmarks (lm_dtype, DK_F32 or DK_BF16) with strides ls, rows
 *              [B, Hkv, C] of d.
 * sel_idx    : out, int32 [B, Hkv, T, k_max]: the kept chunk ids ascending, then -1.
 * sel_count  : out, int32 [B, Hkv, T]: chunks kept (1..k_max).
 * sel_score  : out or NULL, fp32 [B, Hkv, T, k_max]: the fp32 chunk scores of the
 *              kept ids, then -inf.
 * union_ids, member, union_count, overlap : NULL, or the outputs of
 *              dk_union_select with T*k_max slots per (b, g): the union of the T
 *              kept sets (ascending, then -1), member bits (bit t: in query t's
 *              set; 0 on padding), its size, and the size of the intersection.
 * ws         : dk_coverage_workspace_size(B, Hkv, T, C) bytes; contents ignored.
 * Rounding   : masses and their sums are fp32; a set whose mass lands within
 *              fp32 rounding of gamma * total may differ by one chunk from an
 *              exact evaluation.  Equal inputs give equal outputs.
 * Errors     : DK_ERR_INVALID_ARG unless sizes >= 1, T is 1 or 2, Hq % Hkv == 0,
 *              1 <= k_max <= C, 0 < gamma <= 1, scale finite, q, lm, sel_idx,
 *              sel_count non-NULL (and member, union_count with union_ids),
 *              ws_bytes large enough; DK_ERR_UNSUPPORTED unless d is 64 or 128,
 *              C <= 16384, G*T is a power of two <= 8 for max, and the 16-byte
 *              alignment rule holds.  Scores must be finite (not checked).
 */
size_t dk_coverage_workspace_size(int B, int Hkv, int T, int C);
dk_status dk_score_coverage(const float* q, int B, int T, int Hq, const void* lm, dk_dtype lm_dtype,
                            dk_strides ls, int Hkv, int C, int d, float scale, dk_group_reduce reduce,
                            float gamma, int k_max, int32_t* sel_idx, int32_t* sel_count, float* sel_score,
                            int32_t* union_ids, uint8_t* member, int32_t* union_count, int32_t* overlap,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * dk_score_topk_union - dk_score_topk and dk_union_select (without a cache
 * plan) of the same step in one call.
 *
 * DualDecoder "4.1": the index comes from the queries and the landmarks;
 * Adaptive DHiSparse, Figure 3 (2): the queries' selections are resolved
 * together.  With a landmark shadow one selection block per (b, g) selects for
 * both tokens and merges the union from its LDS, so the step needs no separate
 * union launch; otherwise the union runs as dk_union_select would.  Every output equals what
 * dk_score_topk followed by dk_union_select(plan = NULL) writes.
 *
 * Arguments: as dk_score_topk, plus the union outputs of dk_union_select
 * (union_ids int32 [B, Hkv, T*k], member uint8 [B, Hkv, T*k], union_count
 * int32 [B, Hkv], overlap int32 [B, Hkv] or NULL).  ws: the same workspace as
 * dk_score_topk; contents on entry are ignored.
 * Errors: those of dk_score_topk; DK_ERR_INVALID_ARG if a union output other
 * than overlap is NULL; DK_ERR_UNSUPPORTED beyond dk_union_select's limits.
 */
dk_status dk_score_topk_union(const float* q, int B, int T, int Hq,
                              const void* lm, dk_dtype lm_dtype, dk_strides ls, int Hkv, int C,
                              int d, int k, float scale, dk_group_reduce reduce,
                              const dk_landmark_shadow* shadow,
                              int32_t* topk_idx, float* topk_score,
                              int32_t* union_ids, uint8_t* member, int32_t* union_count,
                              int32_t* overlap, void* ws, size_t ws_bytes, void* stream);

/*
 * Hot-cache plan for the host-pool path (NULL in HBM-pool mode).
 *
 * Adaptive DHiSparse, Figure 2: a selected row that the hot cache does not hold
 * is copied from host DRAM into the hot cache before attention reads it.
 * OasisKV summary, "Asynchronous Prefetch Pipeline": the selection stage
 * compares the predicted set with the resident set and builds a transfer plan.
 *
 * Rule: union chunks already resident are hits and keep their slot; misses, in
 * ascending chunk order, take the free slots (slots whose chunk is not in the
 * new union, or empty) in ascending slot order; afterwards the cache holds
 * exactly the new union and every other slot is -1.
 */
typedef struct {
    int32_t* resident;       /* in/out [B, Hkv, slots]: chunk held by each slot, -1 = empty */
    int      slots;          /* slots per (b, g); must be >= T*k                            */
    int32_t* slot_of_union;  /* out [B, Hkv, T*k]: slot of each union entry, -1 padded      */
    int32_t* miss_chunk;     /* out [B, Hkv, T*k]: chunk id of each miss, -1 padded         */
    int32_t* miss_slot;      /* out [B, Hkv, T*k]: destination slot of each miss            */
    int32_t* miss_count;     /* out [B, Hkv]                                                */
    int32_t* hit_count;      /* out [B, Hkv]                                                */
} dk_cache_plan;

/*
 * dk_capped_plan - one step of a bounded per-(request, KV head) working set
 * under delta selection with capped eviction.
 *
 * OasisKV, "Delta Selection and Capped Eviction": predicted blocks already
 * resident cost no traffic; resident blocks outside the predicted set are ranked
 * by the step of their last selection; each admitted non-resident block is
 * paired with one eviction target, least recently selected first; at most `cap`
 * pairs are admitted per step and KV head.
 *
 * Rule: hits keep their slot and their stamp becomes `step`.  Targets are the
 * slots whose chunk is not predicted: empty slots first, then the oldest stamp,
 * then the lower slot.  The admitted misses are the best min(cap, misses,
 * targets) by (score descending, id ascending; all tied when sel_score is NULL),
 * paired in ascending chunk order with the targets in ascending slot order; the
 * target takes the chunk and the stamp `step`.  Other misses get no slot.
 *
 * sel_ids      : int32, row (b, g) at sel_ids + (b*Hkv + g) * sel_stride: N entries,
 *                the first sel_count of them strictly ascending chunk ids >= 0
 *                (e.g. one query's row of dk_score_topk output: offset t*k, stride T*k).
 * sel_score    : fp32 priorities in the same layout, or NULL.
 * sel_count    : int32 at sel_count + (b*Hkv + g) * count_stride (clamped to [0, N]), or NULL (N).
 * resident     : in/out int32 [B, Hkv, slots]: chunk per slot, -1 empty; distinct chunks.
 * stamp        : in/out int32 [B, Hkv, slots]: step of the slot's last selection.
 * sel_slot     : out int32 [B, Hkv, N]: slot of each entry after the step, -1 when
 *                not admitted or past the count.
 * admit_chunk, admit_slot : out int32 [B, Hkv, cap]: the transfers (chunk -> slot)
 *                in ascending chunk order, -1 padded (may be NULL when cap == 0);
 *                dk_gather_kv(src_chunk = admit_chunk, dst_slot = admit_slot,
 *                count = admit_count) performs them.
 * admit_count  : out int32 [B, Hkv].   hit_count : out int32 [B, Hkv] or NULL.
 * Errors       : DK_ERR_INVALID_ARG unless B, Hkv, N, slots >= 1, sel_stride >= N,
 *                count_stride >= 1 with sel_count, 0 <= cap <= 2^20 and the required
 *                pointers are non-NULL; DK_ERR_UNSUPPORTED if N or slots > 4096.
 *                Row contents are not checked: ids that are not ascending or
 *                resident chunks that repeat give an unspecified (in-bounds) plan.
 */
dk_status dk_capped_plan(const int32_t* sel_ids, const float* sel_score, const int32_t* sel_count, int B, int Hkv,
                         int N, int sel_stride, int count_stride, int32_t* resident, int32_t* stamp, int slots,
                         int cap, int32_t step, int32_t* sel_slot, int32_t* admit_chunk, int32_t* admit_slot,
                         int32_t* admit_count, int32_t* hit_count, void* stream);

/*
 * dk_union_select - the distinct chunks of the T selections of every (b, g).
 *
 * Adaptive DHiSparse, Figure 3 (2): the top-k selections of several queries of
 * one request and KV source are resolved together, so each distinct chunk is
 * moved once, and each query still attends over its own selection.  DualDecoder
 * "6.3 Accuracy Analysis": the overlap of the predicted (speculative) and true
 * (real) sets is the prediction accuracy.
 *
 * topk_idx    : int32 [B, Hkv, T, k], each row strictly ascending in [0, C)
 *               (as written by dk_score_topk).
 * union_ids   : out int32 [B, Hkv, T*k]: ascending distinct ids, -1 padded.
 * member      : out uint8 [B, Hkv, T*k]: bit t set iff the chunk is in query t's set, 0 padded.
 * union_count : out int32 [B, Hkv].
 * overlap     : out int32 [B, Hkv]: |S_0 & S_1| (k when T == 1), or NULL.
 * plan        : hot-cache plan (see above) or NULL.
 * Errors      : DK_ERR_INVALID_ARG unless 1 <= T <= 2, 1 <= k <= C <= 2^30, outputs
 *               non-NULL and, with a plan, all its arrays non-NULL and slots >= T*k;
 *               DK_ERR_UNSUPPORTED if T*k > 8192 or slots > 8192.
 */
dk_status dk_union_select(const int32_t* topk_idx, int B, int Hkv, int T, int k, int C,
                          int32_t* union_ids, uint8_t* member, int32_t* union_count,
                          int32_t* overlap, const dk_cache_plan* plan, void* stream);

/*
 * dk_gather_kv - copy selected chunks of a KV pool into destination slots.
 *
 * DualDecoder "5.4 Layer-Scoped KV Memory Management", GPU-side sparse KV
 * assembly: selected blocks are moved into GPU memory and placed into the
 * attention layout by a GPU kernel; Adaptive DHiSparse, Figure 2 step 3: missed
 * rows are copied from host DRAM into the hot cache.
 *
 * For every (b, g) and j < count[b, g]: rows [c*chunk, (c+1)*chunk) of K_src and
 * V_src, c = src_chunk[b, g, j], go to rows [s*chunk, (s+1)*chunk) of K_dst and
 * V_dst, s = dst_slot[b, g, j] (s = j when dst_slot is NULL).
 *
 * src_chunk, dst_slot : int32 [B, Hkv, N].   count : int32 [B, Hkv] (NULL: N each).
 * src_blocks          : chunks in the source pool; ids outside [0, src_blocks) are skipped.
 * dst_blocks          : slots in the destination; ids outside [0, dst_blocks) are skipped.
 * src_kind = DK_SRC_DEVICE      : K_src/V_src and the lists are device memory;
 *                                 one kernel on `stream`.
 * src_kind = DK_SRC_HOST_COPY   : K_src/V_src are pinned host memory (hipHostMalloc)
 *                                 and src_chunk, dst_slot, count are host-readable and
 *                                 final when the call is made; the call issues one
 *                                 hipMemcpyAsync (2-D when rows are strided) per run of
 *                                 consecutive chunks on `stream` and returns after
 *                                 issuing.  Every copy costs a few microseconds of host
 *                                 time, so scattered misses are API-bound.  A HIP
 *                                 failure partway returns DK_ERR_HIP with the earlier
 *                                 copies still enqueued (destination slots undefined).
 * src_kind = DK_SRC_HOST_MAPPED : K_src/V_src are pinned host memory, the lists are
 *                                 device memory; one kernel on `stream` reads the pool
 *                                 through its device mapping over PCIe.  Fully
 *                                 asynchronous: no host synchronisation on the lists.
 * Errors              : DK_ERR_INVALID_ARG unless sizes >= 1, N >= 0, pointers
 *                       non-NULL (dst_slot and count may be NULL), src_kind is one
 *                       of the above and, for the host kinds, K_src and V_src are
 *                       pinned host memory known to HIP; DK_ERR_UNSUPPORTED unless
 *                       the 16-byte alignment rule holds.
 */
dk_status dk_gather_kv(const void* K_src, const void* V_src, dk_dtype dt, dk_strides src_s,
                       int B, int Hkv, int chunk, int d,
                       const int32_t* src_chunk, const int32_t* dst_slot, const int32_t* count,
                       int N, int src_blocks,
                       void* K_dst, void* V_dst, dk_strides dst_s, int dst_blocks,
                       int src_kind, void* stream);

/*
 * dk_sparse_decode_attn - attention of every query head over its own chunks,
 * both queries in one pass over the union.
 *
 * DualDecoder "4.2" and "5.3": the result must equal attention over the true
 * retrieval index; "5.2" and "6.4": the real and speculative tokens are
 * processed by one attention launch instead of two.  Adaptive DHiSparse Figure 3
 * (2): each query attends over its own selection.
 *
 * For query head h (KV head g = h / G) and query t, with R the rows of the chunks
 * i < count[b, g] whose member bit t is set:
 *   z = scale * K[b, g, R] q[b, t, h],  out[b, t, h] = softmax(z) V[b, g, R],
 *   lse[b, t, h] = log sum exp z   (out = 0 and lse = -inf when R is empty).
 * Each union chunk is read once for all G*T query rows.
 *
 * q          : fp32 [B, T, Hq, dk] contiguous.  With bf16 K, q is read as bf16
 *              (exact for bf16-valued queries); fp32 K uses q as is.
 * K, V       : pools (kv_dtype) with strides ks, vs; block_ids index chunks of
 *              `chunk` rows in them (pool chunk ids, or hot-cache slot ids).
 * block_ids  : int32 [B, Hkv, N]; ids outside [0, pool_blocks) are skipped.
 * member     : uint8 [B, Hkv, N] query bits, or NULL when T == 1 (all rows belong).
 * count      : int32 [B, Hkv] valid entries (<= N), or NULL for N.
 * out, lse   : out fp32 [B, T, Hq, dv] and [B, T, Hq] (lse may be NULL).
 * ws         : workspace of dk_attn_workspace_size(...) bytes (NULL when 0).
 *
 * Latent rows (dk = 576, dv = 512, token-level selection; Adaptive DHiSparse
 * Figure 2: attention reads the rows the indexer selected): K holds one bf16
 * latent row per token (512 content + 64 position columns), V must be the same
 * pointer with the same strides (the value is the first 512 columns of each
 * row), chunk == 1, block_ids are token ids (pool_blocks = tokens), and every
 * query head of a KV head reads the same rows.  The product runs on the matrix
 * cores; Hq/Hkv must be a multiple of 64/T.  The workspace is
 * dk_attn_workspace_size(B, Hkv, T, Hq, 512, N, 1).
 *
 * Errors     : DK_ERR_INVALID_ARG unless sizes >= 1, Hq % Hkv == 0, 1 <= T <= 2,
 *              pointers non-NULL as stated and ws_bytes large enough;
 *              DK_ERR_UNSUPPORTED unless dk == dv in {64, 128} with G*T <= 16, or
 *              the latent form above holds, and the 16-byte alignment rule holds.
 */
size_t dk_attn_workspace_size(int B, int Hkv, int T, int Hq, int dv, int N, int chunk);
dk_status dk_sparse_decode_attn(const float* q, int B, int T, int Hq, int Hkv,
                                const void* K, const void* V, dk_dtype kv_dtype,
                                dk_strides ks, dk_strides vs, int dk, int dv, int chunk,
                                const int32_t* block_ids, const uint8_t* member,
                                const int32_t* count, int N, int pool_blocks, float scale,
                                float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * dk_sparse_decode_attn_noalloc - dk_sparse_decode_attn without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that forbid allocation, harnesses without
 * hipMalloc).
 *
 * The result is the one dk_sparse_decode_attn writes: the same kernels run on
 * the same plan.  The split partials go to a fixed 64 MiB device array inside
 * the library instead of a caller workspace; each device the library runs on
 * holds its own copy from the first call on it until the process ends.  The
 * call allocates nothing (no hipMalloc, no hipFree); its first call on a device
 * looks the array's device address up once.  Nothing in the array needs to
 * start at zero: every partial is written before it is read.
 *
 * Concurrency: every call on one device shares that device's array.  Calls
 * whose execution overlaps on one device (different streams, or host threads
 * with no ordering between their streams) race on it and give undefined
 * results; calls ordered on one stream are safe.
 *
 * Arguments: as dk_sparse_decode_attn, without ws and ws_bytes.
 * Errors: those of dk_sparse_decode_attn; DK_ERR_UNSUPPORTED when the shape
 * needs more scratch than the array holds (dk_attn_workspace_size(...) of the
 * same arguments above 64 MiB); DK_ERR_HIP when the device address cannot be
 * looked up.
 */
dk_status dk_sparse_decode_attn_noalloc(const float* q, int B, int T, int Hq, int Hkv,
                                        const void* K, const void* V, dk_dtype kv_dtype,
                                        dk_strides ks, dk_strides vs, int dk, int dv, int chunk,
                                        const int32_t* block_ids, const uint8_t* member,
                                        const int32_t* count, int N, int pool_blocks, float scale,
                                        float* out, float* lse, void* stream);

/*
 * dk_sparse_decode_attn_tail - dk_sparse_decode_attn plus the rows every query
 * attends besides its chunks.
 *
 * DualDecoder "5.2 Dual-Token Decoding Pipeline": the step's real and
 * speculative tokens lie one after the other along the sequence, and a mask
 * keeps the real token from the speculative token's data while the speculative
 * token sees every earlier token, the real one included.  Adaptive DHiSparse
 * Figure 2: each request's tail of recent rows is resolved for every lookup,
 * besides the selected rows.
 *
 * For query head h (KV head g) and query t the key rows are its own chunks' rows
 * (as in dk_sparse_decode_attn), the first tail_len[b] rows of the tail, and the
 * new rows of the step's tokens t' <= t; the softmax runs over all of them.
 *
 * extra->K_tail, V_tail : [B, Hkv, tail_max, dk] pools (kv_dtype) with element
 *                         strides tail_k_s, tail_v_s, or both NULL (no tail).
 * extra->tail_len       : int32 [B], clamped to [0, tail_max], or NULL (tail_max).
 * extra->K_new, V_new   : [B, T, Hkv, dk] contiguous (kv_dtype): the step's own
 *                         tokens' keys and values, or both NULL.
 * ws                    : dk_attn_tail_workspace_size(...) bytes; contents on
 *                         entry are ignored.  The size allows the tail a partial
 *                         result of its own; on the bf16 d = 128, G = 4, T = 2 path
 *                         the last chunk range attends the tail rows itself and
 *                         the workspace is used as for dk_sparse_decode_attn.
 * Other arguments and errors: as dk_sparse_decode_attn; DK_ERR_INVALID_ARG also
 * for a NULL extra, a half-given K/V pair or negative tail sizes.
 */
typedef struct {
    const void* K_tail;
    const void* V_tail;
    dk_strides tail_k_s, tail_v_s;
    const int32_t* tail_len;
    int tail_max;
    const void* K_new;
    const void* V_new;
} dk_attn_extra;
size_t dk_attn_tail_workspace_size(int B, int Hkv, int T, int Hq, int dv, int N, int chunk);
dk_status dk_sparse_decode_attn_tail(const float* q, int B, int T, int Hq, int Hkv,
                                     const void* K, const void* V, dk_dtype kv_dtype,
                                     dk_strides ks, dk_strides vs, int dk, int dv, int chunk,
                                     const int32_t* block_ids, const uint8_t* member,
                                     const int32_t* count, int N, int pool_blocks,
                                     const dk_attn_extra* extra, float scale,
                                     float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * dk_decode_step - one layer's decode step in one call: dk_score_topk_union
 * followed by dk_sparse_decode_attn over the union it wrote.
 *
 * DualDecoder "4.1" (the index from the query and the landmarks), "4.2" and
 * "5.3" (attention over the retrieved chunks equals attention over the true
 * index), "5.2" and "6.4" (both tokens in one pass); Adaptive DHiSparse
 * Figure 3 (2) (each query attends over its own selection, each union chunk is
 * read once).
 *
 * The arguments are those of the two calls: q, B, T, Hq, Hkv, lm (DK_F32),
 * ls, C, d, k, scale, reduce and shadow as for dk_score_topk_union; K, V,
 * kv_dtype, ks, vs and chunk as for dk_sparse_decode_attn with dk = dv = d, the
 * union as its block_ids / member / count, N = T*k and pool_blocks = C.  The
 * outputs are both calls' outputs (topk_score and overlap may be NULL, lse may
 * be NULL) and equal theirs bit for bit.  extra: NULL, or the tail rows and the
 * step's own rows of dk_sparse_decode_attn_tail (which then replaces
 * dk_sparse_decode_attn, with its causal rule).  ws:
 * dk_decode_step_workspace_size bytes (with_tail: extra is given; NULL when 0).
 * Errors are those of the two calls, checked before anything is enqueued.
 *
 * With a shadow, the mean reduction, T = 2, G = 4, d = 128, bf16 K/V, chunk a
 * multiple of 32, k <= 128 and B*Hkv > 256, one kernel does both: each block
 * scores, selects and merges one (b, g), then attends over that union, so the
 * blocks that finish their selection early stream their attention while others
 * still select.  Other shapes, and calls with extra, run the two calls' kernels
 * in turn.
 */
size_t dk_decode_step_workspace_size(int B, int Hkv, int T, int Hq, int C, int d, int k, int chunk,
                                     int with_shadow, int with_tail);
dk_status dk_decode_step(const float* q, int B, int T, int Hq, int Hkv, const void* lm, dk_dtype lm_dtype,
                         dk_strides ls, int C, int d, int k, float scale, dk_group_reduce reduce,
                         const dk_landmark_shadow* shadow, const void* K, const void* V, dk_dtype kv_dtype,
                         dk_strides ks, dk_strides vs, int chunk, const dk_attn_extra* extra,
                         int32_t* topk_idx, float* topk_score,
                         int32_t* union_ids, uint8_t* member, int32_t* union_count, int32_t* overlap, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DUALKV_H */
