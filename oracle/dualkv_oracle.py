"""Plain CPU reference ("oracle") for one dual-query sparse KV retrieval decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's compute
path never calls it, and it shares no code with the HIP kernels: it is written
from the pages' description of the method, in numpy float64, as slowly and
plainly as possible, so that a reader can check each function against the
passage it cites.

What one step computes, per request b, KV head g and query t (t = 0 the real
token, t = 1 the speculative look-ahead token):

1. chunk landmarks: the mean key of each fixed-size chunk of adjacent KV
   entries (DualDecoder, "2.2 Dynamic Sparse KV Cache": adjacent entries are
   segmented into chunks summarised by GPU-resident landmarks; "4.1 KV Retrieval
   Predictability": landmarks are made before decoding and stay fixed);
2. chunk scores from the current query and the landmarks (DualDecoder, "4.1":
   the retrieval index is determined by the current query and the landmarks;
   the speculative token with the landmarks predicts the next step's index);
3. the k best chunks of each query (fixed sparse budget);
4. the union of the two queries' chunk sets, each distinct chunk once, with a
   membership bit per query (Adaptive DHiSparse, Figure 3 (2): the selections of
   several queries are resolved together so each distinct missing row moves
   once, while each query still attends over its own selection);
5. attention of every query head over the KV rows of its own query's chunks only
   (DualDecoder, "4.2" and "5.3": misses are corrected before attention so the
   result equals attention over the true index).

The overlap of the real and speculative chunk sets is the prediction accuracy
(DualDecoder, "6.3 Accuracy Analysis": overlap ratio of predicted and
ground-truth sparse indices).

Readings where the pages are silent:
* a landmark is the arithmetic mean of the chunk's keys;
* the G query heads of one KV head are combined by the mean of their scaled
  dot products ("max" is offered as an alternative);
* the score scale is 1/sqrt(d) unless given; it does not change the ranking;
* ties in score go to the lower chunk id; a selected set is reported as
  ascending chunk ids;
* every query attends over the pool rows of its own chunk set only; there is no
  tail of fresh rows and L must be a multiple of the chunk size.

Token-level selection over a latent KV head (Adaptive DHiSparse, Figure 2: an
indexer reads its index state and emits the top-k token positions, and
attention reads the selected rows; Table 3: 2,048 selections per selecting
layer) is the same step with chunk = 1: the indexer keys are their own
landmarks, and one latent head serves every query head.  Readings for it:
* a token's index score is the mean over the indexer heads of the scaled dot
  products of the indexer query with the token's indexer key (the same rule as
  the chunk score);
* attention uses the whole latent row (content part and position part) as the
  key, the first dv columns of the same row as the value, and the scale the
  caller passes (1/sqrt of the key width in the workloads).

Selection variants replace the landmark score or the fixed budget k:
* min/max chunk summaries (OasisKV, "Look-ahead Attention"): a chunk's score
  is the largest scaled dot product any key in the box between its coordinate-
  wise minimum and maximum can reach, combined over heads like chunk scores;
* coverage budgets (MOIRA, abstract): a chunk's estimated attention mass is the
  softmax of its chunk score over the row; the kept set is the shortest prefix
  of the (score descending, id ascending) order whose mass reaches gamma, at
  least one chunk and at most k_max (the caller's buffer); the union of the two
  queries' sets is taken over their own counts;
* capped eviction (OasisKV, "Delta Selection and Capped Eviction"): see
  capped_plan for the readings of the order of admissions, eviction targets
  and their pairing.

Parity of each function is pinned by the not-gpu tests (closed forms, brute
force on tiny inputs, a library attention routine, hand-worked fixtures under
tests/golden/).  The absolute prediction-accuracy level on synthetic data has
no value on the pages to compare with: parity unpinned for that level (the GPU
must reproduce the oracle's value; the oracle's own overlap count is pinned).
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the bf16 word is the upper half of an fp32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# step 1: chunk landmarks
# ----------------------------------------------------------------------------

def chunk_landmarks(K: np.ndarray, chunk: int) -> np.ndarray:
    """Mean key of every chunk.

    K: [B, Hkv, L, d] keys; chunk: tokens per chunk (L % chunk == 0).
    Returns lm: [B, Hkv, C, d] with lm[b, g, c] = mean of K[b, g, c*chunk:(c+1)*chunk].
    """
    K = np.asarray(K, dtype=np.float64)
    B, H, L, d = K.shape
    if chunk <= 0 or L % chunk != 0:
        raise ValueError("L must be a positive multiple of chunk")
    C = L // chunk
    lm = np.zeros((B, H, C, d), dtype=np.float64)
    for c in range(C):
        rows = K[:, :, c * chunk:(c + 1) * chunk, :]
        lm[:, :, c, :] = rows.sum(axis=2) / chunk
    return lm


# ----------------------------------------------------------------------------
# step 2: chunk scores
# ----------------------------------------------------------------------------

def chunk_scores(q: np.ndarray, lm: np.ndarray, scale: float, reduce: str = "mean") -> np.ndarray:
    """Score every chunk landmark against each query.

    q: [B, T, Hq, d]; lm: [B, Hkv, C, d]; query head h belongs to KV head h // G.
    s[b, g, t, c] = reduce over the G heads h of KV head g of scale * <q[b, t, h], lm[b, g, c]>,
    reduce = "mean" (default) or "max".  Returns [B, Hkv, T, C].
    """
    q = np.asarray(q, dtype=np.float64)
    lm = np.asarray(lm, dtype=np.float64)
    B, T, Hq, d = q.shape
    Hkv, C = lm.shape[1], lm.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    s = np.zeros((B, Hkv, T, C), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            for t in range(T):
                heads = q[b, t, g * G:(g + 1) * G, :]            # [G, d]
                per_head = scale * (heads @ lm[b, g].T)          # [G, C]
                if reduce == "mean":
                    s[b, g, t] = per_head.mean(axis=0)
                elif reduce == "max":
                    s[b, g, t] = per_head.max(axis=0)
                else:
                    raise ValueError("reduce must be 'mean' or 'max'")
    return s


# ----------------------------------------------------------------------------
# step 3: top-k chunks per query
# ----------------------------------------------------------------------------

def topk_chunks(s: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring chunk ids of every score row, as an ascending id list.

    Full sort of each row by (score descending, id ascending), keep the first k.
    s: [..., C]; returns int64 [..., k].
    """
    s = np.asarray(s, dtype=np.float64)
    C = s.shape[-1]
    if not 1 <= k <= C:
        raise ValueError("need 1 <= k <= C")
    flat = s.reshape(-1, C)
    out = np.zeros((flat.shape[0], k), dtype=np.int64)
    ids = np.arange(C)
    for r in range(flat.shape[0]):
        order = np.lexsort((ids, -flat[r]))   # primary: -score, secondary: id
        out[r] = np.sort(order[:k])
    return out.reshape(s.shape[:-1] + (k,))


# ----------------------------------------------------------------------------
# step 4: union of the two queries' sets
# ----------------------------------------------------------------------------

def union_select(idx: np.ndarray):
    """Union of the T chunk sets of every (request, KV head), duplicates removed.

    idx: [B, Hkv, T, k] chunk ids (T = 1 or 2).
    Returns (union_ids [B, Hkv, T*k] ascending, -1 padded;
             member [B, Hkv, T*k] uint8, bit t set iff the chunk is in query t's set;
             count [B, Hkv] distinct chunks;
             overlap [B, Hkv] = |S_0 & S_1| (= k when T = 1)).
    """
    idx = np.asarray(idx)
    B, H, T, k = idx.shape
    union_ids = np.full((B, H, T * k), -1, dtype=np.int64)
    member = np.zeros((B, H, T * k), dtype=np.uint8)
    count = np.zeros((B, H), dtype=np.int64)
    overlap = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for g in range(H):
            sets = [set(int(c) for c in idx[b, g, t]) for t in range(T)]
            u = sorted(set().union(*sets))
            count[b, g] = len(u)
            for i, c in enumerate(u):
                union_ids[b, g, i] = c
                bits = 0
                for t in range(T):
                    if c in sets[t]:
                        bits |= 1 << t
                member[b, g, i] = bits
            overlap[b, g] = len(sets[0] & sets[1]) if T == 2 else len(sets[0])
    return union_ids, member, count, overlap


def prediction_accuracy(overlap: np.ndarray, k: int) -> float:
    """Mean over (request, KV head[, layer]) of |S_real & S_spec| / k."""
    return float(np.mean(np.asarray(overlap, dtype=np.float64) / k))


# ----------------------------------------------------------------------------
# step 5: attention over each query's own selected rows
# ----------------------------------------------------------------------------

def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sel: np.ndarray,
                     chunk: int, scale: float):
    """Softmax attention of every query head over the rows of its own chunk set.

    q: [B, T, Hq, dk]; K: [B, Hkv, L, dk]; V: [B, Hkv, L, dv];
    sel: [B, Hkv, T, k] chunk ids of each query's own set.
    For query head h (KV head g = h // G) and query t the rows are
    R = union over c in sel[b, g, t] of [c*chunk, (c+1)*chunk), and
        z = scale * K[b, g, R] @ q[b, t, h],  m = max z,  p = exp(z - m),
        out = (p @ V[b, g, R]) / sum p,       lse = m + log(sum p).
    Returns out [B, T, Hq, dv] and lse [B, T, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, T, Hq, dk = q.shape
    Hkv = K.shape[1]
    dv = V.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, dv), dtype=np.float64)
    lse = np.zeros((B, T, Hq), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            for h in range(Hq):
                g = h // G
                rows = np.concatenate([np.arange(int(c) * chunk, (int(c) + 1) * chunk)
                                       for c in sel[b, g, t]])
                z = scale * (K[b, g, rows] @ q[b, t, h])
                m = z.max()
                p = np.exp(z - m)
                out[b, t, h] = (p @ V[b, g, rows]) / p.sum()
                lse[b, t, h] = m + math.log(p.sum())
    return out, lse


def sparse_attention_tail(q: np.ndarray, K: np.ndarray, V: np.ndarray, sel: np.ndarray, chunk: int,
                          scale: float, K_tail=None, V_tail=None, tail_len=None, K_new=None, V_new=None):
    """sparse_attention plus the rows every query attends besides its chunks.

    DualDecoder "5.2 Dual-Token Decoding Pipeline": the step's real token T_i and
    speculative token T'_{i+1} are placed one after the other along the sequence,
    and a mask keeps the real token from using the speculative token's data,
    while the speculative token sees every earlier token, the real one included.
    Adaptive DHiSparse, Figure 2: a per-request tail of recent rows is resolved
    for every lookup, besides the selected rows.

    K_tail, V_tail: [B, Hkv, Lt, d] and tail_len [B]: the first tail_len[b] rows
    are attended by every query of request b (None: no tail).
    K_new, V_new: [B, T, Hkv, d]: the step's own tokens; query t attends the rows
    of tokens t' <= t (None: no fresh rows).
    For query head h (KV head g = h // G) and query t the key rows are the rows of
    its chunks, then the tail rows, then the allowed fresh rows; the softmax is
    the same dense one as in sparse_attention over all of them.
    Returns out [B, T, Hq, dv] and lse [B, T, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, T, Hq, dk = q.shape
    Hkv = K.shape[1]
    dv = V.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, dv), dtype=np.float64)
    lse = np.zeros((B, T, Hq), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            for h in range(Hq):
                g = h // G
                keys, vals = [], []
                for c in sel[b, g, t]:
                    keys.append(K[b, g, int(c) * chunk:(int(c) + 1) * chunk])
                    vals.append(V[b, g, int(c) * chunk:(int(c) + 1) * chunk])
                if K_tail is not None:
                    n = int(tail_len[b])
                    keys.append(np.asarray(K_tail[b, g, :n], dtype=np.float64))
                    vals.append(np.asarray(V_tail[b, g, :n], dtype=np.float64))
                if K_new is not None:
                    for tp in range(t + 1):           # tokens up to and including t
                        keys.append(np.asarray(K_new[b, tp, g], dtype=np.float64)[None, :])
                        vals.append(np.asarray(V_new[b, tp, g], dtype=np.float64)[None, :])
                Kr = np.concatenate(keys, axis=0)
                Vr = np.concatenate(vals, axis=0)
                z = scale * (Kr @ q[b, t, h])
                m = z.max()
                p = np.exp(z - m)
                out[b, t, h] = (p @ Vr) / p.sum()
                lse[b, t, h] = m + math.log(p.sum())
    return out, lse


# ----------------------------------------------------------------------------
# host-pool hot cache: which union chunks are already resident
# ----------------------------------------------------------------------------

def cache_plan(resident: np.ndarray, union_ids: np.ndarray, count: np.ndarray):
    """Plan one step of the HBM hot cache that holds the previous step's union.

    The hot cache of each (request, KV head) has S slots; resident[b, g, s] is the
    chunk held by slot s, or -1.  The chunks of the new union that are already
    resident are hits and keep their slot; the others are misses that must be
    copied from host memory before attention reads them (Adaptive DHiSparse,
    Figure 2, step 3; OasisKV summary, "KV selection" compares the predicted set
    with the resident set and builds a transfer plan).  Misses, in ascending
    chunk order, take the free slots (slots whose chunk is not in the new union)
    in ascending slot order.  Afterwards the cache holds exactly the new union;
    every other slot is empty.

    resident: [B, Hkv, S]; union_ids: [B, Hkv, N] ascending, -1 padded; count: [B, Hkv].
    Returns a dict with new_resident [B, Hkv, S], slot_of_union [B, Hkv, N] (-1 pad),
    miss_chunk, miss_slot [B, Hkv, N] (-1 pad), miss_count, hit_count [B, Hkv].
    """
    resident = np.asarray(resident)
    B, H, S = resident.shape
    N = union_ids.shape[2]
    new_res = np.full((B, H, S), -1, dtype=np.int64)
    slot_of_union = np.full((B, H, N), -1, dtype=np.int64)
    miss_chunk = np.full((B, H, N), -1, dtype=np.int64)
    miss_slot = np.full((B, H, N), -1, dtype=np.int64)
    miss_count = np.zeros((B, H), dtype=np.int64)
    hit_count = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for g in range(H):
            u = [int(c) for c in union_ids[b, g, :int(count[b, g])]]
            if len(u) > S:
                raise ValueError("hot cache has fewer slots than the union")
            where = {int(c): s for s, c in enumerate(resident[b, g]) if c >= 0}
            in_u = set(u)
            free = [s for s in range(S) if int(resident[b, g, s]) not in in_u]
            nm = 0
            for i, c in enumerate(u):
                if c in where:
                    slot = where[c]
                    hit_count[b, g] += 1
                else:
                    slot = free[nm]
                    miss_chunk[b, g, nm] = c
                    miss_slot[b, g, nm] = slot
                    nm += 1
                slot_of_union[b, g, i] = slot
                new_res[b, g, slot] = c
            miss_count[b, g] = nm
    return dict(new_resident=new_res, slot_of_union=slot_of_union, miss_chunk=miss_chunk,
                miss_slot=miss_slot, miss_count=miss_count, hit_count=hit_count)


# ----------------------------------------------------------------------------
# one decode step
# ----------------------------------------------------------------------------

def decode_step(q, K, V, chunk: int, k: int, scale: float | None = None,
                reduce: str = "mean", lm: np.ndarray | None = None):
    """Landmarks (unless given) -> scores -> top-k -> union -> attention for one layer."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if lm is None:
        lm = chunk_landmarks(K, chunk)
    s = chunk_scores(q, lm, scale, reduce)
    sel = topk_chunks(s, k)
    union_ids, member, count, overlap = union_select(sel)
    out, lse = sparse_attention(q, K, V, sel, chunk, scale)
    return dict(lm=lm, scores=s, topk=sel, union_ids=union_ids, member=member, count=count,
                overlap=overlap, accuracy=prediction_accuracy(overlap, k), out=out, lse=lse)


# ----------------------------------------------------------------------------
# token-level selection over one latent KV head
# ----------------------------------------------------------------------------

def indexer_topk(qi: np.ndarray, Kidx: np.ndarray, k: int, scale: float) -> np.ndarray:
    """Top-k token positions of every query from the indexer.

    Adaptive DHiSparse, Figure 2: the indexer turns the index state into the top-k
    positions the step reads.  qi: [B, T, Hi, di] indexer queries; Kidx: [B, 1, L, di]
    indexer keys, one per token.  A token's score is the mean over the Hi indexer
    heads of scale * <qi[b, t, h], Kidx[b, 0, n]> (chunk_scores with the keys as
    their own landmarks); the k best tokens, ties to the lower position, are
    returned ascending.  Returns [B, 1, T, k].
    """
    return topk_chunks(chunk_scores(qi, Kidx, scale, "mean"), k)


def mla_attention(q: np.ndarray, latent: np.ndarray, sel: np.ndarray, dv: int, scale: float):
    """Attention of every query head over its own selected latent rows.

    q: [B, T, Hq, dk] with dk the latent width (content + position parts);
    latent: [B, 1, L, dk], one latent row per token shared by every query head;
    sel: [B, 1, T, k] token positions of each query.  The key is the whole latent
    row and the value its first dv columns; otherwise this is sparse_attention
    with chunk = 1.  Returns out [B, T, Hq, dv] and lse [B, T, Hq].
    """
    latent = np.asarray(latent, dtype=np.float64)
    return sparse_attention(q, latent, latent[..., :dv], sel, 1, scale)


def mla_decode_step(qi, Kidx, q, latent, k: int, dv: int, index_scale: float, scale: float):
    """Indexer top-k -> union -> latent attention for one layer of token-level selection."""
    sel = indexer_topk(qi, Kidx, k, index_scale)
    union_ids, member, count, overlap = union_select(sel)
    out, lse = mla_attention(q, latent, sel, dv, scale)
    return dict(topk=sel, union_ids=union_ids, member=member, count=count, overlap=overlap,
                accuracy=prediction_accuracy(overlap, k), out=out, lse=lse)


# ----------------------------------------------------------------------------
# selection variants: min/max chunk summaries (upper-bound scores)
# ----------------------------------------------------------------------------

def chunk_minmax(K: np.ndarray, chunk: int):
    """Coordinate-wise minimum and maximum key of every chunk.

    OasisKV summary, "Look-ahead Attention": the draft query scans compressed
    key summaries, two vectors per block (coordinate-wise min and max).
    K: [B, Hkv, L, d] with L a multiple of chunk.  Returns (kmin, kmax), each
    [B, Hkv, C, d].
    """
    K = np.asarray(K, dtype=np.float64)
    B, H, L, d = K.shape
    if L % chunk != 0:
        raise ValueError("L must be a multiple of chunk")
    Kc = K.reshape(B, H, L // chunk, chunk, d)
    return Kc.min(axis=3), Kc.max(axis=3)


def minmax_scores(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray, scale: float,
                  reduce: str = "mean") -> np.ndarray:
    """Upper-bound chunk scores from min/max summaries.

    For one query head h and chunk c the largest dot product any key inside the
    box [kmin, kmax] can reach is sum_d max(q_d * kmin_d, q_d * kmax_d); the
    score is scale times that bound, combined over the G heads of KV head g by
    the chunk-score rule (mean by default, or max).  Returns [B, Hkv, T, C].
    """
    q = np.asarray(q, dtype=np.float64)
    kmin = np.asarray(kmin, dtype=np.float64)
    kmax = np.asarray(kmax, dtype=np.float64)
    B, T, Hq, d = q.shape
    Hkv, C = kmin.shape[1], kmin.shape[2]
    G = Hq // Hkv
    s = np.zeros((B, Hkv, T, C), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            for t in range(T):
                per_head = np.zeros((G, C))
                for i in range(G):
                    qh = q[b, t, g * G + i]                      # [d]
                    lo = kmin[b, g] * qh                         # [C, d]
                    hi = kmax[b, g] * qh
                    per_head[i] = scale * np.maximum(lo, hi).sum(axis=1)
                if reduce == "mean":
                    s[b, g, t] = per_head.mean(axis=0)
                elif reduce == "max":
                    s[b, g, t] = per_head.max(axis=0)
                else:
                    raise ValueError("reduce must be 'mean' or 'max'")
    return s


def minmax_topk(q, kmin, kmax, k: int, scale: float, reduce: str = "mean") -> np.ndarray:
    """The k chunks with the largest upper-bound score (ties to the lower id), ascending."""
    return topk_chunks(minmax_scores(q, kmin, kmax, scale, reduce), k)


# ----------------------------------------------------------------------------
# selection variants: coverage budgets (estimated attention mass)
# ----------------------------------------------------------------------------

def coverage_select(s: np.ndarray, gamma: float, k_max: int):
    """Smallest set of chunks whose estimated attention mass reaches gamma.

    MOIRA (abstract): per request, layer, KV head and step a coverage rule keeps
    the smallest set of pages whose estimated attention mass reaches a fraction
    gamma.  The estimate used here is the softmax of the chunk scores (the
    chunk's landmark logit), and the set is the shortest prefix of the chunks in
    (score descending, id ascending) order whose mass reaches gamma of the
    total, at least 1 and at most k_max chunks (the output buffer).
    s: [..., C].  Returns (idx [..., k_max] ascending ids, -1 padded;
    count [...] chunks kept).
    """
    s = np.asarray(s, dtype=np.float64)
    C = s.shape[-1]
    if not 1 <= k_max <= C:
        raise ValueError("need 1 <= k_max <= C")
    if not 0.0 < gamma <= 1.0:
        raise ValueError("need 0 < gamma <= 1")
    flat = s.reshape(-1, C)
    idx = np.full((flat.shape[0], k_max), -1, dtype=np.int64)
    count = np.zeros(flat.shape[0], dtype=np.int64)
    ids = np.arange(C)
    for r in range(flat.shape[0]):
        w = np.exp(flat[r] - flat[r].max())
        mass = w / w.sum()
        order = np.lexsort((ids, -flat[r]))
        total = 0.0
        n = 0
        while n < C:
            total += mass[order[n]]
            n += 1
            if total >= gamma:
                break
        n = max(1, min(n, k_max))
        idx[r, :n] = np.sort(order[:n])
        count[r] = n
    return idx.reshape(s.shape[:-1] + (k_max,)), count.reshape(s.shape[:-1])


def union_select_ragged(idx: np.ndarray, count: np.ndarray):
    """union_select for sets of different sizes: row t of idx[b, g] holds count[b, g, t] ids.

    Returns the same four arrays as union_select, with T * k_max union slots.
    """
    idx = np.asarray(idx)
    B, H, T, k = idx.shape
    union_ids = np.full((B, H, T * k), -1, dtype=np.int64)
    member = np.zeros((B, H, T * k), dtype=np.uint8)
    ucount = np.zeros((B, H), dtype=np.int64)
    overlap = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for g in range(H):
            sets = [set(int(c) for c in idx[b, g, t, :int(count[b, g, t])]) for t in range(T)]
            u = sorted(set().union(*sets))
            ucount[b, g] = len(u)
            for i, c in enumerate(u):
                union_ids[b, g, i] = c
                member[b, g, i] = sum(1 << t for t in range(T) if c in sets[t])
            overlap[b, g] = len(sets[0] & sets[1]) if T == 2 else len(sets[0])
    return union_ids, member, ucount, overlap


# ----------------------------------------------------------------------------
# selection variants: delta selection with capped LRU eviction
# ----------------------------------------------------------------------------

def capped_plan(sel_ids, sel_score, sel_count, resident, stamp, cap: int, step: int):
    """One step of a bounded per-(request, KV head) working set under capped eviction.

    OasisKV, "Delta Selection and Capped Eviction": resident blocks of the
    predicted set cost no traffic; resident blocks outside it are ranked by the
    step at which they were last selected; each admitted non-resident block is
    paired with one eviction target, least recently selected first; at most
    `cap` pairs are admitted per step and KV head.

    Readings: the predicted set P of (b, g) is sel_ids[b, g, :sel_count[b, g]]
    (ascending chunk ids) with priorities sel_score (None: all equal).  Hits keep
    their slot and their stamp becomes `step`.  Eviction targets are the slots
    whose chunk is not in P, empty slots first, then the oldest stamp, then the
    lower slot.  The admitted misses are the min(cap, #misses, #targets) best by
    (score descending, id ascending); they are paired in ascending chunk order
    with the chosen targets in ascending slot order, and stamped `step`.  Misses
    not admitted stay out of the working set for this step (slot -1).

    resident, stamp: [B, Hkv, S] (chunk per slot or -1; last-selected step).
    Returns a dict: resident, stamp (new arrays), sel_slot [B, Hkv, N] (slot of
    each entry after the step, -1 when dropped or padding), admit_chunk,
    admit_slot [B, Hkv, cap] (-1 padded), admit_count, hit_count [B, Hkv].
    """
    sel_ids = np.asarray(sel_ids)
    B, H, N = sel_ids.shape
    resident = np.array(resident, dtype=np.int64, copy=True)
    stamp = np.array(stamp, dtype=np.int64, copy=True)
    S = resident.shape[2]
    score = np.zeros(sel_ids.shape) if sel_score is None else np.asarray(sel_score, dtype=np.float64)
    count = np.full((B, H), N) if sel_count is None else np.asarray(sel_count)
    sel_slot = np.full((B, H, N), -1, dtype=np.int64)
    admit_chunk = np.full((B, H, cap), -1, dtype=np.int64)
    admit_slot = np.full((B, H, cap), -1, dtype=np.int64)
    admit_count = np.zeros((B, H), dtype=np.int64)
    hit_count = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for g in range(H):
            n = int(count[b, g])
            P = [int(c) for c in sel_ids[b, g, :n]]
            res, st = resident[b, g], stamp[b, g]
            where = {int(c): s for s, c in enumerate(res) if c >= 0}
            in_p = set(P)
            misses = []
            for i, c in enumerate(P):
                if c in where:
                    sel_slot[b, g, i] = where[c]
                    st[where[c]] = step
                    hit_count[b, g] += 1
                else:
                    misses.append(i)
            targets = [s for s in range(S) if res[s] < 0 or int(res[s]) not in in_p]
            targets.sort(key=lambda s: (res[s] >= 0, st[s] if res[s] >= 0 else 0, s))
            misses.sort(key=lambda i: (-score[b, g, i], P[i]))
            a = min(cap, len(misses), len(targets))
            admitted = sorted(misses[:a], key=lambda i: P[i])
            for r, (i, s) in enumerate(zip(admitted, sorted(targets[:a]))):
                res[s] = P[i]
                st[s] = step
                sel_slot[b, g, i] = s
                admit_chunk[b, g, r] = P[i]
                admit_slot[b, g, r] = s
            admit_count[b, g] = a
    return dict(resident=resident, stamp=stamp, sel_slot=sel_slot, admit_chunk=admit_chunk,
                admit_slot=admit_slot, admit_count=admit_count, hit_count=hit_count)
