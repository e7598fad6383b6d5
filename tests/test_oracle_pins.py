"""Pins of the CPU oracle against what the pages and mathematics fix.

Each check is written as a function of the oracle routine it pins, so that the
mutation tests at the bottom can hand it a plausibly wrong variant (a dropped
term, a wrong index, a reversed tie rule, the union's rows instead of a query's
own rows) and show that the pin fails on it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dualkv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# landmarks: mean key of each chunk
# ----------------------------------------------------------------------------

def check_landmarks(fn):
    fx = golden("landmarks_hand.json")
    lm = fn(np.array(fx["K"], dtype=np.float64), fx["chunk"])
    np.testing.assert_array_equal(lm, np.array(fx["expected_lm"], dtype=np.float64))
    rng = np.random.default_rng(1)
    K = rng.standard_normal((2, 3, 12, 5))
    # chunk = 1: every key is its own landmark
    np.testing.assert_array_equal(fn(K, 1), K)
    # keys constant inside each chunk: the landmark is that constant
    vals = rng.integers(-9, 9, size=(2, 3, 3, 5)).astype(np.float64)
    Kc = np.repeat(vals, 4, axis=2)
    np.testing.assert_array_equal(fn(Kc, 4), vals)
    # one chunk spanning L: the landmark is the mean over all keys (numpy's mean)
    np.testing.assert_allclose(fn(K, 12)[:, :, 0], np.mean(K, axis=2), rtol=0, atol=1e-14)


def test_landmarks_pins():
    check_landmarks(O.chunk_landmarks)


def test_landmarks_reject_ragged_length():
    with pytest.raises(ValueError):
        O.chunk_landmarks(np.zeros((1, 1, 10, 2)), 4)


# ----------------------------------------------------------------------------
# scores
# ----------------------------------------------------------------------------

def check_scores(fn):
    fx = golden("scores_hand.json")
    q = np.array(fx["q"], dtype=np.float64)
    lm = np.array(fx["lm"], dtype=np.float64)
    np.testing.assert_allclose(fn(q, lm, fx["scale"], "mean"), np.array(fx["expected_mean"]), atol=1e-15)
    np.testing.assert_allclose(fn(q, lm, fx["scale"], "max"), np.array(fx["expected_max"]), atol=1e-15)
    rng = np.random.default_rng(2)
    # G = 1: mean and max of one head agree
    q1 = rng.standard_normal((2, 2, 3, 7))
    lm1 = rng.standard_normal((2, 3, 11, 7))
    np.testing.assert_array_equal(fn(q1, lm1, 0.3, "mean"), fn(q1, lm1, 0.3, "max"))
    # group of 4 heads, rectangular shapes: compare with a brute-force triple loop
    q4 = rng.standard_normal((2, 2, 8, 6))
    lm4 = rng.standard_normal((2, 2, 9, 6))
    s = fn(q4, lm4, 0.25, "mean")
    sm = fn(q4, lm4, 0.25, "max")
    for b, g, t, c in itertools.product(range(2), range(2), range(2), range(9)):
        dots = [0.25 * sum(q4[b, t, h, i] * lm4[b, g, c, i] for i in range(6))
                for h in range(4 * g, 4 * g + 4)]
        assert abs(s[b, g, t, c] - sum(dots) / 4) < 1e-12
        assert abs(sm[b, g, t, c] - max(dots)) < 1e-12


def test_scores_pins():
    check_scores(O.chunk_scores)


# ----------------------------------------------------------------------------
# top-k
# ----------------------------------------------------------------------------

def brute_force_topk(row, k):
    """Among all k-subsets with the largest score sum, the lexicographically smallest."""
    best = None
    for sub in itertools.combinations(range(len(row)), k):
        key = (-sum(row[i] for i in sub), sub)
        if best is None or key < best:
            best = key
    return list(best[1])


def check_topk(fn):
    fx = golden("topk_ties_hand.json")
    for k, want in fx["cases"]:
        assert list(fn(np.array(fx["scores"], dtype=np.float64), k)) == want
    rng = np.random.default_rng(3)
    for trial in range(60):
        C = int(rng.integers(1, 11))
        k = int(rng.integers(1, C + 1))
        if trial % 2:
            row = rng.integers(0, 4, size=C).astype(np.float64)   # many ties
        else:
            row = rng.standard_normal(C)
        assert list(fn(row, k)) == brute_force_topk(row, k), (row, k)
    # distinct scores: the same set as torch.topk
    s = rng.standard_normal((4, 3, 200))
    got = fn(s, 17)
    ref = torch.topk(torch.from_numpy(s), 17, dim=-1).indices.sort(dim=-1).values.numpy()
    np.testing.assert_array_equal(got, ref)
    # k = C keeps everything
    np.testing.assert_array_equal(fn(s[0, 0], 200), np.arange(200))


def test_topk_pins():
    check_topk(O.topk_chunks)


# ----------------------------------------------------------------------------
# union
# ----------------------------------------------------------------------------

def check_union(fn):
    fx = golden("union_hand.json")
    u, m, c, o = fn(np.array(fx["idx"]))
    np.testing.assert_array_equal(u, fx["expected_union"])
    np.testing.assert_array_equal(m, fx["expected_member"])
    np.testing.assert_array_equal(c, fx["expected_count"])
    np.testing.assert_array_equal(o, fx["expected_overlap"])
    rng = np.random.default_rng(4)
    C, k = 40, 9
    idx = np.stack([np.stack([np.sort(rng.choice(C, k, replace=False)) for _ in range(2)])
                    for _ in range(6)]).reshape(2, 3, 2, k)
    u, m, c, o = fn(idx)
    for b, g in itertools.product(range(2), range(3)):
        n = c[b, g]
        ids = u[b, g, :n]
        assert n == 2 * k - o[b, g]
        assert k <= n <= min(2 * k, C)
        assert np.all(np.diff(ids) > 0)
        assert np.all(u[b, g, n:] == -1) and np.all(m[b, g, n:] == 0)
        for t in range(2):
            assert set(ids[(m[b, g, :n] >> t) & 1 == 1].tolist()) == set(idx[b, g, t].tolist())
        assert np.all(m[b, g, :n] > 0)
    # identical selections: union = each set, full overlap, accuracy exactly 1
    same = np.repeat(idx[:, :, :1], 2, axis=2)
    u, m, c, o = fn(same)
    assert np.all(c == k) and np.all(o == k) and np.all(m[:, :, :k] == 3)
    assert O.prediction_accuracy(o, k) == 1.0


def test_union_pins():
    check_union(O.union_select)


def test_union_single_query():
    idx = np.array([[[[2, 5, 6]]]])
    u, m, c, o = O.union_select(idx)
    assert u.tolist() == [[[2, 5, 6]]] and m.tolist() == [[[1, 1, 1]]]
    assert c.tolist() == [[3]] and o.tolist() == [[3]]


# ----------------------------------------------------------------------------
# attention over each query's own rows
# ----------------------------------------------------------------------------

def sdpa_masked(q, K, V, rows_mask, scale):
    """torch's scaled_dot_product_attention in fp64 on CPU with a boolean row mask."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None, :], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None], attn_mask=torch.from_numpy(rows_mask)[None, None, None, :],
        scale=scale)
    return out[0, 0, 0].numpy()


def check_attention(fn):
    fx = golden("attention_hand.json")
    out, lse = fn(np.array(fx["q"]), np.array(fx["K"]), np.array(fx["V"]), np.array(fx["sel"]),
                  fx["chunk"], fx["scale"])
    np.testing.assert_allclose(out, fx["expected_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, fx["expected_lse"], rtol=0, atol=1e-12)

    rng = np.random.default_rng(5)
    B, T, Hq, Hkv, dk, dv, chunk, C = 2, 2, 4, 2, 6, 5, 3, 7
    L = C * chunk
    q = rng.standard_normal((B, T, Hq, dk))
    K = rng.standard_normal((B, Hkv, L, dk))
    V = rng.standard_normal((B, Hkv, L, dv))
    G = Hq // Hkv
    # k = C: sparse attention is dense attention (library routine, fp64)
    sel_all = np.broadcast_to(np.arange(C), (B, Hkv, T, C))
    out, lse = fn(q, K, V, sel_all, chunk, 0.4)
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        ref = sdpa_masked(q[b, t, h], K[b, h // G], V[b, h // G], np.ones(L, dtype=bool), 0.4)
        np.testing.assert_allclose(out[b, t, h], ref, rtol=0, atol=1e-12)
        z = 0.4 * K[b, h // G] @ q[b, t, h]
        assert abs(lse[b, t, h] - math.log(np.sum(np.exp(z)))) < 1e-12
    # own sets differ per query: masked library attention over exactly those rows
    sel = np.zeros((B, Hkv, T, 3), dtype=np.int64)
    for b, g, t in itertools.product(range(B), range(Hkv), range(T)):
        sel[b, g, t] = np.sort(rng.choice(C, 3, replace=False))
    out, lse = fn(q, K, V, sel, chunk, 0.4)
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        mask = np.zeros(L, dtype=bool)
        for c in sel[b, h // G, t]:
            mask[c * chunk:(c + 1) * chunk] = True
        ref = sdpa_masked(q[b, t, h], K[b, h // G], V[b, h // G], mask, 0.4)
        np.testing.assert_allclose(out[b, t, h], ref, rtol=0, atol=1e-12)
    # one selected row: the output is that row's value, lse its logit
    sel1 = np.full((B, Hkv, T, 1), 4)
    out, lse = fn(q, K, V, sel1, 1, 0.4)
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        np.testing.assert_array_equal(out[b, t, h], V[b, h // G, 4])
        assert abs(lse[b, t, h] - 0.4 * K[b, h // G, 4] @ q[b, t, h]) < 1e-14
    # zero keys: uniform weights over the own rows, lse = log(#rows)
    out, lse = fn(q, np.zeros_like(K), V, sel, chunk, 0.4)
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        rows = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in sel[b, h // G, t]])
        np.testing.assert_allclose(out[b, t, h], V[b, h // G, rows].mean(axis=0), atol=1e-14)
        assert abs(lse[b, t, h] - math.log(len(rows))) < 1e-14


def test_attention_pins():
    check_attention(O.sparse_attention)


# ----------------------------------------------------------------------------
# attention with the tail and the step's own (fresh) rows
# ----------------------------------------------------------------------------

def tail_inputs(rng, B=2, T=2, Hq=4, Hkv=2, dk=6, dv=5, chunk=3, C=7, Lt=5):
    q = rng.standard_normal((B, T, Hq, dk))
    K = rng.standard_normal((B, Hkv, C * chunk, dk))
    V = rng.standard_normal((B, Hkv, C * chunk, dv))
    sel = np.zeros((B, Hkv, T, 3), dtype=np.int64)
    for b, g, t in itertools.product(range(B), range(Hkv), range(T)):
        sel[b, g, t] = np.sort(rng.choice(C, 3, replace=False))
    Kt = rng.standard_normal((B, Hkv, Lt, dk))
    Vt = rng.standard_normal((B, Hkv, Lt, dv))
    tl = np.array([Lt, 2][:B])
    Kn = rng.standard_normal((B, T, Hkv, dk))
    Vn = rng.standard_normal((B, T, Hkv, dv))
    return q, K, V, sel, chunk, Kt, Vt, tl, Kn, Vn


def check_attention_tail(fn):
    fx = golden("attention_tail_hand.json")
    out, lse = fn(np.array(fx["q"]), np.array(fx["K"]), np.array(fx["V"]), np.array(fx["sel"]), fx["chunk"],
                  fx["scale"], np.array(fx["K_tail"]), np.array(fx["V_tail"]), np.array(fx["tail_len"]),
                  np.array(fx["K_new"]), np.array(fx["V_new"]))
    np.testing.assert_allclose(out, fx["expected_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, fx["expected_lse"], rtol=0, atol=1e-12)

    rng = np.random.default_rng(11)
    q, K, V, sel, chunk, Kt, Vt, tl, Kn, Vn = tail_inputs(rng)
    B, T, Hq, _ = q.shape
    G = Hq // K.shape[1]
    out, lse = fn(q, K, V, sel, chunk, 0.4, Kt, Vt, tl, Kn, Vn)
    # the same rows laid out as one sequence (pool, tail, real, speculative) with a
    # boolean mask, through the library's masked attention in fp64
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        g = h // G
        Kall = np.concatenate([K[b, g], Kt[b, g], Kn[b, :, g]])
        Vall = np.concatenate([V[b, g], Vt[b, g], Vn[b, :, g]])
        L, Lt = K.shape[2], Kt.shape[2]
        mask = np.zeros(len(Kall), dtype=bool)
        for c in sel[b, g, t]:
            mask[c * chunk:(c + 1) * chunk] = True
        mask[L:L + tl[b]] = True
        mask[L + Lt:L + Lt + t + 1] = True        # causal: tokens up to t
        ref = sdpa_masked(q[b, t, h], Kall, Vall, mask, 0.4)
        np.testing.assert_allclose(out[b, t, h], ref, rtol=0, atol=1e-12)
        z = 0.4 * Kall[mask] @ q[b, t, h]
        assert abs(lse[b, t, h] - math.log(np.sum(np.exp(z)))) < 1e-12
    # causality: the speculative token's fresh row never reaches the real query ...
    Kn2, Vn2 = Kn.copy(), Vn.copy()
    Kn2[:, 1] = 50.0 * rng.standard_normal(Kn2[:, 1].shape)
    Vn2[:, 1] = 9.0
    out2, lse2 = fn(q, K, V, sel, chunk, 0.4, Kt, Vt, tl, Kn2, Vn2)
    np.testing.assert_array_equal(out2[:, 0], out[:, 0])
    np.testing.assert_array_equal(lse2[:, 0], lse[:, 0])
    # ... while the real token's fresh row reaches both
    Vn3 = Vn.copy()
    Vn3[:, 0] += 1.0
    out3, _ = fn(q, K, V, sel, chunk, 0.4, Kt, Vt, tl, Kn, Vn3)
    assert np.all(np.abs(out3[:, 0] - out[:, 0]) > 1e-9) and np.all(np.abs(out3[:, 1] - out[:, 1]) > 1e-9)
    # no tail and no fresh rows: plain sparse attention; an empty tail adds nothing
    o0, l0 = fn(q, K, V, sel, chunk, 0.4)
    r0, rl0 = O.sparse_attention(q, K, V, sel, chunk, 0.4)
    np.testing.assert_allclose(o0, r0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l0, rl0, rtol=0, atol=1e-13)
    o1, l1 = fn(q, K, V, sel, chunk, 0.4, Kt, Vt, np.zeros(B, dtype=np.int64))
    np.testing.assert_allclose(o1, r0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, rl0, rtol=0, atol=1e-13)


def test_attention_tail_pins():
    check_attention_tail(O.sparse_attention_tail)


# ----------------------------------------------------------------------------
# hot-cache plan
# ----------------------------------------------------------------------------

def check_cache_plan(fn):
    fx = golden("cache_plan_hand.json")
    p = fn(np.array(fx["resident"]), np.array(fx["union"]), np.array(fx["count"]))
    for key in ("new_resident", "slot_of_union", "miss_chunk", "miss_slot", "miss_count", "hit_count"):
        np.testing.assert_array_equal(p[key], fx["expected_" + key], err_msg=key)
    rng = np.random.default_rng(6)
    S, C, n = 12, 30, 8
    res = np.full((2, 2, S), -1)
    for step in range(6):
        u = np.full((2, 2, S), -1)
        cnt = np.zeros((2, 2), dtype=np.int64)
        for b, g in itertools.product(range(2), range(2)):
            m = int(rng.integers(1, n + 1))
            u[b, g, :m] = np.sort(rng.choice(C, m, replace=False))
            cnt[b, g] = m
        p = fn(res, u, cnt)
        for b, g in itertools.product(range(2), range(2)):
            m = cnt[b, g]
            ids = u[b, g, :m]
            new = p["new_resident"][b, g]
            assert sorted(new[new >= 0].tolist()) == sorted(ids.tolist())
            assert p["hit_count"][b, g] + p["miss_count"][b, g] == m
            old = {int(c): s for s, c in enumerate(res[b, g]) if c >= 0}
            for i, c in enumerate(ids):
                s = p["slot_of_union"][b, g, i]
                assert new[s] == c
                if c in old:
                    assert s == old[c]
            for j in range(p["miss_count"][b, g]):
                c, s = p["miss_chunk"][b, g, j], p["miss_slot"][b, g, j]
                assert c not in old and (res[b, g, s] < 0 or res[b, g, s] not in ids)
        # the same union again: every chunk is a hit
        p2 = fn(p["new_resident"], u, cnt)
        assert np.all(p2["miss_count"] == 0) and np.all(p2["hit_count"] == cnt)
        res = p["new_resident"]


def test_cache_plan_pins():
    check_cache_plan(O.cache_plan)


# ----------------------------------------------------------------------------
# whole step: sizes and composition
# ----------------------------------------------------------------------------

def test_pool_size_closed_form():
    from sparse_kv_retrieval_amd.workloads import WORKLOADS
    # OasisKV summary Eq. (1) for one layer: B * L * 2 * N_kv * d_h * s bytes
    w = WORKLOADS["b64_l128k"]
    assert w.pool_bytes() == 64 * 131072 * 2 * 8 * 128 * 2 == 34_359_738_368
    assert WORKLOADS["llama8b_l32k"].landmark_bytes() == 16 * 8 * 1024 * 128 * 4


def test_decode_step_identical_queries_full_accuracy():
    rng = np.random.default_rng(7)
    q1 = rng.standard_normal((2, 1, 4, 8))
    q = np.concatenate([q1, q1], axis=1)
    K = rng.standard_normal((2, 2, 64, 8))
    V = rng.standard_normal((2, 2, 64, 8))
    r = O.decode_step(q, K, V, chunk=4, k=5)
    assert r["accuracy"] == 1.0
    np.testing.assert_array_equal(r["out"][:, 0], r["out"][:, 1])


# ----------------------------------------------------------------------------
# the pins bite: each fails on a plausibly wrong oracle
# ----------------------------------------------------------------------------

def _landmarks_off_by_one(K, chunk):
    B, H, L, d = K.shape
    return K.reshape(B, H, L // chunk, chunk, d)[:, :, :, 1:, :].sum(axis=3) / chunk


def _landmarks_wrong_divisor(K, chunk):
    B, H, L, d = K.shape
    return K.reshape(B, H, L // chunk, chunk, d).sum(axis=3) / max(chunk - 1, 1)


def _scores_wrong_group(q, lm, scale, reduce="mean"):
    # query head h read against KV head h % Hkv instead of h // G
    B, T, Hq, d = q.shape
    Hkv = lm.shape[1]
    perm = np.concatenate([np.arange(g, Hq, Hkv) for g in range(Hkv)])
    return O.chunk_scores(q[:, :, perm], lm, scale, reduce)


def _scores_no_scale(q, lm, scale, reduce="mean"):
    return O.chunk_scores(q, lm, 1.0, reduce)


def _topk_ties_high_id(s, k):
    s = np.asarray(s, dtype=np.float64)
    C = s.shape[-1]
    flat = s.reshape(-1, C)
    out = np.zeros((flat.shape[0], k), dtype=np.int64)
    for r in range(flat.shape[0]):
        order = np.lexsort((-np.arange(C), -flat[r]))
        out[r] = np.sort(order[:k])
    return out.reshape(s.shape[:-1] + (k,))


def _union_overlap_wrong(idx):
    u, m, c, o = O.union_select(idx)
    return u, m, c, c - idx.shape[-1]


def _attention_over_union(q, K, V, sel, chunk, scale):
    # every query reads the union of the two sets instead of its own set
    B, T, Hq, dk = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, V.shape[3]))
    lse = np.zeros((B, T, Hq))
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        ids = sorted(set(sel[b, h // G].reshape(-1).tolist()))
        rows = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in ids])
        z = scale * K[b, h // G, rows] @ q[b, t, h]
        p = np.exp(z - z.max())
        out[b, t, h] = p @ V[b, h // G, rows] / p.sum()
        lse[b, t, h] = z.max() + math.log(p.sum())
    return out, lse


def _attention_lse_missing_max(q, K, V, sel, chunk, scale):
    out, lse = O.sparse_attention(q, K, V, sel, chunk, scale)
    return out, lse * 0.5


def _cache_plan_misses_descending_slots(resident, union_ids, count):
    # misses fill the free slots from the highest slot down
    B, H, S = resident.shape
    new = np.full((B, H, S), -1)
    sou = np.full(union_ids.shape, -1)
    mc = np.full(union_ids.shape, -1)
    ms = np.full(union_ids.shape, -1)
    mn = np.zeros((B, H), dtype=np.int64)
    hn = np.zeros((B, H), dtype=np.int64)
    for b, g in itertools.product(range(B), range(H)):
        u = [int(c) for c in union_ids[b, g, :int(count[b, g])]]
        where = {int(c): s for s, c in enumerate(resident[b, g]) if c >= 0}
        free = [s for s in range(S - 1, -1, -1) if int(resident[b, g, s]) not in set(u)]
        for i, c in enumerate(u):
            if c in where:
                s = where[c]
                hn[b, g] += 1
            else:
                s = free[mn[b, g]]
                mc[b, g, mn[b, g]] = c
                ms[b, g, mn[b, g]] = s
                mn[b, g] += 1
            sou[b, g, i] = s
            new[b, g, s] = c
    return dict(new_resident=new, slot_of_union=sou, miss_chunk=mc, miss_slot=ms,
                miss_count=mn, hit_count=hn)


def _tail_no_causal_mask(q, K, V, sel, chunk, scale, K_tail=None, V_tail=None, tail_len=None, K_new=None,
                         V_new=None):
    # every query sees every fresh row: the speculative token leaks into the real one
    if K_new is None:
        return O.sparse_attention_tail(q, K, V, sel, chunk, scale, K_tail, V_tail, tail_len)
    out = np.zeros(q.shape[:3] + (V.shape[3],))
    lse = np.zeros(q.shape[:3])
    for t in range(q.shape[1]):
        o, l = _tail_all_fresh(q[:, [t]], K, V, sel[:, :, [t]], chunk, scale, K_tail, V_tail, tail_len, K_new,
                               V_new)
        out[:, t], lse[:, t] = o[:, 0], l[:, 0]
    return out, lse


def _tail_all_fresh(q, K, V, sel, chunk, scale, K_tail, V_tail, tail_len, K_new, V_new):
    B, T1, Hq, dk = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, 1, Hq, V.shape[3]))
    lse = np.zeros((B, 1, Hq))
    for b, h in itertools.product(range(B), range(Hq)):
        g = h // G
        rows = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in sel[b, g, 0]])
        Kr = np.concatenate([K[b, g, rows]] + ([K_tail[b, g, :tail_len[b]]] if K_tail is not None else [])
                            + [K_new[b, :, g]])
        Vr = np.concatenate([V[b, g, rows]] + ([V_tail[b, g, :tail_len[b]]] if K_tail is not None else [])
                            + [V_new[b, :, g]])
        z = scale * Kr @ q[b, 0, h]
        p = np.exp(z - z.max())
        out[b, 0, h] = p @ Vr / p.sum()
        lse[b, 0, h] = z.max() + math.log(p.sum())
    return out, lse


def _tail_ignores_tail_len(q, K, V, sel, chunk, scale, K_tail=None, V_tail=None, tail_len=None, K_new=None,
                           V_new=None):
    full = None if tail_len is None else np.full_like(np.asarray(tail_len), K_tail.shape[2])
    return O.sparse_attention_tail(q, K, V, sel, chunk, scale, K_tail, V_tail, full, K_new, V_new)


# ----------------------------------------------------------------------------
# token-level selection over one latent KV head (indexer top-k, latent attention)
# ----------------------------------------------------------------------------

def check_indexer(fn):
    fx = golden("mla_token_hand.json")
    sel = fn(np.array(fx["qi"], dtype=np.float64), np.array(fx["Kidx"], dtype=np.float64), fx["k"],
             fx["index_scale"])
    np.testing.assert_array_equal(sel, fx["expected_topk"])
    ui, mb, ct, ov = O.union_select(sel)
    np.testing.assert_array_equal(ui, fx["expected_union_ids"])
    np.testing.assert_array_equal(mb, fx["expected_member"])
    np.testing.assert_array_equal(ct, fx["expected_count"])
    np.testing.assert_array_equal(ov, fx["expected_overlap"])

    rng = np.random.default_rng(11)
    B, T, Hi, di, L, k = 2, 2, 4, 8, 40, 6
    qi = rng.standard_normal((B, T, Hi, di))
    Kidx = rng.standard_normal((B, 1, L, di))
    sel = fn(qi, Kidx, k, 0.3)
    # linearity: the mean over heads of the scaled dots is the scaled dot with the
    # mean query, so the selection is the top-k of that single product (distinct scores)
    for b, t in itertools.product(range(B), range(T)):
        sc = 0.3 * (Kidx[b, 0] @ qi[b, t].mean(axis=0))
        assert len(set(np.round(sc, 9))) == L
        np.testing.assert_array_equal(sel[b, 0, t], np.sort(np.argsort(-sc)[:k]))
    # one-hot keys and one indexer head: the score of token n is scale * q[n % di], so the
    # k best tokens are the positions of the k largest query components (lowest
    # position first among the copies of a component)
    qi1 = rng.standard_normal((1, 1, 1, di))
    K1 = np.zeros((1, 1, 2 * di, di))
    for n in range(2 * di):
        K1[0, 0, n, n % di] = 1.0
    sel = fn(qi1, K1, 3, 0.5)
    top = np.argsort(-qi1[0, 0, 0])[:2]
    expect = sorted([int(top[0]), int(top[0]) + di, int(top[1])])
    np.testing.assert_array_equal(sel[0, 0, 0], expect)


def test_indexer_pins():
    check_indexer(O.indexer_topk)


def check_mla(fn):
    fx = golden("mla_token_hand.json")
    out, lse = fn(np.array(fx["q"]), np.array(fx["latent"], dtype=np.float64),
                  np.array(fx["expected_topk"]), fx["dv"], fx["scale"])
    np.testing.assert_allclose(out, fx["expected_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, fx["expected_lse"], rtol=0, atol=1e-12)

    rng = np.random.default_rng(12)
    B, T, Hq, dk, dv, L = 2, 2, 5, 9, 6, 12
    q = rng.standard_normal((B, T, Hq, dk))
    lat = rng.standard_normal((B, 1, L, dk))
    # every token selected: dense attention with the value aliasing the key's first dv
    # columns (library routine, fp64)
    sel_all = np.broadcast_to(np.arange(L), (B, 1, T, L))
    out, lse = fn(q, lat, sel_all, dv, 0.25)
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        Kb = lat[b, 0]
        ref = sdpa_masked(q[b, t, h], Kb, np.ascontiguousarray(Kb[:, :dv]), np.ones(L, dtype=bool), 0.25)
        np.testing.assert_allclose(out[b, t, h], ref, rtol=0, atol=1e-12)
    # own token sets: masked library attention
    sel = np.zeros((B, 1, T, 4), dtype=np.int64)
    for b, t in itertools.product(range(B), range(T)):
        sel[b, 0, t] = np.sort(rng.choice(L, 4, replace=False))
    out, lse = fn(q, lat, sel, dv, 0.25)
    for b, t, h in itertools.product(range(B), range(T), range(Hq)):
        mask = np.zeros(L, dtype=bool)
        mask[sel[b, 0, t]] = True
        Kb = lat[b, 0]
        ref = sdpa_masked(q[b, t, h], Kb, np.ascontiguousarray(Kb[:, :dv]), mask, 0.25)
        np.testing.assert_allclose(out[b, t, h], ref, rtol=0, atol=1e-12)


def test_mla_pins():
    check_mla(O.mla_attention)


def test_mla_decode_step_composes():
    fx = golden("mla_token_hand.json")
    r = O.mla_decode_step(np.array(fx["qi"], dtype=np.float64), np.array(fx["Kidx"], dtype=np.float64),
                          np.array(fx["q"]), np.array(fx["latent"], dtype=np.float64), fx["k"], fx["dv"],
                          fx["index_scale"], fx["scale"])
    np.testing.assert_array_equal(r["topk"], fx["expected_topk"])
    np.testing.assert_allclose(r["out"], fx["expected_out"], atol=1e-12)
    assert r["accuracy"] == 0.5


def _indexer_max_over_heads(qi, Kidx, k, scale):
    return O.topk_chunks(O.chunk_scores(qi, Kidx, scale, "max"), k)


def _indexer_first_head_only(qi, Kidx, k, scale):
    return O.topk_chunks(O.chunk_scores(qi[:, :, :1], Kidx, scale, "mean"), k)


def _mla_value_from_last_columns(q, latent, sel, dv, scale):
    latent = np.asarray(latent, dtype=np.float64)
    return O.sparse_attention(q, latent, latent[..., -dv:], sel, 1, scale)


def _mla_key_content_only(q, latent, sel, dv, scale):
    latent = np.asarray(latent, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    return O.sparse_attention(q[..., :dv], latent[..., :dv], latent[..., :dv], sel, 1, scale)


# ----------------------------------------------------------------------------
# min/max chunk summaries and their upper-bound scores
# ----------------------------------------------------------------------------

def check_minmax(fn):
    """fn(q, kmin, kmax, scale, reduce) -> scores; pins the bound and its summaries."""
    fx = golden("minmax_hand.json")
    mn, mx = O.chunk_minmax(np.array(fx["K"], dtype=np.float64), fx["chunk"])
    np.testing.assert_array_equal(mn, fx["expected_kmin"])
    np.testing.assert_array_equal(mx, fx["expected_kmax"])
    q = np.array(fx["q"], dtype=np.float64)
    np.testing.assert_allclose(fn(q, mn, mx, fx["scale"], "mean"), fx["expected_scores_mean"], atol=1e-12)
    np.testing.assert_allclose(fn(q, mn, mx, fx["scale"], "max"), fx["expected_scores_max"], atol=1e-12)
    np.testing.assert_array_equal(O.topk_chunks(fn(q, mn, mx, fx["scale"], "mean"), fx["k"]),
                                  fx["expected_topk_mean"])

    rng = np.random.default_rng(21)
    B, T, Hq, Hkv, d, chunk, C = 2, 2, 4, 2, 6, 4, 9
    K = rng.standard_normal((B, Hkv, C * chunk, d))
    q = rng.standard_normal((B, T, Hq, d))
    mn, mx = O.chunk_minmax(K, chunk)
    G = Hq // Hkv
    # one head per KV head: the score bounds every key's dot product in the chunk, and
    # is reached when the chunk holds the corner the query's signs pick
    for h in range(Hq):
        g = h // G
        s1 = fn(q[:, :, h:h + 1], mn[:, g:g + 1], mx[:, g:g + 1], 0.7, "mean")
        for b, t, c in itertools.product(range(B), range(T), range(C)):
            dots = 0.7 * K[b, g, c * chunk:(c + 1) * chunk] @ q[b, t, h]
            assert s1[b, 0, t, c] >= dots.max() - 1e-12
    Kc = K.copy()
    for b, g, c in itertools.product(range(B), range(Hkv), range(C)):
        qs = q[b, 0, g * G]
        lo, hi = mn[b, g, c], mx[b, g, c]
        Kc[b, g, c * chunk] = np.where(qs >= 0, hi, lo)      # the corner is one of the keys
    mnc, mxc = O.chunk_minmax(Kc, chunk)
    s1 = fn(q[:, :1, ::G], mnc, mxc, 0.7, "mean")
    for b, g, c in itertools.product(range(B), range(Hkv), range(C)):
        dots = 0.7 * Kc[b, g, c * chunk:(c + 1) * chunk] @ q[b, 0, g * G]
        assert abs(s1[b, g, 0, c] - dots.max()) < 1e-12
    # chunk 1: the box is the key, the bound is the exact score
    mn1, mx1 = O.chunk_minmax(K, 1)
    np.testing.assert_allclose(fn(q, mn1, mx1, 0.3, "mean"), O.chunk_scores(q, K, 0.3, "mean"), atol=1e-12)
    np.testing.assert_allclose(fn(q, mn1, mx1, 0.3, "max"), O.chunk_scores(q, K, 0.3, "max"), atol=1e-12)


def test_minmax_pins():
    check_minmax(O.minmax_scores)


def _minmax_lower_bound(q, kmin, kmax, scale, reduce="mean"):
    # the smallest dot product in the box instead of the largest
    return -O.minmax_scores(-np.asarray(q), kmin, kmax, scale, reduce)


def _minmax_no_sign_branch(q, kmin, kmax, scale, reduce="mean"):
    return O.chunk_scores(q, np.asarray(kmax), scale, reduce)



# ----------------------------------------------------------------------------
# coverage budgets: smallest set of chunks reaching a fraction of the mass
# ----------------------------------------------------------------------------

def check_coverage(fn):
    """fn(s, gamma, k_max) -> (idx, count); pins the coverage rule."""
    fx = golden("coverage_hand.json")
    s = np.array(fx["scores"], dtype=np.float64)
    for case in fx["cases"]:
        idx, n = fn(s, case["gamma"], case["k_max"])
        np.testing.assert_array_equal(idx, case["idx"], err_msg=str(case))
        np.testing.assert_array_equal(n, case["count"], err_msg=str(case))

    # brute force over every subset: the count is the size of the smallest set whose
    # softmax mass reaches gamma (at most k_max), and the kept set has the largest
    # mass among the sets of that size
    rng = np.random.default_rng(31)
    checked = 0
    for _ in range(300):
        C = int(rng.integers(1, 8))
        row = np.round(rng.standard_normal(C) * 2) / 2          # half-steps: ties occur
        gamma = float(rng.uniform(0.05, 1.0))
        k_max = int(rng.integers(1, C + 1))
        m = np.exp(row - row.max())
        m = m / m.sum()
        sub = [(sum(m[list(S)]), S) for r in range(1, C + 1) for S in itertools.combinations(range(C), r)]
        if min(abs(v - gamma) for v, _ in sub) < 1e-9:
            continue                                           # a boundary the sum order decides
        n_bf = min(len(S) for v, S in sub if v >= gamma)
        n_bf = min(n_bf, k_max)
        idx, n = fn(row[None], gamma, k_max)
        assert int(n[0]) == n_bf, (row, gamma, k_max, n, n_bf)
        kept = idx[0, :n_bf]
        assert np.all(np.diff(kept) > 0) and np.all(idx[0, n_bf:] == -1)
        best = max(v for v, S in sub if len(S) == n_bf)
        assert sum(m[kept]) >= best - 1e-12
        checked += 1
    assert checked > 200

    rows = rng.standard_normal((3, 5, 40)) * 3
    # softmax masses: adding a constant to every score changes nothing
    for gamma in (0.2, 0.6, 0.95):
        a = fn(rows, gamma, 40)
        b = fn(rows + 3.7, gamma, 40)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
    # a tiny gamma keeps the best chunk only; gamma = 1 keeps k_max chunks
    idx, n = fn(rows, 1e-9, 7)
    assert np.all(n == 1) and np.all(idx[..., 0] == rows.argmax(axis=-1))
    idx, n = fn(rows, 1.0, 7)
    assert np.all(n == 7)
    np.testing.assert_array_equal(idx, O.topk_chunks(rows, 7))
    # equal scores: masses 1/C, the first ceil(gamma C) ids
    idx, n = fn(np.zeros((1, 16)), 3 / 8, 16)
    assert n[0] == 6 and idx[0, :6].tolist() == list(range(6))
    # one dominant chunk carries nearly all of the mass
    row = np.zeros((1, 9))
    row[0, 4] = 40.0
    idx, n = fn(row, 0.99, 9)
    assert n[0] == 1 and idx[0, 0] == 4


def test_coverage_pins():
    check_coverage(O.coverage_select)


def test_coverage_rejects():
    with pytest.raises(ValueError):
        O.coverage_select(np.zeros((1, 4)), 0.0, 2)
    with pytest.raises(ValueError):
        O.coverage_select(np.zeros((1, 4)), 1.5, 2)
    with pytest.raises(ValueError):
        O.coverage_select(np.zeros((1, 4)), 0.5, 5)


def check_union_ragged(fn):
    """fn(idx, count) -> union_select's four arrays, for rows of different sizes."""
    rng = np.random.default_rng(32)
    C, k = 30, 8
    idx = np.stack([np.sort(rng.choice(C, k, replace=False)) for _ in range(12)]).reshape(2, 3, 2, k)
    # full rows: the same as the fixed-size union
    full = fn(idx, np.full((2, 3, 2), k))
    for a, b in zip(full, O.union_select(idx)):
        np.testing.assert_array_equal(a[..., :b.shape[-1]], b)
        assert np.all(a[..., b.shape[-1]:] <= 0)
    # ragged rows: ids past a row's count are padding and take no part
    count = rng.integers(1, k + 1, size=(2, 3, 2))
    padded = idx.copy()
    for b, g, t in itertools.product(range(2), range(3), range(2)):
        padded[b, g, t, count[b, g, t]:] = -1
    u, m, c, o = fn(padded, count)
    for b, g in itertools.product(range(2), range(3)):
        sets = [set(idx[b, g, t, :count[b, g, t]].tolist()) for t in range(2)]
        n = c[b, g]
        assert n == len(sets[0] | sets[1]) == count[b, g, 0] + count[b, g, 1] - o[b, g]
        assert o[b, g] == len(sets[0] & sets[1])
        ids = u[b, g, :n]
        assert np.all(np.diff(ids) > 0) and np.all(u[b, g, n:] == -1) and np.all(m[b, g, n:] == 0)
        for t in range(2):
            assert set(ids[(m[b, g, :n] >> t) & 1 == 1].tolist()) == sets[t]


def test_union_ragged_pins():
    check_union_ragged(O.union_select_ragged)


def _coverage_strict(s, gamma, k_max):
    # stops only once the mass exceeds gamma
    return O.coverage_select(s, min(1.0, gamma * (1 + 1e-12)), k_max)


def _coverage_raw_scores(s, gamma, k_max):
    # mass proportional to the shifted scores instead of their exponentials
    s = np.asarray(s, dtype=np.float64)
    lin = np.log(s - s.min(axis=-1, keepdims=True) + 1e-3)
    return O.coverage_select(lin, gamma, k_max)


def _coverage_ties_high_id(s, gamma, k_max):
    s = np.asarray(s, dtype=np.float64)
    idx, n = O.coverage_select(s[..., ::-1], gamma, k_max)
    C = s.shape[-1]
    out = np.where(idx >= 0, C - 1 - idx, -1)
    out = np.sort(np.where(out >= 0, out, C + 1), axis=-1)
    return np.where(out <= C, out, -1), n


def _coverage_stop_before(s, gamma, k_max):
    # keeps the chunks before the one that reaches gamma
    s = np.asarray(s, dtype=np.float64)
    idx, n = O.coverage_select(s, gamma, k_max)
    n2 = np.maximum(n - 1, 1)
    res = np.full(idx.shape, -1).reshape(-1, idx.shape[-1])
    rows = s.reshape(-1, s.shape[-1])
    for r, c in enumerate(n2.reshape(-1)):
        res[r, :c] = np.sort(O.topk_chunks(rows[r:r + 1], int(c))[0])
    return res.reshape(idx.shape), n2


def _union_ragged_ignores_count(idx, count):
    return O.union_select_ragged(idx, np.full(np.asarray(count).shape, np.asarray(idx).shape[-1]))


# ----------------------------------------------------------------------------
# delta selection with capped LRU eviction
# ----------------------------------------------------------------------------

def lru_reference(seq, S):
    """Textbook LRU cache of S entries over an access sequence: (hit, evicted) per access."""
    from collections import OrderedDict
    cache, out = OrderedDict(), []
    for x in seq:
        if x in cache:
            cache.move_to_end(x)
            out.append((True, None))
            continue
        ev = None
        if len(cache) == S:
            ev, _ = cache.popitem(last=False)
        cache[x] = True
        out.append((False, ev))
    return out, set(cache)


def check_capped(fn):
    """fn(sel_ids, sel_score, sel_count, resident, stamp, cap, step) -> dict; pins the capped plan."""
    fx = golden("capped_plan_hand.json")
    for case in fx["cases"]:
        r = fn(np.array(fx["sel_ids"])[None, None], np.array(fx["sel_score"])[None, None] if case["scores"] else None,
               None, np.array(fx["resident"])[None, None], np.array(fx["stamp"])[None, None], case["cap"], fx["step"])
        for key in ("resident", "stamp", "sel_slot", "admit_chunk", "admit_slot"):
            np.testing.assert_array_equal(r[key][0, 0], case[key], err_msg=f"{key} {case['cap']}")
        assert r["admit_count"][0, 0] == case["admit_count"] and r["hit_count"][0, 0] == case["hit_count"]

    # one block per step and one admission per step: a textbook LRU cache
    rng = np.random.default_rng(41)
    S, seq = 5, rng.integers(0, 12, size=300).tolist()
    ref, final = lru_reference(seq, S)
    res, st = np.full((1, 1, S), -1), np.full((1, 1, S), -1)
    for step, (x, (hit, ev)) in enumerate(zip(seq, ref)):
        before = set(res[0, 0].tolist())
        r = fn(np.array([[[x]]]), None, None, res, st, 1, step)
        res, st = r["resident"], r["stamp"]
        assert (r["hit_count"][0, 0] == 1) == hit, step
        after = set(res[0, 0].tolist())
        if ev is not None:
            assert before - after == {ev}, (step, before, after, ev)
        assert x in after
    assert set(res[0, 0].tolist()) == final

    # from an empty cache with room for every miss: the uncapped cache plan
    B, H, S, N = 2, 3, 40, 12
    ids = np.stack([np.sort(rng.choice(100, N, replace=False)) for _ in range(B * H)]).reshape(B, H, N)
    cnt = rng.integers(1, N + 1, size=(B, H))
    sc = rng.standard_normal((B, H, N))
    empty = np.full((B, H, S), -1)
    r = fn(ids, sc, cnt, empty, empty, N, 3)
    u = np.where(np.arange(N) < cnt[..., None], ids, -1)
    cp = O.cache_plan(empty, u, cnt)
    np.testing.assert_array_equal(r["sel_slot"], cp["slot_of_union"])
    np.testing.assert_array_equal(r["resident"], cp["new_resident"])

    # invariants over random multi-step traces
    res = np.full((B, H, S), -1)
    st = np.full((B, H, S), -1)
    for step in range(12):
        ids = np.stack([np.sort(rng.choice(60, N, replace=False)) for _ in range(B * H)]).reshape(B, H, N)
        cnt = rng.integers(1, N + 1, size=(B, H))
        sc = np.round(rng.standard_normal((B, H, N)), 1)
        cap = int(rng.integers(0, 6))
        r = fn(ids, sc, cnt, res, st, cap, step)
        for b, g in itertools.product(range(B), range(H)):
            n = cnt[b, g]
            P = ids[b, g, :n].tolist()
            old, new = res[b, g], r["resident"][b, g]
            a = int(r["admit_count"][b, g])
            assert a <= cap
            occ = new[new >= 0]
            assert len(set(occ.tolist())) == len(occ)                          # distinct chunks
            changed = np.nonzero(old != new)[0]
            assert len(changed) == a and set(changed.tolist()) == set(r["admit_slot"][b, g, :a].tolist())
            for s in changed:
                assert old[s] < 0 or old[s] not in P                           # hits are never evicted
            # least recently selected first: no surviving candidate is older than an evicted one
            surv = [s for s in range(S) if s not in changed and (old[s] < 0 or old[s] not in P)]
            for s in changed:
                for t in surv:
                    ks = (old[s] >= 0, st[b, g, s] if old[s] >= 0 else 0, s)
                    kt = (old[t] >= 0, st[b, g, t] if old[t] >= 0 else 0, t)
                    assert ks < kt, (step, b, g, s, t)
            # the best misses are admitted
            miss = [i for i in range(n) if P[i] not in old.tolist()]
            adm = [i for i in miss if r["sel_slot"][b, g, i] >= 0]
            drop = [i for i in miss if r["sel_slot"][b, g, i] < 0]
            assert len(adm) == a and len(drop) == len(miss) - a
            for i in adm:
                for j in drop:
                    assert (-sc[b, g, i], P[i]) < (-sc[b, g, j], P[j])
            for i in range(n):
                s = r["sel_slot"][b, g, i]
                assert s < 0 or new[s] == P[i]
                if s >= 0:
                    assert r["stamp"][b, g, s] == step
        res, st = r["resident"], r["stamp"]


def test_capped_pins():
    check_capped(O.capped_plan)


def _capped_mru(sel_ids, sel_score, sel_count, resident, stamp, cap, step):
    # evicts the most recently selected block first
    r = O.capped_plan(sel_ids, sel_score, sel_count, resident, -np.asarray(stamp), cap, step)
    r["stamp"] = np.where(r["stamp"] == step, step, np.asarray(stamp))
    return r


def _capped_ignores_cap(sel_ids, sel_score, sel_count, resident, stamp, cap, step):
    r = O.capped_plan(sel_ids, sel_score, sel_count, resident, stamp, 10 ** 6, step)
    r["admit_chunk"] = r["admit_chunk"][..., :cap]
    r["admit_slot"] = r["admit_slot"][..., :cap]
    return r


def _capped_low_score_first(sel_ids, sel_score, sel_count, resident, stamp, cap, step):
    neg = None if sel_score is None else -np.asarray(sel_score)
    return O.capped_plan(sel_ids, neg, sel_count, resident, stamp, cap, step)


def _capped_hits_not_restamped(sel_ids, sel_score, sel_count, resident, stamp, cap, step):
    r = O.capped_plan(sel_ids, sel_score, sel_count, resident, stamp, cap, step)
    kept = np.asarray(resident) == r["resident"]
    r["stamp"] = np.where(kept, np.asarray(stamp), r["stamp"])
    return r


@pytest.mark.parametrize("check,bad", [
    (check_capped, _capped_mru),
    (check_capped, _capped_ignores_cap),
    (check_capped, _capped_low_score_first),
    (check_capped, _capped_hits_not_restamped),
    (check_coverage, _coverage_strict),
    (check_coverage, _coverage_raw_scores),
    (check_coverage, _coverage_ties_high_id),
    (check_coverage, _coverage_stop_before),
    (check_union_ragged, _union_ragged_ignores_count),
    (check_minmax, _minmax_lower_bound),
    (check_minmax, _minmax_no_sign_branch),
    (check_indexer, _indexer_max_over_heads),
    (check_indexer, _indexer_first_head_only),
    (check_mla, _mla_value_from_last_columns),
    (check_mla, _mla_key_content_only),
    (check_attention_tail, _tail_no_causal_mask),
    (check_attention_tail, _tail_ignores_tail_len),
    (check_landmarks, _landmarks_off_by_one),
    (check_landmarks, _landmarks_wrong_divisor),
    (check_scores, _scores_wrong_group),
    (check_scores, _scores_no_scale),
    (check_topk, _topk_ties_high_id),
    (check_union, _union_overlap_wrong),
    (check_attention, _attention_over_union),
    (check_attention, _attention_lse_missing_max),
    (check_cache_plan, _cache_plan_misses_descending_slots),
])
def test_pins_reject_planted_mistakes(check, bad):
    with pytest.raises(AssertionError):
        check(bad)
