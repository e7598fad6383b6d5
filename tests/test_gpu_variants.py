"""GPU parity of the selection variants against the oracle.

Min/max chunk summaries (dk_build_minmax) are bit-exact; their upper-bound
top-k (dk_score_topk_minmax) matches the oracle's minmax_topk except at counted
near-ties, its reported scores lie within a derived fp32 bound, and its union
equals the oracle's union of the GPU's own sets.

Coverage budgets (dk_score_coverage): each row's count is one the oracle's
cumulative masses allow within a derived fp32 bound (equal to the oracle's count
away from that band), the kept ids are the oracle's best `count` chunks except at
counted score near-ties, and the union of the ragged sets is exact against the
oracle's union of the GPU's own sets.
"""
import numpy as np
import pytest
import torch

from oracle import dualkv_oracle as O
from sparse_kv_retrieval_amd import synth
from sparse_kv_retrieval_amd.workloads import WORKLOADS, shrink

from parity_utils import compare_topk

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def dkb():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a GPU")
    from sparse_kv_retrieval_amd import binding   # raises if libdualkv.so is missing
    return binding


def workload(name, B=None, L=None, **kw):
    w = WORKLOADS[name]
    if B is not None or L is not None:
        w = shrink(w, B=B, L=L)
    return w.with_(**kw) if kw else w


@pytest.mark.parametrize("name,B,L,strided", [("tiny", None, None, False), ("llama8b_l32k", 2, 4096, False),
                                               ("llama8b_l32k", 2, 4096, True)])
def test_build_minmax(dkb, name, B, L, strided):
    w = workload(name, B, L)
    q = synth.make_queries(w, 5, device="cuda")
    K, _ = synth.make_kv_pool(w, 5, device="cuda", q0=q)
    if strided:   # a [B, L, Hkv, d] buffer read through a permuted view
        K = K.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    mn, mx = dkb.build_minmax(K, w.chunk)
    torch.cuda.synchronize()
    rmn, rmx = O.chunk_minmax(synth.to_numpy_f64(K), w.chunk)
    np.testing.assert_array_equal(synth.to_numpy_f64(mn), rmn)
    np.testing.assert_array_equal(synth.to_numpy_f64(mx), rmx)


def check_minmax_topk(dkb, w, q, K, reduce, union=False):
    mn, mx = dkb.build_minmax(K, w.chunk)
    red = dkb.DK_REDUCE_MAX if reduce == "max" else dkb.DK_REDUCE_MEAN
    res = dkb.score_topk_minmax(q, mn, mx, w.k, w.scale, red, union=union)
    torch.cuda.synchronize()
    idx, sc = res[0], res[1]
    qh = q.cpu().numpy().astype(np.float64)
    mnh, mxh = synth.to_numpy_f64(mn), synth.to_numpy_f64(mx)
    s_ref = O.minmax_scores(qh, mnh, mxh, w.scale, reduce)
    idx_ref = O.topk_chunks(s_ref, w.k)
    gi = idx.cpu().numpy().astype(np.int64)
    rows_diff, near, hard = compare_topk(gi, idx_ref, s_ref)
    assert not hard, hard[:5]
    # reported scores: fp32 rounding of the head means (G terms) and of the 2d-term
    # sum over centre and radius, bounded through |centre| + |radius| <= |min| + |max|
    B, T, Hq, d = qh.shape
    G = Hq // w.Hkv
    qa = np.abs(qh).reshape(B, T, w.Hkv, G, d).mean(axis=3)
    mag = abs(w.scale) * np.einsum("btgd,bgcd->bgtc", qa, np.abs(mnh) + np.abs(mxh))
    if reduce == "max":
        mag = abs(w.scale) * np.einsum("btgid,bgcd->bgtc", np.abs(qh).reshape(B, T, w.Hkv, G, d),
                                       np.abs(mnh) + np.abs(mxh))
    err = np.abs(sc.cpu().numpy().astype(np.float64) - np.take_along_axis(s_ref, gi, axis=-1))
    bound = (G + 2 * d + 8) * U32 * np.take_along_axis(mag, gi, axis=-1) * 1.01 + 1e-30
    assert np.all(err <= bound), float((err / bound).max())
    if union:
        uid, mem, cnt, ov = res[2:]
        ru, rm, rc, ro = O.union_select(gi)
        np.testing.assert_array_equal(uid.cpu().numpy(), ru)
        np.testing.assert_array_equal(mem.cpu().numpy(), rm)
        np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
        np.testing.assert_array_equal(ov.cpu().numpy(), ro)
    return near


@pytest.mark.parametrize("name,B,L,reduce,union", [
    ("tiny", None, None, "mean", True),
    ("tiny", None, None, "max", False),
    ("llama8b_l32k", 2, 4096, "mean", True),
    ("llama8b_l32k", 2, 4096, "max", True),
    ("llama8b_l32k", 3, 8192, "mean", False),
])
def test_minmax_topk(dkb, name, B, L, reduce, union):
    w = workload(name, B, L)
    print(f"case {name} B={B} L={L} {reduce} union={union}", flush=True)
    q = synth.make_queries(w, 7, device="cuda")
    K, _ = synth.make_kv_pool(w, 7, device="cuda", q0=q)
    check_minmax_topk(dkb, w, q, K, reduce, union)


def test_minmax_topk_one_query(dkb):
    w = workload("llama8b_l32k", 2, 4096, T=1)
    q = synth.make_queries(w, 8, device="cuda")
    K, _ = synth.make_kv_pool(w, 8, device="cuda", q0=q)
    check_minmax_topk(dkb, w, q, K, "mean", True)


def test_minmax_topk_full_128k_sampled(dkb):
    """b64_l128k's shape (C = 4096 chunks per (b, g)); oracle on sampled (b, g)."""
    w = WORKLOADS["b64_l128k"]
    q = synth.make_queries(w, 9, device="cuda")
    K, _ = synth.make_kv_pool(w, 9, device="cuda", q0=q)
    mn, mx = dkb.build_minmax(K, w.chunk)
    del K
    idx, _, uid, mem, cnt, ov = dkb.score_topk_minmax(q, mn, mx, w.k, w.scale, union=True)
    torch.cuda.synchronize()
    for b, g in ((0, 0), (31, 3), (63, 7)):
        qh = q[b:b + 1, :, g * w.G:(g + 1) * w.G].cpu().numpy().astype(np.float64)
        mnh = synth.to_numpy_f64(mn[b:b + 1, g:g + 1])
        mxh = synth.to_numpy_f64(mx[b:b + 1, g:g + 1])
        s_ref = O.minmax_scores(qh, mnh, mxh, w.scale)
        gi = idx[b:b + 1, g:g + 1].cpu().numpy().astype(np.int64)
        rows_diff, near, hard = compare_topk(gi, O.topk_chunks(s_ref, w.k), s_ref)
        assert not hard, (b, g, hard[:5])
        ru, rm, rc, _ = O.union_select(gi)
        np.testing.assert_array_equal(uid[b:b + 1, g:g + 1].cpu().numpy(), ru)
        np.testing.assert_array_equal(cnt[b:b + 1, g:g + 1].cpu().numpy(), rc)


# ----------------------------------------------------------------------------
# coverage budgets
# ----------------------------------------------------------------------------

def check_coverage(dkb, q, lm, gamma, k_max, scale, reduce="mean", union=False, label=""):
    """GPU coverage selection against the oracle on the same inputs; returns the
    number of rows whose count differs from the oracle's (inside the rounding band)."""
    red = dkb.DK_REDUCE_MAX if reduce == "max" else dkb.DK_REDUCE_MEAN
    res = dkb.score_coverage(q, lm, gamma, k_max, scale, red, union=union)
    torch.cuda.synchronize()
    idx, cnt, sc = res[0], res[1], res[2]
    qh = q.cpu().numpy().astype(np.float64)
    lh = synth.to_numpy_f64(lm)
    B, T, Hq, d = qh.shape
    Hkv, C = lh.shape[1], lh.shape[2]
    G = Hq // Hkv
    s_ref = O.chunk_scores(qh, lh, scale, reduce)
    _, n_ref = O.coverage_select(s_ref, gamma, k_max)
    gi = idx.cpu().numpy().astype(np.int64)
    gn = cnt.cpu().numpy().astype(np.int64)
    gs = sc.cpu().numpy().astype(np.float64)
    # score error: fp32 head mean (G terms) or per-head products, d-term dot products
    qa = np.abs(qh).reshape(B, T, Hkv, G, d)
    per_head = abs(scale) * np.einsum("btgid,bgcd->bgtci", qa, np.abs(lh))
    mag = per_head.max(axis=-1) if reduce == "max" else per_head.mean(axis=-1)
    err_s = (G + d + 4) * U32 * mag * 1.01 + 1e-30
    # masses move by at most 2 max|score error| (relative) under score errors; the
    # fp32 sums add at most (terms per thread + 6 butterfly + 16 waves) roundings,
    # exp and the target a few more
    ept = 1 << max(0, int(np.ceil(np.log2(max(C, 1024) / 1024))))
    delta = 2 * err_s.max(axis=-1) + (ept + 6 + 16 + 8) * U32
    rows = gi.reshape(-1, k_max)
    counts = gn.reshape(-1)
    srows = s_ref.reshape(-1, C)
    drows = delta.reshape(-1)
    moved, near_total = 0, 0
    for r in range(rows.shape[0]):
        n = int(counts[r])
        assert 1 <= n <= k_max, (label, r, n)
        row = srows[r]
        m = np.exp(row - row.max())
        m /= m.sum()
        order = np.lexsort((np.arange(C), -row))
        cum = np.cumsum(m[order])
        if n < k_max:
            assert cum[n - 1] >= gamma - drows[r], (label, r, n, cum[n - 1], gamma)
        if n > 1:
            assert cum[n - 2] < gamma + drows[r], (label, r, n, cum[n - 2], gamma)
        moved += n != int(n_ref.reshape(-1)[r])
        kept = rows[r, :n]
        assert np.all(rows[r, n:] == -1), (label, r)
        _, near, hard = compare_topk(kept[None], O.topk_chunks(row[None], n), row[None])
        assert not hard, (label, r, hard[:5])
        near_total += near
        e = np.abs(gs.reshape(-1, k_max)[r, :n] - row[kept])
        assert np.all(e <= err_s.reshape(-1, C)[r, kept]), (label, r, float(e.max()))
        assert np.all(np.isneginf(gs.reshape(-1, k_max)[r, n:]))
    if union:
        uid, mem, ucnt, ov = res[3:]
        ru, rm, rc, ro = O.union_select_ragged(gi, gn)
        np.testing.assert_array_equal(uid.cpu().numpy(), ru[..., :T * k_max])
        np.testing.assert_array_equal(mem.cpu().numpy(), rm[..., :T * k_max])
        np.testing.assert_array_equal(ucnt.cpu().numpy(), rc)
        np.testing.assert_array_equal(ov.cpu().numpy(), ro)
    print(f"{label}: counts moved by rounding {moved}/{rows.shape[0]}, near-ties {near_total}, "
          f"mean count {counts.mean():.1f}", flush=True)
    return moved


def pool_landmarks(dkb, w, seed):
    q = synth.make_queries(w, seed, device="cuda")
    K, _ = synth.make_kv_pool(w, seed, device="cuda", q0=q)
    return q, dkb.build_landmarks(K, w.chunk)


@pytest.mark.parametrize("name,B,L,gamma,k_max,scale,reduce,dtype,union", [
    ("tiny", None, None, 0.5, 128, None, "mean", "f32", True),
    ("tiny", None, None, 0.9, 40, None, "mean", "f32", True),          # clamped at k_max
    ("llama8b_l32k", 2, 4096, 0.9, 128, 1.0, "mean", "f32", True),    # sharper scores
    ("llama8b_l32k", 2, 4096, 0.5, 64, None, "max", "f32", True),
    ("llama8b_l32k", 2, 4096, 0.7, 128, 1.0, "mean", "bf16", False),
    ("llama8b_l32k", 3, 40000, 0.8, 600, 1.0, "mean", "f32", True),   # C = 1250: a ragged second slab
    ("llama8b_l32k", 1, 32768, 1.0, 300, None, "mean", "f32", True),  # gamma 1: the top k_max
])
def test_coverage(dkb, name, B, L, gamma, k_max, scale, reduce, dtype, union):
    w = workload(name, B, L)
    print(f"case {name} B={B} L={L} gamma={gamma} k_max={k_max} scale={scale} {reduce} {dtype}", flush=True)
    q, lm = pool_landmarks(dkb, w, 11)
    if dtype == "bf16":
        lm = lm.to(torch.bfloat16)
    check_coverage(dkb, q, lm, gamma, k_max, w.scale if scale is None else scale, reduce, union,
                   label=f"{name} {gamma} {k_max}")


def test_coverage_one_query(dkb):
    w = workload("llama8b_l32k", 2, 4096, T=1)
    q, lm = pool_landmarks(dkb, w, 13)
    check_coverage(dkb, q, lm, 0.6, 128, 1.0, "mean", True, label="one query")


def test_coverage_equal_scores(dkb):
    # every score 0: masses 1/C exactly, the first ceil(gamma C) ids; exact counts
    B, T, Hq, Hkv, d, C = 2, 2, 8, 2, 128, 3000
    g = torch.Generator(device="cuda").manual_seed(14)
    q = synth.round_bf16(torch.randn(B, T, Hq, d, generator=g, device="cuda"))
    lm = torch.zeros(B, Hkv, C, d, device="cuda")
    idx, cnt, _, uid, mem, ucnt, ov = dkb.score_coverage(q, lm, 0.25, C, 0.1, union=True)
    torch.cuda.synchronize()
    assert torch.all(cnt == 750)
    assert torch.equal(idx[..., :750].cpu(), torch.arange(750, dtype=torch.int32).expand(B, Hkv, T, 750))
    assert torch.all(ucnt == 750) and torch.all(ov == 750) and torch.all(mem[..., :750] == 3)


def test_coverage_wide_rows(dkb):
    # 12000 chunks per row (16 per thread), random landmarks, both queries
    g = torch.Generator(device="cuda").manual_seed(15)
    q = synth.round_bf16(torch.randn(1, 2, 4, 64, generator=g, device="cuda"))
    lm = torch.randn(1, 2, 12000, 64, generator=g, device="cuda")
    check_coverage(dkb, q, lm, 0.5, 6000, 0.5, "mean", True, label="wide")


def test_coverage_full_128k_sampled(dkb):
    """b64_l128k's shape (C = 4096 chunks per (b, g)); oracle on sampled (b, g)."""
    w = WORKLOADS["b64_l128k"]
    q, lm = pool_landmarks(dkb, w, 16)
    idx, cnt, sc, uid, mem, ucnt, ov = dkb.score_coverage(q, lm, 0.9, 1024, 1.0, union=True)
    torch.cuda.synchronize()
    for b, g in ((0, 0), (31, 3), (63, 7)):
        qh = q[b:b + 1, :, g * w.G:(g + 1) * w.G]
        lmh = lm[b:b + 1, g:g + 1]
        i2, c2, _, u2, m2, uc2, o2 = dkb.score_coverage(qh.contiguous(), lmh.contiguous(), 0.9, 1024, 1.0,
                                                         union=True)
        torch.cuda.synchronize()
        # one (b, g) alone gives the same answer as inside the full batch
        assert torch.equal(i2[0, 0], idx[b, g]) and torch.equal(c2[0, 0], cnt[b, g])
        assert torch.equal(u2[0, 0], uid[b, g]) and torch.equal(uc2[0], ucnt[b:b + 1, g])
        check_coverage(dkb, qh.contiguous(), lmh.contiguous(), 0.9, 1024, 1.0, "mean", True,
                       label=f"b64_l128k ({b}, {g})")

