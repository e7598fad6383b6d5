"""GPU parity of token-level selection over one latent KV head.

The indexer (dk_score_topk / dk_score_topk_union with bf16 per-token keys) is
compared with the oracle's indexer_topk: token ids bit-exact except at counted
near-ties, the union bit-exact against the oracle's union of the GPU's own sets,
and the reported scores within a derived fp32 error bound.
"""
import numpy as np
import pytest
import torch

from oracle import dualkv_oracle as O
from sparse_kv_retrieval_amd import synth
from sparse_kv_retrieval_amd.workloads import MLA_WORKLOADS

from parity_utils import compare_topk

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def dkb():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a GPU")
    from sparse_kv_retrieval_amd import binding   # raises if libdualkv.so is missing
    return binding


def bf16_keys(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def check_index(dkb, qi, keys, k, scale, union=False, label=""):
    """GPU token-level selection against the oracle on the same values; returns near-tie count."""
    qh = qi.detach().cpu().numpy().astype(np.float64)
    kh = synth.to_numpy_f64(keys)
    if union:
        idx, sc, uid, mem, cnt, ov = dkb.score_topk_union(qi, keys, k, scale, want_scores=True)
    else:
        idx, sc = dkb.score_topk(qi, keys, k, scale)
    torch.cuda.synchronize()
    s_ref = O.chunk_scores(qh, kh, scale, "mean")
    idx_ref = O.indexer_topk(qh, kh, k, scale)
    gi = idx.cpu().numpy().astype(np.int64)
    rows_diff, near, hard = compare_topk(gi, idx_ref, s_ref)
    assert not hard, (label, hard[:5])
    # reported scores: the GPU's fp32 scores of its own ids, within the rounding of
    # the fp32 head mean (G terms) and of the d-term dot product
    B, T, Hq, d = qh.shape
    Hkv = kh.shape[1]
    G = Hq // Hkv
    s_sel = np.take_along_axis(s_ref, gi, axis=-1)
    qa = np.abs(qh).reshape(B, T, Hkv, G, d).mean(axis=3)
    mag = abs(scale) * np.einsum("btgd,bgcd->bgtc", qa, np.abs(kh))
    mag_sel = np.take_along_axis(mag, gi, axis=-1)
    err = np.abs(sc.cpu().numpy().astype(np.float64) - s_sel)
    assert np.all(err <= (G + d + 3) * U32 * mag_sel * 1.01 + 1e-30), (label, float(err.max()))
    if union:
        ru, rm, rc, ro = O.union_select(gi)
        np.testing.assert_array_equal(uid.cpu().numpy(), ru)
        np.testing.assert_array_equal(mem.cpu().numpy(), rm)
        np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
        np.testing.assert_array_equal(ov.cpu().numpy(), ro)
    return near


def mla_inputs(w, seed):
    qi, q = synth.make_mla_queries(w, seed, device="cuda")
    Kidx, lat = synth.make_mla_pools(w, seed, device="cuda")
    return qi, q, Kidx, lat


@pytest.mark.parametrize("name,kw", [
    ("mla_b1_l2k", {}),
    ("mla_b2_l16k", {}),
    ("mla_b1_l2k", dict(T=1)),
    ("mla_b1_l2k", dict(k=2048)),          # every token
    ("mla_b1_l2k", dict(L=3076, k=700)),   # tokens not a multiple of the scoring block
    ("mla_b1_l2k", dict(L=50004, k=700)),  # split selection: three slices, the last one short
    ("mla_b2_l16k", dict(L=65536, k=2048)),  # split selection: four slices per row
])
def test_index_topk(dkb, name, kw):
    w = MLA_WORKLOADS[name].with_(**kw)
    print(f"case {name} {kw}", flush=True)
    qi, _, Kidx, _ = mla_inputs(w, 31)
    check_index(dkb, qi, Kidx, w.k, w.index_scale, label=name)


@pytest.mark.parametrize("B,rows_per_block", [(128, 2048), (200, 4096)])
def test_index_topk_long_scoring_blocks(dkb, B, rows_per_block):
    """Many rows of 10000 tokens: the scoring kernel takes 2048- or 4096-token blocks
    (the longest that keep 512 blocks), and the last block of every row is short
    (10000 - 8192 = 1808 tokens)."""
    g = torch.Generator(device="cuda").manual_seed(12)
    qi = synth.round_bf16(torch.randn(B, 2, 4, 128, generator=g, device="cuda"))
    keys = bf16_keys(torch.randn(B, 1, 10000, 128, generator=g, device="cuda"))
    print(f"B={B}: {rows_per_block}-token scoring blocks", flush=True)
    check_index(dkb, qi, keys, 700, 1.0 / 128 ** 0.5, union=True, label=f"B={B}")


def test_index_topk_union(dkb):
    w = MLA_WORKLOADS["mla_b2_l16k"]
    qi, _, Kidx, _ = mla_inputs(w, 32)
    check_index(dkb, qi, Kidx, w.k, w.index_scale, union=True)


def test_index_topk_grouped_heads_d64(dkb):
    # two key heads, four indexer heads each, width 64
    g = torch.Generator(device="cuda").manual_seed(9)
    qi = synth.round_bf16(torch.randn(3, 2, 8, 64, generator=g, device="cuda"))
    keys = bf16_keys(torch.randn(3, 2, 4096, 64, generator=g, device="cuda"))
    check_index(dkb, qi, keys, 333, 0.125, union=True)


@pytest.mark.parametrize("kind,C", [("zeros", 8192), ("quantised", 8192), ("zeros", 40000), ("quantised", 40000)])
def test_index_topk_ties(dkb, kind, C):
    # equal scores over whole bins: the radix fallback and the position rule; at
    # C = 40000 the split selection flags the rows and falls back to one block per row
    g = torch.Generator(device="cuda").manual_seed(10)
    qi = synth.round_bf16(torch.randn(2, 2, 4, 128, generator=g, device="cuda"))
    if kind == "zeros":
        keys = torch.zeros(2, 1, C, 128, dtype=torch.bfloat16, device="cuda")
    else:
        # keys in {-1, 0, 1} on 2 dims: a handful of distinct scores, thousands each
        keys = torch.zeros(2, 1, C, 128, device="cuda")
        keys[..., :2] = torch.randint(-1, 2, (2, 1, C, 2), generator=g, device="cuda").float()
        keys = bf16_keys(keys)
    near = check_index(dkb, qi, keys, 3000, 0.1, union=True, label=kind)
    assert near == 0


def test_index_topk_full_size_sampled(dkb):
    """The full shape (B=32, 131072 tokens, top-2048), oracle on sampled requests."""
    w = MLA_WORKLOADS["mla_b32_l128k"]
    qi, _, Kidx, _ = mla_inputs(w, 1)
    idx, sc, uid, mem, cnt, ov = dkb.score_topk_union(qi, Kidx, w.k, w.index_scale, want_scores=True)
    torch.cuda.synchronize()
    near_total = 0
    for b in (0, 17, 31):
        qh = qi[b:b + 1].cpu().numpy().astype(np.float64)
        kh = synth.to_numpy_f64(Kidx[b:b + 1])
        s_ref = O.chunk_scores(qh, kh, w.index_scale, "mean")
        idx_ref = O.topk_chunks(s_ref, w.k)
        gi = idx[b:b + 1].cpu().numpy().astype(np.int64)
        rows_diff, near, hard = compare_topk(gi, idx_ref, s_ref)
        assert not hard, (b, hard[:5])
        near_total += near
        ru, rm, rc, ro = O.union_select(gi)
        np.testing.assert_array_equal(uid[b:b + 1].cpu().numpy(), ru)
        np.testing.assert_array_equal(mem[b:b + 1].cpu().numpy(), rm)
        np.testing.assert_array_equal(cnt[b:b + 1].cpu().numpy(), rc)
    print(f"near-ties over 3 sampled requests: {near_total}", flush=True)


# ----------------------------------------------------------------------------
# latent attention (matrix cores) over each query's own tokens
# ----------------------------------------------------------------------------

def to_dev(a, dtype=torch.int32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def check_mla_attention(dkb, w, q, lat, sel, label="", count_override=None):
    """GPU latent attention on the oracle's union of `sel` against the oracle."""
    ru, rm, rc, _ = O.union_select(sel)
    if count_override is not None:
        rc = count_override
    member = None if w.T == 1 else to_dev(rm, torch.uint8)
    out, lse = dkb.mla_decode_attn(q, lat, to_dev(ru), member, to_dev(rc), w.scale)
    torch.cuda.synchronize()
    qh = q.cpu().numpy().astype(np.float64)
    lh = synth.to_numpy_f64(lat)
    if count_override is None:
        ro, rl = O.mla_attention(qh, lh, sel, w.dv, w.scale)
    else:
        ro, rl = np.zeros(out.shape), np.full(lse.shape, -np.inf)
    from parity_utils import ATOL, max_abs
    eo, el = max_abs(out.cpu().numpy(), ro), max_abs(lse.cpu().numpy(), rl)
    print(f"{label}: max|out err| {eo:.3g}, max|lse err| {el:.3g}", flush=True)
    assert eo <= ATOL["bf16"] and el <= ATOL["bf16"], (label, eo, el)


@pytest.mark.parametrize("name,kw", [
    ("mla_b1_l2k", {}),                     # ranges merged, ragged last tile
    ("mla_b1_l2k", dict(k=24)),             # one range: direct output
    ("mla_b1_l2k", dict(T=1)),              # one query, no member bits
    ("mla_b2_l16k", {}),
    ("mla_b1_l2k", dict(Hq=64)),            # one 64-row group
])
def test_mla_attention(dkb, name, kw):
    w = MLA_WORKLOADS[name].with_(**kw)
    print(f"case {name} {kw}", flush=True)
    qi, q, Kidx, lat = mla_inputs(w, 41)
    sel = O.indexer_topk(qi.cpu().numpy().astype(np.float64), synth.to_numpy_f64(Kidx), w.k, w.index_scale)
    check_mla_attention(dkb, w, q, lat, sel, label=f"{name} {kw}")


def test_mla_attention_empty_selection(dkb):
    w = MLA_WORKLOADS["mla_b1_l2k"].with_(B=2)
    qi, q, Kidx, lat = mla_inputs(w, 42)
    sel = O.indexer_topk(qi.cpu().numpy().astype(np.float64), synth.to_numpy_f64(Kidx), w.k, w.index_scale)
    check_mla_attention(dkb, w, q, lat, sel, label="empty", count_override=np.zeros((2, 1), dtype=np.int64))


def test_mla_step_full_size_sampled(dkb):
    """Indexer + union + latent attention at the full shape (B=32, 131072 tokens,
    top-2048, 128 heads), in the bench's launch configuration; oracle on sampled requests."""
    w = MLA_WORKLOADS["mla_b32_l128k"]
    qi, q, Kidx, lat = mla_inputs(w, 2)
    idx, _, uid, mem, cnt, ov = dkb.score_topk_union(qi, Kidx, w.k, w.index_scale)
    out, lse = dkb.mla_decode_attn(q, lat, uid, mem, cnt, w.scale)
    torch.cuda.synchronize()
    from parity_utils import ATOL, max_abs
    for b in (0, 21, 31):
        gi = idx[b:b + 1].cpu().numpy().astype(np.int64)
        qh = q[b:b + 1].cpu().numpy().astype(np.float64)
        lh = synth.to_numpy_f64(lat[b:b + 1])
        ro, rl = O.mla_attention(qh, lh, gi, w.dv, w.scale)
        eo = max_abs(out[b:b + 1].cpu().numpy(), ro)
        el = max_abs(lse[b:b + 1].cpu().numpy(), rl)
        print(f"request {b}: max|out err| {eo:.3g}, max|lse err| {el:.3g}", flush=True)
        assert eo <= ATOL["bf16"] and el <= ATOL["bf16"], (b, eo, el)
