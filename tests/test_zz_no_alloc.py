"""dk_sparse_decode_attn_noalloc (the library's fixed device scratch instead of a
caller workspace) against dk_sparse_decode_attn (a caller workspace) on the same
inputs: two calls in a row per kernel family, the second with a smaller input,
so a stale partial left in the shared scratch by the first call would show.

The two entry points run the same kernels on the same plan, so the outputs must
be identical; the test also holds them to the attention parity bar (1e-4 fp32,
2e-2 bf16) as a floor.
"""
import numpy as np
import pytest
import torch

from sparse_kv_retrieval_amd import synth
from sparse_kv_retrieval_amd.workloads import MLA_WORKLOADS, WORKLOADS, shrink

from parity_utils import ATOL, max_abs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dkb():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from sparse_kv_retrieval_amd import binding   # raises if libdualkv.so is missing
    return binding


def chunk_union(dkb, w, seed):
    """Seeded inputs and the library's own union of the two queries' top-k sets."""
    q = synth.make_queries(w, seed, device="cuda")
    K, V = synth.make_kv_pool(w, seed, device="cuda", q0=q)
    lm = dkb.build_landmarks(K, w.chunk)
    _, _, uid, mem, cnt, _ = dkb.score_topk_union(q, lm, w.k, w.scale)
    return q, K, V, uid, mem, cnt


def compare(a, b, tol, label):
    (oa, la), (ob, lb) = a, b
    torch.cuda.synchronize()
    e_out = max_abs(oa.cpu().numpy(), ob.cpu().numpy())
    e_lse = max_abs(la.cpu().numpy(), lb.cpu().numpy())
    print(f"{label}: max|out diff| {e_out:.3e}  max|lse diff| {e_lse:.3e}", flush=True)
    assert e_out <= tol and e_lse <= tol, label
    assert torch.equal(oa, ob), label
    assert torch.equal(la.nan_to_num(), lb.nan_to_num()), label


@pytest.mark.parametrize("family,cases", [
    # bf16 d = 128, G = 4, T = 2 (the fast kernel): 4 x 8 then 2 x 8 (b, g) pairs
    ("fast", [("llama8b_l32k", 4, 8192, {}), ("llama8b_l32k", 2, 4096, dict(k=32))]),
    # fp32 generic kernel, several (b, g), then one
    ("generic", [("tiny", 3, None, dict(Hq=8, Hkv=2)), ("tiny", 1, 1024, {})]),
])
def test_noalloc_matches_workspace_call(dkb, family, cases):
    for i, (name, B, L, kw) in enumerate(cases):
        w = shrink(WORKLOADS[name], B=B, L=L).with_(**kw)
        q, K, V, uid, mem, cnt = chunk_union(dkb, w, 50 + i)
        print(f"[{family} call {i}] B={w.B} Hkv={w.Hkv} L={w.L} k={w.k} "
              f"ws={dkb.attn_workspace_size(w.B, w.Hkv, w.T, w.Hq, w.d, w.T * w.k, w.chunk)}", flush=True)
        ref = dkb.sparse_decode_attn(q, K, V, uid, mem, cnt, w.chunk, w.scale)
        got = dkb.sparse_decode_attn_noalloc(q, K, V, uid, mem, cnt, w.chunk, w.scale)
        compare(got, ref, ATOL[w.kv_dtype], f"{family} call {i}")


def test_noalloc_latent_rows(dkb):
    """Latent attention (dk 576 / dv 512): two calls, the second with fewer requests
    and a shorter token list."""
    for i, (B, L, k) in enumerate([(2, 16384, 512), (1, 2048, 96)]):
        w = MLA_WORKLOADS["mla_b2_l16k"].with_(B=B, L=L, k=k)
        qi, q = synth.make_mla_queries(w, 60 + i, device="cuda")
        Kidx, lat = synth.make_mla_pools(w, 60 + i, device="cuda")
        _, _, uid, mem, cnt, _ = dkb.score_topk_union(qi, Kidx, w.k, w.index_scale)
        print(f"[latent call {i}] B={B} L={L} k={k} "
              f"ws={dkb.attn_workspace_size(B, 1, w.T, w.Hq, w.dv, w.T * w.k, 1)}", flush=True)
        ref = dkb.mla_decode_attn(q, lat, uid, mem, cnt, w.scale)
        got = dkb.sparse_decode_attn_noalloc(q, lat, lat[..., :w.dv], uid, mem, cnt, 1, w.scale,
                                             pool_blocks=lat.shape[2])
        compare(got, ref, ATOL["bf16"], f"latent call {i}")


def test_noalloc_rejects_oversized_scratch(dkb):
    """A shape whose plan needs more than the fixed scratch is refused before any launch."""
    import ctypes
    lib = dkb.lib
    fake = ctypes.c_void_p(0x1000)
    for B, N in [(2, 1 << 20), (8, 1 << 20), (64, 1 << 22)]:
        need = dkb.attn_workspace_size(B, 8, 2, 32, 128, N, 32)
        if need > (64 << 20):
            break
    else:
        pytest.skip("no candidate shape needs more than the fixed scratch")
    st = lib.dk_sparse_decode_attn_noalloc(fake, B, 2, 32, 8, fake, fake, dkb.DK_BF16,
                                           dkb.dk_strides(1 << 30, 1 << 27, 128), dkb.dk_strides(1 << 30, 1 << 27, 128),
                                           128, 128, 32, fake, fake, fake, N, 1 << 20, 0.088, fake, fake, None)
    assert st == dkb.DK_ERR_UNSUPPORTED
    assert "scratch" in lib.dk_last_error().decode()
