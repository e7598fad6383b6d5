"""The seeded input generator: shapes, determinism and the stated recipe."""
import math

import torch

from sparse_kv_retrieval_amd import synth
from sparse_kv_retrieval_amd.workloads import WORKLOADS, shrink


def test_queries_are_bf16_values_and_deterministic():
    w = shrink(WORKLOADS["llama8b_l32k"], B=2, L=1024)
    q = synth.make_queries(w, seed=3)
    assert q.shape == (2, 2, 32, 128) and q.dtype == torch.float32
    assert torch.equal(q, synth.round_bf16(q))
    assert torch.equal(q, synth.make_queries(w, seed=3))
    assert not torch.equal(q, synth.make_queries(w, seed=4))
    # the speculative query is the real one plus about 0.1 of noise
    diff = (q[:, 1] - q[:, 0]).std().item()
    assert 0.08 < diff < 0.12


def test_kv_pool_recipe():
    w = shrink(WORKLOADS["llama8b_l32k"], B=2, L=2048)
    q0 = synth.make_queries(w, seed=5)
    K, V = synth.make_kv_pool(w, seed=5, q0=q0)
    assert K.shape == V.shape == (2, 8, 2048, 128) and K.dtype == torch.bfloat16
    assert K.nbytes + V.nbytes == w.pool_bytes()
    # heavy hitters: floor(0.01 L) keys per (request, KV head) carry alpha * z
    zhat = synth.heavy_hitter_directions(w, q0)
    proj = torch.einsum("bgld,bgd->bgl", K.float(), zhat)
    alpha = 4 * math.sqrt(128)
    n_hh = (proj > alpha / 2).sum(dim=-1)
    assert torch.all((n_hh >= 20) & (n_hh <= 22))   # 20 planted, about 0 by chance
    K2, V2 = synth.make_kv_pool(w, seed=5, q0=q0)
    assert torch.equal(K, K2) and torch.equal(V, V2)


def test_tiny_is_fp32_without_heavy_hitters():
    w = WORKLOADS["tiny"]
    K, V = synth.make_kv_pool(w, seed=0)
    assert K.dtype == torch.float32 and K.shape == (1, 1, 2048, 64)
    assert abs(K.float().mean().item()) < 0.02 and abs(K.float().std().item() - 1) < 0.02


def test_query_sequence_drift():
    w = shrink(WORKLOADS["host_b32_l128k"], B=2, L=1024)
    seq = synth.make_query_sequence(w, seed=1, steps=3)
    assert len(seq) == 3
    # next real query = previous speculative query + 0.05 noise
    d = (seq[1][:, 0] - seq[0][:, 1]).std().item()
    assert 0.04 < d < 0.06


def test_bf16_to_f64_is_exact():
    x = torch.randn(1000).to(torch.bfloat16)
    a = synth.to_numpy_f64(x)
    assert (a == x.float().numpy().astype("float64")).all()


def test_mla_inputs_shapes_values_and_slices():
    from sparse_kv_retrieval_amd.workloads import MLA_WORKLOADS
    w = MLA_WORKLOADS["mla_b1_l2k"].with_(B=2, L=256)
    qi, q = synth.make_mla_queries(w, 3)
    assert qi.shape == (2, 2, w.Hi, w.di) and q.shape == (2, 2, w.Hq, w.dk)
    for x in (qi, q):
        assert x.dtype == torch.float32
        assert torch.equal(x, x.to(torch.bfloat16).to(torch.float32))      # bf16 values
    # the speculative query is the real one plus a small perturbation
    d = (q[:, 1] - q[:, 0]).std().item()
    assert 0.05 < d < 0.2
    Kidx, lat = synth.make_mla_pools(w, 3)
    assert Kidx.shape == (2, 1, w.L, w.di) and lat.shape == (2, 1, w.L, w.dk)
    assert Kidx.dtype == torch.bfloat16 and lat.dtype == torch.bfloat16
    kb, lb = synth.fill_mla_slice(w, 3, 1, "cpu")
    assert torch.equal(Kidx[1, 0], kb.to(torch.bfloat16)) and torch.equal(lat[1, 0], lb.to(torch.bfloat16))
    assert abs(lat.float().std().item() - 1.0) < 0.05
