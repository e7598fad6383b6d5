"""Seeded synthetic inputs for the dual-query sparse KV retrieval decode step.

The same generated tensors feed both the HIP path and the CPU oracle.  This
module draws random numbers and lays them out; it contains none of the
method's arithmetic (no landmarks, scores, selection or attention).

Recipe (one layer):

* K, V ~ N(0, 1), drawn in fp32 and rounded to bf16 with round-to-nearest-even
  (or kept in fp32 for fp32 workloads).
* Real queries q_real ~ N(0, 1); speculative queries q_spec = q_real + sigma * N(0, 1)
  with sigma = 0.1.  Both are rounded to bf16 values and stored as fp32, so any
  consumer sees exactly representable values.
* Heavy hitters (bf16 workloads): for each (request, KV head), floor(0.01 * L)
  distinct positions are drawn uniformly and their keys get alpha * z added
  before rounding, where z is the unit vector of the mean real query of the
  KV head's query group (layer 0, step 0) and alpha = 4 * sqrt(d), about four
  times the norm of an N(0, 1) key.
* Host-pool query dynamics: q_real(step + 1) = q_spec(step) + 0.05 * N(0, 1).
* Token-level latent workloads: indexer keys and latent rows ~ N(0, 1) in
  bf16 (no heavy hitters); indexer queries and attention queries follow the
  real / speculative rule above.

Sub-streams are keyed by (seed, purpose, index) so that any slice can be
regenerated on its own.  Values differ between devices (torch's CPU and GPU
generators are different algorithms); the recipe is the same.
"""
from __future__ import annotations

import hashlib
import math

import torch

from .workloads import MlaWorkload, Workload


def sub_seed(base: int, *tags) -> int:
    h = hashlib.sha256(repr((int(base),) + tuple(tags)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def round_bf16(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32."""
    return x.to(torch.bfloat16).to(torch.float32)


def make_queries(w: Workload, seed: int, layer: int = 0, device="cpu",
                 sigma: float | None = None) -> torch.Tensor:
    """q [B, T, Hq, d] fp32 holding bf16 values; t=0 real, t=1 speculative."""
    sigma = w.sigma_spec if sigma is None else sigma
    q_real = torch.randn(w.B, w.Hq, w.d, generator=_gen(device, sub_seed(seed, "q_real", layer)),
                         device=device)
    noise = torch.randn(w.B, w.Hq, w.d, generator=_gen(device, sub_seed(seed, "q_spec", layer)),
                        device=device)
    q_spec = q_real + sigma * noise
    q = torch.stack([round_bf16(q_real), round_bf16(q_spec)], dim=1)
    return q[:, : w.T].contiguous()


def make_query_sequence(w: Workload, seed: int, steps: int, layer: int = 0, device="cpu",
                        drift: float = 0.05, sigma: float | None = None):
    """Queries for consecutive decode steps of the host-pool workload.

    Step 0 is ``make_queries``; afterwards the next real query is the previous
    speculative query plus drift * N(0, 1), and the new speculative query is the
    new real query plus sigma * N(0, 1).
    """
    sigma = w.sigma_spec if sigma is None else sigma
    out = [make_queries(w, seed, layer, device, sigma)]
    for s in range(1, steps):
        prev_spec = out[-1][:, min(1, w.T - 1)]
        n1 = torch.randn(w.B, w.Hq, w.d, generator=_gen(device, sub_seed(seed, "q_drift", layer, s)),
                         device=device)
        n2 = torch.randn(w.B, w.Hq, w.d, generator=_gen(device, sub_seed(seed, "q_spec", layer, s)),
                         device=device)
        q_real = prev_spec + drift * n1
        q_spec = q_real + sigma * n2
        q = torch.stack([round_bf16(q_real), round_bf16(q_spec)], dim=1)[:, : w.T]
        out.append(q.contiguous())
    return out


def heavy_hitter_directions(w: Workload, q0: torch.Tensor) -> torch.Tensor:
    """Unit vector of each KV head's mean real query, [B, Hkv, d] fp32."""
    qg = q0[:, 0].reshape(w.B, w.Hkv, w.G, w.d).mean(dim=2)
    return qg / qg.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def fill_kv_slice(w: Workload, seed: int, b: int, device, zhat_b: torch.Tensor | None):
    """Generate K[b], V[b] ([Hkv, L, d] fp32 values before the dtype cast)."""
    Kb = torch.randn(w.Hkv, w.L, w.d, generator=_gen(device, sub_seed(seed, "K", b)), device=device)
    if w.heavy_hitters and zhat_b is not None:
        n_hh = int(math.floor(0.01 * w.L))
        alpha = 4.0 * math.sqrt(w.d)
        gp = _gen(device, sub_seed(seed, "hh_pos", b))
        for g in range(w.Hkv):
            pos = torch.randperm(w.L, generator=gp, device=device)[:n_hh]
            Kb[g, pos] += alpha * zhat_b[g]
    Vb = torch.randn(w.Hkv, w.L, w.d, generator=_gen(device, sub_seed(seed, "V", b)), device=device)
    return Kb, Vb


def kv_torch_dtype(w: Workload):
    return torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32


def make_kv_pool(w: Workload, seed: int, device="cpu", q0: torch.Tensor | None = None,
                 out_device=None, pin_memory: bool = False):
    """K, V pools [B, Hkv, L, d] in the workload's dtype.

    ``q0`` is the layer-0 query tensor used for the heavy-hitter direction (made
    with ``make_queries(w, seed, 0)`` if omitted).  Generation runs on ``device``;
    the pools are stored on ``out_device`` (default: ``device``), optionally in
    pinned host memory.
    """
    out_device = device if out_device is None else out_device
    dt = kv_torch_dtype(w)
    if w.heavy_hitters:
        if q0 is None:
            q0 = make_queries(w, seed, 0, device)
        zhat = heavy_hitter_directions(w, q0.to(device))
    else:
        zhat = None
    shape = (w.B, w.Hkv, w.L, w.d)
    K = torch.empty(shape, dtype=dt, device=out_device, pin_memory=pin_memory)
    V = torch.empty(shape, dtype=dt, device=out_device, pin_memory=pin_memory)
    for b in range(w.B):
        Kb, Vb = fill_kv_slice(w, seed, b, device, None if zhat is None else zhat[b])
        K[b].copy_(Kb.to(dt))
        V[b].copy_(Vb.to(dt))
        del Kb, Vb
    return K, V


def to_numpy_f64(x: torch.Tensor):
    """Exact fp64 copy of an fp32 or bf16 tensor, through its bit pattern for bf16."""
    import numpy as np
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        bits = x.view(torch.int16).numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.numpy().astype(np.float64)


def _real_spec(shape, seed: int, tag: str, layer: int, device, sigma: float) -> torch.Tensor:
    """[B, 2, ...] fp32 holding bf16 values: t=0 real ~ N(0, 1), t=1 real + sigma * N(0, 1)."""
    real = torch.randn(shape, generator=_gen(device, sub_seed(seed, tag + "_real", layer)), device=device)
    noise = torch.randn(shape, generator=_gen(device, sub_seed(seed, tag + "_spec", layer)), device=device)
    return torch.stack([round_bf16(real), round_bf16(real + sigma * noise)], dim=1)


def make_mla_queries(w: MlaWorkload, seed: int, layer: int = 0, device="cpu"):
    """Indexer queries qi [B, T, Hi, di] and attention queries q [B, T, Hq, dk], fp32 bf16 values."""
    qi = _real_spec((w.B, w.Hi, w.di), seed, "qi", layer, device, w.sigma_spec)[:, : w.T]
    q = _real_spec((w.B, w.Hq, w.dk), seed, "qa", layer, device, w.sigma_spec)[:, : w.T]
    return qi.contiguous(), q.contiguous()


def fill_mla_slice(w: MlaWorkload, seed: int, b: int, device):
    """Indexer keys [L, di] and latent rows [L, dk] of request b, fp32 values before the bf16 cast."""
    Kidx = torch.randn(w.L, w.di, generator=_gen(device, sub_seed(seed, "Kidx", b)), device=device)
    lat = torch.randn(w.L, w.dk, generator=_gen(device, sub_seed(seed, "latent", b)), device=device)
    return Kidx, lat


def make_mla_pools(w: MlaWorkload, seed: int, device="cpu"):
    """Indexer keys [B, 1, L, di] and latent cache [B, 1, L, dk], both bf16."""
    Kidx = torch.empty((w.B, 1, w.L, w.di), dtype=torch.bfloat16, device=device)
    lat = torch.empty((w.B, 1, w.L, w.dk), dtype=torch.bfloat16, device=device)
    for b in range(w.B):
        kb, lb = fill_mla_slice(w, seed, b, device)
        Kidx[b, 0].copy_(kb.to(torch.bfloat16))
        lat[b, 0].copy_(lb.to(torch.bfloat16))
        del kb, lb
    return Kidx, lat
