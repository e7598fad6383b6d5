"""Workload shapes for one dual-query sparse KV retrieval decode step.

Each workload fixes the shapes of one decode step: B requests, T query tokens per
request (t=0 the real token, t=1 the speculative look-ahead token), Hq query heads
sharing Hkv KV heads (GQA group G = Hq / Hkv, query head h reads KV head h // G),
head dimension d, context length L split into C = L / chunk fixed-size chunks,
and k chunks kept per query.

The shapes stand in for the long-context decode workloads on the pages:
Llama-3-8B-style GQA (32 query heads over 8 KV heads of width 128, as used in the
DualDecoder evaluation, "6.1 Experiment Setup"), 32K-128K contexts, and sparse
budgets of 1024-2048 tokens (DualDecoder Table 1 and "6.4 Modular Study";
OasisKV summary, single-GPU results).  No dataset item is used anywhere: every
tensor is drawn from a seeded generator (see ``synth.py``).

This module holds shapes only.  It contains none of the method's arithmetic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    chunk: int
    k: int
    T: int = 2
    layers: int = 1
    kv_dtype: str = "bf16"          # "bf16" or "f32"
    heavy_hitters: bool = True      # 1 % of keys pushed toward the query direction
    sigma_spec: float = 0.1         # spec query = real query + sigma * N(0, 1)
    host_pool: bool = False         # KV pool in pinned host memory (hot cache in HBM)
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def C(self) -> int:
        return self.L // self.chunk

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.kv_dtype == "bf16" else 4

    def pool_bytes(self) -> int:
        """K plus V pool bytes for one layer: B * L * 2 * Hkv * d * s.

        This is the per-layer form of the KV footprint equation in the OasisKV
        summary (Eq. 1, M_KV = B * L * N_layer * 2 * N_kv * d_h * s).
        """
        return self.B * self.L * 2 * self.Hkv * self.d * self.elem_bytes

    def landmark_bytes(self) -> int:
        """fp32 landmark table bytes for one layer: B * Hkv * C * d * 4."""
        return self.B * self.Hkv * self.C * self.d * 4

    def chunk_kv_bytes(self) -> int:
        """Bytes of one chunk of K plus V for one (request, KV head)."""
        return 2 * self.chunk * self.d * self.elem_bytes

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny correctness case: fp32 K/V, no heavy hitters.
    "tiny": Workload(
        name="tiny", B=1, Hq=4, Hkv=1, d=64, L=2048, chunk=16, k=8,
        kv_dtype="f32", heavy_hitters=False,
        description="B=1 Hq=4 Hkv=1 d=64 L=2048 chunk=16 (C=128) k=8 T=2, fp32 K/V"),
    # One Llama-3-8B-shaped layer at 32K context.
    "llama8b_l32k": Workload(
        name="llama8b_l32k", B=16, Hq=32, Hkv=8, d=128, L=32768, chunk=32, k=64,
        description="B=16 Hq=32 Hkv=8 d=128 L=32768 chunk=32 (C=1024) k=64 T=2, bf16 K/V"),
    # 128K decode with the KV pool resident in HBM, 32 layers in sequence.
    "b64_l128k": Workload(
        name="b64_l128k", B=64, Hq=32, Hkv=8, d=128, L=131072, chunk=32, k=64, layers=32,
        description="B=64 Hq=32 Hkv=8 d=128 L=131072 chunk=32 (C=4096) k=64 T=2, "
                    "bf16 K/V resident in HBM, 32 layers"),
    # 128K decode with the KV pool in pinned host memory and an HBM hot cache.
    "host_b32_l128k": Workload(
        name="host_b32_l128k", B=32, Hq=32, Hkv=8, d=128, L=131072, chunk=32, k=64, layers=32,
        host_pool=True,
        description="B=32 Hq=32 Hkv=8 d=128 L=131072 chunk=32 (C=4096) k=64 T=2, "
                    "bf16 K/V in pinned host memory, HBM hot cache of the previous union"),
}


@dataclass(frozen=True)
class MlaWorkload:
    """Token-level selection over one latent KV head (multi-head latent attention).

    Adaptive DHiSparse, Figure 2 and Table 3: an indexer picks k token positions
    per query (2,048 per selecting layer for the GLM model on the pages), and
    attention reads those rows of a latent cache shared by every query head.
    Each token has an indexer key of width di and a latent row of width
    dk = d_c + d_r (content part, position part); the value is the first
    dv = d_c columns of the latent row.  Hq attention heads and Hi indexer heads
    per query token, T query tokens per request.
    """
    name: str
    B: int
    L: int
    k: int
    Hq: int = 128
    d_c: int = 512
    d_r: int = 64
    Hi: int = 4
    di: int = 128
    T: int = 2
    layers: int = 1
    sigma_spec: float = 0.1
    description: str = ""

    @property
    def dk(self) -> int:
        return self.d_c + self.d_r

    @property
    def dv(self) -> int:
        return self.d_c

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)

    @property
    def index_scale(self) -> float:
        return 1.0 / math.sqrt(self.di)

    def index_key_bytes(self) -> int:
        """bf16 indexer keys read by one scoring pass: B * L * di * 2."""
        return self.B * self.L * self.di * 2

    def latent_row_bytes(self) -> int:
        return self.dk * 2

    def with_(self, **kw) -> "MlaWorkload":
        return replace(self, **kw)


MLA_WORKLOADS = {
    # The full shape: 32 requests at 128K context, 2,048 tokens per query.
    "mla_b32_l128k": MlaWorkload(
        name="mla_b32_l128k", B=32, L=131072, k=2048,
        description="B=32 Hq=128 on one latent head (dk 576 = 512 + 64, dv 512), L=131072, "
                    "indexer 4 heads x 128 (bf16 keys), token top-k=2048, T=2"),
    # Test sizes with the same head layout.
    "mla_b2_l16k": MlaWorkload(
        name="mla_b2_l16k", B=2, L=16384, k=512,
        description="B=2 Hq=128 latent dk 576 / dv 512, L=16384, indexer 4 x 128, top-k=512, T=2"),
    "mla_b1_l2k": MlaWorkload(
        name="mla_b1_l2k", B=1, L=2048, k=96,
        description="B=1 Hq=128 latent dk 576 / dv 512, L=2048, indexer 4 x 128, top-k=96, T=2"),
}


def shrink(w: Workload, B: int | None = None, L: int | None = None,
           layers: int | None = None) -> Workload:
    """Same head layout and budget, fewer requests / shorter context (test sizes)."""
    return replace(w, name=w.name + "_small",
                   B=B if B is not None else w.B,
                   L=L if L is not None else w.L,
                   layers=layers if layers is not None else w.layers)
