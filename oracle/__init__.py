"""CPU reference for the dual-query sparse KV retrieval decode step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the
benchmark's CPU-baseline leg, never by the library's compute path.
"""
from .dualkv_oracle import (  # noqa: F401
    bf16_bits_to_f64, chunk_landmarks, chunk_scores, topk_chunks, union_select,
    prediction_accuracy, sparse_attention, cache_plan, decode_step,
)
