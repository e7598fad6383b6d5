"""libdualkv: dual-query sparse KV retrieval decode on MI355X (gfx950).

The compute path is the HIP library ``libdualkv.so`` built in-tree from
``csrc/``; ``binding`` wraps its C ABI for torch tensors and streams.  Importing
the package itself loads nothing: ``binding`` raises if the library is missing.
"""
__all__ = ["workloads", "synth"]
