"""Decode steps over a KV pool held in pinned host memory, with an HBM hot cache.

DualDecoder (arXiv 2607.26475), "4.1" and "5.4": the index of the next step is
predicted by the speculative token, so the chunks it needs can be fetched from
host memory while the GPU works on something else; Adaptive DHiSparse,
Figure 2: a per-head hot cache in HBM, a resolver that copies only the missed
rows from host DRAM, and attention that reads the hot cache afterwards.

Per layer the hot cache holds exactly the previous step's union of the two
queries' chunk sets (T*k slots per (b, g)).  With buffers="ping-pong" the
layers share max(2, lookahead) such buffers instead (layer l uses buffer
l mod that count; DualDecoder "5.3", the two-layer buffer of Figure 9(a)):
HBM holds two layers' selected KV instead of every layer's, and since a buffer
last held another layer's chunks, every chunk of a layer's union is copied at
every step.  One step, per layer l:

  compute stream : dk_score_topk(l), dk_union_select(l, plan)  -> misses of l
  copy stream    : dk_gather_kv(l)  host pool -> free slots of l's hot cache
  compute stream : dk_sparse_decode_attn(l) over l's hot cache, after gather(l)

Layer-aware schedule (DualDecoder "5.3", Figure 9(a)): the selection and
transfer for layer l + lookahead are issued right after the attention of layer
l, so the copy stream moves one layer's misses while the compute stream scores
later layers and attends earlier ones.  The default lookahead of 2 is the pages'
schedule.  With the synthetic per-layer queries used here a layer's query does
not depend on the previous layer's output; in a model it would, and the
transfers would overlap the layer's other work instead.  Two source kinds are
offered:

  "mapped" : the gather kernel reads the pinned pool through its device
             mapping; the miss lists never leave the GPU (no host sync);
  "copy"   : the miss lists are copied to pinned host buffers, the host waits
             for them and issues one hipMemcpyAsync per run of chunks.

This module only orders library calls on streams; every step runs in libdualkv.
"""
from __future__ import annotations

import torch

from . import binding as dkb


def buffer_layout(layers, lookahead, buffers):
    """(buffer count, buffer of each layer, whether buffers change layers).

    "per-layer": one buffer per layer, so residency carries over to the next step.
    "ping-pong": max(2, lookahead) buffers (at most one per layer), layer l in
    buffer l mod count.  The refill for layer l + count is queued behind layer l's
    attention in both schedules of HostPoolDecoder.step, so it never overwrites
    rows still being read; two buffers are the least the "copy" schedule needs,
    since it queues layer l + 1's selection before layer l's attention."""
    if buffers not in ("per-layer", "ping-pong"):
        raise ValueError("buffers must be 'per-layer' or 'ping-pong'")
    if layers < 1 or lookahead < 1:
        raise ValueError("layers and lookahead must be >= 1")
    nbuf = layers if buffers == "per-layer" else min(layers, max(2, lookahead))
    return nbuf, [l % nbuf for l in range(layers)], nbuf < layers


class HostPoolDecoder:
    def __init__(self, K_host, V_host, lm, shadow, *, T, Hq, k, scale, layers, mode="mapped",
                 device="cuda", reduce=dkb.DK_REDUCE_MEAN, lookahead=2, buffers="per-layer"):
        if mode not in ("mapped", "copy"):
            raise ValueError("mode must be 'mapped' or 'copy'")
        if K_host.is_cuda or not (K_host.is_pinned() and V_host.is_pinned()):
            raise ValueError("the KV pool must be in pinned host memory")
        B, Hkv, L, d = K_host.shape
        C = lm.shape[2]
        chunk = L // C
        self.B, self.T, self.Hq, self.Hkv, self.d, self.C, self.chunk, self.k = B, T, Hq, Hkv, d, C, chunk, k
        self.scale, self.layers, self.mode, self.reduce = scale, layers, mode, reduce
        if lookahead < 1:
            raise ValueError("lookahead must be >= 1")
        self.lookahead = lookahead
        self.K_host, self.V_host, self.lm, self.shadow = K_host, V_host, lm, shadow
        self.slots = T * k
        n = T * k
        self.buffers = buffers
        self.nbuf, self.buf, self.shared = buffer_layout(layers, lookahead, buffers)
        i32 = dict(dtype=torch.int32, device=device)
        cache_shape = (self.nbuf, B, Hkv, self.slots * chunk, d)
        self.Kc = torch.zeros(cache_shape, dtype=K_host.dtype, device=device)
        self.Vc = torch.zeros(cache_shape, dtype=V_host.dtype, device=device)
        self.plans = [dkb.CachePlan.empty(B, Hkv, T, k, self.slots, device) for _ in range(layers)]
        self.topk_idx = torch.empty(layers, B, Hkv, T, k, **i32)
        self.union_ids = torch.empty(layers, B, Hkv, n, **i32)
        self.member = torch.empty(layers, B, Hkv, n, dtype=torch.uint8, device=device)
        self.count = torch.empty(layers, B, Hkv, **i32)
        self.overlap = torch.empty(layers, B, Hkv, **i32)
        self.out = torch.empty(layers, B, T, Hq, d, dtype=torch.float32, device=device)
        self.lse = torch.empty(layers, B, T, Hq, dtype=torch.float32, device=device)
        ws = dkb.score_topk_workspace_size(B, Hkv, T, C, k, shadow is not None)
        self.ws_topk = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        wa = dkb.attn_workspace_size(B, Hkv, T, Hq, d, n, chunk)
        self.ws_attn = torch.empty(max(wa, 1), dtype=torch.uint8, device=device)
        self.copy_stream = torch.cuda.Stream(device=device)
        self.ev_union = [torch.cuda.Event() for _ in range(layers)]
        self.ev_gather = [torch.cuda.Event() for _ in range(layers)]
        if mode == "copy":
            pin = dict(dtype=torch.int32, pin_memory=True)
            self.h_miss_chunk = torch.empty(layers, B, Hkv, n, **pin)
            self.h_miss_slot = torch.empty(layers, B, Hkv, n, **pin)
            self.h_miss_count = torch.empty(layers, B, Hkv, **pin)

    def reset(self):
        """Empty every hot cache (the next step is a cold step)."""
        for p in self.plans:
            p.resident.fill_(-1)

    # ---- the three stages of one layer ---------------------------------
    def _select(self, l, q, timer):
        cs = torch.cuda.current_stream()
        if timer:
            timer.begin("select", l, cs)
        if self.shared:
            self.plans[l].resident.fill_(-1)       # the buffer holds another layer's chunks
        dkb.score_topk(q, self.lm, self.k, self.scale, self.reduce, self.topk_idx[l], None, self.ws_topk,
                       shadow=self.shadow)
        dkb.union_select(self.topk_idx[l], self.C, self.union_ids[l], self.member[l], self.count[l],
                         self.overlap[l], plan=self.plans[l])
        if self.mode == "copy":
            p = self.plans[l]
            self.h_miss_chunk[l].copy_(p.miss_chunk, non_blocking=True)
            self.h_miss_slot[l].copy_(p.miss_slot, non_blocking=True)
            self.h_miss_count[l].copy_(p.miss_count, non_blocking=True)
        if timer:
            timer.end("select", l, cs)
        self.ev_union[l].record(cs)

    def _gather(self, l, timer):
        cps = self.copy_stream
        p = self.plans[l]
        if self.mode == "copy":
            self.ev_union[l].synchronize()          # the host reads the miss lists
        cps.wait_event(self.ev_union[l])
        if timer:
            timer.begin("gather", l, cps)
        if self.mode == "mapped":
            dkb.gather_kv(self.K_host, self.V_host, p.miss_chunk, p.miss_count, self.chunk, self.Kc[self.buf[l]],
                          self.Vc[self.buf[l]], dst_slot=p.miss_slot, stream=cps)
        else:
            dkb.gather_kv(self.K_host, self.V_host, self.h_miss_chunk[l], self.h_miss_count[l], self.chunk,
                          self.Kc[self.buf[l]], self.Vc[self.buf[l]], dst_slot=self.h_miss_slot[l], stream=cps)
        if timer:
            timer.end("gather", l, cps)
        self.ev_gather[l].record(cps)

    def _attend(self, l, q, timer):
        cs = torch.cuda.current_stream()
        cs.wait_event(self.ev_gather[l])
        if timer:
            timer.begin("attn", l, cs)
        dkb.sparse_decode_attn(q, self.Kc[self.buf[l]], self.Vc[self.buf[l]], self.plans[l].slot_of_union,
                               self.member[l],
                               self.count[l], self.chunk, self.scale, pool_blocks=self.slots,
                               out=self.out[l], lse=self.lse[l], ws=self.ws_attn)
        if timer:
            timer.end("attn", l, cs)

    def step(self, qs, timer=None):
        """One decode step over every layer; qs[l] is layer l's [B, T, Hq, d] query."""
        L = self.layers
        if self.mode == "mapped":
            # compute: sel(0..a-1) | att(0) sel(a) | att(1) sel(a+1) | ... ; copy: gat(0) gat(1) ...
            a = min(self.lookahead, L)
            for l in range(a):
                self._select(l, qs[l], timer)
                self._gather(l, timer)
            for l in range(L):
                self._attend(l, qs[l], timer)
                if l + a < L:
                    self._select(l + a, qs[l + a], timer)
                    self._gather(l + a, timer)
        else:
            # the host must see layer l's lists before it issues l's copies, so the
            # selection of l+1 is queued first to keep the GPU busy meanwhile
            self._select(0, qs[0], timer)
            for l in range(L):
                if l + 1 < L:
                    self._select(l + 1, qs[l + 1], timer)
                self._gather(l, timer)
                self._attend(l, qs[l], timer)


class StageTimer:
    """HIP events around each stage of each layer of the recorded steps."""

    def __init__(self):
        self.pairs = {}

    def begin(self, stage, l, stream):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        self.pairs.setdefault(stage, []).append([e, None])

    def end(self, stage, l, stream):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        self.pairs[stage][-1][1] = e

    def total_ms(self, stage):
        return sum(a.elapsed_time(b) for a, b in self.pairs.get(stage, []))

    def count(self, stage):
        return len(self.pairs.get(stage, []))
