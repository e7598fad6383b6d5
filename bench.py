"""Benchmark: dual-query sparse decode steps/s and selected-KV GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b64_l128k]

A step is one pass of the whole hot path over every layer of the workload: per
layer, chunk scores, top-k of both queries and their union in one call
(dk_score_topk_union), and attention of both queries over their own chunks,
read once per union chunk straight from the HBM pool (dk_sparse_decode_attn).
Landmarks (and their 8-bit shadow) are built once before timing: they are fixed
for the whole decode.
Inputs are seeded synthetic tensors resident in HBM before the timed region.

Prints one JSON line.  `value` comes from steps timed with nothing between the
library calls; a second pass of the same steps, with events around every call,
gives `kernels` (every call's measured duration and algorithmic bytes) and
`roofline` (the call that takes the most time per step).  `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload, one worker process per
host core.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, 8 TB/s
PCIE_PEAK_GBPS = 64.0    # PCIe 5.0 x16, one direction
METRIC = "dual-query sparse decode steps/s + selected-KV GB/s (% HBM peak), B=64 L=128K"
METRIC_HOST = "dual-query sparse decode steps/s, KV pool in pinned host memory, B=32 L=128K"
METRIC_MLA = "token-level dual-query sparse decode steps/s (one layer, 128 heads on one latent head), B=32 L=128K"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="b64_l128k")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle sample budget (0 disables the CPU baseline)")
    ap.add_argument("--flush-mb", type=int, default=None,
                    help="write this many MiB between timed steps, outside the timed intervals, so the "
                         "256 MB Infinity Cache does not serve a step's bytes from the step before "
                         "(default: 1024 for one-layer workloads, whose working set fits that cache; 0 otherwise)")
    ap.add_argument("--no-events", action="store_true",
                    help="skip the second pass that times every call with events")
    ap.add_argument("--two-calls", action="store_true",
                    help="time the step as score_topk_union + sparse_decode_attn instead of one dk_decode_step")
    ap.add_argument("--no-shadow", action="store_true",
                    help="score from the fp32 landmarks only (no 8-bit landmark shadow)")
    ap.add_argument("--host-copy", choices=("mapped", "copy"), default="mapped",
                    help="host-pool workloads: gather kernel over the mapped pool, or hipMemcpyAsync")
    ap.add_argument("--tail", type=int, default=0,
                    help="attend, besides the chunks, a per-request tail of up to this many rows "
                         "(lengths drawn in [tail/2, tail]) and the step's two fresh rows "
                         "(dk_sparse_decode_attn_tail)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the card's read ceilings (register loads and the attention's LDS-DMA ring, "
                         "contiguous and as random 8 KiB K/V chunk pairs) and the host-pool transfer paths")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB + 1 GiB device copy (dk_gather_kv over consecutive "
                         "chunks) three times: the known-size reference for HBM byte counters")
    ap.add_argument("--selection", choices=("landmark", "minmax", "coverage", "capped"), default="landmark",
                    help="chunk selection of the step: landmark top-k (default), top-k by min/max summary "
                         "bounds, coverage budgets, or landmark top-k plus a capped-eviction working-set plan")
    ap.add_argument("--gamma", type=float, default=0.9, help="coverage: fraction of the estimated mass")
    ap.add_argument("--k-max", type=int, default=None, help="coverage: most chunks per query (default 2k)")
    ap.add_argument("--cov-scale", type=float, default=0.5,
                    help="coverage: logit scale of the mass estimate (the synthetic keys' logits are flat at "
                         "1/sqrt(d))")
    ap.add_argument("--cap", type=int, default=8, help="capped: admissions per step and KV head")
    ap.add_argument("--slots", type=int, default=None, help="capped: working-set slots per (b, g) (default 4k)")
    ap.add_argument("--lookahead", type=int, default=2,
                    help="host-pool workloads: layers between a selection/transfer and its attention")
    ap.add_argument("--host-buffers", choices=("per-layer", "ping-pong"), default="per-layer",
                    help="host-pool workloads: a hot cache per layer (residency kept across steps) or "
                         "max(2, lookahead) buffers shared by the layers (every union chunk copied every step)")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "sparse_kv_retrieval_amd", "csrc")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, call):
    """HBM bytes per launch of `call` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE passes, each scaled by the same counter's reading
    for a plain copy of known size), or None when there is no summary for this
    workload or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = next((json.loads(line[5:]) for line in fh if line.startswith("json:")), None)
    c = (rec or {}).get("calls", {}).get(call)
    if not c or source_digest(c["sources"]) != c["digest"]:
        return None
    return c["bytes_per_launch"]


def near_tie_report(gpu_sel, ref_sel, scores):
    """Compare GPU and oracle top-k rows: a chunk in one set but not the other is
    a near-tie when its oracle score is within 1e-5 * max(|s_(k)|, rms(row)) of
    the k-th largest oracle score s_(k); any other difference is a mismatch."""
    import numpy as np
    rows = diff_rows = near = hard = 0
    for gi, oi, sc in zip(gpu_sel.reshape(-1, gpu_sel.shape[-1]), ref_sel.reshape(-1, ref_sel.shape[-1]),
                          scores.reshape(-1, scores.shape[-1])):
        rows += 1
        sym = set(gi.tolist()) ^ set(oi.tolist())
        if not sym:
            continue
        diff_rows += 1
        sk = sc[oi].min()
        tol = 1e-5 * max(abs(sk), float(np.sqrt(np.mean(sc ** 2))))
        for c in sym:
            if abs(sc[c] - sk) <= tol:
                near += 1
            else:
                hard += 1
    return rows, diff_rows, near, hard


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, unchanged, on every host core.  A pool of
# worker processes (one BLAS thread each) is forked before anything touches the
# GPU; each worker times the oracle on units of one sampled (request, KV head)
# of the same workload for the whole budget, so the workers run side by side
# and their rates add up.  Inputs reach the workers as raw bf16 bit patterns
# (or fp32) and are widened there, untimed.
# ---------------------------------------------------------------------------
MAX_CPU_WORKERS = 16      # the host share of one GPU on the boxes this runs on
_POOL = None


def cpu_pool_size():
    aff = len(os.sched_getaffinity(0))
    return max(1, min(aff, MAX_CPU_WORKERS)), aff


def start_cpu_pool():
    """Fork the oracle workers (call before the GPU is initialised)."""
    import multiprocessing as mp
    global _POOL
    n, _ = cpu_pool_size()
    _POOL = mp.get_context("fork").Pool(n)


def stop_cpu_pool():
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def raw_host(t):
    """A torch tensor as numpy: uint16 bit patterns for bf16, the values otherwise."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _widen(a):
    import numpy as np
    from oracle import dualkv_oracle as O
    return O.bf16_bits_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)


def run_cpu_pool(worker, tasks):
    """Run one task per worker; returns the results and the summed rate in units/s."""
    if _POOL is None:
        raise RuntimeError("the CPU worker pool was not started")
    res = _POOL.map(worker, tasks, chunksize=1)
    rate = sum(r["units"] / r["spent"] for r in res if r["spent"] > 0)
    return res, rate


def cpu_record(rate, units_per_step, res, what, slice_="(request, KV head)"):
    n, aff = cpu_pool_size()
    units = sum(r["units"] for r in res)
    spent = sum(r["spent"] for r in res)
    per_unit = spent / max(units, 1)
    return {"value": rate / units_per_step, "unit": "steps/s", "cores": len(res), "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cores": aff,
            "sample": f"{units} {what} on {len(res)} worker processes (one per core, one BLAS thread each; "
                      f"{spent:.1f} s of CPU time, {per_unit * 1e3:.1f} ms per unit), each worker on one sampled "
                      f"{slice_} for the whole budget; the summed rate scaled to {units_per_step} units per step"}


def _chunk_step_worker(task):
    """The oracle's chunk step (scores, top-k, union, attention) on one (b, g),
    layer after layer, for `budget` seconds; with the GPU's sets, the sampled
    selections are compared too."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import dualkv_oracle as O
    Kr, Vr, qs, gsel, chunk, k, scale, budget = task
    units, spent, layer = 0, 0.0, 0
    cmp = [0, 0, 0, 0]
    ov = [0, 0]
    with threadpool_limits(1):
        Kh, Vh = _widen(Kr)[None, None], _widen(Vr)[None, None]
        lm = O.chunk_landmarks(Kh, chunk)            # built once per prefill: not timed
        while spent < budget:
            li = layer % len(qs)
            qh = qs[li]
            t0 = time.perf_counter()
            s = O.chunk_scores(qh, lm, scale, "mean")
            sel = O.topk_chunks(s, k)
            O.union_select(sel)
            O.sparse_attention(qh, Kh, Vh, sel, chunk, scale)
            spent += time.perf_counter() - t0
            units += 1
            if gsel is not None and layer < len(qs):
                for i, x in enumerate(near_tie_report(gsel[li], sel, s)):
                    cmp[i] += x
                if sel.shape[2] == 2:
                    g_ = gsel[li]
                    ov[0] += len(set(g_[0, 0, 0].tolist()) & set(g_[0, 0, 1].tolist()))
                    ov[1] += len(set(sel[0, 0, 0].tolist()) & set(sel[0, 0, 1].tolist()))
            layer += 1
    return {"units": units, "spent": spent, "cmp": cmp, "ov": ov}


def cpu_baseline(w, qs_host, K, V, budget_s, seed, gpu_topk=None):
    """Time the fp64 CPU oracle on sampled (request, KV head, layer) units on every
    host core; with the GPU's top-k of every layer, also compare the sampled
    selections."""
    import numpy as np
    n, _ = cpu_pool_size()
    rng = np.random.default_rng(seed)
    flat = rng.choice(w.B * w.Hkv, size=min(n, w.B * w.Hkv), replace=False)
    tasks = []
    for f in flat:
        b, g = divmod(int(f), w.Hkv)
        qs = [q[b:b + 1, :, g * w.G:(g + 1) * w.G] for q in qs_host]
        gsel = None if gpu_topk is None else [t[b:b + 1, g:g + 1] for t in gpu_topk]
        tasks.append((raw_host(K[b, g]), raw_host(V[b, g]), qs, gsel, w.chunk, w.k, w.scale, budget_s))
    res, rate = run_cpu_pool(_chunk_step_worker, tasks)
    out = cpu_record(rate, w.B * w.Hkv * len(qs_host), res,
                     f"(request, KV head, layer) units of the {w.name} step (landmarks precomputed)")
    if gpu_topk is not None:
        cmp = [sum(r["cmp"][i] for r in res) for i in range(4)]
        out["selection_check"] = {"rows": cmp[0], "rows_differing": cmp[1], "near_tie_chunks": cmp[2],
                                  "mismatched_chunks": cmp[3], "overlap_gpu": sum(r["ov"][0] for r in res),
                                  "overlap_oracle": sum(r["ov"][1] for r in res)}
    return out


def hbm_copy_gbps(torch, dkb, reps=5):
    """Plain device copy rate (1 GiB read + 1 GiB written per launch) through
    dk_gather_kv over consecutive chunks; bytes moved (read + written) per second."""
    rows, d, chunk = 1 << 21, 128, 32
    C = rows // chunk
    src = [torch.ones(1, 1, rows, d, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    dst = [torch.empty_like(src[0]) for _ in range(2)]
    ids = torch.arange(C, dtype=torch.int32, device="cuda").reshape(1, 1, C)
    dkb.gather_kv(src[0], src[1], ids, None, chunk, dst[0], dst[1])
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dkb.gather_kv(src[0], src[1], ids, None, chunk, dst[0], dst[1])
        b.record()
        b.synchronize()
        best = max(best, 4 * src[0].nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return best


def h2d_peak_gbps(torch, nbytes=1 << 28, reps=5):
    """Contiguous pinned-host -> HBM copy rate (the link's practical peak)."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        b.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    return best


def bench_host_pool(args, w):
    """Decode steps with the KV pool in pinned host memory and a hot cache per layer."""
    import numpy as np
    import torch

    from sparse_kv_retrieval_amd import binding as dkb
    from sparse_kv_retrieval_amd import synth
    from sparse_kv_retrieval_amd.host_pool import HostPoolDecoder, StageTimer

    dev = "cuda"
    # one cold step, warm-up, the timed steps, then (with events) the same number of
    # steps again with events around every stage
    timed0 = 1 + args.warmup
    total = timed0 + args.steps * (1 if args.no_events else 2)
    t0 = time.time()
    qseq = [synth.make_query_sequence(w, args.seed, total, layer=l, device=dev) for l in range(w.layers)]
    K, V = synth.make_kv_pool(w, args.seed, device=dev, q0=qseq[0][0])
    lm = dkb.build_landmarks(K, w.chunk)                # prefill: built before the pool moves out
    shadow = None if args.no_shadow else dkb.build_landmark_shadow(lm)
    Kh = torch.empty(K.shape, dtype=K.dtype, pin_memory=True)
    Vh = torch.empty(V.shape, dtype=V.dtype, pin_memory=True)
    Kh.copy_(K)
    Vh.copy_(V)
    del K, V
    torch.cuda.empty_cache()
    dec = HostPoolDecoder(Kh, Vh, lm, shadow, T=w.T, Hq=w.Hq, k=w.k, scale=w.scale, layers=w.layers,
                          mode=args.host_copy, lookahead=args.lookahead, buffers=args.host_buffers)
    link_gbps = h2d_peak_gbps(torch)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s: host pool {2 * Kh.nbytes / 1e9:.2f} GB pinned, "
          f"hot caches {2 * dec.Kc.nbytes / 1e9:.2f} GB, contiguous H2D {link_gbps:.1f} GB/s",
          file=sys.stderr, flush=True)

    def qs_at(s):
        return [qseq[l][s] for l in range(w.layers)]

    for s in range(timed0):
        dec.step(qs_at(s))
    torch.cuda.synchronize()
    # headline: event-free steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(timed0, timed0 + args.steps):
        dec.step(qs_at(s))
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    # stage durations: the following steps with events around every stage
    timer = None if args.no_events else StageTimer()
    if timer:
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start.record()
        for s in range(timed0 + args.steps, total):
            dec.step(qs_at(s), timer)
        t_end.record()
        torch.cuda.synchronize()
        timer_ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # Statistics from a deterministic replay of the same steps (untimed).
    dec.reset()
    prev_spec = [None] * w.layers
    hits = unions = misses = overlap_sum = temporal_hits = 0
    misses_timer = 0      # misses of the stage-timed steps (their copies give the PCIe rate)
    n_units = 0
    for s in range(total):
        dec.step(qs_at(s))
        torch.cuda.synchronize()
        for l in range(w.layers):
            idx = dec.topk_idx[l]
            if s >= timed0 + args.steps:
                misses_timer += int(dec.plans[l].miss_count.sum())
            if timed0 <= s < timed0 + args.steps:
                p = dec.plans[l]
                hits += int(p.hit_count.sum())
                misses += int(p.miss_count.sum())
                unions += int(dec.count[l].sum())
                overlap_sum += int(dec.overlap[l].sum())
                real = idx[:, :, 0]
                temporal_hits += int((real.unsqueeze(-1) == prev_spec[l].unsqueeze(-2)).any(-1).sum())
                n_units += w.B * w.Hkv
            prev_spec[l] = idx[:, :, w.T - 1].clone()
    chunk_bytes = w.chunk_kv_bytes()
    miss_bytes_step = misses * chunk_bytes / args.steps
    union_bytes_step = unions * chunk_bytes / args.steps
    out = {
        "metric": METRIC_HOST, "value": round(1000.0 / ms_per_step, 3), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "chunk": w.chunk, "k": w.k, "T": w.T, "layers": w.layers, "seed": args.seed,
                   "landmark_shadow": shadow is not None, "host_copy": args.host_copy,
                   "hot_cache_slots": dec.slots, "drift": 0.05, "lookahead": dec.lookahead,
                   "host_buffers": dec.buffers, "hot_cache_GB": round(2 * dec.Kc.nbytes / 1e9, 2)},
        "hit_rate": round(hits / max(unions, 1), 5),
        "misses_per_bg_layer": round(misses / max(n_units, 1), 3),
        "miss_bytes_per_step": int(miss_bytes_step),
        "prediction_accuracy": round(overlap_sum / max(n_units, 1) / w.k, 5),
        "temporal_prediction_accuracy": round(temporal_hits / max(n_units, 1) / w.k, 5),
        "h2d_contiguous_GBps": round(link_gbps, 1),
    }
    if timer:
        g_ms = timer.total_ms("gather") / args.steps
        sel_ms = timer.total_ms("select") / args.steps
        att_ms = timer.total_ms("attn") / args.steps
        pcie = misses_timer * chunk_bytes / args.steps / (g_ms * 1e-3) / 1e9
        hidden = (g_ms + sel_ms + att_ms - timer_ms_per_step) / g_ms if g_ms > 0 else 0.0
        out["pcie_GBps"] = round(pcie, 2)
        out["pcie_frac_of_contiguous"] = round(pcie / link_gbps, 4)
        out["copy_ms_per_step"] = round(g_ms, 3)
        out["compute_ms_per_step"] = round(sel_ms + att_ms, 3)
        out["copy_hidden_frac"] = round(min(max(hidden, 0.0), 1.0), 4)
        out["hot_cache_attn_GBps"] = round(union_bytes_step / (att_ms * 1e-3) / 1e9, 1)
        out["roofline"] = {"bound": "pcie", "kernel": "gather_kv", "achieved": round(pcie, 2),
                           "peak": PCIE_PEAK_GBPS, "unit": "GB/s", "frac": round(pcie / PCIE_PEAK_GBPS, 4),
                           "traffic": None}
        out["kernels"] = {
            "select (score_topk + union_select)": {"avg_us": round(sel_ms * 1e3 / w.layers, 2)},
            "gather_kv": {"avg_us": round(g_ms * 1e3 / w.layers, 2),
                          "bytes_per_launch": int(misses_timer * chunk_bytes / args.steps / w.layers)},
            "sparse_decode_attn": {"avg_us": round(att_ms * 1e3 / w.layers, 2),
                                   "bytes_per_launch": int(union_bytes_step / w.layers)},
        }
    else:
        out["roofline"] = None
    if args.cpu_seconds > 0:
        qs_host = [q.cpu().numpy().astype(np.float64) for q in qs_at(total - 1)]
        out["cpu_baseline"] = cpu_baseline(w, qs_host, Kh, Vh, args.cpu_seconds, args.seed)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_mla(args, w):
    """Token-level selection over one latent KV head (one layer): the indexer call
    (dk_score_topk_union on bf16 per-token keys) and latent attention on the matrix
    cores (dk_sparse_decode_attn with dk 576 / dv 512)."""
    import numpy as np
    import torch
    from sparse_kv_retrieval_amd import binding as dkb
    from sparse_kv_retrieval_amd import synth

    dev = "cuda"
    t0 = time.time()
    qi, q = synth.make_mla_queries(w, args.seed, device=dev)
    Kidx, lat = synth.make_mla_pools(w, args.seed, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    N = w.T * w.k
    topk = torch.empty(w.B, 1, w.T, w.k, **i32)
    uid = torch.empty(w.B, 1, N, **i32)
    mem = torch.empty(w.B, 1, N, dtype=torch.uint8, device=dev)
    cnt = torch.empty(w.B, 1, **i32)
    ov = torch.empty(w.B, 1, **i32)
    ws_i = torch.empty(dkb.index_topk_workspace_size(w.B, 1, w.T, w.L), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(1, dkb.attn_workspace_size(w.B, 1, w.T, w.Hq, w.dv, N, 1)), dtype=torch.uint8,
                       device=dev)
    out = torch.empty(w.B, w.T, w.Hq, w.dv, dtype=torch.float32, device=dev)
    lse = torch.empty(w.B, w.T, w.Hq, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s: indexer keys {Kidx.nbytes / 1e9:.2f} GB, "
          f"latent {lat.nbytes / 1e9:.2f} GB", file=sys.stderr, flush=True)

    calls = ("index_topk_union", "mla_attention")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(record):
        e = ev[record - 1] if record else None
        if record:
            e[0].record()
        dkb.score_topk_union(qi, Kidx, w.k, w.index_scale, dkb.DK_REDUCE_MEAN, topk, None, uid, mem, cnt, ov,
                             ws_i)
        if record:
            e[1].record()
        dkb.mla_decode_attn(q, lat, uid, mem, cnt, w.scale, out=out, lse=lse, ws=ws_a)
        if record:
            e[2].record()

    step(0)
    torch.cuda.synchronize()
    union_tokens = int(cnt.sum().item())
    accuracy = float(ov.double().mean().item()) / w.k
    for _ in range(args.warmup):
        step(0)
    torch.cuda.synchronize()
    # headline: event-free steps, one event per step boundary
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    bounds[0].record()
    for s_ in range(args.steps):
        step(0)
        bounds[s_ + 1].record()
    torch.cuda.synchronize()
    ms_per_step = bounds[0].elapsed_time(bounds[-1]) / args.steps
    step_ms = [bounds[s_].elapsed_time(bounds[s_ + 1]) for s_ in range(args.steps)]
    # call durations: the same steps again with events around every call
    for s_ in range(args.steps):
        step(s_ + 1)
    torch.cuda.synchronize()
    call_ms = {c: sum(ev[s_][i].elapsed_time(ev[s_][i + 1]) for s_ in range(args.steps)) / args.steps
               for i, c in enumerate(calls)}

    # algorithmic work: the indexer streams every key once (queries and the
    # selected ids besides); attention reads each union row once and does
    # 2 * (dk + dv) flops per (query row, own token)
    idx_bytes = w.B * w.L * w.di * 2 + w.B * w.T * w.Hi * w.di * 4 + w.B * w.T * w.k * 4 * 3
    attn_bytes = union_tokens * w.latent_row_bytes() + w.B * w.T * w.Hq * (w.dk * 4 + (w.dv + 1) * 4)
    attn_flops = 2.0 * w.B * w.T * w.Hq * w.k * (w.dk + w.dv)
    ki, ka = call_ms["index_topk_union"], call_ms["mla_attention"]
    kernels = {
        "index_topk_union": {"avg_us": round(ki * 1e3, 2), "bytes_per_launch": int(idx_bytes),
                             "GBps": round(idx_bytes / (ki * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(idx_bytes / (ki * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "mla_attention": {"avg_us": round(ka * 1e3, 2), "bytes_per_launch": int(attn_bytes),
                          "flops_per_launch": attn_flops,
                          "TFLOPs": round(attn_flops / (ka * 1e-3) / 1e12, 1),
                          "frac_mfma_bf16_peak": round(attn_flops / (ka * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                          "GBps": round(attn_bytes / (ka * 1e-3) / 1e9, 1)},
    }
    dominant = max(kernels, key=lambda c: kernels[c]["avg_us"])
    if dominant == "mla_attention":
        kd = kernels[dominant]
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": kd["TFLOPs"],
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": kd["frac_mfma_bf16_peak"],
                    "traffic": measured_traffic(w.name, dominant)}
    else:
        kd = kernels[dominant]
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": kd["GBps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": kd["frac_hbm_peak"], "traffic": measured_traffic(w.name, dominant)}
    res = {
        "metric": METRIC_MLA,
        "value": round(1000.0 / ms_per_step, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "Hq": w.Hq, "dk": w.dk, "dv": w.dv, "Hi": w.Hi,
                   "di": w.di, "k": w.k, "T": w.T, "seed": args.seed},
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(np.min(step_ms)), 4),
        "timing": "value: event-free steps; kernels and roofline: a second pass with events around every call",
        "mean_union_tokens": round(union_tokens / w.B, 1),
        "prediction_accuracy": round(accuracy, 5),
        "roofline": roofline,
        "kernels": kernels,
    }
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_mla(w, qi, q, Kidx, lat, topk, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


METRIC_VARIANT = {
    "minmax": "dual-query sparse decode steps/s, chunks ranked by min/max summary bounds, B=64 L=128K",
    "coverage": "dual-query sparse decode steps/s, coverage budgets (smallest chunk sets reaching gamma of the "
                "estimated mass), B=64 L=128K",
    "capped": "dual-query sparse decode steps/s with a capped-eviction working-set plan per layer, B=64 L=128K",
}


def bench_variant(args, w):
    """The HBM-pool step with a selection variant: per layer, the variant's selection
    and union (plus, for `capped`, the working-set plan of the speculative query's
    top-k), then attention of both queries over their own chunks."""
    import numpy as np
    import torch

    from sparse_kv_retrieval_amd import binding as dkb
    from sparse_kv_retrieval_amd import synth

    dev, sel = "cuda", args.selection
    B, T, Hq, Hkv, d, C, k = w.B, w.T, w.Hq, w.Hkv, w.d, w.C, w.k
    i32 = dict(dtype=torch.int32, device=dev)
    t0 = time.time()
    # layer l's queries drift l steps from the planted layer-0 queries, so every layer
    # meets the pool's heavy hitters (independent queries see flat chunk masses)
    qs = synth.make_query_sequence(w, args.seed, w.layers, device=dev)
    K, V = synth.make_kv_pool(w, args.seed, device=dev, q0=qs[0])
    k_max = args.k_max or 2 * k
    N = T * (k_max if sel == "coverage" else k)
    union_ids = torch.empty(B, Hkv, N, **i32)
    member = torch.empty(B, Hkv, N, dtype=torch.uint8, device=dev)
    count = torch.empty(B, Hkv, **i32)
    overlap = torch.empty(B, Hkv, **i32)
    ws_attn = torch.empty(max(dkb.attn_workspace_size(B, Hkv, T, Hq, d, N, w.chunk), 1), dtype=torch.uint8,
                          device=dev)
    out = torch.empty(B, T, Hq, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, T, Hq, dtype=torch.float32, device=dev)
    summary_bytes = 0
    if sel == "minmax":
        kmin, kmax = dkb.build_minmax(K, w.chunk)
        summary_bytes = kmin.nbytes + kmax.nbytes
        topk_idx = torch.empty(B, Hkv, T, k, **i32)
        ws_sel = torch.empty(dkb.index_topk_workspace_size(B, Hkv, T, C), dtype=torch.uint8, device=dev)
    else:
        lm = dkb.build_landmarks(K, w.chunk)
        summary_bytes = lm.nbytes
    if sel == "coverage":
        cov_idx = torch.empty(B, Hkv, T, k_max, **i32)
        cov_cnt = torch.empty(B, Hkv, T, **i32)
        ws_sel = torch.empty(dkb.coverage_workspace_size(B, Hkv, T, C), dtype=torch.uint8, device=dev)
    if sel == "capped":
        shadow = dkb.build_landmark_shadow(lm)
        topk_idx = torch.empty(B, Hkv, T, k, **i32)
        topk_score = torch.empty(B, Hkv, T, k, dtype=torch.float32, device=dev)
        ws_sel = torch.empty(max(dkb.score_topk_workspace_size(B, Hkv, T, C, k, True), 1), dtype=torch.uint8,
                             device=dev)
        S = args.slots or 4 * k
        resident = torch.full((w.layers, B, Hkv, S), -1, **i32)
        stamp = torch.full((w.layers, B, Hkv, S), -1, **i32)
        sel_slot = torch.empty(B, Hkv, k, **i32)
        admit_chunk = torch.empty(B, Hkv, max(args.cap, 1), **i32)
        admit_slot = torch.empty(B, Hkv, max(args.cap, 1), **i32)
        admit_count = torch.empty(w.layers, B, Hkv, **i32)
        hit_count = torch.empty(w.layers, B, Hkv, **i32)
    torch.cuda.synchronize()
    print(f"[bench] {sel} inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    plan_step = [0]

    def select(l):
        q = qs[l]
        if sel == "minmax":
            dkb.score_topk_minmax(q, kmin, kmax, k, w.scale, topk_idx=topk_idx, union=True, union_ids=union_ids,
                                  member=member, count=count, overlap=overlap, ws=ws_sel, want_scores=False)
        elif sel == "coverage":
            dkb.score_coverage(q, lm, args.gamma, k_max, args.cov_scale, sel_idx=cov_idx, sel_count=cov_cnt,
                               union=True, union_ids=union_ids, member=member, count=count, overlap=overlap,
                               ws=ws_sel, want_scores=False)
        else:
            dkb.score_topk_union(q, lm, k, w.scale, dkb.DK_REDUCE_MEAN, topk_idx, topk_score, union_ids, member,
                                 count, overlap, ws_sel, shadow=shadow)

    def plan(l):
        dkb.capped_plan(topk_idx[:, :, 1], resident[l], stamp[l], args.cap, plan_step[0],
                        sel_score=topk_score[:, :, 1], sel_slot=sel_slot, admit_chunk=admit_chunk,
                        admit_slot=admit_slot, admit_count=admit_count[l], hit_count=hit_count[l])

    def attend(l):
        dkb.sparse_decode_attn(qs[l], K, V, union_ids, member, count, w.chunk, w.scale, out=out, lse=lse,
                               ws=ws_attn)

    calls = ("select", "plan", "attn") if sel == "capped" else ("select", "attn")
    fns = {"select": select, "plan": plan, "attn": attend}

    # per-layer union sizes (deterministic for the stateless selections)
    sel_chunks, ov = [], []
    for l in range(w.layers):
        select(l)
        sel_chunks.append(int(count.sum().item()))
        ov.append(overlap.double().mean().item())
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(w.layers)]
          for _ in range(args.steps)]

    def step(record):
        for l in range(w.layers):
            e = ev[record - 1][l] if record else None
            if record:
                e[0].record()
            for i, c in enumerate(calls):
                fns[c](l)
                if record:
                    e[i + 1].record()
        plan_step[0] += 1

    for _ in range(args.warmup):
        step(0)
    torch.cuda.synchronize()
    # headline: event-free steps, one event per step boundary
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    bounds[0].record()
    for s_ in range(args.steps):
        step(0)
        bounds[s_ + 1].record()
    torch.cuda.synchronize()
    ms_per_step = bounds[0].elapsed_time(bounds[-1]) / args.steps
    step_ms = [bounds[s_].elapsed_time(bounds[s_ + 1]) for s_ in range(args.steps)]
    # call durations: the same steps again with events around every call
    for s_ in range(args.steps):
        step(s_ + 1)
    torch.cuda.synchronize()
    call_ms = {c: 0.0 for c in calls}
    for s_ in range(args.steps):
        for l in range(w.layers):
            for i, c in enumerate(calls):
                call_ms[c] += ev[s_][l][i].elapsed_time(ev[s_][l][i + 1])

    chunk_bytes = w.chunk_kv_bytes()
    sel_bytes_step = sum(sel_chunks) * chunk_bytes
    q_bytes = B * T * Hq * d * 4
    rows_bytes = 2 * B * Hkv * T * C * 4            # fp32 score rows written, then read
    if sel == "capped":
        # the shadow selection keeps its score rows in LDS
        score_bytes = (w.landmark_bytes() // 4 + B * Hkv * C * 4 + B * Hkv * T * k * d * 4 + q_bytes
                       + B * Hkv * T * k * 4 * 4)
    else:
        score_bytes = summary_bytes + rows_bytes + q_bytes + B * Hkv * N * 5
    S_ = args.slots or 4 * k
    per_call_bytes = {
        "select": score_bytes,
        "plan": B * Hkv * (k * 8 + S_ * 16 + k * 4 + 2 * args.cap * 4),
        "attn": sel_bytes_step / w.layers,
    }
    n_launch = args.steps * w.layers
    kernels = {}
    for c in calls:
        avg_ms = call_ms[c] / n_launch
        gbps = per_call_bytes[c] / (avg_ms * 1e-3) / 1e9
        kernels[c] = {"avg_us": round(avg_ms * 1e3, 2), "bytes_per_launch": int(per_call_bytes[c]),
                      "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    dominant = max(kernels, key=lambda c: kernels[c]["avg_us"])
    kd = kernels[dominant]
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": kd["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(kd["GBps"] / HBM_PEAK_GBPS, 4), "traffic": None}
    attn_gbps = sel_bytes_step / (call_ms["attn"] / args.steps * 1e-3) / 1e9
    cfg = {"workload": w.name, "B": B, "L": w.L, "Hq": Hq, "Hkv": Hkv, "d": d, "chunk": w.chunk, "k": k, "T": T,
           "layers": w.layers, "seed": args.seed, "selection": sel, "queries": "drifting sequence over layers"}
    if sel == "coverage":
        cfg.update(gamma=args.gamma, k_max=k_max, estimate_scale=args.cov_scale)
    if sel == "capped":
        cfg.update(cap=args.cap, slots=S_)
    res = {
        "metric": METRIC_VARIANT[sel],
        "value": round(1000.0 / ms_per_step, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "timing": "value: event-free steps; kernels and roofline: a second pass with events around every call",
        "selected_kv_GBps": round(attn_gbps, 1),
        "selected_kv_frac_hbm_peak": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "mean_union_chunks": round(sum(sel_chunks) / (w.layers * B * Hkv), 2),
        "mean_overlap_chunks": round(float(np.mean(ov)), 2),
        "roofline": roofline,
        "kernels": kernels,
    }
    if sel == "coverage":
        res["mean_kept_chunks_per_query"] = round(float(cov_cnt.double().mean().item()), 2)
    if sel == "capped":
        res["mean_admits_per_head_step"] = round(float(admit_count.double().mean().item()), 2)
        res["mean_hits_per_head_step"] = round(float(hit_count.double().mean().item()), 2)
    res["cpu_baseline"] = cpu_baseline_variant(w, sel, qs, K, V, args) if args.cpu_seconds > 0 else None
    print(json.dumps(res), flush=True)


def _variant_worker(task):
    """The oracle's variant step (selection, union, for `capped` the plan from an
    empty working set, then attention) on one (b, g), layer after layer."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import dualkv_oracle as O
    Kr, Vr, qs, sel, chunk, k, scale, T, k_max, S, cap, gamma, cov_scale, budget = task
    units, spent, layer = 0, 0.0, 0
    with threadpool_limits(1):
        Kh, Vh = _widen(Kr)[None, None], _widen(Vr)[None, None]
        if sel == "minmax":
            mn, mx = O.chunk_minmax(Kh, chunk)        # summaries: built once, not timed
        else:
            lm = O.chunk_landmarks(Kh, chunk)
        res, st = np.full((1, 1, S), -1), np.full((1, 1, S), -1)
        while spent < budget:
            qh = qs[layer % len(qs)]
            t0 = time.perf_counter()
            if sel == "minmax":
                chosen = O.minmax_topk(qh, mn, mx, k, scale)
                O.union_select(chosen)
            elif sel == "coverage":
                s = O.chunk_scores(qh, lm, cov_scale, "mean")
                idx, n = O.coverage_select(s, gamma, k_max)
                O.union_select_ragged(idx, n)
                chosen = [[[idx[0, 0, t, :n[0, 0, t]] for t in range(T)]]]
            else:
                s = O.chunk_scores(qh, lm, scale, "mean")
                chosen = O.topk_chunks(s, k)
                O.union_select(chosen)
                sc = np.take_along_axis(s, chosen, axis=-1)
                r = O.capped_plan(chosen[:, :, 1], sc[:, :, 1], None, res, st, cap, layer)
                res, st = r["resident"], r["stamp"]
            if sel == "coverage":
                for t in range(T):
                    sel_t = np.asarray(chosen[0][0][t])[None, None, None]
                    O.sparse_attention(qh[:, t:t + 1], Kh, Vh, sel_t, chunk, scale)
            else:
                O.sparse_attention(qh, Kh, Vh, chosen, chunk, scale)
            spent += time.perf_counter() - t0
            units += 1
            layer += 1
    return {"units": units, "spent": spent}


def cpu_baseline_variant(w, sel, qs, K, V, args):
    """Time the fp64 CPU oracle of the variant step on sampled (request, KV head,
    layer) units on every host core."""
    import numpy as np
    n, _ = cpu_pool_size()
    rng = np.random.default_rng(args.seed)
    flat = rng.choice(w.B * w.Hkv, size=min(n, w.B * w.Hkv), replace=False)
    qs_h = [q.cpu().numpy().astype(np.float64) for q in qs]
    tasks = []
    for f in flat:
        b, g = divmod(int(f), w.Hkv)
        tasks.append((raw_host(K[b, g]), raw_host(V[b, g]), [q[b:b + 1, :, g * w.G:(g + 1) * w.G] for q in qs_h],
                      sel, w.chunk, w.k, w.scale, w.T, args.k_max or 2 * w.k, args.slots or 4 * w.k, args.cap,
                      args.gamma, args.cov_scale, args.cpu_seconds))
    res, rate = run_cpu_pool(_variant_worker, tasks)
    return cpu_record(rate, w.B * w.Hkv * w.layers, res,
                      f"(request, KV head, layer) units of the {w.name} {sel} step (summaries precomputed)")


def _mla_worker(task):
    """The oracle's token-level step (indexer top-k, union, latent attention) on
    one request, repeated for `budget` seconds; the GPU's sets are compared."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import dualkv_oracle as O
    qih, qh, Kr, Lr, gsel, k, index_scale, dv, scale, budget = task
    units, spent = 0, 0.0
    cmp = [0, 0, 0, 0]
    with threadpool_limits(1):
        kh, lh = _widen(Kr)[None, None], _widen(Lr)[None, None]
        while spent < budget:
            t0 = time.perf_counter()
            s = O.chunk_scores(qih, kh, index_scale, "mean")
            sel = O.topk_chunks(s, k)
            O.union_select(sel)
            O.mla_attention(qh, lh, sel, dv, scale)
            spent += time.perf_counter() - t0
            if units == 0:
                cmp = list(near_tie_report(gsel, sel, s))
            units += 1
    return {"units": units, "spent": spent, "cmp": cmp}


def cpu_baseline_mla(w, qi, q, Kidx, lat, gpu_topk, budget_s):
    """Time the fp64 CPU oracle (indexer top-k, union, latent attention) on sampled
    whole requests on every host core; compare the sampled selections with the
    GPU's."""
    import numpy as np
    n, _ = cpu_pool_size()
    reqs = list(range(min(n, w.B)))
    qih, qh, gt = (x.cpu().numpy() for x in (qi, q, gpu_topk))
    tasks = [(qih[b:b + 1].astype(np.float64), qh[b:b + 1].astype(np.float64), raw_host(Kidx[b, 0]),
              raw_host(lat[b, 0]), gt[b:b + 1], w.k, w.index_scale, w.dv, w.scale, budget_s) for b in reqs]
    res, rate = run_cpu_pool(_mla_worker, tasks)
    out = cpu_record(rate, w.B, res, f"whole requests of the {w.name} layer", "request")
    cmp = [sum(r["cmp"][i] for r in res) for i in range(4)]
    out["selection_check"] = {"rows": cmp[0], "rows_differing": cmp[1], "near_tie_chunks": cmp[2],
                              "mismatched_chunks": cmp[3]}
    return out


def bench_ceiling(args):
    """Read ceilings of the card in the attention's geometry (1536 blocks of 256
    threads, 24 tiles of 16 KiB each: 604 MB), with the probe library, and the
    rate of three ways to move scattered 8 KiB chunks from pinned host memory."""
    import ctypes
    import numpy as np
    import torch
    from sparse_kv_retrieval_amd import binding as dkb

    path = os.path.join(ROOT, "sparse_kv_retrieval_amd", "libdkprobe.so")
    if not os.path.exists(path):
        raise SystemExit("libdkprobe.so is not built (python -m sparse_kv_retrieval_amd.build)")
    probe = ctypes.CDLL(path)
    probe.dkp_read_pass.restype = ctypes.c_int
    probe.dkp_read_pass.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nch = 1 << 19                                      # 8 KiB chunks per array: 4 GiB each
    K = torch.ones(nch * 4096, dtype=torch.bfloat16, device="cuda")
    V = torch.ones(nch * 4096, dtype=torch.bfloat16, device="cuda")
    blocks, tpb = 1536, 24
    ntile = blocks * tpb
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed)
    ids = torch.randint(0, nch, (ntile,), generator=g, device="cuda", dtype=torch.int64)
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for mode, mname in ((0, "register_loads"), (1, "lds_dma_ring")):
        for gather in (False, True):
            best = float("inf")
            for r in range(7):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                rc = probe.dkp_read_pass(mode, ctypes.c_void_p(K.data_ptr()), ctypes.c_void_p(V.data_ptr()),
                                         ctypes.c_void_p(ids.data_ptr()) if gather else None, blocks, tpb,
                                         ctypes.c_void_p(sink.data_ptr()), st)
                b.record()
                b.synchronize()
                if rc != 0:
                    raise SystemExit(f"dkp_read_pass failed: {rc}")
                if r:
                    best = min(best, a.elapsed_time(b))
            res[f"{mname}_{'gather_8KiB' if gather else 'contiguous'}"] = {
                "us": round(best * 1e3, 1), "GBps": round(ntile * 16384 / (best * 1e-3) / 1e9, 1)}
    del K, V
    torch.cuda.empty_cache()
    # scattered 8 KiB chunks of a pinned host pool into an HBM cache: 64 (b, g) of
    # 1024 chunks each, 78 missed chunks per (b, g) (4992 in all)
    B_, H_, per, chunk, d = 8, 8, 78, 32, 128
    Ch = 1024
    Kh = torch.ones(B_, H_, Ch * chunk, d, dtype=torch.bfloat16, pin_memory=True)
    Vh = torch.ones(B_, H_, Ch * chunk, d, dtype=torch.bfloat16, pin_memory=True)
    Kd = torch.empty(B_, H_, per * chunk, d, dtype=torch.bfloat16, device="cuda")
    Vd = torch.empty_like(Kd)
    rng = np.random.default_rng(args.seed)
    src = torch.from_numpy(np.stack([np.sort(rng.choice(Ch, per, replace=False)) for _ in range(B_ * H_)])
                           .astype(np.int32)).reshape(B_, H_, per)
    host_src = src.pin_memory()
    dev_src = src.cuda()
    n = B_ * H_ * per
    nbytes = 2 * n * chunk * d * 2
    host = {}
    for name, fn in (("hipMemcpyAsync_per_chunk", lambda: dkb.gather_kv(Kh, Vh, host_src, None, chunk, Kd, Vd)),
                     ("mapped_gather_kernel", lambda: dkb.gather_kv(Kh, Vh, dev_src, None, chunk, Kd, Vd)),
                     ("one_contiguous_copy", lambda: (Kd.view(-1).copy_(Kh.view(-1)[:Kd.numel()], non_blocking=True),
                                                      Vd.view(-1).copy_(Vh.view(-1)[:Vd.numel()], non_blocking=True)))):
        best = float("inf")
        for r in range(4):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            if r:
                best = min(best, time.perf_counter() - t0)
        host[name] = {"ms": round(best * 1e3, 3), "GBps": round(nbytes / best / 1e9, 2)}
    print(json.dumps({"ceiling": "read", "geometry": f"{blocks} blocks x {tpb} tiles of 16 KiB ({ntile * 16384} B)",
                      "device_read": res,
                      "host_pool_scattered_chunks": {"chunks": n, "bytes": nbytes, **host}}), flush=True)


def calibrate_copy():
    """Three plain copies of 512 MiB K + 512 MiB V (1 GiB read, 1 GiB written each)."""
    import torch

    from sparse_kv_retrieval_amd import binding as dkb

    rows, d, chunk = 1 << 21, 128, 32
    C = rows // chunk
    src = [torch.ones(1, 1, rows, d, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    dst = [torch.empty_like(src[0]) for _ in range(2)]
    ids = torch.arange(C, dtype=torch.int32, device="cuda").reshape(1, 1, C)
    for _ in range(3):
        dkb.gather_kv(src[0], src[1], ids, None, chunk, dst[0], dst[1])
    torch.cuda.synchronize()
    assert torch.equal(dst[0], src[0]) and torch.equal(dst[1], src[1])
    nbytes = 2 * src[0].nbytes
    print(json.dumps({"calibration": "copy", "kernel": "k_gather", "launches": 3,
                      "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode step has no "
              "cross-GPU exchange and this benchmark measures a single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.cpu_seconds > 0 and not args.calibrate_copy and not args.ceiling:
        start_cpu_pool()          # forked before anything touches the GPU
    try:
        run(args)
    finally:
        stop_cpu_pool()


def run(args):
    import numpy as np
    import torch

    from sparse_kv_retrieval_amd import binding as dkb   # fails loudly without libdualkv.so
    from sparse_kv_retrieval_amd import synth
    from sparse_kv_retrieval_amd.workloads import MLA_WORKLOADS, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload in MLA_WORKLOADS:
        torch.cuda.set_device(0)
        bench_mla(args, MLA_WORKLOADS[args.workload])
        return
    w = WORKLOADS[args.workload]
    if args.layers:
        w = w.with_(layers=args.layers)
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.ceiling:
        bench_ceiling(args)
        return
    if w.host_pool:
        bench_host_pool(args, w)
        return
    if args.selection != "landmark":
        bench_variant(args, w)
        return

    t0 = time.time()
    qs = [synth.make_queries(w, args.seed, layer=l, device=dev) for l in range(w.layers)]
    K, V = synth.make_kv_pool(w, args.seed, device=dev, q0=qs[0])
    lm = dkb.build_landmarks(K, w.chunk)
    shadow = None if args.no_shadow else dkb.build_landmark_shadow(lm)
    st = dkb.DecodeStep(w.B, w.T, w.Hq, w.Hkv, w.d, w.C, w.chunk, w.k, w.scale, dev, want_scores=False,
                        shadow=shadow)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s: pool {2 * K.nbytes / 1e9:.2f} GB, "
          f"landmarks {lm.nbytes / 1e9:.3f} GB", file=sys.stderr, flush=True)

    # Per-layer union sizes (deterministic): the selected-KV bytes of each layer.
    sel_chunks, overlap, gpu_topk, max_chunks = [], [], [], 0
    for l in range(w.layers):
        st.run(qs[l], lm, K, V)
        sel_chunks.append(int(st.count.sum().item()))
        max_chunks = max(max_chunks, int(st.count.max().item()))
        overlap.append(st.overlap.double().mean().item())
        gpu_topk.append(st.topk_idx.cpu().numpy())
    torch.cuda.synchronize()
    chunk_bytes = w.chunk_kv_bytes()
    sel_bytes_step = sum(sel_chunks) * chunk_bytes
    lm_bytes_layer = w.landmark_bytes()
    accuracy = float(np.mean(overlap)) / w.k

    attn_call = "sparse_decode_attn_tail" if args.tail else "sparse_decode_attn"
    # the step as one dk_decode_step call (one fused kernel at this shape; with tail
    # rows the call runs the two calls' kernels) unless --two-calls asks for the
    # separate calls
    fused = not args.two_calls
    split_calls = ("score_topk_union", attn_call)
    step_kernels = "the two calls' kernels, tail rows included" if args.tail else "one fused kernel"
    calls = ("decode_step",) if fused else split_calls
    if args.tail:
        # one tail and one pair of fresh rows, shared by the layers like the pool
        gt = torch.Generator(device=dev)
        gt.manual_seed(args.seed + 7)
        kvdt = K.dtype
        K_tail = torch.randn(w.B, w.Hkv, args.tail, w.d, generator=gt, device=dev).to(kvdt)
        V_tail = torch.randn(w.B, w.Hkv, args.tail, w.d, generator=gt, device=dev).to(kvdt)
        tail_len = torch.randint(args.tail // 2, args.tail + 1, (w.B,), generator=gt, device=dev,
                                 dtype=torch.int32)
        K_new = torch.randn(w.B, w.T, w.Hkv, w.d, generator=gt, device=dev).to(kvdt)
        V_new = torch.randn(w.B, w.T, w.Hkv, w.d, generator=gt, device=dev).to(kvdt)
        ws_tail = torch.empty(dkb.attn_tail_workspace_size(w.B, w.Hkv, w.T, w.Hq, w.d, w.T * w.k, w.chunk),
                              dtype=torch.uint8, device=dev)
        tail_rows = int(tail_len.sum().item())
        ws_step = torch.empty(max(1, dkb.decode_step_workspace_size(w.B, w.Hkv, w.T, w.Hq, w.C, w.d, w.k, w.chunk,
                                                                    shadow is not None, True)),
                              dtype=torch.uint8, device=dev)
        tail_kw = dict(K_tail=K_tail, V_tail=V_tail, tail_len=tail_len, K_new=K_new, V_new=V_new)
    else:
        ws_step, tail_kw = st.ws_step, {}
    use_events = not args.no_events
    call_ms = {c: 0.0 for c in calls + (split_calls if fused else ())}

    def step(ev_step=None, one_call=fused):
        """One decode step over every layer; with ev_step, events around every call."""
        for l in range(w.layers):
            q = qs[l]
            e = ev_step[l] if ev_step else None
            if e:
                e[0].record()
            if one_call:
                dkb.decode_step(q, lm, K, V, w.chunk, w.k, w.scale, dkb.DK_REDUCE_MEAN, shadow, st.topk_idx, None,
                                st.union_ids, st.member, st.count, st.overlap, st.out, st.lse, ws_step, **tail_kw)
                if e:
                    e[1].record()
                continue
            dkb.score_topk_union(q, lm, w.k, w.scale, dkb.DK_REDUCE_MEAN, st.topk_idx, None, st.union_ids,
                                 st.member, st.count, st.overlap, st.ws_topk, shadow=shadow)
            if e:
                e[1].record()
            if args.tail:
                dkb.sparse_decode_attn_tail(q, K, V, st.union_ids, st.member, st.count, w.chunk, w.scale,
                                            K_tail=K_tail, V_tail=V_tail, tail_len=tail_len, K_new=K_new,
                                            V_new=V_new, out=st.out, lse=st.lse, ws=ws_tail)
            else:
                dkb.sparse_decode_attn(q, K, V, st.union_ids, st.member, st.count, w.chunk, w.scale,
                                       out=st.out, lse=st.lse, ws=st.ws_attn)
            if e:
                e[2].record()

    flush_mb = args.flush_mb if args.flush_mb is not None else (1024 if w.layers == 1 else 0)
    flush_buf = torch.empty(flush_mb << 20, dtype=torch.uint8, device=dev) if flush_mb else None

    def flush():
        if flush_buf is not None:
            flush_buf.fill_(1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The headline: K steps with nothing between the calls but one event at each
    # step boundary (with a cache flush, each step between its own pair of events,
    # the flush outside them).
    if flush_buf is None:
        bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        bounds[0].record()
        for s in range(args.steps):
            step()
            bounds[s + 1].record()
        torch.cuda.synchronize()
        step_ms = [bounds[s].elapsed_time(bounds[s + 1]) for s in range(args.steps)]
        total_ms = bounds[0].elapsed_time(bounds[-1])
    else:
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for s in range(args.steps):
            flush()
            pairs[s][0].record()
            step()
            pairs[s][1].record()
        torch.cuda.synchronize()
        step_ms = [a.elapsed_time(b) for a, b in pairs]
        total_ms = sum(step_ms)
    ms_per_step = total_ms / args.steps
    # Call durations: the same K steps again, with events around every call (on the
    # launch stream), read only afterwards.
    call_pass_ms = None
    if use_events:
        ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(w.layers)]
              for _ in range(args.steps)]
        for s in range(args.steps):
            flush()
            step(ev[s])
        torch.cuda.synchronize()
        for s in range(args.steps):
            for l in range(w.layers):
                for i, c in enumerate(calls):
                    call_ms[c] += ev[s][l][i].elapsed_time(ev[s][l][i + 1])
        call_pass_ms = sum(ev[s][0][0].elapsed_time(ev[s][w.layers - 1][len(calls)])
                           for s in range(args.steps)) / args.steps
        if fused:
            # the same steps once more as the two separate calls, for their own durations
            ev2 = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(w.layers)]
                   for _ in range(args.steps)]
            for s in range(args.steps):
                flush()
                step(ev2[s], one_call=False)
            torch.cuda.synchronize()
            for s in range(args.steps):
                for l in range(w.layers):
                    for i, c in enumerate(split_calls):
                        call_ms[c] += ev2[s][l][i].elapsed_time(ev2[s][l][i + 1])
    steps_per_s = 1000.0 / ms_per_step

    kernels = {}
    n_launch = args.steps * w.layers
    q_bytes = w.B * w.T * w.Hq * w.d * 4
    if shadow is None:
        score_bytes = lm_bytes_layer + q_bytes
    else:
        # 8-bit codes and one fp32 scale per chunk + at least k fp32 landmark rows
        # re-scored per (b, g, t) (the shadow scores stay in LDS)
        score_bytes = (lm_bytes_layer // 4 + w.B * w.Hkv * w.C * 4
                       + w.B * w.Hkv * w.T * w.k * w.d * 4 + q_bytes)
    per_call_bytes = {
        # scores and selection, then the union: both sets read back, ids + bits written
        "score_topk_union": score_bytes + w.B * w.Hkv * w.T * w.k * 4 * 3,
        attn_call: sel_bytes_step / w.layers
        + (w.Hkv * (tail_rows + w.B * w.T) * w.d * 2 * K.element_size() if args.tail else 0),
    }
    # the fused call: the selection's bytes (its union stays in the block) and the selected KV
    per_call_bytes["decode_step"] = per_call_bytes["score_topk_union"] + per_call_bytes[attn_call]
    for c in calls + (split_calls if fused else ()):
        if not use_events:
            break
        avg_ms = call_ms[c] / n_launch
        gbps = per_call_bytes[c] / (avg_ms * 1e-3) / 1e9
        kernels[c] = {"avg_us": round(avg_ms * 1e3, 2), "bytes_per_launch": int(per_call_bytes[c]),
                      "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    attn_ms_step = call_ms[attn_call] / args.steps if use_events else float("nan")
    sel_gbps = sel_bytes_step / (attn_ms_step * 1e-3) / 1e9 if use_events else float("nan")

    # every byte the step moves: landmark scoring, union chunks, queries, outputs, indices
    out_bytes = w.B * w.T * w.Hq * (w.d + 1) * 4          # out and lse
    full_bytes_step = w.layers * (per_call_bytes["score_topk_union"] + q_bytes + out_bytes) + sel_bytes_step
    copy_gbps = hbm_copy_gbps(torch, dkb)

    dominant = max(kernels, key=lambda c: kernels[c]["avg_us"]) if kernels else None
    if fused and kernels:
        dominant = "decode_step"      # the one call of the timed step
    roofline = None
    if dominant:
        kd = kernels[dominant]
        # the counter summaries are of runs without tail rows
        traffic = None if args.tail else measured_traffic(w.name, dominant)
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": kd["GBps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(kd["GBps"] / HBM_PEAK_GBPS, 4),
                    "traffic": None if traffic is None else int(traffic)}

    out = {
        "metric": METRIC if w.name == "b64_l128k" else
        f"dual-query sparse decode steps/s + selected-KV GB/s (% HBM peak), B={w.B} L={w.L}, {w.layers} layer(s)",
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "chunk": w.chunk, "k": w.k, "T": w.T, "layers": w.layers, "seed": args.seed,
                   "landmark_shadow": shadow is not None, "tail_max": args.tail,
                   "cache_flush_MiB_between_steps": flush_mb},
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(np.min(step_ms)), 4),
        "timing": "value and ms_per_step: event-free steps (one event per step boundary); kernels and "
                  "roofline: a second pass of the same steps with events around every call"
                  + (f"; the step is one dk_decode_step call per layer ({step_kernels}), "
                     f"and a third pass times the same work as its two separate calls (score_topk_union, "
                     f"{attn_call}: selected_kv_GBps is the selected KV over the separate attention call's time)"
                     if fused else ""),
        "step_call": "dk_decode_step" if fused else "dk_score_topk_union + " + ("dk_sparse_decode_attn_tail" if args.tail else "dk_sparse_decode_attn"),
        "ms_per_step_call_pass": None if call_pass_ms is None else round(call_pass_ms, 4),
        "selected_kv_GBps": round(sel_gbps, 1),
        "selected_kv_frac_hbm_peak": round(sel_gbps / HBM_PEAK_GBPS, 4),
        "hbm_copy_GBps": round(copy_gbps, 1),
        "selected_kv_frac_of_copy": round(sel_gbps / copy_gbps, 4),
        "full_step_GBps": round(full_bytes_step / (ms_per_step * 1e-3) / 1e9, 1),
        "full_step_frac_hbm_peak": round(full_bytes_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "selected_kv_bytes_per_step": int(sel_bytes_step),
        "mean_union_chunks": round(sum(sel_chunks) / (w.layers * w.B * w.Hkv), 2),
        "max_union_chunks": max_chunks,
        "prediction_accuracy": round(accuracy, 5),
        "roofline": roofline,
        "kernels": kernels,
    }
    if args.cpu_seconds > 0:
        qs_host = [q.cpu().numpy().astype(np.float64) for q in qs]
        out["cpu_baseline"] = cpu_baseline(w, qs_host, K, V, args.cpu_seconds, args.seed, gpu_topk)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
