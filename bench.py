#!/usr/bin/env python3
"""Benchmark of the paged fused-MoE layer on one MI355X.

One step = one pass of the layer over one batch of resident inputs: top-k
routing + alignment (moe_route), the gate/up GEMM with SiLU*mul, the down GEMM
with the weighted combine (moe_paged_forward), reading every expert in place
from pool pages or from the active load buffer.  The load-buffer fill of the
next layer (pinned host -> device over PCIe on a side stream) is measured in
the same run and reported under "loadbuf": its bound is the host link, not HBM.

Consecutive steps rotate over R copies of the layer's pool and load buffers
(R large enough that R working sets exceed the 256 MB Infinity Cache), as the
layers of a model would, so each step streams its weights from HBM.

Prints ONE JSON line.  Default workload: the Mixtral-8x7B-shaped layer (T=4096,
d=4096, f=14336, E=8, top-2, Zipf(1.2) routing; all experts paged in a
fragmented pool), the largest configuration; every other configuration (the
tiny, Qwen1.5-MoE-shaped and Qwen3-Next-shaped layers and the decode sweep
T = 1, 2, 4, 8, 32, 128, 512) is timed in the same run and reported under
"configs" (step time, fractions of the rooflines, paged vs contiguous, the
dominant kernel's roofline; for batches of up to 512 tokens also the step
replayed from a HIP graph).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged fused-MoE TFLOP/s & HBM GB/s (%roofline) + overhead vs contiguous"
HBM_PEAK_GBS = 8000.0
# HBM bytes per launch of the roofline kernel (k_gemm1, or the decode form's gate/up launch)
# measured with rocprofv3 (FETCH_SIZE scaled by 2.0, the factor a 1 GiB copy reads back, plus
# WRITE_SIZE), keyed by workload, T, block_m, atomic combine and a hash of that kernel's
# sources as the counters were taken on them.  Reported only while that hash matches.
MEASURED_TRAFFIC = {
    ("mixtral", 4096, 256, False, "d6fda7df82d698e1"): 3812226821,
    ("qwen15", 1024, 128, False, "d6fda7df82d698e1"): 718600108,
    ("qwen3n", 8192, 128, False, "d6fda7df82d698e1"): 2774475391,
    ("decode", 1, 16, False, "fe5e8ea014cba59d"): 46334585,
    ("decode", 8, 16, False, "fe5e8ea014cba59d"): 300421338,
    ("decode", 32, 16, False, "d6fda7df82d698e1"): 577641550,
}
GEMM_SOURCES = ("paged_expert_weight_amd/csrc/moe_gemm.hip", "paged_expert_weight_amd/csrc/internal.h")
DECODE_SOURCES = ("paged_expert_weight_amd/csrc/decode.hip", "paged_expert_weight_amd/csrc/route_token.h",
                  "paged_expert_weight_amd/csrc/internal.h")
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20

WORKLOAD_TEXT = {
    "tiny": "tiny MoE layer T=16 d=128 f=64 E=8 top-2; 6 experts paged in a 32-page pool, 2 via load buffer",
    "qwen15": "Qwen1.5-MoE-14B-shaped MoE layer T=1024 d=2048 f=1408 E=60 top-4; 48 experts paged in a "
              "256-page pool (random order), 12 via double-buffered load buffer",
    "decode": "Qwen1.5-MoE-shaped decode layer d=2048 f=1408 E=60 top-4; 30 experts paged, 30 via load buffer",
    "mixtral": "Mixtral-8x7B-shaped MoE layer T=4096 d=4096 f=14336 E=8 top-2, Zipf(1.2) routing; all experts "
               "paged in a 32-page pool with 8 pages carved into KV pages",
    "qwen3n": "Qwen3-Next-80B-A3B-shaped MoE layer T=8192 d=2048 f=512 E=512 top-10 + 1 shared expert, "
              "Zipf(1.1) routing; pool of 2 MiB pages interleaved with 16-token KV pages; 64 experts via load buffer",
}


def source_hash(paths=GEMM_SOURCES) -> str:
    """Hash of kernel sources' code (the grouped GEMMs', by default): comments,
    trailing blanks and empty lines removed, so that the measured traffic stays
    keyed to the code it was taken on and only a change of code (not of a
    comment) drops it.  The sources hold no string literal with a comment marker."""
    import hashlib
    import re
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for p in paths:
        with open(os.path.join(root, p), encoding="utf-8") as fh:
            code = re.sub(r"//[^\n]*|/\*.*?\*/", "", fh.read(), flags=re.S)
        lines = [ln.rstrip() for ln in code.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def gemm_source_hash() -> str:
    return source_hash(GEMM_SOURCES)


def decode_source_hash() -> str:
    return source_hash(DECODE_SOURCES)


def measured_traffic(name, T, bm, atomic, decode_form):
    h = decode_source_hash() if decode_form else gemm_source_hash()
    return MEASURED_TRAFFIC.get((name, T, bm, bool(atomic), h))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--only", action="store_true",
                    help="time the chosen workload alone (default: also every other configuration, as sub-objects)")
    ap.add_argument("--T", type=int, default=None, help="tokens (default: the workload's own; decode: 1)")
    ap.add_argument("--block-m", type=int, default=0, help="GEMM tile height (default: moe_suggest_block_m)")
    ap.add_argument("--atomic", action="store_true", help="fp32-atomic combine instead of the ordered one")
    ap.add_argument("--rotate", type=int, default=0, help="layer copies to rotate over (default: automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-contig", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed steps of the small batches")
    ap.add_argument("--no-fill", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target seconds of oracle work")
    ap.add_argument("--pipeline", action="store_true",
                    help="time an L-layer pass through moe_pipeline_* instead (one JSON line of its own)")
    ap.add_argument("--layers", type=int, default=8, help="--pipeline: layers per pass")
    ap.add_argument("--offloaded", type=int, default=1, help="--pipeline: experts per layer via the load buffer")
    ap.add_argument("--allocator", action="store_true",
                    help="time the three-tier page allocator under a serving churn (host only; one JSON line)")
    ap.add_argument("--placement", default="synth", choices=("synth", "allocator"),
                    help="pages of the pool experts: a seeded permutation, or handed out by the page allocator "
                         "during a seeded KV / eviction churn")
    ap.add_argument("--vmm", action="store_true",
                    help="compare the paged forward with the contiguous kernels over remapped expert views "
                         "(moe_vmm_*) on the same physical pages (one JSON line of its own)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB fp32 read + 1 GiB write elementwise kernel (scales HBM counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain elementwise kernel of known traffic: reads 1 GiB, writes 1 GiB."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"read_bytes": src.numel() * 4, "write_bytes": dst.numel() * 4,
                                           "launches": 3}}))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.pipeline and args.gpus == 1:
        pipeline_bench(args)
        return
    if args.allocator:
        allocator_bench(args)
        return
    if args.vmm and args.gpus == 1:
        vmm_bench(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer's hot path runs on a single MI355X and there is no "
              "multi-GPU path (experts would shard across GPUs with an all-to-all of routed tokens, not "
              "implemented here). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_expert_weight_amd as pm
    from workloads import synth

    pm.lib()  # fails loudly without the HIP library
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    name = args.workload
    T = args.T if args.T is not None else (1 if name == "decode" else synth.SPECS[name].T)
    layer = make_host_layer(name, T, args.placement)
    line, extra = bench_layer(layer, args, full=True)

    # every other configuration, timed in the same run: step time, fractions of the rooflines,
    # paged vs contiguous and the dominant kernel's roofline (one layer resident at a time)
    if not args.only:
        subs = {}
        for sub_name, sub_T in ALL_CONFIGS:
            if (sub_name, sub_T) == (name, T):
                continue
            sub_layer = make_host_layer(sub_name, sub_T, "synth")
            sub, _ = bench_layer(sub_layer, args, full=False)
            subs[f"{sub_name}_T{sub_T}"] = sub
            del sub_layer
            torch.cuda.empty_cache()
        line["configs"] = subs

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layer, args.cpu_seconds)
    line.update(extra)
    print(json.dumps(line), flush=True)


# The configurations every default run times besides the headline one (the decode sweep
# as one entry per batch size, with 2 and 4 tokens beside the sweep's 1, 8, 32, 128, 512).
ALL_CONFIGS = (("tiny", 16), ("qwen15", 1024), ("decode", 1), ("decode", 2), ("decode", 4), ("decode", 8),
               ("decode", 32), ("decode", 128), ("decode", 512), ("mixtral", 4096), ("qwen3n", 8192))
_HOST_LAYERS = {}


def make_host_layer(name, T, placement):
    """The seeded host layer of a workload with its first T tokens (the decode sweep
    slices one 512-token draw, so its weights are generated once)."""
    from workloads import synth
    t0 = time.time()
    s = synth.SPECS[name]
    key = (name, placement)
    if key not in _HOST_LAYERS:
        _HOST_LAYERS.clear()
        full = synth.make_layer(s)
        if placement == "allocator":
            full = allocator_placed(full)
        _HOST_LAYERS[key] = full
    full = _HOST_LAYERS[key]
    layer = synth.Layer(s, full.x[:T].copy(), full.logits[:T].copy(), full.w13, full.w2, full.placement)
    print(f"# layer {name} T={T} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    return layer


def carve(dev, s, torch):
    """One device allocation holding a copy of the pool, both load buffers and the
    contiguous twin's w13 / w2, so that the paged path and its twin read memory of
    the same placement."""
    parts = [dev.pool, dev.loadbuf[0], dev.loadbuf[1], dev.w13, dev.w2]
    n = [t.numel() for t in parts]
    big = torch.empty(sum(n), dtype=torch.bfloat16, device=dev.pool.device)
    views, off = [], 0
    for t, k in zip(parts, n):
        v = big[off:off + k].view(t.shape)
        v.copy_(t)
        views.append(v)
        off += k
    return big, views


def bench_layer(layer, args, full):
    """Time one layer: the paged step (routing + forward in one call), its contiguous
    twin in alternating blocks, per-stage HIP-event times and the dominant kernel's
    roofline.  full: also the load-buffer fill, the per-step spread and the adjuster's
    host cost.  Returns (line, extra keys for the top level)."""
    import numpy as np
    import torch

    import paged_expert_weight_amd as pm
    from workloads import device as wdev
    from workloads import synth

    s = layer.spec
    name, T = s.name, layer.T
    dev = wdev.to_device(layer)
    fd = s.f * s.d
    # working set of one step (weights of touched experts are at most all experts)
    ws_bytes_est = min(s.E_tot, T * s.k_eff) * 3 * fd * 2
    R = args.rotate or max(2, min(16, math.ceil(1.0 * MALL_BYTES / max(1, ws_bytes_est)) + 1))

    slots = sorted(dev.host_blobs)
    # the same layer over the twin's own bytes: w13 and w2 lie back to back in the carved
    # allocation, so as a pool of 3(E+S) pages they hold W1_e on page 2e, W3_e on 2e+1 and W2_e on
    # 2(E+S)+e (every expert, the load-buffer ones included).  Paged reads of this pool touch exactly
    # the addresses the contiguous kernels read: the difference is the page lookup alone.
    same_locs = layer.placement.locs.copy()
    for e in range(s.E_tot):
        same_locs[e]["kind"] = synth.LOC_POOL
        same_locs[e]["idx"] = (2 * e, 2 * e + 1, 2 * s.E_tot + e)
    copies = []
    for r in range(R):
        big, (pool, lb0, lb1, w13, w2) = carve(dev, s, torch)
        h = pm.moe_pool_create(pool, s.pool_pages, s.d, s.f, s.E, s.k, s.S, s.loadbuf_slots, (lb0, lb1))
        pm.moe_set_expert_locs(h, layer.placement.locs)
        h_same = pm.moe_pool_create(w13, 3 * s.E_tot, s.d, s.f, s.E, s.k, s.S, s.loadbuf_slots, (lb0, lb1))
        pm.moe_set_expert_locs(h_same, same_locs)
        if s.loadbuf_slots:
            pm.moe_loadbuf_fill(h, 0, slots, [dev.host_blobs[k] for k in slots])
        copies.append(dict(h=h, h_same=h_same, big=big, pool=pool, lbs=(lb0, lb1), w13=w13, w2=w2))
    torch.cuda.synchronize()
    dev.pool = dev.w13 = dev.w2 = None
    dev.loadbuf = None
    torch.cuda.empty_cache()

    h0 = copies[0]["h"]
    bm = args.block_m or pm.moe_suggest_block_m(h0, T)
    flags = pm.MOE_FLAG_ATOMIC_COMBINE if args.atomic else 0
    ws = pm.workspace(h0, T, bm, flags)
    rt = pm.RouteOut(h0, T, bm)
    y = torch.empty_like(dev.x)
    stream = torch.cuda.current_stream()
    # the headline takes exactly --steps; the short steps of the other configurations take more
    K = args.steps if full or ws_bytes_est * 8 > 2e9 else max(args.steps, 100)
    W = args.warmup

    # One step = routing + the layer, in one call (for a decode step the routing runs inside the gate/up
    # launch).  The load buffer is refilled only by the concurrent-fill measurement (buffer 1): the
    # "buffer read" mark of buffer 0 is deferred to its next fill instead of a stream marker per step.
    def step(i, mode="paged", st=None):
        c = copies[i % R]
        st = stream if st is None else st
        if mode == "contiguous":
            pm.moe_route_contiguous_forward(c["h"], c["w13"], c["w2"], dev.logits, dev.x, bm, rt.topk_ids,
                                            rt.topk_w, rt.sorted_ids, rt.block_expert, rt.num_padded, y, ws, flags,
                                            st)
        else:
            pm.moe_route_forward(c["h_same" if mode == "paged_same" else "h"], dev.logits, dev.x, bm, rt.topk_ids,
                                 rt.topk_w, rt.sorted_ids, rt.block_expert, rt.num_padded, 0, y, ws,
                                 flags | pm.MOE_FLAG_DEFER_READ_DONE, st)

    def timed(K, W, mode="paged"):
        for i in range(W):
            step(i, mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            step(i, mode)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    # ---- paging overhead: the contiguous twin (same kernels, dense weight arrays, same inputs and
    # routing) against the paged path over the twin's own bytes (the page lookup is the only difference)
    # and over the layer's pool (pages in the workload's order, carved from the same allocation), in
    # alternating blocks (three rounds of the three modes, rotated), so that all three see the same clock
    # and thermal state.  It runs before the timed region.
    contig_ms = same_ms = paged_alt_ms = None
    if not args.no_contig:
        # blocks of about 30 ms each, and every mode in every position of the rotation once (a block that
        # follows a host synchronisation can start at a lower clock)
        K_cmp = min(2000, max(K, math.ceil(30.0 / max(1e-3, timed(5, W)))))
        modes = ("contiguous", "paged_same", "paged")
        runs = {m: [] for m in modes}
        for rnd in range(3):
            for i in range(3):
                mode = modes[(rnd + i) % 3]
                runs[mode].append(timed(K_cmp, W, mode))
        contig_ms, same_ms, paged_alt_ms = (sum(runs[m]) / 3 for m in modes)
        print(f"# {name} T={T}: contiguous {contig_ms * 1e3:.1f} us/step, paged over the same bytes "
              f"{same_ms * 1e3:.1f}, paged over the pool {paged_alt_ms * 1e3:.1f}", file=sys.stderr, flush=True)

    # ---- the timed region (paged)
    ms = timed(K, W)
    print(f"# {name} T={T}: paged {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    # ---- the same steps captured in a HIP graph and replayed (what a serving loop that captures its
    # layers sees): the stream-launched figure above includes the host launch path and the gaps between
    # launches, the replayed one the kernels and the command processor's dispatch only.  The step
    # launches kernels only (the load buffer's fill is complete, its read mark deferred).
    graph = None
    if T <= GRAPH_MAX_T and not args.no_graph:
        graph = graph_timed(step, R, K, W, stream)
        print(f"# {name} T={T}: paged, graph replay {graph['paged'] * 1e3:.1f} us/step, contiguous "
              f"{graph['contiguous'] * 1e3:.1f}", file=sys.stderr, flush=True)

    ids = rt.topk_ids.cpu().numpy()
    n = T * s.k_eff
    touched = int(np.unique(ids).size)
    flops = 6.0 * s.d * s.f * n
    bytes_alg = touched * 3 * fd * 2 + T * s.d * 2 + 2 * n * s.f * 2 + T * s.d * 2
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = bytes_alg / (ms * 1e-3) / 1e9

    # ---- per-stage times from HIP events on the launch stream (the library's events around its launches;
    # a decode step's routing is part of its first launch, a larger batch's is timed around moe_route)
    decode_form = pm.moe_forward_form(h0, T) == pm.MOE_FORM_DECODE
    routed_form = pm.moe_route_forward_form(h0, T) == pm.MOE_FORM_DECODE_ROUTED
    for c in copies:
        pm.moe_stage_timing(c["h"], True)
    ra0, ra1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    route_ms = 0.0
    for i in range(K):
        c = copies[i % R]
        if routed_form:
            step(i)
            continue
        ra0.record(stream)
        pm.moe_route(c["h"], dev.logits, bm, rt.topk_ids, rt.topk_w, rt.sorted_ids, rt.block_expert,
                     rt.num_padded, ws, stream)
        ra1.record(stream)
        pm.moe_paged_forward(c["h"], dev.x, bm, rt.topk_ids, rt.topk_w, rt.sorted_ids, rt.block_expert,
                             rt.num_padded, 0, y, ws, flags | pm.MOE_FLAG_DEFER_READ_DONE, stream)
        ra1.synchronize()
        route_ms += ra0.elapsed_time(ra1)
    torch.cuda.synchronize()
    stage = [0.0, 0.0, 0.0]
    cnt = 0
    for c in copies:
        msv, k = pm.moe_stage_times(c["h"])
        pm.moe_stage_timing(c["h"], False)
        stage = [a + b for a, b in zip(stage, msv)]
        cnt += k
    stage_us = [v / max(1, cnt) * 1e3 for v in stage]
    route_us = route_ms / K * 1e3

    # ---- roofline of the dominant kernel (the gate/up launch: 2/3 of the flops and of the weight bytes)
    g1_flops = 4.0 * n * s.f * s.d
    g1_bytes = touched * 2 * fd * 2 + T * s.d * 2 + n * s.f * 2
    g1_ai = g1_flops / g1_bytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    g1_s = stage_us[0] * 1e-6
    if g1_ai < ridge:
        roof = {"bound": "hbm", "achieved": round(g1_bytes / g1_s / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(g1_flops / g1_s / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(name, T, bm, args.atomic, routed_form or decode_form)
    roof["kernel"] = ("k_dec_route_gate_up (routing + paged gate/up, decode form: weight rows dotted with the "
                      "picks' x rows + SiLU*mul)" if routed_form else
                      "k_dec_gate_up (paged gate/up, decode form: weight rows dotted with the picks' x rows + SiLU*mul)"
                      if decode_form else "k_gemm1 (paged gate/up GEMM + SiLU*mul)")
    roof["avg_launch_us"] = round(stage_us[0], 2)
    roof["algorithmic_bytes_per_launch"] = int(g1_bytes)
    roof["algorithmic_flops_per_launch"] = int(g1_flops)

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[name] if name != "decode" else f"{WORKLOAD_TEXT[name]}; T={T}",
                   "name": name, "T": T, "block_m": bm, "placement": args.placement if full else "synth",
                   "gemm_form": "decode, routing in its gate/up launch" if routed_form else
                   "decode" if decode_form else "tiles",
                   "combine": "atomic" if args.atomic else "ordered", "layer_copies_rotated": R},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "algorithmic": {"flops": int(flops), "bytes": int(bytes_alg), "experts_touched": touched},
        "contig_ms_per_step": round(contig_ms, 5) if contig_ms else None,
        # the cost of the page lookup: paged reads of the twin's own bytes against the twin
        "overhead_vs_contiguous_pct": round((same_ms / contig_ms - 1) * 100, 3) if contig_ms else None,
        # the layer's pool (pages in the workload's order, load-buffer experts in the load buffer)
        # against the twin: the lookup plus where the weights lie in memory
        "pool_vs_contiguous_pct": round((paged_alt_ms / contig_ms - 1) * 100, 3) if contig_ms else None,
        "graph_replay": None if graph is None else {
            "us_per_step": round(graph["paged"] * 1e3, 2),
            "tflops": round(flops / (graph["paged"] * 1e-3) / 1e12, 3),
            "hbm_gbs": round(bytes_alg / (graph["paged"] * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_alg / (graph["paged"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "contig_us_per_step": round(graph["contiguous"] * 1e3, 2),
            "pool_vs_contiguous_pct": round((graph["paged"] / graph["contiguous"] - 1) * 100, 3),
            "steps_per_graph": graph["steps_per_graph"]},
        "stages_us": {"route_align": round(route_us, 2), "gate_up": round(stage_us[0], 2),
                      "down": round(stage_us[1], 2),
                      # the decode form combines inside its down launch: no stage of its own
                      "combine": None if decode_form else round(stage_us[2], 2)},
        "roofline": roof,
    }
    extra = {}
    if not full:
        for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "dtype", "data"):
            line.pop(k)
        for c in copies:
            c["h"].close()
            c["h_same"].close()
        return line, extra

    # ---- load-buffer fill (host link) and its effect on compute
    loadbuf = None
    if s.loadbuf_slots and not args.no_fill:
        copy = torch.cuda.Stream()
        hc = copies[0]["h"]
        blobs = [dev.host_blobs[k] for k in slots]
        nbytes = len(slots) * 3 * fd * 2
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        pm.moe_loadbuf_fill(hc, 1, slots, blobs, copy)
        copy.synchronize()
        f0.record(copy)
        for _ in range(reps):
            pm.moe_loadbuf_fill(hc, 1, slots, blobs, copy)
        f1.record(copy)
        copy.synchronize()
        fill_ms = f0.elapsed_time(f1) / reps
        # compute on buffer 0 while buffer 1 keeps filling
        for _ in range(max(1, int(K * ms / fill_ms) + 1)):
            pm.moe_loadbuf_fill(hc, 1, slots, blobs, copy)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            step(0)
        e1.record(stream)
        torch.cuda.synchronize()
        busy_ms = e0.elapsed_time(e1) / K
        loadbuf = {"experts_per_fill": len(slots), "bytes_per_fill": nbytes, "fill_ms": round(fill_ms, 3),
                   "h2d_gbs": round(nbytes / (fill_ms * 1e-3) / 1e9, 2),
                   "step_us_with_concurrent_fill": round(busy_ms * 1e3, 2),
                   "step_slowdown_pct": round((busy_ms / ms - 1) * 100, 2),
                   "fill_hidden_behind_one_step": fill_ms <= ms}

    # ---- per-step spread (events around every step of one more timed pass)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    spread = {q: round(float(np.percentile(per_step, p)), 2) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}
    extra = {"step_us_spread": spread, "loadbuf": loadbuf, "adjuster": adjuster_timing(s.E)}
    if roof["bound"] == "mfma":
        extra["dense_library_gemm"] = dense_library_gemm(int(rt.num_padded.item()), s.d, s.f)
    for c in copies:
        c["h"].close()
        c["h_same"].close()
    return line, extra


def allocator_placed(layer):
    """The layer with its pool experts placed by the page allocator during a seeded
    serving churn (KV pages of f*d*2 / kv_pages_per_hole bytes, else 64 KiB)."""
    import numpy as np

    import paged_expert_weight_amd as pm
    from paged_expert_weight_amd import placement
    from workloads import churn, synth
    s = layer.spec
    locs0 = layer.placement.locs
    slots = {e: int(locs0[e]["idx"][0]) for e in range(s.E_tot) if locs0[e]["kind"] == synth.LOC_LOADBUF}
    pool_experts = [e for e in range(s.E_tot) if e not in slots]
    e_bytes = s.f * s.d * 2
    kv_bytes = e_bytes // s.kv_pages_per_hole if s.kv_pages_per_hole else 64 * 1024
    alloc = pm.PageAllocator(s.pool_pages * e_bytes, e_bytes, kv_bytes)
    spare = s.pool_pages - 3 * len(pool_experts)
    r = placement.replay(alloc, pool_experts, churn.events(s.seed, len(pool_experts), 300,
                                                           arrivals=max(1.0, spare / 8.0)))
    locs = placement.location_table(s.E_tot, r["pages"], slots)
    per = e_bytes // kv_bytes
    holes = sorted({q // per for v in r["kv"].values() for q in v})
    used = sorted(p for v in r["pages"].values() for p in v)
    free = sorted(set(range(s.pool_pages)) - set(used) - set(holes))
    pl = synth.Placement(locs, np.asarray(used, np.int64), np.asarray(holes, np.int64), np.asarray(free, np.int64),
                         layer.placement.slot_expert)
    runs = 1 + sum(1 for a, b in zip(used, used[1:]) if b != a + 1)
    print(f"# allocator placement: expert pages in {runs} runs, {len(holes)} pages split into KV pages",
          file=sys.stderr, flush=True)
    return synth.Layer(s, layer.x, layer.logits, layer.w13, layer.w2, pl)


def allocator_bench(args):
    """The page allocator under a serving churn on a 64 GiB pool of 2 MiB expert
    pages (Qwen3-Next-shaped: f=512, d=2048) and 32 KiB KV pages (16 tokens):
    host microseconds per call through the C ABI, and the space that KV pages
    trap inside expert pages, with and without same-request packing."""
    import numpy as np

    import paged_expert_weight_amd as pm
    from workloads import churn

    e_bytes, kv_bytes = 512 * 2048 * 2, 32 * 1024
    n_pages = 32768
    n_experts = 6000  # 18 000 expert pages resident at the start
    ev = churn.events(7, n_experts, 4000, arrivals=12.0, mean_life=60.0, evict_rate=0.5)
    out = {}
    for packing in (True, False):
        a = pm.PageAllocator(n_pages * e_bytes, e_bytes, kv_bytes, packing=packing)
        pages = {e: a.alloc_expert(3) for e in range(n_experts)}
        kv = {}
        trapped, avail = [], []
        calls = 0
        t_alloc = t_free = 0.0
        n_kv_pages = 0
        n_alloc_calls = 0
        refused = 0
        for i, e in enumerate(ev):
            t0 = time.perf_counter()
            if e[0] == "req" or (e[0] == "grow" and e[1] in kv):
                try:
                    got = a.alloc_small(pm.MOE_PAGE_KV, e[1], e[2])
                    kv[e[1]] = kv.get(e[1], []) + got
                    n_kv_pages += e[2]
                    n_alloc_calls += 1
                except pm.MoeError:
                    refused += 1
                t_alloc += time.perf_counter() - t0
            elif e[0] == "done":
                if kv.pop(e[1], None) is not None:
                    a.free_request(e[1])
                t_free += time.perf_counter() - t0
            elif e[0] == "evict" and e[1] in pages:
                a.free_expert(pages.pop(e[1]))
            elif e[0] == "add" and e[1] not in pages:
                try:
                    pages[e[1]] = a.alloc_expert(3)
                except pm.MoeError:
                    pass
            calls += 1
            if i % 50 == 0:
                st = a.stats()
                trapped.append(st["trapped_bytes"])
                avail.append(st["expert_available"])
        st = a.stats()
        n_done = sum(1 for e in ev if e[0] == "done")
        out["packing" if packing else "no_packing"] = {
            "mean_trapped_mib": round(float(np.mean(trapped)) / 2**20, 1),
            "max_trapped_mib": round(float(np.max(trapped)) / 2**20, 1),
            "mean_expert_pages_available": round(float(np.mean(avail)), 1),
            "refused_requests": refused,
            "us_per_alloc_call": round(t_alloc / max(1, n_alloc_calls) * 1e6, 2),
            "us_per_kv_page": round(t_alloc / max(1, n_kv_pages) * 1e6, 3),
            "us_per_request_free": round(t_free / max(1, n_done) * 1e6, 2),
            "final_split_pages": st["split"][0],
        }
        print(f"# packing={packing}: {out['packing' if packing else 'no_packing']}", file=sys.stderr, flush=True)
        a.close()
    line = {"metric": "three-tier page allocator: host us per call and trapped KV space under churn",
            "value": out["packing"]["us_per_kv_page"], "unit": "us/KV page", "higher_is_better": False,
            "n_gpus": 0, "data": "synthetic",
            "config": {"workload": "64 GiB pool of 2 MiB expert pages, 32 KiB KV pages (16 tokens); 6000 experts "
                                   "resident at the start; 4000 decode steps; log-normal prompt lengths (median "
                                   "300 tokens), one more KV page per 16 generated tokens, random expert evictions "
                                   "and re-adds", "events": len(ev)},
            "results": out}
    print(json.dumps(line), flush=True)


def vmm_bench(args):
    """One layer on physical pages that are mapped twice: into the pool view the
    paged kernels read through the location table, and into remapped expert
    views the contiguous kernels read unchanged.  Times route + forward for the
    paged path, the remapped views and the contiguous twin on ordinary
    allocations (interleaved, second round reported), and the cost of
    remapping."""
    import ctypes

    import numpy as np
    import torch

    import paged_expert_weight_amd as pm
    from workloads import synth

    name = args.workload
    s = synth.SPECS[name]
    T = args.T if args.T is not None else (32 if name == "decode" else s.T)
    layer = synth.make_layer(s, T)
    P, fd = s.f * s.d * 2, s.f * s.d
    try:
        ev = pm.ExpertViews(P, s.pool_pages, s.loadbuf_slots, s.E_tot)
    except pm.MoeError as e:
        print(json.dumps({"metric": "remapped expert views", "error": str(e), "workload": name}), flush=True)
        return
    gmin, grec = ev.granularity()
    v = ev.views()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemsetD16.argtypes = [ctypes.c_void_p, ctypes.c_uint16, ctypes.c_size_t]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    w13, w2, x = dev(layer.w13), dev(layer.w2), dev(layer.x)
    logits = torch.from_numpy(layer.logits).cuda()
    torch.cuda.synchronize()
    assert hip.hipMemsetD16(v["pool"], 0x7FC0, s.pool_pages * fd) == 0
    locs = layer.placement.locs.copy()

    def write(e, pages):
        for m, p in enumerate(pages):
            src = w13[e, m * s.f:(m + 1) * s.f] if m < 2 else w2[e]
            assert hip.hipMemcpy(v["pool"] + int(p) * P, src.data_ptr(), P, 3) == 0

    for e in range(s.E_tot):
        if locs[e]["kind"] == synth.LOC_POOL:
            write(e, locs[e]["idx"])
    pool = pm.moe_pool_create(v["pool"], s.pool_pages, s.d, s.f, s.E, s.k, s.S, s.loadbuf_slots,
                              (v["loadbuf0"], v["loadbuf1"]))
    pm.moe_set_expert_locs(pool, locs)
    blobs = {}
    for e in range(s.E_tot):
        b = torch.empty(3 * fd, dtype=torch.bfloat16, pin_memory=True)
        b.view(torch.int16).copy_(torch.from_numpy(synth.expert_blob(s, layer.w13, layer.w2, e).view(np.int16)))
        blobs[e] = b

    def fill(buf):
        lb = [e for e in range(s.E_tot) if locs[e]["kind"] == synth.LOC_LOADBUF]
        if lb:
            pm.moe_loadbuf_fill(pool, buf, [int(locs[e]["idx"][0]) for e in lb], [blobs[e] for e in lb])
        torch.cuda.synchronize()

    fill(0)
    t0 = time.perf_counter()
    n_first = ev.map_experts(locs, 0)
    first_ms = (time.perf_counter() - t0) * 1e3
    bm = args.block_m or pm.moe_suggest_block_m(pool, T)
    ws = pm.workspace(pool, T, bm)
    rt = pm.RouteOut(pool, T, bm)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    wv = ev.views()

    def step(mode):
        pm.moe_route(pool, logits, bm, rt.topk_ids, rt.topk_w, rt.sorted_ids, rt.block_expert, rt.num_padded, ws,
                     stream)
        if mode == "paged":
            pm.moe_paged_forward(pool, x, bm, rt.topk_ids, rt.topk_w, rt.sorted_ids, rt.block_expert,
                                 rt.num_padded, 0, y, ws, 0, stream)
        elif mode == "vmm":
            ev.forward(pool, x, rt, ws, y=y, stream=stream)
        else:
            pm.moe_contiguous_forward(pool, w13, w2, x, bm, rt.topk_ids, rt.topk_w, rt.sorted_ids,
                                      rt.block_expert, rt.num_padded, y, ws, 0, stream)

    def timed(mode, K, W):
        for _ in range(W):
            step(mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            step(mode)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K * 1e3

    outs = {}
    for mode in ("paged", "vmm", "contiguous"):
        step(mode)
        torch.cuda.synchronize()
        outs[mode] = y.view(torch.int16).cpu().numpy().copy()
    identical = bool(np.array_equal(outs["paged"], outs["vmm"]) and np.array_equal(outs["vmm"], outs["contiguous"]))
    us = {}
    for rnd in range(2):
        for mode in ("paged", "vmm", "contiguous"):
            us[mode] = round(timed(mode, args.steps, args.warmup), 2)
            print(f"# round {rnd} {mode}: {us[mode]} us/step", file=sys.stderr, flush=True)
    # remap costs: one expert evicted into a free slot and one cached in free pages; a buffer swap
    remap = {"first_full_map_ms": round(first_ms, 2), "first_full_map_pages": n_first}
    pool_e = [e for e in range(s.E) if locs[e]["kind"] == synth.LOC_POOL]
    lb_e = [e for e in range(s.E) if locs[e]["kind"] == synth.LOC_LOADBUF]
    used = {int(p) for e in range(s.E_tot) if locs[e]["kind"] == synth.LOC_POOL for p in locs[e]["idx"]}
    free = [p for p in range(s.pool_pages) if p not in used]
    if pool_e and lb_e and len(free) >= 3:
        ev_e, add_e = pool_e[0], lb_e[0]
        slot = int(locs[add_e]["idx"][0])
        locs[add_e]["kind"] = synth.LOC_POOL
        locs[add_e]["idx"] = free[:3]
        write(add_e, free[:3])
        locs[ev_e]["kind"] = synth.LOC_LOADBUF
        locs[ev_e]["idx"] = (slot, 0, 0)
        fill(0)
        t0 = time.perf_counter()
        n = ev.map_experts(locs, 0)
        remap["evict_and_add_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
        remap["evict_and_add_pages"] = n
    if s.loadbuf_slots:
        fill(1)
        t0 = time.perf_counter()
        n = ev.map_experts(locs, 1)
        remap["buffer_swap_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
        remap["buffer_swap_pages"] = n
    # two experts trade pages (timing only: no forward runs on this table)
    pe = [e for e in range(s.E_tot) if locs[e]["kind"] == synth.LOC_POOL]
    if len(pe) >= 2:
        a, b = pe[0], pe[1]
        ia, ib = locs[a]["idx"].copy(), locs[b]["idx"].copy()
        locs[a]["idx"], locs[b]["idx"] = ib, ia
        t0 = time.perf_counter()
        n = ev.map_experts(locs, 1 if s.loadbuf_slots else 0)
        remap["swap_two_experts_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
        remap["swap_two_experts_pages"] = n
    line = {"metric": "remapped expert views (PagedTensor) vs in-kernel page lookup, us per step",
            "value": us["vmm"], "unit": "us/step", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": WORKLOAD_TEXT[name], "name": name, "T": T, "block_m": bm,
                       "page_bytes": P, "granularity": {"minimum": gmin, "recommended": grec}},
            "us_per_step": us,
            "vs_contiguous_pct": {m: round((us[m] / us["contiguous"] - 1) * 100, 2) for m in ("paged", "vmm")},
            "outputs_bit_identical": identical,
            "remap": remap}
    print(json.dumps(line), flush=True)
    pool.close()
    ev.close()


def pipeline_bench(args):
    """An L-layer pass of Qwen1.5-MoE-shaped layers over one shared pool: every
    layer keeps E - n experts in its own pool pages and takes n through the
    alternating load buffers, filled from pinned host memory on a copy stream.
    Timed four ways, passes back to back with the host at most one pass ahead:
    overlapped (prefetch of layer l + 1 issued ahead of the forward of layer
    l), serialized (each fill waits for the previous forward), fills alone and
    forwards alone; plus a pass in which every layer switches tables (the
    copy-before-switch wait and the table upload), one pass at a time from an
    idle GPU, and the host cost of each call."""
    import numpy as np
    import torch

    import paged_expert_weight_amd as pm
    from workloads import device as wdev
    from workloads import synth

    pm.lib()
    L, n_lb = args.layers, args.offloaded
    T = args.T or 1024
    base = synth.SPECS["qwen15"]
    E = base.E
    s = synth.spec("qwen15", T=max(T, base.T), pool_pages=3 * (E - n_lb),
                   loadbuf_experts=tuple(range(E - n_lb, E)), loadbuf_slots=n_lb)
    t0 = time.time()
    layer = synth.make_layer(s, T)
    dev = wdev.to_device(layer)
    print(f"# layer generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    Pl = s.pool_pages
    fd = s.f * s.d
    pool = torch.empty((L * Pl, fd), dtype=torch.bfloat16, device="cuda")
    for l in range(L):
        pool[l * Pl:(l + 1) * Pl].copy_(dev.pool)  # every layer reads pages of its own
    del dev.pool
    lbuf = tuple(dev.loadbuf)
    slots = sorted(dev.host_blobs)
    blobs = [dev.host_blobs[k] for k in slots]
    tables = []
    hs = []
    for l in range(L):
        t = layer.placement.locs.copy()
        for e in range(s.E_tot):
            if t[e]["kind"] == synth.LOC_POOL:
                t[e]["idx"] = t[e]["idx"] + l * Pl
        tables.append(t)
        h = pm.moe_pool_create(pool, L * Pl, s.d, s.f, s.E, s.k, s.S, n_lb, lbuf)
        pm.moe_set_expert_locs(h, t)
        pm.moe_loadbuf_fill(h, l % 2, slots, blobs)  # for the forwards-alone timing
        hs.append(h)
    torch.cuda.synchronize()
    bm = pm.moe_suggest_block_m(hs[0], T)
    ws = pm.workspace(hs[0], T, bm)
    r = pm.route(hs[0], dev.logits, bm, ws)
    y = torch.empty_like(dev.x)
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    pipe = pm.MoePipeline(hs, copy)

    def fwd(l):
        pipe.forward(l, dev.x, r, ws, y=y, stream=comp)

    def pass_overlapped():
        pipe.prefetch(0, slots, blobs)
        for l in range(L):
            if l + 1 < L:
                pipe.prefetch(l + 1, slots, blobs)
            fwd(l)

    def pass_serialized():
        for l in range(L):
            copy.wait_stream(comp)
            pipe.prefetch(l, slots, blobs)
            fwd(l)

    def pass_fills():
        for l in range(L):
            pm.moe_loadbuf_fill(hs[l], l % 2, slots, blobs, copy)

    def pass_forwards():
        for l in range(L):
            pm.moe_paged_forward(hs[l], dev.x, bm, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert,
                                 r.num_padded, l % 2, y, ws, 0, comp)

    def pass_switch():
        for l in range(L):
            pipe.stage_table(l, tables[l])
        pass_overlapped()

    def bounded(fn, n):
        """n passes back to back, the host at most one pass ahead of the GPU (as a
        serving loop that enqueues the next step while the current one runs)."""
        prev = None
        for _ in range(n):
            if prev is not None:
                prev[0].synchronize()
                prev[1].synchronize()
            e = (torch.cuda.Event(), torch.cuda.Event())
            e[0].record(comp)
            e[1].record(copy)
            fn()
            prev = e

    def timed(fn, K, W):
        bounded(fn, W)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        copy.wait_stream(comp)
        bounded(fn, K)
        comp.wait_stream(copy)
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K * 1e3

    def isolated(fn, K):
        """One pass at a time from an idle GPU, start of the first copy or kernel to the end of the last."""
        tot = 0.0
        for _ in range(K):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(comp)
            copy.wait_stream(comp)
            fn()
            comp.wait_stream(copy)
            e1.record(comp)
            e1.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / K * 1e3

    K, W = max(1, args.steps // 2), max(2, args.warmup // 2)
    us = {}
    # two interleaved rounds; the second (warm) one is reported
    for rnd in range(2):
        for key, fn in (("overlapped", pass_overlapped), ("serialized", pass_serialized),
                        ("fills_alone", pass_fills), ("forwards_alone", pass_forwards),
                        ("overlapped_with_table_switch", pass_switch)):
            us[key] = round(timed(fn, K, W), 1)
            print(f"# round {rnd} {key}: {us[key]} us/pass", file=sys.stderr, flush=True)
        us["isolated_overlapped"] = round(isolated(pass_overlapped, K), 1)
        print(f"# round {rnd} isolated_overlapped: {us['isolated_overlapped']} us/pass", file=sys.stderr, flush=True)
    # host cost per call (enqueue only)
    torch.cuda.synchronize()
    reps = 200
    t0 = time.perf_counter()
    for i in range(reps):
        pm.moe_paged_forward(hs[0], dev.x, bm, r.topk_ids, r.topk_w, r.sorted_ids, r.block_expert, r.num_padded, 0,
                             y, ws, 0, comp)
    plain_us = (time.perf_counter() - t0) / reps * 1e6
    torch.cuda.synchronize()
    pipe.prefetch(0, slots, blobs)
    t0 = time.perf_counter()
    for i in range(reps):
        fwd(0)
    pipe_us = (time.perf_counter() - t0) / reps * 1e6
    torch.cuda.synchronize()
    copy_l = us["fills_alone"] / L
    comp_l = us["forwards_alone"] / L
    # back to back, the first fill of a pass overlaps the end of the previous one
    ideal = L * max(copy_l, comp_l)
    ideal_iso = L * max(copy_l, comp_l) + min(copy_l, comp_l)
    hideable = us["serialized"] - ideal
    nbytes = n_lb * 3 * fd * 2
    line = {
        "metric": "multi-layer pipeline pass time (us)",
        "value": us["overlapped"],
        "unit": "us/pass",
        "higher_is_better": False,
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{L} Qwen1.5-MoE-shaped layers (d=2048 f=1408 E=60 top-4) over one pool, "
                               f"{n_lb} expert(s) per layer via the alternating load buffers",
                   "layers": L, "T": T, "block_m": bm, "offloaded_per_layer": n_lb,
                   "fill_bytes_per_layer": nbytes},
        "pass_us": us,
        "per_layer_us": {"fill": round(copy_l, 1), "forward": round(comp_l, 1)},
        "h2d_gbs": round(nbytes / (copy_l * 1e-6) / 1e9, 2),
        "ideal_us": {"overlapped": round(ideal, 1), "isolated_overlapped": round(ideal_iso, 1)},
        "frac_of_ideal": {"overlapped": round(ideal / us["overlapped"], 3),
                          "isolated_overlapped": round(ideal_iso / us["isolated_overlapped"], 3)},
        "overlap_efficiency": round((us["serialized"] - us["overlapped"]) / hideable, 3) if hideable > 0 else None,
        "table_switch_cost_us_per_layer": round((us["overlapped_with_table_switch"] - us["overlapped"]) / L, 2),
        "host_us_per_call": {"moe_paged_forward": round(plain_us, 2), "moe_pipeline_forward": round(pipe_us, 2)},
    }
    print(json.dumps(line), flush=True)
    pipe.close()
    for h in hs:
        h.close()


GRAPH_MAX_T = 512  # batches whose graph-replayed step is reported


def graph_timed(step, R, K, W, stream):
    """Per-step time of `step` captured in one HIP graph (a whole number of rotations of the layer
    copies, about 20 steps) and replayed, for the paged path over the layer's pool and for the
    contiguous twin, in alternating blocks of replays."""
    import torch
    G = R * max(1, math.ceil(20 / R))
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graphs = {}
    for mode in ("paged", "contiguous"):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
            for i in range(G):
                step(i, mode, side)
        graphs[mode] = g
    torch.cuda.synchronize()
    reps = max(1, math.ceil(K / G))
    out = {"paged": 0.0, "contiguous": 0.0, "steps_per_graph": G}
    for rnd in range(3):
        for mode in (("paged", "contiguous") if rnd % 2 == 0 else ("contiguous", "paged")):
            g = graphs[mode]
            for _ in range(max(1, math.ceil(W / G))):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            out[mode] += e0.elapsed_time(e1) / (reps * G) / 3
    del graphs
    torch.cuda.synchronize()
    return out


def dense_library_gemm(rows: int, d: int, f: int, reps: int = 10):
    """Context for the MFMA fraction of the grouped GEMMs: the vendor library's dense bf16 GEMM
    (torch.matmul, hipBLASLt on ROCm) on the same executed shapes, all padded rows of the aligned
    order as one dense matrix: gate/up [rows, d] x [d, 2f], down [rows, f] x [f, d]."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    out = {"rows": rows}
    for name, (m, k, n) in (("gate_up", (rows, d, 2 * f)), ("down", (rows, f, d))):
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16, generator=g).contiguous()
        c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, b, out=c)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        out[f"{name}_us"] = round(ms * 1e3, 1)
        out[f"{name}_mfma_frac"] = round(2.0 * m * k * n / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        del a, b, c
    torch.cuda.empty_cache()
    return out


def adjuster_timing(E: int, layers: int = 48, rounds: int = 2000):
    """Host cost of one adjuster round (amounts + selection) for a model of `layers`
    MoE layers of E experts: grows of 5 and shrinks of 3 alternating."""
    import numpy as np
    import paged_expert_weight_amd as pm
    g = np.random.default_rng(0)
    ranking = np.stack([g.permutation(E) for _ in range(layers)]).astype(np.int32)
    prob = -np.sort(-g.random((layers, E)).astype(np.float32), axis=1)
    resident = [E // 2] * layers
    t0 = time.perf_counter()
    for r in range(rounds):
        ev, add = pm.adjust_amounts(8 if r % 2 else 0, 0 if r % 2 else 24)
        _, resident = pm.adjust_select(ranking, prob, resident, E, ev, add)
    us = (time.perf_counter() - t0) / rounds * 1e6
    return {"layers": layers, "experts": E, "us_per_round": round(us, 2),
            "note": "host-side policy incl. Python marshalling of the C calls"}


def cpu_baseline(layer, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle

    s = layer.spec
    T = layer.T
    per_tok = 6.0 * s.d * s.f * s.k_eff
    t = time.time()
    ids, w = oracle.route(layer.logits, s.k, s.S)
    oracle.align(ids, s.E_tot, 64)
    route_s = time.time() - t
    # probe the rate on a few tokens, then size the sample to ~`seconds`
    probe = list(range(min(T, 8)))
    t = time.time()
    oracle.moe(layer.x, layer.w13, layer.w2, ids, w, tokens=probe)
    rate = len(probe) * per_tok / max(1e-6, time.time() - t)
    ntok = int(max(1, min(T, seconds * rate / per_tok)))
    toks = np.linspace(0, T - 1, ntok).astype(np.int64)
    done, flops, t = 0, 0.0, time.time()
    while True:
        oracle.moe(layer.x, layer.w13, layer.w2, ids, w, tokens=toks)
        done += 1
        flops += ntok * per_tok
        if time.time() - t >= seconds * 0.8 or done >= 50:
            break
    el = time.time() - t + route_s
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"routing + alignment of all {T} tokens, then the per-token expert sum for {ntok} of "
                      f"the {T} tokens (evenly spaced) x{done}; {el:.1f} s of CPU work in fp64"}


if __name__ == "__main__":
    main()
