#!/usr/bin/env python3
"""MoE FFN layer benchmark on one MI355X.

A step is one pass of the whole layer -- top-k routing, Align & Sort, the
grouped SwiGLU FFN (gate/up, down) and the weighted combine -- over one batch
of seeded synthetic input already resident in HBM.  The default workload is the
one-GPU expert-parallel prefill share: 2048 tokens, each routed to one of 32
local experts (64 per expert), hidden 7168, expert intermediate 2048, bf16,
block_size_m 64.

Prints ONE JSON line.  `value` is layer tokens/s; per-kernel durations come
from HIP events recorded on the launch stream around every kernel inside the
timed steps; `roofline` is for the dominant kernel (the gate/up GEMM);
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload prefill_bf16] [--B 64]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                                   # MI355X HBM3E
# dense matrix-core peaks; E4M3 x E2M1 products run on the f8f6f4 instruction
# with an E4M3 operand and are priced at the fp8 peak
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0, "e2m1": 5000.0, "f32": 157.3}
ESZ = {"f32": 4, "bf16": 2, "e4m3": 1, "e2m1": 0.5}
DTYPE_NAME = {"f32": "f32", "bf16": "bf16", "e4m3": "fp8_e4m3", "e2m1": "fp8_e4m3 x mxfp4"}
PROFILE_DIR = os.path.join(ROOT, "profiles")
NUM_XCD = 8                                             # XCDs of an MI355X (one GRBM instance each)


def layer_flops(slots: int, hidden: int, inter: int) -> int:
    """Useful FLOPs of the expert FFN for ``slots`` routed token slots:
    gate+up is a [slots,H]x[H,2I] GEMM (2*H*2I flops per slot) and down a
    [slots,I]x[I,H] GEMM (2*I*H per slot): 6*H*I per slot."""
    return 6 * slots * hidden * inter


def algorithmic_bytes(cfg, ids_np, E_slabs):
    """Bytes the method itself must move per kernel (each counted once):
    gate/up: W13 of every expert hit (+ its fp32 row scales, or its E8M0
    block scales: one byte per 32 weights) and x;
    down: W2 of every expert hit (+ scales) and the fp32 y_slots rows written;
    combine: y_slots read, out written (bf16 / fp32)."""
    import numpy as np
    T, H, I = cfg["T"], cfg["H"], cfg["I"]
    dt = cfg["dtype"]
    e = ESZ[dt]
    flat = ids_np.ravel()
    hit = np.unique(flat[(flat >= 0) & (flat < E_slabs)])
    D = int(hit.size)
    S_valid = int(((flat >= 0) & (flat < E_slabs)).sum())
    xb = T * H * (4 if dt == "f32" else 2)
    # scale bytes per weight row of W13 (H long) and of W2 (I long)
    sc1 = 4 if dt == "e4m3" else H // 32 if dt == "e2m1" else 0
    sc2 = 4 if dt == "e4m3" else I // 32 if dt == "e2m1" else 0
    out_b = T * H * (4 if dt == "f32" else 2)
    return {
        "experts_hit": D,
        "stage1": int(D * 2 * I * H * e) + D * 2 * I * sc1 + xb,
        "stage2": int(D * H * I * e) + D * H * sc2 + S_valid * H * 4,
        "combine": S_valid * H * 4 + out_b,
        "weights": int(D * 3 * I * H * e) + D * (2 * I * sc1 + H * sc2),
        "slots": S_valid,
    }


def _mean(v):
    return sum(v) / len(v) if v else 0.0


def run_layer_timed(cfg, B, steps, warmup, dev, seed=0, rows="by_token", rotate=1, graph=True,
                    schedule="two_launch", slot_rows="fp32"):
    """Generate one workload, run `warmup` + `steps` layer passes with events
    around every kernel; return timings and what the roofline needs.
    rows="sorted": the layer permutes the token rows into the sorted order
    first and combines back through the inverse map.
    rotate > 1: that many distinct input sets (x, logits; seeds seed..) are
    resident and step s uses set s % rotate, so no step reads the input the
    previous step just read (a fresh activation per layer, as in a model)."""
    import torch

    import moe_synth as ms
    import routing_align_sort_amd as moe

    L = ms.make_layer(cfg, device=dev, seed=seed)
    w13, w2, s13, s2 = L["w13"], L["w2"], L.get("w13_scale"), L.get("w2_scale")
    if cfg["dtype"] == "e2m1":          # generator bytes -> the binding's MXFP4 dtypes
        w13, w2, s13, s2 = w13.view(moe.FP4), w2.view(moe.FP4), s13.view(moe.E8M0), s2.view(moe.E8M0)
    layer = moe.MoELayer(w13, w2, T=cfg["T"], K=cfg["K"], B=B, score=cfg["score"],
                         n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                         renormalize=cfg["renormalize"], shared=bool(cfg.get("shared")),
                         w13_scale=s13, w2_scale=s2,
                         x_dtype=L["x"].dtype,
                         out_dtype=torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16,
                         rows=rows, schedule=schedule,
                         slot_dtype=torch.bfloat16 if slot_rows == "bf16" else torch.float32)
    x, logits, bias = L["x"], L["logits"], L["bias"]
    inputs = [(x, logits)]
    for j in range(1, rotate):
        Lj = ms.make_layer(cfg, device=dev, seed=seed + j, weights=False)
        inputs.append((Lj["x"], Lj["logits"]))
    for s in range(warmup):
        layer.forward(*inputs[s % rotate], bias)
    torch.cuda.synchronize()
    # 1. the layer as a caller runs it: the four calls back to back, nothing
    #    else on the stream; wall clock between device synchronisations
    t0 = time.perf_counter()
    for s in range(steps):
        layer.forward(*inputs[s % rotate], bias)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # a top-1 layer runs its FFN and combine as one call; the same steps with
    # the two calls apart, for comparison
    wall_sep = float("nan")
    if layer.top1:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            xs, ls = inputs[s % rotate]
            layer.route(ls, bias)
            layer.align()
            layer.ffn(xs)
            layer.combine()
        torch.cuda.synchronize()
        wall_sep = time.perf_counter() - t0
    # with E4M3 / MXFP4 weights the forward routes and quantises x in one
    # launch; the same steps with the quantisation inside the FFN call
    wall_quant_in_ffn = float("nan")
    if layer.route_quant:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            xs, ls = inputs[s % rotate]
            layer.route(ls, bias)
            layer.align()
            if layer.top1:
                layer.ffn_top1(xs)
            else:
                layer.ffn(xs)
                layer.combine()
        torch.cuda.synchronize()
        wall_quant_in_ffn = time.perf_counter() - t0
    # 2. the same four calls captured once in a HIP graph and replayed
    wall_graph = float("nan")
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(x, logits, bias)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        wall_graph = time.perf_counter() - t0
        del g
    # 3. per-stage durations: events around every kernel (each event adds a
    #    few us of stream time, so these steps are not the wall-clock figure)
    NE = 9
    ev = moe.HipEvents(NE * max(steps, 1))
    torch.cuda.synchronize()
    for s in range(steps):
        b = NE * s
        xs, ls = inputs[s % rotate]
        ev.record(b + 0)
        layer.route(ls, bias)
        ev.record(b + 1)
        layer.align()
        ev.record(b + 2)
        if layer.rows_sorted:
            layer.permute(xs)
        layer.ffn(xs, stage_events=ev.handles[b + 3:b + 8])
        layer.combine()
        ev.record(b + 8)
    torch.cuda.synchronize()
    names = ["route", "align", "permute" if layer.rows_sorted else None, "quant", "gate_up", "requant",
             "down", "combine"]
    per = {n: [] for n in names if n}
    total = []
    for s in range(steps):
        b = NE * s
        for i, n in enumerate(names):
            if n:
                per[n].append(ev.elapsed_ms(b + i, b + i + 1) * 1e3)
        total.append(ev.elapsed_ms(b, b + 8) * 1e3)
    ev.close()
    ids_np = layer.topk_ids.cpu().numpy()
    res = {
        "wall_s": wall,
        "wall_sep_s": wall_sep,
        "wall_quant_in_ffn_s": wall_quant_in_ffn,
        "wall_graph_s": wall_graph,
        "us": {n: _mean(v) for n, v in per.items()},
        "us_step_events": _mean(total),
        "P": int(layer.ntpp.item()),
        "ids": ids_np,
        "weights_np": layer.topk_weights.cpu().numpy(),
        "E_slabs": layer.E_slabs,
        "L": L,
        "layer": layer,
        "steps": steps,
    }
    return res


def summarize(cfg, B, r):
    ab = algorithmic_bytes(cfg, r["ids"], r["E_slabs"])
    us = r["us"]
    flops = layer_flops(ab["slots"], cfg["H"], cfg["I"])
    gemm_us = us["gate_up"] + us["down"]
    dt = cfg["dtype"]
    steps = r["steps"]
    return {
        "block_size_m": B,
        "tokens_per_s": cfg["T"] * steps / r["wall_s"],
        "us_per_step": r["wall_s"] / steps * 1e6,
        "graph_us_per_step": r["wall_graph_s"] / steps * 1e6 if r["wall_graph_s"] == r["wall_graph_s"] else None,
        "us_per_step_ffn_then_combine": (r["wall_sep_s"] / steps * 1e6 if r["wall_sep_s"] == r["wall_sep_s"]
                                         else None),
        # E4M3 / MXFP4: the steps with the activation quantisation in the FFN
        # call instead of in the routing launch
        "us_per_step_quant_in_ffn": (r["wall_quant_in_ffn_s"] / steps * 1e6
                                     if r["wall_quant_in_ffn_s"] == r["wall_quant_in_ffn_s"] else None),
        "event_timed_us_per_step": r["us_step_events"],
        "us": {k: round(v, 2) for k, v in us.items()},
        "experts_hit": ab["experts_hit"],
        "num_tokens_post_padded": r["P"],
        "grouped_gemm_tflops": flops / (gemm_us * 1e-6) / 1e12,
        "grouped_gemm_mfma_frac": flops / (gemm_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS[dt],
        "gate_up_hbm_gbs": ab["stage1"] / (us["gate_up"] * 1e-6) / 1e9,
        "down_hbm_gbs": ab["stage2"] / (us["down"] * 1e-6) / 1e9,
        "weights_gb": ab["weights"] / 1e9,
        "layer_weight_stream_frac": ab["weights"] / (r["wall_s"] / steps) / 1e9 / HBM_PEAK_GBS,
    }


_SPIN = {}


def _spin_cycles(dev, target_ms=3.0):
    """Argument of torch.cuda._sleep that keeps the GPU busy for ~target_ms."""
    import torch

    import routing_align_sort_amd as moe

    if dev not in _SPIN:
        ev = moe.HipEvents(2)
        n = 1 << 20
        torch.cuda.synchronize()
        ev.record(0)
        torch.cuda._sleep(n)
        ev.record(1)
        torch.cuda.synchronize()
        ms = max(ev.elapsed_ms(0, 1), 1e-3)
        ev.close()
        _SPIN[dev] = int(n * target_ms / ms)
    return _SPIN[dev]


def align_timed(dev, T, iters=200, cold=False, K=8, E=256, B=64, zipf_s=1.1):
    """Align & Sort alone on T tokens x top-K of E experts (Zipf), event-timed
    per call.  cold=True rewrites a 512 MB buffer between calls so that the
    ids and outputs are not in L2 or the infinity cache."""
    import numpy as np
    import torch

    import moe_synth as ms
    import routing_align_sort_amd as moe

    ids_np = ms.zipf_topk_ids(0, ms.TAG_IDS, T, K, E, zipf_s)
    ids = torch.from_numpy(ids_np).to(dev)
    ws_b = moe.moe_align_sort_workspace_bytes(T, K, E, B)
    ws = torch.zeros(max(ws_b, 1), dtype=torch.uint8, device=dev)   # zero before first use
    out = moe.moe_align_sort(ids, E, B, workspace=ws)            # allocates the outputs once
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold else None
    ev = moe.HipEvents(2 * iters)
    for _ in range(10):
        moe.moe_align_sort(ids, E, B, workspace=ws, **out)
    torch.cuda.synchronize()
    # A GPU-side spin ahead of every batch lets the host queue the batch
    # before the GPU reaches it, so the events time the kernels and not the
    # host's launch latency.
    spin = _spin_cycles(dev)
    batch = 20
    for i in range(iters):
        if i % batch == 0:
            torch.cuda._sleep(spin)
        if cold:
            scrub.fill_(i & 0xFF)
        ev.record(2 * i)
        moe.moe_align_sort(ids, E, B, workspace=ws, **out)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    t = sorted(ev.elapsed_ms(2 * i, 2 * i + 1) * 1e3 for i in range(iters))
    ev.close()
    P = int(out["num_tokens_post_padded"].item())
    S = ids_np.size
    C = out["sorted_token_ids"].numel()
    # algorithmic bytes: ids read, sorted_token_ids written to capacity, expert_ids written
    nbytes = 4 * S + 4 * C + 4 * (C // B)
    med = t[len(t) // 2]
    del scrub
    return {"tokens": T, "cold": cold, "us_median": round(med, 2), "us_p10": round(t[len(t) // 10], 2),
            "us_p90": round(t[9 * len(t) // 10], 2), "num_tokens_post_padded": P,
            "algorithmic_bytes": nbytes, "gbs": round(nbytes / (med * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


ALIGN_SWEEP_T = (64, 1024, 16384, 131072, 1048576)


def align_only(dev, iters=200):
    """Align & Sort on 16384 tokens x top-8 of 256 experts (Zipf 1.1), block 64:
    warm (ids just written) and cold; plus the token-count sweep (warm)."""
    warm = align_timed(dev, 16384, iters)
    cold = align_timed(dev, 16384, iters, cold=True)
    sweep = [align_timed(dev, T, 50 if T >= 131072 else iters) for T in ALIGN_SWEEP_T]
    return {"workload": "16384 tokens x top-8 of 256 experts, Zipf(1.1), block_size_m 64",
            "us_median": warm["us_median"], "us_p10": warm["us_p10"], "us_p90": warm["us_p90"],
            "num_tokens_post_padded": warm["num_tokens_post_padded"],
            "algorithmic_bytes": warm["algorithmic_bytes"], "gbs": warm["gbs"],
            "cold_us_median": cold["us_median"],
            "sweep": [{k: r[k] for k in ("tokens", "us_median", "gbs", "hbm_frac")} for r in sweep]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--B", type=int, default=None)
    ap.add_argument("--rows", default="by_token", choices=("by_token", "sorted"),
                    help="sorted: permute the token rows into the sorted order before the FFN "
                         "and combine back through the inverse map")
    ap.add_argument("--schedule", default="two_launch", choices=("two_launch", "fused"),
                    help="fused: both GEMMs in one persistent launch")
    ap.add_argument("--slot-rows", default="fp32", choices=("fp32", "bf16"),
                    help="type of the slot rows between the FFN and the combine (layers with a combine)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the align-only and secondary-workload figures")
    ap.add_argument("--align-only", action="store_true",
                    help="time Align & Sort alone (16k tokens warm / cold and the token-count sweep), "
                         "print its JSON and exit")
    ap.add_argument("--backward-only", action="store_true",
                    help="time the training backward of the prefill bf16 layer, print its JSON and exit")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates rocprofv3 byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-probe run into the traffic record under profiles/ and exit")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PMC_DIR", "OUT_JSON"),
                    help="reduce one rocprofv3 --pmc output directory to per-kernel medians of every "
                         "counter (the library's kernels and the copy probe), with per-dispatch "
                         "durations when it also holds a kernel trace, "
                         "write them as JSON and exit")
    args = ap.parse_args()
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.workload,
                           args.B or None)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the layer runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); it is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_synth as ms
    import routing_align_sort_amd as moe
    if not os.path.exists(moe.LIB_PATH):
        from routing_align_sort_amd import build as hip_build
        hip_build.build()
    moe.load_library()
    dev = torch.device("cuda:0")
    if args.align_only:
        print(json.dumps(align_only(dev)), flush=True)
        return
    if args.backward_only:
        print(json.dumps(backward_step(dev)), flush=True)
        return
    cfg = ms.CONFIGS[args.workload]
    B = args.B or cfg["B"]

    r = run_layer_timed(cfg, B, args.steps, args.warmup, dev, rows=args.rows, schedule=args.schedule,
                        slot_rows=args.slot_rows)
    summ = summarize(cfg, B, r)
    ab = algorithmic_bytes(cfg, r["ids"], r["E_slabs"])
    ms_per_step = r["wall_s"] / args.steps * 1e3
    value = cfg["T"] * args.steps / r["wall_s"]
    st1_us = r["us"]["gate_up"]
    achieved = ab["stage1"] / (st1_us * 1e-6) / 1e9
    roofline = {"kernel": "ffn_stage1 (gate/up GEMM + SiLU*up)", "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload, B),
                "algorithmic_bytes_per_launch": ab["stage1"], "avg_launch_us": round(st1_us, 2)}
    line = {
        "metric": "MoE layer tokens/s + grouped-GEMM TFLOPS (% MFMA peak); align-sort us",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[cfg["dtype"]],
        "data": "synthetic (seeded counter-based generator; random-init expert weights)",
        "config": {"workload": describe(args.workload, cfg, B), "tokens": cfg["T"],
                   "experts": cfg["E"], "top_k": cfg["K"], "hidden": cfg["H"], "inter": cfg["I"],
                   "block_size_m": B, "shared_expert": bool(cfg.get("shared")), "rows": args.rows,
                   "schedule": args.schedule, "slot_rows": args.slot_rows},
        "layer": summ,
        "roofline": roofline,
    }
    del r
    torch.cuda.empty_cache()
    if not args.no_extras:
        # the same steps over 32 rotating resident input sets (940 MB, beyond
        # the 256 MB last-level cache): no step reads an x left in that cache
        rr = run_layer_timed(cfg, B, args.steps, args.warmup, dev, rotate=32, graph=False)
        line["layer"]["us_per_step_rotating_inputs"] = round(rr["wall_s"] / args.steps * 1e6, 1)
        line["layer"]["gate_up_us_rotating_inputs"] = round(rr["us"]["gate_up"], 2)
        del rr
        torch.cuda.empty_cache()
        line["hbm_probe"] = hbm_probe(dev)
        line["mfma_probe"] = mfma_probe(dev)
        line["vendor_gemm"] = vendor_gemm(dev)
        line["align_sort_16k"] = align_only(dev)
        extra = {}
        # the HBM-bound secondary shapes at their own block size; the
        # compute-bound 512-tokens-per-expert shapes at block 128
        for name, b2 in (("prefill_fp8", None), ("prefill_fp8_uniform", None), ("decode_bf16", None),
                         ("prefill_bf16_512", 128),
                         ("prefill_fp8_512", 128), ("decode_fp4", None), ("prefill_fp4", None),
                         ("prefill_fp4_512", 128)):
            if name == args.workload:
                continue
            c2 = ms.CONFIGS[name]
            b2 = b2 or c2["B"]
            r2 = run_layer_timed(c2, b2, 10, 3, dev)
            extra[name] = {"workload": describe(name, c2, b2), **summarize(c2, b2, r2)}
            if not r2["layer"].top1:
                # the same layer with bf16 slot rows between the FFN and the combine
                del r2
                r2 = run_layer_timed(c2, b2, 10, 3, dev, graph=False, slot_rows="bf16")
                s16 = summarize(c2, b2, r2)
                extra[name]["bf16_slot_rows"] = {"us_per_step": round(s16["us_per_step"], 1),
                                                 "down_us": s16["us"]["down"], "combine_us": s16["us"]["combine"]}
            if name == "prefill_fp8_uniform":
                # the pages' figure for this shape, on another machine: context only
                extra[name]["pages_context"] = {"kernel": "aiter a8w8 fused MoE, block 32x512", "gpu": "MI300",
                                                "us": 484, "tflops": 372.7}
            del r2
            torch.cuda.empty_cache()
        line["other_workloads"] = extra
        # the headline workload at the other block sizes the pages tune over
        sweep = {}
        for b2 in (32, 64, 128):
            if b2 == B:
                sm = line["layer"]
            else:
                r2 = run_layer_timed(cfg, b2, 10, 3, dev)
                sm = summarize(cfg, b2, r2)
                del r2
                torch.cuda.empty_cache()
            sweep[str(b2)] = {"us_per_step": round(sm["us_per_step"], 1), "gate_up_us": sm["us"]["gate_up"],
                              "down_us": sm["us"]["down"], "grouped_gemm_tflops": round(sm["grouped_gemm_tflops"], 1)}
        line["block_size_sweep"] = sweep
        # the fp8 workload (Zipf routing + shared expert) over the same block
        # sizes: its heavy experts re-read their weights once per block
        if args.workload != "prefill_fp8":
            c2 = ms.CONFIGS["prefill_fp8"]
            sw8 = {}
            for b2 in (32, 64, 128):
                r2 = run_layer_timed(c2, b2, 10, 3, dev, graph=False)
                sm = summarize(c2, b2, r2)
                del r2
                torch.cuda.empty_cache()
                sw8[str(b2)] = {"us_per_step": round(sm["us_per_step"], 1), "gate_up_us": sm["us"]["gate_up"],
                                "down_us": sm["us"]["down"], "num_tokens_post_padded": sm["num_tokens_post_padded"]}
            line["block_size_sweep_prefill_fp8"] = sw8
        line["permute_path"] = permute_path(dev)
        line["ffn_input_state"] = ffn_input_state(dev)
        line["one_stage_schedule"] = one_stage(dev)
        line["backward"] = backward_step(dev)
    if args.copy_probe:
        copy_probe(dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline(cfg, B, dev)
    print(json.dumps(line), flush=True)


def permute_path(dev):
    """The layer with the token rows moved into the sorted order first (what an
    expert-parallel dispatch sends) against the layer that gathers inside the
    FFN, on the prefill bf16 and fp8 workloads, both over 32 rotating input
    sets (no step finds its input in the last-level cache): step time of both, and the permute and unpermute-combine kernels
    with their HBM rates on algorithmic bytes (permute: each placed row read
    once, each row below num_tokens_post_padded written; unpermute-combine:
    every placed row read, out written), and the unpermute-combine's gradient
    (event-timed alone, 10 calls)."""
    import torch

    import moe_synth as ms
    res = {}
    for name in ("prefill_bf16", "prefill_fp8"):
        cfg = ms.CONFIGS[name]
        B = cfg["B"]
        r = run_layer_timed(cfg, B, 16, 8, dev, rows="sorted", rotate=32, graph=False)
        layer = r["layer"]
        C, H = layer.C, layer.H
        S_valid = int((layer.sorted < layer.T * layer.KO).sum().item())
        xb = 2                                          # bf16 rows are moved in both workloads
        P = int(layer.ntpp.item())
        perm_bytes = S_valid * H * xb + P * H * xb
        unperm_bytes = S_valid * H * 4 + cfg["T"] * H * 2
        base = run_layer_timed(cfg, B, 16, 8, dev, rotate=32, graph=False)
        # the unpermute-combine's gradient on the same layout (training): each
        # placed row reads d_out's row and y_perm's row, every row below P
        # writes d_y_perm (bf16, the GEMMs' operand type)
        import routing_align_sort_amd as moe
        d_out = torch.randn((layer.T, H), dtype=torch.float32, device=dev)
        d_y = torch.empty((C, H), dtype=torch.bfloat16, device=dev)
        d_w = torch.empty((layer.T, layer.KO), dtype=torch.float32, device=dev)
        ev = moe.HipEvents(2 * 10)
        for i in range(13):
            if i >= 3:
                ev.record(2 * (i - 3))
            moe.moe_unpermute_combine_backward(d_out, layer.y_slots, layer.topk_weights, layer.topk_ids, layer.sorted,
                                               layer.ntpp, layer.E_slabs, B, d_y_perm_dtype=torch.bfloat16,
                                               d_y_perm=d_y, d_topk_weights=d_w)
            if i >= 3:
                ev.record(2 * (i - 3) + 1)
        torch.cuda.synchronize()
        ub_us = _mean([ev.elapsed_ms(2 * i, 2 * i + 1) * 1e3 for i in range(10)])
        ev.close()
        ub_bytes = S_valid * H * 4 * 2 + P * H * 2
        del d_out, d_y, d_w
        res[name] = {
            "block_size_m": B,
            "us_per_step_sorted_rows": round(r["wall_s"] / r["steps"] * 1e6, 1),
            "us_per_step_gathered_rows": round(base["wall_s"] / base["steps"] * 1e6, 1),
            "gate_up_us_sorted_rows": round(r["us"]["gate_up"], 1),
            "gate_up_us_gathered_rows": round(base["us"]["gate_up"], 1),
            "permute_us": round(r["us"]["permute"], 2),
            "permute_gbs": round(perm_bytes / (r["us"]["permute"] * 1e-6) / 1e9, 1),
            "unpermute_combine_us": round(r["us"]["combine"], 2),
            "unpermute_combine_gbs": round(unperm_bytes / (r["us"]["combine"] * 1e-6) / 1e9, 1),
            "unpermute_combine_backward_us": round(ub_us, 2),
            "unpermute_combine_backward_gbs": round(ub_bytes / (ub_us * 1e-6) / 1e9, 1),
            "stage_us": {k: round(v, 2) for k, v in r["us"].items()},
        }
        del r, base, layer
        torch.cuda.empty_cache()
    return res


def backward_step(dev, steps=10, warmup=3):
    """The training step of the headline layer (prefill bf16, 2048 tokens x 32
    experts, B 64, canonical weights).  The training forward keeps the slot
    rows and the fp32 gate/up values; the backward reads them and computes dx,
    dW13, dW2, the combine weights' and the logits' gradients.  Wall clock of
    back-to-back calls of each; the backward's useful FLOPs are data
    gradients 2SHI + 4SHI and weight gradients 2SHI + 4SHI (12SHI).  Also the
    backward that recomputes gate/up itself (16SHI with the recompute), and the
    one that writes the weight gradients in bf16."""
    import torch

    import moe_synth as ms
    import routing_align_sort_amd as moe
    cfg = ms.CONFIGS["prefill_bf16"]
    L = ms.make_layer(cfg, device=dev)
    layer = moe.MoELayer(L["w13"], L["w2"], T=cfg["T"], K=1, B=cfg["B"], score="softmax", renormalize=False,
                         train=True)
    x, logits = L["x"], L["logits"]
    d_out = torch.randn((cfg["T"], cfg["H"]), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_ffn_backward_workspace_bytes(cfg["T"], 1, cfg["E"], cfg["H"], cfg["I"], cfg["B"]),
                     dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    fwd = timed(lambda: layer.forward(x, logits))
    us = timed(lambda: layer.backward(x, logits, d_out, workspace=ws))
    us_re = timed(lambda: layer.backward(x, logits, d_out, workspace=ws, recompute=True))
    layer.grad_dtype = torch.bfloat16
    us_bf16 = timed(lambda: layer.backward(x, logits, d_out, workspace=ws))
    S = int((layer.topk_ids >= 0).sum().item())
    shi = S * cfg["H"] * cfg["I"]
    res = {"workload": describe("prefill_bf16", cfg, cfg["B"]) + ", training backward",
           "us_per_step": round(us, 1), "forward_us_per_step": round(fwd, 1),
           "tflops": round(12 * shi / (us * 1e-6) / 1e12, 1),
           "mfma_frac": round(12 * shi / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
           "us_per_step_recomputing_gate_up": round(us_re, 1),
           "us_per_step_bf16_weight_grads": round(us_bf16, 1)}
    del layer, L, ws
    torch.cuda.empty_cache()
    return res


def one_stage(dev):
    """Layer step time with both GEMMs in one persistent launch against two
    launches (back-to-back steps, no events), per workload at its block size."""
    import torch

    import moe_synth as ms
    res = {}
    for name, B in (("prefill_bf16", 64), ("prefill_fp8", 64), ("decode_bf16", 16), ("decode_fp4", 16),
                    ("prefill_fp4", 64), ("prefill_bf16_512", 128), ("prefill_fp8_512", 128)):
        cfg = ms.CONFIGS[name]
        row = {"block_size_m": B}
        for sched in ("two_launch", "fused"):
            r = run_layer_timed(cfg, B, 10, 3, dev, graph=False, schedule=sched)
            row[sched + "_us_per_step"] = round(r["wall_s"] / r["steps"] * 1e6, 1)
            row[sched + "_ffn_event_us"] = round(sum(r["us"][k] for k in ("quant", "gate_up", "requant", "down")), 1)
            del r
            torch.cuda.empty_cache()
        res[name] = row
    return res


def ffn_input_state(dev, n=15):
    """The grouped FFN of the headline workload (both GEMMs, event-timed,
    median of n) after three different things ran before it: nothing but the
    previous step (its x read before), a kernel that rewrote x (as the
    previous layer of a model does), and a kernel that wrote 512 MB
    elsewhere.  Separates the cost of reading an input from the cost of
    following a kernel that wrote a lot."""
    import torch

    import moe_synth as ms
    import routing_align_sort_amd as moe
    cfg = ms.CONFIGS["prefill_bf16"]
    L = ms.make_layer(cfg, device=dev)
    x, logits = L["x"], L["logits"]
    xsrc = x.clone()
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    layer = moe.MoELayer(L["w13"], L["w2"], T=cfg["T"], K=1, B=cfg["B"], score="softmax",
                         renormalize=False)
    layer.forward(x, logits)
    torch.cuda.synchronize()

    def run(before):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for i in range(n):
            before()
            torch.cuda._sleep(20000)          # keep the host's launch latency out of the events
            ev[2 * i].record()
            layer.ffn(x)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        return round(sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(n))[n // 2], 1)

    res = {"ffn_us_after_previous_step": run(lambda: None),
           "ffn_us_after_x_rewritten": run(lambda: x.copy_(xsrc)),
           "ffn_us_after_512MB_written": run(lambda: scrub.add_(1))}
    del layer, scrub, L
    torch.cuda.empty_cache()
    return res


COPY_PROBE_BYTES = 1 << 30


def copy_probe(dev, reps=3):
    """A plain device copy of COPY_PROBE_BYTES (ordinary 16-byte loads and
    stores, read once, written once; routing_align_sort_amd/probe): the
    reference the profiler's byte counters are scaled against."""
    import ctypes

    import torch

    from routing_align_sort_amd import build as hip_build
    if not os.path.exists(hip_build.PROBE_LIB):
        hip_build.build_probe()
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    lib.moe_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(reps):
        if lib.moe_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                              COPY_PROBE_BYTES, stream) != 0:
            raise RuntimeError("copy probe launch failed")
    torch.cuda.synchronize()


def hbm_probe(dev, nbytes=4 << 30, reps=10):
    """Bandwidth plain kernels reach: a 16-byte-per-thread copy (reads and
    writes nbytes/2 each), a grid-strided read of nbytes, and a read of nbytes
    shaped like the GEMMs' weight stream (1 KB per wave load, 8 in flight,
    non-temporal, a contiguous slab per workgroup) at several grid sizes;
    event-timed, best of `reps`."""
    import ctypes

    import torch

    import routing_align_sort_amd as moe
    from routing_align_sort_amd import build as hip_build
    if not os.path.exists(hip_build.PROBE_LIB):
        hip_build.build_probe()
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    for f in (lib.moe_probe_copy, lib.moe_probe_read):
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.moe_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.c_void_p]
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    half = nbytes // 2
    out = torch.empty(4096, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ev = moe.HipEvents(4 * reps)
    res = {}
    for name, call, moved in (
            ("copy", lambda: lib.moe_probe_copy(ctypes.c_void_p(buf.data_ptr()),
                                                ctypes.c_void_p(buf.data_ptr() + half), half, stream),
             2 * half),
            ("read", lambda: lib.moe_probe_read(ctypes.c_void_p(buf.data_ptr()),
                                                ctypes.c_void_p(out.data_ptr()), nbytes, stream),
             nbytes),
            # 1 KB per wave load instruction, 8 in flight, non-temporal, one
            # contiguous slab per workgroup (the GEMMs' weight stream)
            *[(f"stream_{g}wg", (lambda g=g: lib.moe_probe_stream(ctypes.c_void_p(buf.data_ptr()),
                                                                   ctypes.c_void_p(out.data_ptr()), nbytes, g,
                                                                   stream)),
               nbytes) for g in (512, 1024, 2048, 4096)]):
        call()
        torch.cuda.synchronize()
        for i in range(reps):
            ev.record(2 * i)
            if call() != 0:
                raise RuntimeError("probe launch failed")
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        best = min(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)) * 1e-3
        res[name + "_gbs"] = round(moved / best / 1e9, 1)
    ev.close()
    del buf
    torch.cuda.empty_cache()
    return res


def mfma_probe(dev, reps=5):
    """Matrix-core throughput a kernel with no memory traffic reaches: 8
    independent MFMA chains per wave, two waves per SIMD, bf16 and fp8,
    event-timed, best of `reps` (the practical ceiling under sustained load)."""
    import ctypes

    import torch

    import routing_align_sort_amd as moe
    from routing_align_sort_amd import build as hip_build
    if not os.path.exists(hip_build.PROBE_LIB):
        hip_build.build_probe()
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    lib.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    blocks, iters = 256 * 2 * 4, 2000
    out = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ev = moe.HipEvents(2 * reps)
    res = {}
    # (name, probe kind, K of the instruction, published dense peak in TFLOP/s)
    for name, kind, k, peak in (("bf16", 0, 16, 2500.0), ("fp8", 1, 64, 5000.0),
                                ("fp8_x_fp4", 2, 64, 5000.0), ("fp4", 3, 64, 10100.0)):
        flops = blocks * 4 * iters * 8 * 2 * 32 * 32 * k
        lib.moe_probe_mfma(kind, ctypes.c_void_p(out.data_ptr()), blocks, iters, stream)
        torch.cuda.synchronize()
        for i in range(reps):
            ev.record(2 * i)
            if lib.moe_probe_mfma(kind, ctypes.c_void_p(out.data_ptr()), blocks, iters, stream) != 0:
                raise RuntimeError("probe launch failed")
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        best = min(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)) * 1e-3
        tf = flops / best / 1e12
        res[name + "_tflops"] = round(tf, 1)
        res[name + "_frac_of_peak"] = round(tf / peak, 4)
    ev.close()
    return res


def vendor_gemm(dev, reps=10):
    """Context for the compute-bound shapes: the vendor GEMM library
    (hipBLASLt, called through torch) on the per-expert products of the
    512-tokens-per-expert workload -- rows already grouped, no gather, no
    SiLU, no scales in bf16 -- and on one dense product with all 16384 rows.
    bf16: one batched call over the 32 experts; fp8 (E4M3, row-wise scales,
    bf16 out): one call per expert, as the library has no grouped form here.
    TFLOP/s from event timing, mean of `reps` after 3 warm-up calls."""
    import torch

    def timed(fn):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    g = torch.Generator(device=dev)
    g.manual_seed(0)
    res = {}
    E, M, H, I = 32, 512, 7168, 2048
    for name, (m, k, n) in (("gate_up", (M, H, 2 * I)), ("down", (M, I, H))):
        x = torch.randn(E, m, k, device=dev, dtype=torch.bfloat16, generator=g)
        w = torch.randn(E, k, n, device=dev, dtype=torch.bfloat16, generator=g)    # contiguous [K, N]
        t = timed(lambda: torch.bmm(x, w))
        res[f"bf16_{name}_512_per_expert_tflops"] = round(2.0 * E * m * k * n / t / 1e12, 1)
        del x, w
        f8 = torch.float8_e4m3fn
        x = (torch.randn(E, m, k, device=dev, generator=g) * 0.5).to(f8)
        w = (torch.randn(E, n, k, device=dev, generator=g) * 0.5).to(f8)            # [N, K]: column-major operand
        sx, sw = torch.ones(m, 1, device=dev), torch.ones(1, n, device=dev)
        t = timed(lambda: [torch._scaled_mm(x[e], w[e].t(), scale_a=sx, scale_b=sw, out_dtype=torch.bfloat16)
                           for e in range(E)])
        res[f"fp8_{name}_512_per_expert_tflops"] = round(2.0 * E * m * k * n / t / 1e12, 1)
        del x, w
        torch.cuda.empty_cache()
    m, k, n = E * M, H, 2 * I
    x = torch.randn(m, k, device=dev, dtype=torch.bfloat16, generator=g)
    w = torch.randn(k, n, device=dev, dtype=torch.bfloat16, generator=g)
    t = timed(lambda: x @ w)
    res["bf16_gate_up_dense_16384_rows_tflops"] = round(2.0 * m * k * n / t / 1e12, 1)
    del x, w
    x = (torch.randn(m, k, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn)
    w = (torch.randn(n, k, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn)
    sx, sw = torch.ones(m, 1, device=dev), torch.ones(1, n, device=dev)
    t = timed(lambda: torch._scaled_mm(x, w.t(), scale_a=sx, scale_b=sw, out_dtype=torch.bfloat16))
    res["fp8_gate_up_dense_16384_rows_tflops"] = round(2.0 * m * k * n / t / 1e12, 1)
    del x, w
    torch.cuda.empty_cache()
    return res


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_sq(pmc_dir, out_json):
    """Per-kernel medians over the dispatches of every counter in a rocprofv3
    --pmc run (counters summed over their instances; the library's kernels and
    the copy probe), and, when the run also took a kernel trace, each
    dispatch's duration from the kernel trace and its cycle count
    (GRBM_GUI_ACTIVE is one instance per XCD, so cycles = its sum / 8)."""
    import statistics
    names, per, dur = {}, {}, {}
    for r in _counter_rows(os.path.join(pmc_dir, "run_counter_collection.csv")):
        name = r["Kernel_Name"].replace("void ", "", 1).split("(")[0]
        if not (name.startswith("moe::") or name.startswith("copy_probe_kernel")):
            continue
        did = r["Dispatch_Id"]
        names[did] = name
        c = per.setdefault(did, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    trace = os.path.join(pmc_dir, "run_kernel_trace.csv")
    if os.path.exists(trace):
        for r in _counter_rows(trace):
            if r.get("Dispatch_Id") in names:
                dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    by_kernel = {}
    for did, name in names.items():
        by_kernel.setdefault(name, []).append(did)
    out = {}
    for name, ids in by_kernel.items():
        rec = {"dispatches": len(ids)}
        for c in per[ids[0]]:
            rec[c] = statistics.median(per[i][c] for i in ids)
        timed = [i for i in ids if i in dur]
        if timed:
            rec["us_median"] = statistics.median(dur[i] for i in timed)
            rec["per_dispatch_us_cycles"] = [(round(dur[i], 1), per[i].get("GRBM_GUI_ACTIVE", 0.0) / NUM_XCD)
                                             for i in timed]
        out[name] = rec
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(f"{out_json}: {sorted(out)}")



def summarize_counters(fetch_csv, write_csv, workload, B):
    """HBM bytes per launch of the gate/up kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch, summed over the XCD instances) each scaled by the
    factor that makes the same counter read the known bytes of the plain
    copy kernel; written to profiles/ffn_stage1_<workload>_B<B>_counters.json
    with the hash of the kernel source it was measured on."""
    import hashlib
    import statistics

    import moe_synth as ms
    cfg = ms.CONFIGS[workload]
    B = B or cfg["B"]

    def per_dispatch(path, counter):
        vals = {}
        for r in _counter_rows(path):
            if r.get("Counter_Name") != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        by_kernel = {}
        for (name, _), v in vals.items():
            by_kernel.setdefault(name, []).append(v)
        return by_kernel

    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    pick = lambda d, pat: statistics.median(next(v for k, v in d.items() if pat(k)))
    biggest = lambda d: max(v for k, vs in d.items() if "copy_probe_kernel" in k for v in vs)
    is_st1 = lambda k: "ffn_stage1" in k
    copy_kib_r, copy_kib_w = biggest(fetch), biggest(write)
    f_fetch = COPY_PROBE_BYTES / (copy_kib_r * 1024.0)
    f_write = COPY_PROBE_BYTES / (copy_kib_w * 1024.0)
    st1_r, st1_w = pick(fetch, is_st1), pick(write, is_st1)
    src = os.path.join(ROOT, "routing_align_sort_amd", "csrc", "ffn_mfma.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    rec = {"kernel": "ffn_stage1", "workload": workload, "block_size_m": B,
           "fetch_kib_per_launch": st1_r, "write_kib_per_launch": st1_w,
           "copy_probe_bytes": COPY_PROBE_BYTES, "copy_fetch_kib": copy_kib_r,
           "copy_write_kib": copy_kib_w, "fetch_scale": f_fetch, "write_scale": f_write,
           "hbm_bytes_per_launch": round(st1_r * 1024 * f_fetch + st1_w * 1024 * f_write),
           "kernel_source_sha256": digest}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    out = os.path.join(PROFILE_DIR, f"ffn_stage1_{workload}_B{B}_counters.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def describe(name, cfg, B):
    if name == "align_16k":
        return "align-sort 16384x8 over 256 experts"
    s = f"{name}: {cfg['T']} tokens x top-{cfg['K']} of {cfg['E']} experts"
    if cfg.get("shared"):
        s += " + 1 shared expert"
    s += f", hidden {cfg['H']}, inter {cfg['I']}, SwiGLU, {cfg['dtype']}, block_size_m {B}"
    return s


def measured_traffic(workload, B):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source; else None."""
    import hashlib
    path = os.path.join(PROFILE_DIR, f"ffn_stage1_{workload}_B{B}_counters.json")
    src = os.path.join(ROOT, "routing_align_sort_amd", "csrc", "ffn_mfma.hip")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("kernel_source_sha256") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def run_cpu_baseline(cfg, B, dev, budget_s=12.0):
    """The CPU oracle as it stands, on a bounded sample of the same workload:
    routing and Align & Sort over all tokens, then the expert FFN + combine of
    a seeded sample of tokens sized to ~budget_s of CPU time; tokens/s is the
    per-token cost extrapolated to the whole batch."""
    import numpy as np
    import torch

    import moe_synth as ms
    import oracle

    L = ms.make_layer(cfg, device="cpu", weights=False)
    logits = L["logits"].numpy()
    bias = None if L["bias"] is None else L["bias"].numpy()
    T = cfg["T"]
    t0 = time.perf_counter()
    ids, w = oracle.route_topk(logits, cfg["K"], score=cfg["score"], bias=bias,
                               n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                               renormalize=cfg["renormalize"],
                               append_shared=bool(cfg.get("shared")))
    E_slabs = cfg["E"] + (1 if cfg.get("shared") else 0)
    oracle.align_sort(ids, E_slabs, B)
    t_ra = time.perf_counter() - t0

    # host copies of the inputs (generated on the GPU, bit-identical to the host generator)
    G = ms.make_weights(cfg, device=dev)
    hb = lambda t: (t.cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16
                    else t.cpu().view(torch.uint8).numpy() if t.dtype == torch.float8_e4m3fn
                    else t.cpu().numpy())
    w13, w2 = hb(G["w13"]), hb(G["w2"])
    s13 = G["w13_scale"].cpu().numpy() if "w13_scale" in G else None
    s2 = G["w2_scale"].cpu().numpy() if "w2_scale" in G else None
    del G
    torch.cuda.empty_cache()
    x = L["x"]
    xh = hb(x)
    wdt = cfg["dtype"]
    xdt = "f32" if wdt == "f32" else "bf16"
    rng = np.random.default_rng(0)
    order = rng.permutation(T)

    def ffn(toks):
        t1 = time.perf_counter()
        oracle.moe_layer(xh[toks], w13, w2, ids[toks], w[toks], w_dtype=wdt, x_dtype=xdt,
                         inter="e4m3" if wdt == "e2m1" else wdt, w13_scale=s13, w2_scale=s2,
                         E=E_slabs)
        return time.perf_counter() - t1

    n0 = int(min(T, 4 * oracle.num_threads()))   # enough tokens to occupy every oracle thread
    t_probe = ffn(np.sort(order[:n0]))
    n = int(min(T, max(n0, budget_s / max(t_probe / n0, 1e-9))))
    t_ffn = ffn(np.sort(order[:n]))
    per_token = t_ra / T + t_ffn / n
    # the same oracle on one core: a smaller seeded sample (about a quarter of the budget)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t_one = ffn(np.sort(order[:1]))
        n1 = int(min(T, max(1, 0.25 * budget_s / max(t_one, 1e-9))))
        t_ffn1 = ffn(np.sort(order[:n1]))
    finally:
        oracle.set_num_threads(threads)
    per_token1 = t_ra / T + t_ffn1 / n1
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    # the Align & Sort oracle alone (serial C, one core) on the 16384 x top-8 workload
    a16 = ms.CONFIGS["align_16k"]
    ids16 = ms.zipf_topk_ids(0, ms.TAG_IDS, a16["T"], a16["K"], a16["E"], a16["zipf_s"])
    t1 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        oracle.align_sort(ids16, a16["E"], a16["B"])
    align_ms = (time.perf_counter() - t1) / reps * 1e3
    return {"value": round(1.0 / per_token, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "align_sort_16k_single_core_ms": round(align_ms, 3),
            "single_core_tokens_per_s": round(1.0 / per_token1, 3),
            "single_core_sample": f"expert FFN + combine for {n1} seeded tokens on one thread ({t_ffn1:.2f} s)",
            "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "sample": f"routing + Align & Sort over all {T} tokens ({t_ra:.3f} s), expert FFN + "
                      f"combine for {n} seeded tokens ({t_ffn:.2f} s), double precision; "
                      f"tokens/s extrapolated per token"}


if __name__ == "__main__":
    main()
