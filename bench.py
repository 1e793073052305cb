"""Benchmark: one MI355X forward pass through the routed grouped-GEMM MoE layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral]

A step is one moe_layer call (route, permute, persistent expert-FFN + combine)
over the seeded synthetic Mixtral-shape batch (T=4096, d=4096, f=14336, E=8,
top-2), inputs resident in HBM.  W untimed steps, then K timed steps between
two device synchronisations.  Each timed step also passes four HIP events to
the library (moe_layer_opts.events), which records them around its launches;
their medians over the K steps give the per-stage times (X-Stage, §5.1,
reports medians).  Prints one JSON line with the layer throughput (tokens/s),
the grouped-GEMM TFLOP/s of the persistent kernel, its roofline entry, the
route / permute / combine bandwidth against HBM, and the CPU oracle timed on
bounded samples of every workload.

Memory-bound stage probes (route, permute, combine as standalone C-ABI calls)
rotate through copies of their inputs totalling more than the 256 MB
Infinity Cache, so their bytes come from HBM.

Other modes:
  --mode copy        a plain device copy of known size (scales the FETCH_SIZE
                     and WRITE_SIZE counters of rocprofv3 to bytes)
  --mode ffn_fp8 / ffn_bf16 / layer_fp8
                     the staged W8A8 or bf16 expert FFN alone, or the W8A8 layer
                     (its default staged launches and its persistent kernel)
  --mode mfma_rate   the sustained bf16 matrix-core rate of a loop of
                     independent MFMAs on every CU, with zero and with
                     random operands (the achievable share of the nominal
                     peak under the chip's power limit)
  --summarize-trace DIR
                     per-kernel medians of the timed dispatches in the
                     rocprofv3 kernel trace (csv) under DIR, skipping the
                     warm-up dispatches (give the run's --warmup / --steps)
  --summarize-counters DIR
                     per-kernel means of the rocprofv3 counters (csv) under DIR
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
INFINITY_CACHE_BYTES = 256 << 20
METRIC = "MoE-layer tokens/s and grouped-GEMM TFLOP/s (% of MFMA bf16 peak), 1 GPU"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "routed_grouped_gemm_moe_amd", "csrc", "*"))):
        with open(p, "rb") as fh:
            h.update(os.path.basename(p).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch of the persistent kernel from the committed counter
    summary of this workload, or None if absent or taken from other sources."""
    path = os.path.join(ROOT, "profiles", f"layer_kernel_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def median(v):
    return float(statistics.median(v)) if v else 0.0


# ------------------------------------------------------------ trace summary

def short_name(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("moe::", "")
    n = re.sub(r"^void\s+", "", n)
    n = re.sub(r"\(.*$", "", n)              # drop the argument list
    return n.strip()


def summarize_trace(args) -> None:
    rows = []
    for p in sorted(glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_trace.csv"),
                              recursive=True)):
        with open(p) as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                             short_name(r["Kernel_Name"])))
    rows.sort()
    by = {}
    for t0, t1, n in rows:
        by.setdefault(n, []).append((t1 - t0) / 1000.0)
    calls = args.warmup + args.steps
    print(f"kernel trace: {len(rows)} dispatches; warm-up dispatches dropped: the first "
          f"warmup/(warmup+steps) = {args.warmup}/{calls} of each kernel's calls")
    total = sum(sum(v) for v in by.values())
    for n, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        per = len(v) // calls if len(v) % calls == 0 and len(v) >= calls else 0
        timed = v[per * args.warmup:] if per else v
        print(f"  {n:48s} calls={len(v):4d} timed={len(timed):4d} "
              f"median_us={median(timed):10.2f} mean_us={sum(timed) / len(timed):10.2f} "
              f"min_us={min(timed):10.2f} max_us={max(timed):10.2f} "
              f"pct_all={100 * sum(v) / total:6.2f}" + ("" if per else "  (not per-step)"))


def summarize_counters(args) -> None:
    """Per-kernel mean of every counter in the rocprofv3 counter collections
    (csv) under DIR, over all dispatches of that kernel."""
    acc = {}
    for p in sorted(glob.glob(os.path.join(args.summarize_counters, "**",
                                           "*counter_collection.csv"), recursive=True)):
        with open(p) as fh:
            for r in csv.DictReader(fh):
                key = (short_name(r["Kernel_Name"]), r["Counter_Name"])
                acc.setdefault(key, {})
                d = acc[key]
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    for (k, c), d in sorted(acc.items()):
        v = list(d.values())
        print(f"  {k:40s} {c:28s} dispatches={len(v):3d} mean={sum(v) / len(v):.6e}")


# ------------------------------------------------------------ modes

def copy_mode(args) -> None:
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": args.steps}), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_sample(cfg, arrs, n_tokens: int):
    """Time the oracle on n_tokens evenly spaced tokens of the workload."""
    import numpy as np
    import oracle
    toks = np.unique(np.linspace(0, cfg.T - 1, min(n_tokens, cfg.T)).astype(np.int64))
    t0 = time.perf_counter()
    _, ids, _ = oracle.layer_tokens(toks, arrs["x"], arrs["w_router"], arrs["w_gate"],
                                    arrs["w_up"], arrs["w_down"], cfg.k, cfg.e_lo, cfg.E_hi,
                                    bias=arrs["bias"])
    dt = time.perf_counter() - t0
    pairs = int(((ids >= cfg.e_lo) & (ids < cfg.E_hi)).sum())
    return {"tokens": int(len(toks)), "seconds": round(dt, 3),
            "tokens_per_s": round(len(toks) / dt, 2),
            "gflops": round(6.0 * cfg.d * cfg.f * pairs / dt / 1e9, 2),
            "full_layer_s_est": round(cfg.T * dt / len(toks), 1)}


def cpu_baseline(cfg, arrs, n_tokens: int, per_config: bool):
    """The oracle as it stands, on this host's cores: the headline sample of
    the benchmarked workload, bounded samples of every workload, and the tiny
    workload once more on one thread, with the host's CPU model."""
    import moe_workloads as W
    import oracle
    threads = oracle.num_threads()
    head = oracle_sample(cfg, arrs, n_tokens)
    rec = {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{head['tokens']} evenly spaced tokens of the same {cfg.name} batch, each "
                     f"routed and run through its selected experts' float64 SwiGLU and combine "
                     f"({head['seconds']} s; {head['gflops']} GFLOP/s)"}
    if per_config:
        sizes = {"tiny": 256, "mixtral": 128, "fine": 1024, "skewed": 128, "dsv3_share": 1024}
        pc = {}
        for name, n in sizes.items():
            c = W.CONFIGS[name]
            a = arrs if name == cfg.name else W.generate(c)
            pc[name] = oracle_sample(c, a, n)
            del a
        oracle.set_num_threads(1)
        try:
            one = oracle_sample(W.CONFIGS["tiny"], W.generate(W.CONFIGS["tiny"]), 256)
        finally:
            oracle.set_num_threads(threads)
        rec["per_config"] = pc
        rec["tiny_one_thread"] = one
    return rec


def stage_probes(args, cfg, M, torch, D, x, wr, bias, n_rows, t_local):
    """Route, permute and combine as standalone C-ABI calls, inputs rotated
    through copies totalling more than the Infinity Cache; median of
    args.steps calls each, against the algorithmic bytes of each stage."""
    def copies(t):
        n = max(2, -(-int(1.25 * INFINITY_CACHE_BYTES) // (t.numel() * t.element_size())))
        return [t.clone() for _ in range(n)]

    def timed(fn, n_in):
        for i in range(args.warmup):
            fn(i % n_in)
        torch.cuda.synchronize()
        ms = []
        for i in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn((args.warmup + i) % n_in)
            e1.record()
            ms.append((e0, e1))
        torch.cuda.synchronize()
        return median([a.elapsed_time(b) for a, b in ms])

    T, d, k, E = cfg.T, cfg.d, cfg.k, cfg.E
    xs = copies(x)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    rws = torch.empty(max(M.moe_route_workspace_bytes(D), 256), dtype=torch.uint8, device="cuda")
    route_ms = timed(lambda i: M.moe_route(D, xs[i], wr, bias, topk_ids=ids, topk_w=gates, ws=rws),
                     len(xs))
    route_bytes = T * d * 2 + E * d * 2 + T * k * 8
    cap = max(T * k, 1)
    counts = torch.empty(D.e_hi - D.e_lo, dtype=torch.int32, device="cuda")
    offsets = torch.empty(D.e_hi - D.e_lo + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(cap, dtype=torch.int32, device="cuda")
    inv = torch.empty((T, k), dtype=torch.int32, device="cuda")
    xp = torch.empty((cap, d), dtype=torch.bfloat16, device="cuda")
    pws = torch.empty(M.moe_permute_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    perm_ms = timed(lambda i: M.moe_permute(D, xs[i], ids, counts, offsets, perm, inv, xp, ws=pws),
                    len(xs))
    # read every token row with a local slot once, write the routed rows and indices
    perm_bytes = t_local * d * 2 + n_rows * d * 2 + T * k * 8 + n_rows * 4
    del xs
    ys = copies(xp)
    out_f32 = bool(cfg.out_fp32)
    out = torch.empty((T, d), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    dt = M.MOE_F32 if out_f32 else M.MOE_BF16
    comb_ms = timed(lambda i: M.moe_combine(D, ys[i], inv, gates, out=out, out_dtype=dt), len(ys))
    comb_bytes = n_rows * d * 2 + T * k * 8 + T * d * (4 if out_f32 else 2)
    del ys

    def entry(ms, nbytes, what):
        gbs = nbytes / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        return {"us": round(ms * 1e3, 2), "algorithmic_bytes": int(nbytes), "GBps": round(gbs, 1),
                "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "call": what}
    return {"route": entry(route_ms, route_bytes, "moe_route"),
            "permute": entry(perm_ms, perm_bytes, "moe_permute (row-major x_perm)"),
            "combine": entry(comb_ms, comb_bytes, "moe_combine"),
            "rotation": "inputs rotated through copies > 1.25 x 256 MB; median of "
                        f"{args.steps} calls after {args.warmup} warm-up"}


def mfma_rate_mode(args) -> None:
    """Sustained matrix-core rate (moe_probe_mfma_rate): one workgroup of 4
    waves per CU, each wave 16 independent v_mfma_f32_32x32x16_bf16 per
    iteration; median of `steps` timed launches after `warmup`, for zero and
    for pseudo-random operands."""
    import torch
    import routed_grouped_gemm_moe_amd as M
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    flops = cus * 4 * iters * 16 * 32768.0
    sink = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    res = {}
    for name, seed in (("zero_operands", 0), ("random_operands", 12345)):
        for _ in range(max(args.warmup, 1)):
            M.moe_probe_mfma_rate(cus, iters, seed, sink)
        ms = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            M.moe_probe_mfma_rate(cus, iters, seed, sink)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = median(ms)
        res[name] = {"ms_median": round(t, 4), "tflops": round(flops / (t * 1e-3) / 1e12, 1),
                     "frac_of_peak": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    print(json.dumps({"mode": "mfma_rate", "metric": "sustained bf16 MFMA rate, 1 GPU",
                      "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS, "cus": cus,
                      "flops_per_launch": flops, "steps": args.steps, "warmup": args.warmup,
                      **res}), flush=True)


def ffn_mode(args, cfg, M, torch, D, x, wr, wg, wu, wd, bias) -> None:
    """Time the staged expert FFN (fp8 or bf16) on the workload's routed rows."""
    ids, _, _ = M.moe_route(D, x, wr, bias)
    _, offsets, _, _, xp = M.moe_permute(D, x, ids)
    n_rows = int(offsets[-1].item())
    flops = 6.0 * cfg.d * cfg.f * n_rows
    y = torch.empty((max(cfg.T * cfg.k, 1), cfg.d), dtype=torch.bfloat16, device="cuda")
    fp8 = args.mode == "ffn_fp8"
    if fp8:
        (gq, gs), (uq, us), (dq, ds) = (M.moe_quantize_fp8(w) for w in (wg, wu, wd))
        ws = torch.empty(M.moe_expert_ffn_fp8_workspace_bytes(D), dtype=torch.uint8, device="cuda")
        step = lambda: M.moe_expert_ffn_fp8(D, xp, offsets, gq, gs, uq, us, dq, ds, y_perm=y, ws=ws)
    else:
        ws = torch.empty(M.moe_expert_ffn_workspace_bytes(D), dtype=torch.uint8, device="cuda")
        step = lambda: M.moe_expert_ffn(D, xp, offsets, wg, wu, wd, y_perm=y, ws=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = median([a.elapsed_time(b) for a, b in evs])
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    print(json.dumps({
        "mode": args.mode,
        "metric": "staged expert-FFN TFLOP/s (" + ("W8A8 E4M3" if fp8 else "bf16") + "), 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_call_median": round(ms, 4),
        "steps": args.steps, "warmup": args.warmup, "peak": peak, "frac": round(tflops / peak, 4),
        "dtype": "fp8_e4m3" if fp8 else "bf16", "routed_rows": n_rows,
        "flops_per_call": flops,
        "config": {"workload": f"{cfg.name}: {cfg.note}", "T": cfg.T, "d": cfg.d, "f": cfg.f,
                   "E": cfg.E, "k": cfg.k, "local_experts": [cfg.e_lo, cfg.E_hi]},
    }), flush=True)


def w8a8_layer(args, cfg, M, torch, D, x, wr, wg, wu, wd, bias, out, dt, n_local=None):
    """The same workload through moe_layer_fp8 (weights quantised once,
    outside the timed steps): its default schedule (the staged launches) and
    its persistent kernel.  fp8_tflops: Weave §3.1's 6*H*I per routed row
    over the median time of the launches after the permute (x quantisation,
    expert FFN, combine), against the 5 PF dense fp8 peak."""
    (gq, gs), (uq, us), (dq, ds) = (M.moe_quantize_fp8(w) for w in (wg, wu, wd))
    ws8 = torch.empty(M.moe_layer_fp8_workspace_bytes(D), dtype=torch.uint8, device="cuda")

    def run(schedule):
        step8 = lambda o: M.moe_layer_fp8(D, x, wr, gq, gs, uq, us, dq, ds, bias=bias, out=out,
                                          out_dtype=dt, ws=ws8, opts=o)
        plain = M.layer_opts(schedule=schedule)
        for _ in range(args.warmup):
            step8(plain)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        opts = [M.layer_opts(events=e, schedule=schedule) for e in evs]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for o in opts:
            step8(o)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        ffn_us = median([e[2].elapsed_time(e[3]) for e in evs]) * 1e3
        return el, median([e[0].elapsed_time(e[3]) for e in evs]), ffn_us

    el, med, ffn_us = run(M.MOE_SCHEDULE_AUTO)   # the staged launches
    el_p, med_p, ffn_us_p = run(M.MOE_SCHEDULE_PERSISTENT)
    tf = lambda us: 6.0 * cfg.d * cfg.f * n_local / (us * 1e-6) / 1e12 if n_local else None
    rec = {"value": round(cfg.T * args.steps / el, 1), "unit": "tokens/s",
           "ms_per_step": round(el / args.steps * 1e3, 4), "ms_per_step_median": round(med, 4),
           "dtype": "fp8_e4m3", "entry_point": "moe_layer_fp8 (default schedule: staged launches)",
           "ffn_combine_median_us": round(ffn_us, 2),
           "persistent_schedule": {"value": round(cfg.T * args.steps / el_p, 1),
                                   "ms_per_step_median": round(med_p, 4),
                                   "ffn_combine_median_us": round(ffn_us_p, 2)}}
    if n_local:
        rec.update({"fp8_tflops": round(tf(ffn_us), 2),
                    "pct_fp8_peak": round(100 * tf(ffn_us) / PEAK_FP8_TFLOPS, 2)})
        rec["persistent_schedule"].update({"fp8_tflops": round(tf(ffn_us_p), 2)})
    return rec


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--mode", default="layer",
                    choices=["layer", "copy", "ffn_fp8", "ffn_bf16", "layer_fp8", "mfma_rate"])
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-per-config", action="store_true",
                    help="oracle baseline on the benchmarked workload only")
    ap.add_argument("--no-w8a8", action="store_true",
                    help="skip the extra W8A8 layer measurement of the default mode")
    ap.add_argument("--no-stage-probe", action="store_true",
                    help="skip the standalone route / permute / combine measurements")
    ap.add_argument("--tile-order", type=int, default=0, choices=[0, 1, 2, 3, 4],
                    help="moe_layer tile order (moe_tile_order)")
    ap.add_argument("--lead", type=int, default=0, help="dependency lead of tile order 2")
    ap.add_argument("--chunks", type=int, default=0, help="token chunks of tile order 4")
    ap.add_argument("--dispatch", default="packed", choices=["packed", "gather"],
                    help="moe_layer dispatch: packed x_perm (default) or gather rows on load")
    ap.add_argument("--summarize-trace", default=None, metavar="DIR")
    ap.add_argument("--summarize-counters", default=None, metavar="DIR")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.mode == "copy":
        copy_mode(args)
        return
    if args.mode == "mfma_rate":
        mfma_rate_mode(args)
        return

    import moe_workloads as W
    import routed_grouped_gemm_moe_amd as M

    cfg = W.CONFIGS[args.config]
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    arrs = W.generate(cfg)
    dev = lambda v: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to("cuda").view(
        torch.bfloat16)
    x, wr = dev(arrs["x"]), dev(arrs["w_router"])
    wg, wu, wd = dev(arrs["w_gate"]), dev(arrs["w_up"]), dev(arrs["w_down"])
    bias = torch.from_numpy(arrs["bias"]).to("cuda") if arrs["bias"] is not None else None
    D = M.MoEDims.make(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.e_lo, cfg.E_hi)
    if args.mode in ("ffn_fp8", "ffn_bf16"):
        ffn_mode(args, cfg, M, torch, D, x, wr, wg, wu, wd, bias)
        return
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32 if cfg.out_fp32 else torch.bfloat16,
                      device="cuda")
    if args.mode == "layer_fp8":
        ids8 = M.moe_route(D, x, wr, bias)[0].cpu().numpy()
        n8 = int(((ids8 >= cfg.e_lo) & (ids8 < cfg.E_hi)).sum())
        rec = w8a8_layer(args, cfg, M, torch, D, x, wr, wg, wu, wd, bias, out, dt, n_local=n8)
        rec.update({"mode": "layer_fp8",
                    "metric": "MoE-layer tokens/s with the W8A8 (E4M3) expert FFN, 1 GPU",
                    "steps": args.steps, "warmup": args.warmup,
                    "config": {"workload": f"{cfg.name}: {cfg.note}", "T": cfg.T, "d": cfg.d,
                               "f": cfg.f, "E": cfg.E, "k": cfg.k,
                               "local_experts": [cfg.e_lo, cfg.E_hi]}})
        print(json.dumps(rec), flush=True)
        return

    base = dict(dispatch=M.MOE_DISPATCH_GATHER if args.dispatch == "gather" else
                M.MOE_DISPATCH_PACKED, tile_order=args.tile_order, lead=args.lead,
                chunks=args.chunks)
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")

    def step(opts):
        M.moe_layer(D, x, wr, wg, wu, wd, bias=bias, out=out, out_dtype=dt, topk_ids_out=ids,
                    topk_w_out=gates, ws=ws, opts=opts)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    warm_opts = M.layer_opts(**base)
    for _ in range(args.warmup):
        step(warm_opts)
    torch.cuda.synchronize()
    if M.moe_device_status(D, ws) != 0:
        raise RuntimeError("device status not OK after warmup")

    # local rows (all T*k for a full-local config)
    ids_h = ids.cpu().numpy()
    local = (ids_h >= cfg.e_lo) & (ids_h < cfg.E_hi)
    n_local = int(local.sum())
    t_local = int(local.any(axis=1).sum())
    flops = 6.0 * cfg.d * cfg.f * n_local   # Weave §3.1: 6*H*I per token-expert pair

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    opts = [M.layer_opts(**base, events=e) for e in evs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for o in opts:
        step(o)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if M.moe_device_status(D, ws) != 0:
        raise RuntimeError("device status not OK after timed steps")
    route_ms = median([e[0].elapsed_time(e[1]) for e in evs])
    perm_ms = median([e[1].elapsed_time(e[2]) for e in evs])
    ffn_ms = median([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = median([e[0].elapsed_time(e[3]) for e in evs])

    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = cfg.T * args.steps / elapsed
    ffn_tflops = flops / (ffn_ms * 1e-3) / 1e12 if ffn_ms > 0 else 0.0
    layer_tflops = flops / (ms_per_step * 1e-3) / 1e12
    # algorithmic bytes of the fused layer's route and permute stages
    route_bytes = cfg.T * cfg.d * 2 + cfg.E * cfg.d * 2 + cfg.T * cfg.k * 8
    perm_bytes = t_local * cfg.d * 2 + n_local * cfg.d * 2 + cfg.T * cfg.k * 8 + n_local * 4

    def gb(nbytes, ms):
        g = nbytes / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        return {"us": round(ms * 1e3, 2), "algorithmic_bytes": int(nbytes), "GBps": round(g, 1),
                "frac_hbm": round(g / PEAK_HBM_GBS, 4)}

    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian activations and weights, Gaussian router)",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "T": cfg.T, "d": cfg.d, "f": cfg.f,
                   "E": cfg.E, "k": cfg.k, "local_experts": [cfg.e_lo, cfg.E_hi],
                   "dispatch": args.dispatch, "tile_order": args.tile_order,
                   "lead": args.lead, "chunks": args.chunks,
                   "parallelism": "none (one GPU)"},
        "grouped_gemm_tflops": round(ffn_tflops, 2),
        "grouped_gemm_pct_mfma_peak": round(100 * ffn_tflops / PEAK_BF16_TFLOPS, 2),
        "layer_tflops": round(layer_tflops, 2),
        "stages_median": {"route": gb(route_bytes, route_ms), "permute": gb(perm_bytes, perm_ms),
                          "expert_ffn_combine_persistent_us": round(ffn_ms * 1e3, 2),
                          "source": "HIP events of moe_layer_opts.events, median of the "
                                    f"{args.steps} timed steps"},
        "roofline": {"bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ffn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(cfg.name),
                     "kernel": "layer_kernel (persistent gate/up, down, combine tiles)",
                     "algorithmic_flops_per_launch": flops,
                     "duration": "median over the timed steps of the launch's HIP events"},
    }
    if not args.no_stage_probe:
        print("[bench] stage probes", file=sys.stderr, flush=True)
        rec["memory_bound_stages"] = stage_probes(args, cfg, M, torch, D, x, wr, bias, n_local,
                                                  t_local)
    if not args.no_w8a8 and cfg.f % 256 == 0:
        print("[bench] W8A8 layer", file=sys.stderr, flush=True)
        rec["w8a8_layer"] = w8a8_layer(args, cfg, M, torch, D, x, wr, wg, wu, wd, bias, out, dt,
                                       n_local=n_local)
    if not args.no_cpu_baseline:
        del x, wr, wg, wu, wd, ws
        torch.cuda.empty_cache()
        print(f"[bench] cpu baseline ({args.cpu_tokens} tokens + per-workload samples)",
              file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, arrs, args.cpu_tokens,
                                           not args.no_cpu_per_config)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
