"""Benchmark: one MI355X forward pass through the routed grouped-GEMM MoE layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral]

A step is one moe_layer call (route, permute, persistent expert-FFN + combine)
over the seeded synthetic Mixtral-shape batch (T=4096, d=4096, f=14336, E=8,
top-2), inputs resident in HBM.  W untimed steps, then K timed steps between
two device synchronisations.  Prints one JSON line with the layer throughput
(tokens/s), the grouped-GEMM TFLOP/s of the persistent kernel, its roofline
entry and the CPU oracle timed on a bounded sample of the same workload.

--mode copy runs a plain device-to-device copy of known size (used to scale
the FETCH_SIZE / WRITE_SIZE counters of rocprofv3 to bytes).

--mode ffn_fp8 / ffn_bf16 time the staged expert FFN alone (moe_expert_ffn_fp8
on E4M3 weights quantised once beforehand, or moe_expert_ffn in bf16) on the
same workload's routed rows, and print one JSON line in TFLOP/s of 6*d*f per
routed row against the MFMA peak of that precision.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer_kernel_mixtral_traffic.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "routed_grouped_gemm_moe_amd", "csrc", "*"))):
        with open(p, "rb") as fh:
            h.update(os.path.basename(p).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the persistent kernel from the committed counter
    summary, or None if absent or taken from different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


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


def cpu_baseline(cfg, arrs, n_tokens: int):
    import numpy as np
    import oracle
    toks = np.linspace(0, cfg.T - 1, n_tokens).astype(np.int64)
    t0 = time.perf_counter()
    oracle.layer_tokens(toks, arrs["x"], arrs["w_router"], arrs["w_gate"], arrs["w_up"],
                        arrs["w_down"], cfg.k, cfg.e_lo, cfg.E_hi, bias=arrs["bias"])
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_tokens} evenly spaced tokens of the same {cfg.name} batch, each routed "
                      f"and run through its {cfg.k} selected experts' float64 SwiGLU and combine "
                      f"({dt:.1f} s)"}


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
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    print(json.dumps({
        "mode": args.mode,
        "metric": "staged expert-FFN TFLOP/s (" + ("W8A8 E4M3" if fp8 else "bf16") + "), 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_call": round(ms, 4),
        "steps": args.steps, "warmup": args.warmup, "peak": peak, "frac": round(tflops / peak, 4),
        "dtype": "fp8_e4m3" if fp8 else "bf16", "routed_rows": n_rows,
        "flops_per_call": flops,
        "config": {"workload": f"{cfg.name}: {cfg.note}", "T": cfg.T, "d": cfg.d, "f": cfg.f,
                   "E": cfg.E, "k": cfg.k, "local_experts": [cfg.e_lo, cfg.E_hi]},
    }), flush=True)


def layer_fp8_mode(args, cfg, M, torch, D, x, wr, wg, wu, wd, bias) -> None:
    """Time moe_layer_fp8 (route, permute, W8A8 FFN, combine) on the workload;
    the weights are quantised once beforehand."""
    (gq, gs), (uq, us), (dq, ds) = (M.moe_quantize_fp8(w) for w in (wg, wu, wd))
    ws = torch.empty(M.moe_layer_fp8_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32 if cfg.out_fp32 else torch.bfloat16,
                      device="cuda")
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    step = lambda: M.moe_layer_fp8(D, x, wr, gq, gs, uq, us, dq, ds, bias=bias, out=out,
                                   out_dtype=dt, topk_ids_out=ids, ws=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    n_local = int(((ids_h >= cfg.e_lo) & (ids_h < cfg.E_hi)).sum())
    flops = 6.0 * cfg.d * cfg.f * n_local
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    print(json.dumps({
        "mode": "layer_fp8",
        "metric": "MoE-layer tokens/s with the W8A8 (E4M3) expert FFN, 1 GPU",
        "value": round(cfg.T * args.steps / elapsed, 1), "unit": "tokens/s",
        "ms_per_step": round(ms, 4), "steps": args.steps, "warmup": args.warmup,
        "layer_tflops": round(flops / (ms * 1e-3) / 1e12, 2), "dtype": "fp8_e4m3",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "T": cfg.T, "d": cfg.d, "f": cfg.f,
                   "E": cfg.E, "k": cfg.k, "local_experts": [cfg.e_lo, cfg.E_hi]},
    }), flush=True)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--mode", default="layer",
                    choices=["layer", "copy", "ffn_fp8", "ffn_bf16", "layer_fp8"])
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-w8a8", action="store_true",
                    help="skip the extra W8A8 layer measurement of the default mode")
    ap.add_argument("--tile-order", type=int, default=0, choices=[0, 1],
                    help="moe_layer persistent-kernel tile order: 0 by kind, 1 interleaved")
    ap.add_argument("--dispatch", default="packed", choices=["packed", "gather"],
                    help="moe_layer dispatch: packed x_perm (default) or gather rows on load")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.mode == "copy":
        copy_mode(args)
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
    if args.mode == "layer_fp8":
        layer_fp8_mode(args, cfg, M, torch, D, x, wr, wg, wu, wd, bias)
        return
    M.moe_set_gather_dispatch(args.dispatch == "gather")
    M.moe_set_tile_order(args.tile_order)
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32 if cfg.out_fp32 else torch.bfloat16,
                      device="cuda")
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")

    def step():
        M.moe_layer(D, x, wr, wg, wu, wd, bias=bias, out=out, out_dtype=dt, topk_ids_out=ids,
                    topk_w_out=gates, ws=ws)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if M.moe_device_status(D, ws) != 0:
        raise RuntimeError("device status not OK after warmup")

    # local rows (all T*k for a full-local config)
    ids_h = ids.cpu().numpy()
    n_local = int(((ids_h >= cfg.e_lo) & (ids_h < cfg.E_hi)).sum())
    flops = 6.0 * cfg.d * cfg.f * n_local   # Weave §3.1: 6*H*I per token-expert pair

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    M.moe_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_ev, (route_ms, perm_ms, ffn_ms) = M.moe_timing_read()
    M.moe_timing_enable(False)
    if M.moe_device_status(D, ws) != 0:
        raise RuntimeError("device status not OK after timed steps")

    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = cfg.T * args.steps / elapsed
    ffn_tflops = flops / (ffn_ms * 1e-3) / 1e12 if ffn_ms > 0 else 0.0
    layer_tflops = flops / (ms_per_step * 1e-3) / 1e12
    traffic = read_traffic()

    rec = {
        "metric": "MoE-layer tokens/s and grouped-GEMM TFLOP/s (% of MFMA bf16 peak), 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian activations and weights, Gaussian router)",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "T": cfg.T, "d": cfg.d, "f": cfg.f,
                   "E": cfg.E, "k": cfg.k, "local_experts": [cfg.e_lo, cfg.E_hi],
                   "dispatch": args.dispatch, "tile_order": args.tile_order,
                   "parallelism": "none (one GPU)"},
        "grouped_gemm_tflops": round(ffn_tflops, 2),
        "grouped_gemm_pct_mfma_peak": round(100 * ffn_tflops / PEAK_BF16_TFLOPS, 2),
        "layer_tflops": round(layer_tflops, 2),
        "stages_ms": {"route": round(route_ms, 4), "permute": round(perm_ms, 4),
                      "expert_ffn_combine_persistent": round(ffn_ms, 4), "events": n_ev},
        "roofline": {"bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ffn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "layer_kernel (persistent gate/up, down, combine tiles)",
                     "algorithmic_flops_per_launch": flops},
    }
    if not args.no_w8a8 and cfg.f % 256 == 0:
        # the same workload through moe_layer_fp8 (weights quantised once,
        # outside the timed steps); reported beside the bf16 line, not as it
        print("[bench] W8A8 layer", file=sys.stderr, flush=True)
        (gq, gs), (uq, us), (dq, ds) = (M.moe_quantize_fp8(w) for w in (wg, wu, wd))
        ws8 = torch.empty(M.moe_layer_fp8_workspace_bytes(D), dtype=torch.uint8, device="cuda")
        step8 = lambda: M.moe_layer_fp8(D, x, wr, gq, gs, uq, us, dq, ds, bias=bias, out=out,
                                        out_dtype=dt, ws=ws8)
        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step8()
        torch.cuda.synchronize()
        el8 = time.perf_counter() - t0
        rec["w8a8_layer"] = {"value": round(cfg.T * args.steps / el8, 1), "unit": "tokens/s",
                             "ms_per_step": round(el8 / args.steps * 1e3, 4),
                             "dtype": "fp8_e4m3", "entry_point": "moe_layer_fp8 (staged)"}
        del ws8, gq, uq, dq
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({args.cpu_tokens} tokens)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, arrs, args.cpu_tokens)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
