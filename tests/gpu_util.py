"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np

import moe_workloads as W

TOL_LAYER = 2e-2       # max relative error of layer / FFN outputs (bf16 in and out)
TOL_GATE = 2e-6        # absolute error of float32 gates vs the float64-evaluated oracle


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host_bits(t) -> np.ndarray:
    """bf16 device tensor -> uint16 numpy bits."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(host_bits(t))
    return t.detach().float().cpu().numpy()


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """Max relative error of a layer output, token by token:
    max over (t, i) of |o[t,i] - r[t,i]| / max(|r[t,i]|, rms(r[t,:])).
    A token whose reference row is exactly zero (no local expert) must come out
    exactly zero: any nonzero value there counts as an infinite error."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    out2 = out.reshape(-1, ref.shape[-1])
    ref2 = ref.reshape(-1, ref.shape[-1])
    rms = np.sqrt(np.mean(ref2 * ref2, axis=1, keepdims=True))
    floor = np.maximum(np.abs(ref2), rms)
    num = np.abs(out2 - ref2)
    zero = floor == 0
    if np.any(num[zero] > 0):
        return float("inf")
    return float(np.max(np.where(zero, 0.0, num / np.where(zero, 1.0, floor))))


def upload(cfg: W.MoEConfig, arrs) -> dict:
    t = {k: dev_bf16(v) for k, v in arrs.items() if v is not None and k != "bias"}
    t["bias"] = dev(arrs["bias"]) if arrs.get("bias") is not None else None
    return t


def sample_tokens(T: int, n: int, seed: int = 0, must=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    base = {0, T - 1} | set(int(m) for m in must)
    extra = rng.choice(T, size=min(T, n), replace=False).tolist()
    return np.array(sorted(base | set(extra))[: max(n, len(base))], dtype=np.int64)
