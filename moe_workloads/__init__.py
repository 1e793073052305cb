"""Seeded synthetic inputs for the routed grouped-GEMM MoE layer.

This module only draws numbers and lays them out; it performs none of the
layer's arithmetic (no routing, no matmul, no activation).  Both the CPU
oracle's tests and the GPU path's tests/bench take their inputs from here, so
the two sides always see byte-identical bf16 tensors.

Workload shapes: the model-shape rows used below are the DeepSeek-V3 and
Qwen3-30B rows of Table 1 ("MoE model configurations") on the Weave page
(Huang et al., "Weave: Fine-Grained Dynamic SM Scheduling in an MoE
Megakernel", §5.1).  The pages route real prompts (ShareGPT, CodeSearchNet);
here Gaussian activations and a Gaussian router stand in for them.

Layouts (all row-major, bf16 stored as uint16 bit patterns):
  x         [T, d]                 activations
  w_router  [E, d]                 router weight, one row per expert
  w_gate    [E_loc, f, d]          gate projection, one row per output unit
  w_up      [E_loc, f, d]          up projection
  w_down    [E_loc, d, f]          down projection
  bias      [E] float32 or None    additive router bias (skewed workload only)
"""
from __future__ import annotations

import concurrent.futures as _cf
import hashlib
import json
import os
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

__all__ = [
    "MoEConfig", "CONFIGS", "generate", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "tensor_digest", "SKEW_BIAS_PATH", "load_skew_bias", "zipf_probs",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
SKEW_BIAS_PATH = os.path.join(_HERE, "skew_bias.json")

# Tensor ids for the per-tensor seed sequences.
_TID = {"x": 0, "w_router": 1, "w_gate": 2, "w_up": 3, "w_down": 4}
# Elements per independently seeded block: makes the stream independent of
# the number of generator threads.
_BLOCK = 1 << 22


@dataclass(frozen=True)
class MoEConfig:
    """One MoE layer workload.  Local experts are [e_lo, e_hi)."""
    name: str
    config_id: int
    T: int
    d: int
    f: int
    E: int
    k: int
    e_lo: int = 0
    e_hi: Optional[int] = None
    skew: Optional[str] = None          # "zipf1.2" for the skewed router
    out_fp32: bool = False              # fp32 partial outputs (expert-parallel share)
    seed: int = 0
    note: str = ""

    @property
    def E_hi(self) -> int:
        return self.E if self.e_hi is None else self.e_hi

    @property
    def E_loc(self) -> int:
        return self.E_hi - self.e_lo

    def scaled(self, **kw) -> "MoEConfig":
        """A copy with some fields replaced (used for reduced-size test cases)."""
        d = dict(self.__dict__)
        d.update(kw)
        return MoEConfig(**d)


CONFIGS: Dict[str, MoEConfig] = {
    c.name: c for c in [
        MoEConfig("tiny", 1, T=256, d=512, f=1024, E=8, k=2,
                  note="tiny layer, E=8 top-2"),
        MoEConfig("mixtral", 2, T=4096, d=4096, f=14336, E=8, k=2,
                  note="Mixtral-shape layer on one GPU, near-uniform load"),
        MoEConfig("fine", 3, T=8192, d=2048, f=768, E=128, k=8,
                  note="fine-grained, Qwen3-30B row of Weave Table 1"),
        MoEConfig("skewed", 4, T=4096, d=4096, f=14336, E=8, k=2, skew="zipf1.2",
                  note="Mixtral shapes, router biased to Zipf(1.2) expert load"),
        MoEConfig("dsv3_share", 5, T=8192, d=7168, f=2048, E=256, k=8, e_lo=0, e_hi=32,
                  out_fp32=True,
                  note="one GPU's expert-parallel share at DeepSeek-V3 shape "
                       "(Weave Table 1): experts 0-31 of 256, fp32 partials"),
    ]
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); return uint16 bits.

    Inputs here are finite; NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(shape, std: float, seed: int, config_id: int, tensor_id: int,
                 pool: Optional[_cf.Executor]) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nblk = (n + _BLOCK - 1) // _BLOCK

    def fill(b: int) -> None:
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        ss = np.random.SeedSequence([seed, config_id, tensor_id, b])
        g = np.random.Generator(np.random.PCG64(ss))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(v)

    if pool is None or nblk == 1:
        for b in range(nblk):
            fill(b)
    else:
        list(pool.map(fill, range(nblk)))
    return out.reshape(shape)


def zipf_probs(n: int, s: float) -> np.ndarray:
    """Zipf(s) probabilities over n ranks: p_i proportional to 1/i^s, i = 1..n."""
    w = 1.0 / np.arange(1, n + 1, dtype=np.float64) ** s
    return w / w.sum()


def load_skew_bias(cfg: MoEConfig) -> np.ndarray:
    """Stored router bias for the skewed workload (written by the calibration
    script that sits beside the oracle)."""
    with open(SKEW_BIAS_PATH) as fh:
        doc = json.load(fh)
    key = f"{cfg.name}:T{cfg.T}:d{cfg.d}:E{cfg.E}:k{cfg.k}:seed{cfg.seed}"
    if key not in doc["bias"]:
        raise KeyError(f"no stored skew bias for {key}; run oracle/calibrate_skew_bias.py")
    return np.array(doc["bias"][key], dtype=np.float32)


def generate(cfg: MoEConfig, with_weights: bool = True, threads: Optional[int] = None,
             bias_override: Optional[np.ndarray] = None) -> Dict[str, Optional[np.ndarray]]:
    """Draw the seeded inputs of one workload.

    x ~ N(0,1); w_gate, w_up ~ N(0, std=1/sqrt(d)); w_down ~ N(0, std=1/sqrt(f));
    w_router ~ N(0, std=0.02).  Each is drawn in float32 and rounded to bf16.
    Only the local experts' FFN weights are drawn (experts [e_lo, e_hi)).
    """
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    pool = _cf.ThreadPoolExecutor(max_workers=threads) if threads > 1 else None
    try:
        s, cid = cfg.seed, cfg.config_id
        out: Dict[str, Optional[np.ndarray]] = {}
        out["x"] = _normal_bf16((cfg.T, cfg.d), 1.0, s, cid, _TID["x"], pool)
        out["w_router"] = _normal_bf16((cfg.E, cfg.d), 0.02, s, cid, _TID["w_router"], pool)
        if with_weights:
            out["w_gate"] = _normal_bf16((cfg.E_loc, cfg.f, cfg.d), 1.0 / np.sqrt(cfg.d), s, cid,
                                         _TID["w_gate"], pool)
            out["w_up"] = _normal_bf16((cfg.E_loc, cfg.f, cfg.d), 1.0 / np.sqrt(cfg.d), s, cid,
                                       _TID["w_up"], pool)
            out["w_down"] = _normal_bf16((cfg.E_loc, cfg.d, cfg.f), 1.0 / np.sqrt(cfg.f), s, cid,
                                         _TID["w_down"], pool)
        if bias_override is not None:
            out["bias"] = np.ascontiguousarray(bias_override, dtype=np.float32)
        elif cfg.skew is not None:
            out["bias"] = load_skew_bias(cfg)
        else:
            out["bias"] = None
        return out
    finally:
        if pool is not None:
            pool.shutdown()


def tensor_digest(arrs: Dict[str, Optional[np.ndarray]]) -> str:
    """SHA-256 over the generated tensors (names, shapes, bytes)."""
    h = hashlib.sha256()
    for name in sorted(arrs):
        a = arrs[name]
        if a is None:
            continue
        h.update(name.encode())
        h.update(str(a.shape).encode())
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
