"""Calibrate the router bias of the skewed workload (run by hand; output committed).

The skewed workload keeps the Mixtral shapes but biases the router so the
per-expert load follows Zipf(s=1.2) over 8 experts.  The pages speak of
balanced and skewed routing (X-Stage, §5.3) without fixing a distribution; the
reading taken here: a per-expert float32 bias b is added to each logit (it
enters both selection and gates), started at b_e = ln p_e and refined by
b_e += 0.5 (ln p_e - ln share_e) on the seeded activations until every
expert's share of the T*k assignments is within 0.5 percentage points of p_e.
Zipf(1.2) over 8 ranks puts 42.9% of the load on the first expert.

This script calls only the oracle's router (it lives beside the oracle for that
reason) and writes moe_workloads/skew_bias.json.

    python oracle/calibrate_skew_bias.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, _ROOT)

import oracle  # noqa: E402
import moe_workloads as W  # noqa: E402


def calibrate(cfg: W.MoEConfig, s: float = 1.2, tol: float = 0.005, max_iter: int = 200):
    a = W.generate(cfg, with_weights=False, bias_override=np.zeros(cfg.E, np.float32))
    p = W.zipf_probs(cfg.E, s)
    b = np.log(p).astype(np.float32)
    share = None
    for it in range(max_iter):
        ids, _ = oracle.route(a["x"], a["w_router"], cfg.k, bias=b)
        share = np.bincount(ids.ravel(), minlength=cfg.E) / ids.size
        err = np.abs(share - p).max()
        print(f"iter {it}: max |share - p| = {err:.5f}  shares={np.round(share, 4).tolist()}")
        if err < tol:
            break
        b = (b + 0.5 * (np.log(p) - np.log(np.maximum(share, 1e-9)))).astype(np.float32)
    else:
        raise RuntimeError("calibration did not converge")
    return b, share, p


def main() -> None:
    doc = {"comment": "router bias of the skewed workload; written by "
                      "oracle/calibrate_skew_bias.py (calls only the oracle router)",
           "bias": {}, "shares": {}, "target": {}}
    for name in ("skewed",):
        cfg = W.CONFIGS[name]
        b, share, p = calibrate(cfg)
        key = f"{cfg.name}:T{cfg.T}:d{cfg.d}:E{cfg.E}:k{cfg.k}:seed{cfg.seed}"
        doc["bias"][key] = [float(v) for v in b]
        doc["shares"][key] = [float(v) for v in share]
        doc["target"][key] = [float(v) for v in p]
    with open(W.SKEW_BIAS_PATH, "w") as fh:
        json.dump(doc, fh, indent=1)
    print("wrote", W.SKEW_BIAS_PATH)


if __name__ == "__main__":
    main()
