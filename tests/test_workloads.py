"""Seeded input generator: bf16 rounding, determinism, distributions, and the
skewed workload's achieved expert shares."""
import numpy as np
import pytest

import moe_workloads as W
import oracle


def test_bf16_round_to_nearest_even_known_values():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38,
                     1.0 + 2 ** -8 + 2 ** -20], np.float32)
    bits = W.f32_to_bf16_bits(vals)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties to even -> 1.0 (0x3F80)
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 0x3F82
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x7F62, 0x3F81]
    assert W.bf16_bits_to_f32(np.array([0x3F80, 0xC020], np.uint16)).tolist() == [1.0, -2.5]


def test_generation_is_deterministic_and_seed_dependent():
    cfg = W.CONFIGS["tiny"]
    a = W.generate(cfg, threads=1)
    b = W.generate(cfg, threads=4)
    assert W.tensor_digest(a) == W.tensor_digest(b)
    c = W.generate(cfg.scaled(seed=1))
    assert W.tensor_digest(a) != W.tensor_digest(c)


def test_distributions():
    cfg = W.CONFIGS["tiny"]
    a = W.generate(cfg)
    f = lambda k: W.bf16_bits_to_f32(a[k]).astype(np.float64)
    assert abs(f("x").std() - 1.0) < 0.01
    assert abs(f("w_router").std() / 0.02 - 1.0) < 0.05
    assert abs(f("w_gate").std() * np.sqrt(cfg.d) - 1.0) < 0.01
    assert abs(f("w_up").std() * np.sqrt(cfg.d) - 1.0) < 0.01
    assert abs(f("w_down").std() * np.sqrt(cfg.f) - 1.0) < 0.01
    assert a["w_gate"].shape == (cfg.E_loc, cfg.f, cfg.d)
    assert a["w_down"].shape == (cfg.E_loc, cfg.d, cfg.f)
    assert a["bias"] is None


def test_ep_share_generates_only_local_expert_weights():
    cfg = W.CONFIGS["dsv3_share"]
    assert (cfg.E_loc, cfg.e_lo, cfg.E_hi) == (32, 0, 32)
    small = cfg.scaled(T=8, d=64, f=32)
    a = W.generate(small)
    assert a["w_gate"].shape == (32, 32, 64) and a["w_router"].shape == (256, 64)


def test_skewed_workload_follows_zipf_1_2():
    cfg = W.CONFIGS["skewed"]
    a = W.generate(cfg, with_weights=False)
    ids, _ = oracle.route(a["x"], a["w_router"], cfg.k, bias=a["bias"])
    share = np.bincount(ids.ravel(), minlength=cfg.E) / ids.size
    p = W.zipf_probs(cfg.E, 1.2)
    assert np.abs(share - p).max() < 0.005
    assert 0.42 < share[0] < 0.46


@pytest.mark.parametrize("name", ["mixtral", "fine"])
def test_gaussian_router_gives_near_uniform_load(name):
    cfg = W.CONFIGS[name].scaled(T=2048)
    a = W.generate(cfg, with_weights=False)
    ids, _ = oracle.route(a["x"], a["w_router"], cfg.k)
    share = np.bincount(ids.ravel(), minlength=cfg.E) / ids.size
    assert share.max() < 3.0 / cfg.E
