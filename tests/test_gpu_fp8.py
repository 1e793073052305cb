"""GPU parity of the W8A8 (E4M3) path against the oracle.

The quantiser decides integers (codes) from exact inputs, so its codes and
scales must equal the oracle's bit for bit.  The fp8 FFN is compared with the
oracle's float64 evaluation of the same quantised operands.  The fp8 matrix
cores do not add a 64-product step exactly: measured on gfx950, one
v_mfma_f32_32x32x64_f8f6f4 is off by up to 2.8e-4 of the sum of the
products' magnitudes (about 12-bit alignment).  That error moves a few h
values across an E4M3 rounding boundary (about 0.2% of h codes differ from
the oracle's), and each such code moves y by one E4M3 step of that h element
times its weights.  A step is at most 2^-3 of the element; against a row of
y, whose rms grows as sqrt(f) times the rms of h and of the weights, one
moved code weighs about 2^-3 * (|h_j| / rms h) * (|w_ij| / rms w) / sqrt(f),
and the two magnitude ratios together reach about 16 in the tails of these
Gaussian inputs.  Bounds: max(6e-2, 2 / sqrt(f)) per token (the rel_err
metric of the bf16 path; 2.9e-2 measured at f = 1024, 7.2e-2 at f = 512
with k = 1, where no second expert's share dilutes it) and 6e-3 for the
root-mean-square error over all checked outputs (a wrong operand, scale or
k-step gives errors of 1e-1 and more).
Inputs: the seeded workloads; the permutation is the oracle's own.
"""
import numpy as np
import pytest

import moe_workloads as W
import oracle
from gpu_util import dev, dev_bf16, host_f32, rel_err, say

TOL_FP8_RMS = 6e-3


def tol_fp8_token(f):
    return max(6e-2, 2.0 / np.sqrt(f))


torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_grouped_gemm_moe_amd as M


def _quant_both(name, w_bits):
    """Quantise a bf16 weight tensor [EL, out, K] on the GPU and in the
    oracle; assert equal codes and scales; return both sides."""
    EL, n_out, K = w_bits.shape
    say(f"moe_quantize_fp8 {name} {EL}x{n_out}x{K}")
    q, s = M.moe_quantize_fp8(dev_bf16(w_bits))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_rows_e4m3(w_bits.reshape(-1, K))
    assert np.array_equal(q.cpu().numpy().reshape(-1, K), rq), f"{name} codes"
    assert np.array_equal(s.cpu().numpy().reshape(-1).view(np.uint32), rs.view(np.uint32)), \
        f"{name} scales"
    return (q, s), (rq.reshape(EL, n_out, K), rs.reshape(EL, n_out))


def test_quantizer_bit_exact_on_edge_rows():
    rng = np.random.default_rng(21)
    rows, cols = 64, 512
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= (2.0 ** rng.integers(-30, 30, (rows, 1))).astype(np.float32)
    x[0] = 0.0                                   # all-zero row: scale 1, codes 0
    x[1] = 0.0
    x[1, 7] = 448.0                              # exact maximum
    x[2, :] = 1e-38                              # tiny row (scale clamped at 2^-126)
    x[3, 5] = 3.0e38                             # huge element
    x[4] = np.linspace(-1, 1, cols)              # many exact midpoints after scaling
    x[5, ::2] = -0.0
    xb = W.f32_to_bf16_bits(x)
    say("moe_quantize_fp8 edge rows")
    q, s = M.moe_quantize_fp8(dev_bf16(xb))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_rows_e4m3(xb)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


FP8_CASES = {
    "tiny": W.CONFIGS["tiny"],
    "ragged_T300": W.CONFIGS["tiny"].scaled(T=300, d=256, f=512, seed=3),
    "local_subset_e16k4": W.CONFIGS["tiny"].scaled(T=200, d=512, f=256, E=16, k=4, e_lo=3,
                                                   e_hi=11, out_fp32=True, seed=4),
    "e128k8": W.CONFIGS["tiny"].scaled(T=160, d=256, f=256, E=128, k=8, seed=7),
    "multi_tile_rows": W.CONFIGS["tiny"].scaled(T=1000, d=256, f=256, E=4, k=2, seed=10),
    "k_equals_E": W.CONFIGS["tiny"].scaled(T=64, d=256, f=256, E=4, k=4, seed=5),
    "single_expert": W.CONFIGS["tiny"].scaled(T=77, d=256, f=256, E=1, k=1, seed=8),
    "one_token": W.CONFIGS["tiny"].scaled(T=1, d=256, f=256, E=8, k=2, seed=9),
    "mixtral": W.CONFIGS["mixtral"],
}


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_ffn_matches_oracle(name):
    cfg = FP8_CASES[name].scaled(name=name)
    arrs = W.generate(cfg)
    D = M.MoEDims.make(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.e_lo, cfg.E_hi)
    r_ids, _ = oracle.route(arrs["x"], arrs["w_router"], cfg.k, bias=arrs["bias"])
    _, ro, rp, _ = oracle.permute(r_ids, cfg.E, cfg.e_lo, cfg.E_hi)
    N = int(ro[-1])
    (gq, gs), (rgq, rgs) = _quant_both("w_gate", arrs["w_gate"])
    (uq, us), (ruq, rus) = _quant_both("w_up", arrs["w_up"])
    (dq, ds), (rdq, rds) = _quant_both("w_down", arrs["w_down"])
    cap = cfg.T * cfg.k
    xp = np.zeros((max(cap, 1), cfg.d), np.uint16)
    xp[:N] = arrs["x"][rp]
    say(f"moe_expert_ffn_fp8 {name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k} N={N}")
    y = M.moe_expert_ffn_fp8(D, dev_bf16(xp), dev(ro.astype(np.int32)), gq, gs, uq, us, dq, ds)
    torch.cuda.synchronize()
    if N == 0:
        return
    rows = np.arange(N) if N <= 1200 else np.unique(
        np.concatenate([[0, N - 1], ro[1:-1].clip(0, N - 1),
                        np.random.default_rng(1).choice(N, 40, replace=False)]))
    expert_of_row = (np.searchsorted(ro, rows, side="right") - 1).astype(np.int32)
    ref = oracle.expert_rows_fp8(arrs["x"][rp[rows]], expert_of_row, rgq, rgs, ruq, rus, rdq, rds)
    got = host_f32(y[torch.as_tensor(rows, device="cuda")])
    err = rel_err(got, ref)
    rms = float(np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2)))
    say(f"  fp8 ffn rel err {err:.3e}, rms err {rms:.3e} over {len(rows)} rows")
    assert err <= tol_fp8_token(cfg.f)
    assert rms <= TOL_FP8_RMS
    # repeatable: a second call gives the same bits
    y2 = M.moe_expert_ffn_fp8(D, dev_bf16(xp), dev(ro.astype(np.int32)), gq, gs, uq, us, dq, ds)
    torch.cuda.synchronize()
    assert torch.equal(y[:N].view(torch.int16), y2[:N].view(torch.int16))


LAYER_CASES = {k: FP8_CASES[k] for k in ("tiny", "ragged_T300", "local_subset_e16k4", "mixtral")}


def _random_fp8_case(seed):
    """A seeded shape across the W8A8 path's range (f a multiple of 256):
    ragged T, E across both router paths, a random local expert range."""
    g = np.random.default_rng(3000 + seed)
    E = int(g.choice([1, 4, 8, 16, 17, 40]))
    k = int(g.integers(1, min(E, 4) + 1))
    e_lo = int(g.integers(0, E))
    e_hi = int(g.integers(e_lo + 1, E + 1))
    return W.CONFIGS["tiny"].scaled(
        T=int(g.integers(1, 500)), d=int(g.choice([256, 512, 768])),
        f=int(g.choice([256, 512, 768, 1280])), E=E, k=k, e_lo=e_lo, e_hi=e_hi,
        out_fp32=bool(g.integers(0, 2)), seed=400 + seed)


LAYER_CASES.update({f"rand{i}": _random_fp8_case(i) for i in range(6)})


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_fp8_layer_matches_oracle_and_staged_calls(name):
    """moe_layer_fp8 against the oracle's route -> permute -> W8A8 FFN ->
    combine on sampled tokens, and bit for bit against the staged C-ABI calls
    (moe_route, moe_permute, moe_expert_ffn_fp8, moe_combine)."""
    from gpu_util import TOL_GATE, sample_tokens
    cfg = LAYER_CASES[name].scaled(name=name)
    arrs = W.generate(cfg)
    D = M.MoEDims.make(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.e_lo, cfg.E_hi)
    (gq, gs), (rgq, rgs) = _quant_both("w_gate", arrs["w_gate"])
    (uq, us), (ruq, rus) = _quant_both("w_up", arrs["w_up"])
    (dq, ds), (rdq, rds) = _quant_both("w_down", arrs["w_down"])
    x, wr = dev_bf16(arrs["x"]), dev_bf16(arrs["w_router"])
    bias = dev(arrs["bias"]) if arrs["bias"] is not None else None
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    say(f"moe_layer_fp8 {name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    out = M.moe_layer_fp8(D, x, wr, gq, gs, uq, us, dq, ds, bias=bias, out_dtype=dt,
                          topk_ids_out=ids, topk_w_out=gates)
    torch.cuda.synchronize()
    # staged calls, same kernels
    say(f"staged fp8 calls {name}")
    s_ids, s_gates, _ = M.moe_route(D, x, wr, bias)
    _, offsets, _, inv, xp = M.moe_permute(D, x, s_ids)
    y = M.moe_expert_ffn_fp8(D, xp, offsets, gq, gs, uq, us, dq, ds)
    staged = M.moe_combine(D, y, inv, s_gates, out_dtype=dt)
    torch.cuda.synchronize()
    bits = torch.int32 if dt == M.MOE_F32 else torch.int16
    assert torch.equal(out.view(bits), staged.view(bits)), "moe_layer_fp8 != staged calls"
    # oracle
    r_ids, r_g = oracle.route(arrs["x"], arrs["w_router"], cfg.k, bias=arrs["bias"])
    _, ro, rp, ri = oracle.permute(r_ids, cfg.E, cfg.e_lo, cfg.E_hi)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert np.abs(gates.cpu().numpy() - r_g).max() <= TOL_GATE
    tokens = np.arange(cfg.T) if cfg.T <= 400 else sample_tokens(cfg.T, 24, seed=2)
    need = np.unique(ri[tokens][ri[tokens] >= 0])
    yref = np.zeros((max(int(ro[-1]), 1), cfg.d))
    if need.size:
        eor = (np.searchsorted(ro, need, side="right") - 1).astype(np.int32)
        yref[need] = oracle.expert_rows_fp8(arrs["x"][rp[need]], eor, rgq, rgs, ruq, rus, rdq, rds)
    ref = oracle.combine(yref, ri[tokens], gates.cpu().numpy()[tokens])
    got = host_f32(out[torch.as_tensor(tokens, device="cuda")])
    err = rel_err(got, ref)
    rms = float(np.sqrt(np.mean((got - ref) ** 2) / max(np.mean(ref ** 2), 1e-300)))
    say(f"  fp8 layer rel err {err:.3e}, rms err {rms:.3e} over {len(tokens)} tokens")
    assert err <= tol_fp8_token(cfg.f)
    assert rms <= TOL_FP8_RMS


def test_fp8_layer_no_local_rows_gives_exact_zeros():
    """Every token routed away from the local experts: no rows, zero output."""
    cfg = W.CONFIGS["tiny"].scaled(T=96, d=256, f=256, E=8, k=2, e_lo=4, e_hi=8, out_fp32=True,
                                   seed=12, name="fp8_no_local")
    arrs = W.generate(cfg)
    bias = np.zeros(cfg.E, np.float32)
    bias[:2] = 1000.0  # experts 0 and 1 win every token; both are remote
    D = M.MoEDims.make(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.e_lo, cfg.E_hi)
    (gq, gs), _ = _quant_both("w_gate", arrs["w_gate"])
    (uq, us), _ = _quant_both("w_up", arrs["w_up"])
    (dq, ds), _ = _quant_both("w_down", arrs["w_down"])
    say("moe_layer_fp8 no local rows")
    out = M.moe_layer_fp8(D, dev_bf16(arrs["x"]), dev_bf16(arrs["w_router"]), gq, gs, uq, us, dq,
                          ds, bias=dev(bias), out_dtype=M.MOE_F32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
