"""GPU parity of the W8A8 (E4M3) path against the oracle, one GEMM at a time.

The quantiser decides integers (codes) from exact inputs, so its codes and
scales must equal the oracle's bit for bit.  The two GEMMs are then checked
separately, each against the oracle evaluated on the GPU's own inputs, with
bounds fixed here before any run:

 * GEMM0 + SiLU-mul (moe_gate_up_fp8): h against the oracle's unrounded h,
   |h_gpu - h| <= TOL_H * max(|h|, rms of the row's h).  h is rounded to bf16
   (half an ulp: at most 2^-8 of |h|), and g and u carry the fp8 matrix
   core's step error, at most ALPHA_F8 = 2^-11 of (sum |p| + |accumulator|)
   per 64-product step (tests/test_gpu_premises.py measures it: 2^-11.3 at
   most) -- for these inputs a few 1e-4 of the products' magnitude sum, i.e.
   well under an ulp of h at the row's rms; TOL_H = 2^-6 is two ulps plus
   margin.
 * That error moves h across an E4M3 rounding boundary now and then, so some
   of h's codes differ from the oracle's.  At most FLIP_CAP = 1% of them may,
   and a row's scale may differ in at most 1% of the rows (a changed row
   maximum).  A differing code may lie more than one step away: the error
   is relative to the row while an E4M3 step is relative to the element, so
   for an element far below the row maximum one bf16 ulp of the row's rms can
   span two steps (the GPU's codes are still the oracle quantiser's codes of
   the GPU's h, which the quantiser tests pin).
 * GEMM1 (moe_down_fp8) against the oracle's down projection of the GPU's own
   h codes and scales: the R10 per-token metric within TOL_LAYER = 2e-2 (y is
   rounded to bf16; the matrix-core error adds a few 1e-3).
 * combine against the oracle's weighted sum of the GPU's own y: bf16 output
   within 2^-8, float32 within 1e-5.
 * End to end against the whole W8A8 oracle (its own h codes): the root mean
   square error over all checked outputs within 6e-3 (a wrong operand, scale
   or k-step gives 1e-1 and more); the per-token differences there are the
   flipped codes above, each one E4M3 step of one h element times its weights.

moe_expert_ffn_fp8 and moe_layer_fp8 must equal the chained halves bit for bit.
Inputs: the seeded workloads; the permutation is the oracle's own.
"""
import zlib

import numpy as np
import pytest

import moe_workloads as W
import oracle
from gpu_util import TOL_LAYER, dev, dev_bf16, host_bits, host_f32, rel_err, say

TOL_H = 2.0 ** -6
FLIP_CAP = 1e-2
TOL_FP8_RMS = 6e-3

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


def test_quantizer_bit_exact_on_every_bf16_value():
    """Every finite bf16 value of magnitude at most 448, once each, in rows
    whose maximum is 448 (scale 1, so each value is encoded as it is): the
    codes of the whole input domain of the encoder, subnormal codes, ties and
    signed zeros included, against the oracle bit for bit.  (A row with
    another power-of-two scale feeds the encoder the same set of floats,
    shifted exactly; magnitudes below 2^-10 all round to zero.)"""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = W.bf16_bits_to_f32(b)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    vals = b[keep]
    cols = 256
    rows = -(-vals.size // (cols - 1))
    grid = np.zeros((rows, cols - 1), np.uint16)
    grid.reshape(-1)[:vals.size] = vals
    xb = np.concatenate([np.full((rows, 1), W.f32_to_bf16_bits(np.float32([448.0]))[0],
                                 np.uint16), grid], axis=1)
    say(f"moe_quantize_fp8 every bf16 value: {vals.size} values in {rows} rows")
    q, s = M.moe_quantize_fp8(dev_bf16(xb))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_rows_e4m3(xb)
    assert np.all(rs == 1.0)
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


def _signed_index(q):
    """Position of an E4M3 code in value order (+-0 both 0)."""
    q = q.astype(np.int64)
    return np.where(q & 0x80, -(q & 0x7F), q & 0x7F)


def _check_gemm_halves(cfg, xrows, eor, h_dev, y_dev, rows, ref_w):
    """GEMM0 and GEMM1 of the W8A8 FFN on the given routed rows, each against
    the oracle on the GPU's own inputs (bounds in the module docstring).
    Returns (y_gpu, y_full) float64 for the end-to-end rms check."""
    rgq, rgs, ruq, rus, rdq, rds = ref_w
    h_ref = oracle.gate_up_rows_fp8(xrows, eor, rgq, rgs, ruq, rus)
    hb_gpu = host_bits(h_dev[torch.as_tensor(rows, device="cuda")])
    err_h = rel_err(W.bf16_bits_to_f32(hb_gpu), h_ref)
    y_full, h_round = oracle.expert_rows_fp8(xrows, eor, rgq, rgs, ruq, rus, rdq, rds,
                                             want_h=True)
    q_gpu, s_gpu = oracle.quantize_rows_e4m3(hb_gpu)   # the GPU's own codes (quantiser pinned)
    q_ref, s_ref = oracle.quantize_rows_e4m3(W.f32_to_bf16_bits(h_round.astype(np.float32)))
    same_scale = s_gpu == s_ref
    diff = (q_gpu != q_ref) & same_scale[:, None]
    flips = float(diff.sum()) / max(int(same_scale.sum()) * q_gpu.shape[1], 1)
    step = np.abs(_signed_index(q_gpu) - _signed_index(q_ref))[same_scale]
    say(f"  GEMM0: h rel err {err_h:.3e}; {flips:.2e} of h codes differ "
        f"(max {int(step.max()) if step.size else 0} step); "
        f"{int((~same_scale).sum())} of {len(rows)} rows with another scale")
    assert err_h <= TOL_H
    assert flips <= FLIP_CAP
    assert (~same_scale).sum() <= max(1, 0.01 * len(rows))
    y_ref = oracle.down_rows_fp8(q_gpu, s_gpu, eor, rdq, rds)
    y_gpu = host_f32(y_dev[torch.as_tensor(rows, device="cuda")]).astype(np.float64)
    err_y = rel_err(y_gpu, y_ref)
    say(f"  GEMM1 on the GPU's own h codes: rel err {err_y:.3e}")
    assert err_y <= TOL_LAYER
    return y_gpu, y_full


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_ffn_matches_oracle(name):
    cfg = FP8_CASES[name].scaled(name=name)
    arrs = W.generate(cfg)
    r_ids, _ = oracle.route(arrs["x"], arrs["w_router"], cfg.k, bias=arrs["bias"])
    _, ro, rp, _ = oracle.permute(r_ids, cfg.E, cfg.e_lo, cfg.E_hi)
    _fp8_ffn_case(name, cfg, arrs, ro, rp)


def test_fp8_ffn_partly_filled_m_tiles_every_row_block_count():
    # the row counts of the bf16 test of the same name: every pair of valid
    # 32-row blocks in the two halves of an expert's last m-tile
    counts = np.array([1, 31, 32, 33, 64, 80, 97, 128, 129, 160, 180, 224, 255, 256, 257, 300,
                       513])
    E, N = len(counts), int(counts.sum())
    cfg = W.CONFIGS["tiny"].scaled(name="partial_tiles", T=N, d=256, f=512, E=E, k=1, seed=22)
    arrs = W.generate(cfg)
    ro = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    _fp8_ffn_case("partial_tiles", cfg, arrs, ro, np.arange(N), all_rows=True)


def _fp8_ffn_case(name, cfg, arrs, ro, rp, all_rows=False):
    D = M.MoEDims.make(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.e_lo, cfg.E_hi)
    N = int(ro[-1])
    (gq, gs), (rgq, rgs) = _quant_both("w_gate", arrs["w_gate"])
    (uq, us), (ruq, rus) = _quant_both("w_up", arrs["w_up"])
    (dq, ds), (rdq, rds) = _quant_both("w_down", arrs["w_down"])
    cap = cfg.T * cfg.k
    xp = np.zeros((max(cap, 1), cfg.d), np.uint16)
    xp[:N] = arrs["x"][rp]
    xp_d, off_d = dev_bf16(xp), dev(ro.astype(np.int32))
    say(f"moe_gate_up_fp8 / moe_down_fp8 {name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} "
        f"k={cfg.k} N={N}")
    h = M.moe_gate_up_fp8(D, xp_d, off_d, gq, gs, uq, us)
    y = M.moe_down_fp8(D, h, off_d, dq, ds)
    say(f"moe_expert_ffn_fp8 {name}")
    y_all = M.moe_expert_ffn_fp8(D, xp_d, off_d, gq, gs, uq, us, dq, ds)
    torch.cuda.synchronize()
    if N == 0:
        return
    assert torch.equal(y_all[:N].view(torch.int16), y[:N].view(torch.int16)), \
        "moe_expert_ffn_fp8 != moe_down_fp8(moe_gate_up_fp8)"
    rows = np.arange(N) if N <= 1200 or all_rows else np.unique(
        np.concatenate([[0, N - 1], ro[1:-1].clip(0, N - 1),
                        np.random.default_rng(1).choice(N, 40, replace=False)]))
    eor = (np.searchsorted(ro, rows, side="right") - 1).astype(np.int32)
    y_gpu, y_full = _check_gemm_halves(cfg, arrs["x"][rp[rows]], eor, h, y, rows,
                                       (rgq, rgs, ruq, rus, rdq, rds))
    rms = float(np.sqrt(np.mean((y_gpu - y_full) ** 2) / np.mean(y_full ** 2)))
    say(f"  end to end: rms err {rms:.3e} over {len(rows)} rows")
    assert rms <= TOL_FP8_RMS
    # repeatable: a second call gives the same bits
    y2 = M.moe_expert_ffn_fp8(D, xp_d, off_d, gq, gs, uq, us, dq, ds)
    torch.cuda.synchronize()
    assert torch.equal(y_all[:N].view(torch.int16), y2[:N].view(torch.int16))


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
    """moe_layer_fp8 (its default schedule, its persistent kernel, and the
    persistent kernel under a seeded adversarial schedule: producers delayed
    before they publish, claims reversed) bit for bit against the staged C-ABI
    calls (moe_route, moe_permute, moe_gate_up_fp8, moe_down_fp8,
    moe_combine); routing against the oracle exactly; each GEMM and the
    combine against the oracle on the GPU's own inputs, on the rows of sampled
    tokens."""
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
    say(f"moe_layer_fp8 persistent kernel {name}")
    P = M.MOE_SCHEDULE_PERSISTENT
    out_ps = M.moe_layer_fp8(D, x, wr, gq, gs, uq, us, dq, ds, bias=bias, out_dtype=dt,
                             opts=M.layer_opts(schedule=P))
    seed = zlib.crc32(name.encode()) | 1
    say(f"moe_layer_fp8 persistent kernel, perturbed schedule {name} seed={seed}")
    ws = torch.empty(M.moe_layer_fp8_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    out_pt = M.moe_layer_fp8(D, x, wr, gq, gs, uq, us, dq, ds, bias=bias, out_dtype=dt, ws=ws,
                             opts=M.layer_opts(schedule=P, perturb_seed=seed))
    torch.cuda.synchronize()
    assert M.moe_device_status(D, ws) == 0, "a flag wait timed out"
    bits = torch.int32 if dt == M.MOE_F32 else torch.int16
    assert torch.equal(out.view(bits), out_ps.view(bits)), "persistent != staged schedule"
    assert torch.equal(out.view(bits), out_pt.view(bits)), "perturbed != staged schedule"
    say(f"staged fp8 calls {name}")
    s_ids, s_gates, _ = M.moe_route(D, x, wr, bias)
    _, offsets, _, inv, xp = M.moe_permute(D, x, s_ids)
    h = M.moe_gate_up_fp8(D, xp, offsets, gq, gs, uq, us)
    y = M.moe_down_fp8(D, h, offsets, dq, ds)
    staged = M.moe_combine(D, y, inv, s_gates, out_dtype=dt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(bits), staged.view(bits)), "moe_layer_fp8 != staged calls"
    r_ids, r_g = oracle.route(arrs["x"], arrs["w_router"], cfg.k, bias=arrs["bias"])
    _, ro, rp, ri = oracle.permute(r_ids, cfg.E, cfg.e_lo, cfg.E_hi)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert np.abs(gates.cpu().numpy() - r_g).max() <= TOL_GATE
    tokens = np.arange(cfg.T) if cfg.T <= 400 else sample_tokens(cfg.T, 24, seed=2)
    need = np.unique(ri[tokens][ri[tokens] >= 0])
    g_h = gates.cpu().numpy()[tokens]
    got = host_f32(out[torch.as_tensor(tokens, device="cuda")])
    if need.size == 0:
        assert not np.any(got)
        return
    eor = (np.searchsorted(ro, need, side="right") - 1).astype(np.int32)
    y_gpu, y_full = _check_gemm_halves(cfg, arrs["x"][rp[need]], eor, h, y, need,
                                       (rgq, rgs, ruq, rus, rdq, rds))
    ycomb = np.zeros((max(int(ro[-1]), 1), cfg.d))
    ycomb[need] = y_gpu
    cref = oracle.combine(ycomb, ri[tokens], g_h)
    err_c = rel_err(got, cref)
    say(f"  combine of the GPU's own y: rel err {err_c:.3e}")
    assert err_c <= (1e-5 if dt == M.MOE_F32 else 2.0 ** -8)
    yfull = np.zeros_like(ycomb)
    yfull[need] = y_full
    ref = oracle.combine(yfull, ri[tokens], g_h)
    rms = float(np.sqrt(np.mean((got - ref) ** 2) / max(np.mean(ref ** 2), 1e-300)))
    say(f"  end to end: rms err {rms:.3e}, per-token {rel_err(got, ref):.3e} over "
        f"{len(tokens)} tokens")
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
    for sched in (M.MOE_SCHEDULE_AUTO, M.MOE_SCHEDULE_PERSISTENT, M.MOE_SCHEDULE_STAGED):
        say(f"moe_layer_fp8 no local rows, schedule {sched}")
        out = M.moe_layer_fp8(D, dev_bf16(arrs["x"]), dev_bf16(arrs["w_router"]), gq, gs, uq, us,
                              dq, ds, bias=dev(bias), out_dtype=M.MOE_F32,
                              opts=M.layer_opts(schedule=sched))
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0
