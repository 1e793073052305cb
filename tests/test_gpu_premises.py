"""The matrix-core rounding that two correctness arguments rest on, measured.

1. The fast router (E > 16) selects from bf16 matrix-core logit partials and
   keeps every expert whose logit could still reach the top k under a bound
   eps of |approx - logit|.  Its ids equal the exact path's only if that bound
   holds.  The bound assumes that one v_mfma_f32_32x32x16_bf16 step errs by at
   most BETA_BF16 * (sum over its products of |p| + |accumulator|).
2. The W8A8 FFN's GEMMs run on v_mfma_f32_32x32x64_f8f6f4, which does not add
   a 64-product step exactly; the fp8 parity bounds take its step error as at
   most ALPHA_F8 * (sum |p| + |accumulator|).

Both constants are stated here before the measurement and checked against
exact sums (float64 sums of exact products, whose own rounding is below
2^-48 of the same scale) on adversarial operands: wide exponent spreads
inside one step, one large product with many small ones of one sign,
cancelling halves, and an accumulator far larger or smaller than the step.
A chain of steps is checked against the per-step model summed over the
chain.  The router premise is then checked where it is used: on the fast
path's own approximate logits and bounds (moe_route_bounds) for router rows
with the same adversarial structure.
"""
import zlib

import numpy as np
import pytest

import moe_workloads as W
import oracle
from gpu_util import dev, dev_bf16, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_grouped_gemm_moe_amd as M

BETA_BF16 = 2.0 ** -20   # bf16 step: as if each of its 16 additions rounded once (u = 2^-24)
ALPHA_F8 = 2.0 ** -11    # E4M3 step: about 12-bit alignment of the 64 products


def _bf16(a):
    bits = W.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    return bits, W.bf16_bits_to_f32(bits).astype(np.float64)


def _spread(rng, shape, e_lo, e_hi, positive=False):
    """Values m * 2^e with 8-bit significands m in [1, 2) and e uniform in [e_lo, e_hi]."""
    m = 1.0 + rng.integers(0, 128, shape) / 128.0
    s = 1.0 if positive else np.where(rng.integers(0, 2, shape) == 1, 1.0, -1.0)
    return s * m * 2.0 ** rng.integers(e_lo, e_hi + 1, shape)


def _bf16_family(name, rng, n, steps=1):
    K = 16
    shp = (n, steps, 32, K)
    c = np.zeros((n, 32, 32))
    if name == "gauss":
        a, b = rng.standard_normal(shp), rng.standard_normal(shp)
    elif name == "gauss_acc":
        a, b = rng.standard_normal(shp), rng.standard_normal(shp)
        c = rng.standard_normal((n, 32, 32)) * 4.0 * 2.0 ** rng.integers(-12, 13, (n, 32, 32))
    elif name == "wide_exponents":
        a, b = _spread(rng, shp, -24, 0), _spread(rng, shp, -24, 0)
    elif name == "one_big_many_small":
        # per row: k = 0 large, the other 15 products 2^-s smaller, all positive
        a = _spread(rng, shp, 0, 0, positive=True)
        b = _spread(rng, shp, 0, 0, positive=True)
        sh = rng.integers(4, 31, (n, steps, 32, 1))
        a[..., 1:] *= 2.0 ** -sh
    elif name == "cancelling_halves":
        a = _spread(rng, shp, -6, 6)
        b = _spread(rng, shp, -6, 6)
        a[..., 8:] = a[..., :8]
        b[..., 8:] = -b[..., :8]
        b[..., 15] *= 1.0 + 2.0 ** -7  # leave a small residue
    elif name == "acc_dominant":
        a, b = rng.standard_normal(shp), rng.standard_normal(shp)
        c = rng.standard_normal((n, 32, 32)) * 2.0 ** rng.integers(8, 20, (n, 32, 32))
    else:
        raise ValueError(name)
    (ab, af), (bb, bf) = _bf16(a), _bf16(b)
    c = c.astype(np.float32).astype(np.float64)
    return ab, af, bb, bf, c


def _e4m3_lut():
    return np.array([oracle.e4m3_value(x) if (x & 0x7F) != 0x7F else 0.0 for x in range(256)])


def _f8_codes(rng, shape, lo=0, hi=0x7E, positive=False):
    q = rng.integers(lo, hi + 1, shape)
    if not positive:
        q = q | (rng.integers(0, 2, shape) << 7)
    return q.astype(np.uint8)


def _f8_family(name, rng, n, steps=1):
    shp = (n, steps, 32, 64)
    c = np.zeros((n, 32, 32))
    if name == "random_codes":
        a, b = _f8_codes(rng, shp), _f8_codes(rng, shp)
    elif name == "positive_codes":
        a, b = _f8_codes(rng, shp, positive=True), _f8_codes(rng, shp, positive=True)
    elif name == "one_big_many_small":
        a = _f8_codes(rng, shp, 0x01, 0x30, positive=True)
        b = _f8_codes(rng, shp, 0x01, 0x30, positive=True)
        a[..., 0] = 0x7E
        b[..., 0] = 0x7E
    elif name == "random_acc":
        a, b = _f8_codes(rng, shp), _f8_codes(rng, shp)
        c = rng.standard_normal((n, 32, 32)) * 2.0 ** rng.integers(-4, 24, (n, 32, 32))
    else:
        raise ValueError(name)
    lut = _e4m3_lut()
    c = c.astype(np.float32).astype(np.float64)
    return a, lut[a.astype(np.int64)], b, lut[b.astype(np.int64)], c


def _run_probe(kind, a_dev, b_dev, c):
    d = M.moe_probe_mfma(kind, a_dev, b_dev, dev(c.astype(np.float32)))
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


def _step_model(af, bf, c):
    """Exact result, and the per-step model's scale summed over the chain:
    sum over steps s of (sum_k |a b| of step s + |exact accumulator before s|)."""
    p = np.einsum("nsrk,nsck->nsrc", af, bf)
    ap = np.einsum("nsrk,nsck->nsrc", np.abs(af), np.abs(bf))
    acc = c[:, None] + np.concatenate([np.zeros_like(p[:, :1]), np.cumsum(p, axis=1)[:, :-1]],
                                      axis=1)
    return c + p.sum(axis=1), (ap + np.abs(acc)).sum(axis=1)


@pytest.mark.parametrize("family", ["gauss", "gauss_acc", "wide_exponents",
                                    "one_big_many_small", "cancelling_halves", "acc_dominant"])
def test_bf16_matrix_core_step_error(family):
    rng = np.random.default_rng(zlib.crc32(b'bf16' + family.encode()))
    ab, af, bb, bf, c = _bf16_family(family, rng, 256)
    say(f"moe_probe_mfma bf16 one step, {family}")
    d = _run_probe(0, dev_bf16(ab), dev_bf16(bb), c)
    exact, scale = _step_model(af, bf, c)
    ratio = np.abs(d - exact) / np.maximum(scale, 1e-300)
    say(f"  bf16 step {family}: max |err| / (sum|p| + |c|) = {ratio.max():.3e} "
        f"(= 2^{np.log2(max(ratio.max(), 1e-300)):.2f}); assumed {BETA_BF16:.3e}")
    assert ratio.max() <= BETA_BF16


@pytest.mark.parametrize("family", ["gauss", "wide_exponents", "cancelling_halves"])
def test_bf16_matrix_core_chain_error(family):
    """64 dependent steps (one split-K partial of the router at d = 1024 per
    part): the error stays within the per-step model summed over the chain."""
    rng = np.random.default_rng(zlib.crc32(b'chain' + family.encode()))
    ab, af, bb, bf, c = _bf16_family(family, rng, 48, steps=64)
    say(f"moe_probe_mfma bf16 64-step chain, {family}")
    d = _run_probe(0, dev_bf16(ab), dev_bf16(bb), c)
    exact, scale = _step_model(af, bf, c)
    ratio = np.abs(d - exact) / np.maximum(scale, 1e-300)
    say(f"  bf16 chain {family}: max |err| / sum_s(sum|p_s| + |acc_s|) = {ratio.max():.3e}")
    assert ratio.max() <= BETA_BF16


@pytest.mark.parametrize("family", ["random_codes", "positive_codes", "one_big_many_small",
                                    "random_acc"])
def test_fp8_matrix_core_step_error(family):
    rng = np.random.default_rng(zlib.crc32(b'fp8' + family.encode()))
    a, af, b, bf, c = _f8_family(family, rng, 256)
    say(f"moe_probe_mfma E4M3 one step, {family}")
    d = _run_probe(1, dev(a), dev(b), c)
    exact, scale = _step_model(af, bf, c)
    ratio = np.abs(d - exact) / np.maximum(scale, 1e-300)
    say(f"  fp8 step {family}: max |err| / (sum|p| + |c|) = {ratio.max():.3e} "
        f"(= 2^{np.log2(max(ratio.max(), 1e-300)):.2f}); assumed {ALPHA_F8:.3e}")
    assert ratio.max() <= ALPHA_F8


def _router_rows(kind, rng, T, d, E):
    if kind == "gauss":
        x = rng.standard_normal((T, d))
        w = rng.standard_normal((E, d)) * 0.02
    elif kind == "wide_exponents":
        x = _spread(rng, (T, d), -20, 4)
        w = _spread(rng, (E, d), -20, 0)
    elif kind == "one_big_many_small":
        # in every 16-wide k-step one large product, the rest 2^-s smaller, one sign
        x = _spread(rng, (T, d), 0, 0, positive=True)
        w = _spread(rng, (E, d), -6, -6, positive=True)
        x.reshape(T, d // 16, 16)[..., 1:] *= 2.0 ** -rng.integers(4, 25, (T, d // 16, 1))
    elif kind == "cancelling":
        # within every 16-wide k-step the second half cancels the first up to
        # a small residue, so each logit is tiny next to sum |x w|
        x = _spread(rng, (T, d), -4, 4)
        w = _spread(rng, (E, d), -8, -4)
        x.reshape(T, d // 16, 16)[..., 8:] = x.reshape(T, d // 16, 16)[..., :8]
        w3 = w.reshape(E, d // 16, 16)
        w3[..., 8:] = -w3[..., :8]
        w3[..., 15] *= 1.0 + 2.0 ** -7
    elif kind == "near_ties":
        x = rng.standard_normal((T, d))
        w = rng.standard_normal((E, d)) * 0.02
        w[1::2] = w[0::2] * (1.0 + 2.0 ** -7)  # pairs of experts a hair apart
    else:
        raise ValueError(kind)
    return W.f32_to_bf16_bits(x.astype(np.float32)), W.f32_to_bf16_bits(w.astype(np.float32))


@pytest.mark.parametrize("shape", [(384, 2048, 128, 8), (256, 7168, 256, 8)],
                         ids=["d2048_E128", "d7168_E256"])
@pytest.mark.parametrize("kind", ["gauss", "wide_exponents", "one_big_many_small", "cancelling",
                                  "near_ties"])
def test_fast_router_bound_holds_and_ids_exact(shape, kind):
    T, d, E, k = shape
    rng = np.random.default_rng(zlib.crc32(f'{kind}{d}'.encode()))
    xb, wb = _router_rows(kind, rng, T, d, E)
    D = M.MoEDims.make(T, d, 1024, E, k)
    x, wr = dev_bf16(xb), dev_bf16(wb)
    say(f"moe_route_bounds {kind} T={T} d={d} E={E}")
    approx, eps = M.moe_route_bounds(D, x, wr)
    torch.cuda.synchronize()
    logits = oracle.router_logits(xb, wb)   # defined-order float32, as the exact path
    err = np.abs(approx.cpu().numpy().astype(np.float64) - logits)
    ratio = err / eps.cpu().numpy().astype(np.float64)
    say(f"  router {kind} d={d}: max |approx - logit| / eps = {ratio.max():.3e}")
    assert np.all(np.isfinite(ratio)) and ratio.max() <= 1.0
    # and the fast path's ids and gates equal the exact path's
    say(f"moe_route exact and fast paths {kind} d={d}")
    ids_x, g_x, _ = M.moe_route(D, x, wr, want_logits=True)
    ids_f, g_f, _ = M.moe_route(D, x, wr)
    torch.cuda.synchronize()
    r_ids, _ = oracle.topk_gates(logits, k)
    assert np.array_equal(ids_x.cpu().numpy(), r_ids)
    assert torch.equal(ids_f, ids_x)
    assert torch.equal(g_f.view(torch.int32), g_x.view(torch.int32))
