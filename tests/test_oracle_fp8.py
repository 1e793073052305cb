"""Pins of the oracle's W8A8 (fp8) functions against facts fixed outside the
oracle: the values the OCP 8-bit floating point definition gives E4M3 codes,
a closed-form rounding evaluated with numpy, exact cases, and a float64 dense
SwiGLU written with numpy matmuls (X-Stage §5.3 evaluates MegaMoE in W8A8)."""
import math

import numpy as np
import pytest

import moe_workloads as W
import oracle


def finite_values():
    """(code, value) of the 127 finite non-negative E4M3 codes."""
    return [(c, oracle.e4m3_value(c)) for c in range(0x7F)]


# ------------------------------------------------------------ E4M3 values

def test_e4m3_values_fixed_by_the_format():
    # exponent bias 7, 3 mantissa bits, subnormals at exponent field 0
    assert oracle.e4m3_value(0x00) == 0.0
    assert oracle.e4m3_value(0x38) == 1.0          # 0 0111 000
    assert oracle.e4m3_value(0x40) == 2.0          # 0 1000 000
    assert oracle.e4m3_value(0x3C) == 1.5          # 0 0111 100
    assert oracle.e4m3_value(0x7E) == 448.0        # largest finite: 2^8 * 1.75
    assert oracle.e4m3_value(0x08) == 2.0 ** -6    # smallest normal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9    # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    z = oracle.e4m3_value(0x80)
    assert z == 0.0 and math.copysign(1.0, z) < 0
    for c in range(0x7F):
        assert oracle.e4m3_value(c | 0x80) == -oracle.e4m3_value(c)


def test_e4m3_values_strictly_increasing():
    vals = [v for _, v in finite_values()]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    # each binade [2^k, 2^(k+1)) above the subnormals holds 8 evenly spaced values
    for k in range(-6, 9):
        binade = [v for v in vals if 2.0 ** k <= v < 2.0 ** (k + 1)]
        assert len(binade) == (7 if k == 8 else 8)
        assert np.allclose(np.diff(binade), 2.0 ** (k - 3), rtol=0, atol=0)


# ------------------------------------------------------------ E4M3 encode

def test_encode_round_trips_every_finite_code():
    for c, v in finite_values():
        assert oracle.e4m3_encode(v) == c
        if c:
            assert oracle.e4m3_encode(-v) == c | 0x80


def test_encode_midpoints_go_to_even_code():
    fv = finite_values()
    for (c0, v0), (c1, v1) in zip(fv, fv[1:]):
        mid = (v0 + v1) / 2  # exact in float32 (4 significant bits)
        assert np.float32(mid) == mid
        even = c0 if c0 % 2 == 0 else c1
        assert oracle.e4m3_encode(mid) == even
        # just off the midpoint: the nearer value
        lo = float(np.nextafter(np.float32(mid), np.float32(0)))
        hi = float(np.nextafter(np.float32(mid), np.float32(1e9)))
        assert oracle.e4m3_encode(lo) == c0 and oracle.e4m3_encode(hi) == c1


def closed_form_value(a):
    """Nearest E4M3 magnitude of a in [0, 448] by the format's quantum:
    2^(floor(log2 a) - 3) for normals, 2^-9 below 2^-6; numpy's round is
    half-to-even, which on these quanta is the even-code rule."""
    a = np.asarray(a, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    q = 2.0 ** (e - 3)
    return np.minimum(np.round(a / q) * q, 448.0)


def test_encode_matches_closed_form_rounding_on_a_sweep():
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.uniform(0, 448, 3000), 2.0 ** rng.uniform(-12, 8.8, 3000)])
    a = a.astype(np.float32).astype(np.float64)
    want = closed_form_value(a)
    got = np.array([oracle.e4m3_value(oracle.e4m3_encode(v)) for v in a])
    assert np.array_equal(got, want)


def test_encode_saturates_and_underflows():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.9) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # tie between 0 and 2^-9: even
    assert oracle.e4m3_encode(-2.0 ** -11) == 0x80     # rounds to -0
    assert oracle.e4m3_encode(1.5 * 2.0 ** -10) == 0x01


# ------------------------------------------------------------ row quantiser

def to_bf16(a):
    return W.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_quantize_rows_scale_is_smallest_power_of_two():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((40, 96)) * 2.0 ** rng.integers(-20, 20, (40, 1))).astype(np.float32)
    xb = to_bf16(x)
    xf = W.bf16_bits_to_f32(xb).astype(np.float64)
    q, s = oracle.quantize_rows_e4m3(xb)
    amax = np.abs(xf).max(axis=1)
    e = np.log2(s.astype(np.float64))
    assert np.array_equal(e, np.round(e))                       # powers of two
    assert np.all(amax <= 448.0 * s) and np.all(amax > 224.0 * s)  # smallest such
    # per element: within half a code step of x / s
    v = np.vectorize(oracle.e4m3_value)(q.astype(np.int64))
    t = xf / s[:, None]
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -6))) - 3)
    assert np.all(np.abs(v - t) <= step / 2)


def test_quantize_rows_exact_for_scaled_e4m3_rows_and_zero_row():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, (6, 64))
    codes[:, 5] = 0x7E  # row max 448 -> the scale is exactly the row's 2^e
    codes = codes | (rng.integers(0, 2, codes.shape) << 7)
    vals = np.vectorize(oracle.e4m3_value)(codes)
    e = np.array([-7, -3, 0, 2, 5, 11])
    x = vals * 2.0 ** e[:, None]
    q, s = oracle.quantize_rows_e4m3(to_bf16(x))
    assert np.array_equal(s, (2.0 ** e).astype(np.float32))
    # codes equal up to the sign of zero
    assert np.array_equal(np.where((codes & 0x7F) == 0, 0, codes), np.where((q & 0x7F) == 0, 0, q))
    qz, sz = oracle.quantize_rows_e4m3(np.zeros((2, 32), np.uint16))
    assert np.all(qz == 0) and np.all(sz == 1.0)


# ------------------------------------------------------------ fp8 FFN

def dec(q):
    lut = np.array([oracle.e4m3_value(c) for c in range(256)])
    return lut[np.asarray(q, dtype=np.int64)]


def test_fp8_ffn_equals_dense_swiglu_on_exact_operands():
    """Operands exact in E4M3 with non-uniform per-row / per-channel scales:
    GEMM0 must equal numpy's float64 dense products; GEMM1 is checked on the
    oracle's own (pinned) quantisation of h."""
    rng = np.random.default_rng(9)
    n, d, f, EL = 5, 64, 32, 2

    def exact_rows(rows, cols, e_lo, e_hi):
        c = rng.integers(0, 0x7F, (rows, cols)) | (rng.integers(0, 2, (rows, cols)) << 7)
        c[:, 0] = 0x7E  # fixes each row's scale at 2^e
        e = rng.integers(e_lo, e_hi, rows)
        return c.astype(np.uint8), (2.0 ** e).astype(np.float32)

    xc, xs = exact_rows(n, d, -12, -6)
    x = dec(xc) * xs[:, None].astype(np.float64)
    xb = to_bf16(x)
    assert np.array_equal(W.bf16_bits_to_f32(xb), x.astype(np.float32))
    wg, sg = zip(*[exact_rows(f, d, -14, -9) for _ in range(EL)])
    wu, su = zip(*[exact_rows(f, d, -14, -9) for _ in range(EL)])
    wd, sd = zip(*[exact_rows(d, f, -14, -9) for _ in range(EL)])
    wg, wu, wd = np.stack(wg), np.stack(wu), np.stack(wd)
    sg, su, sd = np.stack(sg), np.stack(su), np.stack(sd)
    eor = np.array([0, 1, 1, 0, 1], np.int32)
    y, h = oracle.expert_rows_fp8(xb, eor, wg, sg, wu, su, wd, sd, want_h=True)
    for r in range(n):
        e = eor[r]
        Wg = dec(wg[e]) * sg[e][:, None]
        Wu = dec(wu[e]) * su[e][:, None]
        g = Wg @ x[r]
        u = Wu @ x[r]
        href = g / (1.0 + np.exp(-g)) * u
        # h is href rounded to bf16
        assert np.all(np.abs(h[r] - href) <= np.abs(href) * 2.0 ** -8 + 1e-300)
        hb = to_bf16(h[r])
        assert np.array_equal(W.bf16_bits_to_f32(hb).astype(np.float64), h[r])
        hq, hs = oracle.quantize_rows_e4m3(hb[None, :])
        Wd = dec(wd[e]) * sd[e][:, None]
        yref = Wd @ (dec(hq[0]) * float(hs[0]))
        assert np.allclose(y[r], yref, rtol=1e-12, atol=1e-300)


def test_fp8_ffn_close_to_unquantised_ffn():
    """Quantisation error only: the W8A8 FFN of random bf16 data stays within
    E4M3's relative step of the float64 FFN (oracle.expert_rows, pinned)."""
    rng = np.random.default_rng(2)
    n, d, f, EL = 6, 128, 64, 2
    x = to_bf16(rng.standard_normal((n, d)))
    wg = to_bf16(rng.standard_normal((EL, f, d)) / math.sqrt(d))
    wu = to_bf16(rng.standard_normal((EL, f, d)) / math.sqrt(d))
    wd = to_bf16(rng.standard_normal((EL, d, f)) / math.sqrt(f))
    q = lambda w: oracle.quantize_rows_e4m3(w.reshape(-1, w.shape[-1]))
    (gq, gs), (uq, us), (dq, ds) = q(wg), q(wu), q(wd)
    eor = rng.integers(0, EL, n).astype(np.int32)
    y8 = oracle.expert_rows_fp8(x, eor, gq.reshape(wg.shape), gs.reshape(EL, f),
                                uq.reshape(wu.shape), us.reshape(EL, f),
                                dq.reshape(wd.shape), ds.reshape(EL, d))
    y = oracle.expert_rows(x, eor, wg, wu, wd)
    # E4M3 rounds each operand with relative error <= 2^-4 (rms ~2^-4/sqrt(3)
    # for uniform rounding); three roundings on the path stay well under 0.15
    rel = np.sqrt(((y8 - y) ** 2).mean(axis=1) / (y ** 2).mean(axis=1))
    assert np.all(rel < 0.15), rel
    assert np.all(rel > 1e-3), rel  # the quantisation is really applied


def test_fp8_gemm_halves_equal_dense_products_and_the_whole_ffn():
    """oracle.gate_up_rows_fp8 against numpy float64 dense products of the
    decoded codes with the row and channel scales (the textbook definition,
    computed here independently of the oracle's loops); its bf16 rounding is
    expert_rows_fp8's h.  oracle.down_rows_fp8 against a numpy dense product
    of given codes and scales; fed the oracle's own quantised h it reproduces
    expert_rows_fp8's y.  Non-uniform scales catch a scale on the wrong axis,
    random signs a dropped or mis-signed term, f != d a transposed operand."""
    rng = np.random.default_rng(31)
    n, d, f, EL = 7, 96, 48, 3
    x = to_bf16(rng.standard_normal((n, d)) * 2.0 ** rng.integers(-4, 4, (n, 1)))
    q = lambda w: oracle.quantize_rows_e4m3(w.reshape(-1, w.shape[-1]))
    wg = to_bf16(rng.standard_normal((EL, f, d)) * 2.0 ** rng.integers(-9, -2, (EL, f, 1)))
    wu = to_bf16(rng.standard_normal((EL, f, d)) * 2.0 ** rng.integers(-9, -2, (EL, f, 1)))
    wd = to_bf16(rng.standard_normal((EL, d, f)) * 2.0 ** rng.integers(-9, -2, (EL, d, 1)))
    (gq, gs), (uq, us), (dq, ds) = q(wg), q(wu), q(wd)
    gq, uq, dq = gq.reshape(wg.shape), uq.reshape(wu.shape), dq.reshape(wd.shape)
    gs, us, ds = gs.reshape(EL, f), us.reshape(EL, f), ds.reshape(EL, d)
    eor = rng.integers(0, EL, n).astype(np.int32)
    h = oracle.gate_up_rows_fp8(x, eor, gq, gs, uq, us)
    xq, xs = oracle.quantize_rows_e4m3(x)
    for r in range(n):
        e = eor[r]
        xr = dec(xq[r]) * float(xs[r])
        g = (dec(gq[e]) * gs[e][:, None].astype(np.float64)) @ xr
        u = (dec(uq[e]) * us[e][:, None].astype(np.float64)) @ xr
        href = g / (1.0 + np.exp(-g)) * u
        assert np.allclose(h[r], href, rtol=1e-12, atol=1e-300)
    y_whole, h_whole = oracle.expert_rows_fp8(x, eor, gq, gs, uq, us, dq, ds, want_h=True)
    hb = to_bf16(h)
    assert np.array_equal(W.bf16_bits_to_f32(hb).astype(np.float64), h_whole)
    # GEMM1 from arbitrary codes and scales
    hq = (rng.integers(0, 0x7F, (n, f)) | (rng.integers(0, 2, (n, f)) << 7)).astype(np.uint8)
    hs = (2.0 ** rng.integers(-10, 3, n)).astype(np.float32)
    y = oracle.down_rows_fp8(hq, hs, eor, dq, ds)
    for r in range(n):
        e = eor[r]
        yref = (dec(dq[e]) * ds[e][:, None].astype(np.float64)) @ (dec(hq[r]) * float(hs[r]))
        assert np.allclose(y[r], yref, rtol=1e-12, atol=1e-300)
    # the oracle's own quantised h reproduces the whole FFN
    hq2, hs2 = oracle.quantize_rows_e4m3(hb)
    assert np.array_equal(oracle.down_rows_fp8(hq2, hs2, eor, dq, ds), y_whole)
