"""GPU parity: every C-ABI call against the CPU oracle.

Small and ragged cases are compared element by element; the five workload
shapes at full size are compared bit-exactly on routing and dispatch, on the
layer output of every token, and on FFN rows (all of them, or the first and
last row of every m-tile).  The fused moe_layer must also equal the staged
route -> permute -> expert_ffn -> combine path bit for bit: both run the same
tiles, so any difference is a scheduling or signaling error in the persistent
kernel -- under every tile order, and under a seeded adversarial schedule.
"""
import numpy as np
import pytest

import moe_workloads as W
import oracle
from gpu_util import (TOL_GATE, TOL_LAYER, dev, dev_bf16, host_bits, host_f32, rel_err, say,
                      sample_tokens, upload)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_grouped_gemm_moe_amd as M


def _dims(cfg):
    return M.MoEDims.make(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.e_lo, cfg.E_hi)


SMALL = {
    "tiny": W.CONFIGS["tiny"],
    "ragged_T300": W.CONFIGS["tiny"].scaled(T=300, d=256, f=384, seed=3),
    "local_subset_e16k4": W.CONFIGS["tiny"].scaled(T=200, d=512, f=256, E=16, k=4, e_lo=3,
                                                   e_hi=11, out_fp32=True, seed=4),
    "k_equals_E": W.CONFIGS["tiny"].scaled(T=64, d=256, f=128, E=4, k=4, seed=5),
    "k1": W.CONFIGS["tiny"].scaled(T=130, d=256, f=256, E=6, k=1, seed=6),
    "e128k8": W.CONFIGS["tiny"].scaled(T=160, d=256, f=128, E=128, k=8, seed=7),
    "single_expert": W.CONFIGS["tiny"].scaled(T=77, d=256, f=128, E=1, k=1, seed=8),
    "one_token": W.CONFIGS["tiny"].scaled(T=1, d=256, f=128, E=8, k=2, seed=9),
    "multi_tile_rows": W.CONFIGS["tiny"].scaled(T=1000, d=256, f=256, E=4, k=2, seed=10),
    "e32k4": W.CONFIGS["tiny"].scaled(T=300, d=512, f=128, E=32, k=4, seed=13),
    "e1024k64": W.CONFIGS["tiny"].scaled(T=40, d=256, f=128, E=1024, k=64, seed=14),
    "e256k8_local": W.CONFIGS["tiny"].scaled(T=700, d=1024, f=128, E=256, k=8, e_lo=32,
                                             e_hi=64, out_fp32=True, seed=15),
    # odd E above 16: the refine kernel's per-wave LDS regions must stay aligned
    "e17k3": W.CONFIGS["tiny"].scaled(T=150, d=256, f=128, E=17, k=3, seed=16),
}


def _bias_all_to_one(E, e):
    b = np.zeros(E, np.float32)
    b[e] = 1000.0
    return b


def _check_route(cfg, t, arrs):
    D = _dims(cfg)
    say(f"moe_route {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k}")
    ids, gates, logits = M.moe_route(D, t["x"], t["w_router"], t["bias"], want_logits=True)
    torch.cuda.synchronize()
    r_ids, r_g, r_l = oracle.route(arrs["x"], arrs["w_router"], cfg.k, bias=arrs["bias"],
                                   want_logits=True)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), r_l.view(np.uint32)), "logits"
    assert np.array_equal(ids.cpu().numpy(), r_ids), "topk ids"
    assert np.abs(gates.cpu().numpy() - r_g).max() <= TOL_GATE, "gates"
    # without the logits output the router takes its fast path (LDS-staged for
    # E <= 16, MFMA bounds + exact candidates above); same ids and gate bits
    say(f"moe_route fast path {cfg.name}")
    f_ids, f_gates, _ = M.moe_route(D, t["x"], t["w_router"], t["bias"])
    torch.cuda.synchronize()
    assert torch.equal(f_ids, ids), "fast-path ids"
    assert torch.equal(f_gates.view(torch.int32), gates.view(torch.int32)), "fast-path gates"
    return ids, gates, r_ids, r_g


def _check_permute(cfg, t, arrs, ids_dev, r_ids):
    D = _dims(cfg)
    say(f"moe_permute {cfg.name}")
    counts, offsets, perm, inv, xp = M.moe_permute(D, t["x"], ids_dev)
    torch.cuda.synchronize()
    rc, ro, rp, ri = oracle.permute(r_ids, cfg.E, cfg.e_lo, cfg.E_hi)
    N = int(ro[-1])
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy()[:N], rp)
    assert np.array_equal(inv.cpu().numpy(), ri)
    assert np.array_equal(host_bits(xp[:N]), arrs["x"][rp]), "x_perm rows"
    return offsets, inv, xp, ro, rp, ri, N


def _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N, rows=None):
    D = _dims(cfg)
    say(f"moe_expert_ffn {cfg.name} N={N}")
    y = M.moe_expert_ffn(D, xp, offsets, t["w_gate"], t["w_up"], t["w_down"])
    torch.cuda.synchronize()
    if N == 0:
        return y
    rows = np.arange(N) if rows is None else rows
    expert_of_row = (np.searchsorted(ro, rows, side="right") - 1).astype(np.int32)
    ref = oracle.expert_rows(arrs["x"][rp[rows]], expert_of_row, arrs["w_gate"], arrs["w_up"],
                             arrs["w_down"])
    got = host_f32(y[torch.as_tensor(rows, device="cuda")])
    err = rel_err(got, ref)
    say(f"  ffn rel err {err:.3e}")
    assert err <= TOL_LAYER
    return y


def _check_combine(cfg, t, y, inv, gates_dev, ri, r_g, N):
    D = _dims(cfg)
    yy = host_f32(y[:max(N, 1)]).astype(np.float64)
    ref = oracle.combine(yy, ri, gates_dev.cpu().numpy())
    for dt, tol in ((M.MOE_BF16, 2.0 ** -8), (M.MOE_F32, 1e-5)):
        say(f"moe_combine {cfg.name} dtype={dt}")
        out = M.moe_combine(D, y, inv, gates_dev, out_dtype=dt)
        torch.cuda.synchronize()
        assert rel_err(host_f32(out), ref) <= tol


def _check_layer(cfg, t, arrs, staged_out=None, tokens=None, opts=None):
    D = _dims(cfg)
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    say(f"moe_layer {cfg.name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k} "
        f"local=[{cfg.e_lo},{cfg.E_hi})")
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    out = M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t["bias"],
                      out_dtype=dt, topk_ids_out=ids, topk_w_out=gates, ws=ws, opts=opts)
    assert M.moe_device_status(D, ws) == 0
    tokens = np.arange(cfg.T) if tokens is None else tokens
    ref, r_ids, r_g = oracle.layer_tokens(tokens, arrs["x"], arrs["w_router"], arrs["w_gate"],
                                          arrs["w_up"], arrs["w_down"], cfg.k, cfg.e_lo, cfg.E_hi,
                                          bias=arrs["bias"])
    assert np.array_equal(ids.cpu().numpy()[tokens], r_ids)
    assert np.abs(gates.cpu().numpy()[tokens] - r_g).max() <= TOL_GATE
    got = host_f32(out[torch.as_tensor(tokens, device="cuda")])
    err = rel_err(got, ref)
    say(f"  layer rel err {err:.3e} over {len(tokens)} tokens")
    assert err <= TOL_LAYER
    if staged_out is not None:
        assert torch.equal(out.view(torch.int32) if dt == M.MOE_F32 else out.view(torch.int16),
                           staged_out.view(torch.int32) if dt == M.MOE_F32
                           else staged_out.view(torch.int16)), "fused != staged"
    return out


def _staged(cfg, t, y, inv, gates_dev):
    D = _dims(cfg)
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    return M.moe_combine(D, y, inv, gates_dev, out_dtype=dt)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_case_all_stages(name):
    cfg = SMALL[name].scaled(name=name)
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    offsets, inv, xp, ro, rp, ri, N = _check_permute(cfg, t, arrs, ids, r_ids)
    y = _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N)
    _check_combine(cfg, t, y, inv, gates, ri, r_g, N)
    staged = _staged(cfg, t, y, inv, gates)
    _check_layer(cfg, t, arrs, staged_out=staged)


def _random_case(seed):
    """A seeded shape drawn across the supported ranges: ragged T, d and f of
    several tiles, E across both router paths, k up to 6, a random local
    expert range and output dtype."""
    g = np.random.default_rng(1000 + seed)
    E = int(g.choice([1, 2, 3, 5, 8, 12, 16, 17, 24, 33, 64]))
    k = int(g.integers(1, min(E, 6) + 1))
    e_lo = int(g.integers(0, E))
    e_hi = int(g.integers(e_lo + 1, E + 1))
    return W.CONFIGS["tiny"].scaled(
        name=f"rand{seed}", T=int(g.integers(1, 600)), d=int(g.choice([256, 512, 768, 1280])),
        f=int(g.choice([128, 256, 384, 640, 896])), E=E, k=k, e_lo=e_lo, e_hi=e_hi,
        out_fp32=bool(g.integers(0, 2)), seed=200 + seed)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_all_stages(seed):
    cfg = _random_case(seed)
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    offsets, inv, xp, ro, rp, ri, N = _check_permute(cfg, t, arrs, ids, r_ids)
    y = _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N)
    staged = _staged(cfg, t, y, inv, gates)
    _check_layer(cfg, t, arrs, staged_out=staged)


@pytest.mark.parametrize("hot,k", [(5, 1), (2, 2)])
def test_degenerate_one_expert_takes_everything(hot, k):
    cfg = W.CONFIGS["tiny"].scaled(name=f"hot{hot}k{k}", T=260, d=256, f=256, E=8, k=k, seed=11)
    arrs = W.generate(cfg, bias_override=_bias_all_to_one(8, hot))
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    assert np.all(r_ids[:, 0] == hot)
    offsets, inv, xp, ro, rp, ri, N = _check_permute(cfg, t, arrs, ids, r_ids)
    assert np.diff(ro)[hot] == cfg.T
    y = _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N)
    staged = _staged(cfg, t, y, inv, gates)
    _check_layer(cfg, t, arrs, staged_out=staged)


def test_expert_with_more_m_tiles_than_one_group():
    # One expert takes all 4600 tokens: 18 m-tiles, so the expert-aligned
    # tile order splits it into groups of 16 and 2 m-tiles.  Fused must equal
    # staged bit for bit, and both must match the oracle.
    cfg = W.CONFIGS["tiny"].scaled(name="hot18", T=4600, d=256, f=256, E=8, k=1, seed=19)
    arrs = W.generate(cfg, bias_override=_bias_all_to_one(8, 2))
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    assert np.all(r_ids[:, 0] == 2)
    offsets, inv, xp, ro, rp, ri, N = _check_permute(cfg, t, arrs, ids, r_ids)
    assert (N + 255) // 256 == 18
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=40, replace=False)]))
    y = _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N, rows=rows)
    staged = _staged(cfg, t, y, inv, gates)
    _check_layer(cfg, t, arrs, staged_out=staged, tokens=sample_tokens(cfg.T, 40, seed=6))


# Row counts per expert whose last m-tile (count % 256 rows, 256 when that
# is 0) gives the two halves of the eight-wave tile every pair of valid
# 32-row blocks a last m-tile can have -- (1,0) (2,0) (3,0) (4,0) (4,1)
# (4,2) (4,3) (4,4) and full -- plus experts of several m-tiles.  Each wave
# runs a K loop specialised on its half's count, so each one is exercised.
PARTIAL_TILE_COUNTS = np.array([1, 31, 32, 33, 64, 80, 97, 128, 129, 160, 180, 224, 255, 256,
                                257, 300, 513])


def test_partly_filled_m_tiles_every_row_block_count():
    counts = PARTIAL_TILE_COUNTS
    E, N = len(counts), int(counts.sum())
    cfg = W.CONFIGS["tiny"].scaled(name="partial_tiles", T=N, d=256, f=384, E=E, k=1, seed=21)
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    D = _dims(cfg)
    ro = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    say(f"moe_expert_ffn partly filled m-tiles E={E} N={N}")
    y = M.moe_expert_ffn(D, t["x"], torch.as_tensor(ro, device="cuda"), t["w_gate"], t["w_up"],
                         t["w_down"])
    torch.cuda.synchronize()
    eor = np.repeat(np.arange(E, dtype=np.int32), counts)
    ref = oracle.expert_rows(arrs["x"], eor, arrs["w_gate"], arrs["w_up"], arrs["w_down"])
    err = rel_err(host_f32(y[:N]), ref)
    say(f"  ffn rel err {err:.3e}")
    assert err <= TOL_LAYER


def test_no_local_rows_gives_zero_output():
    # every token routes only to experts outside the local range
    cfg = W.CONFIGS["tiny"].scaled(name="nolocal", T=50, d=256, f=128, E=8, k=1, e_lo=0, e_hi=2,
                                   out_fp32=True, seed=12)
    arrs = W.generate(cfg, bias_override=_bias_all_to_one(8, 6))
    t = upload(cfg, arrs)
    out = _check_layer(cfg, t, arrs)
    assert torch.count_nonzero(out).item() == 0


def test_repeated_calls_reuse_workspace_and_stay_identical():
    cfg = SMALL["multi_tile_rows"]
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    D = _dims(cfg)
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    say("moe_layer repeated x5 on one workspace")
    outs = [M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], ws=ws)
            for _ in range(5)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert M.moe_device_status(D, ws) == 0


def test_bounded_wait_reports_timeout_then_recovers():
    cfg = SMALL["multi_tile_rows"]
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    D = _dims(cfg)
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    say("moe_layer with a 1 us flag-wait timeout")
    M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], ws=ws,
                opts=M.layer_opts(wait_timeout_us=1))
    st = M.moe_device_status(D, ws)
    assert st in (0, -5)
    say("moe_layer with the default timeout")
    M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], ws=ws)
    assert M.moe_device_status(D, ws) == 0


# ------------------------------------------------------------ full-size shapes

FULL = ["tiny", "mixtral", "fine", "skewed", "dsv3_share"]


def _mtile_rows(ro, rng, extra=16):
    """The first and last row of every 256-row m-tile of every expert segment
    (so every m-tile of the grouped GEMMs is compared), plus random rows."""
    rows = []
    for e in range(len(ro) - 1):
        for r0 in range(int(ro[e]), int(ro[e + 1]), 256):
            rows += [r0, min(r0 + 255, int(ro[e + 1]) - 1)]
    N = int(ro[-1])
    return np.unique(np.concatenate([np.array(rows, np.int64),
                                     rng.choice(N, size=min(N, extra), replace=False)]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    """The five workloads at full size: routing and dispatch bit-exact, the
    FFN on every row (tiny, fine) or on the first and last row of every
    m-tile (the rest), and the layer output of EVERY token against the
    oracle, fused == staged bit for bit."""
    cfg = W.CONFIGS[name]
    say(f"generate {name}")
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    offsets, inv, xp, ro, rp, ri, N = _check_permute(cfg, t, arrs, ids, r_ids)
    rows = None if name in ("tiny", "fine") else _mtile_rows(ro, np.random.default_rng(1))
    y = _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N, rows=rows)
    staged = _staged(cfg, t, y, inv, gates)
    _check_layer(cfg, t, arrs, staged_out=staged, tokens=np.arange(cfg.T))
    del t, xp, y, staged
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,hot", [("spread", None), ("one_hot_expert", 3)])
def test_fused_visibility_poisoned_workspace_alternating_inputs(name, hot):
    # Two different inputs through one workspace whose scratch regions start
    # as NaN bytes: a tile that read a row before its producer's write was
    # visible would carry NaNs or the previous input's values into the output,
    # so fused must equal staged bit for bit on both calls.
    base = W.CONFIGS["tiny"].scaled(name=name, T=2048, d=512, f=512, E=8, k=2)
    D = _dims(base)
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    for seed in (21, 22):
        cfg = base.scaled(seed=seed)
        bias = _bias_all_to_one(8, hot) if hot is not None else None
        arrs = W.generate(cfg, bias_override=bias)
        t = upload(cfg, arrs)
        say(f"moe_layer poisoned ws {name} seed={seed}")
        out = M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t["bias"],
                          ws=ws)
        assert M.moe_device_status(D, ws) == 0
        ids, gates, _ = M.moe_route(D, t["x"], t["w_router"], t["bias"], want_logits=True)
        counts, offsets, perm, inv, xp = M.moe_permute(D, t["x"], ids)
        y = M.moe_expert_ffn(D, xp, offsets, t["w_gate"], t["w_up"], t["w_down"])
        staged = M.moe_combine(D, y, inv, gates)
        torch.cuda.synchronize()
        assert not torch.isnan(out.float()).any()
        assert torch.equal(out.view(torch.int16), staged.view(torch.int16)), "fused != staged"


@pytest.mark.parametrize("pattern", ["duplicated_rows", "all_equal", "scaled_copies",
                                     "block_equal"])
def test_router_fast_path_on_constructed_ties(pattern):
    # Router weights built so that logits tie exactly (duplicated expert rows),
    # all tie (identical rows: every expert is a candidate), sit at the
    # tolerance edge (rows that are exact power-of-two multiples of others),
    # or tie in a block of 40 (a token that ranks that row among its top k has
    # 40 or more candidates: several candidate batches, selected by rank):
    # the fast path must still return the exact-order selection and gates.
    cfg = W.CONFIGS["tiny"].scaled(name=f"ties_{pattern}", T=257, d=512, f=128, E=96, k=6,
                                   seed=16)
    arrs = W.generate(cfg)
    wr = W.bf16_bits_to_f32(arrs["w_router"]).reshape(cfg.E, cfg.d)
    if pattern == "duplicated_rows":
        wr[1::2] = wr[0::2]
    elif pattern == "all_equal":
        wr[:] = wr[0]
    elif pattern == "block_equal":
        wr[:40] = wr[0]
    else:
        wr[48:] = wr[:48] * 2.0
    arrs["w_router"] = W.f32_to_bf16_bits(wr.astype(np.float32))
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    if pattern == "all_equal":
        assert np.array_equal(r_ids[0], np.arange(cfg.k))


# With E > 16 and a wide hidden dimension, a refine wave stages its token row
# in two windows of pieces per chunk (the row would otherwise leave LDS for
# fewer than 16 waves per CU): windows of 16 and 18 pieces (d = 4352), of 16
# (d = 4096, duplicated expert rows: exact ties), and every expert a
# candidate at d = 7168 (all rows equal), so each batch of 16 candidates
# stages both windows again; and a block of 40 equal rows at d = 7168 (40 to
# 64 candidates where the block ranks high: several batches, each staging
# both windows, selected by rank).
TWO_WINDOW_ROUTER = {
    "d4352_e256": dict(T=300, d=4352, E=256, k=8, pattern=None),
    "d4096_e256_duplicated": dict(T=200, d=4096, E=256, k=6, pattern="duplicated_rows"),
    "d7168_e256_all_equal": dict(T=129, d=7168, E=256, k=8, pattern="all_equal"),
    "d7168_e256_block_equal": dict(T=257, d=7168, E=256, k=8, pattern="block_equal"),
}


@pytest.mark.parametrize("name", list(TWO_WINDOW_ROUTER))
def test_router_two_window_staging(name):
    spec = dict(TWO_WINDOW_ROUTER[name])
    pattern = spec.pop("pattern")
    cfg = W.CONFIGS["tiny"].scaled(name=name, f=128, seed=60 + list(TWO_WINDOW_ROUTER).index(name),
                                   **spec)
    arrs = W.generate(cfg)
    if pattern is not None:
        wr = W.bf16_bits_to_f32(arrs["w_router"]).reshape(cfg.E, cfg.d)
        if pattern == "duplicated_rows":
            wr[1::2] = wr[0::2]
        elif pattern == "block_equal":
            wr[:40] = wr[0]
        else:
            wr[:] = wr[0]
        arrs["w_router"] = W.f32_to_bf16_bits(wr.astype(np.float32))
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    if pattern == "all_equal":
        assert np.array_equal(r_ids[0], np.arange(cfg.k))


# The E <= 16 router stages the activations through LDS when d is a multiple
# of 1024 (up to four 32 KiB steps in flight, a ring beyond that): step
# counts 1, 2, 3, 5 and 8, ragged and single-token blocks, E below 8 and
# between 9 and 16; every stage, and the layer, whose router also counts the
# permute's histogram.
LDS_ROUTER = {
    "d1024_e8": dict(T=1000, d=1024, E=8, k=2),
    "d2048_e16": dict(T=333, d=2048, E=16, k=4),
    "d3072_e5": dict(T=130, d=3072, E=5, k=2),
    "d5120_e12": dict(T=200, d=5120, E=12, k=3),
    "d8192_e8": dict(T=64, d=8192, E=8, k=1),
    "d4096_t65": dict(T=65, d=4096, E=8, k=2),
    "d1024_one_token": dict(T=1, d=1024, E=2, k=1),
}


@pytest.mark.parametrize("name", list(LDS_ROUTER))
def test_router_lds_staged_shapes(name):
    cfg = W.CONFIGS["tiny"].scaled(name=name, f=128, seed=40 + list(LDS_ROUTER).index(name),
                                   **LDS_ROUTER[name])
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    offsets, inv, xp, ro, rp, ri, N = _check_permute(cfg, t, arrs, ids, r_ids)
    y = _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N)
    staged = _staged(cfg, t, y, inv, gates)
    _check_layer(cfg, t, arrs, staged_out=staged)


@pytest.mark.parametrize("f,parts", [(8448, 2), (8192, 4)])
def test_cut_down_tiles(f, parts):
    # Deep down GEMMs (f >= 8192) cut the down tiles of the schedule's last
    # partial round into K parts (2 when f is not a multiple of 512, else 4),
    # both in moe_layer's persistent kernel and in moe_expert_ffn: more than
    # 256 down tiles (the MI355X grid) make the last round partial.  Fused
    # must equal staged bit for bit, and both must match the oracle.
    cfg = W.CONFIGS["tiny"].scaled(name=f"cut{parts}", T=2400, d=4096, f=f, E=2, k=2, seed=17)
    say(f"generate cut-tile case f={f}")
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    ids, gates, r_ids, r_g = _check_route(cfg, t, arrs)
    offsets, inv, xp, ro, rp, ri, N = _check_permute(cfg, t, arrs, ids, r_ids)
    counts = np.diff(ro)
    n_down_tiles = int(sum((c + 255) // 256 for c in counts)) * (cfg.d // 256)
    assert n_down_tiles > 256 and n_down_tiles % 256 > 0, n_down_tiles
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=10, replace=False)]))
    y = _check_ffn(cfg, t, arrs, xp, offsets, ro, rp, N, rows=rows)
    staged = _staged(cfg, t, y, inv, gates)
    toks = sample_tokens(cfg.T, 24, seed=4, must=[0, cfg.T - 1])
    _check_layer(cfg, t, arrs, staged_out=staged, tokens=toks)
    del t, xp, y, staged
    torch.cuda.empty_cache()


def _named_case(name):
    if name.startswith("rand"):
        return _random_case(int(name[4:]))
    return (SMALL[name] if name in SMALL else W.CONFIGS[name]).scaled(name=name)


@pytest.mark.parametrize("name", ["tiny", "ragged_T300", "local_subset_e16k4", "e128k8", "mixtral",
                                  "rand1", "rand2", "rand6", "rand9"])
def test_gather_on_load_dispatch(name):
    # Gather-on-load dispatch: gate/up tiles fetch their rows of x through
    # perm_src (x_perm never written).  Same tile k-order as the packed path,
    # so the layer output must equal the packed-dispatch output bit for bit,
    # and match the oracle.
    cfg = _named_case(name)
    D = _dims(cfg)
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    say(f"moe_layer packed dispatch {cfg.name}")
    packed = M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t["bias"],
                         out_dtype=dt)
    torch.cuda.synchronize()
    say(f"moe_layer gather dispatch {cfg.name}")
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # a packed x_perm left from elsewhere must not be read
    out = M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"],
                      t["bias"], out_dtype=dt, ws=ws,
                      opts=M.layer_opts(dispatch=M.MOE_DISPATCH_GATHER))
    torch.cuda.synchronize()
    assert M.moe_device_status(D, ws) == 0
    bits = torch.int32 if dt == M.MOE_F32 else torch.int16
    assert torch.equal(out.view(bits), packed.view(bits)), "gather != packed dispatch"
    toks = sample_tokens(cfg.T, 32, seed=5)
    ref, _, _ = oracle.layer_tokens(toks, arrs["x"], arrs["w_router"], arrs["w_gate"], arrs["w_up"],
                                    arrs["w_down"], cfg.k, cfg.e_lo, cfg.E_hi, bias=arrs["bias"])
    err = rel_err(host_f32(out[torch.as_tensor(toks, device="cuda")]), ref)
    say(f"  gather dispatch rel err {err:.3e}")
    assert err <= TOL_LAYER
    del t
    torch.cuda.empty_cache()


ORDERS = [1, 2, 3, 4]


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("name", ["tiny", "local_subset_e16k4", "e128k8", "mixtral",
                                  "rand1", "rand2", "rand6", "rand9"])
def test_tile_orders_same_bits_and_match_oracle(name, order):
    """Every tile order runs the same tiles with the same arithmetic: the
    output bits equal the default order's, and match the oracle."""
    cfg = _named_case(name)
    arrs = W.generate(cfg)
    t = upload(cfg, arrs)
    D = _dims(cfg)
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    say(f"moe_layer tile order 0 {name}")
    ref = M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t["bias"],
                      out_dtype=dt, ws=ws)
    torch.cuda.synchronize()
    ws.fill_(0xFF)
    say(f"moe_layer tile order {order} {name}")
    out = M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"],
                      t["bias"], out_dtype=dt, ws=ws, opts=M.layer_opts(tile_order=order))
    torch.cuda.synchronize()
    assert M.moe_device_status(D, ws) == 0
    bits = torch.int32 if dt == M.MOE_F32 else torch.int16
    assert torch.equal(out.view(bits), ref.view(bits))
    toks = np.arange(cfg.T) if cfg.T <= 1200 else sample_tokens(cfg.T, 64, seed=8)
    oref, _, _ = oracle.layer_tokens(toks, arrs["x"], arrs["w_router"], arrs["w_gate"],
                                     arrs["w_up"], arrs["w_down"], cfg.k, cfg.e_lo, cfg.E_hi,
                                     bias=arrs["bias"])
    err = rel_err(host_f32(out[torch.as_tensor(toks, device="cuda")]), oref)
    say(f"  tile order {order} rel err {err:.3e} over {len(toks)} tokens")
    assert err <= TOL_LAYER
    del t
    torch.cuda.empty_cache()


def _perturb_case(name):
    if name == "cut4":
        return W.CONFIGS["tiny"].scaled(name="cut4", T=2400, d=4096, f=8192, E=2, k=2, seed=17)
    if name == "hot18":
        return W.CONFIGS["tiny"].scaled(name="hot18", T=4600, d=256, f=256, E=8, k=1, seed=19)
    return _named_case(name)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("order", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("name,seed", [("tiny", 1), ("multi_tile_rows", 2), ("e128k8", 3),
                                       ("local_subset_e16k4", 4), ("hot18", 5), ("cut4", 6),
                                       ("fine", 7)])
def test_adversarial_schedule_same_bits_and_match_oracle(name, seed, order):
    """The flag protocol under adversarial timing: producers wait seeded
    pseudo-random delays (up to ~100 us) between writing their tiles and
    publishing them, and each kind's tiles are claimed from the far end of
    every range (not in the dependency-lead and chunked orders, whose merged
    streams must be claimed in order).  A consumer that read before its producer's release would
    see the NaN bytes the workspace starts with, or stale rows; the output
    must instead equal the staged calls bit for bit and match the oracle."""
    cfg = _perturb_case(name)
    arrs = W.generate(cfg, bias_override=_bias_all_to_one(8, 2) if name == "hot18" else None)
    t = upload(cfg, arrs)
    D = _dims(cfg)
    dt = M.MOE_F32 if cfg.out_fp32 else M.MOE_BF16
    say(f"staged calls {name}")
    ids, gates, _ = M.moe_route(D, t["x"], t["w_router"], t["bias"])
    _, offsets, _, inv, xp = M.moe_permute(D, t["x"], ids)
    y = M.moe_expert_ffn(D, xp, offsets, t["w_gate"], t["w_up"], t["w_down"], check_status=True)
    staged = M.moe_combine(D, y, inv, gates, out_dtype=dt)
    torch.cuda.synchronize()
    del xp, y
    ws = torch.empty(M.moe_layer_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    say(f"moe_layer perturbed schedule {name} seed={seed} order={order}")
    out = M.moe_layer(D, t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], t["bias"],
                      out_dtype=dt, ws=ws, opts=M.layer_opts(tile_order=order, perturb_seed=seed),
                      check_status=True)
    bits = torch.int32 if dt == M.MOE_F32 else torch.int16
    assert torch.equal(out.view(bits), staged.view(bits)), "perturbed fused != staged"
    toks = np.arange(cfg.T) if cfg.T <= 600 else sample_tokens(cfg.T, 48, seed=seed)
    oref, _, _ = oracle.layer_tokens(toks, arrs["x"], arrs["w_router"], arrs["w_gate"],
                                     arrs["w_up"], arrs["w_down"], cfg.k, cfg.e_lo, cfg.E_hi,
                                     bias=arrs["bias"])
    err = rel_err(host_f32(out[torch.as_tensor(toks, device="cuda")]), oref)
    say(f"  perturbed rel err {err:.3e} over {len(toks)} tokens")
    assert err <= TOL_LAYER
    del t, ws
    torch.cuda.empty_cache()
