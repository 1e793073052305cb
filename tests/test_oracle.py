"""Pins of the CPU oracle against facts fixed outside the oracle itself:
hand-worked values, exact integer arithmetic, brute force, textbook dense
SwiGLU written with numpy matmuls, and the special cases the method reduces to
(Weave, §2.1 and Figure 3: top-k gating, dispatch, GEMM0 up+gate, SiLU-mul,
GEMM1 down, weighted-sum combine)."""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import moe_workloads as W
import oracle

U = 2.0 ** -24  # float32 unit roundoff


def bf16(v):
    """Exact bf16 bits of values that are representable (asserted)."""
    a = np.asarray(v, dtype=np.float32)
    b = W.f32_to_bf16_bits(a)
    assert np.array_equal(W.bf16_bits_to_f32(b), a), "value not bf16-representable"
    return b


# ------------------------------------------------------------------ router

def test_logits_equal_exact_integer_dot_products():
    rng = np.random.default_rng(11)
    T, d, E = 7, 96, 5
    xi = rng.integers(-8, 9, size=(T, d))
    wi = rng.integers(-8, 9, size=(E, d))
    bi = rng.integers(-3, 4, size=E).astype(np.float32)
    l = oracle.router_logits(bf16(xi), bf16(wi), bias=bi)
    exact = xi.astype(np.int64) @ wi.T.astype(np.int64) + bi.astype(np.int64)
    assert np.array_equal(l, exact.astype(np.float32))
    # without bias
    l0 = oracle.router_logits(bf16(xi), bf16(wi))
    assert np.array_equal(l0, (xi @ wi.T).astype(np.float32))


def test_logits_defined_order_chunks_then_tree_hand_case():
    # d = 32: sixteen chunks of two elements.  Products chunk0 = [1, 2^24],
    # chunk1 = [1, -2^24], rest 0.  Chunk sums: fl(1 + 2^24) = 2^24 (tie to
    # even), fl(1 - 2^24) = -(2^24 - 1) exactly; tree: 2^24 - (2^24 - 1) = 1.
    # A plain left-to-right float32 sum would give 0, the real sum is 2.
    d = 32
    x = np.zeros(d)
    w = np.zeros(d)
    x[0:4] = [1, 2 ** 12, 1, 2 ** 12]
    w[0:4] = [1, 2 ** 12, 1, -2 ** 12]
    l = oracle.router_logits(bf16(x[None]), bf16(w[None]))
    assert l[0, 0] == np.float32(1.0)


def test_logits_tree_pairs_adjacent_chunks_hand_case():
    # chunk sums s0 = 2^24, s1 = 1, s2 = 0, s3 = 1, rest 0.
    # (s0+s1) = fl(2^24 + 1) = 2^24 (tie to even), (s2+s3) = 1, and then
    # fl(2^24 + 1) = 2^24 again.  A tree pairing (s0+s2)+(s1+s3) would give
    # 2^24 + 2 exactly.  (A sequential fold over chunks also gives 2^24 here,
    # but fails the next variant and the previous test.)
    d = 32
    x = np.zeros(d)
    w = np.zeros(d)
    x[0], w[0] = 2 ** 12, 2 ** 12      # chunk 0
    x[2], w[2] = 1, 1                  # chunk 1
    x[6], w[6] = 1, 1                  # chunk 3
    l = oracle.router_logits(bf16(x[None]), bf16(w[None]))
    assert l[0, 0] == np.float32(2 ** 24)
    # second variant: s0 = 2^24, s1 = 0, s2 = 1, s3 = 1 -> (2^24) + 2 exact
    x = np.zeros(d)
    w = np.zeros(d)
    x[0], w[0] = 2 ** 12, 2 ** 12
    x[4], w[4] = 1, 1
    x[6], w[6] = 1, 1
    l = oracle.router_logits(bf16(x[None]), bf16(w[None]))
    assert l[0, 0] == np.float32(2 ** 24 + 2)


def test_logits_bias_added_after_tree():
    # tree result 2^24 (one product 2^12 * 2^12); bias 3 is added last:
    # fl(2^24 + 3) = 2^24 + 4 (halfway between 2^24+2 and 2^24+4, ties to even).
    # Starting a chunk accumulator at the bias instead would also round, but a
    # dropped or double-counted bias gives 2^24 or 2^24 + 6.
    d = 32
    x = np.zeros(d)
    w = np.zeros(d)
    x[0], w[0] = 2 ** 12, 2 ** 12
    l = oracle.router_logits(bf16(x[None]), bf16(w[None]), bias=np.array([3.0], np.float32))
    assert l[0, 0] == np.float32(2 ** 24 + 4)


def test_logits_within_float32_error_bound_of_f64():
    cfg = W.CONFIGS["tiny"]
    a = W.generate(cfg, with_weights=False)
    bias = np.linspace(-0.5, 0.5, cfg.E).astype(np.float32)
    l32 = oracle.router_logits(a["x"], a["w_router"], bias=bias).astype(np.float64)
    l64, absd = oracle.router_logits_f64(a["x"], a["w_router"], bias=bias)
    # recursive summation depth d/16 - 1 inside a chunk, 4 tree levels, 1 bias add
    n = cfg.d // 16 + 4
    bound = (n * U / (1 - n * U)) * (absd + np.abs(bias)[None, :]) + U * np.abs(l64)
    err = np.abs(l32 - l64)
    assert (err <= bound).all()
    assert err.max() > 0  # the float32 order really rounds on these inputs


def _brute_force_selection(l, k):
    E = len(l)
    key = lambda e: (l[e], -e)  # larger logit first, then lower id
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [u for u in range(E) if u not in S]
        if all(key(s) > key(u) for s in S for u in rest):
            winners.append(S)
    assert len(winners) == 1
    return sorted(winners[0], key=lambda e: (-l[e], e))


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (7, 7), (8, 2)])
def test_topk_matches_brute_force_including_exact_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    T = 40
    # integer-valued logits in a small range force many exact ties
    xi = np.zeros((T, 32), np.int64)
    wi = np.zeros((E, 32), np.int64)
    xi[:, :3] = rng.integers(-1, 2, size=(T, 3))
    wi[:, :3] = rng.integers(-1, 2, size=(E, 3))
    l = oracle.router_logits(bf16(xi), bf16(wi))
    ids, g = oracle.topk_gates(l, k)
    n_ties = 0
    for t in range(T):
        want = _brute_force_selection(l[t].tolist(), k)
        assert ids[t].tolist() == want
        n_ties += len(set(l[t].tolist())) < E
    assert n_ties > T // 2


def test_gates_special_cases():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 8)).astype(np.float32)
    # k = 1: the single gate is exactly 1
    ids, g = oracle.topk_gates(l, 1)
    assert np.all(g == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(l, axis=1))
    # equal logits: 1/k each, ids 0..k-1 (ties to the lower id)
    ids, g = oracle.topk_gates(np.zeros((3, 8), np.float32), 4)
    assert np.all(g == np.float32(0.25))
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))
    # k = E: the full softmax (textbook, scipy) in the selection order
    ids, g = oracle.topk_gates(l, 8)
    sm = scipy.special.softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(sm, ids.astype(np.int64), 1), rtol=1e-6,
                               atol=0)
    # gates sum to one, are non-increasing along the slots
    ids, g = oracle.topk_gates(l, 3)
    np.testing.assert_allclose(g.astype(np.float64).sum(1), 1.0, atol=4 * U)
    assert np.all(np.diff(g, axis=1) <= 0)


def test_renormalised_softmax_equals_full_softmax_renormalised():
    # the gate reading: softmax over all E, keep the top-k, renormalise
    rng = np.random.default_rng(5)
    l = (rng.standard_normal((64, 16)) * 2).astype(np.float32)
    ids, g = oracle.topk_gates(l, 4)
    full = scipy.special.softmax(l.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    np.testing.assert_allclose(g, sel / sel.sum(1, keepdims=True), rtol=2e-7)


# ---------------------------------------------------------------- dispatch

def _random_ids(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,e_lo,e_hi", [(50, 8, 2, 0, 8), (64, 16, 4, 4, 10),
                                             (33, 5, 5, 0, 5), (1, 4, 1, 0, 4),
                                             (0, 4, 2, 0, 4)])
def test_permute_equals_stable_sort(T, E, k, e_lo, e_hi):
    rng = np.random.default_rng(T + E)
    ids = _random_ids(rng, T, E, k) if T else np.zeros((0, k), np.int32)
    counts, offsets, perm, inv = oracle.permute(ids, E, e_lo, e_hi)
    flat = ids.ravel()
    local = (flat >= e_lo) & (flat < e_hi)
    assert np.array_equal(counts, np.bincount(flat[local] - e_lo, minlength=e_hi - e_lo))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    # library stable sort of the local slots by expert, slots in (t, j) order
    slot = np.nonzero(local)[0]
    order = slot[np.argsort(flat[slot], kind="stable")]
    assert np.array_equal(perm, order // k)
    want_inv = -np.ones(T * k, np.int64)
    want_inv[order] = np.arange(len(order))
    assert np.array_equal(inv.ravel(), want_inv)
    # bijection between local slots and positions
    pos = inv.ravel()[local]
    assert sorted(pos.tolist()) == list(range(int(offsets[-1])))
    assert np.array_equal(perm[pos], (np.nonzero(local)[0] // k))


def test_permute_degenerate_one_expert_takes_all_and_empty_experts():
    ids = np.zeros((20, 1), np.int32) + 2
    counts, offsets, perm, inv = oracle.permute(ids, 4)
    assert counts.tolist() == [0, 0, 20, 0]
    assert offsets.tolist() == [0, 0, 0, 20, 20]
    assert perm.tolist() == list(range(20))
    assert inv[:, 0].tolist() == list(range(20))


def test_counts_sum_to_T_times_k_on_workload():
    cfg = W.CONFIGS["tiny"]
    a = W.generate(cfg, with_weights=False)
    ids, _ = oracle.route(a["x"], a["w_router"], cfg.k)
    counts, offsets, perm, inv = oracle.permute(ids, cfg.E)
    assert counts.sum() == cfg.T * cfg.k == offsets[-1]


# -------------------------------------------------------------- expert FFN

def _dense_swiglu(x, wg, wu, wd):
    """Textbook SwiGLU with numpy float64 matmuls; weights are [out, in]."""
    g = x @ wg.T
    u = x @ wu.T
    h = g / (1.0 + np.exp(-g)) * u
    return h @ wd.T


def _f(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def test_expert_rows_hand_worked_2x2():
    # x = [1, 2]; Wg = I; Wu = [[1, 1], [0, 1]]; Wd = I.
    # g = [1, 2], u = [3, 2], h = [3 sigmoid(1), 2 * 2 sigmoid(2)], y = h.
    sig1 = 0.7310585786300049  # 1 / (1 + e^-1)
    sig2 = 0.8807970779778823  # 1 / (1 + e^-2)
    x = bf16([[1, 2]])
    wg = bf16([[[1, 0], [0, 1]]])
    wu = bf16([[[1, 1], [0, 1]]])
    wd = bf16([[[1, 0], [0, 1]]])
    y = oracle.expert_rows(x, [0], wg, wu, wd)
    np.testing.assert_allclose(y[0], [3 * sig1, 4 * sig2], rtol=1e-15)


def test_single_expert_layer_equals_dense_swiglu():
    cfg = W.CONFIGS["tiny"].scaled(T=48, d=64, f=96, E=1, k=1)
    a = W.generate(cfg)
    r = oracle.layer_full(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], 1)
    assert np.all(r["gates"] == 1.0)
    dense = _dense_swiglu(_f(a["x"]), _f(a["w_gate"][0]), _f(a["w_up"][0]), _f(a["w_down"][0]))
    np.testing.assert_allclose(r["out"], dense, rtol=1e-10, atol=1e-12)


def test_one_hot_k1_gives_the_selected_experts_ffn():
    cfg = W.CONFIGS["tiny"].scaled(T=40, d=64, f=80, E=4, k=1)
    a = W.generate(cfg)
    r = oracle.layer_full(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], 1)
    x = _f(a["x"])
    for t in range(cfg.T):
        e = r["ids"][t, 0]
        want = _dense_swiglu(x[t:t + 1], _f(a["w_gate"][e]), _f(a["w_up"][e]), _f(a["w_down"][e]))
        np.testing.assert_allclose(r["out"][t], want[0], rtol=1e-10, atol=1e-12)


def test_identical_experts_reduce_to_dense_ffn():
    cfg = W.CONFIGS["tiny"].scaled(T=32, d=64, f=64, E=6, k=3)
    a = W.generate(cfg)
    wg = np.repeat(a["w_gate"][:1], 6, axis=0)
    wu = np.repeat(a["w_up"][:1], 6, axis=0)
    wd = np.repeat(a["w_down"][:1], 6, axis=0)
    r = oracle.layer_full(a["x"], a["w_router"], wg, wu, wd, 3)
    dense = _dense_swiglu(_f(a["x"]), _f(wg[0]), _f(wu[0]), _f(wd[0]))
    gsum = r["gates"].astype(np.float64).sum(1, keepdims=True)
    np.testing.assert_allclose(r["out"], dense * gsum, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["out"], dense, rtol=1e-6, atol=1e-7)


def test_combine_hand_worked_and_linear_in_gates():
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    inv = np.array([[2, 0], [-1, 1]], np.int32)
    g = np.array([[0.5, 0.25], [1.0, 0.75]], np.float32)
    out = oracle.combine(y, inv, g)
    np.testing.assert_array_equal(out, [[50.25, 100.5], [7.5, 15.0]])
    np.testing.assert_array_equal(oracle.combine(y, inv, 2 * g), 2 * out)


def test_expert_parallel_shards_sum_to_full_layer():
    cfg = W.CONFIGS["tiny"].scaled(T=24, d=64, f=48, E=8, k=3)
    a = W.generate(cfg)
    full = oracle.layer_full(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], 3)
    acc = np.zeros_like(full["out"])
    for lo in range(0, 8, 2):
        sh = oracle.layer_full(a["x"], a["w_router"], a["w_gate"][lo:lo + 2],
                               a["w_up"][lo:lo + 2], a["w_down"][lo:lo + 2], 3, e_lo=lo,
                               e_hi=lo + 2)
        assert np.array_equal(sh["ids"], full["ids"])  # gates over the global top-k
        acc += sh["out"]
    np.testing.assert_allclose(acc, full["out"], rtol=1e-12, atol=1e-14)


def test_token_path_agrees_with_staged_path():
    cfg = W.CONFIGS["tiny"]
    a = W.generate(cfg)
    full = oracle.layer_full(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], cfg.k)
    toks = [0, 1, 100, 255]
    out, ids, g = oracle.layer_tokens(toks, a["x"], a["w_router"], a["w_gate"], a["w_up"],
                                      a["w_down"], cfg.k)
    assert np.array_equal(ids, full["ids"][toks])
    np.testing.assert_allclose(out, full["out"][toks], rtol=1e-12, atol=1e-14)


def test_oracle_rejects_bad_arguments():
    x = np.zeros((2, 30), np.uint16)  # d not a multiple of 16
    with pytest.raises(ValueError):
        oracle.router_logits(x, np.zeros((3, 30), np.uint16))
    with pytest.raises(ValueError):
        oracle.topk_gates(np.zeros((2, 3), np.float32), 4)
