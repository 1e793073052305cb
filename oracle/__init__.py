"""CPU oracle of the routed grouped-GEMM MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, see its header for the
definition followed and every reading taken where the pages are silent).
This module only builds that file and marshals numpy arrays into it.

Parity status of each function (what pins it, in tests/test_oracle_*.py):
  router_logits   pinned: exact small-integer dot products; a hand-worked case
                  where the defined chunk/tree order differs from a plain
                  sequential sum; float64 agreement within the float32 bound.
  topk_gates      pinned: brute force over all C(E,k) subsets incl. exact ties;
                  k=1 gives gate 1; equal logits give 1/k; k=E gives the full
                  softmax (scipy); gates sum to 1.
  permute         pinned: equals a stable sort by expert (numpy), bijection,
                  counts equal numpy bincount.
  expert_rows     pinned: E=1 equals a dense SwiGLU written with numpy float64
                  matmuls; a hand-worked 2x2 case.
  combine         pinned: hand-worked small case; linearity in the gates.
  e4m3_value      pinned: values the OCP 8-bit float definition fixes (1, 2,
                  448, 2^-6, 2^-9, NaN pattern, signed zero), monotone order.
  e4m3_encode     pinned: every finite value round-trips; midpoints go to the
                  even code; a closed-form rounding (numpy half-to-even on the
                  value's own quantum) agrees on a dense sweep; saturation.
  quantize_rows_e4m3  pinned: the scale is the smallest admissible power of
                  two; exact when the row is already E4M3 times 2^e; error
                  within half a code step.
  expert_rows_fp8 pinned: with inputs exact in E4M3 it equals the float64
                  dense SwiGLU of the decoded operands (numpy matmuls) up to
                  the bf16/E4M3 rounding of h; per-row and per-channel scales
                  land on their own axes (non-uniform scales).
  gate_up_rows_fp8  pinned: equals numpy float64 products of the decoded
                  codes with the row and channel scales, then silu(g)*u; its
                  bf16 rounding equals expert_rows_fp8's h.
  down_rows_fp8   pinned: equals a numpy float64 dense product of decoded
                  codes and scales; fed the oracle's own quantised h it gives
                  expert_rows_fp8's y.
  layer_tokens    pinned: k=1 one-hot reduces to one expert's FFN; identical
                  experts reduce to the dense FFN (gates sum to 1); sum of
                  expert-parallel shard partials equals the unsharded layer.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
               "-fPIC", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = C.CDLL(_LIB)
        i64, vp = C.c_int64, C.c_void_p
        lib.oracle_router_logits.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        lib.oracle_router_logits_f64.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_topk_gates.argtypes = [i64, i64, i64, vp, vp, vp]
        lib.oracle_route.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_permute.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_expert_rows.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_combine.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        lib.oracle_layer_tokens.argtypes = [i64, vp, i64, i64, i64, i64, i64, i64, i64, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_e4m3_value.argtypes = [C.c_int32]
        lib.oracle_e4m3_value.restype = C.c_double
        lib.oracle_e4m3_encode.argtypes = [C.c_float]
        lib.oracle_e4m3_encode.restype = C.c_int32
        lib.oracle_quantize_rows_e4m3.argtypes = [i64, i64, vp, vp, vp]
        lib.oracle_quantize_rows_e4m3.restype = C.c_int
        lib.oracle_expert_rows_fp8.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, vp]
        lib.oracle_expert_rows_fp8.restype = C.c_int
        lib.oracle_gate_up_rows_fp8.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_gate_up_rows_fp8.restype = C.c_int
        lib.oracle_down_rows_fp8.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_down_rows_fp8.restype = C.c_int
        lib.oracle_num_threads.restype = C.c_int
        lib.oracle_set_num_threads.argtypes = [C.c_int]
        lib.oracle_set_num_threads.restype = None
        for name in ("oracle_router_logits", "oracle_router_logits_f64", "oracle_topk_gates",
                     "oracle_route", "oracle_permute", "oracle_expert_rows", "oracle_combine",
                     "oracle_layer_tokens"):
            getattr(lib, name).restype = C.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Set the OpenMP thread count of later oracle calls."""
    _load().oracle_set_num_threads(int(n))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    x, w = _u16(x), _u16(w_router)
    T, d = x.shape
    E = w.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float32)
    _check(_load().oracle_router_logits(T, d, E, _p(x), _p(w), _p(b), _p(out)), "router_logits")
    return out


def router_logits_f64(x, w_router, bias=None) -> Tuple[np.ndarray, np.ndarray]:
    x, w = _u16(x), _u16(w_router)
    T, d = x.shape
    E = w.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float64)
    absd = np.empty((T, E), dtype=np.float64)
    _check(_load().oracle_router_logits_f64(T, d, E, _p(x), _p(w), _p(b), _p(out), _p(absd)),
           "router_logits_f64")
    return out, absd


def topk_gates(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    l = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = l.shape
    ids = np.empty((T, k), dtype=np.int32)
    g = np.empty((T, k), dtype=np.float32)
    _check(_load().oracle_topk_gates(T, E, k, _p(l), _p(ids), _p(g)), "topk_gates")
    return ids, g


def route(x, w_router, k: int, bias=None, want_logits: bool = False):
    x, w = _u16(x), _u16(w_router)
    T, d = x.shape
    E = w.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    g = np.empty((T, k), dtype=np.float32)
    l = np.empty((T, E), dtype=np.float32) if want_logits else None
    _check(_load().oracle_route(T, d, E, k, _p(x), _p(w), _p(b), _p(ids), _p(g), _p(l)), "route")
    return (ids, g, l) if want_logits else (ids, g)


def permute(ids: np.ndarray, E: int, e_lo: int = 0, e_hi: Optional[int] = None):
    """Returns counts [E_loc], offsets [E_loc+1], perm_src [N], inv_perm [T,k]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    e_hi = E if e_hi is None else e_hi
    EL = e_hi - e_lo
    counts = np.empty(EL, dtype=np.int32)
    offsets = np.empty(EL + 1, dtype=np.int32)
    perm = np.empty(max(1, T * k), dtype=np.int32)
    inv = np.empty((T, k), dtype=np.int32)
    _check(_load().oracle_permute(T, k, E, e_lo, e_hi, _p(ids), _p(counts), _p(offsets), _p(perm),
                                  _p(inv)), "permute")
    return counts, offsets, perm[: int(offsets[-1])].copy(), inv


def expert_rows(x_rows, expert_of_row, w_gate, w_up, w_down, want_h: bool = False):
    x_rows = _u16(x_rows)
    e = np.ascontiguousarray(expert_of_row, dtype=np.int32)
    wg, wu, wd = _u16(w_gate), _u16(w_up), _u16(w_down)
    n, d = x_rows.shape
    EL, f, _ = wg.shape
    y = np.empty((n, d), dtype=np.float64)
    h = np.empty((n, f), dtype=np.float64) if want_h else None
    _check(_load().oracle_expert_rows(n, d, f, EL, _p(x_rows), _p(e), _p(wg), _p(wu), _p(wd),
                                      _p(y), _p(h)), "expert_rows")
    return (y, h) if want_h else y


def combine(y_perm: np.ndarray, inv_perm: np.ndarray, gates: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y_perm, dtype=np.float64)
    inv = np.ascontiguousarray(inv_perm, dtype=np.int32)
    g = np.ascontiguousarray(gates, dtype=np.float32)
    T, k = inv.shape
    d = y.shape[1]
    out = np.empty((T, d), dtype=np.float64)
    _check(_load().oracle_combine(T, k, d, _p(y), _p(inv), _p(g), _p(out)), "combine")
    return out


def layer_tokens(tokens: Sequence[int], x, w_router, w_gate, w_up, w_down, k: int,
                 e_lo: int = 0, e_hi: Optional[int] = None, bias=None):
    """Layer output (float64) for the listed tokens; also their ids and gates."""
    toks = np.ascontiguousarray(tokens, dtype=np.int64)
    x, wr = _u16(x), _u16(w_router)
    wg, wu, wd = _u16(w_gate), _u16(w_up), _u16(w_down)
    T, d = x.shape
    E = wr.shape[0]
    f = wg.shape[1]
    e_hi = E if e_hi is None else e_hi
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    n = toks.shape[0]
    ids = np.empty((n, k), dtype=np.int32)
    g = np.empty((n, k), dtype=np.float32)
    out = np.empty((n, d), dtype=np.float64)
    _check(_load().oracle_layer_tokens(n, _p(toks), T, d, f, E, k, e_lo, e_hi, _p(x), _p(wr),
                                       _p(b), _p(wg), _p(wu), _p(wd), _p(ids), _p(g), _p(out)),
           "layer_tokens")
    return out, ids, g


def layer_full(x, w_router, w_gate, w_up, w_down, k: int, e_lo: int = 0,
               e_hi: Optional[int] = None, bias=None):
    """Whole layer through the staged oracle (route -> permute -> FFN -> combine).

    Returns dict with ids, gates, counts, offsets, perm_src, inv_perm, y_perm, out.
    For small sizes only.
    """
    E = np.asarray(w_router).shape[0]
    e_hi = E if e_hi is None else e_hi
    ids, g = route(x, w_router, k, bias=bias)
    counts, offsets, perm, inv = permute(ids, E, e_lo, e_hi)
    x = _u16(x)
    x_perm = x[perm]
    expert_of_row = np.repeat(np.arange(e_hi - e_lo, dtype=np.int32), counts)
    y = expert_rows(x_perm, expert_of_row, w_gate, w_up, w_down) if len(perm) else \
        np.zeros((0, x.shape[1]))
    out = combine(y, inv, g)
    return dict(ids=ids, gates=g, counts=counts, offsets=offsets, perm_src=perm, inv_perm=inv,
                y_perm=y, out=out)


# ------------------------------------------------------------ W8A8 (fp8)

def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code (0..255)."""
    return float(_load().oracle_e4m3_value(int(code)))


def e4m3_encode(v: float) -> int:
    """Nearest E4M3 code of a float32 value (ties to even, saturating)."""
    return int(_load().oracle_e4m3_encode(float(np.float32(v))))


def quantize_rows_e4m3(x) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row power-of-two scaled E4M3 codes of a bf16 matrix [rows, cols]:
    (codes uint8 [rows, cols], scales float32 [rows])."""
    x = _u16(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(rows, dtype=np.float32)
    _check(_load().oracle_quantize_rows_e4m3(rows, cols, _p(x), _p(q), _p(s)), "quantize_rows_e4m3")
    return q, s


def expert_rows_fp8(x_rows, expert_of_row, wq_gate, s_gate, wq_up, s_up, wq_down, s_down,
                    want_h: bool = False):
    """W8A8 SwiGLU FFN of rows (float64 y; h as its bf16-rounded values)."""
    x_rows = _u16(x_rows)
    e = np.ascontiguousarray(expert_of_row, dtype=np.int32)
    u8 = lambda a: np.ascontiguousarray(a, dtype=np.uint8)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    wg, wu, wd = u8(wq_gate), u8(wq_up), u8(wq_down)
    sg, su, sd = f32(s_gate), f32(s_up), f32(s_down)
    n, d = x_rows.shape
    EL, f, _ = wg.shape
    y = np.empty((n, d), dtype=np.float64)
    h = np.empty((n, f), dtype=np.float64) if want_h else None
    _check(_load().oracle_expert_rows_fp8(n, d, f, EL, _p(x_rows), _p(e), _p(wg), _p(sg), _p(wu),
                                          _p(su), _p(wd), _p(sd), _p(y), _p(h)),
           "expert_rows_fp8")
    return (y, h) if want_h else y


def gate_up_rows_fp8(x_rows, expert_of_row, wq_gate, s_gate, wq_up, s_up) -> np.ndarray:
    """GEMM0 + SiLU-mul of the W8A8 FFN: h [n, f] float64, not rounded."""
    x_rows = _u16(x_rows)
    e = np.ascontiguousarray(expert_of_row, dtype=np.int32)
    u8 = lambda a: np.ascontiguousarray(a, dtype=np.uint8)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    wg, wu, sg, su = u8(wq_gate), u8(wq_up), f32(s_gate), f32(s_up)
    n, d = x_rows.shape
    EL, f, _ = wg.shape
    h = np.empty((n, f), dtype=np.float64)
    _check(_load().oracle_gate_up_rows_fp8(n, d, f, EL, _p(x_rows), _p(e), _p(wg), _p(sg),
                                           _p(wu), _p(su), _p(h)), "gate_up_rows_fp8")
    return h


def down_rows_fp8(hq, sh, expert_of_row, wq_down, s_down) -> np.ndarray:
    """GEMM1 of the W8A8 FFN from given E4M3 codes hq [n, f] and row scales
    sh [n] of h: y [n, d] float64."""
    hq = np.ascontiguousarray(hq, dtype=np.uint8)
    sh = np.ascontiguousarray(sh, dtype=np.float32)
    e = np.ascontiguousarray(expert_of_row, dtype=np.int32)
    wd = np.ascontiguousarray(wq_down, dtype=np.uint8)
    sd = np.ascontiguousarray(s_down, dtype=np.float32)
    n, f = hq.shape
    EL, d, _ = wd.shape
    y = np.empty((n, d), dtype=np.float64)
    _check(_load().oracle_down_rows_fp8(n, d, f, EL, _p(hq), _p(sh), _p(e), _p(wd), _p(sd),
                                        _p(y)), "down_rows_fp8")
    return y
