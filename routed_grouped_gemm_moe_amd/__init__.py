"""Python binding of the MI355X routed grouped-GEMM MoE library (gfx950 HIP).

Thin ctypes marshalling over the C ABI in include/moe.h: the functions below
carry the same names as the C entry points, take torch tensors that already
live on the GPU, pass their data pointers and the current HIP stream, and
raise on a non-OK status.  Every step of the computation runs in the HIP
kernels of libmoe_mi355x.so; torch only provides device memory and streams.
Output tensors that are not passed in are allocated here with torch.

If the shared library has not been built, every call raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional, Tuple

__all__ = [
    "MoEDims", "lib_path", "load", "exported_abi_names", "header_abi_names",
    "moe_route", "moe_route_bounds", "moe_probe_mfma", "moe_probe_mfma_rate", "moe_gate_up_fp8",
    "moe_down_fp8",
    "moe_permute", "moe_permute_noalloc", "moe_expert_ffn", "moe_combine", "moe_layer",
    "moe_route_workspace_bytes",
    "moe_permute_workspace_bytes", "moe_expert_ffn_workspace_bytes",
    "moe_layer_workspace_bytes", "moe_device_status", "moe_status_string",
    "MoELayerOpts", "layer_opts", "moe_wall_clock_hz", "MoEError",
    "MOE_DISPATCH_PACKED", "MOE_DISPATCH_GATHER", "MOE_ORDER_BY_KIND", "MOE_ORDER_READY_DOWN",
    "MOE_ORDER_LEAD", "MOE_ORDER_COMBINE_FIRST", "MOE_ORDER_CHUNKED",
    "MOE_BF16", "MOE_F32",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_BF16, MOE_F32 = 0, 1
MOE_DISPATCH_PACKED, MOE_DISPATCH_GATHER = 0, 1
MOE_ORDER_BY_KIND, MOE_ORDER_READY_DOWN, MOE_ORDER_LEAD, MOE_ORDER_COMBINE_FIRST = 0, 1, 2, 3
MOE_ORDER_CHUNKED = 4
MOE_SCHEDULE_AUTO = 0
MOE_SCHEDULE_PERSISTENT = 1
MOE_SCHEDULE_STAGED = 2
_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
           -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP", -5: "MOE_ERR_DEVICE_TIMEOUT"}


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({status})")


class MoEDims(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("T", "d", "f", "E", "k", "e_lo", "e_hi")]

    @classmethod
    def make(cls, T, d, f, E, k, e_lo=0, e_hi=None) -> "MoEDims":
        return cls(int(T), int(d), int(f), int(E), int(k), int(e_lo),
                   int(E if e_hi is None else e_hi))


class MoELayerOpts(C.Structure):
    """Per-call options of moe_layer / moe_layer_fp8 (include/moe.h)."""
    _fields_ = [("dispatch", C.c_int32), ("tile_order", C.c_int32), ("lead", C.c_int32),
                ("chunks", C.c_int32), ("perturb_seed", C.c_uint32), ("schedule", C.c_int32),
                ("wait_timeout_us", C.c_int64),
                ("trace", C.c_void_p), ("trace_records", C.c_int64),
                ("events", C.c_void_p * 4)]


def _event_handle(ev) -> Optional[int]:
    """hipEvent_t of a torch.cuda.Event (created on first record)."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return int(ev.cuda_event)


def layer_opts(dispatch: int = MOE_DISPATCH_PACKED, tile_order: int = MOE_ORDER_BY_KIND,
               lead: int = 0, chunks: int = 0, perturb_seed: int = 0, wait_timeout_us: int = 0,
               trace=None, trace_records: int = 0, events=None,
               schedule: int = 0) -> MoELayerOpts:
    """Build a MoELayerOpts.  trace: int64 device tensor of 1 + 4*trace_records
    elements (element 0 zeroed by the caller); events: up to 4 torch.cuda.Event
    (or None) recorded before the route, after the route, after the permute
    and after the last launch."""
    o = MoELayerOpts()
    o.dispatch, o.tile_order, o.lead, o.chunks = int(dispatch), int(tile_order), int(lead), int(chunks)
    o.perturb_seed, o.wait_timeout_us = int(perturb_seed), int(wait_timeout_us)
    o.schedule = int(schedule)
    if trace is not None:
        o.trace, o.trace_records = trace.data_ptr(), int(trace_records)
    for i, ev in enumerate(list(events or [])[:4]):
        o.events[i] = _event_handle(ev)
    return o


def lib_path() -> str:
    return _LIB


_lib = None


def load():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        raise ImportError(f"{_LIB} is missing: build it with "
                          "`python -m routed_grouped_gemm_moe_amd.build` (no fallback exists)")
    lib = C.CDLL(_LIB)
    vp, i32, i64, sz, dp = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.POINTER(MoEDims)
    sig = {
        "moe_status_string": ([i32], C.c_char_p),
        "moe_version": ([], i32),
        "moe_route_workspace_bytes": ([dp], sz),
        "moe_route": ([dp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_route_bounds": ([dp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_probe_mfma": ([i32, i64, i32, vp, vp, vp, vp, vp], i32),
        "moe_probe_mfma_rate": ([i64, i32, C.c_uint32, vp, vp], i32),
        "moe_gate_up_fp8": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_down_fp8": ([dp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_permute_workspace_bytes": ([dp], sz),
        "moe_permute": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_permute_noalloc_max_ints": ([], sz),
        "moe_permute_noalloc": ([dp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "moe_expert_ffn_workspace_bytes": ([dp], sz),
        "moe_expert_ffn": ([dp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_quantize_fp8": ([vp, i64, i64, vp, vp, vp], i32),
        "moe_expert_ffn_fp8_workspace_bytes": ([dp], sz),
        "moe_expert_ffn_fp8": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_layer_fp8_workspace_bytes": ([dp], sz),
        "moe_layer_fp8": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz,
                           C.POINTER(MoELayerOpts), vp], i32),
        "moe_combine": ([dp, vp, vp, vp, vp, i32, vp], i32),
        "moe_layer_workspace_bytes": ([dp], sz),
        "moe_layer": ([dp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, C.POINTER(MoELayerOpts),
                       vp], i32),
        "moe_device_status": ([dp, vp, sz, vp], i32),
        "moe_wall_clock_hz": ([], i64),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def header_abi_names():
    """Function names declared in include/moe.h."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def exported_abi_names():
    lib = load()
    return [n for n in header_abi_names() if hasattr(lib, n)]


# ------------------------------------------------------------------ helpers

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise MoEError(rc, what)


def _dims(dims) -> MoEDims:
    if isinstance(dims, MoEDims):
        return dims
    if isinstance(dims, dict):
        return MoEDims.make(**dims)
    return MoEDims.make(dims.T, dims.d, dims.f, dims.E, dims.k, dims.e_lo, dims.E_hi)


def _require(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: want contiguous cuda {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


def _workspace(nbytes: int, device, stream=None):
    """A workspace allocated here for one call.  Allocated on torch's current
    stream; if the call runs on another stream, that use is recorded so the
    caching allocator does not hand the block out before the call's kernels
    are done with it."""
    import torch
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


# ------------------------------------------------------------------ ABI calls

def moe_status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def moe_route_workspace_bytes(dims) -> int:
    return int(load().moe_route_workspace_bytes(C.byref(_dims(dims))))


def moe_permute_workspace_bytes(dims) -> int:
    return int(load().moe_permute_workspace_bytes(C.byref(_dims(dims))))


def moe_expert_ffn_workspace_bytes(dims) -> int:
    return int(load().moe_expert_ffn_workspace_bytes(C.byref(_dims(dims))))


def moe_layer_workspace_bytes(dims) -> int:
    return int(load().moe_layer_workspace_bytes(C.byref(_dims(dims))))


def moe_route(dims, x, w_router, bias=None, topk_ids=None, topk_w=None, logits=None,
              want_logits: bool = False, ws=None, use_workspace: bool = True, stream=None):
    """Top-k gating.  Returns (topk_ids int32 [T,k], topk_w f32 [T,k], logits or None).

    A workspace (allocated here when not given and use_workspace is true)
    enables the fast path for E > 16; without one every logit is evaluated in
    the defined order.  Both give the same ids and gates."""
    import torch
    D = _dims(dims)
    dev = x.device
    _require(x, torch.bfloat16, (D.T, D.d), "x")
    _require(w_router, torch.bfloat16, (D.E, D.d), "w_router")
    if bias is not None:
        _require(bias, torch.float32, (D.E,), "bias")
    if topk_ids is None:
        topk_ids = torch.empty((D.T, D.k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((D.T, D.k), dtype=torch.float32, device=dev)
    if logits is None and want_logits:
        logits = torch.empty((D.T, D.E), dtype=torch.float32, device=dev)
    if ws is None and use_workspace:
        nb = moe_route_workspace_bytes(D)
        ws = _workspace(nb, dev, stream) if nb > 0 else None
    rc = load().moe_route(C.byref(D), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_ids),
                          _ptr(topk_w), _ptr(logits), _ptr(ws),
                          ws.numel() if ws is not None else 0, _stream(stream))
    _check(rc, "moe_route")
    return topk_ids, topk_w, logits


def moe_route_bounds(dims, x, w_router, bias=None, approx=None, eps=None, ws=None, stream=None):
    """The fast router's approximate logits and their error bounds (E > 16).
    Returns (approx f32 [T,E], eps f32 [T,E])."""
    import torch
    D = _dims(dims)
    dev = x.device
    _require(x, torch.bfloat16, (D.T, D.d), "x")
    _require(w_router, torch.bfloat16, (D.E, D.d), "w_router")
    if bias is not None:
        _require(bias, torch.float32, (D.E,), "bias")
    approx = torch.empty((D.T, D.E), dtype=torch.float32, device=dev) if approx is None else approx
    eps = torch.empty((D.T, D.E), dtype=torch.float32, device=dev) if eps is None else eps
    ws = _workspace(moe_route_workspace_bytes(D), dev, stream) if ws is None else ws
    rc = load().moe_route_bounds(C.byref(D), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(approx),
                                 _ptr(eps), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check(rc, "moe_route_bounds")
    return approx, eps


def moe_probe_mfma(kind: int, a, b, c, d=None, stream=None):
    """Matrix-core probe: kind 0 bf16 (a, b bf16 [n, steps, 32, 16]), kind 1
    E4M3 (a, b uint8 [n, steps, 32, 64]); c f32 [n, 32, 32].  Returns d =
    c + sum over steps of a_s . b_s^T as computed by the matrix cores."""
    import torch
    want = (torch.bfloat16, 16) if kind == 0 else (torch.uint8, 64)
    if a.dtype != want[0] or b.dtype != want[0] or a.dim() != 4 or tuple(a.shape) != tuple(b.shape) \
            or tuple(a.shape[2:]) != (32, want[1]) or not a.is_contiguous() or not b.is_contiguous():
        raise ValueError("a, b: contiguous [n, steps, 32, K] operands of the probe's kind")
    n, steps = int(a.shape[0]), int(a.shape[1])
    _require(c, torch.float32, (n, 32, 32), "c")
    d = torch.empty_like(c) if d is None else d
    _check(load().moe_probe_mfma(int(kind), n, steps, _ptr(a), _ptr(b), _ptr(c), _ptr(d),
                                 _stream(stream)), "moe_probe_mfma")
    return d


def moe_probe_mfma_rate(workgroups: int, iters: int, seed: int, sink=None, stream=None):
    """Matrix-core rate probe: `workgroups` x 4 waves, each iters x 16
    independent bf16 MFMAs on zero (seed 0) or pseudo-random operands; the
    caller times it.  Returns the sink tensor (f32 [workgroups * 256])."""
    import torch
    if sink is None:
        sink = torch.empty(max(int(workgroups), 1) * 256, dtype=torch.float32, device="cuda")
    _check(load().moe_probe_mfma_rate(int(workgroups), int(iters), int(seed) & 0xFFFFFFFF,
                                      _ptr(sink), _stream(stream)), "moe_probe_mfma_rate")
    return sink


def moe_permute(dims, x, topk_ids, counts=None, offsets=None, perm_src=None, inv_perm=None,
                x_perm=None, ws=None, stream=None):
    """Dispatch.  Returns (counts, offsets, perm_src, inv_perm, x_perm) device tensors
    (perm_src and x_perm sized for T*k rows; the first offsets[-1] are valid)."""
    import torch
    D = _dims(dims)
    dev = x.device
    EL, cap = D.e_hi - D.e_lo, D.T * D.k
    _require(x, torch.bfloat16, (D.T, D.d), "x")
    _require(topk_ids, torch.int32, (D.T, D.k), "topk_ids")
    counts = torch.empty(EL, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(EL + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm_src = torch.empty(max(cap, 1), dtype=torch.int32, device=dev) if perm_src is None else perm_src
    inv_perm = torch.empty((D.T, D.k), dtype=torch.int32, device=dev) if inv_perm is None else inv_perm
    x_perm = torch.empty((max(cap, 1), D.d), dtype=torch.bfloat16, device=dev) if x_perm is None else x_perm
    need = moe_permute_workspace_bytes(D)
    ws = _workspace(need, dev, stream) if ws is None else ws
    rc = load().moe_permute(C.byref(D), _ptr(x), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                            _ptr(perm_src), _ptr(inv_perm), _ptr(x_perm), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "moe_permute")
    return counts, offsets, perm_src, inv_perm, x_perm


def moe_permute_noalloc(dims, x, topk_ids, counts, offsets, perm_src, inv_perm, x_perm,
                        stream=None):
    """moe_permute without a workspace and without any allocation: the caller
    passes every output (counts [E_loc], offsets [E_loc+1], perm_src [T*k],
    inv_perm [T,k], x_perm [T*k, d]); the library's per-GPU scratch array holds
    the per-block counts.  Calls that overlap on one GPU race."""
    import torch
    D = _dims(dims)
    EL, cap = D.e_hi - D.e_lo, D.T * D.k
    _require(x, torch.bfloat16, (D.T, D.d), "x")
    _require(topk_ids, torch.int32, (D.T, D.k), "topk_ids")
    _require(counts, torch.int32, (EL,), "counts")
    _require(offsets, torch.int32, (EL + 1,), "offsets")
    _require(inv_perm, torch.int32, (D.T, D.k), "inv_perm")
    if perm_src.dtype != torch.int32 or perm_src.numel() < cap or x_perm.dtype != torch.bfloat16 \
            or x_perm.shape[0] < cap or x_perm.shape[1] != D.d:
        raise ValueError("perm_src must hold T*k int32 rows, x_perm T*k bf16 rows of d")
    rc = load().moe_permute_noalloc(C.byref(D), _ptr(x), _ptr(topk_ids), _ptr(counts),
                                    _ptr(offsets), _ptr(perm_src), _ptr(inv_perm), _ptr(x_perm),
                                    _stream(stream))
    _check(rc, "moe_permute_noalloc")
    return counts, offsets, perm_src, inv_perm, x_perm


def moe_expert_ffn(dims, x_perm, offsets, w_gate, w_up, w_down, y_perm=None, ws=None,
                   check_status: bool = False, stream=None):
    """Grouped SwiGLU FFN over expert-contiguous rows.  Returns y_perm bf16 [T*k, d].
    check_status: synchronise and raise MoEError on a nonzero device status."""
    import torch
    D = _dims(dims)
    dev = x_perm.device
    EL, cap = D.e_hi - D.e_lo, D.T * D.k
    _require(w_gate, torch.bfloat16, (EL, D.f, D.d), "w_gate")
    _require(w_up, torch.bfloat16, (EL, D.f, D.d), "w_up")
    _require(w_down, torch.bfloat16, (EL, D.d, D.f), "w_down")
    _require(offsets, torch.int32, (EL + 1,), "offsets")
    if x_perm.shape[0] < cap or x_perm.shape[1] != D.d:
        raise ValueError("x_perm must have at least T*k rows of d")
    y_perm = torch.empty((max(cap, 1), D.d), dtype=torch.bfloat16, device=dev) if y_perm is None else y_perm
    need = moe_expert_ffn_workspace_bytes(D)
    ws = _workspace(need, dev, stream) if ws is None else ws
    rc = load().moe_expert_ffn(C.byref(D), _ptr(x_perm), _ptr(offsets), _ptr(w_gate), _ptr(w_up),
                               _ptr(w_down), _ptr(y_perm), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream))
    _check(rc, "moe_expert_ffn")
    if check_status:
        _check(moe_device_status(D, ws, stream), "moe_expert_ffn (device status)")
    return y_perm


def moe_quantize_fp8(x, q=None, scale=None, stream=None):
    """Per-row E4M3 codes of a bf16 matrix [..., K] with power-of-two row
    scales.  Returns (q uint8 [..., K], scale f32 [...])."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous bf16 tensor")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if scale is None else scale
    _check(load().moe_quantize_fp8(_ptr(x), rows, cols, _ptr(q), _ptr(scale), _stream(stream)),
           "moe_quantize_fp8")
    return q, scale


def moe_expert_ffn_fp8_workspace_bytes(dims) -> int:
    return int(load().moe_expert_ffn_fp8_workspace_bytes(C.byref(_dims(dims))))


def moe_expert_ffn_fp8(dims, x_perm, offsets, wq_gate, s_gate, wq_up, s_up, wq_down, s_down,
                       y_perm=None, ws=None, stream=None):
    """W8A8 grouped SwiGLU FFN over expert-contiguous bf16 rows (E4M3 weights
    from moe_quantize_fp8).  Returns y_perm bf16 [T*k, d]."""
    import torch
    D = _dims(dims)
    dev = x_perm.device
    EL, cap = D.e_hi - D.e_lo, D.T * D.k
    _require(wq_gate, torch.uint8, (EL, D.f, D.d), "wq_gate")
    _require(wq_up, torch.uint8, (EL, D.f, D.d), "wq_up")
    _require(wq_down, torch.uint8, (EL, D.d, D.f), "wq_down")
    _require(s_gate, torch.float32, (EL, D.f), "s_gate")
    _require(s_up, torch.float32, (EL, D.f), "s_up")
    _require(s_down, torch.float32, (EL, D.d), "s_down")
    _require(offsets, torch.int32, (EL + 1,), "offsets")
    if x_perm.dtype != torch.bfloat16 or x_perm.shape[0] < cap or x_perm.shape[1] != D.d:
        raise ValueError("x_perm must be bf16 with at least T*k rows of d")
    y_perm = torch.empty((max(cap, 1), D.d), dtype=torch.bfloat16, device=dev) if y_perm is None else y_perm
    need = moe_expert_ffn_fp8_workspace_bytes(D)
    ws = _workspace(need, dev, stream) if ws is None else ws
    rc = load().moe_expert_ffn_fp8(C.byref(D), _ptr(x_perm), _ptr(offsets), _ptr(wq_gate),
                                   _ptr(s_gate), _ptr(wq_up), _ptr(s_up), _ptr(wq_down),
                                   _ptr(s_down), _ptr(y_perm), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "moe_expert_ffn_fp8")
    return y_perm


def moe_gate_up_fp8(dims, x_perm, offsets, wq_gate, s_gate, wq_up, s_up, h=None, ws=None,
                    stream=None):
    """GEMM0 + SiLU-mul of the W8A8 FFN.  Returns h bf16 [T*k, f]."""
    import torch
    D = _dims(dims)
    dev = x_perm.device
    EL, cap = D.e_hi - D.e_lo, D.T * D.k
    _require(wq_gate, torch.uint8, (EL, D.f, D.d), "wq_gate")
    _require(wq_up, torch.uint8, (EL, D.f, D.d), "wq_up")
    _require(s_gate, torch.float32, (EL, D.f), "s_gate")
    _require(s_up, torch.float32, (EL, D.f), "s_up")
    _require(offsets, torch.int32, (EL + 1,), "offsets")
    if x_perm.dtype != torch.bfloat16 or x_perm.shape[0] < cap or x_perm.shape[1] != D.d:
        raise ValueError("x_perm must be bf16 with at least T*k rows of d")
    h = torch.empty((max(cap, 1), D.f), dtype=torch.bfloat16, device=dev) if h is None else h
    ws = _workspace(moe_expert_ffn_fp8_workspace_bytes(D), dev, stream) if ws is None else ws
    rc = load().moe_gate_up_fp8(C.byref(D), _ptr(x_perm), _ptr(offsets), _ptr(wq_gate),
                                _ptr(s_gate), _ptr(wq_up), _ptr(s_up), _ptr(h), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "moe_gate_up_fp8")
    return h


def moe_down_fp8(dims, h, offsets, wq_down, s_down, y_perm=None, ws=None, stream=None):
    """GEMM1 of the W8A8 FFN on bf16 rows h [T*k, f].  Returns y_perm bf16 [T*k, d]."""
    import torch
    D = _dims(dims)
    dev = h.device
    EL, cap = D.e_hi - D.e_lo, D.T * D.k
    _require(wq_down, torch.uint8, (EL, D.d, D.f), "wq_down")
    _require(s_down, torch.float32, (EL, D.d), "s_down")
    _require(offsets, torch.int32, (EL + 1,), "offsets")
    if h.dtype != torch.bfloat16 or h.shape[0] < cap or h.shape[1] != D.f:
        raise ValueError("h must be bf16 with at least T*k rows of f")
    y_perm = torch.empty((max(cap, 1), D.d), dtype=torch.bfloat16, device=dev) if y_perm is None else y_perm
    ws = _workspace(moe_expert_ffn_fp8_workspace_bytes(D), dev, stream) if ws is None else ws
    rc = load().moe_down_fp8(C.byref(D), _ptr(h), _ptr(offsets), _ptr(wq_down), _ptr(s_down),
                             _ptr(y_perm), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream))
    _check(rc, "moe_down_fp8")
    return y_perm


def moe_layer_fp8_workspace_bytes(dims) -> int:
    return int(load().moe_layer_fp8_workspace_bytes(C.byref(_dims(dims))))


def moe_layer_fp8(dims, x, w_router, wq_gate, s_gate, wq_up, s_up, wq_down, s_down, bias=None,
                  out=None, out_dtype: int = MOE_BF16, topk_ids_out=None, topk_w_out=None,
                  ws=None, opts: Optional[MoELayerOpts] = None, stream=None):
    """Forward pass with the W8A8 expert FFN: separate launches by default
    (MOE_SCHEDULE_AUTO / MOE_SCHEDULE_STAGED), one persistent kernel with
    opts.schedule = MOE_SCHEDULE_PERSISTENT (same bits).  Returns out [T, d]."""
    import torch
    D = _dims(dims)
    dev = x.device
    EL = D.e_hi - D.e_lo
    _require(x, torch.bfloat16, (D.T, D.d), "x")
    _require(w_router, torch.bfloat16, (D.E, D.d), "w_router")
    _require(wq_gate, torch.uint8, (EL, D.f, D.d), "wq_gate")
    _require(wq_up, torch.uint8, (EL, D.f, D.d), "wq_up")
    _require(wq_down, torch.uint8, (EL, D.d, D.f), "wq_down")
    _require(s_gate, torch.float32, (EL, D.f), "s_gate")
    _require(s_up, torch.float32, (EL, D.f), "s_up")
    _require(s_down, torch.float32, (EL, D.d), "s_down")
    if bias is not None:
        _require(bias, torch.float32, (D.E,), "bias")
    dt = torch.float32 if out_dtype == MOE_F32 else torch.bfloat16
    out = torch.empty((D.T, D.d), dtype=dt, device=dev) if out is None else out
    need = moe_layer_fp8_workspace_bytes(D)
    ws = _workspace(need, dev, stream) if ws is None else ws
    rc = load().moe_layer_fp8(C.byref(D), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(wq_gate),
                              _ptr(s_gate), _ptr(wq_up), _ptr(s_up), _ptr(wq_down), _ptr(s_down),
                              _ptr(out), out_dtype, _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
                              ws.numel() * ws.element_size(),
                              C.byref(opts) if opts is not None else None, _stream(stream))
    _check(rc, "moe_layer_fp8")
    return out


def moe_combine(dims, y_perm, inv_perm, topk_w, out=None, out_dtype: int = MOE_BF16, stream=None):
    """Gate-weighted combine.  Returns out [T, d] (bf16 or f32)."""
    import torch
    D = _dims(dims)
    dev = y_perm.device
    _require(inv_perm, torch.int32, (D.T, D.k), "inv_perm")
    _require(topk_w, torch.float32, (D.T, D.k), "topk_w")
    dt = torch.float32 if out_dtype == MOE_F32 else torch.bfloat16
    out = torch.empty((D.T, D.d), dtype=dt, device=dev) if out is None else out
    rc = load().moe_combine(C.byref(D), _ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(out),
                            int(out_dtype), _stream(stream))
    _check(rc, "moe_combine")
    return out


def moe_layer(dims, x, w_router, w_gate, w_up, w_down, bias=None, out=None,
              out_dtype: int = MOE_BF16, topk_ids_out=None, topk_w_out=None, ws=None,
              opts: Optional[MoELayerOpts] = None, check_status: bool = False, stream=None):
    """Whole layer forward.  Returns out [T, d].  opts: a MoELayerOpts (see
    layer_opts) or None for the defaults.  check_status: synchronise and raise
    MoEError if a device-side wait timed out (the workspace's status word)."""
    import torch
    D = _dims(dims)
    dev = x.device
    EL = D.e_hi - D.e_lo
    _require(x, torch.bfloat16, (D.T, D.d), "x")
    _require(w_router, torch.bfloat16, (D.E, D.d), "w_router")
    _require(w_gate, torch.bfloat16, (EL, D.f, D.d), "w_gate")
    _require(w_up, torch.bfloat16, (EL, D.f, D.d), "w_up")
    _require(w_down, torch.bfloat16, (EL, D.d, D.f), "w_down")
    if bias is not None:
        _require(bias, torch.float32, (D.E,), "bias")
    dt = torch.float32 if out_dtype == MOE_F32 else torch.bfloat16
    out = torch.empty((D.T, D.d), dtype=dt, device=dev) if out is None else out
    need = moe_layer_workspace_bytes(D)
    ws = _workspace(need, dev, stream) if ws is None else ws
    rc = load().moe_layer(C.byref(D), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
                          _ptr(w_up), _ptr(w_down), _ptr(out), int(out_dtype), _ptr(topk_ids_out),
                          _ptr(topk_w_out), _ptr(ws), ws.numel() * ws.element_size(),
                          C.byref(opts) if opts is not None else None, _stream(stream))
    _check(rc, "moe_layer")
    if check_status:
        _check(moe_device_status(D, ws, stream), "moe_layer (device status)")
    return out


def moe_device_status(dims, ws, stream=None) -> int:
    return int(load().moe_device_status(C.byref(_dims(dims)), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def moe_wall_clock_hz() -> int:
    return int(load().moe_wall_clock_hz())
