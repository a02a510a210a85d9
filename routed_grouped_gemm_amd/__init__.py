"""Python binding of libmoe.so, the MI355X MoE-layer forward (C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch is used for device memory (tensor storage and data_ptr()) and for
the current HIP stream; nothing here computes any part of the layer.

    import routed_grouped_gemm_amd as moe
    p = moe.problem(T, d, n, E, k, act="bf16", w="bf16", layout="packed")
    packed = moe.pack_weights(p, weights)         # once, at load time (rowmajor: skip)
    ws = moe.alloc_workspace(p)                   # caller-owned, initialised once
    out = moe.forward(p, hidden, w_router, None, packed, ws)

If the library has not been built, importing works but every call raises; there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = ["MoEError", "problem", "workspace_size", "plan_describe", "alloc_workspace", "workspace_init", "route",
           "permute", "forward", "forward_noalloc", "pack_weights", "last_device_error", "abi_version", "status_string",
           "MoELayer", "LIB_PATH", "HEADER_PATH", "header_functions", "F32", "BF16", "FP8_E4M3",
           "ROWMAJOR", "PACKED", "NOALLOC_SCRATCH_BYTES"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

F32, BF16, FP8_E4M3 = 0, 1, 2
AQ_NONE, AQ_FP8 = 0, 1  # moe_act_quant
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
ROWMAJOR, PACKED = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h
_LAYOUT = {"rowmajor": ROWMAJOR, "packed": PACKED}
_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP", 5: "MOE_ERR_DEVICE_FAULT"}


class MoEError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_STATUS.get(code, code)}")


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("n", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("scale_block", ctypes.c_int32), ("w_layout", ctypes.c_int32),
                ("act_quant", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down",
                 "sh_s_gate", "sh_s_up", "sh_s_down")]


class RouteOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_ids", "topk_weights", "logits", "counts", "offsets", "perm", "inv_perm")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("m_tile_rows", ctypes.c_int32), ("gateup_cols", ctypes.c_int32), ("down_cols", ctypes.c_int32),
                ("router_k_split", ctypes.c_int32), ("max_m_tiles", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("fp8_activations", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class LaunchOptions(ctypes.Structure):
    _fields_ = [("grid_wgs", ctypes.c_int32), ("schedule", ctypes.c_int32), ("trace", ctypes.c_void_p),
                ("trace_bytes", ctypes.c_int64), ("m_tile_rows", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m routed_grouped_gemm_amd.build` "
                           "(there is no fallback implementation)")
    import torch  # noqa: F401  (torch's HIP runtime must be the one the library binds to)
    L = ctypes.CDLL(LIB_PATH)
    P, VP, SZ, I = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.moe_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    L.moe_workspace_init.argtypes = [VP, SZ, VP]
    L.moe_plan_describe.argtypes = [P, ctypes.POINTER(PlanInfo)]
    L.moe_route.argtypes = [P, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
    L.moe_permute.argtypes = [P, VP, VP, VP, VP, VP, VP, SZ, VP]
    L.moe_forward.argtypes = [P, VP, VP, VP, ctypes.POINTER(Weights), VP, ctypes.POINTER(RouteOut), VP, SZ, VP]
    L.moe_forward_ex.argtypes = L.moe_forward.argtypes + [ctypes.POINTER(LaunchOptions)]
    L.moe_forward_noalloc.argtypes = [P, VP, VP, VP, ctypes.POINTER(Weights), VP, ctypes.POINTER(RouteOut), VP]
    L.moe_pack_weights.argtypes = [P, ctypes.POINTER(Weights), ctypes.POINTER(Weights), VP]
    L.moe_last_device_error.argtypes = [VP, VP]
    L.moe_status_string.argtypes = [I]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_abi_version.argtypes = []
    for fn in ("moe_workspace_size", "moe_workspace_init", "moe_plan_describe", "moe_route", "moe_permute", "moe_forward",
               "moe_forward_ex", "moe_forward_noalloc", "moe_pack_weights", "moe_last_device_error", "moe_abi_version"):
        getattr(L, fn).restype = I
    _lib = L
    return L


def lib():
    return _load()


def header_functions():
    """Names of the functions include/moe.h declares."""
    src = open(HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def _check(code: int, where: str):
    if code != 0:
        raise MoEError(code, where)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


_ESIZE = {F32: 4, BF16: 2, FP8_E4M3: 1}


def _sized(t, numel, esize, name):
    """The library reads and writes through bare pointers: a tensor smaller than the problem
    needs, or of another element width, would take it out of bounds, so it is refused here."""
    if t is None:
        return
    if t.numel() < numel or t.element_size() != esize:
        raise ValueError(f"{name}: needs {numel} elements of {esize} bytes, got {t.numel()} of "
                         f"{t.element_size()}")


def _check_inputs(p: Problem, hidden, w_router, bias, out=None):
    a = _ESIZE.get(p.act_dtype, 0)
    _sized(hidden, p.T * p.d, a, "hidden")
    _sized(w_router, p.E * p.d, a, "w_router")
    _sized(bias, p.E, 4, "bias")
    _sized(out, p.T * p.d, a, "out")


def _check_weights(p: Problem, weights: dict):
    """Sizes of the expert (and shared-expert) matrices and, for fp8, their block scales."""
    w = _ESIZE.get(p.w_dtype, 0)
    E, d, n = p.E, p.d, p.n
    sh = p.n_shared > 0
    for key, rows in (("w_gate", E), ("w_up", E), ("w_down", E), ("sh_gate", 1), ("sh_up", 1), ("sh_down", 1)):
        if key.startswith("sh_") and not sh:
            continue
        _sized(weights.get(key), rows * n * d, w, key)
    if p.w_dtype == FP8_E4M3:
        nb = (n // 128) * (d // 128)
        for key, rows in (("s_gate", E), ("s_up", E), ("s_down", E), ("sh_s_gate", 1), ("sh_s_up", 1),
                          ("sh_s_down", 1)):
            if key.startswith("sh_") and not sh:
                continue
            _sized(weights.get(key), rows * nb, 4, key)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def abi_version() -> int:
    return _load().moe_abi_version()


def status_string(code: int) -> str:
    return _load().moe_status_string(code).decode()


def problem(T, d, n, E, k, n_shared=0, act="bf16", w="bf16", layout="rowmajor", act_quant=False) -> Problem:
    """act_quant: the fp8-activation mode of the expert GEMMs (moe_problem.act_quant, fp8
    weights only)."""
    wd = _DT[w]
    return Problem(int(T), int(d), int(n), int(E), int(k), int(n_shared), _DT[act], wd,
                   128 if wd == FP8_E4M3 else 0, _LAYOUT[layout], AQ_FP8 if act_quant else AQ_NONE)


def workspace_size(p: Problem) -> int:
    out = ctypes.c_size_t(0)
    _check(_load().moe_workspace_size(ctypes.byref(p), ctypes.byref(out)), "moe_workspace_size")
    return out.value


def plan_describe(p: Problem) -> dict:
    """The tiling the library chooses for problem p (moe_plan_describe): m-tile rows, columns
    per gate/up and down work item, router K split, bound on routed m-tiles."""
    info = PlanInfo()
    _check(_load().moe_plan_describe(ctypes.byref(p), ctypes.byref(info)), "moe_plan_describe")
    return {f[0]: getattr(info, f[0]) for f in PlanInfo._fields_ if f[0] != "reserved"}


def workspace_init(ws: torch.Tensor):
    _check(_load().moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream()), "moe_workspace_init")


def alloc_workspace(p: Problem, device="cuda", extra: int = 0) -> torch.Tensor:
    """A caller-owned workspace for problem p (256-byte aligned), initialised."""
    nbytes = workspace_size(p) + extra
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + nbytes]
    workspace_init(ws)
    return ws


def _ws(ws):
    return _ptr(ws), ws.numel() * ws.element_size()


def route(p: Problem, hidden, w_router, bias, ws, want_logits=False):
    dev = hidden.device
    T, k, E = p.T, p.k, p.E
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    _check_inputs(p, hidden, w_router, bias)
    wp, wb = _ws(ws)
    _check(_load().moe_route(ctypes.byref(p), _ptr(hidden), _ptr(w_router), _ptr(bias), _ptr(ids), _ptr(wts),
                             _ptr(logits), wp, wb, _stream()), "moe_route")
    return ids, wts, logits


def permute(p: Problem, ids, ws):
    dev = ids.device
    T, k, E = p.T, p.k, p.E
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    _sized(ids, T * k, 4, "ids")
    wp, wb = _ws(ws)
    _check(_load().moe_permute(ctypes.byref(p), _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv),
                               wp, wb, _stream()), "moe_permute")
    return counts, offsets, perm, inv


_WKEYS = [f[0] for f in Weights._fields_]


def make_weights(weights: dict) -> Weights:
    return Weights(*[_ptr(weights.get(key)) for key in _WKEYS])


def forward(p: Problem, hidden, w_router, bias, weights, ws, out=None, route_out=False, grid_wgs=0,
            schedule=0, trace=None, m_tile_rows=0, group_m=0):
    """The whole layer.  weights: dict with w_gate, w_up, w_down (+ s_*, sh_*) device tensors,
    or a prebuilt Weights struct.  trace: optional device tensor receiving one 32-byte record
    per work item; m_tile_rows, group_m: overrides of the tile table (see moe_launch_options
    in include/moe.h).  Returns out, or (out, dict of routing tensors)."""
    dev = hidden.device
    T, k, E, d = p.T, p.k, p.E, p.d
    if out is None:
        out = torch.empty((T, d), dtype=hidden.dtype, device=dev)
    _check_inputs(p, hidden, w_router, bias, out)
    if not isinstance(weights, Weights):
        _check_weights(p, weights)
    W = weights if isinstance(weights, Weights) else make_weights(weights)
    ro = None
    rdict = None
    if route_out:
        rdict = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                     topk_weights=torch.empty((T, k), dtype=torch.float32, device=dev),
                     logits=torch.empty((T, E), dtype=torch.float32, device=dev),
                     counts=torch.empty(E, dtype=torch.int32, device=dev),
                     offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                     perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                     inv_perm=torch.empty(T * k, dtype=torch.int32, device=dev))
        ro = RouteOut(*[_ptr(rdict[f[0]]) for f in RouteOut._fields_])
    wp, wb = _ws(ws)
    L = _load()
    if grid_wgs or schedule or trace is not None or m_tile_rows or group_m:
        opts = LaunchOptions(int(grid_wgs), int(schedule), _ptr(trace),
                             0 if trace is None else trace.numel() * trace.element_size(), int(m_tile_rows),
                             int(group_m))
        code = L.moe_forward_ex(ctypes.byref(p), _ptr(hidden), _ptr(w_router), _ptr(bias), ctypes.byref(W),
                                _ptr(out), ctypes.byref(ro) if ro is not None else None, wp, wb, _stream(),
                                ctypes.byref(opts))
    else:
        code = L.moe_forward(ctypes.byref(p), _ptr(hidden), _ptr(w_router), _ptr(bias), ctypes.byref(W),
                             _ptr(out), ctypes.byref(ro) if ro is not None else None, wp, wb, _stream())
    _check(code, "moe_forward")
    return (out, rdict) if route_out else out


def _route_dict(T, k, E, dev):
    return dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                topk_weights=torch.empty((T, k), dtype=torch.float32, device=dev),
                logits=torch.empty((T, E), dtype=torch.float32, device=dev),
                counts=torch.empty(E, dtype=torch.int32, device=dev),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                inv_perm=torch.empty(T * k, dtype=torch.int32, device=dev))


def forward_noalloc(p: Problem, hidden, w_router, bias, weights, out=None, route_out=False):
    """The whole layer through moe_forward_noalloc: no workspace argument, the library's fixed
    device scratch instead (see include/moe.h).  Returns out, or (out, dict of routing
    tensors)."""
    dev = hidden.device
    T, k, E, d = p.T, p.k, p.E, p.d
    if out is None:
        out = torch.empty((T, d), dtype=hidden.dtype, device=dev)
    _check_inputs(p, hidden, w_router, bias, out)
    if not isinstance(weights, Weights):
        _check_weights(p, weights)
    W = weights if isinstance(weights, Weights) else make_weights(weights)
    rdict = _route_dict(T, k, E, dev) if route_out else None
    ro = RouteOut(*[_ptr(rdict[f[0]]) for f in RouteOut._fields_]) if route_out else None
    code = _load().moe_forward_noalloc(ctypes.byref(p), _ptr(hidden), _ptr(w_router), _ptr(bias), ctypes.byref(W),
                                       _ptr(out), ctypes.byref(ro) if ro is not None else None, _stream())
    _check(code, "moe_forward_noalloc")
    return (out, rdict) if route_out else out


_MATS = ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")


def pack_weights(p: Problem, weights: dict) -> dict:
    """Row-major expert weights -> a new dict whose matrices are in the packed layout
    (moe_pack_weights, on the current stream); scales are passed through unchanged."""
    _check_weights(p, weights)
    out = dict(weights)
    for key in _MATS:
        if weights.get(key) is not None:
            out[key] = torch.empty_like(weights[key])
    _check(_load().moe_pack_weights(ctypes.byref(p), ctypes.byref(make_weights(weights)),
                                    ctypes.byref(make_weights(out)), _stream()), "moe_pack_weights")
    return out


def last_device_error(ws) -> int:
    """Synchronizes the current stream; 0 if no device-side fault was flagged."""
    return _load().moe_last_device_error(_ptr(ws), _stream())


class MoELayer:
    """Holds device weights and a workspace; call with hidden [T, d] for the layer output."""

    def __init__(self, d, n, E, k, w_router, weights: dict, bias=None, n_shared=0, act="bf16", w="bf16"):
        """weights: row-major expert weights; they are packed once, here."""
        self.d, self.n, self.E, self.k, self.n_shared, self.act, self.w = d, n, E, k, n_shared, act, w
        self.w_router, self.bias = w_router, bias
        self.weights = pack_weights(problem(1, d, n, E, k, n_shared, act, w), weights)
        self._W = make_weights(self.weights)
        self._ws = None
        self._ws_T = -1

    def __call__(self, hidden, route_out=False):
        T = hidden.shape[0]
        p = problem(T, self.d, self.n, self.E, self.k, self.n_shared, self.act, self.w, layout="packed")
        if self._ws is None or workspace_size(p) > self._ws.numel():
            self._ws = alloc_workspace(p, hidden.device)
        return forward(p, hidden, self.w_router, self.bias, self._W, self._ws, route_out=route_out)
