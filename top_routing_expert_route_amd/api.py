"""Thin Python binding over the C ABI in include/moe.h.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the layer runs in the HIP kernels of libmoe_hip.so.
There is no fallback: if the library is missing, every call raises.

The low-level functions (``lib().moe_route`` ...) are the C entry points with
ctypes signatures; the functions of this module with the same names allocate
outputs and workspaces with torch and call them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_hip.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (status %d)" % (msg, status))
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("capacity_factor", ctypes.c_float), ("expert_begin", ctypes.c_int32),
                ("num_local_experts", ctypes.c_int32), ("has_shared", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("dtype", ctypes.c_int)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w1", "b1", "w2", "b2", "ws1", "bs1", "ws2", "bs2", "sel_bias")]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_router", "db_router", "dw1", "db1", "dw2", "db2", "dws1", "dbs1", "dws2", "dbs2",
                 "dlogits")]


class Outputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "expert_count", "f", "P", "l_aux", "seg_offsets", "kept_count",
                 "slot_row", "row_src", "n_dropped")]


EXPORTS = ["moe_abi_version", "moe_status_string", "moe_last_error", "moe_max_rows", "moe_route_workspace_size",
           "moe_route", "moe_dispatch_workspace_size", "moe_dispatch", "moe_dispatch_noalloc_scratch_bytes",
           "moe_dispatch_noalloc", "moe_grouped_gemm_workspace_size",
           "moe_grouped_gemm", "moe_expert_ffn", "moe_combine", "moe_forward_workspace_size", "moe_forward",
           "moe_forward_overlap_workspace_size", "moe_forward_overlap", "moe_backward_workspace_size",
           "moe_backward", "moe_forward_save", "moe_backward_saved"]

_lib = None


def lib():
    """The loaded C library with ctypes signatures (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoe_hip.so is not built (%s); run __graft_entry__.build() or "
                           "python top_routing_expert_route_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.moe_abi_version.argtypes, L.moe_abi_version.restype = [], I
    L.moe_status_string.argtypes, L.moe_status_string.restype = [I], ctypes.c_char_p
    L.moe_last_error.argtypes, L.moe_last_error.restype = [], ctypes.c_char_p
    L.moe_max_rows.argtypes, L.moe_max_rows.restype = [I64, I, I, F, I], I64
    L.moe_route_workspace_size.argtypes, L.moe_route_workspace_size.restype = [I64, I, I], SZ
    L.moe_route.argtypes = [P, I, P, P, P, I64, I, I, I, F, P, P, P, P, P, P, P, SZ, P]
    L.moe_route.restype = I
    L.moe_dispatch_workspace_size.argtypes, L.moe_dispatch_workspace_size.restype = [I64, I, I], SZ
    L.moe_dispatch.argtypes = [P, I, P, I64, I, I, I, F, I, I, P, P, P, P, P, I64, P, P, SZ, P]
    L.moe_dispatch.restype = I
    L.moe_dispatch_noalloc_scratch_bytes.argtypes, L.moe_dispatch_noalloc_scratch_bytes.restype = [], SZ
    L.moe_dispatch_noalloc.argtypes = [P, I, P, I64, I, I, I, F, I, I, P, P, P, P, P, I64, P, P]
    L.moe_dispatch_noalloc.restype = I
    L.moe_grouped_gemm_workspace_size.argtypes, L.moe_grouped_gemm_workspace_size.restype = [], SZ
    L.moe_grouped_gemm.argtypes = [P, P, I, I64, I, I, I, P, P, I, P, P, SZ, P]
    L.moe_grouped_gemm.restype = I
    L.moe_expert_ffn.argtypes = [P, P, I, I64, I, I, I, P, P, P, P, P, P, P, SZ, P]
    L.moe_expert_ffn.restype = I
    L.moe_combine.argtypes = [P, I64, P, P, P, I64, I, I, I, P, P]
    L.moe_combine.restype = I
    L.moe_forward_workspace_size.argtypes = [ctypes.POINTER(Problem)]
    L.moe_forward_workspace_size.restype = SZ
    L.moe_forward.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Weights), P, P, ctypes.POINTER(Outputs), P,
                              SZ, P]
    L.moe_forward.restype = I
    L.moe_forward_overlap_workspace_size.argtypes = [ctypes.POINTER(Problem)]
    L.moe_forward_overlap_workspace_size.restype = SZ
    L.moe_forward_overlap.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Weights), P, P,
                                      ctypes.POINTER(Outputs), P, SZ, P, P, P, P]
    L.moe_forward_overlap.restype = I
    L.moe_backward_workspace_size.argtypes = [ctypes.POINTER(Problem)]
    L.moe_backward_workspace_size.restype = SZ
    L.moe_backward.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Weights), P, P, F, ctypes.POINTER(Grads), P,
                               SZ, P]
    L.moe_backward.restype = I
    L.moe_forward_save.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Weights), P, P, ctypes.POINTER(Outputs),
                                   P, P, P, SZ, P]
    L.moe_forward_save.restype = I
    L.moe_backward_saved.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Weights), P, P, F, P, P,
                                     ctypes.POINTER(Grads), P, SZ, P]
    L.moe_backward_saved.restype = I
    _lib = L
    return L


def check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode() or lib().moe_status_string(status).decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError("activations and expert weights must be bfloat16 or float32, got %s" % t.dtype)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ws(nbytes: int, dev) -> torch.Tensor:
    """A workspace: zero-filled once at allocation (its leading counters must
    start at zero; every call leaves them zero)."""
    return torch.zeros(max(1, int(nbytes)), dtype=torch.uint8, device=dev)


_ws_cache = {}


def workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-initialised workspace of at least nbytes, cached per device and
    reused by the step functions below (their calls are ordered on the
    current stream; every call leaves the leading counters zero)."""
    dev = torch.device(device)
    buf = _ws_cache.get(dev)
    if buf is None or buf.numel() < nbytes:
        buf = _ws(nbytes, dev)
        _ws_cache[dev] = buf
    return buf


def _check_out(out: dict, spec: dict, dev) -> None:
    """Caller-supplied outputs: each named tensor must have the shape, dtype
    and device the call writes (the library trusts the sizes it is given)."""
    for name, (shape, dtype) in spec.items():
        t = out.get(name)
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != dev \
                or not t.is_contiguous():
            raise ValueError("out[%r]: need a contiguous %s tensor of shape %s on %s" % (name, dtype, shape, dev))


def max_rows(T: int, E: int, k: int, capacity_factor: float = 0.0, num_local_experts: int = 0) -> int:
    return int(lib().moe_max_rows(T, E, k, capacity_factor, num_local_experts))


# ----------------------------------------------------------------- steps --

def moe_route(x: torch.Tensor, w_router: torch.Tensor, b_router: Optional[torch.Tensor], k: int,
              alpha: float = 0.01, sel_bias: Optional[torch.Tensor] = None, out: Optional[dict] = None) -> dict:
    """moe_route; `out` (the dict an earlier call returned, same sizes)
    receives the results instead of new tensors."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    if out is None:
        out = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                   topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
                   expert_count=torch.empty(E, dtype=torch.int32, device=dev),
                   f=torch.empty(E, dtype=torch.float32, device=dev),
                   P=torch.empty(E, dtype=torch.float32, device=dev),
                   l_aux=torch.empty(1, dtype=torch.float32, device=dev))
    else:
        _check_out(out, dict(topk_idx=((T, k), torch.int32), topk_w=((T, k), torch.float32),
                             expert_count=((E,), torch.int32), f=((E,), torch.float32), P=((E,), torch.float32),
                             l_aux=((1,), torch.float32)), dev)
    nb = lib().moe_route_workspace_size(T, d, E)
    ws = workspace(dev, nb)
    check(lib().moe_route(_p(x), _dt(x), _p(w_router), _p(b_router), _p(sel_bias), T, d, E, k, alpha,
                          _p(out["topk_idx"]), _p(out["topk_w"]), _p(out["expert_count"]), _p(out["f"]),
                          _p(out["P"]), _p(out["l_aux"]), _p(ws), nb, _stream(dev)))
    return out


def moe_dispatch(x: Optional[torch.Tensor], topk_idx: torch.Tensor, E: int, capacity_factor: float = 0.0,
                 expert_begin: int = 0, num_local_experts: int = 0, with_x_perm: bool = True,
                 rows: Optional[int] = None, dtype: Optional[torch.dtype] = None, d: Optional[int] = None,
                 noalloc: bool = False, out: Optional[dict] = None) -> dict:
    """moe_dispatch with a torch workspace; with noalloc, moe_dispatch_noalloc
    (the library's static scratch, no workspace).  New outputs have row_src
    filled with -1 past the kept rows (the library writes rows [0, rows));
    `out` (the dict an earlier call returned, same sizes) receives the
    results instead, its rows past the kept ones left as they were."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    E_loc = num_local_experts if num_local_experts > 0 else E
    mr = max_rows(T, E, k, capacity_factor, num_local_experts) if rows is None else rows
    d = x.shape[1] if x is not None else d
    dt = _dt(x) if x is not None else (MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)
    if out is None:
        out = dict(seg_offsets=torch.empty(E_loc + 1, dtype=torch.int32, device=dev),
                   kept_count=torch.empty(E_loc, dtype=torch.int32, device=dev),
                   slot_row=torch.empty((T, k), dtype=torch.int32, device=dev),
                   row_src=torch.full((max(1, mr),), -1, dtype=torch.int32, device=dev),
                   n_dropped=torch.empty(1, dtype=torch.int32, device=dev),
                   x_perm=(torch.empty((max(1, mr), d), dtype=x.dtype, device=dev)
                           if (with_x_perm and x is not None) else None))
    else:
        spec = dict(seg_offsets=((E_loc + 1,), torch.int32), kept_count=((E_loc,), torch.int32),
                    slot_row=((T, k), torch.int32), row_src=((max(1, mr),), torch.int32),
                    n_dropped=((1,), torch.int32))
        if out.get("x_perm") is not None:
            if x is None:
                raise ValueError("out['x_perm'] needs x")
            spec["x_perm"] = ((max(1, mr), d), x.dtype)
        _check_out(out, spec, dev)
    if noalloc:
        check(lib().moe_dispatch_noalloc(_p(x), dt, _p(topk_idx), T, d, E, k, capacity_factor, expert_begin,
                                         num_local_experts, _p(out["seg_offsets"]), _p(out["kept_count"]),
                                         _p(out["slot_row"]), _p(out["row_src"]), _p(out["x_perm"]), mr,
                                         _p(out["n_dropped"]), _stream(dev)))
        out["max_rows"] = mr
        return out
    nb = lib().moe_dispatch_workspace_size(T, k, E_loc)
    ws = workspace(dev, nb)
    check(lib().moe_dispatch(_p(x), dt, _p(topk_idx), T, d, E, k, capacity_factor, expert_begin,
                             num_local_experts, _p(out["seg_offsets"]), _p(out["kept_count"]), _p(out["slot_row"]),
                             _p(out["row_src"]), _p(out["x_perm"]), mr, _p(out["n_dropped"]), _p(ws), nb,
                             _stream(dev)))
    out["max_rows"] = mr
    return out


_gemm_ws = {}


def gemm_workspace(device) -> torch.Tensor:
    """A cached device scratch buffer for the grouped GEMM's split tail."""
    dev = torch.device(device)
    if dev not in _gemm_ws:
        _gemm_ws[dev] = _ws(lib().moe_grouped_gemm_workspace_size(), dev)
    return _gemm_ws[dev]


def moe_grouped_gemm(a: torch.Tensor, seg_offsets: Optional[torch.Tensor], w: torch.Tensor,
                     bias: Optional[torch.Tensor], activation: int, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, use_ws: bool = True) -> torch.Tensor:
    rows, K = a.shape
    S, N, K2 = w.shape
    assert K2 == K
    if out is None:
        out = torch.empty((rows, N), dtype=a.dtype, device=a.device)
    if ws is None and use_ws:
        ws = gemm_workspace(a.device)
    nseg = S if seg_offsets is not None else 1
    check(lib().moe_grouped_gemm(_p(a), _p(seg_offsets), nseg, rows, N, K, _dt(a), _p(w), _p(bias), activation,
                                 _p(out), _p(ws), 0 if ws is None else ws.numel(), _stream(a.device)))
    return out


def moe_expert_ffn(x_perm: torch.Tensor, seg_offsets: torch.Tensor, w1, b1, w2, b2,
                   h: Optional[torch.Tensor] = None, y_perm: Optional[torch.Tensor] = None,
                   use_ws: bool = True):
    rows, d = x_perm.shape
    S, ffn, _ = w1.shape
    if h is None:
        h = torch.empty((rows, ffn), dtype=x_perm.dtype, device=x_perm.device)
    if y_perm is None:
        y_perm = torch.empty((rows, d), dtype=x_perm.dtype, device=x_perm.device)
    ws = gemm_workspace(x_perm.device) if use_ws else None
    check(lib().moe_expert_ffn(_p(x_perm), _p(seg_offsets), S, rows, d, ffn, _dt(x_perm), _p(w1), _p(b1), _p(w2),
                               _p(b2), _p(h), _p(y_perm), _p(ws), 0 if ws is None else ws.numel(),
                               _stream(x_perm.device)))
    return h, y_perm


def moe_combine(y_perm: torch.Tensor, slot_row: torch.Tensor, topk_w: torch.Tensor,
                y_shared: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    rows, d = y_perm.shape
    T, k = slot_row.shape
    if y is None:
        y = torch.empty((T, d), dtype=y_perm.dtype, device=y_perm.device)
    check(lib().moe_combine(_p(y_perm), rows, _p(slot_row), _p(topk_w), _p(y_shared), T, d, k, _dt(y_perm), _p(y),
                            _stream(y_perm.device)))
    return y


class Layer:
    """Device tensors of one layer plus a reusable workspace for moe_forward."""

    def __init__(self, T, d, E, k, ffn, dtype, capacity_factor=0.0, expert_begin=0, num_local_experts=0,
                 alpha=0.01, w_router=None, b_router=None, w1=None, b1=None, w2=None, b2=None,
                 ws1=None, bs1=None, ws2=None, bs2=None, device="cuda", sel_bias=None):
        self.problem = Problem(T, d, E, k, ffn, capacity_factor, expert_begin, num_local_experts,
                               1 if ws1 is not None else 0, alpha, MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)
        self.tensors = dict(w_router=w_router, b_router=b_router, w1=w1, b1=b1, w2=w2, b2=b2,
                            ws1=ws1, bs1=bs1, ws2=ws2, bs2=bs2, sel_bias=sel_bias)
        self.weights = Weights(*[_p(self.tensors[n]) for n, _ in Weights._fields_])
        self.E_loc = num_local_experts if num_local_experts > 0 else E
        self.max_rows = max_rows(T, E, k, capacity_factor, num_local_experts)
        self.device = torch.device(device)
        self.dtype = dtype
        self.outputs = None
        self.out_struct = Outputs()
        self.ws = None

    def alloc_outputs(self):
        p, dev = self.problem, self.device
        self.outputs = dict(
            topk_idx=torch.empty((p.T, p.k), dtype=torch.int32, device=dev),
            topk_w=torch.empty((p.T, p.k), dtype=torch.float32, device=dev),
            expert_count=torch.empty(p.E, dtype=torch.int32, device=dev),
            f=torch.empty(p.E, dtype=torch.float32, device=dev),
            P=torch.empty(p.E, dtype=torch.float32, device=dev),
            l_aux=torch.empty(1, dtype=torch.float32, device=dev),
            seg_offsets=torch.empty(self.E_loc + 1, dtype=torch.int32, device=dev),
            kept_count=torch.empty(self.E_loc, dtype=torch.int32, device=dev),
            slot_row=torch.empty((p.T, p.k), dtype=torch.int32, device=dev),
            row_src=torch.empty(max(1, self.max_rows), dtype=torch.int32, device=dev),
            n_dropped=torch.empty(1, dtype=torch.int32, device=dev))
        self.out_struct = Outputs(*[_p(self.outputs[n]) for n, _ in Outputs._fields_])
        self.ws = None
        return self.outputs

    def workspace_bytes(self, overlap: bool = False) -> int:
        fn = lib().moe_forward_overlap_workspace_size if overlap else lib().moe_forward_workspace_size
        return int(fn(ctypes.byref(self.problem)))

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                side_stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """moe_forward on the current stream; with side_stream, moe_forward_overlap
        (the shared expert runs on side_stream)."""
        overlap = side_stream is not None
        if self.ws is None or getattr(self, "_ws_overlap", None) != overlap:
            self.ws = _ws(self.workspace_bytes(overlap), self.device)
            self._ws_overlap = overlap
        if y is None:
            y = torch.empty((self.problem.T, self.problem.d), dtype=x.dtype, device=x.device)
        if overlap:
            if getattr(self, "_events", None) is None:
                # caller-owned fork/join events, created once per layer (torch
                # creates an event's handle at its first record)
                self._events = (torch.cuda.Event(), torch.cuda.Event())
                for e in self._events:
                    e.record(torch.cuda.current_stream(self.device))
            fork, join = self._events
            check(lib().moe_forward_overlap(ctypes.byref(self.problem), ctypes.byref(self.weights), _p(x), _p(y),
                                            ctypes.byref(self.out_struct), _p(self.ws), self.ws.numel(),
                                            _stream(x.device), ctypes.c_void_p(side_stream.cuda_stream),
                                            ctypes.c_void_p(fork.cuda_event), ctypes.c_void_p(join.cuda_event)))
        else:
            check(lib().moe_forward(ctypes.byref(self.problem), ctypes.byref(self.weights), _p(x), _p(y),
                                    ctypes.byref(self.out_struct), _p(self.ws), self.ws.numel(),
                                    _stream(x.device)))
        return y

    def forward_save(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        """moe_forward_save on the current stream: moe_forward that also keeps
        the first Linear's fp32 pre-activations (self.u_saved, and
        self.u_shared_saved with a shared expert) for backward(saved=True)."""
        p, dev = self.problem, self.device
        if self.ws is None or getattr(self, "_ws_overlap", None):
            self.ws = _ws(self.workspace_bytes(False), dev)
            self._ws_overlap = False
        if getattr(self, "u_saved", None) is None:
            self.u_saved = torch.empty((max(1, self.max_rows), p.ffn), dtype=torch.float32, device=dev)
            self.u_shared_saved = (torch.empty((max(1, p.T), p.ffn), dtype=torch.float32, device=dev)
                                   if p.has_shared else None)
        if y is None:
            y = torch.empty((p.T, p.d), dtype=x.dtype, device=x.device)
        check(lib().moe_forward_save(ctypes.byref(p), ctypes.byref(self.weights), _p(x), _p(y),
                                     ctypes.byref(self.out_struct), _p(self.u_saved), _p(self.u_shared_saved),
                                     _p(self.ws), self.ws.numel(), _stream(x.device)))
        return y

    def backward_workspace_bytes(self) -> int:
        return int(lib().moe_backward_workspace_size(ctypes.byref(self.problem)))

    def backward(self, x: torch.Tensor, dy: torch.Tensor, g_aux: float = 0.0, bias_grads: bool = True,
                 dlogits: bool = False, grads: Optional[dict] = None, saved: bool = False) -> dict:
        """moe_backward on the current stream: float32 gradients of a loss with
        dL/dY = dy and dL/dL_aux = g_aux.  Returns (or fills) a dict with dx,
        dw_router, dw1, dw2 (dws1, dws2 with a shared expert), the bias
        gradients when bias_grads, and dlogits when asked for.  With saved,
        moe_backward_saved on the pre-activations of the last forward_save."""
        p, dev = self.problem, self.device
        if grads is None:
            f32 = dict(dtype=torch.float32, device=dev)
            E_loc, T, d, E, F = self.E_loc, p.T, p.d, p.E, p.ffn
            grads = dict(dx=torch.empty((T, d), **f32), dw_router=torch.empty((E, d), **f32),
                         dw1=torch.empty((E_loc, F, d), **f32), dw2=torch.empty((E_loc, d, F), **f32))
            if bias_grads:
                grads.update(db_router=torch.empty(E, **f32), db1=torch.empty((E_loc, F), **f32),
                             db2=torch.empty((E_loc, d), **f32))
            if p.has_shared:
                grads.update(dws1=torch.empty((F, d), **f32), dws2=torch.empty((d, F), **f32))
                if bias_grads:
                    grads.update(dbs1=torch.empty(F, **f32), dbs2=torch.empty(d, **f32))
            if dlogits:
                grads["dlogits"] = torch.empty((T, E), **f32)
        gs = Grads(*[_p(grads.get(n)) for n, _ in Grads._fields_])
        nb = self.backward_workspace_bytes()
        if getattr(self, "_bws", None) is None or self._bws.numel() < nb:
            self._bws = _ws(nb, dev)
        if saved:
            if getattr(self, "u_saved", None) is None:
                raise RuntimeError("backward(saved=True) needs a forward_save first")
            check(lib().moe_backward_saved(ctypes.byref(self.problem), ctypes.byref(self.weights), _p(x), _p(dy),
                                           float(g_aux), _p(self.u_saved), _p(self.u_shared_saved), ctypes.byref(gs),
                                           _p(self._bws), self._bws.numel(), _stream(x.device)))
        else:
            check(lib().moe_backward(ctypes.byref(self.problem), ctypes.byref(self.weights), _p(x), _p(dy),
                                     float(g_aux), ctypes.byref(gs), _p(self._bws), self._bws.numel(),
                                     _stream(x.device)))
        return grads
