"""CPU oracle for one MoE FFN layer forward (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package; the product path never does.  It wraps the plain C
implementation in ``oracle.c`` (double precision, plain loops) with numpy
marshalling, and shares no code with the HIP library.

See ``oracle.c`` for the passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT_F32 = 0
DT_BF16 = 1


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_route.argtypes = [P, I, P, P, P, i64, I, I, I, P, P, P, P, I]
        lib.oracle_route.restype = I
        lib.oracle_load_stats.argtypes = [P, P, i64, I, I, D, P, P, P, P]
        lib.oracle_load_stats.restype = I
        lib.oracle_capacity.argtypes = [P, i64, I, I, D, I, I, P, P, P, P, P, P]
        lib.oracle_capacity.restype = I
        lib.oracle_combine.argtypes = [P, I, i64, I, I, I, P, i64, P, P, P, I, I,
                                       P, P, P, P, P, P, P, P, P, I]
        lib.oracle_combine.restype = I
        lib.oracle_gelu.argtypes = [D]
        lib.oracle_gelu.restype = D
        lib.oracle_gelu_grad.argtypes = [D]
        lib.oracle_gelu_grad.restype = D
        lib.oracle_backward.argtypes = [P, I, i64, I, I, I, I, P, P, P, P, P, P, D, D, I, I,
                                        P, P, P, P, P, P, P, P, P,
                                        P, P, P, P, P, P, P, P, P, P, P, P, I]
        lib.oracle_backward.restype = I
        lib.oracle_backward_tokens.argtypes = [P, I, i64, I, I, I, I, P, P, P, P, P, P, D, D, I, I,
                                               P, P, P, P, P, P, P, P, P, P, i64, P, P, I]
        lib.oracle_backward_tokens.restype = I
        lib.oracle_ffn_grad_columns.argtypes = [P, I, i64, I, I, P, P, P, P, P, i64, P, P, I, P, P, P, P, I]
        lib.oracle_ffn_grad_columns.restype = I
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _threads(n: Optional[int]) -> int:
    if n is not None:
        return max(1, int(n))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float32:
        return DT_F32
    raise TypeError("oracle takes float32 arrays or uint16 bfloat16 bit patterns, got %s" % a.dtype)


@dataclass
class Route:
    logits: np.ndarray    # [T, E] float64
    probs: np.ndarray     # [T, E] float64
    topk_idx: np.ndarray  # [T, k] int32
    topk_w: np.ndarray    # [T, k] float64
    scores: Optional[np.ndarray] = None  # [T, E] float64: what top-k ranks (logits + sel_bias)


def route(x: np.ndarray, w_router: np.ndarray, b_router: Optional[np.ndarray], k: int,
          threads: Optional[int] = None, want_logits: bool = True,
          sel_bias: Optional[np.ndarray] = None) -> Route:
    """Router Linear, softmax, top-k.  ``sel_bias`` (optional, [E] float32)
    is added to the logits for the top-k choice only."""
    T, d = x.shape
    E = w_router.shape[0]
    x = np.ascontiguousarray(x)
    w_router = np.ascontiguousarray(w_router, dtype=np.float32)
    if b_router is not None:
        b_router = np.ascontiguousarray(b_router, dtype=np.float32)
    if sel_bias is not None:
        sel_bias = np.ascontiguousarray(sel_bias, dtype=np.float32)
    logits = np.empty((T, E), np.float64) if want_logits else None
    probs = np.empty((T, E), np.float64)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = _load().oracle_route(_ptr(x), _dtype_of(x), _ptr(w_router), _ptr(b_router), _ptr(sel_bias), T, d,
                              E, k, _ptr(logits), _ptr(probs), _ptr(idx), _ptr(w), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_route: invalid sizes")
    scores = None
    if logits is not None:
        scores = logits if sel_bias is None else logits + sel_bias.astype(np.float64)[None, :]
    return Route(logits, probs, idx, w, scores)


@dataclass
class Stats:
    count: np.ndarray   # [E] int64
    f: np.ndarray       # [E] float64
    P: np.ndarray       # [E] float64
    l_aux: float


def load_stats(topk_idx: np.ndarray, probs: np.ndarray, alpha: float = 0.01) -> Stats:
    T, k = topk_idx.shape
    E = probs.shape[1]
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    probs = np.ascontiguousarray(probs, dtype=np.float64)
    count = np.empty(E, np.int64)
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    l = np.zeros(1, np.float64)
    rc = _load().oracle_load_stats(_ptr(topk_idx), _ptr(probs), T, E, k, alpha,
                                   _ptr(count), _ptr(f), _ptr(P), _ptr(l))
    if rc != 0:
        raise ValueError("oracle_load_stats: invalid sizes")
    return Stats(count, f, P, float(l[0]))


@dataclass
class Dispatch:
    capacity: int             # -1 = no cap
    slot_row: np.ndarray      # [T, k] int32: row, -1 dropped, -2 remote
    row_src: np.ndarray       # [rows] int32: t*k+j of each row
    seg_offsets: np.ndarray   # [E_loc+1] int32
    kept_count: np.ndarray    # [E_loc] int32
    n_dropped: int


def capacity(topk_idx: np.ndarray, E: int, capacity_factor: float = 0.0,
             expert_begin: int = 0, num_local_experts: int = 0) -> Dispatch:
    T, k = topk_idx.shape
    E_loc = num_local_experts if num_local_experts > 0 else E
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    C = np.zeros(1, np.int64)
    slot_row = np.empty((T, k), np.int32)
    row_src = np.full(max(1, T * k), -1, np.int32)
    seg = np.empty(E_loc + 1, np.int32)
    kept = np.empty(E_loc, np.int32)
    nd = np.zeros(1, np.int64)
    rc = _load().oracle_capacity(_ptr(topk_idx), T, E, k, float(capacity_factor), expert_begin, E_loc,
                                 _ptr(C), _ptr(slot_row), _ptr(row_src), _ptr(seg), _ptr(kept), _ptr(nd))
    if rc != 0:
        raise ValueError("oracle_capacity: invalid sizes")
    rows = int(seg[-1])
    return Dispatch(int(C[0]), slot_row, row_src[:rows].copy(), seg, kept, int(nd[0]))


def combine(x: np.ndarray, tokens: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray,
            slot_row: np.ndarray, w1: np.ndarray, b1, w2: np.ndarray, b2,
            expert_begin: int = 0, ws1=None, bs1=None, ws2=None, bs2=None,
            threads: Optional[int] = None) -> np.ndarray:
    """Layer output (float64 [len(tokens), d]) for the listed tokens."""
    T, d = x.shape
    k = topk_idx.shape[1]
    E_loc, ffn, _ = w1.shape
    dt = _dtype_of(x)
    for a in (w1, w2, b1, b2, ws1, bs1, ws2, bs2):
        if a is not None and _dtype_of(a) != dt:
            raise TypeError("expert tensors must share the activation dtype")
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    x = np.ascontiguousarray(x)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float64)
    slot_row = np.ascontiguousarray(slot_row, dtype=np.int32)
    y = np.empty((len(tokens), d), np.float64)
    rc = _load().oracle_combine(_ptr(x), dt, T, d, k, ffn, _ptr(tokens), len(tokens),
                                _ptr(topk_idx), _ptr(topk_w), _ptr(slot_row), expert_begin, E_loc,
                                _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                _ptr(ws1), _ptr(bs1), _ptr(ws2), _ptr(bs2), _ptr(y), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_combine: invalid sizes or token ids")
    return y


def gelu(u: float) -> float:
    return float(_load().oracle_gelu(float(u)))


@dataclass
class Forward:
    route: Route
    stats: Stats
    dispatch: Dispatch
    tokens: np.ndarray
    y: np.ndarray


def forward(inp, tokens: Optional[np.ndarray] = None, threads: Optional[int] = None,
            topk_idx: Optional[np.ndarray] = None) -> Forward:
    """Whole layer on a workloads.LayerInputs.

    ``tokens`` restricts the (expensive) expert FFN to a subset of tokens; the
    routing, statistics and capacity always cover all T tokens.  If
    ``topk_idx`` is given (e.g. another implementation's selection), the
    statistics, capacity and output are conditioned on it, with the oracle's
    own probabilities at those indices as routing weights.
    """
    w = inp.w
    r = route(inp.x, inp.w_router, inp.b_router, w.k, threads=threads, sel_bias=getattr(inp, "sel_bias", None))
    idx = r.topk_idx if topk_idx is None else np.ascontiguousarray(topk_idx, dtype=np.int32)
    wts = np.take_along_axis(r.probs, idx.astype(np.int64).clip(0, w.E - 1), axis=1)
    st = load_stats(idx, r.probs, w.alpha)
    # the capacity factor is a float32 parameter of the layer
    dp = capacity(idx, w.E, float(np.float32(w.capacity_factor)), w.expert_begin, w.num_local_experts)
    if tokens is None:
        tokens = np.arange(w.T, dtype=np.int64)
    y = combine(inp.x, tokens, idx, wts, dp.slot_row, inp.w1, inp.b1, inp.w2, inp.b2,
                w.expert_begin, inp.ws1, inp.bs1, inp.ws2, inp.bs2, threads=threads)
    return Forward(r, st, dp, np.asarray(tokens), y)


def gelu_grad(u: float) -> float:
    return float(_load().oracle_gelu_grad(float(u)))


@dataclass
class Grads:
    dx: np.ndarray        # [T, d]
    dW_r: np.ndarray      # [E, d]
    db_r: np.ndarray      # [E]
    dW1: np.ndarray       # [E_loc, ffn, d]
    db1: np.ndarray       # [E_loc, ffn]
    dW2: np.ndarray       # [E_loc, d, ffn]
    db2: np.ndarray       # [E_loc, d]
    dWs1: Optional[np.ndarray]
    dbs1: Optional[np.ndarray]
    dWs2: Optional[np.ndarray]
    dbs2: Optional[np.ndarray]
    dlogits: np.ndarray   # [T, E]


def backward(inp, dY: np.ndarray, g_aux: float = 0.0, threads: Optional[int] = None,
             topk_idx: Optional[np.ndarray] = None) -> Grads:
    """Gradients of a scalar loss L through the whole layer, in float64.

    dY = dL/dY [T, d]; g_aux = dL/dL_aux.  The forward is recomputed here
    (route, statistics, capacity); ``topk_idx`` conditions it on another
    implementation's selection, as in ``forward``.
    """
    w = inp.w
    T, d, E, k, ffn = w.T, w.d, w.E, w.k, w.ffn
    r = route(inp.x, inp.w_router, inp.b_router, k, threads=threads, sel_bias=getattr(inp, "sel_bias", None))
    idx = r.topk_idx if topk_idx is None else np.ascontiguousarray(topk_idx, dtype=np.int32)
    wts = np.ascontiguousarray(np.take_along_axis(r.probs, idx.astype(np.int64).clip(0, E - 1), axis=1))
    st = load_stats(idx, r.probs, w.alpha)
    dp = capacity(idx, E, float(np.float32(w.capacity_factor)), w.expert_begin, w.num_local_experts)
    E_loc = w.E_loc
    sh = inp.ws1 is not None
    g = Grads(dx=np.empty((T, d)), dW_r=np.empty((E, d)), db_r=np.empty(E), dW1=np.empty((E_loc, ffn, d)),
              db1=np.empty((E_loc, ffn)), dW2=np.empty((E_loc, d, ffn)), db2=np.empty((E_loc, d)),
              dWs1=np.empty((ffn, d)) if sh else None, dbs1=np.empty(ffn) if sh else None,
              dWs2=np.empty((d, ffn)) if sh else None, dbs2=np.empty(d) if sh else None,
              dlogits=np.empty((T, E)))
    c = lambda a: None if a is None else np.ascontiguousarray(a)
    dY = np.ascontiguousarray(dY, dtype=np.float64)
    f = np.ascontiguousarray(st.f, dtype=np.float64)
    rc = _load().oracle_backward(
        _ptr(np.ascontiguousarray(inp.x)), _dtype_of(inp.x), T, d, E, k, ffn,
        _ptr(np.ascontiguousarray(inp.w_router, dtype=np.float32)), _ptr(r.probs), _ptr(idx), _ptr(wts),
        _ptr(dp.slot_row), _ptr(f), float(w.alpha), float(g_aux), w.expert_begin, E_loc,
        _ptr(c(inp.w1)), _ptr(c(inp.b1)), _ptr(c(inp.w2)), _ptr(c(inp.b2)),
        _ptr(c(inp.ws1)), _ptr(c(inp.bs1)), _ptr(c(inp.ws2)), _ptr(c(inp.bs2)), _ptr(dY),
        _ptr(g.dx), _ptr(g.dW_r), _ptr(g.db_r), _ptr(g.dW1), _ptr(g.db1), _ptr(g.dW2), _ptr(g.db2),
        _ptr(g.dWs1), _ptr(g.dbs1), _ptr(g.dWs2), _ptr(g.dbs2), _ptr(g.dlogits), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_backward: invalid sizes (%d)" % rc)
    return g


def backward_tokens(inp, dY: np.ndarray, tokens, g_aux: float = 0.0, threads: Optional[int] = None,
                    topk_idx: Optional[np.ndarray] = None):
    """dx [n, d] and dlogits [n, E] of the tokens ``tokens`` only, with the
    arithmetic of ``backward`` (no weight gradients).  dY is the full [T, d]
    gradient (only the listed rows are read)."""
    w = inp.w
    T, d, E, k, ffn = w.T, w.d, w.E, w.k, w.ffn
    r = route(inp.x, inp.w_router, inp.b_router, k, threads=threads, sel_bias=getattr(inp, "sel_bias", None))
    idx = r.topk_idx if topk_idx is None else np.ascontiguousarray(topk_idx, dtype=np.int32)
    wts = np.ascontiguousarray(np.take_along_axis(r.probs, idx.astype(np.int64).clip(0, E - 1), axis=1))
    st = load_stats(idx, r.probs, w.alpha)
    dp = capacity(idx, E, float(np.float32(w.capacity_factor)), w.expert_begin, w.num_local_experts)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    dx = np.empty((tok.size, d))
    dl = np.empty((tok.size, E))
    c = lambda a: None if a is None else np.ascontiguousarray(a)
    rc = _load().oracle_backward_tokens(
        _ptr(np.ascontiguousarray(inp.x)), _dtype_of(inp.x), T, d, E, k, ffn,
        _ptr(np.ascontiguousarray(inp.w_router, dtype=np.float32)), _ptr(r.probs), _ptr(idx), _ptr(wts),
        _ptr(dp.slot_row), _ptr(np.ascontiguousarray(st.f, dtype=np.float64)), float(w.alpha), float(g_aux),
        w.expert_begin, w.E_loc, _ptr(c(inp.w1)), _ptr(c(inp.b1)), _ptr(c(inp.w2)), _ptr(c(inp.b2)),
        _ptr(c(inp.ws1)), _ptr(c(inp.bs1)), _ptr(c(inp.ws2)), _ptr(c(inp.bs2)),
        _ptr(np.ascontiguousarray(dY, dtype=np.float64)), _ptr(tok), tok.size, _ptr(dx), _ptr(dl),
        _threads(threads))
    if rc != 0:
        raise ValueError("oracle_backward_tokens: invalid arguments (%d)" % rc)
    return dx, dl


@dataclass
class FfnColumns:
    dW1_rows: np.ndarray   # [nq, d]: rows qs of dW1
    db1: np.ndarray        # [nq]
    dW2_cols: np.ndarray   # [nq, d]: columns qs of dW2
    db2: np.ndarray        # [d]


def ffn_grad_columns(x: np.ndarray, w1: np.ndarray, b1, w2: np.ndarray, tokens, weights, dY: np.ndarray, qs,
                     threads: Optional[int] = None) -> FfnColumns:
    """Hidden features ``qs`` of one FFN's weight gradients (w1 [ffn, d],
    w2 [d, ffn]) over the rows (tokens[r], output weight weights[r]); see
    oracle_ffn_grad_columns."""
    T, d = x.shape
    ffn = w1.shape[0]
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    wt = np.ascontiguousarray(weights, dtype=np.float64)
    q = np.ascontiguousarray(qs, dtype=np.int32)
    out = FfnColumns(np.empty((q.size, d)), np.empty(q.size), np.empty((q.size, d)), np.empty(d))
    c = lambda a: None if a is None else np.ascontiguousarray(a)
    rc = _load().oracle_ffn_grad_columns(
        _ptr(np.ascontiguousarray(x)), _dtype_of(x), T, d, ffn, _ptr(c(w1)), _ptr(c(b1)), _ptr(c(w2)), _ptr(tok),
        _ptr(wt), tok.size, _ptr(np.ascontiguousarray(dY, dtype=np.float64)), _ptr(q), q.size, _ptr(out.dW1_rows),
        _ptr(out.db1), _ptr(out.dW2_cols), _ptr(out.db2), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_ffn_grad_columns: invalid arguments (%d)" % rc)
    return out
