"""Seeded synthetic MoE-layer workloads.

This module only describes workload shapes and draws random inputs; it holds
none of the layer's arithmetic.  Both the HIP path and the CPU oracle are fed
from it, so the same bytes reach both sides.

Shapes follow the workloads the pages speak of (Mixtral 8x7B with 8 experts,
top-2, d=4096 in "Expert Parallelism (MoE)", section "MoE Layer Structure";
DeepSeek-V3 with 256 routed experts, top-8 and a shared expert in the same
page's "Production MoE Models" list and in "Expert Parallelism (EP)", section
"Key math / How it works").  Trained weights and real activations are not
available, so seeded Gaussian layers stand in for them.

Recipe (fixed): numpy PCG64 streams derived from ``SeedSequence(seed)``; one
child stream per tensor slot (x, router weight, W1 of each global expert, W2 of
each global expert, shared W1, shared W2, then bias slots), each tensor drawn in
row chunks that get their own grandchild stream so that generation can run on
several threads and still be bit-reproducible.  Values are drawn as float32
N(0,1), scaled by the stated standard deviation in float32, then rounded to
bfloat16 with round-to-nearest-even where the workload is bf16.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens in the batch
    d: int                 # hidden size
    E: int                 # experts scored by the router
    k: int                 # experts selected per token
    ffn: int               # expert inner size
    dtype: str             # activations / expert weights: "f32" or "bf16"
    capacity_factor: float = 0.0   # <= 0: no capacity cap
    expert_begin: int = 0          # first local expert
    num_local_experts: int = 0     # 0 -> all E experts are local
    shared_expert: bool = False    # one non-routed expert run on every token
    router_bias: str = "zero"      # "zero" | "zipf" (b_i = 2 ln(1/(i+1))) | "gauss"
    expert_bias: str = "zero"      # "zero" | "gauss"
    sel_bias: str = "none"         # "none" | "gauss": selection-only router bias, N(0, 0.3^2)
    alpha: float = 0.01

    @property
    def E_loc(self) -> int:
        return self.num_local_experts if self.num_local_experts > 0 else self.E


# The five workloads.  Index 1 (Mixtral-8x7B-shaped) is the headline one.
WORKLOADS = [
    Workload("tiny-fp32", T=256, d=64, E=8, k=2, ffn=256, dtype=F32),
    Workload("mixtral8x7b-layer", T=4096, d=4096, E=8, k=2, ffn=16384, dtype=BF16),
    Workload("capacity-drop-zipf", T=8192, d=2048, E=64, k=2, ffn=8192, dtype=BF16,
             capacity_factor=1.25, router_bias="zipf"),
    Workload("fine-grained-e128-k8", T=16384, d=2048, E=128, k=8, ffn=768, dtype=BF16),
    Workload("deepseekv3-share-32of256", T=32768, d=7168, E=256, k=8, ffn=2048, dtype=BF16,
             expert_begin=0, num_local_experts=32, shared_expert=True),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def get(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    return BY_NAME[name_or_index]


def scaled(w: Workload, **changes) -> Workload:
    """Same workload with some fields replaced (used for small parity cases)."""
    return replace(w, **changes)


# --------------------------------------------------------------------------
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Generation
# --------------------------------------------------------------------------

_CHUNK_ELEMS = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_gaussian(out_rows: np.ndarray, seq: np.random.SeedSequence, std: float,
                   to_bf16: bool, jobs: list):
    """Queue the jobs that fill a 2-D array [rows, cols] with N(0, std^2)."""
    rows, cols = out_rows.shape
    chunk_rows = max(1, _CHUNK_ELEMS // max(1, cols))
    nchunks = (rows + chunk_rows - 1) // chunk_rows
    subs = seq.spawn(nchunks)
    for c in range(nchunks):
        r0 = c * chunk_rows
        r1 = min(rows, r0 + chunk_rows)

        def job(r0=r0, r1=r1, s=subs[c]):
            g = np.random.Generator(np.random.PCG64(s))
            v = g.standard_normal((r1 - r0, cols), dtype=np.float32)
            if std != 1.0:
                v *= np.float32(std)
            if to_bf16:
                out_rows[r0:r1] = f32_to_bf16_bits(v)
            else:
                out_rows[r0:r1] = v
        jobs.append(job)


@dataclass
class LayerInputs:
    """Host arrays for one MoE layer.  bf16 tensors are uint16 bit patterns."""
    w: Workload
    x: np.ndarray                    # [T, d]
    w_router: np.ndarray             # [E, d] float32
    b_router: Optional[np.ndarray]   # [E] float32 or None
    w1: np.ndarray                   # [E_loc, ffn, d]
    b1: Optional[np.ndarray]         # [E_loc, ffn]
    w2: np.ndarray                   # [E_loc, d, ffn]
    b2: Optional[np.ndarray]         # [E_loc, d]
    ws1: Optional[np.ndarray] = None  # [ffn, d] shared expert
    bs1: Optional[np.ndarray] = None
    ws2: Optional[np.ndarray] = None  # [d, ffn]
    bs2: Optional[np.ndarray] = None
    sel_bias: Optional[np.ndarray] = None  # [E] float32: selection-only router bias
    extra: dict = field(default_factory=dict)


def make_layer(w: Workload, seed: int = 0, threads: Optional[int] = None,
               with_experts: bool = True) -> LayerInputs:
    """Draw the seeded inputs of workload ``w``.

    ``with_experts=False`` skips the expert weights (router-only tests).
    """
    bf = w.dtype == BF16
    act_dt = np.uint16 if bf else np.float32
    E, E_loc, e0 = w.E, w.E_loc, w.expert_begin
    root = np.random.SeedSequence(seed)
    # slots: 0 x, 1 router W, 2..2+E W1[e], 2+E..2+2E W2[e], 2+2E shared W1,
    # 3+2E shared W2, 4+2E router bias, 5+2E b1, 6+2E b2, 7+2E shared biases,
    # 8+2E selection bias
    slots = root.spawn(9 + 2 * E)
    jobs: list = []

    x = np.empty((w.T, w.d), dtype=act_dt)
    _fill_gaussian(x, slots[0], 1.0, bf, jobs)
    w_router = np.empty((E, w.d), dtype=np.float32)
    _fill_gaussian(w_router, slots[1], 1.0 / math.sqrt(w.d), False, jobs)

    if with_experts:
        w1 = np.empty((E_loc, w.ffn, w.d), dtype=act_dt)
        w2 = np.empty((E_loc, w.d, w.ffn), dtype=act_dt)
        for le in range(E_loc):
            ge = e0 + le
            _fill_gaussian(w1[le], slots[2 + ge], 1.0 / math.sqrt(w.d), bf, jobs)
            _fill_gaussian(w2[le], slots[2 + E + ge], 1.0 / math.sqrt(w.ffn), bf, jobs)
    else:
        w1 = np.empty((E_loc, 0, w.d), dtype=act_dt)
        w2 = np.empty((E_loc, w.d, 0), dtype=act_dt)

    ws1 = ws2 = None
    if w.shared_expert and with_experts:
        ws1 = np.empty((w.ffn, w.d), dtype=act_dt)
        ws2 = np.empty((w.d, w.ffn), dtype=act_dt)
        _fill_gaussian(ws1, slots[2 + 2 * E], 1.0 / math.sqrt(w.d), bf, jobs)
        _fill_gaussian(ws2, slots[3 + 2 * E], 1.0 / math.sqrt(w.ffn), bf, jobs)

    nthr = threads or _threads()
    if nthr > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(lambda j: j(), jobs))
    else:
        for j in jobs:
            j()

    # router bias
    if w.router_bias == "zero":
        b_router = None
    elif w.router_bias == "zipf":
        b_router = (2.0 * np.log(1.0 / (np.arange(E, dtype=np.float64) + 1.0))).astype(np.float32)
    elif w.router_bias == "gauss":
        g = np.random.Generator(np.random.PCG64(slots[4 + 2 * E]))
        b_router = g.standard_normal(E, dtype=np.float32) * np.float32(0.5)
    else:
        raise ValueError(w.router_bias)

    b1 = b2 = bs1 = bs2 = None
    if w.expert_bias == "gauss" and with_experts:
        g1 = np.random.Generator(np.random.PCG64(slots[5 + 2 * E]))
        g2 = np.random.Generator(np.random.PCG64(slots[6 + 2 * E]))
        b1f = g1.standard_normal((E, w.ffn), dtype=np.float32)[e0:e0 + E_loc] * np.float32(0.1)
        b2f = g2.standard_normal((E, w.d), dtype=np.float32)[e0:e0 + E_loc] * np.float32(0.1)
        b1 = f32_to_bf16_bits(b1f) if bf else np.ascontiguousarray(b1f)
        b2 = f32_to_bf16_bits(b2f) if bf else np.ascontiguousarray(b2f)
        if w.shared_expert:
            g3 = np.random.Generator(np.random.PCG64(slots[7 + 2 * E]))
            s1 = g3.standard_normal(w.ffn, dtype=np.float32) * np.float32(0.1)
            s2 = g3.standard_normal(w.d, dtype=np.float32) * np.float32(0.1)
            bs1 = f32_to_bf16_bits(s1) if bf else s1
            bs2 = f32_to_bf16_bits(s2) if bf else s2

    if w.sel_bias == "none":
        sel_bias = None
    elif w.sel_bias == "gauss":
        g = np.random.Generator(np.random.PCG64(slots[8 + 2 * E]))
        sel_bias = g.standard_normal(E, dtype=np.float32) * np.float32(0.3)
    else:
        raise ValueError(w.sel_bias)

    return LayerInputs(w, x, w_router, b_router, w1, b1, w2, b2, ws1, bs1, ws2, bs2, sel_bias)


def make_grad_output(w: Workload, seed: int = 0, threads: Optional[int] = None) -> np.ndarray:
    """Seeded dL/dY [T, d] ~ N(0, 1) for the backward pass, in the layer's
    storage dtype (uint16 bf16 bits or float32); drawn from its own seed
    stream, so the layer's inputs do not depend on it."""
    bf = w.dtype == BF16
    dy = np.empty((w.T, w.d), dtype=np.uint16 if bf else np.float32)
    jobs: list = []
    _fill_gaussian(dy, np.random.SeedSequence([seed, 0x6772]), 1.0, bf, jobs)
    n = threads or _threads()
    if n > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(lambda j: j(), jobs))
    else:
        for j in jobs:
            j()
    return dy


def token_sample(T: int, n: int, seed: int = 1234, must_include=()) -> np.ndarray:
    """Sorted seeded sample of ``n`` distinct token ids (plus ``must_include``)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, T, n])))
    n = min(n, T)
    pick = g.choice(T, size=n, replace=False)
    pick = np.union1d(pick, np.asarray(list(must_include), dtype=np.int64))
    return np.sort(pick.astype(np.int64))


def to_torch(a: Optional[np.ndarray], device=None):
    """Host array -> torch tensor (uint16 bit patterns become bfloat16)."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device) if device is not None else t


def device_layer(inp: LayerInputs, device="cuda") -> dict:
    """Every tensor of a layer copied to ``device`` (names as in LayerInputs)."""
    names = ("x", "w_router", "b_router", "w1", "b1", "w2", "b2", "ws1", "bs1", "ws2", "bs2", "sel_bias")
    return {n: to_torch(getattr(inp, n), device) for n in names}
