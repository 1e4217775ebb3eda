"""Algorithmic work of each step of the layer: the bytes a step must move and
the flops it must do, computed from the counts of an actual run.

Conditional computation ("Expert Parallelism (MoE)", sections "MoE Layer
Structure" and "Common Pitfalls"): a token touches only the k experts it
selects, so expert work scales with k (and with the rows actually kept), not
with E.  Nothing here counts the dense E-expert work that the method avoids.
"""
from __future__ import annotations

from dataclasses import dataclass

# MI355X published peaks.
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


def elem_bytes(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


def active_param_fraction(E: int, k: int) -> float:
    """Fraction of the routed-expert parameters one token uses."""
    return k / E


def expert_flops_per_token(d: int, ffn: int, k: int) -> int:
    """Two Linear layers per selected expert: 2*d*ffn flops each."""
    return k * 4 * d * ffn


@dataclass
class RunCounts:
    T: int
    d: int
    E: int
    k: int
    ffn: int
    dtype: str
    rows: int                 # kept local (token, slot) selections
    active_experts: int       # local experts with at least one row
    tokens_with_rows: int     # tokens with at least one kept local selection
    shared: bool = False
    has_router_bias: bool = False
    has_expert_bias: bool = False


def route_bytes(c: RunCounts) -> int:
    s = elem_bytes(c.dtype)
    b = c.T * c.d * s + c.E * c.d * 4 + c.T * c.k * (4 + 4)
    if c.has_router_bias:
        b += c.E * 4
    return b


def route_flops(c: RunCounts) -> int:
    return 2 * c.T * c.d * c.E


def dispatch_bytes(c: RunCounts) -> int:
    """Read each token with a kept local selection once, write its rows, plus
    the index arrays (topk_idx read, slot_row written, row_src written)."""
    s = elem_bytes(c.dtype)
    return c.tokens_with_rows * c.d * s + c.rows * c.d * s + c.T * c.k * 4 * 2 + c.rows * 4


def gemm1_flops(c: RunCounts) -> int:
    return 2 * c.rows * c.d * c.ffn


def gemm2_flops(c: RunCounts) -> int:
    return 2 * c.rows * c.ffn * c.d


def gemm_weight_bytes(c: RunCounts) -> int:
    s = elem_bytes(c.dtype)
    return c.active_experts * 2 * c.d * c.ffn * s


def gemm1_bytes(c: RunCounts) -> int:
    s = elem_bytes(c.dtype)
    return c.active_experts * c.d * c.ffn * s + c.rows * c.d * s + c.rows * c.ffn * s


def gemm2_bytes(c: RunCounts) -> int:
    s = elem_bytes(c.dtype)
    return c.active_experts * c.d * c.ffn * s + c.rows * c.ffn * s + c.rows * c.d * s


def shared_flops(c: RunCounts) -> int:
    return 4 * c.T * c.d * c.ffn if c.shared else 0


def combine_bytes(c: RunCounts) -> int:
    s = elem_bytes(c.dtype)
    b = c.rows * c.d * s + c.T * c.d * s + c.T * c.k * (4 + 4)
    if c.shared:
        b += c.T * c.d * s
    return b


def backward_gemm_flops(c: RunCounts) -> int:
    """Matrix-core work of one moe_backward: per FFN (routed rows, and the
    shared expert over all tokens) five GEMMs of 2 * rows * d * ffn: the
    recomputed first Linear, dh' = W2^T dY, dx = W1^T du, dW2 and dW1."""
    f = 5 * 2 * c.rows * c.d * c.ffn
    if c.shared:
        f += 5 * 2 * c.T * c.d * c.ffn
    return f


def backward_router_flops(c: RunCounts) -> int:
    """fp32 vector work of the router backward: dW_r = dl^T x and the dx term
    dl W_r, 2 * T * E * d each (the router forward recompute is route_flops)."""
    return 2 * 2 * c.T * c.E * c.d
