"""Comparison helpers shared by the GPU parity tests (no GPU work here).

Contract (GPU path vs the fp64 oracle):
  - integers (expert ids, counts, capacity, permutation, drop sets) are
    bit-exact; tokens whose top-k choice is a near tie (fp64 logit gap below
    1e-5, where fp32 rounding may legitimately flip the order) are excluded
    from the exact id check, counted, and checked for validity instead;
  - later stages are conditioned on the GPU's own selection, so a flipped
    near tie cannot cascade;
  - router floats (routing weights, P, L_aux): max|gpu - ref| / max|ref| <= 1e-4;
  - Y: max|gpu - ref| / max|ref| <= 2e-2 for bf16 layers, <= 1e-4 for fp32.
"""
from __future__ import annotations

import numpy as np

NEAR_TIE = 1e-5
TOL_ROUTER = 1e-4
TOL_Y_BF16 = 2e-2
TOL_Y_F32 = 1e-4


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def near_ties(logits: np.ndarray, k: int):
    """(boundary, order) boolean masks over tokens."""
    T, E = logits.shape
    s = -np.sort(-logits, axis=1)
    boundary = np.zeros(T, bool)
    if E > k:
        boundary = (s[:, k - 1] - s[:, k]) < NEAR_TIE
    order = np.zeros(T, bool)
    for j in range(k - 1):
        order |= (s[:, j] - s[:, j + 1]) < NEAR_TIE
    return boundary, order


def check_topk(gpu_idx: np.ndarray, logits: np.ndarray, ref_idx: np.ndarray, k: int) -> dict:
    """Exact ids off near ties; a valid selection on near ties."""
    T, E = logits.shape
    assert gpu_idx.shape == (T, k)
    assert ((gpu_idx >= 0) & (gpu_idx < E)).all(), "expert id out of range"
    srt = np.sort(gpu_idx, axis=1)
    assert (np.diff(srt, axis=1) > 0).all() if k > 1 else True, "repeated expert within a token"
    boundary, order = near_ties(logits, k)
    plain = ~(boundary | order)
    bad = np.flatnonzero(plain & (gpu_idx != ref_idx).any(axis=1))
    assert bad.size == 0, "top-k mismatch at tokens %s" % bad[:10]
    # order near ties (not at the boundary): same set
    o = np.flatnonzero(order & ~boundary)
    assert (np.sort(gpu_idx[o], 1) == np.sort(ref_idx[o], 1)).all(), "set mismatch on an order near tie"
    # boundary near ties: every selected logit >= every unselected - eps
    for t in np.flatnonzero(boundary):
        sel = logits[t, gpu_idx[t]]
        mask = np.ones(E, bool)
        mask[gpu_idx[t]] = False
        assert sel.min() >= logits[t, mask].max() - NEAR_TIE, "invalid selection at near tie %d" % t
    return dict(boundary=int(boundary.sum()), order=int((order & ~boundary).sum()))


def expected_xperm(x_host: np.ndarray, row_src: np.ndarray, k: int) -> np.ndarray:
    return x_host[row_src // k]
