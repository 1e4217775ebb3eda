"""Seeded random layer shapes against the oracle.

Beyond the hand-picked cases: layers drawn from a fixed seed across the
supported size space (E from 1 to 1024 including non-powers of two and values
on both sides of the router's path switches, k up to 32, d and ffn any
multiple of 8, capacity caps, local shares, a shared expert, expert biases,
router biases, selection-only biases, bf16 and fp32).  Every case runs the
forward parity check of the hand-picked cases (integer outputs exact,
routing weights and statistics within the router tolerance, Y within the
layer's tolerance); the cases the backward supports also run its parity
check on every gradient element.
"""
import numpy as np
import pytest

import oracle
from parity import TOL_ROUTER, TOL_Y_BF16, TOL_Y_F32, rel_err
from test_gpu_backward import EXPERT_GRADS, ROUTER_GRADS, SHARED_GRADS, _dy64, _run
from test_gpu_parity import _check_forward, _inputs
from top_routing_expert_route_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _draw(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = wl.BF16 if rng.random() < 0.75 else wl.F32
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 31, 32, 33, 64, 65, 96, 128, 200, 256, 512, 1024]))
        k = int(rng.integers(1, min(E, 32 if rng.random() < 0.15 else 8) + 1))
        if dtype == wl.BF16 and rng.random() < 0.5:
            d = 64 * int(rng.integers(1, 6))
            ffn = 64 * int(rng.integers(1, 7))
        else:
            d = 8 * int(rng.integers(1, 41))
            ffn = 8 * int(rng.integers(1, 49))
        T = int(rng.integers(0, 700))
        cap = float(rng.choice([0.0, 0.0, 0.5, 1.0, 1.25, 2.0]))
        nle = 0
        e0 = 0
        if E > 1 and rng.random() < 0.3:
            nle = int(rng.integers(1, E + 1))
            e0 = int(rng.integers(0, E - nle + 1))
        cases.append(wl.Workload(
            "rand%02d" % i, T=T, d=d, E=E, k=k, ffn=ffn, dtype=dtype, capacity_factor=cap, expert_begin=e0,
            num_local_experts=nle, shared_expert=bool(rng.random() < 0.25),
            router_bias=str(rng.choice(["zero", "gauss"])), expert_bias=str(rng.choice(["zero", "gauss"])),
            sel_bias=str(rng.choice(["none", "none", "gauss"]))))
    return cases


CASES = {w.name: w for w in _draw()}


def _backward_supported(w):
    return w.T > 0 and (w.dtype == wl.F32 or (w.d % 64 == 0 and w.ffn % 64 == 0 and w.d >= 128 and w.ffn >= 128))


@pytest.mark.parametrize("name", list(CASES))
def test_random_shape(name):
    w = CASES[name]
    print("random case", w, flush=True)
    inp, t = _inputs(w, seed=11)
    _check_forward(w, inp, t)
    if not _backward_supported(w):
        return
    g_aux = 0.3
    inp, t, dy, dy_host, layer, outs, grads = _run(w, seed=11, g_aux=g_aux)
    ref = oracle.backward(inp, _dy64(w, dy_host), g_aux=g_aux, topk_idx=outs["topk_idx"].cpu().numpy())
    tol = TOL_Y_BF16 if w.dtype == wl.BF16 else TOL_Y_F32
    for gname, rname in EXPERT_GRADS + (SHARED_GRADS if w.shared_expert else ()):
        err = rel_err(grads[gname].cpu().numpy(), getattr(ref, rname))
        assert err <= tol, (gname, err)
    for gname, rname in ROUTER_GRADS:
        err = rel_err(grads[gname].cpu().numpy(), getattr(ref, rname))
        assert err <= TOL_ROUTER, (gname, err)


def _draw_large(n=8, seed=1001):
    """Larger layers (multi-round GEMMs, split-K tails, the large dispatch
    planner, many route blocks), checked on a token sample of at least 512
    tokens holding every near tie and one token of every 256-row tile."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = wl.BF16 if rng.random() < 0.85 else wl.F32
        E = int(rng.choice([8, 16, 60, 64, 72, 128, 256, 512]))
        k = int(rng.integers(1, min(E, 8) + 1))
        mult = 64 if rng.random() < 0.7 else 8
        d = mult * int(rng.integers(max(1, 256 // mult), 2048 // mult + 1))
        ffn = mult * int(rng.integers(max(1, 128 // mult), 4096 // mult + 1))
        T = int(rng.integers(2000, 40000))
        if dtype == wl.F32:
            d, ffn, T = min(d, 512), min(ffn, 512), min(T, 4000)
        cap = float(rng.choice([0.0, 0.0, 1.0, 1.25]))
        nle = 0
        e0 = 0
        if rng.random() < 0.3:
            nle = int(rng.integers(1, E + 1))
            e0 = int(rng.integers(0, E - nle + 1))
        cases.append(wl.Workload(
            "large%02d" % i, T=T, d=d, E=E, k=k, ffn=ffn, dtype=dtype, capacity_factor=cap, expert_begin=e0,
            num_local_experts=nle, shared_expert=bool(rng.random() < 0.2),
            router_bias=str(rng.choice(["zero", "gauss", "zipf"])), expert_bias=str(rng.choice(["zero", "gauss"])),
            sel_bias=str(rng.choice(["none", "gauss"]))))
    return cases


LARGE = {w.name: w for w in _draw_large()}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(LARGE))
def test_random_large_shape(name):
    w = LARGE[name]
    print("random large case", w, flush=True)
    inp, t = _inputs(w, seed=3)
    _check_forward(w, inp, t, tokens=512)
