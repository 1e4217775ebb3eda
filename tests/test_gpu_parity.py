"""GPU parity: every step of the HIP path against the fp64 oracle, called
through the C ABI, on seeded workloads shaped like the pages' layers.

Small cases span several tiles and ragged tails and are compared on every
element.  The full-size workloads run in the launch configuration the
benchmark times; they compare every integer output on every token, and Y on
every token of the Mixtral-shaped and capacity-drop layers, and on a seeded
sample of at least 512 tokens of the fine-grained and DeepSeek-shaped layers
that also holds every near-tie token and one token of every 256-row tile of
every expert segment (and of the shared expert, which covers all tokens).
"""
import numpy as np
import pytest
import torch

import oracle
from parity import (TOL_ROUTER, TOL_Y_BF16, TOL_Y_F32, check_topk, expected_xperm, near_ties, rel_err)
from top_routing_expert_route_amd import api
from top_routing_expert_route_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"

SMALL = {
    "tiny-fp32": wl.get(0),
    "mixtral-small": wl.scaled(wl.get(1), name="mixtral-small", T=333, d=256, ffn=384),
    "drop-small": wl.scaled(wl.get(2), name="drop-small", T=1000, d=192, ffn=256),
    "fine-small": wl.scaled(wl.get(3), name="fine-small", T=700, d=128, ffn=96),
    "dsv3-small": wl.scaled(wl.get(4), name="dsv3-small", T=500, d=136, ffn=264, expert_begin=32,
                            expert_bias="gauss"),
    "bias-f32": wl.scaled(wl.get(0), name="bias-f32", T=301, d=72, ffn=136, router_bias="gauss",
                          expert_bias="gauss", capacity_factor=1.1),
    # selection-only router bias: the fused small-E router and the E > 64 path
    "selbias-e32": wl.scaled(wl.get(1), name="selbias-e32", T=400, d=192, E=32, k=4, ffn=128,
                             sel_bias="gauss", router_bias="gauss"),
    "selbias-e128": wl.scaled(wl.get(3), name="selbias-e128", T=300, d=128, ffn=96, sel_bias="gauss",
                              capacity_factor=1.5),
    # E > 64 with d = 64: too short a reduction for the router's grouped-GEMM path
    "e128-d64": wl.scaled(wl.get(3), name="e128-d64", T=300, d=64, ffn=96),
    # E > 64 not a multiple of 8 (3E logits per row not in whole 16-byte groups), k = 16
    "e65-k16": wl.scaled(wl.get(3), name="e65-k16", T=325, d=192, E=65, k=16, ffn=128, router_bias="gauss"),
}

FULL = {w.name: w for w in wl.WORKLOADS[1:]}
# Y on every token (None) or on a seeded sample of this many tokens, plus
# every near tie and one token per 256-row tile (see _sample_tokens)
FULL_SAMPLE = {"mixtral8x7b-layer": None, "capacity-drop-zipf": None, "fine-grained-e128-k8": 768,
               "deepseekv3-share-32of256": 640}
TILE = 256  # row tile edge of the grouped GEMM


def _sample_tokens(w, n, scores, seg_offsets, row_src, seed=17):
    """At least n tokens: a seeded sample, every near-tie token, and for every
    256-row tile of every local segment the token of one (seeded) row of it,
    plus each segment's first and last row; with a shared expert (one segment
    of all T tokens in order) one token of every 256-token tile as well."""
    b, o = near_ties(scores, w.k)
    must = [np.flatnonzero(b | o)]
    g = np.random.default_rng([seed, w.T])
    rows = []
    for s in range(len(seg_offsets) - 1):
        lo, hi = int(seg_offsets[s]), int(seg_offsets[s + 1])
        if hi <= lo:
            continue
        rows += [lo, hi - 1]
        for r0 in range(lo, hi, TILE):
            rows.append(int(g.integers(r0, min(r0 + TILE, hi))))
    if rows:
        must.append(np.asarray(row_src)[np.asarray(rows)] // w.k)
    if w.shared_expert:
        must.append(np.array([int(g.integers(t0, min(t0 + TILE, w.T))) for t0 in range(0, w.T, TILE)]))
    return wl.token_sample(w.T, n, must_include=np.concatenate(must).astype(np.int64))

_cache = {}


def _inputs(w, seed=0):
    key = (w, seed)
    if key not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        inp = wl.make_layer(w, seed=seed)
        _cache[key] = (inp, wl.device_layer(inp, DEV))
    return _cache[key]


def _torch_dtype(w):
    return torch.bfloat16 if w.dtype == wl.BF16 else torch.float32


def _ytol(w):
    return TOL_Y_BF16 if w.dtype == wl.BF16 else TOL_Y_F32


def _host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def _x_f64(inp):
    return wl.bf16_bits_to_f32(inp.x) if inp.x.dtype == np.uint16 else inp.x


def _run_stages(w, inp, t):
    """Route, dispatch, expert FFN and combine called one by one."""
    r = api.moe_route(t["x"], t["w_router"], t["b_router"], w.k, w.alpha, sel_bias=t["sel_bias"])
    dp = api.moe_dispatch(t["x"], r["topk_idx"], w.E, w.capacity_factor, w.expert_begin, w.num_local_experts)
    h, y_perm = api.moe_expert_ffn(dp["x_perm"], dp["seg_offsets"], t["w1"], t["b1"], t["w2"], t["b2"])
    y_sh = None
    if w.shared_expert:
        hs = api.moe_grouped_gemm(t["x"], None, t["ws1"].unsqueeze(0), None if t["bs1"] is None else t["bs1"].unsqueeze(0), 1)
        y_sh = api.moe_grouped_gemm(hs, None, t["ws2"].unsqueeze(0), None if t["bs2"] is None else t["bs2"].unsqueeze(0), 0)
    y = api.moe_combine(y_perm, dp["slot_row"], r["topk_w"], y_sh)
    torch.cuda.synchronize()
    return r, dp, y_perm, y_sh, y


def _check_route(w, inp, r, ref_route):
    gidx = r["topk_idx"].cpu().numpy()
    nt = check_topk(gidx, ref_route.scores, ref_route.topk_idx, w.k)
    # routing weight = oracle probability at the GPU's selection
    ref_w = np.take_along_axis(ref_route.probs, gidx.astype(np.int64), 1)
    assert rel_err(r["topk_w"].cpu().numpy(), ref_w) <= TOL_ROUTER
    st = oracle.load_stats(gidx, ref_route.probs, w.alpha)
    cnt = r["expert_count"].cpu().numpy()
    np.testing.assert_array_equal(cnt, st.count)
    # f = fp32(count / T); with no tokens the statistics are zero
    f_ref = np.float32(cnt) / np.float32(w.T) if w.T > 0 else np.zeros(len(cnt), np.float32)
    np.testing.assert_array_equal(r["f"].cpu().numpy(), f_ref)
    assert rel_err(r["P"].cpu().numpy(), st.P) <= TOL_ROUTER
    assert rel_err(r["l_aux"].cpu().numpy(), [st.l_aux]) <= TOL_ROUTER
    own = oracle.load_stats(ref_route.topk_idx, ref_route.probs, w.alpha)
    assert np.abs(own.count - st.count).sum() <= 2 * nt["boundary"]
    return gidx, nt


def _check_dispatch(w, inp, gidx, dp):
    ref = oracle.capacity(gidx, w.E, np.float32(w.capacity_factor), w.expert_begin, w.num_local_experts)
    np.testing.assert_array_equal(dp["seg_offsets"].cpu().numpy(), ref.seg_offsets)
    np.testing.assert_array_equal(dp["kept_count"].cpu().numpy(), ref.kept_count)
    np.testing.assert_array_equal(dp["slot_row"].cpu().numpy(), ref.slot_row)
    rows = int(ref.seg_offsets[-1])
    np.testing.assert_array_equal(dp["row_src"].cpu().numpy()[:rows], ref.row_src)
    assert int(dp["n_dropped"].item()) == ref.n_dropped
    xp = dp["x_perm"][:rows]
    if xp.dtype == torch.bfloat16:
        got = xp.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got = xp.cpu().numpy()
    np.testing.assert_array_equal(got, expected_xperm(inp.x, ref.row_src, w.k))
    return ref


def _oracle_rows(w, inp, gidx, row_src, rows_sel):
    """Expert output (no routing weight) of each selected dispatched row."""
    k = w.k
    out = np.zeros((len(rows_sel), w.d))
    toks = row_src[rows_sel] // k
    slots = row_src[rows_sel] % k
    for j in range(k):
        sel = np.flatnonzero(slots == j)
        if sel.size == 0:
            continue
        tj = toks[sel]
        sr = np.full((w.T, k), -1, np.int32)
        sr[tj, j] = 0
        wts = np.ones((w.T, k))
        y = oracle.combine(inp.x, tj, gidx, wts, sr, inp.w1, inp.b1, inp.w2, inp.b2, w.expert_begin)
        out[sel] = y
    return out


@pytest.mark.parametrize("name", list(SMALL))
def test_stages_small(name):
    w = SMALL[name]
    inp, t = _inputs(w)
    r, dp, y_perm, y_sh, y = _run_stages(w, inp, t)
    ref_route = oracle.route(inp.x, inp.w_router, inp.b_router, w.k, sel_bias=inp.sel_bias)
    gidx, nt = _check_route(w, inp, r, ref_route)
    ref_dp = _check_dispatch(w, inp, gidx, dp)
    rows = int(ref_dp.seg_offsets[-1])
    if rows:
        ref_rows = _oracle_rows(w, inp, gidx, ref_dp.row_src, np.arange(rows))
        assert rel_err(_host(y_perm[:rows]), ref_rows) <= _ytol(w)
    # combine on the GPU's own expert outputs, reference in float64 (rows past
    # the kept count are never read by the combine and are not initialised)
    yp = _host(y_perm[:rows]).astype(np.float64)
    sr = dp["slot_row"].cpu().numpy()
    tw = r["topk_w"].cpu().numpy().astype(np.float64)
    yc = np.zeros((w.T, w.d))
    for j in range(w.k):
        ok = sr[:, j] >= 0
        yc[ok] += tw[ok, j:j + 1] * yp[sr[ok, j]]
    if y_sh is not None:
        yc += _host(y_sh)
    assert rel_err(_host(y), yc) <= (1e-2 if w.dtype == wl.BF16 else 1e-6)
    # whole layer against the oracle, conditioned on the GPU's selection
    ref = oracle.forward(inp, topk_idx=gidx)
    assert rel_err(_host(y), ref.y) <= _ytol(w)


def _layer(w, t, **kw):
    return api.Layer(w.T, w.d, w.E, w.k, w.ffn, _torch_dtype(w), w.capacity_factor, w.expert_begin,
                     w.num_local_experts, w.alpha, t["w_router"], t["b_router"], t["w1"], t["b1"], t["w2"],
                     t["b2"], t["ws1"], t["bs1"], t["ws2"], t["bs2"], device=DEV, sel_bias=t["sel_bias"], **kw)


def _check_forward(w, inp, t, tokens=None):
    layer = _layer(w, t)
    outs = layer.alloc_outputs()
    y = layer.forward(t["x"])
    torch.cuda.synchronize()
    ref_route = oracle.route(inp.x, inp.w_router, inp.b_router, w.k, sel_bias=inp.sel_bias)
    gidx, nt = _check_route(w, inp, outs, ref_route)
    ref_dp = oracle.capacity(gidx, w.E, np.float32(w.capacity_factor), w.expert_begin, w.num_local_experts)
    np.testing.assert_array_equal(outs["slot_row"].cpu().numpy(), ref_dp.slot_row)
    np.testing.assert_array_equal(outs["seg_offsets"].cpu().numpy(), ref_dp.seg_offsets)
    rows = int(ref_dp.seg_offsets[-1])
    np.testing.assert_array_equal(outs["row_src"].cpu().numpy()[:rows], ref_dp.row_src)
    assert int(outs["n_dropped"].item()) == ref_dp.n_dropped
    if tokens is not None:
        tokens = _sample_tokens(w, tokens, ref_route.scores, ref_dp.seg_offsets, ref_dp.row_src)
    ref = oracle.forward(inp, tokens=tokens, topk_idx=gidx)
    yh = _host(y)
    yg = yh if tokens is None else yh[tokens]
    err = rel_err(yg, ref.y)
    assert err <= _ytol(w), err
    ntok = w.T if tokens is None else len(tokens)
    return layer, y, outs, nt, err, ntok


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    w = SMALL[name]
    inp, t = _inputs(w)
    _check_forward(w, inp, t)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(FULL))
def test_forward_full_size(name):
    import time
    w = FULL[name]
    t0 = time.perf_counter()
    inp, t = _inputs(w)
    layer, y, outs, nt, err, ntok = _check_forward(w, inp, t, tokens=FULL_SAMPLE[name])
    print("%s: near ties boundary %d order %d, Y rel err %.3e on %d of %d tokens (%.1f s)"
          % (name, nt["boundary"], nt["order"], err, ntok, w.T, time.perf_counter() - t0), flush=True)
    # bitwise reproducible
    y2 = layer.forward(t["x"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_forward_is_deterministic_small():
    w = SMALL["drop-small"]
    inp, t = _inputs(w)
    layer = _layer(w, t)
    layer.alloc_outputs()
    y1 = layer.forward(t["x"]).clone()
    o1 = {k: v.clone() for k, v in layer.outputs.items()}
    y2 = layer.forward(t["x"])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    for k in o1:
        assert torch.equal(o1[k], layer.outputs[k]), k


@pytest.mark.parametrize("name", ["dsv3-small", "mixtral-small", "deepseekv3-share-32of256"])
def test_forward_overlap_matches_forward(name):
    """moe_forward_overlap (shared expert on a second stream) gives the same
    bits as moe_forward, on two calls in a row (workspace reuse)."""
    w = SMALL[name] if name in SMALL else FULL[name]
    inp, t = _inputs(w)
    ref_layer = _layer(w, t)
    ref_layer.alloc_outputs()
    y_ref = ref_layer.forward(t["x"]).clone()
    layer = _layer(w, t)
    layer.alloc_outputs()
    side = torch.cuda.Stream(device=DEV)
    for _ in range(2):
        y = layer.forward(t["x"], side_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32),
                           y_ref.view(torch.int16) if y_ref.dtype == torch.bfloat16 else y_ref.view(torch.int32))
        rows = int(ref_layer.outputs["seg_offsets"][-1].item())
        for k in ref_layer.outputs:
            a, b = layer.outputs[k], ref_layer.outputs[k]
            if k == "row_src":  # defined for the first `rows` entries only
                a, b = a[:rows], b[:rows]
            assert torch.equal(a, b), k
    if w.shared_expert and name in SMALL:
        ref = oracle.forward(inp, topk_idx=ref_layer.outputs["topk_idx"].cpu().numpy())
        assert rel_err(_host(y), ref.y) <= _ytol(w)


# ------------------------------------------------------------ edge cases --

def test_zero_tokens():
    w = wl.scaled(wl.get(1), T=0, d=64, ffn=128)
    inp = wl.make_layer(w, seed=1)
    t = wl.device_layer(inp, DEV)
    layer = _layer(w, t)
    outs = layer.alloc_outputs()
    for v in outs.values():
        v.fill_(7)
    y = layer.forward(t["x"])
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    assert (outs["seg_offsets"] == 0).all() and (outs["kept_count"] == 0).all()
    assert (outs["expert_count"] == 0).all() and (outs["f"] == 0).all() and (outs["P"] == 0).all()
    assert outs["l_aux"].item() == 0.0 and outs["n_dropped"].item() == 0


@pytest.mark.parametrize("noalloc", [False, True])
def test_dispatch_zero_tokens(noalloc):
    """moe_dispatch (and the allocation-free form) on zero tokens: an empty x
    is allowed, the segment offsets, kept counts and drop count are zero."""
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    out = api.moe_dispatch(x, idx, 8, 1.25, 0, 0, noalloc=noalloc)
    torch.cuda.synchronize()
    assert (out["seg_offsets"] == 0).all() and (out["kept_count"] == 0).all()
    assert out["n_dropped"].item() == 0


@pytest.mark.parametrize("T", [1, 17])
def test_few_tokens(T):
    w = wl.scaled(wl.get(1), T=T, d=128, ffn=256, router_bias="gauss", expert_bias="gauss")
    inp, t = _inputs(w)
    _check_forward(w, inp, t)


@pytest.mark.parametrize("d", [65536, 65544])
def test_large_hidden_size(d):
    """A hidden size far past the benchmark's: the router's per-wave K range
    spans 256 steps and the first expert GEMM 1024 K steps (split along K
    over the chip: eight row tiles); d = 65544 is a multiple of 8 but not of
    64, so the first GEMM takes the 128x128 kernel and the router's last K
    step is ragged."""
    w = wl.scaled(wl.get(1), name="wide-d%d" % d, T=40, d=d, ffn=128, router_bias="gauss",
                  expert_bias="gauss")
    inp, t = _inputs(w)
    _check_forward(w, inp, t)


@pytest.mark.parametrize("cf", [0.0, 1.25])
def test_many_tokens(cf):
    """200 000 tokens of a narrow layer: 12 500 router blocks feeding the
    last-block statistics, and a dispatch past the single-launch bound (the
    histogram, scan, rank and scatter kernels), with and without a cap."""
    w = wl.scaled(wl.get(1), name="many-t-cf%g" % cf, T=200000, d=64, ffn=64, capacity_factor=cf,
                  router_bias="gauss", expert_bias="gauss")
    inp, t = _inputs(w)
    _check_forward(w, inp, t)


def test_single_expert_is_dense_ffn():
    w = wl.scaled(wl.get(1), T=130, d=128, E=1, k=1, ffn=256, expert_bias="gauss")
    inp, t = _inputs(w)
    layer, y, outs, nt, err, _ = _check_forward(w, inp, t)
    assert (outs["topk_w"] == 1.0).all()


def test_all_experts_selected():
    w = wl.scaled(wl.get(1), T=90, d=64, E=4, k=4, ffn=128)
    inp, t = _inputs(w)
    _check_forward(w, inp, t)


def test_capacity_zero_drops_everything():
    # C = floor(64 * 0.05 / 8) = 0
    w = wl.scaled(wl.get(1), T=64, d=64, ffn=128, capacity_factor=0.05)
    inp, t = _inputs(w)
    layer, y, outs, nt, err, _ = _check_forward(w, inp, t)
    assert (outs["slot_row"] == -1).all() and outs["n_dropped"].item() == 64 * 2
    assert (y.float() == 0).all()


def test_capacity_zero_with_shared_expert():
    w = wl.scaled(wl.get(4), T=48, d=64, ffn=128, E=16, k=4, num_local_experts=4, expert_begin=4,
                  capacity_factor=0.05)
    inp, t = _inputs(w)
    _check_forward(w, inp, t)


def test_max_experts_and_k():
    w = wl.scaled(wl.get(3), T=200, d=64, E=1024, k=32, ffn=64)
    inp, t = _inputs(w)
    _check_forward(w, inp, t)


def test_dispatch_ignores_out_of_range_ids():
    T, k, E = 50, 2, 8
    idx = np.random.default_rng(0).integers(0, E, size=(T, k)).astype(np.int32)
    idx[idx[:, 0] == idx[:, 1], 1] = (idx[idx[:, 0] == idx[:, 1], 0] + 1) % E
    idx[3, 1] = -5
    idx[7, 0] = 999
    gi = torch.from_numpy(idx).to(DEV)
    dp = api.moe_dispatch(None, gi, E, 0.0, 2, 4, with_x_perm=False, dtype=torch.bfloat16, d=64)
    torch.cuda.synchronize()
    ref = oracle.capacity(idx, E, 0.0, 2, 4)
    np.testing.assert_array_equal(dp["slot_row"].cpu().numpy(), ref.slot_row)
    np.testing.assert_array_equal(dp["seg_offsets"].cpu().numpy(), ref.seg_offsets)
    assert dp["slot_row"][3, 1].item() == -2 and dp["slot_row"][7, 0].item() == -2


@pytest.mark.parametrize("T,d,E,k,cf", [
    (4096, 4096, 8, 2, 0.0),     # single-launch dispatch, grid = CUs: eight-vector row prefetch
    (5000, 4104, 8, 2, 0.0),     # more blocks than CUs: four-vector prefetch, rest of a ragged row after
    (8192, 512, 64, 2, 0.0),     # four-vector prefetch longer than the row
    (8192, 2048, 64, 2, 1.25),   # capped: no prefetch, two blocks per CU
])
def test_dispatch_single_launch_grids(T, d, E, k, cf):
    """The single-launch dispatch in each of its grid regimes (prefetch of the
    row before the planning or not, one or two blocks per CU) against the
    oracle's capacity, permutation and x_perm, with Zipf-skewed selections."""
    rng = np.random.default_rng(T + d)
    logits = rng.standard_normal((T, E)) + 2.0 * np.log(1.0 / np.arange(1, E + 1))
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    dp = api.moe_dispatch(xt, torch.from_numpy(idx).to(DEV), E, cf)
    torch.cuda.synchronize()
    ref = oracle.capacity(idx, E, np.float32(cf))
    np.testing.assert_array_equal(dp["seg_offsets"].cpu().numpy(), ref.seg_offsets)
    np.testing.assert_array_equal(dp["kept_count"].cpu().numpy(), ref.kept_count)
    np.testing.assert_array_equal(dp["slot_row"].cpu().numpy(), ref.slot_row)
    rows = int(ref.seg_offsets[-1])
    np.testing.assert_array_equal(dp["row_src"].cpu().numpy()[:rows], ref.row_src)
    assert int(dp["n_dropped"].item()) == ref.n_dropped
    got = dp["x_perm"][:rows].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, expected_xperm(x, ref.row_src, k))


def test_pages_dispatch_example_on_gpu():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_dispatch_example.json")))
    idx = torch.tensor(g["topk_idx"], dtype=torch.int32, device=DEV)
    x = torch.arange(4 * 8, dtype=torch.float32, device=DEV).reshape(4, 8)
    dp = api.moe_dispatch(x, idx, g["E"])
    torch.cuda.synchronize()
    assert dp["row_src"][:4].tolist() == g["expected_row_src"]
    assert dp["seg_offsets"].tolist() == g["expected_seg_offsets"]
    assert dp["kept_count"].tolist() == g["expected_kept_count"]
    assert torch.equal(dp["x_perm"][:4], x[torch.tensor(g["expected_row_src"], device=DEV)])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("act", [0, 1])
def test_grouped_gemm_segments(dtype, act):
    """Segments of 0, 1, ragged and multi-tile sizes; K and N with tails."""
    g = torch.Generator().manual_seed(5)
    sizes = [0, 1, 130, 0, 257, 64, 3]
    rows, K, N = sum(sizes) + 9, 200, 136
    S = len(sizes)
    a = torch.randn(rows, K, generator=g).to(dtype)
    w = (torch.randn(S, N, K, generator=g) / K ** 0.5).to(dtype)
    b = (torch.randn(S, N, generator=g) * 0.1).to(dtype)
    seg = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32)
    out = torch.full((rows, N), 7.0, dtype=dtype)
    od = api.moe_grouped_gemm(a.to(DEV), seg.to(DEV), w.to(DEV), b.to(DEV), act, out=out.to(DEV))
    torch.cuda.synchronize()
    got = od.float().cpu()
    for s in range(S):
        lo, hi = int(seg[s]), int(seg[s + 1])
        ref = a[lo:hi].double() @ w[s].double().T + b[s].double()
        if act:
            ref = torch.nn.functional.gelu(ref, approximate="none")
        if hi > lo:
            tol = 1e-2 if dtype == torch.bfloat16 else 1e-5
            assert rel_err(got[lo:hi].numpy(), ref.numpy()) <= tol
    # rows past the last segment are untouched
    assert (got[seg[-1]:] == 7.0).all()


@pytest.mark.parametrize("use_ws", [False, True])
def test_grouped_gemm_256_partial_row_tiles(use_ws):
    """The 256x256 kernel on segments whose last row tile holds 1, 64, 65,
    128, 129 or a whole tile's rows, empty segments included, with and
    without the split-K tail (here every tile is split: 38 tiles on the
    whole chip)."""
    g = torch.Generator().manual_seed(8)
    sizes = [0, 1, 64, 65, 128, 129, 0, 256, 257, 384, 385, 640, 700, 3]
    rows, K, N = sum(sizes) + 5, 256, 512
    S = len(sizes)
    a = torch.randn(rows, K, generator=g).to(torch.bfloat16)
    w = (torch.randn(S, N, K, generator=g) / K ** 0.5).to(torch.bfloat16)
    b = (torch.randn(S, N, generator=g) * 0.1).to(torch.bfloat16)
    seg = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32)
    out = torch.full((rows, N), 7.0, dtype=torch.bfloat16).to(DEV)
    od = api.moe_grouped_gemm(a.to(DEV), seg.to(DEV), w.to(DEV), b.to(DEV), 1, out=out, use_ws=use_ws)
    torch.cuda.synchronize()
    got = od.float().cpu()
    for s_ in range(S):
        lo, hi = int(seg[s_]), int(seg[s_ + 1])
        if hi > lo:
            ref = torch.nn.functional.gelu(a[lo:hi].double() @ w[s_].double().T + b[s_].double(),
                                           approximate="none")
            assert rel_err(got[lo:hi].numpy(), ref.numpy()) <= 1e-2, s_
    assert (got[int(seg[-1]):] == 7.0).all()


def test_grouped_gemm_single_segment_null_offsets():
    g = torch.Generator().manual_seed(6)
    a = torch.randn(300, 128, generator=g).to(torch.bfloat16)
    w = (torch.randn(1, 256, 128, generator=g) / 128 ** 0.5).to(torch.bfloat16)
    od = api.moe_grouped_gemm(a.to(DEV), None, w.to(DEV), None, 0)
    torch.cuda.synchronize()
    ref = a.double() @ w[0].double().T
    assert rel_err(od.float().cpu().numpy(), ref.numpy()) <= 1e-2


def test_route_bitwise_reproducible_and_stats_fixed_order():
    w = SMALL["fine-small"]
    inp, t = _inputs(w)
    r1 = api.moe_route(t["x"], t["w_router"], t["b_router"], w.k)
    r2 = api.moe_route(t["x"], t["w_router"], t["b_router"], w.k)
    torch.cuda.synchronize()
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


@pytest.mark.parametrize("name", ["drop-small", "fine-small"])
def test_route_and_dispatch_into_caller_outputs(name):
    """The binding's out= form (outputs allocated once and reused, as the
    bench's stage timing calls them) gives the bits of fresh outputs, call
    after call, also after another layer's results were written into them."""
    w = SMALL[name]
    inp, t = _inputs(w)
    r0 = api.moe_route(t["x"], t["w_router"], t["b_router"], w.k, w.alpha, sel_bias=t["sel_bias"])
    d0 = api.moe_dispatch(t["x"], r0["topk_idx"], w.E, w.capacity_factor, w.expert_begin, w.num_local_experts)
    r_out = {k: torch.full_like(v, 7) for k, v in r0.items()}
    d_out = {k: (torch.full_like(v, 7) if torch.is_tensor(v) else v) for k, v in d0.items()}
    _, t2 = _inputs(w, seed=3)
    for xs in (t2["x"], t["x"], t["x"]):
        r = api.moe_route(xs, t["w_router"], t["b_router"], w.k, w.alpha, sel_bias=t["sel_bias"], out=r_out)
        d = api.moe_dispatch(xs, r["topk_idx"], w.E, w.capacity_factor, w.expert_begin, w.num_local_experts,
                             out=d_out)
    torch.cuda.synchronize()
    assert r is r_out and d is d_out
    for k in r0:
        assert torch.equal(r[k], r0[k]), k
    rows = int(d0["seg_offsets"][-1])
    for k in ("seg_offsets", "kept_count", "slot_row", "n_dropped"):
        assert torch.equal(d[k], d0[k]), k
    assert torch.equal(d["row_src"][:rows], d0["row_src"][:rows])
    assert torch.equal(d["x_perm"][:rows].view(torch.int16), d0["x_perm"][:rows].view(torch.int16))


def test_route_leaves_workspace_counters_zero():
    """The single-launch router's arrival counter (the workspace's first 256
    bytes) is zero again after every call, whatever the grid size, so the
    workspace is reusable as is (and in graph replays)."""
    for name in ("mixtral-small", "fine-small", "drop-small", "selbias-e32"):
        w = SMALL[name]
        inp, t = _inputs(w)
        for _ in range(2):
            r = api.moe_route(t["x"], t["w_router"], t["b_router"], w.k, w.alpha, sel_bias=t["sel_bias"])
            torch.cuda.synchronize()
            ws = api.workspace(t["x"].device, 0)
            assert int(ws[:256].count_nonzero().item()) == 0, name
            ref_route = oracle.route(inp.x, inp.w_router, inp.b_router, w.k, sel_bias=inp.sel_bias)
            _check_route(w, inp, r, ref_route)


@pytest.mark.parametrize("T,d,E,k,sel", [
    (6007, 256, 64, 2, "none"),    # two token tiles per block, last block 23 tokens
    (4100, 520, 17, 3, "gauss"),   # two tiles, last block 4 tokens, ragged K range per wave, selection bias
    (8205, 256, 64, 2, "none"),    # four tiles, last block 13 tokens
    (8223, 520, 16, 4, "gauss"),   # four tiles, ragged K range per wave, selection bias
    (16421, 200, 33, 3, "none"),   # four tiles, three expert tiles, last block 37 tokens
    (16384, 128, 8, 2, "none"),    # four tiles, whole blocks
    (50000, 64, 64, 8, "gauss"),   # four tiles, 782 blocks: statistics in 28 groups of 28
    (300007, 64, 64, 2, "none"),   # 4688 blocks: 63 groups (the counter limit), ragged last group
])
def test_route_multi_tile_blocks(T, d, E, k, sel):
    """The single-launch router's larger blocks (two or four 16-token tiles,
    taken above 4096 and 8192 tokens on 256 CUs) and its two-level statistics (block
    groups, then the groups) against the oracle on every token, with ragged
    last blocks and groups; bitwise equal on a second call, and the
    workspace's arrival counters back at zero."""
    w = wl.scaled(wl.get(2), name="route-tt", T=T, d=d, E=E, k=k, router_bias="gauss", sel_bias=sel)
    inp = wl.make_layer(w, seed=5, with_experts=False)
    x = wl.to_torch(inp.x, DEV)
    wr = wl.to_torch(inp.w_router, DEV)
    br = wl.to_torch(inp.b_router, DEV)
    sb = wl.to_torch(inp.sel_bias, DEV)
    r = api.moe_route(x, wr, br, k, w.alpha, sel_bias=sb)
    r2 = api.moe_route(x, wr, br, k, w.alpha, sel_bias=sb)
    torch.cuda.synchronize()
    ref = oracle.route(inp.x, inp.w_router, inp.b_router, k, sel_bias=inp.sel_bias)
    _check_route(w, inp, r, ref)
    for key in r:
        assert torch.equal(r[key], r2[key]), key
    ws = api.workspace(x.device, 0)
    assert int(ws[:256].count_nonzero().item()) == 0


def test_route_sel_bias_full_size():
    """The DeepSeek-shaped router (T=32768, d=7168, E=256, top-8, the E > 64
    path) with a selection-only bias, against the oracle on every token."""
    w = wl.scaled(wl.get(4), sel_bias="gauss")
    inp = wl.make_layer(w, seed=0, with_experts=False)
    x = wl.to_torch(inp.x, DEV)
    wr = wl.to_torch(inp.w_router, DEV)
    sb = wl.to_torch(inp.sel_bias, DEV)
    r = api.moe_route(x, wr, None, w.k, w.alpha, sel_bias=sb)
    torch.cuda.synchronize()
    ref = oracle.route(inp.x, inp.w_router, None, w.k, sel_bias=inp.sel_bias)
    _gidx, nt = _check_route(w, inp, r, ref)
    plain = api.moe_route(x, wr, None, w.k, w.alpha)
    torch.cuda.synchronize()
    changed = (plain["topk_idx"] != r["topk_idx"]).any(dim=1).float().mean().item()
    assert changed > 0.1, changed  # the bias moved a real share of the selections
    assert torch.equal(plain["P"], r["P"])  # P is the unbiased mean probability
    # 2048 select blocks: statistics in 45 groups; the arrival counters are back at zero
    ws = api.workspace(x.device, 0)
    assert int(ws[:256].count_nonzero().item()) == 0
    print("sel_bias: near ties boundary %d order %d; %.1f%% of tokens re-routed" %
          (nt["boundary"], nt["order"], 100 * changed))


def test_gelu_epilogue_matches_fp64_erf():
    """The first Linear's GELU (erf from Abramowitz & Stegun 7.1.26, |err| <=
    1.5e-7) against 0.5 u (1 + erf(u / sqrt 2)) in float64: a one-hot weight
    makes the fp32 GEMM output exactly GELU(u)."""
    import math
    u = torch.linspace(-9.0, 9.0, 4001, dtype=torch.float64)
    rows = u.numel()
    a = torch.zeros(rows, 8, dtype=torch.float32)
    a[:, 0] = u.float()
    w = torch.zeros(1, 8, 8, dtype=torch.float32)
    w[0, :, 0] = 1.0
    out = api.moe_grouped_gemm(a.to(DEV), None, w.to(DEV), None, 1)
    torch.cuda.synchronize()
    uu = a[:, 0].double()
    ref = 0.5 * uu * (1.0 + torch.erf(uu / math.sqrt(2.0)))
    err = (out[:, 0].cpu().double() - ref).abs()
    assert (err <= 4e-7 * (1.0 + uu.abs())).all(), float(err.max())
    # bf16 path: same function, output rounded to bf16
    ab = a.to(torch.bfloat16)
    wb = w.to(torch.bfloat16)
    ob = api.moe_grouped_gemm(ab.to(DEV), None, wb.to(DEV), None, 1)
    torch.cuda.synchronize()
    ub = ab[:, 0].double()
    refb = 0.5 * ub * (1.0 + torch.erf(ub / math.sqrt(2.0)))
    assert ((ob[:, 0].cpu().double() - refb).abs() <= 2.0 ** -8 * refb.abs() + 1e-6).all()


@pytest.mark.parametrize("sizes,split", [
    # 17 non-empty segments of at most one row tile x 8 feature tiles = 136
    # tiles on a 256-block grid: more than half a round, so three K ranges per
    # tile and two units per block (the capacity-drop layer's second GEMM)
    ([160] * 6 + [92, 55, 12, 17, 7, 6, 0, 4, 4, 1, 1, 1], True),
    # 200 tiles: more than two thirds of a round, not split
    ([100] * 25, False),
])
def test_grouped_gemm_tail_two_units_per_block(sizes, split):
    """The split-K tail with several units per block: against the fp64
    product (bias, GELU) within bf16 rounding, bitwise reproducible, and, when
    the plan does not split, bitwise equal to the call without a workspace."""
    g = torch.Generator().manual_seed(11)
    rows, K, N = sum(sizes), 1536, 2048
    S = len(sizes)
    a = torch.randn(rows, K, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn(S, N, K, generator=g) / K ** 0.5).to(torch.bfloat16).to(DEV)
    b = (torch.randn(S, N, generator=g) * 0.1).to(torch.bfloat16).to(DEV)
    seg = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32, device=DEV)
    whole = api.moe_grouped_gemm(a, seg, w, b, 1, use_ws=False)
    s1 = api.moe_grouped_gemm(a, seg, w, b, 1)
    s2 = api.moe_grouped_gemm(a, seg, w, b, 1)
    torch.cuda.synchronize()
    assert torch.equal(s1.view(torch.int16), s2.view(torch.int16))
    if not split:
        assert torch.equal(s1.view(torch.int16), whole.view(torch.int16))
    ref = torch.cat([torch.nn.functional.gelu(a[lo:hi].double() @ w[s].double().T + b[s].double(),
                                              approximate="none")
                     for s, (lo, hi) in enumerate(zip(seg[:-1].tolist(), seg[1:].tolist()))])
    assert rel_err(s1.float().cpu().numpy(), ref.cpu().numpy()) <= 1e-2
    assert rel_err(whole.float().cpu().numpy(), ref.cpu().numpy()) <= 1e-2


def test_grouped_gemm_split_tail_matches_whole_tiles():
    """With a workspace, tail tiles are split along K and reduced in a fixed
    order: equal to the unsplit result within bf16 rounding, and bitwise
    reproducible."""
    g = torch.Generator().manual_seed(7)
    sizes = [700, 300, 1000]           # 3 + 2 + 4 row tiles of 256
    rows, K, N = sum(sizes), 1024, 512
    a = torch.randn(rows, K, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn(3, N, K, generator=g) / K ** 0.5).to(torch.bfloat16).to(DEV)
    b = (torch.randn(3, N, generator=g) * 0.1).to(torch.bfloat16).to(DEV)
    seg = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32, device=DEV)
    whole = api.moe_grouped_gemm(a, seg, w, b, 1, use_ws=False)
    split1 = api.moe_grouped_gemm(a, seg, w, b, 1)
    split2 = api.moe_grouped_gemm(a, seg, w, b, 1)
    torch.cuda.synchronize()
    assert torch.equal(split1.view(torch.int16), split2.view(torch.int16))
    assert rel_err(split1.float().cpu().numpy(), whole.float().cpu().numpy()) <= 1e-2
    ref = torch.cat([torch.nn.functional.gelu(a[lo:hi].double() @ w[s].double().T + b[s].double(),
                                              approximate="none")
                     for s, (lo, hi) in enumerate(zip(seg[:-1].tolist(), seg[1:].tolist()))])
    assert rel_err(split1.float().cpu().numpy(), ref.cpu().numpy()) <= 1e-2
