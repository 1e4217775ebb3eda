"""GPU parity of the backward pass (moe_backward through the C ABI) against
the fp64 oracle's gradients, on seeded layers shaped like the pages'
workloads: routed experts with and without capacity drops, a local expert
share with a shared expert, expert biases, the selection-only router bias.

The oracle is conditioned on the GPU's top-k selection (a near tie may pick
either expert; selection has no gradient).  Floating-point gradients are
compared as max|got - ref| / max|ref|: the expert-path gradients (dx, dW1,
db1, dW2, db2 and the shared expert's) within the layer's Y tolerance
(bf16 operands, fp32 accumulation), the router gradients (dlogits, dW_r,
db_r) within the router tolerance, since the routing-weight gradient is
formed from fp32 values only.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL_ROUTER, TOL_Y_BF16, TOL_Y_F32, near_ties, rel_err
from top_routing_expert_route_amd import api
from top_routing_expert_route_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"

BWD_SMALL = {
    "tiny-fp32": wl.get(0),
    "bias-f32": wl.scaled(wl.get(0), name="bias-f32", T=301, d=72, ffn=136, router_bias="gauss",
                          expert_bias="gauss", capacity_factor=1.1),
    "mixtral-small": wl.scaled(wl.get(1), name="mixtral-small", T=333, d=256, ffn=384),
    "drop-small": wl.scaled(wl.get(2), name="drop-small", T=1000, d=192, ffn=256),
    "fine-bwd": wl.scaled(wl.get(3), name="fine-bwd", T=700, d=128, ffn=128),
    "dsv3-bwd": wl.scaled(wl.get(4), name="dsv3-bwd", T=500, d=192, ffn=256, expert_begin=32,
                          expert_bias="gauss"),
    "selbias-bwd": wl.scaled(wl.get(1), name="selbias-bwd", T=400, d=192, E=32, k=4, ffn=128,
                             sel_bias="gauss", router_bias="gauss"),
    # fp32 layer with a local share and a shared expert (fp32 K-segmented path, dx accumulated in place)
    "f32-shared": wl.scaled(wl.get(0), name="f32-shared", T=200, d=64, E=8, k=2, ffn=128, shared_expert=True,
                            expert_begin=2, num_local_experts=4, expert_bias="gauss", router_bias="gauss"),
    # E >= 32 but not a multiple of 8: the router backward stays on the vector units
    "e36-bwd": wl.scaled(wl.get(1), name="e36-bwd", T=300, d=128, E=36, k=3, ffn=128, capacity_factor=1.3),
}

EXPERT_GRADS = (("dx", "dx"), ("dw1", "dW1"), ("db1", "db1"), ("dw2", "dW2"), ("db2", "db2"))
SHARED_GRADS = (("dws1", "dWs1"), ("dbs1", "dbs1"), ("dws2", "dWs2"), ("dbs2", "dbs2"))
ROUTER_GRADS = (("dlogits", "dlogits"), ("dw_router", "dW_r"), ("db_router", "db_r"))


def _torch_dtype(w):
    return torch.bfloat16 if w.dtype == wl.BF16 else torch.float32


def _layer(w, t):
    return api.Layer(w.T, w.d, w.E, w.k, w.ffn, _torch_dtype(w), w.capacity_factor, w.expert_begin,
                     w.num_local_experts, w.alpha, t["w_router"], t["b_router"], t["w1"], t["b1"], t["w2"],
                     t["b2"], t["ws1"], t["bs1"], t["ws2"], t["bs2"], device=DEV, sel_bias=t["sel_bias"])


def _dy64(w, dy_host):
    return (wl.bf16_bits_to_f32(dy_host) if w.dtype == wl.BF16 else dy_host).astype(np.float64)


def _run(w, seed=0, g_aux=0.7):
    print("backward case", w.name, "T=%d d=%d E=%d k=%d ffn=%d" % (w.T, w.d, w.E, w.k, w.ffn), flush=True)
    inp = wl.make_layer(w, seed=seed)
    t = wl.device_layer(inp, DEV)
    dy_host = wl.make_grad_output(w, seed=seed)
    dy = wl.to_torch(dy_host, DEV)
    layer = _layer(w, t)
    outs = layer.alloc_outputs()
    layer.forward(t["x"])
    grads = layer.backward(t["x"], dy, g_aux, dlogits=True)
    torch.cuda.synchronize()
    return inp, t, dy, dy_host, layer, outs, grads


@pytest.mark.parametrize("name", list(BWD_SMALL))
def test_backward_small(name):
    w = BWD_SMALL[name]
    g_aux = 0.7
    inp, t, dy, dy_host, layer, outs, grads = _run(w, g_aux=g_aux)
    gidx = outs["topk_idx"].cpu().numpy()
    ref = oracle.backward(inp, _dy64(w, dy_host), g_aux=g_aux, topk_idx=gidx)
    tol = TOL_Y_BF16 if w.dtype == wl.BF16 else TOL_Y_F32
    pairs = EXPERT_GRADS + (SHARED_GRADS if w.shared_expert else ())
    for gname, rname in pairs:
        err = rel_err(grads[gname].cpu().numpy(), getattr(ref, rname))
        assert err <= tol, (gname, err)
    for gname, rname in ROUTER_GRADS:
        err = rel_err(grads[gname].cpu().numpy(), getattr(ref, rname))
        assert err <= TOL_ROUTER, (gname, err)


@pytest.mark.parametrize("name", ["mixtral-small", "dsv3-bwd", "tiny-fp32"])
def test_backward_deterministic(name):
    """Two calls in a row (workspace reused) give the same bits."""
    w = BWD_SMALL[name]
    inp, t, dy, dy_host, layer, outs, g1 = _run(w)
    g1 = {k: v.clone() for k, v in g1.items()}
    g2 = layer.backward(t["x"], dy, 0.7, dlogits=True)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k].view(torch.int32), g2[k].view(torch.int32)), k


def test_backward_aux_only():
    """dL/dY = 0: only the auxiliary loss reaches the router, and
    dl[t, e] = g_aux alpha / T * p[t, e] (f_e - sum_e' p[t, e'] f_e')."""
    w = BWD_SMALL["mixtral-small"]
    inp = wl.make_layer(w, seed=3)
    t = wl.device_layer(inp, DEV)
    dy = torch.zeros((w.T, w.d), dtype=torch.bfloat16, device=DEV)
    layer = _layer(w, t)
    outs = layer.alloc_outputs()
    layer.forward(t["x"])
    g = layer.backward(t["x"], dy, 2.5, dlogits=True)
    torch.cuda.synchronize()
    for n in ("dw1", "db1", "dw2", "db2"):
        assert torch.count_nonzero(g[n]).item() == 0, n
    r = oracle.route(inp.x, inp.w_router, inp.b_router, w.k)
    f = outs["f"].cpu().numpy().astype(np.float64)
    p = r.probs
    ref = 2.5 * w.alpha / w.T * p * (f[None, :] - (p * f[None, :]).sum(1, keepdims=True))
    assert rel_err(g["dlogits"].cpu().numpy(), ref) <= TOL_ROUTER


def test_backward_all_remote():
    """A selection bias keeps every token off the local experts: every routed
    weight gradient comes from empty segments (zero), dx is the router and
    shared-expert terms only."""
    w = wl.scaled(wl.get(1), name="all-remote", T=300, d=128, E=16, k=2, ffn=128, expert_begin=4,
                  num_local_experts=4, shared_expert=True)
    inp = wl.make_layer(w, seed=2)
    sb = np.zeros(w.E, np.float32)
    sb[4:8] = -100.0
    inp.sel_bias = sb
    t = wl.device_layer(inp, DEV)
    dy_host = wl.make_grad_output(w, seed=2)
    layer = _layer(w, t)
    outs = layer.alloc_outputs()
    layer.forward(t["x"])
    g = layer.backward(t["x"], wl.to_torch(dy_host, DEV), 0.7, dlogits=True)
    torch.cuda.synchronize()
    assert int(outs["seg_offsets"][-1].item()) == 0
    for n in ("dw1", "db1", "dw2", "db2"):
        assert torch.count_nonzero(g[n]).item() == 0, n
    ref = oracle.backward(inp, _dy64(w, dy_host), g_aux=0.7, topk_idx=outs["topk_idx"].cpu().numpy())
    for gname, rname in EXPERT_GRADS + SHARED_GRADS:
        assert rel_err(g[gname].cpu().numpy(), getattr(ref, rname)) <= TOL_Y_BF16, gname
    for gname, rname in ROUTER_GRADS:
        assert rel_err(g[gname].cpu().numpy(), getattr(ref, rname)) <= TOL_ROUTER, gname


def test_backward_zero_tokens():
    w = wl.scaled(wl.get(1), name="zero", T=0, d=128, ffn=128)
    inp = wl.make_layer(w, seed=1)
    t = wl.device_layer(inp, DEV)
    layer = _layer(w, t)
    dy = torch.empty((0, w.d), dtype=torch.bfloat16, device=DEV)
    grads = layer.backward(t["x"], dy, 1.0)
    for v in grads.values():
        v.fill_(7.0)
    grads = layer.backward(t["x"], dy, 1.0, grads=grads)
    torch.cuda.synchronize()
    for k, v in grads.items():
        assert torch.count_nonzero(v).item() == 0, k


def test_backward_rejects_unsupported_bf16_shape():
    w = wl.scaled(wl.get(1), name="odd", T=64, d=136, ffn=264)
    inp = wl.make_layer(w, seed=1)
    t = wl.device_layer(inp, DEV)
    layer = _layer(w, t)
    dy = torch.zeros((w.T, w.d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(api.MoeError) as e:
        layer.backward(t["x"], dy, 0.0)
    assert e.value.status == api.MOE_ERR_UNSUPPORTED


def _f64(w, a):
    if a is None:
        return None
    return (wl.bf16_bits_to_f32(a) if w.dtype == wl.BF16 else a).astype(np.float64)


def _bits(a):
    return a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)


@pytest.mark.parametrize("name", ["mixtral-small", "drop-small", "dsv3-bwd", "f32-shared", "tiny-fp32"])
def test_forward_save_and_backward_saved(name):
    """moe_forward_save writes moe_forward's bits and keeps u = W1 x + b1 of
    the kept rows (checked in fp64 on a row sample: row r of segment e holds
    token row_src[r] // k); moe_backward_saved on it gives moe_backward's
    bits, twice in a row."""
    w = BWD_SMALL[name]
    inp = wl.make_layer(w, seed=4)
    t = wl.device_layer(inp, DEV)
    dy = wl.to_torch(wl.make_grad_output(w, seed=4), DEV)
    layer = _layer(w, t)
    outs = layer.alloc_outputs()
    y_ref = layer.forward(t["x"]).clone()
    o_ref = {k: v.clone() for k, v in outs.items()}
    g_ref = {k: v.clone() for k, v in layer.backward(t["x"], dy, 0.7, dlogits=True).items()}
    y = layer.forward_save(t["x"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))
    for k in ("topk_idx", "topk_w", "seg_offsets", "kept_count", "slot_row"):
        assert torch.equal(outs[k], o_ref[k]), k

    seg = outs["seg_offsets"].cpu().numpy()
    row_src = outs["row_src"].cpu().numpy()
    u = layer.u_saved.cpu().numpy()
    x64, w1, b1 = _f64(w, inp.x), _f64(w, inp.w1), _f64(w, inp.b1)
    kept = int(seg[-1])
    assert kept > 0
    rows = np.random.default_rng(1).choice(kept, size=min(48, kept), replace=False)
    ref = np.empty((len(rows), w.ffn))
    for i, r in enumerate(rows):
        e = int(np.searchsorted(seg, r, side="right")) - 1
        ref[i] = w1[e] @ x64[row_src[r] // w.k] + (b1[e] if b1 is not None else 0.0)
    assert rel_err(u[rows].astype(np.float64), ref) <= 1e-5
    if w.shared_expert:
        us = layer.u_shared_saved.cpu().numpy().astype(np.float64)
        tok = np.random.default_rng(2).choice(w.T, size=min(32, w.T), replace=False)
        ref_s = x64[tok] @ _f64(w, inp.ws1).T + (_f64(w, inp.bs1) if inp.bs1 is not None else 0.0)
        assert rel_err(us[tok], ref_s) <= 1e-5

    for _ in range(2):
        g = layer.backward(t["x"], dy, 0.7, dlogits=True, saved=True)
        torch.cuda.synchronize()
        for k in g_ref:
            assert torch.equal(g[k].view(torch.int32), g_ref[k].view(torch.int32)), k


def test_backward_saved_needs_forward_save():
    w = BWD_SMALL["mixtral-small"]
    inp = wl.make_layer(w, seed=1)
    t = wl.device_layer(inp, DEV)
    layer = _layer(w, t)
    dy = torch.zeros((w.T, w.d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError):
        layer.backward(t["x"], dy, 0.0, saved=True)


# ------------------------------------------------------------- full size --
# The pages' workload shapes at full size, in the launch configuration of the
# benchmark.  The oracle cannot produce every gradient at these sizes in
# seconds, so it is sampled: dx and dlogits on a token sample (dropped and
# kept tokens, every near tie), and one whole 256-wide feature tile (plus the
# first and last feature) of the weight gradients of three experts (and of
# the shared expert): a row of output tiles of the first Linear's weight
# gradient and a column of tiles of the second's.  The router weight
# gradient is checked against its definition dW_r = dl^T x on the GPU's own
# dlogits (which the token sample pins to the oracle).

FULL = {w.name: w for w in wl.WORKLOADS[1:]}
FULL_TOKENS = 256


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(FULL))
def test_backward_full_size_sampled(name):
    w = FULL[name]
    g_aux = 0.7
    inp, t, dy, dy_host, layer, outs, grads = _run(w, g_aux=g_aux)
    gidx = outs["topk_idx"].cpu().numpy()
    dY64 = _dy64(w, dy_host)
    tol = TOL_Y_BF16 if w.dtype == wl.BF16 else TOL_Y_F32
    slot_row = outs["slot_row"].cpu().numpy()
    dropped = np.flatnonzero((slot_row == -1).any(1))
    kept = np.flatnonzero((slot_row >= 0).any(1))
    r = oracle.route(inp.x, inp.w_router, inp.b_router, w.k, sel_bias=inp.sel_bias)
    nb, no = near_ties(r.scores, w.k)
    # a sample of dropped tokens only could be all cancellation (dx ~ 0): keep kept ones in it
    toks = wl.token_sample(w.T, FULL_TOKENS, seed=5,
                           must_include=np.concatenate([dropped[:8], kept[:8], np.flatnonzero(nb | no)]))
    dx_ref, dl_ref = oracle.backward_tokens(inp, dY64, toks, g_aux, topk_idx=gidx)
    dx = grads["dx"][torch.from_numpy(toks).to(DEV)].cpu().numpy()
    dl_all = grads["dlogits"].cpu().numpy()
    assert rel_err(dx, dx_ref) <= tol
    assert rel_err(dl_all[toks], dl_ref) <= TOL_ROUTER
    # router weight and bias gradients: the contraction of the GPU's dlogits
    x64 = (wl.bf16_bits_to_f32(inp.x) if inp.x.dtype == np.uint16 else inp.x).astype(np.float64)
    dl64 = dl_all.astype(np.float64)
    assert rel_err(grads["dw_router"].cpu().numpy(), dl64.T @ x64) <= TOL_ROUTER
    assert rel_err(grads["db_router"].cpu().numpy(), dl64.sum(0)) <= TOL_ROUTER
    del x64, dl64
    # one whole 256-wide tile of hidden features (seeded) plus the first and
    # last feature, for the first, a middle and the last non-empty local expert
    cap = oracle.capacity(gidx, w.E, float(np.float32(w.capacity_factor)), w.expert_begin, w.num_local_experts)
    seg = cap.seg_offsets
    nonempty = [le for le in range(w.E_loc) if seg[le + 1] > seg[le]]
    g = np.random.default_rng([6, w.T])
    j0 = 256 * int(g.integers(0, max(1, w.ffn // 256)))
    qs = np.unique(np.concatenate([[0, w.ffn - 1], np.arange(j0, min(j0 + 256, w.ffn))]))
    for le in sorted({nonempty[0], nonempty[len(nonempty) // 2], nonempty[-1]}):
        slots = cap.row_src[seg[le]:seg[le + 1]].astype(np.int64)
        tk = slots // w.k
        wts = r.probs[tk, gidx.reshape(-1)[slots]]
        c = oracle.ffn_grad_columns(inp.x, inp.w1[le], None if inp.b1 is None else inp.b1[le], inp.w2[le], tk, wts,
                                    dY64, qs)
        assert rel_err(grads["dw1"][le][qs].cpu().numpy(), c.dW1_rows) <= tol, le
        assert rel_err(grads["db1"][le][qs].cpu().numpy(), c.db1) <= tol, le
        assert rel_err(grads["dw2"][le][:, qs].T.cpu().numpy(), c.dW2_cols) <= tol, le
        assert rel_err(grads["db2"][le].cpu().numpy(), c.db2) <= tol, le
    if w.shared_expert:
        c = oracle.ffn_grad_columns(inp.x, inp.ws1, inp.bs1, inp.ws2, np.arange(w.T), np.ones(w.T), dY64, qs)
        assert rel_err(grads["dws1"][qs].cpu().numpy(), c.dW1_rows) <= tol
        assert rel_err(grads["dbs1"][qs].cpu().numpy(), c.db1) <= tol
        assert rel_err(grads["dws2"][:, qs].T.cpu().numpy(), c.dW2_cols) <= tol
        assert rel_err(grads["dbs2"].cpu().numpy(), c.db2) <= tol
