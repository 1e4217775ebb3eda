"""Benchmark of the MoE layer forward on one MI355X.

A step is one moe_forward over one batch: route (router GEMM, softmax, top-k,
load statistics), dispatch (capacity, drops, permutation), the expert FFN
(grouped GEMM + GELU, grouped GEMM) and combine.  Inputs are seeded
synthetic layers already resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Beside the mean step time the line carries the median and minimum of the
same steps timed one by one; the HBM-bound stages (route, dispatch, combine)
timed warm and cold (a 1 GiB copy before each evicts L2 and the MALL); a
plain 1 GiB device copy as the practical HBM ceiling; the step replayed from
a HIP graph captured once (graph_replay); and the oracle on all cores
(cpu_baseline) and on one thread.

The roofline entry covers the dominant kernel (the first grouped GEMM with
the fused GELU): algorithmic flops of one launch (2 * rows * d * ffn, rows =
the kept (token, expert) pairs of the run) over its average duration, timed
with HIP events on the stream the library launches on.  The per-step value is
timed separately on moe_forward itself, with no events inside the step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "mixtral8x7b-layer"


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp"):
        with open(os.path.join(ROOT, "top_routing_expert_route_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or
    None when the kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            t = json.load(f)
        e = t[workload][kernel]
        if e.get("source_hash") != _kernel_source_hash():
            return None
        return e["bytes_per_launch"]
    except (KeyError, ValueError, OSError):
        return None


_ROUTED = {}  # the oracle's routing and capacity plan of a layer, from cpu_baseline


def cpu_baseline_single_thread(inp, budget_s: float = 5.0) -> dict:
    """The oracle on one thread: routing of the first min(T, 512) tokens and
    the expert FFN + combine of a seeded token sample sized to about budget_s
    seconds, each scaled per token (routing and the FFN are per-token work;
    the statistics and capacity passes are integer bookkeeping)."""
    import numpy as np
    import oracle
    from top_routing_expert_route_amd import workloads as wl
    w = inp.w
    n_r = min(w.T, 512)
    t0 = time.perf_counter()
    oracle.route(inp.x[:n_r], inp.w_router, inp.b_router, w.k, threads=1, want_logits=False)
    t_route = (time.perf_counter() - t0) / n_r
    if id(inp) in _ROUTED:
        r, dp = _ROUTED[id(inp)]
    else:
        r = oracle.route(inp.x, inp.w_router, inp.b_router, w.k, threads=len(os.sched_getaffinity(0)),
                         want_logits=False)
        dp = oracle.capacity(r.topk_idx, w.E, float(np.float32(w.capacity_factor)), w.expert_begin,
                             w.num_local_experts)

    def ffn(tokens):
        s = time.perf_counter()
        oracle.combine(inp.x, tokens, r.topk_idx, r.topk_w, dp.slot_row, inp.w1, inp.b1, inp.w2, inp.b2,
                       w.expert_begin, inp.ws1, inp.bs1, inp.ws2, inp.bs2, threads=1)
        return time.perf_counter() - s

    probe = ffn(wl.token_sample(w.T, 1, seed=98))
    n = int(min(w.T, max(1, (budget_s - probe) / max(probe, 1e-9))))
    tok = wl.token_sample(w.T, n, seed=101)
    t_ffn = ffn(tok) / len(tok)
    return {"value": round(1.0 / (t_route + t_ffn), 3), "unit": "tokens/s", "cores": 1,
            "sample": "fp64 oracle on 1 thread: routing of %d tokens (%.3f ms/token), expert FFN+combine of a "
                      "seeded sample of %d tokens (%.1f ms/token)" % (n_r, t_route * 1e3, len(tok), t_ffn * 1e3)}


def cpu_baseline(inp, budget_s: float = 15.0) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload:
    routing, statistics and capacity over all T tokens, the expert FFN and
    combine on a seeded token sample sized to about budget_s seconds."""
    import numpy as np
    import oracle
    from top_routing_expert_route_amd import workloads as wl
    w = inp.w
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    r = oracle.route(inp.x, inp.w_router, inp.b_router, w.k, threads=threads, want_logits=False)
    oracle.load_stats(r.topk_idx, r.probs, w.alpha)
    dp = oracle.capacity(r.topk_idx, w.E, float(np.float32(w.capacity_factor)), w.expert_begin,
                         w.num_local_experts)
    t_route = time.perf_counter() - t0
    _ROUTED[id(inp)] = (r, dp)

    def ffn(tokens):
        s = time.perf_counter()
        oracle.combine(inp.x, tokens, r.topk_idx, r.topk_w, dp.slot_row, inp.w1, inp.b1, inp.w2, inp.b2,
                       w.expert_begin, inp.ws1, inp.bs1, inp.ws2, inp.bs2, threads=threads)
        return time.perf_counter() - s

    n = max(1, threads)
    probe = ffn(wl.token_sample(w.T, n, seed=99))
    per_tok = probe / n
    n2 = int(min(w.T, max(n, (budget_s - probe) / max(per_tok, 1e-9))))
    n2 = max(threads, n2 // threads * threads)
    tok = wl.token_sample(w.T, n2, seed=100)
    t_ffn = ffn(tok)
    sec_per_token = t_route / w.T + t_ffn / len(tok)
    return {"value": round(1.0 / sec_per_token, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle: route+stats+capacity over all %d tokens (%.2f s), expert FFN+combine on a "
                      "seeded sample of %d tokens (%.2f s); tokens/s = 1/(t_route/T + t_ffn/n)"
                      % (w.T, t_route, len(tok), t_ffn)}


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def hbm_copy_ceiling(torch, dev, reps: int = 5) -> dict:
    """A plain 1 GiB device-to-device copy timed with HIP events: the
    practical HBM ceiling beside the nominal 8 TB/s (2 GiB moved a copy)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    stream = torch.cuda.current_stream(dev)
    us = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        e1.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3)
    del a, b
    best = min(us)
    return {"bytes_moved": 2 * n, "us_median": round(_median(us), 1), "us_min": round(best, 1),
            "gbps_best": round(2 * n / (best * 1e-6) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the moe_backward timing")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert-parallel sharding is a "
              "design note only). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from top_routing_expert_route_amd import accounting as acc
    from top_routing_expert_route_amd import api
    from top_routing_expert_route_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return

    api.lib()  # fail loudly if the HIP library is missing
    w = wl.get(args.workload)
    inp = wl.make_layer(w, seed=0)
    t = wl.device_layer(inp, dev)
    dt = torch.bfloat16 if w.dtype == wl.BF16 else torch.float32
    layer = api.Layer(w.T, w.d, w.E, w.k, w.ffn, dt, w.capacity_factor, w.expert_begin, w.num_local_experts,
                      w.alpha, t["w_router"], t["b_router"], t["w1"], t["b1"], t["w2"], t["b2"], t["ws1"],
                      t["bs1"], t["ws2"], t["bs2"], device=dev, sel_bias=t["sel_bias"])
    outs = layer.alloc_outputs()
    x = t["x"]
    y = torch.empty((w.T, w.d), dtype=dt, device=dev)

    # ---- headline: K whole-layer steps of moe_forward ----
    for _ in range(args.warmup):
        layer.forward(x, y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.forward(x, y)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.T * args.steps / elapsed

    # ---- per-step spread: the same steps, each between two HIP events ----
    stream = torch.cuda.current_stream(dev)
    step_ms = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        layer.forward(x, y)
        e1.record(stream)
        e1.synchronize()
        step_ms.append(e0.elapsed_time(e1))

    # ---- the same step replayed from a HIP graph (captured once) ----
    graph = None
    try:
        side_g = torch.cuda.Stream(device=dev)
        side_g.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side_g):
            layer.forward(x, y)
        torch.cuda.current_stream(dev).wait_stream(side_g)
        torch.cuda.synchronize()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            layer.forward(x, y)
        for _ in range(args.warmup):
            cg.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(args.steps):
            cg.replay()
        torch.cuda.synchronize()
        elg = time.perf_counter() - tg
        graph = {"ms_per_step": round(elg * 1e3 / args.steps, 4), "value": round(w.T * args.steps / elg, 1)}
        del cg
    except RuntimeError as e:  # reported, not fatal: the eager line above is the headline
        graph = {"error": str(e)[:200]}

    # ---- with a shared expert: the same step with it on a second stream ----
    overlap = None
    if w.shared_expert:
        side = torch.cuda.Stream(device=dev)
        y_ov = torch.empty_like(y)
        for _ in range(args.warmup):
            layer.forward(x, y_ov, side_stream=side)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            layer.forward(x, y_ov, side_stream=side)
        torch.cuda.synchronize()
        el = time.perf_counter() - t1
        overlap = {"entry_point": "moe_forward_overlap", "ms_per_step": round(el * 1e3 / args.steps, 4),
                   "value": round(w.T * args.steps / el, 1), "speedup": round(elapsed / el, 4),
                   "same_bits": bool(torch.equal(y_ov.view(torch.int16), y.view(torch.int16)))
                   if y.dtype == torch.bfloat16 else bool(torch.equal(y_ov, y))}

    # counts of the actual run
    seg = outs["seg_offsets"].cpu().numpy()
    rows = int(seg[-1])
    per_expert = np.diff(seg)
    slot_row = outs["slot_row"].cpu().numpy()
    counts = acc.RunCounts(T=w.T, d=w.d, E=w.E, k=w.k, ffn=w.ffn, dtype=w.dtype, rows=rows,
                           active_experts=int((per_expert > 0).sum()),
                           tokens_with_rows=int((slot_row >= 0).any(axis=1).sum()), shared=w.shared_expert,
                           has_router_bias=inp.b_router is not None)

    def tflops(flops, us):
        return flops / (us * 1e-6) / 1e12 if us > 0 else 0.0

    def gbps(b, us):
        return b / (us * 1e-6) / 1e9 if us > 0 else 0.0

    # ---- per-stage timing with HIP events on the launch stream ----
    names = ["route", "dispatch", "gemm1_gelu", "gemm2", "shared", "combine"]
    acc_ms = {n: 0.0 for n in names}
    dp_ws = {}

    # the step functions write into outputs allocated once, so that the timed
    # calls launch the library's kernels only (no allocation, no fill)
    r_out = api.moe_route(x, t["w_router"], t["b_router"], w.k, w.alpha, sel_bias=t["sel_bias"])
    dp_out = api.moe_dispatch(x, r_out["topk_idx"], w.E, w.capacity_factor, w.expert_begin, w.num_local_experts)

    def staged_step(record):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] if record else None
        if record:
            ev[0].record(stream)
        r = api.moe_route(x, t["w_router"], t["b_router"], w.k, w.alpha, sel_bias=t["sel_bias"], out=r_out)
        if record:
            ev[1].record(stream)
        dp = api.moe_dispatch(x, r["topk_idx"], w.E, w.capacity_factor, w.expert_begin, w.num_local_experts,
                              out=dp_out)
        if record:
            ev[2].record(stream)
        h = api.moe_grouped_gemm(dp["x_perm"], dp["seg_offsets"], t["w1"], t["b1"], 1,
                                 out=dp_ws.setdefault("h", torch.empty((dp["max_rows"], w.ffn), dtype=dt,
                                                                       device=dev)))
        if record:
            ev[3].record(stream)
        yp = api.moe_grouped_gemm(h, dp["seg_offsets"], t["w2"], t["b2"], 0,
                                  out=dp_ws.setdefault("yp", torch.empty((dp["max_rows"], w.d), dtype=dt,
                                                                         device=dev)))
        if record:
            ev[4].record(stream)
        ysh = None
        if w.shared_expert:
            hs = api.moe_grouped_gemm(x, None, t["ws1"].unsqueeze(0), None, 1)
            ysh = api.moe_grouped_gemm(hs, None, t["ws2"].unsqueeze(0), None, 0)
        if record:
            ev[5].record(stream)
        api.moe_combine(yp, dp["slot_row"], r["topk_w"], ysh, y=y)
        if record:
            ev[6].record(stream)
        return ev

    for _ in range(2):
        staged_step(False)
    torch.cuda.synchronize()
    evs = [staged_step(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for ev in evs:
        for i, n in enumerate(names):
            acc_ms[n] += ev[i].elapsed_time(ev[i + 1])
    avg_us = {n: acc_ms[n] * 1e3 / args.steps for n in names}

    g1_flops = acc.gemm1_flops(counts)
    g1_tf = tflops(g1_flops, avg_us["gemm1_gelu"])
    stages = {
        "route": {"us": round(avg_us["route"], 2), "bytes": acc.route_bytes(counts),
                  "hbm_frac": round(gbps(acc.route_bytes(counts), avg_us["route"]) / acc.PEAK_HBM_GBPS, 4)},
        "dispatch": {"us": round(avg_us["dispatch"], 2), "bytes": acc.dispatch_bytes(counts),
                     "hbm_frac": round(gbps(acc.dispatch_bytes(counts), avg_us["dispatch"]) / acc.PEAK_HBM_GBPS,
                                       4)},
        "gemm1_gelu": {"us": round(avg_us["gemm1_gelu"], 2), "flops": g1_flops,
                       "mfma_frac": round(g1_tf / acc.PEAK_BF16_TFLOPS, 4)},
        "gemm2": {"us": round(avg_us["gemm2"], 2), "flops": acc.gemm2_flops(counts),
                  "mfma_frac": round(tflops(acc.gemm2_flops(counts), avg_us["gemm2"]) / acc.PEAK_BF16_TFLOPS, 4)},
        "combine": {"us": round(avg_us["combine"], 2), "bytes": acc.combine_bytes(counts),
                    "hbm_frac": round(gbps(acc.combine_bytes(counts), avg_us["combine"]) / acc.PEAK_HBM_GBPS, 4)},
    }
    if w.shared_expert:
        stages["shared"] = {"us": round(avg_us["shared"], 2), "flops": acc.shared_flops(counts),
                            "mfma_frac": round(tflops(acc.shared_flops(counts), avg_us["shared"]) /
                                               acc.PEAK_BF16_TFLOPS, 4)}
    staged_total = sum(avg_us.values())

    # ---- cold HBM-bound stages: a 1 GiB copy (512 MiB read, 512 MiB written)
    # before each timed stage evicts L2 and the 256 MB MALL ----
    sa = torch.empty(1 << 29, dtype=torch.uint8, device=dev).fill_(3)
    sb = torch.empty_like(sa)
    cold = {"route": [], "dispatch": [], "combine": []}

    def timed(fn):
        sb.copy_(sa)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = fn()
        e1.record(stream)
        return out, (e0, e1)

    cold_reps = max(5, min(args.steps, 10))
    for _ in range(cold_reps + 1):
        r, ev_r = timed(lambda: api.moe_route(x, t["w_router"], t["b_router"], w.k, w.alpha, sel_bias=t["sel_bias"],
                                              out=r_out))
        dp, ev_d = timed(lambda: api.moe_dispatch(x, r["topk_idx"], w.E, w.capacity_factor, w.expert_begin,
                                                  w.num_local_experts, out=dp_out))
        h = api.moe_grouped_gemm(dp["x_perm"], dp["seg_offsets"], t["w1"], t["b1"], 1, out=dp_ws["h"])
        yp = api.moe_grouped_gemm(h, dp["seg_offsets"], t["w2"], t["b2"], 0, out=dp_ws["yp"])
        ysh = None
        if w.shared_expert:
            hs = api.moe_grouped_gemm(x, None, t["ws1"].unsqueeze(0), None, 1)
            ysh = api.moe_grouped_gemm(hs, None, t["ws2"].unsqueeze(0), None, 0)
        _, ev_c = timed(lambda: api.moe_combine(yp, dp["slot_row"], r["topk_w"], ysh, y=y))
        torch.cuda.synchronize()
        for n, (e0, e1) in (("route", ev_r), ("dispatch", ev_d), ("combine", ev_c)):
            cold[n].append(e0.elapsed_time(e1) * 1e3)
    del sa, sb
    cold_bytes = {"route": acc.route_bytes(counts), "dispatch": acc.dispatch_bytes(counts),
                  "combine": acc.combine_bytes(counts)}
    stages_cold = {}
    for n, v in cold.items():
        v = v[1:]  # the first round warms up the allocator
        med = _median(v)
        stages_cold[n] = {"us_median": round(med, 2), "us_min": round(min(v), 2), "bytes": cold_bytes[n],
                          "hbm_frac_median": round(gbps(cold_bytes[n], med) / acc.PEAK_HBM_GBPS, 4)}

    # ---- backward: K steps of moe_backward on the same layer (dL/dY seeded
    # Gaussian, dL/dL_aux = 1); reported beside the forward, not in `value` ----
    backward = None
    if not args.no_backward and not (w.dtype == wl.BF16 and (w.d % 64 or w.ffn % 64)):
        dy = wl.to_torch(wl.make_grad_output(w, seed=0), dev)
        grads = layer.backward(x, dy, 1.0)
        for _ in range(args.warmup):
            layer.backward(x, dy, 1.0, grads=grads)
        torch.cuda.synchronize()
        tb = time.perf_counter()
        for _ in range(args.steps):
            layer.backward(x, dy, 1.0, grads=grads)
        torch.cuda.synchronize()
        elb = time.perf_counter() - tb
        bflops = acc.backward_gemm_flops(counts)
        btf = bflops * args.steps / elb / 1e12
        backward = {"entry_point": "moe_backward", "ms_per_step": round(elb * 1e3 / args.steps, 4),
                    "value": round(w.T * args.steps / elb, 1), "unit": "tokens/s",
                    "gemm_flops": bflops, "router_flops": acc.backward_router_flops(counts),
                    "gemm_tflops_over_step": round(btf, 2),
                    "mfma_frac_over_step": round(btf / acc.PEAK_BF16_TFLOPS, 4)}
        # the same with the first Linear's pre-activations kept from the
        # forward (moe_forward_save + moe_backward_saved): no GEMM recompute
        y_s = torch.empty_like(y)
        for _ in range(args.warmup):
            layer.forward_save(x, y_s)
            layer.backward(x, dy, 1.0, grads=grads, saved=True)
        torch.cuda.synchronize()
        tf = time.perf_counter()
        for _ in range(args.steps):
            layer.forward_save(x, y_s)
        torch.cuda.synchronize()
        tb2 = time.perf_counter()
        for _ in range(args.steps):
            layer.backward(x, dy, 1.0, grads=grads, saved=True)
        torch.cuda.synchronize()
        te = time.perf_counter()
        backward["saved"] = {"entry_points": "moe_forward_save + moe_backward_saved",
                             "forward_save_ms": round((tb2 - tf) * 1e3 / args.steps, 4),
                             "backward_saved_ms": round((te - tb2) * 1e3 / args.steps, 4),
                             "same_bits_y": bool(torch.equal(y_s.view(torch.int16), y.view(torch.int16)))
                             if y.dtype == torch.bfloat16 else bool(torch.equal(y_s, y))}
        layer.u_saved = layer.u_shared_saved = None
        del grads, dy, y_s

    result = {
        "metric": "MoE layer tokens/sec (1 GPU)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == wl.BF16 else "f32",
        "data": "synthetic (seeded Gaussian layer, uniform routing; no trained weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "ffn": w.ffn,
                   "capacity_factor": w.capacity_factor, "num_local_experts": w.E_loc,
                   "shared_expert": w.shared_expert, "router": "fp32", "rows": rows,
                   "active_experts": counts.active_experts, "tokens_with_rows": counts.tokens_with_rows},
        "roofline": {"bound": "mfma", "achieved": round(g1_tf, 2), "peak": acc.PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(g1_tf / acc.PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic(w.name, "gemm1_gelu"),
                     "kernel": "grouped_gemm_256 (first Linear + GELU)",
                     "flops_per_launch": g1_flops, "avg_us": round(avg_us["gemm1_gelu"], 2)},
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(_median(step_ms), 4),
                    "min": round(min(step_ms), 4)},
        "stages": stages,
        "stages_cold": stages_cold,
        "staged_step_us": round(staged_total, 1),
        "hbm_copy": hbm_copy_ceiling(torch, dev),
    }
    if graph is not None:
        result["graph_replay"] = graph
    if overlap is not None:
        result["shared_overlap"] = overlap
    if backward is not None:
        result["backward"] = backward
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp)
        result["cpu_baseline"]["single_thread"] = cpu_baseline_single_thread(inp)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
