"""Benchmark of one DeepSeekMoE layer forward with bias-based balancing on one MI355X.

A step is one pass of the whole path over one batch: route (router GEMM +
sigmoid + biased group-limited top-k) -> dispatch (count, scan, permute) ->
expert FFN (gate/up GEMM + SwiGLU, down GEMM; routed and shared) -> combine ->
bias update.  Workload: the V3-like prefill layer in bf16 (T=16384 tokens,
hidden 7168, 256 routed experts in 8 groups, at most 4 groups per token,
top-8, 1 shared expert, intermediate 2048, gate scale 2.5), seeded synthetic
inputs resident in HBM before timing starts.

Prints ONE JSON line on stdout (progress goes to stderr).  value = routed
tokens/s of the whole layer.  The roofline object is for the dominant kernel,
the gate/up grouped GEMM, timed live with HIP events on the stream it runs
on.  cpu_baseline times the plain CPU oracle on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer (V3-like bf16); % MFMA peak; route GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_prefill_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decode-size and FP8 measurements that follow the headline one")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="rough budget of the CPU oracle sample")
    ap.add_argument("--train-only", action="store_true",
                    help="diagnostic: time only the training step (forward + backward) and print its JSON")
    ap.add_argument("--dispatch", choices=("gather", "copy"), default="gather",
                    help="gather: dispatch writes the indices and the gate/up GEMM reads its rows from x "
                         "through perm; copy: dispatch also writes x_perm and the GEMM reads that")
    ap.add_argument("--two-stream", action="store_true",
                    help="diagnostic: one batch's expert GEMMs against another batch's dispatch (row copy) + "
                         "combine, one after the other and on two streams (micro-batch overlap); prints its JSON")
    ap.add_argument("--gemm-probe", choices=("random", "zero"), default=None,
                    help="diagnostic: time the grouped gate/up and down GEMMs alone with expert weights drawn on the "
                         "GPU (N(0, sigma), or all zero: the same instructions on data that switches few bits), "
                         "plus a dense hipBLASLt GEMM of the gate/up shape; prints its JSON")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this size 3 times (a plain copy kernel of known "
                         "size, for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def stage_bytes(c, gather=False, scores=False):
    """Algorithmic HBM bytes of the bandwidth-bound stages (per layer pass).  With
    gather, dispatch moves indices only (the rows are read by the gate/up GEMM).
    Without scores the route stage reads x, W_r and the bias and writes idx and w
    (the [T, E] affinities stay on chip); with them it also writes and reads them."""
    a = 2  # bf16
    sc = c.T * c.E * 4 if scores else 0
    route = sc + c.E * 4 + c.T * c.k * 8                                   # (scores in), bias, idx + w out
    router = c.T * c.H * a + c.E * c.H * a + sc                           # x + W_r in, (scores out)
    dispatch = c.T * c.k * 4 * 4                                          # idx in (twice), perm + inv out
    if not gather:
        dispatch += c.T * c.H * a + c.T * c.k * c.H * a                   # x in, x_perm out
    combine = c.T * c.k * c.H * a + c.T * c.H * a * (2 if c.S else 1) + c.T * c.k * 8
    return dict(router=router, topk=route, dispatch=dispatch, combine=combine)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gate_up_v3_prefill_bf16.txt")
TRAFFIC_SOURCES = ["include/moe.h", "biased_top_routing_amd/csrc/common.h", "biased_top_routing_amd/csrc/ffn_layout.h",
                   "biased_top_routing_amd/csrc/ffn.hip", "biased_top_routing_amd/csrc/gemm_bf16.hip"]


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the gate/up GEMM from the committed counter summary, or None
    when the summary is missing, covers another workload, or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("workload") != workload or kv.get("sources_sha256") != sources_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(c, x, w, bias, budget_s):
    """Plain numpy oracle on a bounded sample; returns the layer rate it implies."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    cores = len(os.sched_getaffinity(0))
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t_rows = min(c.T, 1024)
    rows = slice(0, t_rows)
    x32 = oracle.decode_act(x[rows]).astype(np.float64)
    t0 = time.perf_counter()
    s = oracle.affinity(x32, oracle.decode_act(w.w_router), w.logit_offset)
    idx, gates = oracle.route(s, bias, c.G, c.M, c.k, c.group_topr, c.route_scale)
    counts, offsets, perm, inv = oracle.dispatch(idx, c.E)
    t_route = time.perf_counter() - t0
    # expert FFN on whole segments of a few experts until the budget is used
    t0 = time.perf_counter()
    pairs_done = 0
    order = np.argsort(-counts)
    e_used = 0
    for e in order:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xp = oracle.decode_act(x[rows][perm[lo:hi] // c.k])
        oracle.swiglu(xp, oracle.decode_act(w.w_gate_up[e]), oracle.decode_act(w.w_down[e]))
        pairs_done += hi - lo
        e_used += 1
        if time.perf_counter() - t0 > budget_s * 0.6:
            break
    t_routed = time.perf_counter() - t0
    t0 = time.perf_counter()
    sh_rows = min(t_rows, 256)
    ysh = oracle.shared_ffn(x32[:sh_rows], [oracle.decode_act(a) for a in w.ws_gate_up],
                            [oracle.decode_act(a) for a in w.ws_down])
    t_shared = time.perf_counter() - t0
    t0 = time.perf_counter()
    yp = np.zeros((t_rows * c.k, c.H))
    oracle.combine(yp, np.zeros((t_rows, c.H)), inv, gates)
    t_combine = time.perf_counter() - t0
    # extrapolate to the whole batch
    per_token = (t_route + t_combine) / t_rows + t_routed / pairs_done * c.k + t_shared / sh_rows
    layer_s = per_token * c.T
    del ysh
    return {"value": c.T / layer_s, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "host_cores": cores,
            "sample": (f"{t_rows} of {c.T} tokens routed/dispatched/combined in fp64 numpy; expert FFN on "
                       f"{pairs_done} (token,expert) pairs over {e_used} whole expert segments; shared expert "
                       f"on {sh_rows} tokens; rate extrapolated per token to T={c.T}"),
            "measured_s": round(t_route + t_routed + t_shared + t_combine, 2)}


PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
STAGES = ["route", "dispatch", "gate_up", "down", "combine", "bias"]


def time_layer(layer, x, bias, c, steps, warmup):
    """Warm up, then time `steps` whole-layer passes.  Returns (ms per step from the
    host clock, mean ms of each stage from HIP events recorded on the layer's stream)."""
    import numpy as np
    import torch

    from biased_top_routing_amd import _lib as L

    def step(ev=None):
        calls = [lambda: layer.route(x, bias), lambda: layer.dispatch(x),
                 lambda: layer.expert_ffn(x, L.MOE_FFN_GATE_UP), lambda: layer.expert_ffn(x, L.MOE_FFN_DOWN),
                 layer.combine, lambda: layer.update_bias(bias, c.gamma)]
        for j, f in enumerate(calls):
            if ev is not None:
                ev[j].record()
            f()
        if ev is not None:
            ev[len(calls)].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in events])) for j, n in enumerate(STAGES)}
    return wall * 1e3 / steps, stage_ms


def decode_extra(layer, c, w, steps, warmup):
    """The same layer at decode size (T=128): time per step and the rate at which it
    streams the weights of the experts it touches (the decode roofline is HBM)."""
    import torch

    from workloads import CONFIGS
    from workloads.inputs import make_x
    cd = CONFIGS["v3_decode_bf16"]
    layer.alloc(cd.T)
    x = to_dev(make_x(cd, 0))
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    ms, stage_ms = time_layer(layer, x, bias, cd, steps, warmup)
    counts = layer.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    wbytes = (touched + cd.S) * 3 * cd.H * cd.I * 2 + cd.E * cd.H * 2
    # rows of H bf16 per token: x for the router and the shared expert, y out, y_perm
    # written and read, and x_perm written and read (copy) or x gathered (gather)
    rows_per_token = 3 + 2 * cd.k + (cd.k if layer.gather else 2 * cd.k)
    iobytes = cd.T * cd.H * 2 * rows_per_token
    return {"workload": cd.name, "T": cd.T, "ms_per_step": round(ms, 4), "tokens_per_s": round(cd.T / (ms * 1e-3), 1),
            "experts_touched": touched, "hbm_gbs": round((wbytes + iobytes) / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round((wbytes + iobytes) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes": wbytes + iobytes, "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()}}


BWD_STAGES = ["combine_bwd", "expert_ffn_bwd", "route_bwd", "dispatch_bwd"]


def train_extra(c, w, steps, warmup, alpha=1e-3, seq_len=4096):
    """One training step of the layer at the prefill shape: the forward pass (with the
    row copy, whose x_perm the backward reads) and the backward pass (gradients of
    every weight, the input and the balance loss).  Per-call times from HIP events.
    The main figures keep the gate and up outputs in the forward pass
    (moe_expert_ffn_save, 2 (T k + T S) I bf16 values) so that the backward pass
    starts from them; "recompute" times the same step recomputing them instead."""
    import numpy as np
    import torch

    from biased_top_routing_amd import _lib as L
    from biased_top_routing_amd.runner import MoeLayerGPU
    from workloads.inputs import make_x

    layer = MoeLayerGPU(c, w, gather=False, save_gu=True)
    x = to_dev(make_x(c, 0))
    g = torch.Generator(device="cuda").manual_seed(5)
    dy = torch.randn((c.T, c.H), device="cuda", generator=g).to(torch.bfloat16)
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    layer.alloc_backward()
    cfg = layer.cfg

    def ffn_bwd():
        if layer.save_gu:
            L.moe_expert_ffn_backward_saved(cfg, layer.x_perm, x, layer.offsets, layer.weights, layer.saved,
                                            layer.dy_perm, dy, layer.dx_perm, layer.dx_shared, layer.grads,
                                            layer.ws_ffn_bwd)
        else:
            L.moe_expert_ffn_backward(cfg, layer.x_perm, x, layer.offsets, layer.weights, layer.dy_perm, dy,
                                      layer.dx_perm, layer.dx_shared, layer.grads, layer.ws_ffn_bwd)

    calls = [lambda: L.moe_combine_backward(cfg, dy, layer.y_perm, layer.inv, layer.topk_w, layer.dy_perm,
                                            layer.d_topk_w),
             ffn_bwd,
             lambda: L.moe_route_backward(cfg, x, layer.w_router, layer.scores, layer.topk_idx, layer.d_topk_w,
                                          alpha, seq_len, layer.dx_router, layer.g_w_router, layer.loss_bal,
                                          layer.ws_route_bwd),
             lambda: L.moe_dispatch_backward(cfg, layer.dx_perm, layer.dx_shared, layer.dx_router, layer.inv,
                                             layer.dx)]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        layer.forward(x, bias, gamma=c.gamma)
        for j, f in enumerate(calls):
            if ev is not None:
                ev[j + 1].record()
            f()
        if ev is not None:
            ev[len(calls) + 1].record()

    def timed():
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 2)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        fwd = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in events]))
        st = {n: float(np.mean([ev[j + 1].elapsed_time(ev[j + 2]) for ev in events]))
              for j, n in enumerate(BWD_STAGES)}
        return wall, fwd, st

    rows = c.T * (c.k + c.S)
    ffn_bwd_flops = 12 * c.H * c.I * rows            # dh 2HI, dx 4HI, dW_gu 4HI, dW_d 2HI per row
    router_bwd_flops = 4 * c.T * c.E * c.H
    fwd_flops = c.gate_up_flops() + c.down_flops() + c.router_flops()
    wall, fwd, st = timed()
    ffn_tf = ffn_bwd_flops / (st["expert_ffn_bwd"] * 1e-3) / 1e12
    out = {"workload": "v3_prefill_train_bf16", "T": c.T, "alpha": alpha, "seq_len": seq_len,
           "gate_up_outputs_kept": True,
           "ms_per_step": round(wall, 4), "tokens_per_s": round(c.T / (wall * 1e-3), 1),
           "forward_ms": round(fwd, 4), "backward_ms": round(sum(st.values()), 4),
           "backward_stages_ms": {k: round(v, 4) for k, v in st.items()},
           "expert_ffn_bwd_tflops": round(ffn_tf, 2), "expert_ffn_bwd_frac_of_peak": round(ffn_tf / PEAK_BF16_TFLOPS, 4),
           "step_tflops": round((fwd_flops + ffn_bwd_flops + router_bwd_flops) / (wall * 1e-3) / 1e12, 2),
           "loss_bal": float(layer.loss_bal.item())}
    layer.save_gu = False                            # the same step recomputing g, u in the backward pass
    wall_r, fwd_r, st_r = timed()
    out["recompute"] = {"ms_per_step": round(wall_r, 4), "forward_ms": round(fwd_r, 4),
                        "backward_ms": round(sum(st_r.values()), 4),
                        "expert_ffn_bwd_ms": round(st_r["expert_ffn_bwd"], 4)}
    del layer, x, dy
    torch.cuda.empty_cache()
    return out


def two_stream(c, w, reps=5):
    """Micro-batch overlap on one GPU: batch A's gate/up (then down) GEMM on one stream and
    batch B's memory-bound stages (dispatch with the row copy, then combine) on a second
    stream, against the same kernels one after the other.  Both batches share the weights."""
    import copy

    import numpy as np
    import torch

    from biased_top_routing_amd import _lib as L
    from biased_top_routing_amd.runner import MoeLayerGPU
    from workloads.inputs import make_x

    la = MoeLayerGPU(c, w, gather=False, keep_scores=False)
    lb = copy.copy(la)
    lb.alloc(c.T)
    xa, xb = to_dev(make_x(c, 0)), to_dev(make_x(c, 1))
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    for lay, x in ((la, xa), (lb, xb)):
        lay.forward(x, bias)
    torch.cuda.synchronize()
    s1 = torch.cuda.current_stream()
    s2 = torch.cuda.Stream()
    out = {}
    for gemm, phase in (("gate_up", L.MOE_FFN_GATE_UP), ("down", L.MOE_FFN_DOWN)):
        def gemm_a():
            la.expert_ffn(xa, phase)

        def mem_b():
            lb.dispatch(xb)
            lb.combine()

        def timed(fn):
            ts = []
            for _ in range(reps):
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return float(np.median(ts))

        t_gemm = timed(gemm_a)
        t_mem = timed(mem_b)

        def sequential():
            gemm_a()
            mem_b()

        def concurrent():
            s2.wait_stream(s1)
            gemm_a()
            with torch.cuda.stream(s2):
                mem_b()
            s1.wait_stream(s2)

        out[gemm] = {"gemm_ms": round(t_gemm, 4), "dispatch_combine_ms": round(t_mem, 4),
                     "sequential_ms": round(timed(sequential), 4), "two_streams_ms": round(timed(concurrent), 4)}
        log(f"two streams, {gemm}: {out[gemm]}")
    return {"workload": c.name, "T": c.T, "reps": reps, "stages": out,
            "note": "batch A's expert GEMM on the default stream, batch B's dispatch (row copy) + combine on a "
                    "second stream of the same priority; median of the repetitions"}


def gemm_probe(c, w, kind, reps=8):
    """The grouped expert GEMMs alone at the workload's routing (the real router on
    make_x(c, 0)), with expert weights drawn on the GPU: N(0, sigma) ("random") or all
    zero ("zero", the same instruction stream on operands that switch few bits, which
    shows how far the chip's power limit holds the clock down).  Also a dense
    hipBLASLt GEMM (torch.mm) of the gate/up shape for every token with its weights as
    [out, in] and as [in, out]."""
    import numpy as np
    import torch

    from biased_top_routing_amd import _lib as L
    from workloads.inputs import make_x

    dev = "cuda"

    def draw(n, rows, cols):
        t = torch.empty((n, rows, cols), dtype=torch.bfloat16, device=dev)
        for i in range(n):
            if kind == "zero":
                t[i].zero_()
            else:
                t[i].normal_(0.0, c.sigma)
        return t

    wgu, wd = draw(c.E, 2 * c.I, c.H), draw(c.E, c.H, c.I)
    sgu, sd = draw(c.S, 2 * c.I, c.H), draw(c.S, c.H, c.I)
    if c.wgt == "fp8_e4m3":
        q = []
        for t in (wgu, wd, sgu, sd):
            n, r, k = t.shape
            codes = torch.empty((n, r, k), dtype=torch.uint8, device=dev)
            sc = torch.empty((n, r // 128, k // 128), dtype=torch.float32, device=dev)
            if n:
                L.moe_quantize_fp8(t, n, r, k, 128, codes, sc)
            q.append((codes, sc))
        W = L.expert_weights(q[0][0], q[1][0], q[2][0], q[3][0], q[0][1], q[1][1], q[2][1], q[3][1])
    else:
        W = L.expert_weights(wgu, wd, sgu, sd)
    cfg = L.cfg_from(c)
    x = to_dev(make_x(c, 0))
    wr = to_dev(w.w_router)
    off = torch.from_numpy(w.logit_offset).to(dev) if w.logit_offset is not None else None
    bias = torch.from_numpy(w.bias0.copy()).to(dev)
    idx = torch.empty((c.T, c.k), dtype=torch.int32, device=dev)
    gw = torch.empty((c.T, c.k), dtype=torch.float32, device=dev)
    L.moe_route(cfg, x, wr, off, bias, torch.empty((c.T, c.E), device=dev), 0, idx, gw)
    counts = torch.empty(c.E, dtype=torch.int32, device=dev)
    offs = torch.empty(c.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(c.T * c.k, dtype=torch.int32, device=dev)
    inv = torch.empty((c.T, c.k), dtype=torch.int32, device=dev)
    wsd = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_DISPATCH), dtype=torch.uint8, device=dev)
    L.moe_dispatch(cfg, idx, None, counts, offs, perm, inv, None, None, wsd)
    yp = torch.empty((c.T * c.k, c.H), dtype=torch.bfloat16, device=dev)
    ys = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
    wsf = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_FFN), dtype=torch.uint8, device=dev)

    def run(ph):
        L.moe_expert_ffn_gather(cfg, x, perm, offs, W, yp, ys, wsf, ph)

    out = {"workload": c.name, "weights": kind, "reps": reps}
    for name, ph, flops in (("gate_up", L.MOE_FFN_GATE_UP, c.gate_up_flops()), ("down", L.MOE_FFN_DOWN, c.down_flops())):
        for _ in range(3):
            run(L.MOE_FFN_GATE_UP)
            run(ph)
        ts = []
        for _ in range(reps):
            if ph == L.MOE_FFN_DOWN:
                run(L.MOE_FFN_GATE_UP)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run(ph)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
        log(f"gemm probe ({kind}) {name}: {out[name]}")
    M, N, K = c.T * (c.k + c.S), 2 * c.I, c.H
    M = min(M, 32768)
    a = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    b_nk = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    b_kn = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    for t, sd_ in ((a, 1.0), (b_nk, c.sigma), (b_kn, c.sigma)):
        if kind == "zero":
            t.zero_()
        else:
            t.normal_(0.0, sd_)
    for name, f in (("hipblaslt_x_WT", lambda: torch.mm(a, b_nk.t())), ("hipblaslt_x_W", lambda: torch.mm(a, b_kn))):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"M": M, "N": N, "K": K, "ms": round(ms, 4), "tflops": round(2 * M * N * K / ms / 1e9, 1)}
        log(f"gemm probe ({kind}) {name}: {out[name]}")
    return out


def balance_trajectory(layer, c, w, steps, note=None):
    """Per-step expert load over `steps` consecutive batches of the layer with the bias
    update between them.  Batch i's x is make_x(c, i) from the shared seeded generator
    (the oracle can replay every step); per step the max/mean, min/mean and the
    coefficient of variation (std/mean) of the per-expert loads."""
    import numpy as np
    import torch

    from workloads.inputs import make_x
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    mean = c.T * c.k / c.E
    mx, mn, cv = [], [], []
    t0 = time.perf_counter()
    for step in range(steps):
        x = to_dev(make_x(c, step))
        layer.forward(x, bias, gamma=c.gamma)
        counts = layer.counts.cpu().numpy().astype(np.float64)
        mx.append(round(float(counts.max() / mean), 4))
        mn.append(round(float(counts.min() / mean), 4))
        cv.append(round(float(counts.std() / mean), 4))
        if step % 20 == 19:
            log(f"  balance step {step + 1}/{steps} ({time.perf_counter() - t0:.0f} s)")
    hot = int(np.argmax(counts))
    b_end = bias.cpu().numpy()
    out = {"steps": steps, "gamma": c.gamma, "x": "make_x(cfg, step): N(0,1) from the shared seeded generator",
           "max_over_mean": mx, "min_over_mean": mn, "cv": cv,
           "hottest_expert": hot, "hottest_expert_bias_start": float(w.bias0[hot]),
           "hottest_expert_bias_end": float(b_end[hot])}
    if note:
        out["note"] = note
    return out


def route_sweep(c, w, sizes=(16384, 65536, 262144), iters=10):
    """The route stage (router GEMM + sigmoid + biased group-limited top-k + gates) at
    several batch sizes, with a 512 MB write between launches so that no input is served
    from the 256 MB Infinity Cache: "route" without the [T, E] affinities (the forward
    pass; the fused kernel keeps them on chip), "route_scores" writing them (a training
    step's forward pass), and "topk" the selection alone on given affinities."""
    import torch

    from biased_top_routing_amd import _lib as L
    out = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    wr = to_dev(w.w_router)
    off = torch.from_numpy(w.logit_offset).cuda() if w.logit_offset is not None else None
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    for T in sizes:
        cfg = L.cfg_from(c, T=T)
        x = torch.randn(T, c.H, device="cuda").to(torch.bfloat16)
        scores = torch.empty(T, c.E, device="cuda")
        ws = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_ROUTE), dtype=torch.uint8, device="cuda")
        idx = torch.empty(T, c.k, dtype=torch.int32, device="cuda")
        gw = torch.empty(T, c.k, device="cuda")
        res = {}
        xw = T * c.H * 2 + c.E * c.H * 2
        sc = T * c.E * 4
        for name, flags, s_arg, nbytes in (("route", 0, None, xw),
                                           ("route_scores", 0, scores, xw + sc),
                                           ("topk", L.MOE_SCORES_IN, scores, sc)):
            nbytes += c.E * 4 + T * c.k * 8
            L.moe_route(cfg, x, wr, off, bias, s_arg, flags, idx, gw, ws)
            ms = []
            for _ in range(iters):
                flush.fill_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                L.moe_route(cfg, x, wr, off, bias, s_arg, flags, idx, gw, ws)
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            t = sorted(ms)[len(ms) // 2]
            res[name] = {"ms": round(t, 4), "gbs": round(nbytes / (t * 1e-3) / 1e9, 1), "bytes": nbytes}
        out[str(T)] = res
        del x, scores, idx, gw, ws
    del flush
    torch.cuda.empty_cache()
    return out


def permute_copy(c, w, x, iters=10):
    """The dispatch with the row copy (counts, offsets, perm, inv and x_perm[p] =
    x[perm[p] / k]) on the routing of x [T, H], with a 512 MB write between
    launches: the permute as a memory-bound stage of its own (the default path folds
    the copy into the gate/up GEMM's loads)."""
    import torch

    from biased_top_routing_amd import _lib as L
    cfg = L.cfg_from(c)
    dev = "cuda"
    if tuple(x.shape) != (c.T, c.H):
        raise ValueError(f"permute_copy: x is {tuple(x.shape)}, the workload needs {(c.T, c.H)}")
    idx = torch.empty((c.T, c.k), dtype=torch.int32, device=dev)
    gw = torch.empty((c.T, c.k), dtype=torch.float32, device=dev)
    wsr = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_ROUTE), dtype=torch.uint8, device=dev)
    off = torch.from_numpy(w.logit_offset).to(dev) if w.logit_offset is not None else None
    L.moe_route(cfg, x, to_dev(w.w_router), off, torch.from_numpy(w.bias0.copy()).to(dev), None, 0, idx, gw, wsr)
    counts = torch.empty(c.E, dtype=torch.int32, device=dev)
    offs = torch.empty(c.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(c.T * c.k, dtype=torch.int32, device=dev)
    inv = torch.empty((c.T, c.k), dtype=torch.int32, device=dev)
    xp = torch.empty((c.T * c.k, c.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_DISPATCH), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    L.moe_dispatch(cfg, idx, x, counts, offs, perm, inv, xp, None, ws)
    ms = []
    for _ in range(iters):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.moe_dispatch(cfg, idx, x, counts, offs, perm, inv, xp, None, ws)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    t = sorted(ms)[len(ms) // 2]
    nbytes = stage_bytes(c, gather=False)["dispatch"]
    del xp, flush
    torch.cuda.empty_cache()
    return {"ms": round(t, 4), "gbs": round(nbytes / (t * 1e-3) / 1e9, 1), "bytes": nbytes,
            "frac_of_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def small_workload(name, steps, warmup, balance_steps, gather=False):
    """One of the small configurations (tiny fp32, mid bf16): per-step time, rates, and
    the per-step load series over `balance_steps` batches with the bias update between
    them (balance_trajectory)."""
    import torch

    from biased_top_routing_amd.runner import MoeLayerGPU
    from workloads import CONFIGS
    from workloads.inputs import make_weights, make_x
    c = CONFIGS[name]
    w = make_weights(c)
    layer = MoeLayerGPU(c, w, gather=gather, keep_scores=False)
    x = to_dev(make_x(c, 0))
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    ms, stage_ms = time_layer(layer, x, bias, c, steps, warmup)
    flops = c.gate_up_flops() + c.down_flops() + c.router_flops()
    peak = 157.3 if c.act == "f32" else PEAK_BF16_TFLOPS   # fp32 vector (no MFMA used) / bf16 MFMA
    out = {"workload": c.name, "T": c.T, "ms_per_step": round(ms, 4), "tokens_per_s": round(c.T / (ms * 1e-3), 1),
           "pairs_per_s": round(c.T * c.k / (ms * 1e-3), 1),
           "layer_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
           "layer_frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / peak, 4),
           "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()}}
    out["balance"] = balance_trajectory(layer, c, w, balance_steps)
    return out


def gemm_summary(c, ms_per_step, stage_ms):
    peak = PEAK_FP8_TFLOPS if c.wgt == "fp8_e4m3" else PEAK_BF16_TFLOPS
    gu = c.gate_up_flops() / (stage_ms["gate_up"] * 1e-3) / 1e12
    dn = c.down_flops() / (stage_ms["down"] * 1e-3) / 1e12
    return peak, gu, dn


def to_dev(a):
    from biased_top_routing_amd.runner import to_device
    return to_device(a)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the layer library has no multi-GPU path; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from biased_top_routing_amd import _lib as L
    from biased_top_routing_amd.runner import MoeLayerGPU
    from workloads import CONFIGS
    from workloads.inputs import make_weights, make_x

    L.lib()     # fails loudly without the built library
    c = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    if args.gemm_probe:
        from workloads.inputs import make_router
        print(json.dumps(gemm_probe(c, make_router(c), args.gemm_probe)), flush=True)
        return
    log(f"workload {c.name}: generating seeded inputs")
    t0 = time.perf_counter()
    w = make_weights(c)
    xh = make_x(c, 0)
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s; uploading")
    if args.train_only:
        print(json.dumps(train_extra(c, w, args.steps, args.warmup)), flush=True)
        return
    if args.two_stream:
        print(json.dumps(two_stream(c, w, max(args.steps, 3))), flush=True)
        return
    gather = args.dispatch == "gather"
    layer = MoeLayerGPU(c, w, gather=gather, keep_scores=False)
    x = to_dev(xh)
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    torch.cuda.synchronize()
    log(f"uploaded; timing {args.steps} steps after {args.warmup} warm-up steps (dispatch: {args.dispatch})")
    ms_per_step, stage_ms = time_layer(layer, x, bias, c, args.steps, args.warmup)
    value = c.T / (ms_per_step * 1e-3)
    counts = layer.counts.cpu().numpy()
    log(f"{ms_per_step:.3f} ms/step, {value:,.0f} tokens/s; stages {stage_ms}")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n} bytes")
        del src, dst

    peak, gu_tflops, dn_tflops = gemm_summary(c, ms_per_step, stage_ms)
    total_flops = c.gate_up_flops() + c.down_flops() + c.router_flops()
    b = stage_bytes(c, gather, scores=layer.keep_scores)
    route_gbs = (b["router"] + b["topk"]) / (stage_ms["route"] * 1e-3) / 1e9
    fp8 = c.wgt == "fp8_e4m3"
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 experts, bf16 router" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": c.name, "T": c.T, "H": c.H, "E": c.E, "G": c.G, "M": c.M, "k": c.k, "S": c.S,
                   "I": c.I, "route_scale": c.route_scale, "parallelism": "single-gpu",
                   "dispatch": args.dispatch},
        "roofline": {
            "kernel": ("gemm_fp8_kernel<gate_up>" if fp8 else "gemm_bf16_kernel<gate_up>") +
                      " (routed + shared gate/up GEMM with fused SwiGLU)",
            "bound": "mfma",
            "achieved": round(gu_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(gu_tflops / peak, 4),
            "traffic": None if fp8 else measured_traffic(c.name),
            "flops_per_launch": c.gate_up_flops(),
            "avg_launch_ms": round(stage_ms["gate_up"], 4),
        },
        "pairs_per_s": round(c.T * c.k / (ms_per_step * 1e-3), 1),
        "stages": {
            "ms": {k: round(v, 4) for k, v in stage_ms.items()},
            "gate_up_tflops": round(gu_tflops, 2),
            "layer_frac_of_peak": round(total_flops / (ms_per_step * 1e-3) / 1e12 / peak, 4),
            "down_tflops": round(dn_tflops, 2),
            "layer_tflops": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2),
            "route_gbs": round(route_gbs, 1),
            "dispatch_gbs": round(b["dispatch"] / (stage_ms["dispatch"] * 1e-3) / 1e9, 1),
            "combine_gbs": round(b["combine"] / (stage_ms["combine"] * 1e-3) / 1e9, 1),
            "hbm_peak_gbs": PEAK_HBM_GBS,
            "max_over_mean_load": round(float(counts.max() / (c.T * c.k / c.E)), 3),
        },
    }
    if not args.no_extras and c.name == "v3_prefill_bf16":
        extras = {}
        log("extra: the same layer at decode size")
        extras["v3_decode_bf16"] = decode_extra(layer, c, w, max(args.steps, 20), args.warmup)
        log("extra: route stage at several batch sizes (cache flushed between launches)")
        extras["route_sweep"] = route_sweep(c, w)
        log("extra: dispatch with the row copy (the permute as a stage of its own)")
        extras["permute_copy"] = permute_copy(c, w, x)
        del layer, x
        torch.cuda.empty_cache()
        log("extra: one training step (forward + backward) at the prefill shape")
        extras["v3_prefill_train_bf16"] = train_extra(c, w, max(args.steps // 2, 5), 2)
        cf = CONFIGS["v3_fp8"]
        log("extra: the FP8 layer (T=32768, Zipf-skewed routing)")
        wf = make_weights(cf)
        lf = MoeLayerGPU(cf, wf, gather=gather, keep_scores=False)
        xf = to_dev(make_x(cf, 0))
        bf = torch.from_numpy(wf.bias0.copy()).cuda()
        msf, stf = time_layer(lf, xf, bf, cf, args.steps, args.warmup)
        pk, gu8, dn8 = gemm_summary(cf, msf, stf)
        cnt = lf.counts.cpu().numpy()
        extras["v3_fp8"] = {"workload": cf.name, "T": cf.T, "ms_per_step": round(msf, 4),
                            "tokens_per_s": round(cf.T / (msf * 1e-3), 1),
                            "pairs_per_s": round(cf.T * cf.k / (msf * 1e-3), 1),
                            "gate_up_tflops": round(gu8, 2), "gate_up_frac_fp8_peak": round(gu8 / pk, 4),
                            "down_tflops": round(dn8, 2), "down_frac_fp8_peak": round(dn8 / pk, 4),
                            "layer_tflops": round((cf.gate_up_flops() + cf.down_flops() + cf.router_flops()) /
                                                  (msf * 1e-3) / 1e12, 2),
                            "max_over_mean_load": round(float(cnt.max() / (cf.T * cf.k / cf.E)), 3),
                            "stages_ms": {k: round(v, 4) for k, v in stf.items()}}
        log("extra: FP8 layer, 100 batches with the bias update between them")
        extras["v3_fp8"]["balance"] = balance_trajectory(
            lf, cf, wf, cf.steps,
            note=("with Zipf(1.5) logit offsets the hottest experts' offsets (up to +4.6) dwarf what "
                  "100 steps of gamma = 1e-3 can move (0.1), so every token keeps choosing them and "
                  "max/mean stays at T / (T k / E) = E / k = 32; the bias of each such expert falls by "
                  "gamma every step"))
        del lf, xf
        torch.cuda.empty_cache()
        for name in ("tiny_fp32", "mid_bf16"):
            log(f"extra: {name}")
            cs = CONFIGS[name]
            extras[name] = small_workload(name, 50, 5, cs.steps, gather)
        out["other_workloads"] = extras
    if not args.no_cpu_baseline and not fp8:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(c, xh, w, w.bias0, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
