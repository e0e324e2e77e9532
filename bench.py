"""Benchmark of one NVFP4 routed-MoE layer on one MI355X.

A step is the whole hot path on one batch of seeded synthetic input:
moe_route -> nvfp4_quant -> moe_experts_fwd -> moe_finalize, replayed from HIP
graphs of 16 consecutive steps (as a model's forward pass holds its layers
back to back in one graph; the steps past a multiple of 16 one to a graph).
``ms_per_step_one_per_graph`` replays every step from a graph of its own,
which adds a graph launch to each. Each step has its own weight copy: the
weights rotate over enough copies (>= 1 GiB)
that the 256 MB Infinity Cache cannot hold them between uses, so weight bytes
come from HBM (the cold-cache timing the flashinfer_ops page's tuning
configuration asks for). Inputs are resident in HBM before timing starts.

Prints one JSON line. The headline workload is prefill_t4096 (the largest
single-GPU configuration: T=4096, H=4096, I=1536, E=128, top-8); the same line
carries a sub-record under ``workloads`` for each decode configuration
(decode_b8, decode_b64_zipf, expert_tp8_b32), each measured the same way with
its own roofline. ``roofline`` is the dominant kernel (the experts step),
timed with HIP events on its own stream: ``kernel_ms`` over 16 consecutive
steps replayed from one graph (back to back, as the layer runs them), and
``kernel_ms_isolated`` one step at a time behind a sleep kernel, which adds a
launch's dispatch to each. With few routes per expert (decode)
it is bound by HBM: algorithmic bytes per launch (codes + e4m3 scales of the
experts that have a route, the NVFP4 input read once, the NVFP4 intermediate
written and re-read, the GEMM2 rows written) over its average duration. With
many (prefill, the register-tiled kernels) it is bound by the matrix cores:
the routed rows' GEMM FLOPs over the duration, against the f16 MFMA peak. ``cpu_baseline`` is the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload prefill_t4096]
                    [--sub-workloads decode_b8,decode_b64_zipf,expert_tp8_b32]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import math
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill_t4096")
    ap.add_argument("--sub-workloads", default="decode_b8,decode_b64_zipf,expert_tp8_b32",
                    help="comma-separated workloads measured into the line's 'workloads' record ('' for none)")
    ap.add_argument("--sub-steps", type=int, default=400,
                    help="timed layer replays of each sub-workload (at least --steps)")
    ap.add_argument("--cpu-tokens", type=int, default=512,
                    help="tokens of the headline workload in the oracle's CPU-baseline sample (0 disables)")
    ap.add_argument("--rotate-bytes", type=float, default=1.0e9)
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the layer step and the expert step, none of the neighbouring calls "
                         "(for counter runs, whose per-dispatch figures then hold only the step's kernels)")
    return ap.parse_args()


HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # MI355X dense f16 matrix peak
LAYER_GROUP = 16                  # layer steps a timed graph holds
MFMA_F64_PEAK_TFLOPS = 78.6       # MI355X fp64 peak (matrix and vector)
ROOT = os.path.dirname(os.path.abspath(__file__))


def measured_traffic(workload: str):
    """HBM bytes per expert step from the committed PMC summary
    (profiles/experts_<workload>_traffic.json), or None when there is none or
    when the kernel sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"experts_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return float(rec["traffic_bytes"]) if h.hexdigest() == rec["sources_sha256"] else None


def mfma_bound(wl) -> bool:
    """Whether moe_experts_fwd takes the register-tiled MFMA kernels (many routes
    per expert; the library's dispatch rule): then the step is bound by the
    matrix cores and its roofline is f16 MFMA throughput."""
    I_part = wl.I // wl.tp
    return (wl.tile_m % 128 == 0 and wl.H % 256 == 0 and I_part % 256 == 0
            and wl.T * (wl.H // 2) < 2 ** 31 and wl.T * wl.K >= 32 * wl.E)


def algorithmic_flops(wl, counts) -> float:
    """Matrix FLOPs of the routed rows: GEMM1 (2I x H) and GEMM2 (H x I) per route."""
    routes = int(counts.sum())
    return 2.0 * routes * (2 * wl.I * wl.H + wl.H * wl.I)


def algorithmic_bytes(wl, counts, finalize: bool = False) -> dict:
    """Bytes the experts step must move at least once per call (per layer step:
    all expert-TP slices). finalize: the step also finalizes (moe_experts_finalize),
    reading every slice's rows once more and writing the bf16 output."""
    touched = int((counts > 0).sum())
    H, I = wl.H, wl.I
    per_expert = 2 * I * H // 2 + 2 * I * H // 16 + H * I // 2 + H * I // 16   # 27/16 I H
    routes = int(counts.sum())
    act = wl.tp * wl.T * (H // 2 + H // 16)                # NVFP4 input, read once a slice
    inter = 2 * routes * (I // 2 + I // 16)                # NVFP4 intermediate, written and read
    rows = wl.tp * routes * H * 2                          # GEMM2 bf16 rows written, one partial a slice
    fin = (wl.tp * routes * H * 2 + wl.T * H * 2) if finalize else 0   # rows read, output written
    other = act + inter + rows + fin
    return dict(weights=touched * per_expert, touched=touched, other=other,
                total=touched * per_expert + other)


def time_norm_quant(N, x, norm_w, gscale, wl, n: int) -> dict:
    """The pre-expert RMSNorm + NVFP4 quantizer (nvfp4_norm_quant) on the
    workload's activations, event-timed on its stream: 2H bytes read and 9H/16
    written per row (the norm weight, 2H bytes, is read once and cached)."""
    import torch
    T, H = wl.T, wl.H
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device=x.device)
    sf = torch.empty((T, H // 16), dtype=torch.uint8, device=x.device)
    us, us_iso = _event_us(lambda s: N.nvfp4_norm_quant(x, norm_w, 1.0, 1e-6, gscale, codes, sf, s), n)
    nbytes = T * (2 * H + H // 2 + H // 16) + 2 * H
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": us, "us_isolated": us_iso, "bytes": nbytes, "achieved": gbs, "unit": "GB/s",
            "peak": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS, "bound": "hbm" if T >= 1024 else "latency"}


def _event_us(fn, n: int, group: int = 16):
    """Event-timed duration of fn(stream) in microseconds, as (back to back,
    isolated): 16 consecutive calls captured in one graph and replayed between
    two events, and single calls each between two events; a sleep kernel ahead
    of every timed region keeps host enqueue time out of it, and the isolated
    figure also holds one launch's dispatch."""
    import torch
    s = torch.cuda.current_stream()
    for _ in range(3):
        fn(s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        torch.cuda._sleep(20000)
        a.record(s)
        fn(s)
        b.record(s)
    torch.cuda.synchronize()
    iso = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for _ in range(group):
            fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    evg = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(4, n // group))]
    for a, b in evg:
        torch.cuda._sleep(20000)
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    batched = float(np.mean([a.elapsed_time(b) for a, b in evg])) * 1e3 / group
    del g
    return batched, iso


def time_router(N, W, wl, bufs, n: int) -> dict:
    """The router logits (fp32 [T, D] x [E, D], D = H) alone and the full
    routing chain (logits, then moe_route into the layer's buffers). Bytes:
    the input, the weight and the logits, each moved once."""
    import torch
    xr, wr = W.make_router_inputs(wl)
    x = torch.from_numpy(xr).to(bufs.ids.device)
    w = torch.from_numpy(wr).to(bufs.ids.device)
    logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device=x.device)
    us_l, iso_l = _event_us(lambda s: N.moe_router_logits(x, w, logits, s), n)
    us_c, iso_c = _event_us(lambda s: N.moe_router_route(x, w, None, None, wl.K, 1.0, wl.tile_m, 0, wl.E, logits,
                                                          bufs.ids, bufs.weights, bufs.meta, s), n)
    nbytes = 4 * (wl.T * wl.H + wl.E * wl.H + wl.T * wl.E)
    if wl.T > 256:      # the tiled kernel: fp64 matrix products, 2 T E D flops
        flops = 2.0 * wl.T * wl.E * wl.H
        tfs = flops / (us_l * 1e-6) / 1e12
        logits_rec = {"us": us_l, "us_isolated": iso_l, "flops": flops, "bytes": nbytes, "achieved": tfs,
                      "unit": "TFLOP/s",
                      "peak": MFMA_F64_PEAK_TFLOPS, "frac": tfs / MFMA_F64_PEAK_TFLOPS, "bound": "mfma fp64"}
    else:
        gbs = nbytes / (us_l * 1e-6) / 1e9
        logits_rec = {"us": us_l, "us_isolated": iso_l, "bytes": nbytes, "achieved": gbs, "unit": "GB/s",
                      "peak": HBM_PEAK_GBS,
                      "frac": gbs / HBM_PEAK_GBS, "bound": "hbm"}
    return {"moe_router_logits": logits_rec, "moe_router_route": {"us": us_c, "us_isolated": iso_c}}


def time_w4a16(N, wl, x, bufs, weights, ab: dict, n: int) -> dict:
    """The W4A16 expert step (bf16 activations, the same NVFP4 weights) on the
    layer's routing, weight copies rotated as in the main measurement: the same
    weight bytes, plus bf16 activations and a bf16 intermediate."""
    import torch
    L = bufs.layout
    inter = torch.empty((L.rows_max, wl.I), dtype=torch.int16, device=x.device)
    k = [0]

    def call(s):
        w = weights[k[0] % len(weights)]
        k[0] += 1
        N.moe_experts_fwd_w4a16(x, bufs.meta, w, wl.T, wl.K, wl.E, wl.H, wl.I, wl.tile_m, inter, bufs.rows[0], s)

    us, us_iso = _event_us(call, n)
    routes = wl.T * wl.K
    nbytes = ab["weights"] + wl.T * wl.H * 2 + 2 * routes * wl.I * 2 + routes * wl.H * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": us, "us_isolated": us_iso, "bytes": nbytes, "achieved": gbs, "unit": "GB/s",
            "peak": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS, "bound": "hbm"}


def time_bf16(N, W, wl, x, bufs, counts, n: int) -> dict:
    """The BF16 expert layers' GEMMs (bf16 weights: 6 I H bytes per expert) on
    the layer's routing; two weight copies alternate so that the 256 MB
    Infinity Cache does not hold the next call's weights."""
    import torch
    w13h, w2h = W.make_bf16_weights(wl)
    dev = x.device
    copies = [(torch.from_numpy(w13h.view(np.int16)).to(dev), torch.from_numpy(w2h.view(np.int16)).to(dev))
              for _ in range(2)]
    del w13h, w2h
    inter = torch.empty((bufs.layout.rows_max, wl.I), dtype=torch.int16, device=dev)
    k = [0]

    def call(s):
        w13, w2 = copies[k[0] % 2]
        k[0] += 1
        N.moe_experts_fwd_bf16(x, bufs.meta, w13, w2, wl.T, wl.K, wl.E, wl.H, wl.I, wl.tile_m, inter,
                               bufs.rows[0], s)

    us, us_iso = _event_us(call, n)
    routes = wl.T * wl.K
    touched = int((counts > 0).sum())
    nbytes = touched * 6 * wl.I * wl.H + wl.T * wl.H * 2 + 2 * routes * wl.I * 2 + routes * wl.H * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    del copies
    torch.cuda.empty_cache()
    return {"us": us, "us_isolated": us_iso, "bytes": nbytes, "achieved": gbs, "unit": "GB/s",
            "peak": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS, "bound": "hbm"}


def cpu_baseline(inp, n_tokens: int) -> dict:
    """The CPU oracle (as it stands: numpy fp64, exact GEMMs) on the first
    n_tokens tokens of the workload, the whole layer for those tokens (quantizer,
    routing, both GEMMs, finalize), with numpy's BLAS on all the threads it uses
    and again on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle.layer import layer_sampled
    wl = inp.wl
    tokens = np.arange(min(n_tokens, wl.T))
    t0 = time.perf_counter()
    ref = layer_sampled(inp, tokens)
    dt = time.perf_counter() - t0
    routes = int(ref["served"].sum())
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    with threadpool_limits(1):
        t0 = time.perf_counter()
        layer_sampled(inp, tokens)
        dt1 = time.perf_counter() - t0
    return {"value": routes / dt, "unit": "routed rows/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt, "single_thread": {"value": routes / dt1, "seconds": dt1, "cores": 1},
            "sample": f"the whole layer of {wl.name} for its first {len(tokens)} tokens ({routes} routes): "
                      f"{dt:.1f} s with numpy's BLAS on {threads} threads (the NVFP4 dequantization is "
                      f"single-threaded numpy), {dt1:.1f} s on one thread"}


def measure(N, LY, W, name: str, steps: int, warmup: int, rotate_bytes: float, extras: bool) -> dict:
    """One workload: the layer step replayed from graphs (steps timed), the expert
    step timed by events with its roofline, the metadata's sync words checked
    after the timed replays, and (extras) the neighbouring calls."""
    import torch
    dev = "cuda:0"
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl)

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    g1a, g1c, g2a = t(inp.g1_alphas), t(inp.g1_scale_c), t(inp.g2_alphas)
    logical = [t(inp.w13_codes), t(inp.w13_sf), t(inp.w2_codes), t(inp.w2_sf)]
    wbytes = sum(x.numel() for x in logical)
    copies = max(4, int(np.ceil(rotate_bytes / wbytes)))
    weights = [LY.pack_weights(*logical, g1a, g1c, g2a) for _ in range(copies)]
    del logical
    N.moe_validate_weights(weights[0], wl.E, wl.H, wl.I, wl.tp)
    x, gscale, logits = t(inp.x_bf16), t(inp.a1_gscale), t(inp.logits)
    norm_w = t(inp.norm_weight_bf16)
    shape = LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m, wl.tp)
    bufs = LY.Buffers(shape, dev)

    def step(w, stream=None):
        sl = None if wl.tp == 1 else [LY.slice_weights(w, r, wl.tp, wl.H, wl.I) for r in range(wl.tp)]
        LY.run_layer(bufs, x, gscale, logits, None, None, w, norm_w, wl.gain_center, wl.eps,
                     bool(wl.weight_before_norm), slices=sl, stream=stream)

    # eager warm-up, then the graphs, captured on a side stream: one per weight
    # copy holding one layer step, and graphs of LAYER_GROUP consecutive steps,
    # weight copies rotating, as a model's forward pass holds its layers back
    # to back in one graph
    for i in range(3):
        step(weights[i % copies])
    torch.cuda.synchronize()
    bufs.check_sync()
    cap = torch.cuda.Stream()
    graphs = []
    for w in weights:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(w)
        graphs.append(g)
    q, r = divmod(steps, LAYER_GROUP)
    gsteps = []
    for k in range(copies // math.gcd(LAYER_GROUP, copies) if q else 0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for j in range(LAYER_GROUP):
                step(weights[(k * LAYER_GROUP + j) % copies])
        gsteps.append(g)
    torch.cuda.synchronize()

    # the dominant kernel, timed with HIP events on the stream it is launched on
    counts = bufs.meta[bufs.layout.expert_counts:bufs.layout.expert_counts + wl.E].cpu().numpy()
    ab = algorithmic_bytes(wl, counts)
    s = torch.cuda.current_stream()
    n_k = min(max(steps, 64), 400)
    I_part = wl.I // wl.tp

    def expert_step(i, stream, finalize=False):
        """The layer's expert launches: every slice's moe_experts_fwd; with finalize
        the last one is moe_experts_finalize (the finalize in the same launch)."""
        w = weights[i % copies]
        sl = [w] if wl.tp == 1 else [LY.slice_weights(w, r, wl.tp, wl.H, wl.I) for r in range(wl.tp)]
        for r, ww in enumerate(sl):
            if finalize and r == len(sl) - 1:
                N.moe_experts_finalize(bufs.a_codes, bufs.a_sf, bufs.meta, ww, wl.T, wl.K, wl.E, wl.H, I_part,
                                       wl.tile_m, bufs.inter_codes, bufs.inter_sf, bufs.rows, len(sl),
                                       bufs.rows.stride(0), bufs.weights, norm_w, wl.gain_center, wl.eps,
                                       bool(wl.weight_before_norm), bufs.out, stream)
            else:
                N.moe_experts_fwd(bufs.a_codes, bufs.a_sf, bufs.meta, ww, wl.T, wl.K, wl.E, wl.H,
                                  I_part, wl.tile_m, bufs.inter_codes, bufs.inter_sf, bufs.rows[r], stream)

    # (1) one step at a time, a sleep kernel ahead of each so that host enqueue
    # time stays out: the step's duration plus one launch's dispatch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_k)]
    for i in range(n_k):
        torch.cuda._sleep(20000)
        ev[i][0].record(s)
        expert_step(i, s)
        ev[i][1].record(s)
    torch.cuda.synchronize()
    k_ms_isolated = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # (2) 16 consecutive steps (weight copies rotating) captured in one graph and
    # replayed between two events: the launches run back to back, as the
    # layer's do, and the per-step figure is the kernel's own duration plus the
    # gap between consecutive launches
    group = 16
    g_steps = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_steps, stream=cap):
        for j in range(group):
            expert_step(j, torch.cuda.current_stream())
    torch.cuda.synchronize()
    g_steps.replay()
    torch.cuda.synchronize()
    n_g = max(4, n_k // group)
    evg = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_g)]
    for a, b in evg:
        torch.cuda._sleep(20000)
        a.record(s)
        g_steps.replay()
        b.record(s)
    torch.cuda.synchronize()
    bufs.check_sync()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evg])) / group
    achieved = ab["total"] / (k_ms * 1e-3) / 1e9

    # the layer steps: `warmup` untimed replays, then the timed region (after
    # the expert-step timing above, so that the chip is at its working clock)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()

    def timed(replays):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for g in replays:
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    # timed region: `steps` whole-layer steps, LAYER_GROUP to a replay (the
    # rest one to a replay); then the same steps one to a replay, each of which
    # then also pays a graph launch
    ms_per_step = timed([gsteps[i % len(gsteps)] for i in range(q)] +
                        [graphs[(q * LAYER_GROUP + i) % copies] for i in range(r)]) / steps
    ms_single = timed([graphs[i % copies] for i in range(steps)]) / steps
    bufs.check_sync()            # no wait gave up: the timed steps computed valid rows

    routes = wl.T * wl.K
    rec = {
        "value": routes / (ms_per_step * 1e-3), "unit": "routed rows/s", "ms_per_step": ms_per_step,
        "steps": steps, "warmup": warmup, "steps_per_graph": LAYER_GROUP if q else 1,
        "ms_per_step_one_per_graph": ms_single,
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "K": wl.K,
                   "tp": wl.tp, "tile_m": wl.tile_m, "weight_copies": copies},
    }
    traffic = measured_traffic(wl.name)
    unit_t = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    if mfma_bound(wl):
        flops = algorithmic_flops(wl, counts)
        tflops = flops / (k_ms * 1e-3) / 1e12
        rec["roofline"] = {"bound": "mfma", "kernel": "moe_experts_fwd (tiled_fused_kernel: GEMM1+SwiGLU+requant "
                                                      "and GEMM2 in one launch)",
                           "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": traffic, "traffic_unit": unit_t,
                           "algorithmic_flops": flops, "algorithmic_bytes": ab["total"], "hbm_gbs": achieved,
                           "kernel_ms": k_ms, "kernel_ms_isolated": k_ms_isolated}
    else:
        launches = "" if wl.tp == 1 else f"; {wl.tp} slice launches a step, figures per step"
        rec["roofline"] = {"bound": "hbm", "kernel": "moe_experts_fwd (experts_fused_kernel: GEMM1+SwiGLU+requant "
                                                     f"and GEMM2 in one launch{launches})",
                           "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "traffic_unit": unit_t,
                           "algorithmic_bytes": ab["total"], "weight_bytes": ab["weights"],
                           "experts_touched": ab["touched"], "kernel_ms": k_ms,
                           "kernel_ms_isolated": k_ms_isolated}
    if extras and not mfma_bound(wl):
        # the expert step with the finalize in its launch (moe_experts_finalize),
        # against the expert step followed by moe_finalize, back to back
        def with_fin(s_):
            with_fin.i += 1
            expert_step(with_fin.i, s_, finalize=True)
        with_fin.i = 0

        def then_fin(s_):
            then_fin.i += 1
            expert_step(then_fin.i, s_)
            N.moe_finalize(bufs.rows, wl.tp, bufs.rows.stride(0), bufs.exp2perm, bufs.weights, norm_w,
                           wl.gain_center, wl.eps, bool(wl.weight_before_norm), wl.T, wl.K, wl.H, bufs.out, s_)
        then_fin.i = 0
        us_f, iso_f = _event_us(with_fin, min(n_k, 128))
        us_s, iso_s = _event_us(then_fin, min(n_k, 128))
        bufs.check_sync()
        rec["finalize_in_launch"] = {"moe_experts_finalize_us": us_f, "moe_experts_finalize_us_isolated": iso_f,
                                     "moe_experts_fwd_then_moe_finalize_us": us_s,
                                     "moe_experts_fwd_then_moe_finalize_us_isolated": iso_s}
    if extras:
        extra = {"nvfp4_norm_quant": time_norm_quant(N, x, norm_w, gscale, wl, n_k)}
        if wl.tp == 1 and not mfma_bound(wl):      # on the layer's routing, before the router rewrites it
            extra["moe_experts_fwd_w4a16"] = time_w4a16(N, wl, x, bufs, weights, ab, n_k)
            if wl.E * 3 * wl.H * wl.I * 2 <= 1 << 30:   # bf16 weights of at most 1 GiB
                extra["moe_experts_fwd_bf16"] = time_bf16(N, W, wl, x, bufs, counts, n_k)
        extra.update(time_router(N, W, wl, bufs, n_k))
        rec["extra_kernels"] = extra
    del graphs, gsteps, g_steps, weights, bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, inp


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path: expert TP is reproduced sequentially on one GPU.", file=sys.stderr)
        sys.exit(2)
    from nvfp4_block_scaled_route_amd import layer as LY
    from nvfp4_block_scaled_route_amd import native as N
    from nvfp4_block_scaled_route_amd import workloads as W

    N.lib()
    head, inp = measure(N, LY, W, args.workload, args.steps, args.warmup, args.rotate_bytes, not args.no_extras)
    out = {
        "metric": "routed rows/s per MoE layer; HBM GB/s (decode) & MFMA util (prefill) vs peak",
        "value": head["value"],
        "unit": "routed rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "steps_per_graph": head["steps_per_graph"], "ms_per_step_one_per_graph": head["ms_per_step_one_per_graph"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "extra_kernels": head.get("extra_kernels", {}),
    }
    subs = [w for w in args.sub_workloads.split(",") if w and w != args.workload]
    if subs:
        out["workloads"] = {}
        for name in subs:
            rec, _ = measure(N, LY, W, name, max(args.steps, args.sub_steps), max(args.warmup, 20),
                             args.rotate_bytes, name != "expert_tp8_b32" and not args.no_extras)
            out["workloads"][name] = rec
    if args.cpu_tokens > 0:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
