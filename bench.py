#!/usr/bin/env python3
"""Throughput of the GLM-5.2 MoE feed-forward layer on one MI355X.

One step = one full layer call (router, top-k, permutation, grouped gate/up,
grouped down, shared expert + combine) on a batch of seeded synthetic tokens
with GLM-5.2 shapes (hidden 6144, 256 routed experts, top-8, expert width
2048, one shared expert of width 2048, bf16 weights, fp32 router).  Weights and
inputs are resident in HBM before timing starts.

Prints one JSON line: the 8192-token prefill throughput (tokens/s) with the
roofline of its dominant kernel, the 64-token decode step as a second record,
and the CPU oracle timed on a bounded sample of the prefill batch.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s @GLM-5.2 shape (T=64 decode, T=8192 prefill); % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_CLOCK_MHZ = 2400.0     # engine clock of the published MFMA peaks
TRAFFIC = os.path.join(ROOT, "profiles", "traffic_gate_up_glm.json")
KERNEL_SOURCES = ("gemm_bf16.hip", "common.h", "permute.hip", "glm_moe.hip")


def kernel_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_moe_transformer_glm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kind):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC) as fh:
            d = json.load(fh)
    except OSError:
        return None
    if d.get("kernel_source_sha256") != kernel_source_sha() or kind not in d:
        return None
    return d[kind]["hbm_bytes_per_launch"]


def measured_peaks(torch):
    """Hardware ceilings measured on this GPU before the layer runs
    (libglm_peaks.so): bf16 and fp8 MFMA loops with the shader clock each
    observed, the 256 x 256 prefill tile's K step with its operands in L2
    (MFMAs only, copies only, both with the fragment reads, both with the
    copies spread over the step as the prefill kernel issues its weight
    copies, copies and MFMAs without the reads, reads and MFMAs without the
    copies, MFMAs with the copies moved through registers; each also in
    shader-clock cycles), and a streaming read of 8 GiB
    (far above the last-level cache)."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "sparse_moe_transformer_glm_amd", "libglm_peaks.so"))
    vp, i32, f32p, f64p = (ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                           ctypes.POINTER(ctypes.c_double))
    L.glm_peak_mfma.argtypes = [i32, i32, i32, vp, f32p, f64p, f64p, vp]
    L.glm_peak_hbm_read.argtypes = [vp, ctypes.c_size_t, i32, vp, f32p, vp]
    stream = torch.cuda.current_stream().cuda_stream
    scratch = torch.empty(16 + 4096 * 512 * 4, dtype=torch.uint8, device="cuda")
    res = {}
    for name, fp8 in (("bf16", 0), ("fp8", 1)):
        ms, flops, mhz = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
        st = L.glm_peak_mfma(fp8, 100000, 2, scratch.data_ptr(), ctypes.byref(ms),
                             ctypes.byref(flops), ctypes.byref(mhz), stream)
        if st != 0:
            raise RuntimeError(f"glm_peak_mfma({name}) failed: hipError {st}")
        res[f"mfma_{name}_tflops"] = round(flops.value / (ms.value * 1e-3) / 1e12, 1)
        res[f"mfma_{name}_clock_mhz"] = round(mhz.value, 0)
    # the 256 x 256 prefill tile's K step with its operands in L2
    L.glm_peak_gemm_step.argtypes = [i32, i32, vp, vp, f64p, f64p, vp]
    src = torch.ones(512 * 12288 // 2, dtype=torch.bfloat16, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    step = {}
    for name, mode in (("mfma_only", 0), ("copies_only", 1), ("full", 2), ("full_spread", 3),
                       ("copies_mfma", 4), ("reads_mfma", 5), ("regcopies_mfma", 6)):
        us, mhz = ctypes.c_double(), ctypes.c_double()
        st = L.glm_peak_gemm_step(mode, 4000, src.data_ptr(), scratch.data_ptr(),
                                  ctypes.byref(us), ctypes.byref(mhz), stream)
        if st != 0:
            raise RuntimeError(f"glm_peak_gemm_step({name}) failed: hipError {st}")
        step[name] = {"us_per_step": round(us.value, 4), "clock_mhz": round(mhz.value, 0),
                      "cycles_per_step": round(us.value * mhz.value, 0)}
    for name in ("full", "full_spread"):
        step[f"{name}_tflops"] = round(2.0 * 256 * 256 * 64 * cus
                                       / (step[name]["us_per_step"] * 1e-6) / 1e12, 1)
    res["gemm_step_l2"] = step
    del src
    nbytes = 8 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ms = ctypes.c_float()
    st = L.glm_peak_hbm_read(buf.data_ptr(), nbytes, 5, scratch.data_ptr(), ctypes.byref(ms),
                             stream)
    if st != 0:
        raise RuntimeError(f"glm_peak_hbm_read failed: hipError {st}")
    res["hbm_read_gbs"] = round(nbytes / (ms.value * 1e-3) / 1e9, 1)
    res["hbm_read_bytes"] = nbytes
    del buf, scratch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


PEAKS = None  # measured ceilings of this run (main sets it)


def with_measured(roof, peaks=None):
    """Add the fraction of the measured ceiling to a roofline object."""
    peaks = peaks or PEAKS
    if not peaks:
        return roof
    if roof["bound"] == "hbm":
        m = peaks["hbm_read_gbs"]
    elif roof["peak"] == PEAK_FP8_TFLOPS:
        m = peaks["mfma_fp8_tflops"]
    else:
        m = peaks["mfma_bf16_tflops"]
    roof["measured_peak"] = m
    roof["frac_measured"] = round(roof["achieved"] / m, 4)
    return roof


def at_clock(roof, clock):
    """MFMA-bound roofline: also the fraction of the peak scaled to the mean
    shader clock measured over the calls (the published peak is at the
    2400 MHz peak engine clock)."""
    if roof["bound"] != "mfma" or not clock:
        return roof
    clk = clock["mean"]
    roof["clock_mhz_timed"] = clk
    roof["peak_at_clock"] = round(roof["peak"] * clk / PEAK_CLOCK_MHZ, 1)
    roof["frac_at_clock"] = round(roof["achieved"] / roof["peak_at_clock"], 4)
    return roof


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic(w, counts):
    """Work the method itself needs for one call, from the realised routing."""
    T, D, E, k, F, Fs = w.T, w.D, w.E, w.k, w.F, w.Fs
    n_active = int((counts > 0).sum())
    wb = 1 + 1 / 32 if w.dtype == "mxfp8" else 2  # weight bytes per element (MXFP8: + scales)
    f = {
        # routed and shared gate/up (one launch)
        "gate_up": 2.0 * T * k * 2 * F * D + 2.0 * T * 2 * Fs * D,
        # routed and shared down projections (one launch)
        "down": 2.0 * T * k * D * F + 2.0 * T * D * Fs,
        "shared_combine": 0.0,
        "router_fp32": 2.0 * T * E * D,
    }
    b = {
        # active experts' w1+w3, the shared w1+w3, and the input tokens
        "gate_up": (n_active * 2 * F * D + 2 * Fs * D) * wb + T * D * 2,
        # active experts' w2 and the shared w2
        "down": (n_active * D * F + D * Fs) * wb,
        # the combine writes the fp32 output (its slot-buffer reads are overhead)
        "shared_combine": T * D * 4,
    }
    layer_bytes = ((n_active * 3 * F * D + 3 * Fs * D) * wb + E * D * 4 + E * 4
                   + T * D * 2 + T * D * 4)
    layer_flops = f["gate_up"] + f["down"]
    return f, b, layer_flops, layer_bytes, n_active


def probe_clock(torch, call, steps, seconds):
    """Mean shader clock (MHz) over `steps` more calls: a one-wave probe
    (libglm_peaks.so) on a side stream samples the shader clock counter
    against the 100 MHz constant counter every 100 us for `seconds` (set a
    little shorter than the calls) while they run."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "sparse_moe_transformer_glm_amd", "libglm_peaks.so"))
    L.glm_peak_clock_probe.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
    n = 4096
    buf = torch.zeros(2 * n + 1, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    st = L.glm_peak_clock_probe(min(max(seconds, 1e-3), 10.0), 100, n, buf.data_ptr(),
                                side.cuda_stream)
    if st != 0:
        raise RuntimeError(f"glm_peak_clock_probe failed: hipError {st}")
    for _ in range(steps):
        call(None)
    torch.cuda.synchronize()
    b = buf.cpu().numpy().astype("uint64")
    m = int(b[2 * n])
    if m < 3:
        return None
    c = b[0:2 * m:2].astype("float64")
    r = b[1:2 * m:2].astype("float64")
    mhz = 100.0 * (c[1:] - c[:-1]) / (r[1:] - r[:-1])
    return {"mean": round(float(mhz.mean()), 0), "min": round(float(mhz.min()), 0),
            "max": round(float(mhz.max()), 0), "samples": int(m - 1)}


def time_calls(glm, torch, call, steps, warmup):
    """Run ``call(trace)`` warmup + steps times untraced; wall time of the
    timed steps (synchronised on both sides); then the same number of calls
    with the library recording HIP events on the call's stream between its
    stages, for the per-stage (per-kernel) times."""
    for _ in range(warmup):
        call(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call(None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # then the shader clock over as many calls again (a separate pass, so the
    # probe's wave does not take part in the timed one)
    time_calls.clock = probe_clock(torch, call, steps, 0.9 * elapsed)
    tr = glm.Trace(max_calls=steps)
    for _ in range(steps):
        call(tr)
    torch.cuda.synchronize()
    stage_ms, n = tr.read()
    tr.close()
    return elapsed, {s: v / n for s, v in stage_ms.items()}


def call_percentiles(torch, call, n):
    """p10 / median / p90 of single-call times (HIP events on the launch
    stream, one pair per call), from n more calls."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record()
        call(None)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"p10": round(float(np.percentile(t, 10)), 4),
            "p50": round(float(np.median(t)), 4),
            "p90": round(float(np.percentile(t, 90)), 4)}


def time_route(glm, torch, dev, w, steps, warmup, ws):
    """glm_moe_route alone (router logits, top-k, weights): ms per call."""
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        glm.route(dev.x, dev.router_w, dev.corr_bias, w.k, w.scale, workspace=ws,
                  topk_idx=idx, topk_w=wt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        glm.route(dev.x, dev.router_w, dev.corr_bias, w.k, w.scale, workspace=ws,
                  topk_idx=idx, topk_w=wt)
    torch.cuda.synchronize()
    return round((time.perf_counter() - t0) * 1e3 / steps, 4)


def time_layer(glm, torch, dev, w, steps, warmup, ws, **opts):
    out = torch.empty((w.T, w.D), dtype=torch.float32, device="cuda")
    args = dev.args()
    scale = opts.pop("scale", w.scale)
    x = opts.pop("x", args[0])
    args = (x,) + tuple(args[1:])
    fwd = glm.forward_mx if w.dtype == "mxfp8" else glm.forward

    def call(tr):
        fwd(*args, w.k, scale, out=out, workspace=ws, trace=tr, **opts)

    elapsed, per_call = time_calls(glm, torch, call, steps, warmup)
    per_call["_pct"] = call_percentiles(torch, call, steps)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    fwd(*args, w.k, scale, out=out, workspace=ws, topk_idx=idx, **opts)
    counts = torch.bincount(idx.flatten().long(), minlength=w.E).cpu().numpy()
    return elapsed, per_call, counts


def stages(per_call):
    return {s: round(v, 4) for s, v in per_call.items() if not s.startswith("_")}


def record(w, elapsed, steps, per_call, counts, bound, traffic_kind=None):
    f, b, lf, lb, n_active = algorithmic(w, counts)
    ms = elapsed * 1e3 / steps
    dom = max(("gate_up", "down", "shared_combine"), key=lambda s: per_call[s])
    t_dom = per_call[dom] * 1e-3
    peak_mfma = PEAK_FP8_TFLOPS if w.dtype == "mxfp8" else PEAK_BF16_TFLOPS
    if bound == "mfma":
        ach = f[dom] / t_dom / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2),
                "peak": peak_mfma, "unit": "TFLOP/s", "frac": round(ach / peak_mfma, 4),
                "traffic": None, "work_per_launch": f[dom], "avg_launch_ms": round(per_call[dom], 4)}
        if dom == "gate_up" and traffic_kind:
            roof["traffic"] = measured_traffic(traffic_kind)
    else:
        ach = b[dom] / t_dom / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                "work_per_launch": b[dom], "avg_launch_ms": round(per_call[dom], 4)}
        if dom == "gate_up" and traffic_kind:
            roof["traffic"] = measured_traffic(traffic_kind)
    t_layer = ms * 1e-3
    layer = {"tflops": round(lf / t_layer / 1e12, 2),
             "frac_mfma": round(lf / t_layer / 1e12 / peak_mfma, 4),
             "hbm_gbs_algorithmic": round(lb / t_layer / 1e9, 1),
             "frac_hbm": round(lb / t_layer / 1e9 / PEAK_HBM_GBS, 4),
             "flops": lf, "bytes": lb}
    load = {"active_experts": n_active, "max_rows": int(counts.max()),
            "mean_rows": round(float(counts.mean()), 2), "min_rows": int(counts.min())}
    return ms, with_measured(roof), layer, load


def dense_record(glm, torch, w, F, dw, steps, warmup, ws, bound):
    """The dense SiLU-gated FFN (hidden w.D, width F) on the grouped path."""
    T, D = w.T, w.D
    import workloads as wl
    from workloads.device import to_device
    x = to_device(wl.make_x(w))
    out = torch.empty((T, D), dtype=torch.float32, device="cuda")

    def call(tr):
        glm.dense_ffn(x, *dw, out=out, workspace=ws, trace=tr)

    elapsed, pc = time_calls(glm, torch, call, steps, warmup)
    ms = elapsed * 1e3 / steps
    f = {"gate_up": 2.0 * T * 2 * F * D, "down": 2.0 * T * D * F}
    b = {"gate_up": 2 * F * D * 2 + T * D * 2, "down": D * F * 2 + T * F * 2}
    dom = max(("gate_up", "down"), key=lambda s: pc[s])
    t = pc[dom] * 1e-3
    if bound == "mfma":
        ach = f[dom] / t / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "work_per_launch": f[dom], "avg_launch_ms": round(pc[dom], 4)}
    else:
        ach = b[dom] / t / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                "work_per_launch": b[dom], "avg_launch_ms": round(pc[dom], 4)}
    return {"workload": f"dense FFN hidden {D} width {F}, {T} tokens", "tokens": T,
            "value": round(T * steps / elapsed, 1), "unit": "tokens/s", "steps": steps,
            "ms_per_step": round(ms, 4), "roofline": at_clock(with_measured(roof), time_calls.clock),
            "stages_ms": {s: round(v, 4) for s, v in pc.items() if v > 0}}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, n_tokens):
    import numpy as np

    import oracle
    import workloads as wl

    x = wl.make_x(w)[:n_tokens]
    rw, cb = wl.make_router_w(w), wl.make_corr_bias(w)
    need = np.unique(oracle.route(x, rw, cb, w.k, w.scale).idx)
    cache = dict(wl.iter_experts(w, experts=need.tolist()))
    shared = wl.make_shared(w)
    t0 = time.perf_counter()
    oracle.forward(x, rw, cb, lambda e: cache[e], shared, w.k, w.scale)
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt, 4), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": (f"first {n_tokens} tokens of the {w.name} batch (T={w.T}): float64 NumPy "
                       f"oracle, routing + the {len(need)} distinct experts they select + shared "
                       f"expert; weights drawn before timing")}


def variants(glm, torch, wl, dev, wp, wd, ws, norm_w, args):
    """The layer's options and the dense FFN, at the prefill (and decode) sizes."""
    from workloads.device import to_device
    res = {}
    base = None
    # pre-norm block: RMSNorm of the residual stream in, residual add out
    h = to_device(wl.make_hidden(wp))
    e, pc, c = time_layer(glm, torch, dev, wp, args.steps, args.warmup, ws, x=h,
                          norm_weight=norm_w, residual=True)
    nb = wp.T * wp.D * 2 * 2 + wp.D * 4   # read h, write the normalised bf16 input
    res["prefill_block"] = {
        "what": "RMSNorm(h) -> layer -> + h", "value": round(wp.T * args.steps / e, 1),
        "unit": "tokens/s", "ms_per_step": round(e * 1e3 / args.steps, 4),
        "norm_roofline": {"bound": "hbm", "kernel": "rmsnorm", "work_per_launch": nb,
                          "avg_launch_ms": round(pc["norm"], 4),
                          "achieved": round(nb / (pc["norm"] * 1e-3) / 1e9, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(nb / (pc["norm"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "stages_ms": stages(pc)}
    log(f"prefill block: {res['prefill_block']['value']:,.0f} tokens/s, stages {stages(pc)}")
    del h
    # group-limited routing (8 groups of 32, 4 kept) at scale 1.0
    e, pc, c = time_layer(glm, torch, dev, wp, args.steps, args.warmup, ws, n_group=8,
                          topk_group=4, group_topk=2, scale=1.0)
    res["prefill_group_routing"] = {
        "what": "n_group 8, topk_group 4, group_topk 2, scale 1.0",
        "value": round(wp.T * args.steps / e, 1), "unit": "tokens/s",
        "ms_per_step": round(e * 1e3 / args.steps, 4),
        "stages_ms": stages(pc)}
    log(f"prefill group routing: {res['prefill_group_routing']['value']:,.0f} tokens/s, "
        f"stages {stages(pc)}")
    if wd:
        dd = type(dev)(wd, to_device(wl.make_x(wd)), dev.router_w,
                       to_device(wl.make_corr_bias(wd)), dev.w1, dev.w3, dev.w2, dev.sw1,
                       dev.sw3, dev.sw2)
        e, pc, c = time_layer(glm, torch, dd, wd, args.decode_steps, args.warmup, ws, n_group=8,
                              topk_group=4, group_topk=2, scale=1.0)
        res["decode_group_routing"] = {
            "value": round(wd.T * args.decode_steps / e, 1), "unit": "tokens/s",
            "ms_per_step": round(e * 1e3 / args.decode_steps, 4),
            "stages_ms": stages(pc)}
    # skewed routing at the GLM shape: +1.5 on 16 hot experts (every assignment
    # lands on them: MFMA-bound), and +0.2 (about 40% hot: weight streaming)
    for key, name, bound in (("skew_literal", "glm_skew", "mfma"),
                             ("skew_mild", "glm_skew_mild", "hbm")):
        w = wl.WORKLOADS[name]
        d = dev.with_x(to_device(wl.make_x(w)), to_device(wl.make_corr_bias(w)), w)
        e, pc, c = time_layer(glm, torch, d, w, args.steps, args.warmup, ws)
        ms, roof, layer, load = record(w, e, args.steps, pc, c, bound)
        at_clock(roof, time_calls.clock)
        res[key] = {"workload": name, "tokens": w.T, "hot_bias": w.hot_value,
                    "value": round(w.T * args.steps / e, 1), "unit": "tokens/s",
                    "ms_per_step": round(ms, 4), "roofline": roof, "layer_roofline": layer,
                    "routing_load": load, "hot_share": round(float(c[:w.hot_count].sum()) /
                                                             float(c.sum()), 4),
                    "stages_ms": stages(pc), "call_ms": pc["_pct"]}
        log(f"{key}: {res[key]['value']:,.0f} tokens/s, hot share {res[key]['hot_share']}, "
            f"stages {stages(pc)}")
        del d
    # the layer between the decode and prefill sizes (same weights, near-uniform
    # routing); the roofline is whichever of MFMA and HBM binds at that size
    sweep = {}
    for T in (256, 1024, 2048, 4096):
        w = wp.with_(name=f"glm_T{T}", T=T)
        d = dev.with_x(to_device(wl.make_x(w)), to_device(wl.make_corr_bias(w)), w)
        e, pc, c = time_layer(glm, torch, d, w, args.steps, args.warmup, ws)
        _, _, lf, lb, _ = algorithmic(w, c)
        bound = "mfma" if lf / (PEAK_BF16_TFLOPS * 1e12) > lb / (PEAK_HBM_GBS * 1e9) else "hbm"
        ms, roof, layer, load = record(w, e, args.steps, pc, c, bound)
        at_clock(roof, time_calls.clock)
        sweep[str(T)] = {"value": round(T * args.steps / e, 1), "unit": "tokens/s",
                         "ms_per_step": round(ms, 4), "roofline": roof, "layer_roofline": layer,
                         "routing_load": load, "call_ms": pc["_pct"]}
        log(f"T={T}: {sweep[str(T)]['value']:,.0f} tokens/s, {roof['bound']} frac {roof['frac']}")
        del d
    res["token_sweep"] = sweep
    # dense FFN of the leading dense layers (width: see workloads.GLM_DENSE_WIDTH)
    F = wl.GLM_DENSE_WIDTH
    t0 = time.time()
    dw = [to_device(a) for a in wl.make_dense(wp, F)]
    log(f"dense FFN weights ready ({time.time() - t0:.1f}s)")
    need = glm.dense_workspace_size(wp.T, wp.D, F)
    dws = ws if need <= ws.numel() else torch.empty(need, dtype=torch.uint8, device="cuda")
    res["dense_prefill"] = dense_record(glm, torch, wp, F, dw, args.steps, args.warmup, dws,
                                        "mfma")
    log(f"dense prefill: {res['dense_prefill']['value']:,.0f} tokens/s")
    if wd:
        res["dense_decode"] = dense_record(glm, torch, wd, F, dw, args.decode_steps,
                                           args.warmup, dws, "hbm")
        log(f"dense decode: {res['dense_decode']['value']:,.0f} tokens/s")
    del dw, dws
    torch.cuda.empty_cache()
    # MXFP8 expert weights: the same draws encoded as MXFP8
    res.update(mx_records(glm, torch, wl, args))
    return res


def mx_records(glm, torch, wl, args):
    """The layer with MXFP8 expert weights at the prefill and decode sizes."""
    from workloads.device import stream_layer, to_device
    wp, wd = wl.WORKLOADS["glm_prefill_mx"], wl.WORKLOADS["glm_decode_mx"]
    t0 = time.time()
    dev, _ = stream_layer(wp)
    log(f"MXFP8 layer weights resident ({time.time() - t0:.1f}s)")
    n = max(glm.workspace_size(w.T, w.D, w.E, w.F, w.Fs, w.k, weight=glm.MXFP8) for w in (wp, wd))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    res = {}
    for key, w, steps, bound in (("prefill_mxfp8", wp, args.steps, "mfma"),
                                 ("decode_mxfp8", wd, args.decode_steps, "hbm")):
        d = dev if w is wp else dev.with_x(to_device(wl.make_x(w)),
                                           to_device(wl.make_corr_bias(w)), w)
        e, pc, c = time_layer(glm, torch, d, w, steps, args.warmup, ws)
        ms, roof, layer, load = record(w, e, steps, pc, c, bound)
        at_clock(roof, time_calls.clock)
        res[key] = {"workload": w.name, "tokens": w.T, "value": round(w.T * steps / e, 1),
                    "unit": "tokens/s", "steps": steps, "ms_per_step": round(ms, 4),
                    "roofline": roof, "layer_roofline": layer, "routing_load": load,
                    "stages_ms": stages(pc), "call_ms": pc["_pct"]}
        log(f"{key}: {res[key]['value']:,.0f} tokens/s, stages {stages(pc)}")
    del dev, ws
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="glm_prefill")
    ap.add_argument("--decode-workload", default="glm_decode", help="'' to skip")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=120, help="0 to skip the oracle baseline")
    ap.add_argument("--no-variants", dest="variants", action="store_false",
                    help="skip the block / group-routing / dense-FFN measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the MFMA / HBM ceiling microbenchmarks (profiling runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this layer is built and measured on "
              "one GPU only (no expert parallelism or collectives); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_moe_transformer_glm_amd as glm
    import workloads as wl
    from workloads.device import stream_layer, to_device

    torch.cuda.set_device(0)
    global PEAKS
    peaks = None
    if args.peaks:
        peaks = PEAKS = measured_peaks(torch)
        log(f"measured ceilings: {peaks}")
    wp = wl.WORKLOADS[args.workload]
    t0 = time.time()
    log(f"drawing + uploading {wp.name} layer weights (seeded, bf16)")
    dev, _ = stream_layer(wp)
    log(f"weights resident in HBM ({time.time() - t0:.1f}s)")

    wd = wl.WORKLOADS[args.decode_workload] if args.decode_workload else None
    norm_w = to_device(wl.make_norm_weight(wp))
    block_opts = glm.options(norm_weight=norm_w, residual=True, D=wp.D)
    sizes = [glm.workspace_size(wp.T, wp.D, wp.E, wp.F, wp.Fs, wp.k),
             glm.workspace_size(wp.T, wp.D, wp.E, wp.F, wp.Fs, wp.k, opts=block_opts)]
    if wd:
        sizes.append(glm.workspace_size(wd.T, wd.D, wd.E, wd.F, wd.Fs, wd.k))
    ws = torch.empty(max(sizes), dtype=torch.uint8, device="cuda")

    elapsed, per_call, counts = time_layer(glm, torch, dev, wp, args.steps, args.warmup, ws)
    gpu = time_calls.clock
    ms, roof, layer, load = record(wp, elapsed, args.steps, per_call, counts, "mfma",
                                   "prefill" if wp.name == "glm_prefill" else None)
    at_clock(roof, gpu)
    value = wp.T * args.steps / elapsed
    log(f"prefill: {value:,.0f} tokens/s, {ms:.3f} ms/step, stages {stages(per_call)}")
    route_ms = time_route(glm, torch, dev, wp, args.steps, args.warmup, ws)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wp.name, "tokens": wp.T, "hidden": wp.D, "experts": wp.E,
                   "top_k": wp.k, "expert_width": wp.F, "shared_width": wp.Fs,
                   "routed_scale": wp.scale, "corr_bias_std": wp.bias_std,
                   "parallelism": "single GPU"},
        "roofline": roof, "layer_roofline": layer, "routing_load": load,
        "stages_ms": stages(per_call), "call_ms": per_call["_pct"], "route_ms": route_ms,
        "measured_peaks": peaks, "shader_clock_mhz": gpu,
    }

    if wd:
        dd = type(dev)(wd, to_device(wl.make_x(wd)), dev.router_w,
                       to_device(wl.make_corr_bias(wd)), dev.w1, dev.w3, dev.w2, dev.sw1,
                       dev.sw3, dev.sw2)
        e2, pc2, c2 = time_layer(glm, torch, dd, wd, args.decode_steps, args.warmup, ws)
        gpu2 = time_calls.clock
        ms2, roof2, layer2, load2 = record(wd, e2, args.decode_steps, pc2, c2, "hbm",
                                           "decode" if wd.name == "glm_decode" else None)
        v2 = wd.T * args.decode_steps / e2
        log(f"decode: {v2:,.0f} tokens/s, {ms2:.3f} ms/step, stages {stages(pc2)}")
        route2 = time_route(glm, torch, dd, wd, args.decode_steps, args.warmup, ws)
        line["decode"] = {"workload": wd.name, "tokens": wd.T, "value": round(v2, 1),
                          "unit": "tokens/s", "steps": args.decode_steps,
                          "ms_per_step": round(ms2, 4), "roofline": roof2,
                          "layer_roofline": layer2, "routing_load": load2,
                          "stages_ms": stages(pc2), "call_ms": pc2["_pct"],
                          "route_ms": route2, "shader_clock_mhz": gpu2}

    if args.variants:
        line["variants"] = variants(glm, torch, wl, dev, wp, wd, ws, norm_w, args)

    del dev
    torch.cuda.empty_cache()
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    if args.cpu_tokens > 0:
        log(f"timing the CPU oracle on {args.cpu_tokens} tokens")
        line["cpu_baseline"] = cpu_baseline(wp, args.cpu_tokens)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
