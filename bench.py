"""Benchmark of the MoE expert layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config small] [--mode router]
                    [--no-cpu-baseline] [--lean] [--overlap | --serial] [--aux-alpha A]

One step = the whole hot path over one batch of synthetic input, through the C
ABI: router logits, routing (softmax / top-k, histogram, offsets, positions),
rowwise dispatch, grouped SwiGLU GEMMs, combine, and the full backward
(combine backward, dgrad / wgrad grouped GEMMs, unpermute-sum, router
backward).  Inputs are generated once and stay resident in HBM; identical
values are used for every step.

Prints ONE JSON line.  The default workload is the 8-expert top-4 layer
(T=8192 tokens, d_model 2048, SwiGLU hidden 1024, bf16).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s and grouped-GEMM TFLOP/s (% of MFMA peak), 1 GPU"
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0

FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 / MXFP8 MFMA
GEMM_KERNELS = {
    # name: flops per launch as a multiple of R*d*h
    "ggemm_up_swiglu": 4, "ggemm_down": 2, "ggemm_dgrad_down_swiglu": 2, "ggemm_wgrad_down": 2,
    "ggemm_dgrad_up": 4, "ggemm_wgrad_up": 4,
}
GEMM_KERNELS.update({n.replace("ggemm_", "ggemm_mx_"): m for n, m in list(GEMM_KERNELS.items())})


# HBM traffic of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE
# runs (profiles/hbm_traffic.txt).  A line counts only while the kernel's
# sources are unchanged since the counters were taken (their sha256 is part of
# the line); otherwise the traffic is reported as null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = {
    "ggemm_mx_": ["ggemm_mx.hip", "ggemm_impl.h", "common.h", "kernels.h"],
    "ggemm_": ["ggemm.hip", "ggemm_impl.h", "common.h", "kernels.h"],
}


def kernel_sources_sha(kernel):
    import hashlib

    for prefix, files in KERNEL_SOURCES.items():
        if kernel.startswith(prefix):
            h = hashlib.sha256()
            for f in files:
                with open(os.path.join(ROOT, "token_routing_grouped_amd", "csrc", f), "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()
    return None


def measured_traffic(kernel, workload):
    """HBM bytes per launch recorded for (kernel, workload), or None."""
    sha = kernel_sources_sha(kernel)
    if sha is None or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("#") or "|" not in line:
                continue
            parts = [p.strip() for p in line.split("|")]
            if len(parts) >= 8 and parts[0] == kernel and parts[1] == workload and parts[2] == sha:
                return float(parts[7])
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def cpu_baseline(cfg, mode, sample_T, min_seconds=10.0):
    """The oracle as it stands, timed on the host on the first sample_T tokens
    of the same workload (all experts, full d and h)."""
    import numpy as np

    from oracle import moe_ref as ref
    from token_routing_grouped_amd import inputs

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    from oracle import moe_mx_ref as mxl

    inp = inputs.layer_inputs(cfg, T=sample_T)
    forced = None
    if mode != "router":
        forced = inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)[:sample_T]
    args = (inp["x"], inp["wr"], inp["w1"], inp["w3"], inp["w2"])
    if cfg.mx:  # the MXFP8 oracle computes in float64 only
        prec = "float64"
        fwd, bwd = mxl.layer_forward_mx, mxl.layer_backward_mx
    else:  # the float oracle run in fp32, the precision the layer accumulates in
        prec = "float32"
        fwd = lambda *a, **kw: ref.layer_forward(*a, dtype=np.float32, **kw)
        bwd = lambda *a, **kw: ref.layer_backward(*a, dtype=np.float32, **kw)
    times = []
    while True:  # repeat the same sample until ~10 s of CPU work (at most 20 runs)
        t0 = time.perf_counter()
        f = fwd(*args, cfg.k, forced_idx=forced)
        bwd(f, inp["dy"], *args)
        times.append(time.perf_counter() - t0)
        if sum(times) >= min_seconds or len(times) >= 20:
            break
    el = float(np.median(times))
    return {"value": sample_T / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"first {sample_T} of {cfg.T} tokens, all {cfg.E} experts, full d={cfg.d} h={cfg.h}; "
                      f"{prec} numpy {'MXFP8 (quantise-dequantise) ' if cfg.mx else ''}fwd+bwd, median of "
                      f"{len(times)} runs ({sum(times):.1f} s total), BLAS on {threads} threads of "
                      f"{os.cpu_count()} host CPUs ({cpu_model()})",
            "seconds_per_run": el}


def plain_ms_per_step(layer, args, forced, steps, warmup):
    """Milliseconds per step of `steps` back-to-back steps with no events at all
    (wall clock around the loop), and the median of one event pair per step."""
    import numpy as np
    import torch

    for _ in range(warmup):
        layer.step(*args, forced_idx=forced)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.step(*args, forced_idx=forced)
    torch.cuda.synchronize()
    wall = 1000.0 * (time.perf_counter() - t0) / steps
    pairs = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.step(*args, forced_idx=forced)
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return {"ms_per_step": wall, "median_ms": float(np.median([x.elapsed_time(y) for x, y in pairs]))}


def gate_runs(small_tensors, small_ms, steps, warmup, dev):
    """The layer at the other gated shapes, in the same process: the wide
    128-expert layer in bf16 and MXFP8, and the small layer in MXFP8 (its inputs
    are the small bf16 layer's, so MXFP8 and bf16 are value-matched at each
    shape).  Returns ms per step and the two gate checks: the layer's share of
    the bf16 MFMA peak, and MXFP8 faster than bf16 at the same shape."""
    import torch

    from token_routing_grouped_amd import configs, inputs
    from token_routing_grouped_amd.layer import MoELayerGPU

    out = {}
    small = configs.get("small")
    for slug in ("mxfp8_small", "wide", "mxfp8"):
        cfg = configs.get(slug)
        if (cfg.T, cfg.d, cfg.E) == (small.T, small.d, small.E):
            t = small_tensors
        else:
            if "wide_tensors" not in out:
                log(f"bench: gate inputs for {cfg.T}x{cfg.d}, {cfg.E} experts")
                out["wide_tensors"] = inputs.device_inputs(cfg, dev)[0]
            t = out["wide_tensors"]
        layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, dev, mx=cfg.mx, overlap=cfg.overlap)
        args = (t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
        r = plain_ms_per_step(layer, args, None, steps, warmup)
        r["tokens_per_s"] = cfg.T / (r["ms_per_step"] * 1e-3)
        r["layer_tflops"] = (cfg.gemm_flops() + cfg.router_flops()) / (r["ms_per_step"] * 1e-3) / 1e12
        r["streams"] = 2 if layer.overlap else 1
        out[slug] = r
        del layer
        torch.cuda.empty_cache()
        log(f"bench: gate {slug}: {r['ms_per_step']:.3f} ms/step")
    out.pop("wide_tensors", None)
    wide = configs.get("wide")
    sm_fl = small.gemm_flops() + small.router_flops()
    wd_fl = wide.gemm_flops() + wide.router_flops()
    return {
        "ms_per_step": {"small_bf16": small_ms, "small_mxfp8": out["mxfp8_small"]["ms_per_step"],
                        "wide_bf16": out["wide"]["ms_per_step"], "wide_mxfp8": out["mxfp8"]["ms_per_step"]},
        "median_ms": {"small_mxfp8": out["mxfp8_small"]["median_ms"], "wide_bf16": out["wide"]["median_ms"],
                      "wide_mxfp8": out["mxfp8"]["median_ms"]},
        "layer_frac_bf16_peak": {"small": sm_fl / (small_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                 "wide": wd_fl / (out["wide"]["ms_per_step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "mxfp8_faster_than_bf16": {"small": out["mxfp8_small"]["ms_per_step"] < small_ms,
                                   "wide": out["mxfp8"]["ms_per_step"] < out["wide"]["ms_per_step"]},
        "note": "ms_per_step: wall clock of back-to-back steps with no events, each workload's default "
                "stream schedule, router routing, same process and inputs as above (wide and MXFP8-wide share "
                "one input set, small and MXFP8-small another)",
    }


# Dense equivalent (M, N, K) of each grouped GEMM: same flop count as one
# launch, as one plain GEMM over all R routed rows.
def dense_shape(kernel, cfg):
    R, d, h = cfg.R, cfg.d, cfg.h
    shapes = {"ggemm_up_swiglu": (R, 2 * h, d), "ggemm_down": (R, d, h), "ggemm_dgrad_down_swiglu": (R, h, d),
              "ggemm_dgrad_up": (R, d, 2 * h), "ggemm_wgrad_down": (d, h, R), "ggemm_wgrad_up": (2 * h, d, R)}
    return shapes.get(kernel)


def dense_gemm_ref(M, N, K, dev, reps=20):
    """torch.mm (the vendor GEMM library) on one dense bf16 GEMM of the given
    size, contiguous operands, timed with events: what the library reaches on
    the same work without grouping or an epilogue, as a reference for the
    grouped kernel's fraction of peak."""
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = (torch.randn(M, K, device=dev, generator=g) * 0.02).to(torch.bfloat16).contiguous()
    b = (torch.randn(K, N, device=dev, generator=g) * 0.02).to(torch.bfloat16).contiguous()
    c = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    del a, b, c
    return {"M": M, "N": N, "K": K, "dtype": "bf16", "avg_us": us, "tflops": tflops,
            "frac": tflops / BF16_PEAK_TFLOPS, "launches": reps}


def copy_probe(nbytes=1 << 30, reps=5):
    """A plain copy kernel of known size: each launch reads and writes exactly
    nbytes.  Profiled with the FETCH_SIZE / WRITE_SIZE counters it gives the
    factor that turns those counters into HBM bytes."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": reps}), flush=True)



def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="small")
    ap.add_argument("--mode", default=None, help="router | uniform | zipf (default: the config's first mode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--overlap", action="store_true",
                    help="run the weight-gradient GEMMs on a second stream next to the dgrad chain (bf16; "
                         "the default for workloads whose config sets it)")
    ap.add_argument("--serial", action="store_true",
                    help="one stream for the whole step, also where the workload's config overlaps")
    ap.add_argument("--lean", action="store_true",
                    help="memory-lean backward: G and U are not stored by the forward but recomputed")
    ap.add_argument("--aux-alpha", type=float, default=0.0,
                    help="include the router balance loss (weight alpha) in every timed step")
    ap.add_argument("--no-gates", action="store_true",
                    help="skip the extra runs of the other gated shapes (wide bf16, MXFP8 small and wide) that "
                         "the default workload reports next to its own line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    a = ap.parse_args()

    if a.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {a.gpus} is not supported "
              f"(the layer is measured on one GPU's share; there is no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from token_routing_grouped_amd import _abi, configs, inputs
    from token_routing_grouped_amd.layer import MoELayerGPU

    if a.copy_probe:
        copy_probe()
        return

    cfg = configs.get(a.config)
    mode = a.mode or cfg.modes[0]
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    log(f"bench: {cfg.slug} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} {cfg.dtype} mode={mode}")
    t, weights_on = inputs.device_inputs(cfg, dev, log=lambda m: log(f"bench: {m}"))
    forced = None
    if mode != "router":
        forced = torch.from_numpy(inputs.forced_routing(mode, cfg.T, cfg.E, cfg.k, cfg.seed)).to(dev)
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dt, dev, mx=cfg.mx, aux_alpha=a.aux_alpha, lean=a.lean,
                        overlap=(a.overlap or cfg.overlap) and not a.serial)
    args = (t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])

    for _ in range(a.warmup):
        layer.step(*args, forced_idx=forced)
    torch.cuda.synchronize()
    log("bench: warmup done")

    # per-kernel averages: an untimed pass of `steps` steps with HIP events
    # around every library launch (recorded on each launch's stream)
    _abi.prof_reset()
    _abi.prof_only(None)
    _abi.prof_enable(True)
    for _ in range(a.steps):
        layer.step(*args, forced_idx=forced)
    torch.cuda.synchronize()
    _abi.prof_enable(False)
    kern = {}
    for name in _abi.prof_names():
        n, ms = _abi.prof_query(name)
        kern[name] = {"launches": n, "avg_us": 1000.0 * ms / max(n, 1)}
    _abi.prof_reset()
    rdh = cfg.R * cfg.d * cfg.h
    timed_gemms = [n for n in GEMM_KERNELS if n in kern]
    if not timed_gemms:  # the fp32 (tiny) layer has no named matrix-core kernels
        print(f"bench.py: no grouped-GEMM kernel timings for {cfg.slug}; it is a parity case, not a bench "
              "workload", file=sys.stderr)
        sys.exit(2)
    # With the two-stream backward the weight-gradient kernels share the GPU
    # with the dgrad chain, so no backward GEMM's event duration is its own;
    # the dominant kernel is then chosen among the forward GEMMs, which run
    # alone (and the grouped-GEMM sum below counts the overlapped ones in full).
    # With the MXFP8 weights quantised on a second stream, W2's copies are made
    # while the up projection runs, so there only the down projection is alone.
    def alone(n):
        if layer.overlap and ("wgrad" in n or "dgrad" in n):
            return False
        return not (layer.mx and layer.wq_stream is not None and "up_swiglu" in n)

    solo = [n for n in timed_gemms if alone(n)]
    dom = max(solo, key=lambda n: kern[n]["avg_us"])
    log("bench: per-kernel pass done")

    # timed region: exactly `steps` steps, with HIP events recorded on the
    # launch stream around the dominant kernel only (two per launch)
    _abi.prof_only(dom)
    _abi.prof_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        layer.step(*args, forced_idx=forced)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _abi.prof_enable(False)
    n_dom, ms_dom = _abi.prof_query(dom)
    _abi.prof_only(None)
    _abi.prof_reset()
    dom_us = 1000.0 * ms_dom / max(n_dom, 1)
    log("bench: timed steps done")

    # the same steps again without the library's per-kernel events (they add
    # a little host/GPU overhead)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(a.steps):
        layer.step(*args, forced_idx=forced)
    torch.cuda.synchronize()
    elapsed_clean = time.perf_counter() - t1

    # Per-step distribution: one event pair per step on torch's current stream
    # (where the layer launches), back to back, then with the 256 MB Infinity
    # Cache flushed before each step by writing a 1 GiB scratch buffer outside
    # the events.
    def step_distribution(flush):
        pairs = []
        for _ in range(a.steps):
            if flush is not None:
                flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            layer.step(*args, forced_idx=forced)
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        ms = np.array([x.elapsed_time(y) for x, y in pairs])
        return {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
                "p90": float(np.percentile(ms, 90))}

    dist = step_distribution(None)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dist_flushed = step_distribution(scratch)
    del scratch
    log("bench: per-step distributions done")

    ms_step = 1000.0 * elapsed / a.steps
    tokens_per_s = cfg.T * a.steps / elapsed
    gemm_flops = cfg.gemm_flops()
    layer_flops = gemm_flops + cfg.router_flops()
    gemm_us = 0.0
    for name, mult in GEMM_KERNELS.items():
        if name in kern:
            kern[name]["tflops"] = mult * rdh / (kern[name]["avg_us"] * 1e-6) / 1e12
            gemm_us += kern[name]["avg_us"]
    gemm_peak = FP8_PEAK_TFLOPS if cfg.mx else BF16_PEAK_TFLOPS
    dom_flops = GEMM_KERNELS[dom] * rdh
    achieved = dom_flops / (dom_us * 1e-6) / 1e12  # from the timed region's own events

    counts = layer.counts.cpu().numpy()
    # router balance report of the same routing (after the timed region): the
    # balance score next to the actual load of the busiest expert
    bstats = layer.balance(alpha=a.aux_alpha).cpu().numpy()
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if cfg.mx else cfg.dtype,
        "data": "synthetic (seeded: x~N(0,1), weights~N(0,0.02^2), dy~N(0,1); values fixed across steps"
                + ("; expert weights drawn on the device)" if weights_on == "device" else ")"),
        "config": {"workload": f"{cfg.slug}: MoE expert layer fwd+bwd, T={cfg.T} d_model={cfg.d} experts={cfg.E} "
                               f"top-{cfg.k} SwiGLU hidden={cfg.h} "
                               f"{'MXFP8 grouped GEMMs (bf16 router/combine)' if cfg.mx else cfg.dtype}, "
                               f"routing={mode}",
                   "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "h": cfg.h, "routing": mode,
                   "parallelism": "single GPU"},
        "layer_tflops": layer_flops / (ms_step * 1e-3) / 1e12,
        "layer_frac_bf16_peak": layer_flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "ggemm_tflops": gemm_flops / (gemm_us * 1e-6) / 1e12,
        "ggemm_frac_bf16_peak": gemm_flops / (gemm_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
        "ggemm_frac_own_peak": gemm_flops / (gemm_us * 1e-6) / 1e12 / gemm_peak,
        "ms_per_step_no_events": 1000.0 * elapsed_clean / a.steps,
        "step_ms": dist,
        "step_ms_cache_flushed": dist_flushed,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": gemm_peak,
                     "unit": "TFLOP/s", "frac": achieved / gemm_peak,
                     "traffic": measured_traffic(dom, f"{cfg.slug}/{mode}"),
                     "algorithmic_per_launch": f"{GEMM_KERNELS[dom]}*R*d*h = {dom_flops:.4g} flop",
                     "avg_us": dom_us, "launches": n_dom},
        # from the untimed pass with events around every launch
        "kernels_avg_us": {n: round(v["avg_us"], 2) for n, v in sorted(kern.items())},
        "expert_load": {"max": int(counts.max()), "mean": float(counts.mean()), "min": int(counts.min())},
        "balance": {"score": float(bstats[0]), "max_over_mean": float(bstats[2]), "min_over_mean": float(bstats[3]),
                    "aux_alpha": a.aux_alpha, "aux_loss": float(bstats[1])},
        "peak_mem_gib": torch.cuda.max_memory_allocated() / 2 ** 30,
        "streams": 2 if layer.overlap else 1,
        "memory": {"lean": a.lean, "saved_activation_bytes": layer.saved_bytes(),
                   "note": "bytes the layer keeps from the forward to the backward (routing metadata, inputs and "
                           "weights excluded)"},
    }
    shape = dense_shape(dom, cfg)
    if shape is not None and not cfg.mx:
        log("bench: dense GEMM reference")
        out["dense_gemm_ref"] = dict(dense_gemm_ref(*shape, dev), kernel=dom,
                                     note="torch.mm on one dense bf16 GEMM with the dominant kernel's flop "
                                          "count (one expert-free M x N x K; the grouped weight gradients write "
                                          "E times its output), outside the timed region")
    if cfg.slug == "small" and mode == "router" and not (a.no_gates or a.lean or a.aux_alpha or a.serial or a.overlap):
        out["gates"] = gate_runs(t, out["ms_per_step_no_events"], a.steps, a.warmup, dev)
    if not a.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, mode, min(a.cpu_sample_tokens, cfg.T))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
