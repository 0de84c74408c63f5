#!/usr/bin/env python3
"""Benchmark of the routed-expert path on one MI355X.

One step = one ``mega_moe`` call (dispatch -> Linear1 + SwiGLU -> Linear2 ->
combine, one persistent kernel after a zeroing pre-pass) over one batch of
seeded synthetic inputs already resident in HBM.  The default workload is
the A8W8 fp8 layer at 16384 tokens (hidden 7168, intermediate 2048, 32
experts, top-8): the MFMA-bound point.  The same run also times the same
layer at 128 tokens (the HBM-bound, weight-streaming point) and reports it
under "hbm_point".

Prints one JSON line: throughput in TFLOP/s (FLOP = 6 * routes * hidden *
intermediate), the roofline of the dominant kernel (the fused kernel, timed
with HIP events on its stream inside the timed region) against the
datasheet peak, against the MFMA peak at the shader clock the kernel ran at
(sampled inside the kernel) and against a measured device-copy bandwidth, a
per-phase breakdown from the three-call path, and the CPU oracle timed on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed expert-FFN TFLOP/s and tokens/s per MoE layer; % MFMA / HBM roofline"
PEAK = {  # MI355X published dense peaks; the MX use cases run on the f8f6f4 MFMA with an
    # e4m3 operand (fp8 rate; fp4 x fp4 alone would have the 10.1 PFLOP/s peak)
    "bf16": 2500e12, "fp8": 5000e12, "int8": 5000e12, "mxfp8": 5000e12, "mxfp4": 5000e12, "hbm": 8.0e12,
}
WEIGHT_BYTES = {"bf16": 2.0, "fp8": 1.0, "int8": 1.0, "mxfp8": 1.0, "mxfp4": 0.5}   # per weight element
DTYPE = {"bf16": "bf16", "fp8": "fp8_e4m3", "int8": "int8", "mxfp8": "mxfp8_e4m3",
         "mxfp4": "fp8_e4m3 x fp4_e2m1 (mx)"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_fp8_t16384")
    ap.add_argument("--hbm-workload", default="dsv3_fp8_t128",
                    help="weight-streaming point timed in the same run ('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phases", action="store_true", help="skip the three-call per-kernel breakdown")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


CLOCK_DATASHEET_HZ = 2.4e9   # the MI355X peak clock the datasheet peaks assume


def algorithmic(cfg, counts):
    """FLOP and minimal HBM bytes of one step and of Linear1 (see the design notes)."""
    import numpy as np
    R = int(np.sum(counts))
    active = int(np.sum(np.asarray(counts) > 0))
    uc = cfg.usecase
    b = WEIGHT_BYTES[uc]
    a_b = 2 if uc == "bf16" else 1   # activation code bytes
    H, I = cfg.H, cfg.I
    flop = 6.0 * R * H * I
    l1_flop = 4.0 * R * H * I
    w1 = active * H * 2 * I * b
    w2 = active * I * H * b
    if uc in ("fp8", "int8"):
        scales = active * (2 * I + H) * 4            # float32 per output channel
    elif uc in ("mxfp8", "mxfp4"):
        scales = active * 3 * H * I // 32            # one E8M0 byte per 32 weights
    else:
        scales = 0
    step_bytes = w1 + w2 + scales + cfg.T * H * 2 + cfg.T * H * 2 + 8 * cfg.T * cfg.K
    # Linear1 moves its weights, reads the pool rows and writes A once
    l1_bytes = w1 + R * H * a_b + R * I * a_b + (active * 2 * I * 4 if uc in ("fp8", "int8") else 0)
    return dict(R=R, flop=flop, l1_flop=l1_flop, step_bytes=step_bytes, l1_bytes=l1_bytes)


def source_digest():
    """sha256 over the HIP sources the kernels are built from."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_expert_mm_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload, kernel="mega"):
    """HBM bytes per launch of `kernel` from the committed counter summary.

    profiles/hbm_traffic.json holds FETCH_SIZE / WRITE_SIZE of the kernels
    (rocprofv3 --pmc), scaled by a plain-copy calibration.  They are only
    valid for the kernel sources they were taken on: if a source changed
    since, the traffic is unknown (None).
    """
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        prof = json.load(open(path))
    except (OSError, ValueError):
        return None
    entry = prof.get("workloads", {}).get(workload, {})
    if source_digest() != entry.get("source_sha256", prof.get("source_sha256")):
        return None
    ent = entry.get(kernel)
    return None if ent is None else ent["traffic_bytes"]


def copy_bandwidth(dev, nbytes=1 << 30, reps=10):
    """Read + write bytes per second of a plain device-to-device copy."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3), ms


def phase_breakdown(layer, x, ids, wts, steps):
    """Per-kernel milliseconds of the three-call path (same device code as
    the phases of the fused kernel), averaged over `steps` calls."""
    from mixture_experts_expert_mm_amd import binding as B
    import torch
    im = layer.new_intermediates()
    y = layer.new_y()

    def once():
        layer.dispatch(x, ids, im)
        layer.linear1(im)
        layer.linear2_combine(im, wts, y)
    once()
    torch.cuda.synchronize()
    B.mm_trace_collect()
    B.mm_trace_enable(True)
    for _ in range(steps):
        once()
    torch.cuda.synchronize()
    B.mm_trace_enable(False)
    tr = B.mm_trace_collect()
    del im, y
    layer._ws = None
    torch.cuda.empty_cache()
    return {k: v[1] / steps for k, v in tr.items() if v[0]}


def time_layer(cfg, dev, steps, warmup, with_phases):
    """Build the layer of `cfg`, warm up, time `steps` mega_moe calls.

    Returns the measurements and the inputs.  The fused kernel's duration
    comes from HIP events recorded around each of its launches on its stream
    inside the timed region; the clock from its own clock sample.
    """
    import torch
    from mixture_experts_expert_mm_amd import binding as B
    from mixture_experts_expert_mm_amd import moe
    from mixture_experts_expert_mm_amd import workloads as wl
    inp = wl.make_inputs(cfg)
    layer = moe.ExpertLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.usecase, "bf16", dev)
    layer.load_weights(inp.weights.w1, inp.weights.w2, inp.weights.s1, inp.weights.s2)
    x, ids, wts = inp.x.to(dev), inp.topk_ids.to(dev), inp.topk_weights.to(dev)
    y = layer.new_y()
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    layer.workspace(True)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        layer.forward(x, ids, wts, y, counts)
    torch.cuda.synchronize()
    B.mm_trace_collect()
    B.mm_trace_enable(True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        layer.forward(x, ids, wts, y, counts)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    B.mm_trace_enable(False)
    trace = B.mm_trace_collect()
    clocks, ticks = B.mm_read_kernel_clock(layer.plan, layer.workspace(True))
    n_k, t_k = trace["mega"]
    res = dict(ms_per_step=ev0.elapsed_time(ev1) / steps, wall=wall, kernel_ms=t_k / max(n_k, 1),
               kernels={k: v[1] / steps for k, v in trace.items() if v[0]},
               clock_hz=(clocks / ticks * 100e6) if ticks > 0 else None, counts=counts.cpu().numpy())
    if with_phases:
        res["phases"] = phase_breakdown(layer, x, ids, wts, max(2, min(steps, 10)))
    del layer, x, ids, wts, y
    torch.cuda.empty_cache()
    return res, inp


def roofline(cfg, res, copy_bps):
    """Roofline of the fused kernel: bound by MFMA when the step's arithmetic
    intensity is above the dtype's ridge, else by HBM."""
    al = algorithmic(cfg, res["counts"])
    k_s = res["kernel_ms"] * 1e-3
    peak_mfma = PEAK[cfg.usecase]
    if al["flop"] / al["step_bytes"] > peak_mfma / PEAK["hbm"]:
        ach = al["flop"] / k_s
        roof = {"bound": "mfma", "achieved": ach / 1e12, "peak": peak_mfma / 1e12, "unit": "TFLOP/s",
                "frac": ach / peak_mfma, "traffic": None}
        if res["clock_hz"]:
            roof["frac_vs_clock_peak"] = ach / (peak_mfma * res["clock_hz"] / CLOCK_DATASHEET_HZ)
    else:
        ach = al["step_bytes"] / k_s
        roof = {"bound": "hbm", "achieved": ach / 1e9, "peak": PEAK["hbm"] / 1e9, "unit": "GB/s",
                "frac": ach / PEAK["hbm"], "traffic": None}
        roof["frac_vs_copy"] = ach / copy_bps
    roof["traffic"] = measured_traffic(cfg.name)
    roof["algorithmic_bytes"] = al["step_bytes"]
    roof["algorithmic_flop"] = al["flop"]
    roof["kernel"] = "mega (fused persistent kernel: dispatch, Linear1 + SwiGLU, Linear2, combine)"
    roof["kernel_ms"] = res["kernel_ms"]
    roof["shader_clock_ghz"] = None if res["clock_hz"] is None else res["clock_hz"] / 1e9
    return roof, al


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, target_s):
    """The oracle, as it stands, on a bounded token sample of the workload."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    from mixture_experts_expert_mm_amd import workloads as wl
    cfg = inp.cfg
    w = inp.weights

    def expert(e):
        w1, w2 = w.w1[e], w.w2[e]
        if cfg.usecase in wl.MX_USECASES:
            return wl.unpack_codes(w1, cfg), wl.unpack_codes(w2, cfg), w.s1[e].numpy(), w.s2[e].numpy()
        if cfg.usecase == "fp8":
            w1, w2 = w1.view(__import__("torch").uint8), w2.view(__import__("torch").uint8)
        elif cfg.usecase == "bf16":
            w1, w2 = w1.float(), w2.float()
        return (w1.numpy(), w2.numpy(), None if w.s1 is None else w.s1[e].numpy(),
                None if w.s2 is None else w.s2[e].numpy())

    x = inp.x.float().numpy()
    ids = inp.topk_ids.numpy()
    g = inp.topk_weights.numpy()
    rng = np.random.default_rng(0)
    n = min(cfg.T, 16)
    elapsed = 0.0
    while True:
        toks = np.sort(rng.choice(cfg.T, n, replace=False))
        t0 = time.perf_counter()
        oracle.moe_forward(x, ids, g, expert, cfg.usecase, tokens=toks)
        elapsed = time.perf_counter() - t0
        if elapsed >= 0.6 * target_s or n >= cfg.T:
            break
        n = min(cfg.T, max(n * 2, int(n * target_s / max(elapsed, 1e-3) / 2)))
    R = int(np.sum(ids[toks] >= 0))
    flop = 6.0 * R * cfg.H * cfg.I
    blas = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    return {"value": flop / elapsed / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{n} of {cfg.T} tokens ({R} routes), float64 numpy/BLAS, {elapsed:.1f} s "
                      f"(includes decoding the experts' weights)",
            "blas_threads": int(blas), "cpu_model": cpu_model(), "tokens_per_s": n / elapsed}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the expert path here "
              f"runs with all experts local on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_expert_mm_amd import binding as B
    from mixture_experts_expert_mm_amd import workloads as wl

    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        bps, ms = copy_bandwidth(dev)
        print(json.dumps({"copy_bytes": 1 << 30, "copy_ms": ms, "copy_GBps_read_plus_write": bps / 1e9}))
        return
    copy_bps, _ = copy_bandwidth(dev)

    cfg = wl.CONFIGS[args.workload]
    res, inp = time_layer(cfg, dev, args.steps, args.warmup, not args.no_phases)
    roof, al = roofline(cfg, res, copy_bps)
    ms_per_step = res["ms_per_step"]
    tflops = al["flop"] / (ms_per_step * 1e-3) / 1e12
    peak_mfma = PEAK[cfg.usecase]
    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[cfg.usecase],
        "data": "synthetic (seeded randn tokens and weights, top-k of randn router scores)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "intermediate_hidden": cfg.I,
                   "num_experts": cfg.E, "topk": cfg.K, "usecase": cfg.usecase,
                   "parallelism": "none (1 GPU, all experts local)"},
        "tokens_per_s": cfg.T / (ms_per_step * 1e-3),
        "hbm_frac_step": al["step_bytes"] / (ms_per_step * 1e-3) / PEAK["hbm"],
        "mfma_frac_step": al["flop"] / (ms_per_step * 1e-3) / peak_mfma,
        "hbm_copy_GBps": copy_bps / 1e9,
        "wall_s_timed": res["wall"],
        "kernels_ms_per_step": res["kernels"],
        "three_call_phases_ms": res.get("phases"),
        "roofline": roof,
    }
    if args.hbm_workload:
        hcfg = wl.CONFIGS[args.hbm_workload]
        hres, _ = time_layer(hcfg, dev, max(args.steps, 20), args.warmup, False)
        hroof, hal = roofline(hcfg, hres, copy_bps)
        out["hbm_point"] = {
            "workload": hcfg.name, "tokens": hcfg.T, "usecase": hcfg.usecase,
            "ms_per_step": hres["ms_per_step"],
            "tokens_per_s": hcfg.T / (hres["ms_per_step"] * 1e-3),
            "TFLOP_s": hal["flop"] / (hres["ms_per_step"] * 1e-3) / 1e12,
            "hbm_frac_step": hal["step_bytes"] / (hres["ms_per_step"] * 1e-3) / PEAK["hbm"],
            "kernels_ms_per_step": hres["kernels"],
            "roofline": hroof,
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
