#!/usr/bin/env python3
"""Benchmark of the MoE grouped-GEMM hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input with
everything already resident in HBM:
    moe_quant_act -> moe_route_pack -> moe_grouped_gemm_fp8 -> moe_unpermute_combine
(plus the down-projection GEMM for the Qwen3-shaped workload, and the 4-bit
GEMM in place of the FP8 one for the INT4 workload).

Default workload: DeepSeek-V3-shaped prefill (T=4096 tokens, 256 experts,
top-8, K=7168, N=4096, FP8 E4M3 with 1x128 / 128x128 power-of-two scales,
contiguous 128-row-aligned layout).  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--cpu-baseline off]
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

METRIC = "grouped-GEMM FP8 TFLOPS (prefill) & HBM GB/s (decode), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3_prefill",
                    choices=["tiny", "dsv3_prefill", "dsv3_decode", "qwen3_skewed", "int4_decode"])
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-experts", type=int, default=128, help="experts in the timed oracle sample")
    ap.add_argument("--expected-m", type=int, default=0,
                    help="tiling hint passed to the GEMM (default: routes per expert)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times), for scaling "
                         "the HBM byte counters of a profiler run")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE counters calibrate the GEMM's."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}),
          flush=True)


KERNEL_SOURCES = {
    "moe_grouped_gemm_fp8": ["gemm_fp8.hip", "gemm_common.h", "moe_device.h", "moe_internal.h"],
    "moe_grouped_gemm_int4": ["gemm_int4.hip", "gemm_common.h", "moe_device.h", "moe_internal.h"],
}


def sources_sha256(kernel):
    """Hash of the HIP sources a kernel is built from (counter figures are valid only for these)."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int4_weights_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None.

    profiles/traffic.json holds, per kernel and workload, the calibrated byte count and the hash of the
    sources it was measured on; a kernel changed since then reports None."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as fh:
            entry = json.load(fh).get(f"{kernel}/{workload}")
    except (OSError, ValueError):
        return None
    if not entry or entry.get("sources_sha256") != sources_sha256(kernel):
        return None
    return entry["bytes_per_launch"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvent:
    """A timing-only HIP event recorded on torch's current stream (the stream every libmoe call is
    enqueued on), created with hipEventDisableSystemFence: recording it releases to device scope instead
    of writing back and invalidating the caches for the host, which would otherwise land inside the
    interval of the kernel that follows (the HIP runtime documents the flag for timing events).  The
    host reads the times after a device synchronize."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded (same soname)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = hip
        self.ctypes, self.torch = ctypes, torch
        self.ev = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        rc = HipEvent._hip.hipEventRecord(self.ev, ctypes_stream(self.torch))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = self.ctypes.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self.ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self.ev:
            HipEvent._hip.hipEventDestroy(self.ev)


def ctypes_stream(torch):
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Timer:
    """Timing-only HIP events around every kernel of every timed step."""

    def __init__(self, torch, names, steps):
        self.torch = torch
        self.names = names
        self.ev = [[HipEvent(torch) for _ in range(len(names) + 1)] for _ in range(steps)]

    def mark(self, step, i):
        self.ev[step][i].record()

    def mean_ms(self):
        out = {}
        for i, n in enumerate(self.names):
            out[n] = sum(e[i].elapsed_time(e[i + 1]) for e in self.ev) / len(self.ev)
        return out


def spin_calibration(torch):
    """Clock cycles of torch.cuda._sleep per millisecond, measured with events."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(1 << 22)
    b.record()
    torch.cuda.synchronize()
    return (1 << 22) / max(a.elapsed_time(b), 1e-3)


def fp8_weights(torch, moe, synth, cfg, N, K, stream_id, keep=()):
    """Quantised FP8 expert weights generated on the GPU, stored in the fragment-packed order
    (moe_pack_weight_fp8, prepared once like any offline weight layout); bf16 copies of `keep`
    experts on the host."""
    E = cfg.E
    codes = torch.empty(E, N, K, dtype=torch.uint8, device="cuda")
    sfw = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device="cuda")
    kept = {}
    chunk = 16
    rowmajor = torch.empty(chunk, N, K, dtype=torch.uint8, device="cuda")
    for e0 in range(0, E, chunk):
        ex = list(range(e0, min(E, e0 + chunk)))
        w = synth.expert_weights(cfg, N, K, experts=ex, stream=stream_id, device="cuda")
        moe.moe_quant_weight_fp8(w, rowmajor[:len(ex)], sfw[e0:e0 + len(ex)])
        moe.moe_pack_weight_fp8(rowmajor[:len(ex)], codes[e0:e0 + len(ex)])
        for i, e in enumerate(ex):
            if e in keep:
                kept[e] = w[i].cpu()
        del w
    torch.cuda.synchronize()
    return codes, sfw, kept


def run(args):
    import numpy as np
    import torch

    import int4_weights_amd as moe
    import synth
    from int4_weights_amd.layer import MoeFP8Layer, MoeInt4Layer

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    moe.load()
    cfg = synth.config_by_name(args.config)
    dev = "cuda"
    T, E, k, K, N = cfg.T, cfg.E, cfg.topk, cfg.K, cfg.N
    R = T * k
    ids_cpu, tw_cpu = synth.route_inputs(cfg)
    ids, tw = ids_cpu.to(dev), tw_cpu.to(dev)
    x = synth.activations(cfg, T, K).to(dev)
    counts_np = np.bincount(ids_cpu.flatten().numpy(), minlength=E)
    sample = [int(e) for e in np.argsort(-counts_np, kind="stable")[: args.cpu_experts]] if args.cpu_baseline == "on" else []
    log(f"[bench] workload {cfg.name}: T={T} E={E} top-{k} K={K} N={N} ({cfg.layout}, {cfg.weights})")

    t_setup = time.perf_counter()
    names = ["moe_quant_act", "moe_route_pack", "gemm", "moe_unpermute_combine"]
    extra = {}
    if cfg.weights == "fp8":
        codes, sfw, kept = fp8_weights(torch, moe, synth, cfg, N, K, synth.STREAM_WEIGHTS, keep=set(sample))
        layout = moe.LAYOUT_MASKED if cfg.layout == "masked" else moe.LAYOUT_CONTIGUOUS
        am = cfg.max_m if cfg.layout == "masked" else cfg.align
        em = args.expected_m or max(1, R // E)
        layer = MoeFP8Layer(codes, sfw, k, T, layout, am, expected_m=em, weights_packed=True)
        down = None
        if cfg.K_down:
            names = ["moe_quant_act", "moe_route_pack", "gemm", "moe_quant_act_down", "gemm_down",
                     "moe_unpermute_combine"]
            dcodes, dsfw, _ = fp8_weights(torch, moe, synth, cfg, cfg.N_down, cfg.K_down, synth.STREAM_WEIGHTS_DOWN)
            a_down = synth.activations(cfg, layer.rows_cap, cfg.K_down, stream=synth.STREAM_ACT_DOWN, device=dev)
            qd = torch.empty(layer.rows_cap, cfg.K_down, dtype=torch.uint8, device=dev)
            sfd = torch.empty(layer.rows_cap, cfg.K_down // 128, dtype=torch.float32, device=dev)
            Dd = torch.empty(layer.rows_cap, cfg.N_down, dtype=torch.bfloat16, device=dev)
            Zd = torch.empty(T, cfg.N_down, dtype=torch.bfloat16, device=dev)
            down = (dcodes, dsfw, a_down, qd, sfd, Dd, Zd)

        def step(tm, s):
            tm.mark(s, 0)
            layer.quant(x)
            tm.mark(s, 1)
            layer.route(ids)
            tm.mark(s, 2)
            layer.gemm()
            tm.mark(s, 3)
            if down is None:
                layer.combine(tw)
                tm.mark(s, 4)
            else:
                dcodes, dsfw, a_down, qd, sfd, Dd, Zd = down
                moe.moe_quant_act(a_down, qd, sfd)
                tm.mark(s, 4)
                layer.gemm(A=qd, SFA=sfd, D=Dd, w=dcodes, sfw=dsfw, N=cfg.N_down, K=cfg.K_down)
                tm.mark(s, 5)
                layer.combine(tw, D=Dd, Z=Zd)
                tm.mark(s, 6)
    else:
        # 4-bit weights: several copies rotate across steps so the 256 MB cache never holds the weights
        # (one allocation holds all copies, made before the generation temporaries)
        ncopy = 4
        all_q4 = torch.empty(ncopy, E, N, K // 2, dtype=torch.uint8, device=dev)
        all_s16 = torch.empty(ncopy, E, N, K // 128, dtype=torch.float16, device=dev)
        copies = []
        for c in range(ncopy):
            w = synth.expert_weights(cfg, N, K, device=dev, seed=0)
            q4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=dev)
            s16 = torch.empty(E, N, K // 128, dtype=torch.float16, device=dev)
            moe.moe_quant_weight_int4(w, q4, s16)
            del w
            moe.moe_pack_weight_int4(q4, s16, all_q4[c], all_s16[c])
            del q4, s16
            copies.append((all_q4[c], all_s16[c]))
        layer = MoeInt4Layer(copies[0][0], copies[0][1], k, T, moe.LAYOUT_MASKED, cfg.max_m,
                             expected_m=args.expected_m or max(1, R // E), weights_packed=True)
        names = ["moe_route_pack", "gemm", "moe_unpermute_combine"]

        def step(tm, s):
            q4, s16 = copies[s % ncopy]
            tm.mark(s, 0)
            layer.route(x, ids)
            tm.mark(s, 1)
            layer.gemm(q4, s16)
            tm.mark(s, 2)
            layer.combine(tw)
            tm.mark(s, 3)

    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s; warmup {args.warmup} steps")
    wt = Timer(torch, names, max(args.warmup, 1))
    for s in range(args.warmup):
        step(wt, s)
    torch.cuda.synchronize()

    # algorithmic work from the routing the device produced (read outside the timed region)
    counts = layer.counts.cpu().numpy().astype(np.int64)
    rows_valid = int(counts.sum())
    active = int((counts > 0).sum())

    # Launches go through Python, which for the decode workloads takes longer
    # than the kernels themselves.  A spin kernel holds the stream while every
    # timed launch is enqueued, so the K steps then run back to back on the GPU
    # (as from a graph or a native serving loop) and the events see kernel time,
    # not host gaps.  The spin kernel itself lies before the start event.
    cycles_per_ms = spin_calibration(torch)
    tm = Timer(torch, names, args.steps)
    start, end = HipEvent(torch), HipEvent(torch)
    t_host = time.perf_counter()
    for s in range(min(args.steps, 3)):
        step(wt, s % max(args.warmup, 1))
    host_ms = (time.perf_counter() - t_host) * 1e3 / min(args.steps, 3)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(cycles_per_ms * (5.0 + 3.0 * host_ms * args.steps)))
    start.record()
    for s in range(args.steps):
        step(tm, s)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    kern = tm.mean_ms()
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step; " + ", ".join(f"{n} {v:.3f} ms" for n, v in kern.items()))

    if cfg.weights == "fp8":
        flops = 2.0 * rows_valid * N * K
        gemm_bytes = active * N * K + active * (N // 128) * (K // 128) * 4 + rows_valid * (K + 4 * K // 128) \
            + rows_valid * N * 2
        if cfg.K_down:
            flops += 2.0 * rows_valid * cfg.N_down * cfg.K_down
        t_gemm = kern["gemm"] / 1e3
        gemm_flops = 2.0 * rows_valid * N * K
        ai = gemm_flops / gemm_bytes
        ridge = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if ai < ridge:
            roof = {"bound": "hbm", "achieved": gemm_bytes / t_gemm / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": gemm_flops / t_gemm / 1e12, "peak": FP8_PEAK_TFLOPS,
                    "unit": "TFLOP/s"}
        extra["gemm_tflops"] = gemm_flops / t_gemm / 1e12
        extra["gemm_hbm_gbs"] = gemm_bytes / t_gemm / 1e9
        extra["gemm_bytes_per_launch"] = gemm_bytes
        extra["gemm_flops_per_launch"] = gemm_flops
        if cfg.layout == "masked":
            value, unit = gemm_bytes / (ms_step / 1e3) / 1e9, "GB/s"
        else:
            value, unit = flops / (ms_step / 1e3) / 1e12, "TFLOP/s"
        dtype = "fp8_e4m3"
    else:
        gemm_bytes = active * N * (K // 2) + active * N * (K // 128) * 2 + rows_valid * K * 2 + rows_valid * N * 2
        flops = 2.0 * rows_valid * N * K
        t_gemm = kern["gemm"] / 1e3
        roof = {"bound": "hbm", "achieved": gemm_bytes / t_gemm / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        extra["gemm_hbm_gbs"] = gemm_bytes / t_gemm / 1e9
        extra["gemm_bytes_per_launch"] = gemm_bytes
        value, unit = gemm_bytes / (ms_step / 1e3) / 1e9, "GB/s"
        dtype = "int4xbf16"
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "moe_grouped_gemm_fp8" if cfg.weights == "fp8" else "moe_grouped_gemm_int4"
    roof["traffic"] = measured_traffic(roof["kernel"], cfg.name)
    roof["avg_launch_ms"] = kern["gemm"]

    cpu = None
    if args.cpu_baseline == "on" and cfg.weights == "fp8":
        cpu = cpu_baseline(np, torch, synth, cfg, ids_cpu, tw_cpu, x, kept, sample)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic: seeded router logits/activations/weights with the workload's shapes and distributions",
        "config": {"workload": cfg.name, "T": T, "E": E, "topk": k, "K": K, "N": N, "layout": cfg.layout,
                   "weights": cfg.weights, "routing": cfg.routing, "rows_valid": rows_valid,
                   "experts_active": active, "K_down": cfg.K_down or None, "N_down": cfg.N_down or None},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_ms": kern,
        **extra,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(np, torch, synth, cfg, ids_cpu, tw_cpu, x_dev, kept, sample):
    """The oracle timed on the host: the whole step restricted to a few experts."""
    import oracle
    from threadpoolctl import threadpool_info

    E, K, N = cfg.E, cfg.K, cfg.N
    ids = ids_cpu.numpy()
    xb = x_dev.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    # weights of the sample experts, quantised by the oracle (preparation, not timed)
    wq = {e: oracle.quant_weight_fp8(kept[e][None].contiguous().view(torch.int16).numpy().view(np.uint16))
          for e in sample}
    t0 = time.perf_counter()
    r = oracle.route(ids, E, "contiguous", align=cfg.align)
    tok_rows = {e: np.nonzero((ids == e).any(axis=1))[0] for e in sample}
    ys = {}
    flops = 0.0
    for e in sample:
        rows = tok_rows[e]
        a, sa = oracle.quant_act(xb[rows])
        wc, sw = wq[e]
        y = oracle.grouped_gemm_fp8(a, sa, wc, sw, np.array([len(rows)]), np.array([0, len(rows)]))
        ys[e] = (rows, y)
        flops += 2.0 * len(rows) * N * K
    # weighted combine of the sample experts' rows into their tokens
    z = {}
    for e in sample:
        rows, y = ys[e]
        for j, t in enumerate(rows):
            for s in range(cfg.topk):
                if ids[t, s] == e:
                    z[t] = z.get(t, 0.0) + float(tw_cpu[t, s]) * y[j]
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": dt, "cpu": platform.processor() or platform.machine(), "host_cpus": os.cpu_count(),
            "sample": f"{len(sample)} of {E} experts (the most loaded: {int(sum(len(ys[e][0]) for e in sample))} "
                      f"routed rows), full K={K} and N={N}: oracle routing of all {cfg.T * cfg.topk} routes, "
                      f"quantisation of the sample rows, fp64 grouped GEMM, weighted combine"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the hot path runs on one MI355X; "
                                   "multi-GPU expert parallelism is a design note, not a measured path",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    run(args)


if __name__ == "__main__":
    main()
