#!/usr/bin/env python3
"""Benchmark of the MoE grouped-GEMM hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input with
everything already resident in HBM:
    moe_route_pack_quant -> moe_grouped_gemm_fp8 -> moe_unpermute_combine
(moe_route_pack_quant quantises the bf16 token rows to 1x128 FP8 while it
routes and packs them: the same bits as moe_quant_act then moe_route_pack;
for the Qwen3-shaped workload the whole expert FFN: the up-projection with
SwiGLU and the requantisation in its epilogue (moe_grouped_gemm_fp8_swiglu),
the down-projection, then the combine; the 4-bit GEMM in place of the FP8 one
for the INT4 workload).

Default workload: DeepSeek-V3-shaped prefill (T=4096 tokens, 256 experts,
top-8, K=7168, N=4096, FP8 E4M3 with 1x128 / 128x128 power-of-two scales,
contiguous 128-row-aligned layout).  The other workloads (the Qwen3-shaped
skewed prefill, whose up-projection is the MFMA-bound GEMM, the masked FP8
decode and the 4-bit decode) are timed in the same run and reported under
"workloads", and the DeepSeek-V3-shaped steps with MXFP4, INT8 or bf16 expert
weights under "variants".  The HBM-bound rooflines are given against the
nominal 8 TB/s and, as `frac_of_measured_read`, against the rate a plain
8 GiB streaming read reaches on the same GPU (`measured_hbm_read`).  Prints
ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--also NAMES|none] [--variants LIST|none]
                    [--cpu-baseline off] [--clock off] [--ceiling off]
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import threading
import time

METRIC = "grouped-GEMM FP8 TFLOPS (prefill) & HBM GB/s (decode), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (TOP/s)
WORKLOADS = ["tiny", "dsv3_prefill", "dsv3_decode", "qwen3_skewed", "int4_decode"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3_prefill", choices=WORKLOADS)
    ap.add_argument("--also", default="qwen3_skewed,dsv3_decode,int4_decode",
                    help="further workloads timed in the same run (comma-separated, or 'none')")
    ap.add_argument("--variants", default="fp4_dsv3_decode,fp4_dsv3_prefill,int8_dsv3_decode,int8_dsv3_prefill,bf16_dsv3_decode,bf16_dsv3_prefill",
                    help="weight-format variants timed in the same run: <fp4|int8|bf16>_<workload> (or 'none')")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-experts", type=int, default=128, help="experts in the timed oracle sample")
    ap.add_argument("--ceiling", choices=["on", "off"], default="on",
                    help="time a plain 8 GiB streaming read (moe_stream_read) and report each HBM-bound kernel's "
                         "fraction of it beside the nominal peak")
    ap.add_argument("--clock", choices=["on", "off"], default="on",
                    help="sample the GPU clock over back-to-back steps after the timed ones")
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


# the files each kernel is built from (its HIP sources, the generator of its assembly, the build script)
KERNEL_SOURCES = {
    "moe_grouped_gemm_fp8": ["csrc/gemm_fp8.hip", "csrc/gen_fp8_asm.py", "csrc/gemm_common.h", "csrc/moe_device.h",
                             "csrc/moe_internal.h", "build.py"],
    "moe_grouped_gemm_fp8_swiglu": ["csrc/gemm_fp8.hip", "csrc/gen_fp8_asm.py", "csrc/gemm_common.h",
                                    "csrc/moe_device.h", "csrc/moe_internal.h", "build.py"],
    "moe_grouped_gemm_int4": ["csrc/gemm_int4.hip", "csrc/gemm_common.h", "csrc/moe_device.h", "csrc/moe_internal.h",
                              "build.py"],
    "moe_grouped_gemm_fp8_fp4": ["csrc/gemm_fp4.hip", "csrc/gemm_common.h", "csrc/moe_device.h",
                                 "csrc/moe_internal.h", "build.py"],
    "moe_grouped_gemm_int8": ["csrc/gemm_int8.hip", "csrc/gemm_common.h", "csrc/moe_device.h", "csrc/moe_internal.h",
                              "build.py"],
    "moe_grouped_gemm_bf16": ["csrc/gemm_bf16.hip", "csrc/gemm_common.h", "csrc/moe_device.h", "csrc/moe_internal.h",
                              "csrc/gen_fp8_asm.py", "build.py"],
}


def sources_sha256(kernel):
    """Hash of the files a kernel is built from (counter figures are valid only for these)."""
    import hashlib

    h = hashlib.sha256()
    pkg = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int4_weights_amd")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None.

    profiles/traffic.json holds, per kernel and workload, the calibrated byte count and the hash of the
    files it was measured on; a kernel changed since then reports None."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as fh:
            entry = json.load(fh).get(f"{kernel}/{key}")
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

    def per_kernel(self):
        """{name: [ms of each step]}"""
        return {n: [e[i].elapsed_time(e[i + 1]) for e in self.ev] for i, n in enumerate(self.names)}


def stats(xs):
    return {"mean": sum(xs) / len(xs), "median": statistics.median(xs), "min": min(xs), "max": max(xs)}


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


def fp8_gemm_roofline(rows_valid, active, N, K, t_ms, swiglu=False):
    """Algorithmic flops and bytes of one FP8 grouped-GEMM launch and where they put it on the roofline
    (swiglu: the up-projection that writes N/2 FP8 codes and N/256 scales per row instead of N bf16)."""
    flops = 2.0 * rows_valid * N * K
    out_row = (N // 2 + 4 * (N // 256)) if swiglu else 2 * N
    nbytes = active * N * K + active * (N // 128) * (K // 128) * 4 + rows_valid * (K + 4 * K // 128) \
        + rows_valid * out_row
    t = t_ms / 1e3
    ridge = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / nbytes < ridge:
        roof = {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["tflops"] = flops / t / 1e12
    roof["hbm_gbs"] = nbytes / t / 1e9
    roof["flops_per_launch"] = flops
    roof["bytes_per_launch"] = nbytes
    return roof


def build_workload(args, cfg, torch, np, moe, synth, want_cpu):
    """Buffers, weights and the step function of one workload (set-up, untimed)."""
    from int4_weights_amd.layer import MoeFP8Layer, MoeInt4Layer

    dev = "cuda"
    T, E, k, K, N = cfg.T, cfg.E, cfg.topk, cfg.K, cfg.N
    R = T * k
    ids_cpu, tw_cpu = synth.route_inputs(cfg)
    ids, tw = ids_cpu.to(dev), tw_cpu.to(dev)
    x = synth.activations(cfg, T, K).to(dev)
    counts_np = np.bincount(ids_cpu.flatten().numpy(), minlength=E)
    sample = [int(e) for e in np.argsort(-counts_np, kind="stable")[: args.cpu_experts]] if want_cpu else []
    w = {"cfg": cfg, "ids_cpu": ids_cpu, "tw_cpu": tw_cpu, "x": x, "sample": sample}
    if cfg.weights == "fp8":
        codes, sfw, kept = fp8_weights(torch, moe, synth, cfg, N, K, synth.STREAM_WEIGHTS, keep=set(sample))
        layout = moe.LAYOUT_MASKED if cfg.layout == "masked" else moe.LAYOUT_CONTIGUOUS
        am = cfg.max_m if cfg.layout == "masked" else cfg.align
        em = args.expected_m or max(1, R // E)
        layer = MoeFP8Layer(codes, sfw, k, T, layout, am, expected_m=em, weights_packed=True)
        w["kept"] = kept
        if not cfg.K_down:
            # quantisation folded into the pack (moe_route_pack_quant): one pass over the token rows
            names = ["moe_route_pack_quant", "gemm", "moe_unpermute_combine"]

            def step(tm, s):
                tm.mark(s, 0)
                layer.quant_route(x, ids)
                tm.mark(s, 1)
                layer.gemm()
                tm.mark(s, 2)
                layer.combine(tw)
                tm.mark(s, 3)
        else:
            # the whole expert FFN: up-projection (gate and up columns) with SwiGLU + requantisation in its
            # epilogue, down-projection
            names = ["moe_route_pack_quant", "gemm", "gemm_down", "moe_unpermute_combine"]
            assert N == 2 * cfg.K_down
            dcodes, dsfw, _ = fp8_weights(torch, moe, synth, cfg, cfg.N_down, cfg.K_down, synth.STREAM_WEIGHTS_DOWN)
            qd = torch.empty(layer.rows_cap, cfg.K_down, dtype=torch.uint8, device=dev)
            sfd = torch.empty(layer.rows_cap, cfg.K_down // 128, dtype=torch.float32, device=dev)
            Dd = torch.empty(layer.rows_cap, cfg.N_down, dtype=torch.bfloat16, device=dev)
            Zd = torch.empty(T, cfg.N_down, dtype=torch.bfloat16, device=dev)

            def step(tm, s):
                tm.mark(s, 0)
                layer.quant_route(x, ids)
                tm.mark(s, 1)
                layer.gemm_swiglu(qd, sfd)
                tm.mark(s, 2)
                layer.gemm(A=qd, SFA=sfd, D=Dd, w=dcodes, sfw=dsfw, N=cfg.N_down, K=cfg.K_down)
                tm.mark(s, 3)
                layer.combine(tw, D=Dd, Z=Zd)
                tm.mark(s, 4)
    else:
        # 4-bit weights: several copies rotate across steps so the 256 MB cache never holds the weights
        # (one allocation holds all copies, made before the generation temporaries)
        ncopy = 4
        all_q4 = torch.empty(ncopy, E, N, K // 2, dtype=torch.uint8, device=dev)
        all_s16 = torch.empty(ncopy, E, N, K // 128, dtype=torch.float16, device=dev)
        copies = []
        kept = {}
        for c in range(ncopy):
            wb = synth.expert_weights(cfg, N, K, device=dev, seed=0)
            if c == 0:
                kept = {e: wb[e].cpu() for e in sample}
            q4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=dev)
            s16 = torch.empty(E, N, K // 128, dtype=torch.float16, device=dev)
            moe.moe_quant_weight_int4(wb, q4, s16)
            del wb
            moe.moe_pack_weight_int4(q4, s16, all_q4[c], all_s16[c])
            del q4, s16
            copies.append((all_q4[c], all_s16[c]))
        layer = MoeInt4Layer(copies[0][0], copies[0][1], k, T, moe.LAYOUT_MASKED, cfg.max_m,
                             expected_m=args.expected_m or max(1, R // E), weights_packed=True)
        names = ["moe_route_pack", "gemm", "moe_unpermute_combine"]
        w["kept"] = kept

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
    w.update(layer=layer, names=names, step=step)
    return w


def build_variant(args, fmt, cfg, torch, np, moe, synth):
    """The same routing and step as the FP8 workload, with the expert weights in another format:
    fp4 -- MXFP4 weights (E2M1 codes, one E8M0 scale per 32 K values) x FP8 activations;
    int8 -- INT8 (1, 1, 128) activations and weights (per-row / per-channel fp32 scales per 128 K);
    bf16 -- bf16 weights x bf16 activations (the rows are packed as bf16, no quantisation)."""
    dev = "cuda"
    T, E, k, K, N = cfg.T, cfg.E, cfg.topk, cfg.K, cfg.N
    ids_cpu, tw_cpu = synth.route_inputs(cfg)
    ids, tw = ids_cpu.to(dev), tw_cpu.to(dev)
    x = synth.activations(cfg, T, K).to(dev)
    layout = moe.LAYOUT_MASKED if cfg.layout == "masked" else moe.LAYOUT_CONTIGUOUS
    am = cfg.max_m if cfg.layout == "masked" else cfg.align
    rows_cap = moe.moe_packed_rows_cap(T, k, E, am) if layout == moe.LAYOUT_CONTIGUOUS else E * am
    em = args.expected_m or max(1, T * k // E)
    counts = torch.zeros(E, dtype=torch.int32, device=dev)
    seg = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    mi = torch.empty(rows_cap, dtype=torch.int32, device=dev)
    oi = torch.empty(T, k, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(moe.moe_route_pack_workspace_bytes(T, k, E), 16), dtype=torch.uint8, device=dev)
    D = torch.empty(rows_cap, N, dtype=torch.bfloat16, device=dev)
    Z = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    am_gemm = am if layout == moe.LAYOUT_MASKED else rows_cap
    if fmt == "fp4":
        # MXFP4 weights in the fragment-packed order (moe_pack_weight_fp4, prepared once)
        W4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=dev)
        SW = torch.empty(E, N, K // 32, dtype=torch.uint8, device=dev)
        r4 = torch.empty(16, N, K // 2, dtype=torch.uint8, device=dev)
        rs = torch.empty(16, N, K // 32, dtype=torch.uint8, device=dev)
        for e0 in range(0, E, 16):
            ex = list(range(e0, min(E, e0 + 16)))
            w = synth.expert_weights(cfg, N, K, experts=ex, stream=synth.STREAM_WEIGHTS, device=dev)
            moe.moe_quant_weight_fp4(w, r4[:len(ex)], rs[:len(ex)])
            moe.moe_pack_weight_fp4(r4[:len(ex)], rs[:len(ex)], W4[e0:e0 + len(ex)], SW[e0:e0 + len(ex)])
            del w
        P = torch.empty(rows_cap, K, dtype=torch.uint8, device=dev)
        Psf = torch.empty(rows_cap, K // 128, dtype=torch.float32, device=dev)
        names = ["moe_route_pack_quant", "gemm", "moe_unpermute_combine"]

        def step(tm, s):
            tm.mark(s, 0)
            moe.moe_route_pack_quant(ids, E, layout, am, x, P, Psf, counts, seg, mi, oi, st, workspace=ws)
            tm.mark(s, 1)
            moe.moe_grouped_gemm_fp8_fp4(layout | moe.WEIGHTS_PACKED, P, Psf, W4, SW, D, counts, seg, E, am_gemm, N, K,
                                         em)
            tm.mark(s, 2)
            moe.moe_unpermute_combine(D, oi, tw, Z)
            tm.mark(s, 3)
    elif fmt == "int8":
        # INT8 codes in moe_pack_weight_fp8's fragment order, per-channel scales K-block-major (prepared once)
        W8 = torch.empty(E, N, K, dtype=torch.uint8, device=dev)
        SW = torch.empty(E, K // 128, N, dtype=torch.float32, device=dev)
        r8 = torch.empty(16, N, K, dtype=torch.int8, device=dev)
        for e0 in range(0, E, 16):
            ex = list(range(e0, min(E, e0 + 16)))
            w = synth.expert_weights(cfg, N, K, experts=ex, stream=synth.STREAM_WEIGHTS, device=dev)
            moe.moe_quant_weight_int8(w, r8[:len(ex)], SW[e0:e0 + len(ex)])
            moe.moe_pack_weight_fp8(r8[:len(ex)].view(torch.uint8), W8[e0:e0 + len(ex)])
            del w
        del r8
        q = torch.empty(T, K, dtype=torch.int8, device=dev)
        sf = torch.empty(T, K // 128, dtype=torch.float32, device=dev)
        P = torch.empty(rows_cap, K, dtype=torch.int8, device=dev)
        Psf = torch.empty(rows_cap, K // 128, dtype=torch.float32, device=dev)
        names = ["moe_quant_act_int8", "moe_route_pack", "gemm", "moe_unpermute_combine"]

        def step(tm, s):
            tm.mark(s, 0)
            moe.moe_quant_act_int8(x, q, sf)
            tm.mark(s, 1)
            moe.moe_route_pack(ids, E, layout, am, q, P, counts, seg, mi, oi, st, payload2=sf, packed2=Psf,
                               workspace=ws)
            tm.mark(s, 2)
            moe.moe_grouped_gemm_int8(layout | moe.WEIGHTS_PACKED, P, Psf, W8, SW, D, counts, seg, E, am_gemm, N, K,
                                      em)
            tm.mark(s, 3)
            moe.moe_unpermute_combine(D, oi, tw, Z)
            tm.mark(s, 4)
    else:
        # bf16 weights in the fragment-packed order (moe_pack_weight_bf16, prepared once)
        W = torch.empty(E, N, K, dtype=torch.bfloat16, device=dev)
        for e0 in range(0, E, 16):
            w = synth.expert_weights(cfg, N, K, experts=range(e0, min(E, e0 + 16)), stream=synth.STREAM_WEIGHTS,
                                     device=dev)
            moe.moe_pack_weight_bf16(w, W[e0:e0 + w.shape[0]])
            del w
        P = torch.empty(rows_cap, K, dtype=torch.bfloat16, device=dev)
        names = ["moe_route_pack", "gemm", "moe_unpermute_combine"]

        def step(tm, s):
            tm.mark(s, 0)
            moe.moe_route_pack(ids, E, layout, am, x, P, counts, seg, mi, oi, st, workspace=ws)
            tm.mark(s, 1)
            moe.moe_grouped_gemm_bf16(layout | moe.WEIGHTS_PACKED, P, W, D, counts, seg, E, am_gemm, N, K, em)
            tm.mark(s, 2)
            moe.moe_unpermute_combine(D, oi, tw, Z)
            tm.mark(s, 3)
    torch.cuda.synchronize()

    class _L:  # what summarise reads of a layer
        pass

    layer = _L()
    layer.counts = counts
    return {"cfg": cfg, "layer": layer, "names": names, "step": step, "fmt": fmt}


def summarise_variant(np, wl, ms_step, per, host_ms):
    cfg, fmt = wl["cfg"], wl["fmt"]
    E, K, N = cfg.E, cfg.K, cfg.N
    counts = wl["layer"].counts.cpu().numpy().astype(np.int64)
    rows_valid, active = int(counts.sum()), int((counts > 0).sum())
    kern = {n: stats(v) for n, v in per.items()}
    t = kern["gemm"]["mean"] / 1e3
    flops = 2.0 * rows_valid * N * K
    if fmt == "fp4":
        nbytes = active * N * (K // 2 + K // 32) + rows_valid * (K + 4 * K // 128) + rows_valid * N * 2
        peak_f, kernel = FP8_PEAK_TFLOPS, "moe_grouped_gemm_fp8_fp4"
    elif fmt == "int8":
        nbytes = active * N * K * (1 + 4 / 128) + rows_valid * (K + 4 * K // 128) + rows_valid * N * 2
        peak_f, kernel = INT8_PEAK_TOPS, "moe_grouped_gemm_int8"
    else:
        nbytes = active * N * K * 2 + rows_valid * K * 2 + rows_valid * N * 2
        peak_f, kernel = BF16_PEAK_TFLOPS, "moe_grouped_gemm_bf16"
    ridge = peak_f * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / nbytes < ridge:
        roof = {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": peak_f,
                "unit": "TOP/s" if fmt == "int8" else "TFLOP/s"}
    roof.update(frac=roof["achieved"] / roof["peak"], tflops=flops / t / 1e12, hbm_gbs=nbytes / t / 1e9,
                flops_per_launch=flops, bytes_per_launch=nbytes, kernel=kernel, avg_launch_ms=kern["gemm"]["mean"],
                median_launch_ms=kern["gemm"]["median"], min_launch_ms=kern["gemm"]["min"],
                traffic=measured_traffic(kernel, f"{fmt}_{cfg.name}"))
    return {"ms_per_step": ms_step, "kernels_ms": kern, "roofline": roof,
            "dtype": {"fp4": "fp8xe2m1", "int8": "int8"}.get(fmt, "bf16"), "config": {"workload": cfg.name, "weights": fmt, "T": cfg.T, "E": E, "topk": cfg.topk, "K": K,
                               "N": N, "layout": cfg.layout, "rows_valid": rows_valid, "experts_active": active},
            "host_enqueue_ms_per_step": host_ms}


def time_workload(args, torch, wl, cycles_per_ms):
    """Warm-up, then exactly args.steps timed steps back to back; per-kernel event times of every step."""
    names, step = wl["names"], wl["step"]
    wt = Timer(torch, names, max(args.warmup, 1))
    for s in range(args.warmup):
        step(wt, s)
    torch.cuda.synchronize()
    # Launches go through Python, which for the decode workloads takes longer
    # than the kernels themselves.  A spin kernel holds the stream while every
    # timed launch is enqueued, so the K steps then run back to back on the GPU
    # (as from a graph or a native serving loop) and the events see kernel time,
    # not host gaps.  The spin kernel itself lies before the start event.
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
    return start.elapsed_time(end) / args.steps, tm.per_kernel(), host_ms


def clock_pass(torch, wl, seconds=2.2):
    """GPU clock (MHz) while steps run back to back.  The SMI's current GFX clock is refreshed about once a
    second (each value covers the preceding interval), so the pass runs for a little over two seconds, the
    value is read every 10 ms, and only the values published after the pass started are kept."""
    samples, stop = [], threading.Event()
    try:
        torch.cuda.clock_rate()
    except Exception as e:  # no SMI access on this machine
        return {"error": f"clock not readable: {type(e).__name__}"}

    def sampler():
        while not stop.is_set():
            try:
                samples.append(float(torch.cuda.clock_rate()))
            except Exception:
                pass
            time.sleep(0.01)

    tm = Timer(torch, wl["names"], 1)
    th = threading.Thread(target=sampler, daemon=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        wl["step"](tm, 0)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()  # keep the host at most a few steps ahead
    torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return {"error": "no samples"}
    # drop the value current when the pass started (it covers the time before it)
    first_change = next((i for i, v in enumerate(samples) if v != samples[0]), None)
    if first_change is None:
        return {"median_mhz": samples[0], "min_mhz": samples[0], "max_mhz": samples[0], "updates": 0, "steps": n,
                "note": "the SMI value did not change during the pass",
                "source": "torch.cuda.clock_rate() (SMI current GFX clock, refreshed about once a second)"}
    busy = samples[first_change:]
    updates = 1 + sum(1 for a, b in zip(busy, busy[1:]) if a != b)
    return {"median_mhz": statistics.median(busy), "min_mhz": min(busy), "max_mhz": max(busy), "updates": updates,
            "steps": n, "source": "torch.cuda.clock_rate() (SMI current GFX clock, refreshed about once a second), "
                                  "read every 10 ms over back-to-back steps; the value current at the start dropped"}


def summarise(args, np, wl, ms_step, per, host_ms, clock):
    """The result dict of one workload (value, rooflines, per-kernel statistics)."""
    cfg, layer = wl["cfg"], wl["layer"]
    T, E, k, K, N = cfg.T, cfg.E, cfg.topk, cfg.K, cfg.N
    counts = layer.counts.cpu().numpy().astype(np.int64)
    rows_valid = int(counts.sum())
    active = int((counts > 0).sum())
    kern = {n: stats(v) for n, v in per.items()}
    out = {"ms_per_step": ms_step, "kernels_ms": kern}
    if cfg.weights == "fp8":
        roof = fp8_gemm_roofline(rows_valid, active, N, K, kern["gemm"]["mean"], swiglu=bool(cfg.K_down))
        flops = roof["flops_per_launch"]
        if cfg.K_down:
            rd = fp8_gemm_roofline(rows_valid, active, cfg.N_down, cfg.K_down, kern["gemm_down"]["mean"])
            rd.update(kernel="moe_grouped_gemm_fp8", avg_launch_ms=kern["gemm_down"]["mean"],
                      median_launch_ms=kern["gemm_down"]["median"], min_launch_ms=kern["gemm_down"]["min"],
                      traffic=measured_traffic("moe_grouped_gemm_fp8", cfg.name + "_down"))
            out["roofline_down"] = rd
            flops += rd["flops_per_launch"]
        if cfg.layout == "masked":
            value, unit = roof["bytes_per_launch"] / (ms_step / 1e3) / 1e9, "GB/s"
        else:
            value, unit = flops / (ms_step / 1e3) / 1e12, "TFLOP/s"
        dtype = "fp8_e4m3"
        kernel = "moe_grouped_gemm_fp8_swiglu" if cfg.K_down else "moe_grouped_gemm_fp8"
    else:
        nbytes = active * N * (K // 2) + active * N * (K // 128) * 2 + rows_valid * K * 2 + rows_valid * N * 2
        t = kern["gemm"]["mean"] / 1e3
        roof = {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": nbytes / t / 1e9 / HBM_PEAK_GBS, "hbm_gbs": nbytes / t / 1e9, "bytes_per_launch": nbytes,
                "flops_per_launch": 2.0 * rows_valid * N * K}
        value, unit = nbytes / (ms_step / 1e3) / 1e9, "GB/s"
        dtype = "int4xbf16"
        kernel = "moe_grouped_gemm_int4"
    roof.update(kernel=kernel, avg_launch_ms=kern["gemm"]["mean"], median_launch_ms=kern["gemm"]["median"],
                min_launch_ms=kern["gemm"]["min"], traffic=measured_traffic(kernel, cfg.name))
    out.update(value=value, unit=unit, dtype=dtype, roofline=roof,
               config={"workload": cfg.name, "T": T, "E": E, "topk": k, "K": K, "N": N, "layout": cfg.layout,
                       "weights": cfg.weights, "routing": cfg.routing, "rows_valid": rows_valid,
                       "experts_active": active, "K_down": cfg.K_down or None, "N_down": cfg.N_down or None},
               clock=clock, host_enqueue_ms_per_step=host_ms)
    return out


def run(args):
    import numpy as np
    import torch

    import int4_weights_amd as moe
    import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    moe.load()
    also = [] if args.also in ("", "none") else [a for a in args.also.split(",") if a and a != args.config]
    for a in also:
        if a not in WORKLOADS:
            raise SystemExit(f"unknown workload {a}")
    cycles_per_ms = spin_calibration(torch)
    results = {}
    cpu = None
    for i, name in enumerate([args.config] + also):
        cfg = synth.config_by_name(name)
        primary = i == 0
        log(f"[bench] workload {cfg.name}: T={cfg.T} E={cfg.E} top-{cfg.topk} K={cfg.K} N={cfg.N} "
            f"({cfg.layout}, {cfg.weights})")
        t_setup = time.perf_counter()
        wl = build_workload(args, cfg, torch, np, moe, synth, primary and args.cpu_baseline == "on")
        log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s; warmup {args.warmup}, timed {args.steps} steps")
        ms_step, per, host_ms = time_workload(args, torch, wl, cycles_per_ms)
        clock = clock_pass(torch, wl) if args.clock == "on" else None
        res = summarise(args, np, wl, ms_step, per, host_ms, clock)
        log(f"[bench] {name}: {ms_step:.3f} ms/step; " +
            ", ".join(f"{n} {v['median']:.3f} ms" for n, v in res["kernels_ms"].items()) +
            (f"; clock {clock.get('median_mhz')} MHz" if clock else ""))
        if primary and args.cpu_baseline == "on":
            cpu = cpu_baseline(np, torch, wl)
            log(f"[bench] oracle on the host: {cpu['value']:.4f} {cpu['unit']} ({cpu['seconds']:.1f} s)")
        results[name] = res
        del wl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    variants = {}
    for v in ([] if args.variants in ("", "none") else args.variants.split(",")):
        fmt, _, name = v.partition("_")
        if fmt not in ("fp4", "int8", "bf16") or name not in WORKLOADS or synth.config_by_name(name).weights != "fp8":
            raise SystemExit(f"unknown variant {v}")
        t_setup = time.perf_counter()
        wl = build_variant(args, fmt, synth.config_by_name(name), torch, np, moe, synth)
        log(f"[bench] variant {v}: setup {time.perf_counter() - t_setup:.1f}s")
        ms_step, per, host_ms = time_workload(args, torch, wl, cycles_per_ms)
        res = summarise_variant(np, wl, ms_step, per, host_ms)
        log(f"[bench] {v}: {ms_step:.3f} ms/step; " +
            ", ".join(f"{n} {x['median']:.3f} ms" for n, x in res["kernels_ms"].items()) +
            f"; GEMM {res['roofline']['frac'] * 100:.1f}% of the {res['roofline']['bound']} roofline")
        variants[v] = res
        del wl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    ceiling = stream_ceiling(torch, moe) if args.ceiling == "on" else None
    if ceiling and "read_gbs" in ceiling:
        log(f"[bench] HBM streaming read (moe_stream_read, {ceiling['bytes'] / 2**30:.0f} GiB): "
            f"{ceiling['read_gbs']:.0f} GB/s")
        for r in list(results.values()) + list(variants.values()):
            for key in ("roofline", "roofline_down"):
                roof = r.get(key)
                if roof and roof.get("bound") == "hbm":
                    roof["frac_of_measured_read"] = roof["achieved"] / ceiling["read_gbs"]

    p = results[args.config]
    out = {
        "metric": METRIC,
        "value": p["value"],
        "unit": p["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": p["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p["dtype"],
        "data": "synthetic: seeded router logits/activations/weights with the workload's shapes and distributions",
        "config": p["config"],
        "roofline": p["roofline"],
        "cpu_baseline": cpu,
        "kernels_ms": p["kernels_ms"],
        "clock": p["clock"],
    }
    if "roofline_down" in p:
        out["roofline_down"] = p["roofline_down"]
    out["workloads"] = {n: {kk: v for kk, v in r.items()} for n, r in results.items() if n != args.config}
    out["variants"] = variants
    out["measured_hbm_read"] = ceiling
    print(json.dumps(out), flush=True)


def stream_ceiling(torch, moe, gib=8, reps=5):
    """The HBM read rate a plain streaming kernel (moe_stream_read) reaches on this GPU: GB/s over a `gib` GiB
    buffer, the median of `reps` event-timed launches after one untimed."""
    nbytes = gib << 30
    try:
        buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    except RuntimeError as e:  # not enough free memory
        return {"error": f"no {gib} GiB buffer: {type(e).__name__}"}
    words = torch.empty(moe.moe_stream_read_words(), dtype=torch.int32, device="cuda")
    moe.moe_stream_read(buf, words)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_stream_read(buf, words)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del buf
    torch.cuda.empty_cache()
    ms = statistics.median(times)
    return {"read_gbs": nbytes / ms / 1e6, "bytes": nbytes, "median_ms": ms, "min_ms": min(times), "reps": reps,
            "method": "moe_stream_read: every byte read once with 16-byte nontemporal loads, 8 in flight per lane, "
                      "one 256-lane workgroup per CU; HIP events around each launch"}


def cpu_baseline(np, torch, wl):
    """The oracle timed on the host: the whole step restricted to the most-loaded experts."""
    import oracle
    from threadpoolctl import threadpool_info

    cfg, ids_cpu, tw_cpu, kept, sample = wl["cfg"], wl["ids_cpu"], wl["tw_cpu"], wl["kept"], wl["sample"]
    E, K, N = cfg.E, cfg.K, cfg.N
    ids = ids_cpu.numpy()
    xb = wl["x"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    bits = {e: kept[e][None].contiguous().view(torch.int16).numpy().view(np.uint16) for e in sample}
    # weights of the sample experts, quantised by the oracle (preparation, not timed)
    if cfg.weights == "fp8":
        wq = {e: oracle.quant_weight_fp8(bits[e]) for e in sample}
    else:
        wq = {e: oracle.quant_weight_int4(bits[e]) for e in sample}
    layout = "masked" if cfg.layout == "masked" else "contiguous"
    kw = {"max_m": cfg.max_m} if layout == "masked" else {"align": cfg.align}
    t0 = time.perf_counter()
    r = oracle.route(ids, E, layout, **kw)
    tok_rows = {e: np.nonzero((ids == e).any(axis=1))[0] for e in sample}
    ys = {}
    flops = 0.0
    nbytes = 0.0
    for e in sample:
        rows = tok_rows[e]
        if cfg.weights == "fp8":
            a, sa = oracle.quant_act(xb[rows])
            wc, sw = wq[e]
            y = oracle.grouped_gemm_fp8(a, sa, wc, sw, np.array([len(rows)]), np.array([0, len(rows)]))
            nbytes += N * K + len(rows) * (K + N * 2)
        else:
            q4, s4 = wq[e]
            y = oracle.grouped_gemm_int4(xb[rows], q4, s4, np.array([len(rows)]), np.array([0, len(rows)]))
            nbytes += N * K // 2 + N * (K // 128) * 2 + len(rows) * (2 * K + 2 * N)
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
    nrows = int(sum(len(ys[e][0]) for e in sample))
    desc = (f"{len(sample)} of {E} experts (the most loaded: {nrows} routed rows), full K={K} and N={N}: oracle "
            f"routing of all {cfg.T * cfg.topk} routes, " +
            ("quantisation of the sample rows, fp64 grouped GEMM" if cfg.weights == "fp8"
             else "fp64 4-bit weight-only grouped GEMM (dequantised weights)") + ", weighted combine")
    if cfg.layout == "masked" or cfg.weights == "int4":
        value, unit = nbytes / dt / 1e9, "GB/s"
    else:
        value, unit = flops / dt / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "seconds": dt,
            "tflops": flops / dt / 1e12, "cpu": platform.processor() or platform.machine(),
            "host_cpus": os.cpu_count(), "sample": desc}


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
