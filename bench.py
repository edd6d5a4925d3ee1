#!/usr/bin/env python3
"""Throughput of the S3D8 weight-decode-fused linear layer on one MI355X.

Headline workload: the decode-step GEMV of the Llama-3.2-11B text MLP
gate/up shape, M=1 token, K=4096, N=14336 (Y = X W^T), S3D8 weights packed
by the library's packer from N(0, 0.02) fp32 weights, activations N(0,1)
quantised per token on the GPU.  One step = s3d8_forward on one token (one
launch of the streaming GEMV, which quantises the activations in its
prologue), inputs resident in HBM.  The metric is effective weight GB/s:
the S3D8 bytes of the matrix (packed bytes + bf16 channel scales + the
96-byte table) per step time.

To keep the weights out of the 256 MB Infinity Cache the step cycles
through R distinct device copies of the packed matrix (the pages' own
practice of cycling source tensors), R * 19.6 MB >= 2 x 256 MB.  The steps
are captured once in a HIP graph (R steps, one per copy) and replayed, so
host launch overhead does not enter the timed region.

Also reported: the prefill GEMM (M=2048, K=4096, N=14336) in INT8 TOPS
against the INT8 MFMA peak, the same GEMM on the lm_head at 512 tokens and
the vision MLP at 1601 tokens, the dominant kernel's roofline fraction, the
per-call median with a bootstrap interval, measured HBM and INT8 ceilings,
the decode step at M=4 and 8, the decoder layer, the lm_head decode step,
the format and output variants, the standalone dequantisation and device
encoder, and the CPU oracle timed on the host cores (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line on stdout; progress goes to stderr.
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

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA, 5.0 POPS
MALL_BYTES = 256 * 2 ** 20   # Infinity Cache
METRIC = "effective weight GB/s (% HBM peak) at M=1; INT8 TOPS (% MFMA peak) at M=2048"
SETTLE_S = 0.2     # sustained load before the headline region (clock settle)
NSAMPLES = 200     # per-call samples behind the median and its interval
SAMPLE_REPS = 5    # replays of the R-step sequence per sample
BUSY_REPS = 10     # R-step sequences queued ahead of the timed region

# The pages' own throughput figures for this layer, all on Arm CPUs, quoted as
# context (GMAC/s of the fused S3D8 kernel at m = 1, of the S3D8 -> INT8 path
# at m = 128; the paper's Table 2 and Appendix table, the blog's "Fast? How
# fast?" section).  Not a target: other hardware, other precision of timing.
PAGES_CONTEXT = [
    {"shape_mkn": [1, 4096, 14336], "hardware": "Google Pixel 8a, 5 cores", "s3d8_GMACs": 33.8,
     "int8_GMACs": 26.5, "bf16_GMACs": 13.6, "source": "paper Table 2 (text.mlp.up); blog 'Fast? How fast?'"},
    {"shape_mkn": [1, 4096, 14336], "hardware": "AWS Graviton4, 96 Neoverse V2 cores", "s3d8_GMACs": 1031,
     "int8_GMACs": 461, "bf16_GMACs": 236, "source": "paper Appendix table (Graviton4)"},
    {"shape_mkn": [128, 4096, 14336], "hardware": "Google Pixel 8a, 5 cores", "s3d8_GMACs": 197.7,
     "int8_GMACs": 201.1, "bf16_GMACs": 76.3, "source": "paper Table 2 (text.mlp.up, m = 128)"},
    {"shape_mkn": [128, 4096, 14336], "hardware": "AWS Graviton4, 96 Neoverse V2 cores", "s3d8_GMACs": 6994,
     "int8_GMACs": 7700, "bf16_GMACs": 3492, "source": "paper Appendix table (Graviton4)"},
    {"shape_mkn": [1601, 1280, 5120], "hardware": "Google Pixel 8a, 5 cores", "s3d8_GMACs": 211.8,
     "int8_GMACs": 206.1, "bf16_GMACs": 116.5, "source": "paper Table 2 (vision.mlp.up)"},
]


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha():
    """Hash of the kernel source with comments and whitespace removed, so
    that counters taken on it stay valid across comment-only edits."""
    import re
    with open(os.path.join(ROOT, "w2_a8_matmul_amd", "csrc", "s3d8_kernels.hip")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(name, launches_bytes):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, only if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def bootstrap_ci(samples, n_boot=2000, seed=0):
    """95 % percentile-bootstrap interval of the median of `samples`."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, len(samples), size=(n_boot, len(samples)))
    med = np.median(np.asarray(samples)[idx], axis=1)
    return float(np.percentile(med, 2.5)), float(np.percentile(med, 97.5))


def graph_launch_us(torch, fns, reps, warm_s=0.1):
    """Average duration of one call: the calls fns[0..n-1] are captured back
    to back in one HIP graph, replayed `reps` times between two events on
    the launching stream; the interval over n * reps calls includes no host
    time, only the kernels and the gaps between consecutive dispatches.  For
    calls of one kernel launch each this is the kernel's average duration.
    Before the timed replays the graph is replayed for `warm_s` seconds: the
    GPU's clocks take a few tens of milliseconds of sustained load to settle
    (the prefill GEMM runs about 15 % slower in the first 20 ms)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_s
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    g.replay()  # untimed: keeps the GPU busy while the timed replays are submitted
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * len(fns))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # (the warm-up steps are followed by a time-based settle, SETTLE_S)
    ap.add_argument("--steps", type=int, default=5600)
    ap.add_argument("--warmup", type=int, default=280)
    ap.add_argument("--pack-iters", type=int, default=25)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the S3D8 linear runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import w2_a8_matmul_amd as s3d8
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- decode GEMV workload
    lin = workloads.C1[1]
    M, K, N = lin.M, lin.K, lin.N
    T = s3d8.num_triples(N)
    weight_bytes = s3d8.format_bytes(N, K)                   # 19,603,554
    # the fused step kernel reads the weights and fp32 x, writes xq, xs and y
    kernel_bytes = weight_bytes + 4 * M * K + M * K + 4 * M + 4 * M * N
    log(f"workload {lin.name}: M={M} K={K} N={N}, {weight_bytes} S3D8 bytes")
    t0 = time.time()
    W = workloads.weights(lin)
    C, scales, packed = s3d8.pack(W, seed=lin.pack_seed, max_iters=args.pack_iters)
    del W
    log(f"packed in {time.time() - t0:.1f}s")
    R = int(np.ceil(2 * MALL_BYTES / weight_bytes))
    R = max(R, 2)
    dC = torch.from_numpy(C).to(dev)
    dS = torch.from_numpy(scales.view(np.int16)).to(dev)
    tiled0 = s3d8.tile(torch.from_numpy(packed).to(dev), N)
    dP = [tiled0.clone() for _ in range(R)]
    del tiled0
    xs_host = workloads.activations(lin)
    dX = [torch.from_numpy(xs_host).to(dev) for _ in range(R)]
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xsc = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def step(r):
        s3d8.forward(dX[r], dP[r], dC, dS, N, y=y, xq=xq, xs=xsc)

    # eager warm-up, then capture R steps in one graph
    for i in range(3):
        step(i % R)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(R):
            step(r)
    # a longer untimed sequence that keeps the GPU busy while the host
    # submits the timed steps (see below)
    busy = torch.cuda.CUDAGraph()
    with torch.cuda.graph(busy):
        for _ in range(BUSY_REPS):
            for r in range(R):
                step(r)
    torch.cuda.synchronize()

    # warm-up: the W steps asked for (whole replays of the R-step graph),
    # then replays until SETTLE_S seconds of sustained load have passed,
    # whatever W is: the clocks take a few tens of milliseconds to settle
    for i in range(max(1, -(-args.warmup // R))):
        graph.replay()
    torch.cuda.synchronize()
    t_settle = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_settle:
        graph.replay()
        torch.cuda.synchronize()
    log(f"timing {args.steps} steps (graph of {R} steps, R={R} weight copies)")
    # the timed region: exactly `steps` launches between two events on the
    # launching stream: steps // R replays of the R-step graph, then the
    # remaining steps % R as direct calls.  An untimed sequence of BUSY_REPS
    # * R steps is queued in front of the start event, after the
    # synchronisation, so that the GPU is still busy with it while the host
    # submits the timed launches: the region then holds the steps' GPU time
    # and not host submission.  (Direct calls, not a graph, for the remainder:
    # every graph replay carries a fixed cost of several microseconds, which a
    # region of only a few steps would otherwise show.)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    busy.replay()
    start.record()
    for i in range(args.steps // R):
        graph.replay()
    for r in range(args.steps % R):
        step(r)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    value = weight_bytes / (ms_per_step * 1e-3) / 1e9
    # per-call samples for the median and its 95 % bootstrap interval (the
    # pages' own statistic): NSAMPLES replays of a graph of SAMPLE_REPS * R
    # launches, an event after each, whatever `steps` is
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs):
        for _ in range(SAMPLE_REPS):
            for r in range(R):
                step(r)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(NSAMPLES + 1)]
    gs.replay()
    marks[0].record()
    for i in range(NSAMPLES):
        gs.replay()
        marks[i + 1].record()
    torch.cuda.synchronize()
    per_call = np.array([marks[i].elapsed_time(marks[i + 1]) * 1e3 / (SAMPLE_REPS * R) for i in range(NSAMPLES)])
    ci = bootstrap_ci(per_call)
    timing = {"samples": NSAMPLES, "launches_per_sample": SAMPLE_REPS * R, "settle_s": SETTLE_S,
              "per_call_us_median": round(float(np.median(per_call)), 3),
              "per_call_us_ci95": [round(v, 3) for v in ci],
              "per_call_us_min_max": [round(float(per_call.min()), 3), round(float(per_call.max()), 3)],
              "timed_region_us_per_step": round(ms_per_step * 1e3, 3)}

    # dominant kernel: the fused quantise + decode GEMV launched by
    # s3d8_forward.  At M=1 a step is exactly one launch of it, so its
    # average duration is the timed region over the launches in it.
    lin_mean_us = ms_per_step * 1e3
    achieved = kernel_bytes / (lin_mean_us * 1e-6) / 1e9
    traffic = measured_traffic("gemv_c1_m1", kernel_bytes)
    # standalone quantisation kernel (used by s3d8_linear callers), for reference
    qa_mean_us = graph_launch_us(torch, [lambda r=r: s3d8.quant_act(dX[r], xq, xsc) for r in range(R)], 10)
    log(f"step {ms_per_step * 1e3:.2f} us -> {value:.1f} GB/s; forward kernel {lin_mean_us:.2f} us "
        f"-> {achieved:.1f} GB/s; quant_act alone {qa_mean_us:.2f} us")

    # ---------------------------------------------------------------- format and output variants
    # the same decode step with 3D8 weights (a random int8 [256][3] signed
    # table over the same bytes) and with bf16 outputs; effective bytes of
    # 3D8 count its 768-byte table
    T3d = torch.from_numpy(workloads.signed_table([7, 1])).to(dev)
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    variants = {"decode": {"workload": f"{lin.name}: M={M} K={K} N={N}"}}
    for tag, tab, fmt, yy in (("s3d8_f32", dC, "s3d8", y), ("3d8_f32", T3d, "3d8", y),
                              ("s3d8_bf16", dC, "s3d8", yb), ("3d8_bf16", T3d, "3d8", yb)):
        out = "bf16" if yy is yb else "f32"
        fns = [lambda r=r, tab=tab, fmt=fmt, yy=yy, out=out: s3d8.forward(dX[r], dP[r], tab, dS, N, y=yy, xq=xq,
                                                                           xs=xsc, fmt=fmt, out=out)
               for r in range(R)]
        fns[0]()
        v_us = graph_launch_us(torch, fns, 10)
        vbytes = weight_bytes + (768 - 96 if fmt == "3d8" else 0)
        variants["decode"][tag] = {"us": round(v_us, 3), "GBs": round(vbytes / (v_us * 1e-6) / 1e9, 1)}
        log(f"variant {tag}: {v_us:.2f} us -> {variants['decode'][tag]['GBs']} GB/s effective weight bytes")
    # ---------------------------------------------------------------- c1 at M = 4 and 8
    # the other token counts of the c1 decode step: M = 4 through the same
    # one-launch streaming kernel, M = 8 as quantisation plus the streaming
    # GEMV on the INT8 codes (s3d8_forward picks both)
    decode_m = {}
    for mm in (4, 8):
        lm_ = workloads.C1[mm]
        xm_ = [torch.from_numpy(workloads.activations(lm_)).to(dev) for _ in range(R)]
        ym_ = torch.empty((mm, N), dtype=torch.float32, device=dev)
        xqm = torch.empty((mm, K), dtype=torch.int8, device=dev)
        xsm = torch.empty((mm,), dtype=torch.float32, device=dev)
        fns = [lambda r=r, xm_=xm_, ym_=ym_, xqm=xqm, xsm=xsm: s3d8.forward(xm_[r], dP[r], dC, dS, N, y=ym_, xq=xqm,
                                                                            xs=xsm) for r in range(R)]
        fns[0]()
        m_us = graph_launch_us(torch, fns, 10)
        decode_m[str(mm)] = {"us": round(m_us, 3), "GBs": round(weight_bytes / (m_us * 1e-6) / 1e9, 1),
                             "path": "one streaming launch" if mm <= 4 else "quant_act + streaming GEMV on the codes"}
        log(f"c1 decode M={mm}: {m_us:.2f} us -> {decode_m[str(mm)]['GBs']} GB/s effective weight bytes "
            f"({decode_m[str(mm)]['path']})")
        del xm_
    variants["decode_m"] = decode_m
    del dP, dX

    # ---------------------------------------------------------------- measured ceilings
    # HBM: a device-to-device copy of 1 GiB (read + write bytes per second),
    # and a copy of the c1 matrix's size cycling through R buffer pairs (the
    # same transfer size and cache behaviour as the decode step).  INT8
    # matrix cores: the rate probe (independent 32x32x32 INT8 MFMA chains on
    # four waves per SIMD).
    big = [torch.empty((2 ** 30,), dtype=torch.uint8, device=dev) for _ in range(2)]
    cp_us = graph_launch_us(torch, [lambda: big[1].copy_(big[0])], 10)
    del big
    same = [torch.empty((weight_bytes,), dtype=torch.uint8, device=dev) for _ in range(2 * R)]
    cs_us = graph_launch_us(torch, [lambda r=r: same[2 * r + 1].copy_(same[2 * r]) for r in range(R)], 10)
    del same
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    # read-only streams: the c1 matrix's size (rounded down to 16 bytes)
    # through R distinct buffers, and 1 GiB; the probe at 1 to 8 workgroups
    # per CU, the best kept
    rsize = weight_bytes // 16 * 16
    rbufs = [torch.empty((rsize,), dtype=torch.uint8, device=dev) for _ in range(R)]
    rout = torch.empty((8 * cus,), dtype=torch.int32, device=dev)
    rd_us = {}
    for wpc in (1, 2, 4, 8):
        rd_us[wpc] = graph_launch_us(torch, [lambda r=r, wpc=wpc: s3d8.hbm_read_probe(rbufs[r], wpc * cus, out=rout)
                                             for r in range(R)], 10)
    del rbufs
    rd_best = min(rd_us, key=rd_us.get)
    rbig = torch.empty((2 ** 30,), dtype=torch.uint8, device=dev)
    rbig_us = graph_launch_us(torch, [lambda: s3d8.hbm_read_probe(rbig, rd_best * cus, out=rout)], 5)
    del rbig
    pr_out, pr_ops = s3d8.mfma_rate_probe(2000, 4 * cus, 1, device=dev)
    pr_us = graph_launch_us(torch, [lambda: s3d8.mfma_rate_probe(2000, 4 * cus, 1, out=pr_out)], 5)
    ceilings = {"hbm_copy_1GiB_GBs": round(2 * 2 ** 30 / (cp_us * 1e-6) / 1e9, 1),
                "hbm_copy_c1_size_GBs": round(2 * weight_bytes / (cs_us * 1e-6) / 1e9, 1),
                "hbm_copy_c1_size_us": round(cs_us, 3),
                "hbm_read_c1_size_us": round(rd_us[rd_best], 3),
                "hbm_read_c1_size_GBs": round(rsize / (rd_us[rd_best] * 1e-6) / 1e9, 1),
                "hbm_read_c1_size_us_by_workgroups_per_cu": {str(k): round(v, 3) for k, v in rd_us.items()},
                "hbm_read_1GiB_GBs": round(2 ** 30 / (rbig_us * 1e-6) / 1e9, 1),
                "hbm_read_probe": f"s3d8_hbm_read_probe, {rsize} bytes through {R} buffers, 16-byte loads",
                "int8_mfma_probe_TOPS": round(pr_ops / (pr_us * 1e-6) / 1e12, 1),
                "int8_mfma_probe": f"{4 * cus} workgroups x 4 waves, 2000 rounds of 4 independent "
                                   f"v_mfma_i32_32x32x32_i8 each"}
    log(f"ceilings: copy 1 GiB {ceilings['hbm_copy_1GiB_GBs']} GB/s, copy {weight_bytes} B "
        f"{cs_us:.2f} us ({ceilings['hbm_copy_c1_size_GBs']} GB/s), read {rsize} B {rd_us[rd_best]:.2f} us "
        f"({ceilings['hbm_read_c1_size_GBs']} GB/s), read 1 GiB {ceilings['hbm_read_1GiB_GBs']} GB/s, "
        f"INT8 MFMA probe {ceilings['int8_mfma_probe_TOPS']} TOPS")

    # ---------------------------------------------------------------- one decoder-layer step (c2)
    # the seven linears of a decoder layer at one token, each with its own
    # packed weights and activations: seven s3d8_forward launches against
    # one s3d8_forward_batch launch; effective bytes = the seven matrices'
    # S3D8 bytes.  Weight copies cycle as above (R2 copies of the layer).
    layer = None
    if not args.no_layer:
        t0 = time.time()
        mats = []
        for ln in workloads.C2:
            Cl, Sl, Pl = s3d8.pack(workloads.weights(ln), seed=ln.pack_seed, max_iters=args.pack_iters)
            mats.append((ln, Cl, Sl, Pl))
        log(f"decoder layer packed in {time.time() - t0:.1f}s")
        layer_bytes = sum(s3d8.format_bytes(ln.N, ln.K) for ln, _, _, _ in mats)
        R2 = max(2, int(np.ceil(2 * MALL_BYTES / layer_bytes)))
        lay = []
        for r in range(R2):
            items = []
            for ln, Cl, Sl, Pl in mats:
                items.append(dict(x=torch.from_numpy(workloads.activations(ln)).to(dev),
                                  tiled=s3d8.tile(torch.from_numpy(Pl).to(dev), ln.N),
                                  centroids=torch.from_numpy(Cl).to(dev),
                                  scales=torch.from_numpy(Sl.view(np.int16)).to(dev), N=ln.N,
                                  y=torch.empty((ln.M, ln.N), dtype=torch.float32, device=dev),
                                  xq=torch.empty((ln.M, ln.K), dtype=torch.int8, device=dev),
                                  xs=torch.empty((ln.M,), dtype=torch.float32, device=dev)))
            lay.append(items)

        def separate(r):
            for it in lay[r]:
                s3d8.forward(it["x"], it["tiled"], it["centroids"], it["scales"], it["N"], y=it["y"], xq=it["xq"],
                             xs=it["xs"])

        sep_us = graph_launch_us(torch, [lambda r=r: separate(r) for r in range(R2)], 5)
        bat_us = graph_launch_us(torch, [lambda r=r: s3d8.forward_batch(lay[r]) for r in range(R2)], 5)
        gbs = layer_bytes / (bat_us * 1e-6) / 1e9
        layer = {"workload": "c2: q, o 4096x4096; k, v 4096->1024; gate, up 4096->14336; down 14336->4096; M=1",
                 "effective_weight_bytes": layer_bytes, "separate_launches_us": round(sep_us, 2),
                 "one_launch_us": round(bat_us, 2), "one_launch_GBs": round(gbs, 1),
                 "one_launch_frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "weight_copies": R2}
        log(f"decoder layer: 7 launches {sep_us:.2f} us, one batched launch {bat_us:.2f} us "
            f"-> {gbs:.1f} GB/s effective weight bytes")
        del lay

    # ---------------------------------------------------------------- lm_head decode step (c4, M=1)
    # the same streaming GEMV over the 175 MB lm_head matrix (K=4096,
    # N=128256), where the fixed costs of a launch (start-up, prologue, the
    # last tiles) weigh far less than on the 19.6 MB c1 matrix.  Uniform
    # random bytes, table and bf16 scales: a kernel's time does not depend
    # on the byte values, and packing 525 M weights would take the bench
    # minutes.  Four weight copies (700 MB) cycle as above.
    lm_head = None
    if not args.no_layer:
        lh = workloads.C4[0]
        Tl = s3d8.num_triples(lh.N)
        lbytes = s3d8.format_bytes(lh.N, lh.K)
        Pl = torch.from_numpy(workloads.random_packed(lh.config_id, Tl, lh.K, lh.matrix_id)).to(dev)
        dPl = [s3d8.tile(Pl, lh.N) for _ in range(4)]
        del Pl
        dCl = torch.from_numpy(workloads.random_centroids(lh.config_id, lh.matrix_id)).to(dev)
        dSl = torch.from_numpy(workloads.random_scales_bf16(lh.config_id, 3 * Tl, lh.matrix_id).view(np.int16)).to(dev)
        xl = torch.from_numpy(workloads.activations(lh)).to(dev)
        yl = torch.empty((1, lh.N), dtype=torch.float32, device=dev)
        xql = torch.empty((1, lh.K), dtype=torch.int8, device=dev)
        xsl = torch.empty((1,), dtype=torch.float32, device=dev)
        fns = [lambda r=r: s3d8.forward(xl, dPl[r], dCl, dSl, lh.N, y=yl, xq=xql, xs=xsl) for r in range(4)]
        fns[0]()
        l_us = graph_launch_us(torch, fns, 10)
        l_gbs = lbytes / (l_us * 1e-6) / 1e9
        lm_head = {"workload": f"{lh.name}: M=1 K={lh.K} N={lh.N}, uniform random S3D8 bytes",
                   "effective_weight_bytes": lbytes, "us": round(l_us, 2), "GBs": round(l_gbs, 1),
                   "frac_hbm": round(l_gbs / HBM_PEAK_GBS, 4),
                   "frac_of_copy_1GiB": round(l_gbs / ceilings["hbm_copy_1GiB_GBs"], 4)}
        log(f"lm_head decode: {l_us:.2f} us -> {l_gbs:.1f} GB/s effective weight bytes "
            f"({lm_head['frac_hbm'] * 100:.1f}% of HBM peak)")
        del dPl

    # ---------------------------------------------------------------- standalone dequant + copy baselines
    # the pages' own kernel measurement: S3D8 -> channel-INT8 dequantisation
    # against a plain copy of the same matrix in INT8, on the c1 gate/up
    # matrix and on the vision MLP up shape the pages time it on (K=1280,
    # N=5120); read bandwidth counted on the S3D8 source bytes as there
    dequant = {}
    for tag, (Nd, Kd, Pd) in {"c1_gate_up": (N, K, packed),
                              "vision_mlp_up": (5120, 1280, workloads.uniform_bytes([9, 1], s3d8.num_triples(5120),
                                                                                     1280))}.items():
        src = [torch.from_numpy(Pd).to(dev) for _ in range(4)]
        wout = torch.empty((Nd, Kd), dtype=torch.int8, device=dev)
        s3d8.dequant(src[0], dC, Nd, w=wout)
        d_us = graph_launch_us(torch, [lambda r=r: s3d8.dequant(src[r], dC, Nd, w=wout) for r in range(4)], 10)
        i8 = [torch.empty((Nd, Kd), dtype=torch.int8, device=dev) for _ in range(4)]
        i8dst = torch.empty((Nd, Kd), dtype=torch.int8, device=dev)
        c_us = graph_launch_us(torch, [lambda r=r: i8dst.copy_(i8[r]) for r in range(4)], 10)
        sbytes = s3d8.format_bytes(Nd, Kd)
        dequant[tag] = {"N": Nd, "K": Kd, "dequant_us": round(d_us, 3),
                        "dequant_read_GBs": round(sbytes / (d_us * 1e-6) / 1e9, 1),
                        "dequant_total_GBs": round((s3d8.packed_bytes(Nd, Kd) + Nd * Kd) / (d_us * 1e-6) / 1e9, 1),
                        "int8_copy_us": round(c_us, 3),
                        "int8_copy_GBs": round(2 * Nd * Kd / (c_us * 1e-6) / 1e9, 1)}
        log(f"dequant {tag}: {d_us:.2f} us ({dequant[tag]['dequant_read_GBs']} GB/s on S3D8 bytes); "
            f"INT8 copy of the same matrix {c_us:.2f} us")
        del src, wout, i8, i8dst

    # ---------------------------------------------------------------- frozen-centroid encode on the device
    # (the quantiser in front of the path): c1 gate/up fp32 weights with the
    # table the packer fitted, against the host encoder on the same input
    Wd = torch.from_numpy(workloads.weights(lin)).to(dev)
    s3d8.encode_device(Wd, dC)
    e_us = graph_launch_us(torch, [lambda: s3d8.encode_device(Wd, dC)], 3)
    t0 = time.perf_counter()
    s3d8.encode(workloads.weights(lin), C)
    host_s = time.perf_counter() - t0
    encode = {"workload": f"{lin.name} weights fp32 [{N}][{K}]", "device_us": round(e_us, 1),
              "fp32_read_GBs": round(4 * N * K / (e_us * 1e-6) / 1e9, 1), "host_s": round(host_s, 3)}
    log(f"device encode {lin.name}: {e_us:.1f} us ({encode['fp32_read_GBs']} GB/s of fp32 weights); "
        f"host encode {host_s:.3f} s")
    del Wd

    # ---------------------------------------------------------------- prefill GEMM
    prefill = None
    if not args.no_prefill:
        lp = workloads.C3
        t0 = time.time()
        Wp = workloads.weights(lp)
        Cp, Sp, Pp = s3d8.pack(Wp, seed=lp.pack_seed, max_iters=args.pack_iters)
        del Wp
        log(f"prefill weights packed in {time.time() - t0:.1f}s")
        xp = torch.from_numpy(workloads.activations(lp)).to(dev)
        xqp, xsp = s3d8.quant_act(xp)
        Rp = 4
        tp0 = s3d8.tile(torch.from_numpy(Pp).to(dev), lp.N)
        dPp = [tp0.clone() for _ in range(Rp)]
        del tp0
        dCp = torch.from_numpy(Cp).to(dev)
        dSp = torch.from_numpy(Sp.view(np.int16)).to(dev)
        yp = torch.empty((lp.M, lp.N), dtype=torch.float32, device=dev)
        for i in range(2):
            s3d8.linear(xqp, xsp, dPp[i % Rp], dCp, dSp, lp.N, y=yp)
        torch.cuda.synchronize()
        g_mean_us = graph_launch_us(
            torch, [lambda r=r: s3d8.linear(xqp, xsp, dPp[r], dCp, dSp, lp.N, y=yp) for r in range(Rp)], 20)
        ops = 2.0 * lp.M * lp.K * lp.N
        tops = ops / (g_mean_us * 1e-6) / 1e12
        log(f"prefill GEMM {lp.name}: fused {g_mean_us:.1f} us -> {tops:.1f} TOPS")
        # context: the vendor library's plain INT8 GEMM (torch._int_mm, which
        # runs hipBLASLt on ROCm) on the same shape with INT8 weights: no
        # decode, INT32 output, i.e. what an INT8-weight model would run
        lib_gemm = None
        try:
            wi8 = [torch.randint(-127, 128, (lp.N, lp.K), dtype=torch.int8, device=dev) for _ in range(Rp)]
            torch._int_mm(xqp, wi8[0].t())
            torch.cuda.synchronize()
            l_us = graph_launch_us(torch, [lambda r=r: torch._int_mm(xqp, wi8[r].t()) for r in range(Rp)], 20)
            lib_gemm = {"call": "torch._int_mm(xq [M][K] int8, w[N][K].t() int8) -> int32 [M][N]",
                        "us": round(l_us, 2), "TOPS": round(ops / (l_us * 1e-6) / 1e12, 1),
                        "frac": round(ops / (l_us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
            log(f"library INT8 GEMM (torch._int_mm) {l_us:.1f} us -> {lib_gemm['TOPS']} TOPS")
            del wi8
        except Exception as e:  # not every torch build routes _int_mm to a GPU library
            lib_gemm = {"error": f"{type(e).__name__}: {e}"[:200]}
            log(f"library INT8 GEMM unavailable: {lib_gemm['error']}")
        # the pages' strategy for many rows: decode once to INT8, then an
        # INT8 GEMM (two launches per call)
        ws = torch.empty((s3d8.unfused_workspace_bytes(lp.N, lp.K),), dtype=torch.int8, device=dev)
        s3d8.linear_unfused(xqp, xsp, dPp[0], dCp, dSp, lp.N, workspace=ws, y=yp)
        torch.cuda.synchronize()
        u_mean_us = graph_launch_us(
            torch, [lambda r=r: s3d8.linear_unfused(xqp, xsp, dPp[r], dCp, dSp, lp.N, workspace=ws, y=yp)
                    for r in range(Rp)], 20)
        u_tops = ops / (u_mean_us * 1e-6) / 1e12
        log(f"prefill GEMM {lp.name}: unfused (dequant + INT8 GEMM) {u_mean_us:.1f} us -> {u_tops:.1f} TOPS")
        # format and output variants of the fused GEMM
        T3p = torch.from_numpy(workloads.signed_table([7, 3])).to(dev)
        ypb = torch.empty((lp.M, lp.N), dtype=torch.bfloat16, device=dev)
        variants["prefill"] = {"workload": f"{lp.name}: M={lp.M} K={lp.K} N={lp.N}"}
        for tag, tab, fmt, yy in (("3d8_f32", T3p, "3d8", yp), ("s3d8_bf16", dCp, "s3d8", ypb),
                                  ("3d8_bf16", T3p, "3d8", ypb)):
            out = "bf16" if yy is ypb else "f32"
            fns = [lambda r=r, tab=tab, fmt=fmt, yy=yy, out=out: s3d8.linear(xqp, xsp, dPp[r], tab, dSp, lp.N, y=yy,
                                                                              fmt=fmt, out=out)
                   for r in range(Rp)]
            fns[0]()
            v_us = graph_launch_us(torch, fns, 20)
            variants["prefill"][tag] = {"us": round(v_us, 2), "TOPS": round(ops / (v_us * 1e-6) / 1e12, 1)}
            log(f"variant prefill {tag}: {v_us:.1f} us -> {variants['prefill'][tag]['TOPS']} TOPS")
        prefill = {
            "workload": f"{lp.name}: M={lp.M} K={lp.K} N={lp.N}",
            "value": round(tops, 2), "unit": "INT8 TOPS", "us_per_launch": round(g_mean_us, 2),
            "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4),
                         "frac_of_probe": round(tops / ceilings["int8_mfma_probe_TOPS"], 4),
                         "traffic": measured_traffic("gemm_c3", None),
                         "kernel": "gemm_w8_kernel (fused decode + INT8 MFMA, eight waves, via s3d8_linear)"},
            "library_int8_gemm": lib_gemm,
            "unfused": {"value": round(u_tops, 2), "unit": "INT8 TOPS", "us_per_call": round(u_mean_us, 2),
                        "frac": round(u_tops / INT8_PEAK_TOPS, 4),
                        "kernels": "dequant_tiled_kernel + gemm_i8_kernel (s3d8_linear_unfused)"},
        }
        del dPp, ws

        # the c4 prefill shapes through the same fused GEMM: lm_head at 512
        # tokens, the vision-encoder MLP at 1601.  Uniform random bytes,
        # table and scales as for the lm_head decode step; four weight
        # copies cycle.
        for lc in workloads.C4[1:]:
            Tc = s3d8.num_triples(lc.N)
            Pc = torch.from_numpy(workloads.random_packed(lc.config_id, Tc, lc.K, lc.matrix_id)).to(dev)
            dPc = [s3d8.tile(Pc, lc.N) for _ in range(4)]
            del Pc
            dCc = torch.from_numpy(workloads.random_centroids(lc.config_id, lc.matrix_id)).to(dev)
            dSc = torch.from_numpy(
                workloads.random_scales_bf16(lc.config_id, 3 * Tc, lc.matrix_id).view(np.int16)).to(dev)
            xqc, xsc = s3d8.quant_act(torch.from_numpy(workloads.activations(lc)).to(dev))
            yc = torch.empty((lc.M, lc.N), dtype=torch.float32, device=dev)
            fns = [lambda r=r: s3d8.linear(xqc, xsc, dPc[r], dCc, dSc, lc.N, y=yc) for r in range(4)]
            fns[0]()
            c_us = graph_launch_us(torch, fns, 20)
            c_tops = 2.0 * lc.M * lc.K * lc.N / (c_us * 1e-6) / 1e12
            entry = {"workload": f"{lc.name}: M={lc.M} K={lc.K} N={lc.N}, uniform random S3D8 bytes",
                     "us_per_launch": round(c_us, 2), "TOPS": round(c_tops, 1),
                     "frac": round(c_tops / INT8_PEAK_TOPS, 4)}
            log(f"prefill GEMM {lc.name}: fused {c_us:.1f} us -> {c_tops:.1f} TOPS "
                f"({100 * c_tops / INT8_PEAK_TOPS:.1f}% of INT8 peak)")
            # split-K (s3d8_linear_splitk) where the library splits this shape
            sk = s3d8.splitk_auto(lc.M, lc.K, lc.N, torch.cuda.get_device_properties(dev).multi_processor_count)
            if sk > 1:
                wsk = torch.zeros((s3d8.splitk_workspace_bytes(lc.M, lc.K, lc.N, sk),), dtype=torch.uint8,
                                  device=dev)
                fk = [lambda r=r: s3d8.linear_splitk(xqc, xsc, dPc[r], dCc, dSc, lc.N, splits=sk, workspace=wsk,
                                                     y=yc) for r in range(4)]
                fk[0]()
                k_us = graph_launch_us(torch, fk, 20)
                k_tops = 2.0 * lc.M * lc.K * lc.N / (k_us * 1e-6) / 1e12
                entry["splitk"] = {"splits": sk, "us_per_launch": round(k_us, 2), "TOPS": round(k_tops, 1),
                                   "frac": round(k_tops / INT8_PEAK_TOPS, 4),
                                   "entry_point": "s3d8_linear_splitk (column-block ranges, exact INT32 "
                                                  "partial sums added before the epilogue)"}
                log(f"prefill GEMM {lc.name}: split-K x{sk} {k_us:.1f} us -> {k_tops:.1f} TOPS "
                    f"({100 * k_tops / INT8_PEAK_TOPS:.1f}% of INT8 peak)")
                del wsk
            prefill.setdefault("c4", []).append(entry)
            del dPc, yc

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        import json as _json

        with open(os.path.join(ROOT, "tests", "golden", "centroids.json")) as f:
            Cg = np.array(_json.load(f)[f"cfg{lin.config_id}.mat{lin.matrix_id}"]["C"], np.uint8)
        W = workloads.weights(lin)
        alpha_o, packed_o = oracle.encode(W, Cg)
        del W
        x = workloads.activations(lin)
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        n = 0
        t0 = time.perf_counter()
        while True:
            oracle.linear(x, packed_o, Cg, alpha_o, N)
            n += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        cpu = {"value": round(weight_bytes * n / el / 1e9, 4), "unit": "GB/s", "cores": threads,
               "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "kind": "oracle",
               "sample": f"full {lin.name} step (quantise, decode every weight, naive int dot "
                         f"products, fp32 epilogue) repeated {n} times in {el:.1f} s"}
        log(f"cpu oracle: {cpu['value']} GB/s on {threads} threads")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{lin.name}: decode GEMV M={M} K={K} N={N} (Llama-3.2-11B text MLP "
                               f"gate/up), S3D8 weights packed from N(0,0.02), step = s3d8_forward "
                               f"(quantise + decode GEMV, one launch)",
                   "weight_copies": R, "graph_steps": R},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "gemv_stream_kernel (fused quantise + decode GEMV, via s3d8_forward)",
                     "kernel_us": round(lin_mean_us, 3), "algorithmic_bytes": kernel_bytes,
                     "frac_of_copy_1GiB": round(achieved / ceilings["hbm_copy_1GiB_GBs"], 4),
                     "frac_of_same_size_read": round(ceilings["hbm_read_c1_size_us"] / lin_mean_us, 4)},
        "timing": timing,
        "context_pages_arm": {"note": "the pages' own figures (Arm CPUs), quoted with their hardware; "
                                      "context, not a target",
                              "figures": PAGES_CONTEXT,
                              "this_run_GMACs": {"[1, 4096, 14336] fused S3D8, s3d8_forward":
                                                 round(K * N / (ms_per_step * 1e-3) / 1e9, 1),
                                                 "[2048, 4096, 14336] fused S3D8, s3d8_linear":
                                                 None if prefill is None else
                                                 round(prefill["value"] * 1e3 / 2, 1)}},
        "ceilings": ceilings,
        "quant_act_us": round(qa_mean_us, 3),
        "prefill": prefill,
        "decoder_layer": layer,
        "lm_head": lm_head,
        "encode": encode,
        "dequant": dequant,
        "variants": variants,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out, allow_nan=False), flush=True)


if __name__ == "__main__":
    main()
