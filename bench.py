#!/usr/bin/env python3
"""Benchmark of the scaled 8-bit GEMM hot path on one MI355X.

Headline (``value``): the prefill step — per-token-group FP8 quantization of a
bf16 activation [4096, 7168] (groups of 128) followed by the [128,128]-block-
scaled FP8 GEMM against W [7168, 7168] with bf16 output — as whole-step
TFLOP/s (2*M*N*K per step over the measured step time). The dominant kernel
(the GEMM) is timed on its own with HIP events around each of its launches in
the timed steps, and reported against the dense FP8 MFMA peak (roofline).

Secondary paths, each timed the same way and reported under ``paths``:
decode block32 GEMM (M in {1, 4, 16, 64}, N=4096, K=7168, UE8M0 group-32
activation quant) as GB/s against HBM, with weights rotated over enough copies
that the 256 MB Infinity Cache cannot hold them; the quant kernel alone;
INT8 W8A8 (2048 x 8192 x 8192, per-token x per-channel); the MoE step
(routing + quant + expert-grouped GEMM with fused gather/un-permute).

The CPU oracle is timed on a bounded sample of the prefill workload (a
subset of rows) as ``cpu_baseline``.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_INT8_TOPS = 5000.0    # MI355X dense INT8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
EPS = 1e-10
MALL_BYTES = 256 << 20


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class KernelTimer:
    """HIP events around launches on the current stream; mean/median in us."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.s = self.torch.cuda.Event(enable_timing=True)
        self.e = self.torch.cuda.Event(enable_timing=True)
        self.s.record()
        return self

    def __exit__(self, *exc):
        self.e.record()
        self.pairs.append((self.s, self.e))
        return False

    def us(self):
        v = [s.elapsed_time(e) * 1e3 for s, e in self.pairs]
        return {"mean": statistics.fmean(v), "median": statistics.median(v),
                "p10": sorted(v)[len(v) // 10], "p90": sorted(v)[(len(v) * 9) // 10], "n": len(v)}


def tile_kernel_sha():
    """Hash of the sources the prefill tile kernel is built from: its
    parameter block, device helpers and kernel, its host launch code, and the
    shared headers. Other kernels in the same file do not change it."""
    csrc = os.path.join(ROOT, "int8_quantized_gemm_amd", "csrc")
    try:
        with open(os.path.join(csrc, "gemm_block.hip")) as f:
            src = f.read()
        parts = [src[src.index("struct TileParams {"):src.index("// Skinny (decode) kernel")],
                 src[src.index("constexpr int kBM = 256"):src.index("__global__ void invert_permutation")]]
        for n in ("tile_common.h", "q8_device.h"):
            with open(os.path.join(csrc, n)) as f:
                parts.append(f.read())
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for part in parts:
        h.update(part.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, only
    while the kernel source still matches the one that was profiled."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
def bench_prefill(torch, q8, synth, steps, warmup, ramp_ms):
    M, N, K, blk = 4096, 7168, 7168, 128
    dev = "cuda:0"
    x = synth.activations(M, K, "bf16", seed=0).to(dev)
    Wq, Ws = synth.fp8_block_weights(N, K, blk, blk, seed=0)
    Wq, Ws = Wq.to(dev), Ws.to(dev)
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    As = torch.empty((M, K // blk), dtype=torch.float32, device=dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(gt=None, qt=None):
        if qt:
            with qt:
                q8.quant_8bit(x, aq, As, blk, EPS, -448.0, 448.0, False)
        else:
            q8.quant_8bit(x, aq, As, blk, EPS, -448.0, 448.0, False)
        if gt:
            with gt:
                q8.blockwise_scaled_mm(aq, Wq, As, Ws, torch.bfloat16, block=(blk, blk), out=D)
        else:
            q8.blockwise_scaled_mm(aq, Wq, As, Ws, torch.bfloat16, block=(blk, blk), out=D)

    # Clock ramp: from idle the GPU needs ≈ 50 ms of back-to-back work before
    # its clock settles (measured per GEMM launch from a cold start: ≈ 450 us
    # in the first ten launches, 230 us after 15 ms, 204-206 us from ≈ 50 ms
    # on). The step runs untimed for ramp_ms of wall time first, so that a
    # short warm-up does not time the ramp; then the warm-up steps as asked.
    ramp_steps = 0
    t_r = time.perf_counter()
    while (time.perf_counter() - t_r) * 1e3 < ramp_ms:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
        ramp_steps += 8
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # step time: plain launches, bracketed by synchronize
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    # kernel durations: events around each launch, on the launch stream
    gt, qt = KernelTimer(torch), KernelTimer(torch)
    for _ in range(steps):
        step(gt, qt)
    torch.cuda.synchronize()
    flops = 2.0 * M * N * K
    g_us = gt.us()
    return {
        "ms_per_step": ms_per_step,
        "tflops_step": flops / (ms_per_step * 1e-3) / 1e12,
        "gemm_us": g_us, "quant_us": qt.us(),
        "gemm_tflops": flops / (g_us["mean"] * 1e-6) / 1e12,
        "shape": (M, N, K, blk),
        "x": x, "Wq": Wq, "Ws": Ws,
        "clock_ramp": {"ms": ramp_ms, "steps": ramp_steps},
    }


def bench_prefill_variants(torch, q8, synth, pre, reps):
    """The other two prefill GEMM workloads: the same activation against a
    [18432, 7168] weight, and the headline shape with a bf16 bias added in the
    epilogue. GEMM only (the activation is quantized once, beforehand)."""
    M, _, K, blk = pre["shape"]
    dev = "cuda:0"
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    As = torch.empty((M, K // blk), dtype=torch.float32, device=dev)
    q8.quant_8bit(pre["x"], aq, As, blk, EPS, -448.0, 448.0, False)
    out = {}
    for name, N, with_bias in (("4096x18432x7168", 18432, False), ("4096x7168x7168_bias", 7168, True)):
        if N == pre["shape"][1]:
            Wq, Ws = pre["Wq"], pre["Ws"]
        else:
            Wq, Ws = synth.fp8_block_weights(N, K, blk, blk, seed=0)
            Wq, Ws = Wq.to(dev), Ws.to(dev)
        b = synth.bias(N, seed=0).to(dev) if with_bias else None
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gt = KernelTimer(torch)
        for i in range(reps + 5):
            if i >= 5:
                with gt:
                    q8.blockwise_scaled_mm(aq, Wq, As, Ws, torch.bfloat16, bias=b, block=(blk, blk), out=D)
            else:
                q8.blockwise_scaled_mm(aq, Wq, As, Ws, torch.bfloat16, bias=b, block=(blk, blk), out=D)
        torch.cuda.synchronize()
        g = gt.us()
        tf = 2.0 * M * N * K / (g["median"] * 1e-6) / 1e12
        out[name] = {"gemm_us": round(g["median"], 2), "gemm_us_p10": round(g["p10"], 2),
                     "gemm_us_p90": round(g["p90"], 2), "TFLOP/s": round(tf, 1),
                     "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        del D, b
    return out


def batched_us(torch, launch, copies, reps, warmup=3, warmup_s=0.05):
    """Per-launch time of ``copies`` back-to-back launches (each on its own
    buffers) between one pair of HIP events on the launch stream, median over
    ``reps`` batches. Batching amortises the event overhead that would
    otherwise dominate kernels of a few microseconds. Untimed warm-up: at
    least ``warmup`` batches and ``warmup_s`` seconds of them, so that the
    clock has ramped up after the host-side set-up between measurements."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < warmup_s:
        for c in range(copies):
            launch(c)
        i += 1
    torch.cuda.synchronize()
    vals = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for c in range(copies):
            launch(c)
        e.record()
        vals.append((s, e))
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) * 1e3 / copies for s, e in vals)
    return {"median": per[len(per) // 2], "p10": per[len(per) // 10], "p90": per[(len(per) * 9) // 10]}


def graph_us(torch, launch, copies, reps):
    """Per-launch GPU time of ``copies`` launches captured once in a HIP graph
    and replayed between a pair of HIP events (median over ``reps`` replays).
    For kernels shorter than the Python launch path (≈ 9 us per call), where
    back-to-back launches from Python leave the GPU idle between kernels."""
    for c in range(copies):
        launch(c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(copies):
            launch(c)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    vals = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        vals.append((s, e))
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) * 1e3 / copies for s, e in vals)
    return {"median": per[len(per) // 2], "p10": per[len(per) // 10], "p90": per[(len(per) * 9) // 10]}


def bench_decode(torch, q8, synth, reps):
    N, K, blk = 4096, 7168, 32
    dev = "cuda:0"
    wbytes = N * K
    copies = max(2, -(-(MALL_BYTES + (64 << 20)) // wbytes))
    Wq0, Ws0 = synth.fp8_block_weights(N, K, blk, blk, seed=0)
    Ws = Ws0.to(dev)
    Ws_list = [Ws.clone() for _ in range(copies)]
    W_list = [Wq0.to(dev) for _ in range(copies)]
    out = {}
    for M in (1, 4, 16, 64):
        x = synth.activations(M, K, "bf16", outlier_frac=0.01, seed=0).to(dev)
        aq = [torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(copies)]
        As = [torch.empty((M, K // blk), dtype=torch.float32, device=dev) for _ in range(copies)]
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def quant(c):
            q8.quant_8bit(x, aq[c], As[c], blk, EPS, -448.0, 448.0, True)

        for c in range(copies):
            quant(c)
        # the launches are bound once (checked and marshalled up front): a
        # decode GEMM takes about as long as one checked Python call
        ws = torch.empty(max(1, q8.blockwise_scaled_mm_workspace_size(M, N, K, blk, blk)),
                         dtype=torch.uint8, device=dev)
        calls = [q8.bind_blockwise_scaled_mm(aq[c], W_list[c], As[c], Ws_list[c], D, block=(blk, blk),
                                             workspace=ws) for c in range(copies)]

        def gemm(c):
            calls[c]()

        g = batched_us(torch, gemm, copies, reps)
        qv = graph_us(torch, quant, copies, reps)
        nbytes = wbytes + Ws.numel() * 4 + M * K + M * (K // blk) * 4 + M * N * 2
        gbs = nbytes / (g["median"] * 1e-6) / 1e9
        out[f"M{M}"] = {"gemm_us": round(g["median"], 3), "gemm_us_p10": round(g["p10"], 3),
                        "gemm_us_p90": round(g["p90"], 3), "quant_us": round(qv["median"], 3),
                        "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1),
                        "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                        "tflops": round(2.0 * M * N * K / (g["median"] * 1e-6) / 1e12, 2)}
    out["weight_copies_rotated"] = copies
    out["timing"] = ("GEMM: HIP events around batches of back-to-back launches, one weight copy each, "
                     "each launch a pre-marshalled C-ABI call; quant (a few-microsecond kernel): the "
                     "same launches replayed from a HIP graph")
    return out


def bench_quant(torch, q8, synth, reps):
    M, K = 4096, 7168
    dev = "cuda:0"
    copies = max(2, -(-(MALL_BYTES + (64 << 20)) // (M * K * 2)))
    base = synth.activations(M, K, "bf16", seed=0).to(dev)
    xs = [base.clone() for _ in range(copies)]
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    res = {}
    for g, ue in ((128, False), (32, True)):
        As = torch.empty((M, K // g), dtype=torch.float32, device=dev)
        u = batched_us(torch, lambda c: q8.quant_8bit(xs[c], aq, As, g, EPS, -448.0, 448.0, ue),
                       copies, reps)
        nbytes = M * K * 2 + M * K + M * (K // g) * 4
        gbs = nbytes / (u["median"] * 1e-6) / 1e9
        res[f"g{g}{'_ue8m0' if ue else ''}"] = {"us": round(u["median"], 3), "algorithmic_bytes": nbytes,
                                                "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    res["input_copies_rotated"] = copies
    return res


def bench_silu_quant(torch, q8, synth, reps):
    """Fused SiLU-and-mul + group-128 FP8 quant. Dense: [4096, 2 x 7168] bf16
    -> [4096, 7168] codes (inputs rotated past the Infinity Cache). Masked:
    the expert-major layout [64, max_m, 2 x 1024] of the 4096-token top-8
    routing (per-expert counts from the same Zipf ids as the MoE step,
    max_m = the largest count), only the routed rows valid."""
    dev = "cuda:0"
    res = {}
    M, K, g = 4096, 7168, 128
    nbytes = M * 2 * K * 2 + M * K + M * (K // g) * 4
    copies = max(2, -(-(MALL_BYTES + (64 << 20)) // (M * 2 * K * 2)))
    base = synth.activations(M, 2 * K, "bf16", seed=0).to(dev)
    xs = [base.clone() for _ in range(copies)]
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    As = torch.empty((M, K // g), dtype=torch.float32, device=dev)
    u = batched_us(torch, lambda c: q8.quant_8bit(xs[c], aq, As, g, EPS, -448.0, 448.0, False,
                                                  fuse_silu_and_mul=True), copies, reps)
    gbs = nbytes / (u["median"] * 1e-6) / 1e9
    res["dense_4096x7168_g128"] = {"us": round(u["median"], 3), "algorithmic_bytes": nbytes,
                                   "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    del xs, base
    T, E, topk, I = 4096, 64, 8, 1024
    ids = synth.zipf_topk_ids(T, E, topk, seed=0)
    counts = torch.bincount(ids.flatten().long(), minlength=E).to(torch.int32)
    max_m = int(counts.max())
    x3 = synth.activations(E * max_m, 2 * I, "bf16", seed=1).reshape(E, max_m, 2 * I).to(dev)
    mm = counts.to(dev)
    q3 = torch.empty((E, max_m, I), dtype=torch.float8_e4m3fn, device=dev)
    s3 = torch.empty((E, max_m, I // g), dtype=torch.float32, device=dev)
    u = batched_us(torch, lambda c: q8.quant_8bit(x3, q3, s3, g, EPS, -448.0, 448.0, False,
                                                  fuse_silu_and_mul=True, masked_m=mm), 4, reps)
    rows = int(counts.sum())
    mbytes = rows * (2 * I * 2 + I + (I // g) * 4)
    gbs = mbytes / (u["median"] * 1e-6) / 1e9
    res["masked_e64_top8_I1024_g128"] = {"us": round(u["median"], 3), "valid_rows": rows,
                                         "max_m": max_m, "algorithmic_bytes": mbytes,
                                         "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    res["input_copies_rotated"] = copies
    return res


def bench_e8m0(torch, q8, synth, reps):
    """Block32 FP8 GEMMs with power-of-two (E8M0) scales on both operands (the
    MX-scaled MFMA path): prefill 4096 x 7168 x 7168 and decode M in
    {1, 4, 16, 64} x 4096 x 7168 (weights rotated past the Infinity Cache),
    next to the float32-scale block32 kernel on the same prefill shape."""
    dev = "cuda:0"
    res = {}
    M, N, K = 4096, 7168, 7168
    x = synth.activations(M, K, "bf16", seed=0).to(dev)
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    asb = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    q8.quant_8bit(x, aq, asb, 32, EPS, -448.0, 448.0, 2)
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, 32, 32, seed=0)
    Wq, Wsb = Wq.to(dev), Wsb.to(dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = KernelTimer(torch)
    for i in range(reps + 3):
        with (t if i >= 3 else _Null()):
            q8.blockwise_scaled_mm_e8m0(aq, Wq, asb, Wsb, block_n=32, out=D)
    torch.cuda.synchronize()
    us = t.us()["median"]
    tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
    res["prefill_4096x7168x7168_block32"] = {"gemm_us": round(us, 2), "TFLOP/s": round(tf, 1),
                                             "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
    # the float32-scale kernel on the same shape and block size
    As32 = torch.empty((M, K // 32), dtype=torch.float32, device=dev)
    q8.quant_8bit(x, aq, As32, 32, EPS, -448.0, 448.0, True)
    W32, Ws32 = synth.fp8_block_weights(N, K, 32, 32, seed=0)
    W32, Ws32 = W32.to(dev), Ws32.to(dev)
    t = KernelTimer(torch)
    for i in range(max(reps // 2, 5) + 3):
        with (t if i >= 3 else _Null()):
            q8.blockwise_scaled_mm(aq, W32, As32, Ws32, torch.bfloat16, block=(32, 32), out=D)
    torch.cuda.synchronize()
    us32 = t.us()["median"]
    res["prefill_4096x7168x7168_block32_float32_scales"] = {
        "gemm_us": round(us32, 2), "TFLOP/s": round(2.0 * M * N * K / (us32 * 1e-6) / 1e12, 1)}
    del x, aq, asb, D, W32, Ws32, As32, Wq, Wsb
    N, K = 4096, 7168
    copies = max(2, -(-(MALL_BYTES + (64 << 20)) // (N * K)))
    W0, Ws0 = synth.fp8_block_weights_e8m0(N, K, 32, 32, seed=0)
    Wl = [W0.to(dev) for _ in range(copies)]
    Wsl = [Ws0.to(dev) for _ in range(copies)]
    dec = {}
    for Md in (1, 4, 16, 64):
        xd = synth.activations(Md, K, "bf16", outlier_frac=0.01, seed=0).to(dev)
        aqd = torch.empty((Md, K), dtype=torch.float8_e4m3fn, device=dev)
        asd = torch.empty((Md, K // 32), dtype=torch.uint8, device=dev)
        q8.quant_8bit(xd, aqd, asd, 32, EPS, -448.0, 448.0, 2)
        Dd = torch.empty((Md, N), dtype=torch.bfloat16, device=dev)
        wsd = torch.empty(max(1, q8.blockwise_scaled_mm_e8m0_workspace_size(Md, N, K, 32)),
                          dtype=torch.uint8, device=dev)
        calls = [q8.bind_blockwise_scaled_mm_e8m0(aqd, Wl[c], asd, Wsl[c], Dd, block_n=32, workspace=wsd)
                 for c in range(copies)]
        g = batched_us(torch, lambda c: calls[c](), copies, 30)
        nbytes = N * K + Ws0.numel() + Md * K + Md * (K // 32) + Md * N * 2
        gbs = nbytes / (g["median"] * 1e-6) / 1e9
        dec[f"M{Md}"] = {"gemm_us": round(g["median"], 3), "algorithmic_bytes": nbytes,
                         "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    res["decode_4096x7168_block32"] = dec
    return res


def bench_int8(torch, q8, synth, reps):
    M, N, K = 2048, 8192, 8192
    dev = "cuda:0"
    x = synth.activations(M, K, "bf16", seed=0).to(dev)
    Wq, ws = synth.int8_weights(N, K, per_channel=True, seed=0)
    Wq, ws = Wq.to(dev), ws.to(dev)
    b = synth.bias(N, seed=0).to(dev)
    qa = torch.empty((M, K), dtype=torch.int8, device=dev)
    sa = torch.empty((M, 1), dtype=torch.float32, device=dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gt, qt = KernelTimer(torch), KernelTimer(torch)
    for i in range(reps + 5):
        if i >= 5:
            with qt:
                q8.quant_8bit(x, qa, sa, K, EPS, -128.0, 127.0, False)
            with gt:
                q8.scaled_mm_int8(qa, Wq, sa, ws, torch.bfloat16, b, out=D)
        else:
            q8.quant_8bit(x, qa, sa, K, EPS, -128.0, 127.0, False)
            q8.scaled_mm_int8(qa, Wq, sa, ws, torch.bfloat16, b, out=D)
    torch.cuda.synchronize()
    g = gt.us()
    tops = 2.0 * M * N * K / (g["median"] * 1e-6) / 1e12
    return {"gemm_us": round(g["median"], 2), "quant_us": round(qt.us()["median"], 2),
            "TOP/s": round(tops, 1), "frac_int8_peak": round(tops / PEAK_INT8_TOPS, 4)}


def bench_fp8_scaled(torch, q8, synth, reps):
    """Per-token FP8 quant of the prefill activation + FP8 GEMM against
    per-channel FP8 weights (one scale per row), bf16 out."""
    M, N, K = 4096, 7168, 7168
    dev = "cuda:0"
    x = synth.activations(M, K, "bf16", seed=0).to(dev)
    Wq, Ws = synth.fp8_block_weights(N, K, 1, K, seed=0)
    Wq, Ws = Wq.to(dev).view(torch.float8_e4m3fn), Ws.reshape(-1).to(dev)
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    sa = torch.empty((M, 1), dtype=torch.float32, device=dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gt, qt = KernelTimer(torch), KernelTimer(torch)
    for i in range(reps + 5):
        if i >= 5:
            with qt:
                q8.quant_8bit(x, aq, sa, K, EPS, -448.0, 448.0, False)
            with gt:
                q8.scaled_mm_fp8(aq, Wq, sa.reshape(-1), Ws, torch.bfloat16, out=D)
        else:
            q8.quant_8bit(x, aq, sa, K, EPS, -448.0, 448.0, False)
            q8.scaled_mm_fp8(aq, Wq, sa.reshape(-1), Ws, torch.bfloat16, out=D)
    torch.cuda.synchronize()
    g = gt.us()
    tf = 2.0 * M * N * K / (g["median"] * 1e-6) / 1e12
    return {"gemm_us": round(g["median"], 2), "quant_us": round(qt.us()["median"], 2),
            "TFLOP/s": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}


def bench_moe(torch, q8, synth, reps):
    T, E, topk, N, K, blk = 4096, 64, 8, 2048, 7168, 128
    dev = "cuda:0"
    ids = synth.zipf_topk_ids(T, E, topk, seed=0).to(dev)
    x = synth.activations(T, K, "bf16", seed=0).to(dev)
    W, Ws = synth.fp8_block_weights(N, K, blk, blk, experts=E, seed=0)
    W, Ws = W.to(dev), Ws.to(dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ps1 = torch.empty((E, 3), dtype=torch.int32, device=dev)
    ps2 = torch.empty((E, 3), dtype=torch.int32, device=dev)
    ip = torch.empty(T * topk, dtype=torch.int32, device=dev)
    op = torch.empty(T * topk, dtype=torch.int32, device=dev)
    aq = torch.empty((T, K), dtype=torch.float8_e4m3fn, device=dev)
    As = torch.empty((T, K // blk), dtype=torch.float32, device=dev)
    D = torch.empty((T * topk, N), dtype=torch.bfloat16, device=dev)
    Ds = torch.empty((T * topk, N), dtype=torch.bfloat16, device=dev)
    gw = synth.topk_weights(T, topk, seed=0).to(dev)
    out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    rt, qt, gt = KernelTimer(torch), KernelTimer(torch), KernelTimer(torch)
    st, ft = KernelTimer(torch), KernelTimer(torch)
    for i in range(reps + 3):
        timed = i >= 3
        with (rt if timed else _Null()):
            q8.moe_mm_data(ids, off, ps1, ps2, ip, op, E, N, K)
        with (qt if timed else _Null()):
            q8.quant_8bit(x, aq, As, blk, EPS, -448.0, 448.0, False)
        with (gt if timed else _Null()):
            q8.grouped_blockwise_scaled_mm(D, aq, W, As, Ws, off, ps1, a_map=ip, c_map=op)
        # the variant that finalizes: expert-sorted rows (no scatter), then the
        # weighted top-k sum reads them through the output permutation
        with (st if timed else _Null()):
            q8.grouped_blockwise_scaled_mm(Ds, aq, W, As, Ws, off, ps1, a_map=ip)
        with (ft if timed else _Null()):
            q8.moe_finalize(Ds, gw, topk, op, out=out)
    torch.cuda.synchronize()
    g = gt.us()
    fin = ft.us()["median"]
    fin_bytes = T * topk * N * 2 + T * N * 2 + T * topk * 8
    step_us = rt.us()["median"] + qt.us()["median"] + g["median"]
    flops = 2.0 * T * topk * N * K
    nbytes = E * N * K + T * K + T * topk * N * 2 + Ws.numel() * 4 + T * (K // blk) * 4
    return {"routing_us": round(rt.us()["median"], 2), "quant_us": round(qt.us()["median"], 2),
            "grouped_gemm_us": round(g["median"], 2),
            "gemm_tflops": round(flops / (g["median"] * 1e-6) / 1e12, 1),
            "frac_fp8_peak": round(flops / (g["median"] * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "gemm_GB/s_fused": round(nbytes / (g["median"] * 1e-6) / 1e9, 1),
            "step_tflops": round(flops / (step_us * 1e-6) / 1e12, 1),
            "grouped_gemm_sorted_us": round(st.us()["median"], 2),
            "finalize_us": round(fin, 2), "finalize_GB/s": round(fin_bytes / (fin * 1e-6) / 1e9, 1),
            "finalize_frac_hbm": round(fin_bytes / (fin * 1e-6) / 1e9 / 8000.0, 4)}


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def traffic_probe(torch, q8, synth) -> int:
    """Kernels for the HBM byte counters: three prefill GEMM launches, three
    decode GEMM launches each at M=1, 16 and 64, and three MoE grouped GEMM
    launches (a 256 MiB fill before each, so the operands are not resident in
    the Infinity Cache), and three plain 256 MiB device-to-device copies of
    known size (the scale for FETCH_SIZE / WRITE_SIZE)."""
    M, N, K, blk = 4096, 7168, 7168, 128
    dev = "cuda:0"
    x = synth.activations(M, K, "bf16", seed=0).to(dev)
    Wq, Ws = synth.fp8_block_weights(N, K, blk, blk, seed=0)
    Wq, Ws = Wq.to(dev), Ws.to(dev)
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    As = torch.empty((M, K // blk), dtype=torch.float32, device=dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    big = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
    dst = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    for _ in range(3):
        q8.quant_8bit(x, aq, As, blk, EPS, -448.0, 448.0, False)
        big.fill_(1)  # evict: 256 MiB written between launches
        q8.blockwise_scaled_mm(aq, Wq, As, Ws, torch.bfloat16, block=(blk, blk), out=D)
    # decode block32 GEMMs (N=4096, K=7168): M=1 (four rows' block partials per
    # MFMA), M=16 (activations staged in LDS once per workgroup) and M=64
    # (split K: float32 partials in the workspace, then the fixed-order sum)
    Nd, db = 4096, 32
    Wd, Wsd = synth.fp8_block_weights(Nd, K, db, db, seed=0)
    Wd, Wsd = Wd.to(dev), Wsd.to(dev)
    for Md in (1, 16, 64):
        xd = synth.activations(Md, K, "bf16", outlier_frac=0.01, seed=0).to(dev)
        aqd = torch.empty((Md, K), dtype=torch.float8_e4m3fn, device=dev)
        Asd = torch.empty((Md, K // db), dtype=torch.float32, device=dev)
        Dd = torch.empty((Md, Nd), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            q8.quant_8bit(xd, aqd, Asd, db, EPS, -448.0, 448.0, True)
            big.fill_(1)
            q8.blockwise_scaled_mm(aqd, Wd, Asd, Wsd, torch.bfloat16, block=(db, db), out=Dd)
    # MoE grouped GEMM (4096 tokens, top-8 of 64 experts, N=2048, K=7168) with
    # the fused gather and scatter: 939.5 MB of expert weights per launch
    del Wq, Ws, D, Wd, Wsd
    T, E, topk, Ne = 4096, 64, 8, 2048
    ids = synth.zipf_topk_ids(T, E, topk, seed=0).to(dev)
    We, Wse = synth.fp8_block_weights(Ne, K, blk, blk, experts=E, seed=0)
    We, Wse = We.to(dev), Wse.to(dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ps1 = torch.empty((E, 3), dtype=torch.int32, device=dev)
    ps2 = torch.empty((E, 3), dtype=torch.int32, device=dev)
    ip = torch.empty(T * topk, dtype=torch.int32, device=dev)
    op = torch.empty(T * topk, dtype=torch.int32, device=dev)
    De = torch.empty((T * topk, Ne), dtype=torch.bfloat16, device=dev)
    q8.moe_mm_data(ids, off, ps1, ps2, ip, op, E, Ne, K)
    q8.quant_8bit(x, aq, As, blk, EPS, -448.0, 448.0, False)
    for _ in range(3):
        big.fill_(1)
        q8.grouped_blockwise_scaled_mm(De, aq, We, As, Wse, off, ps1, a_map=ip, c_map=op)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("traffic probe done: 3 prefill GEMM launches, 3 decode GEMM launches each at M=1, 16 and 64, "
        "3 MoE grouped GEMM launches, 3 copies of 268435456 bytes")
    return 0


def cpu_baseline(pre, rows: int):
    """The oracle as it stands, on the first ``rows`` rows of the prefill
    workload: quantize those rows, then the block-scaled GEMM against all of W."""
    import numpy as np

    from oracle import gemm as og
    from oracle import quant as oq
    M, N, K, blk = pre["shape"]
    x = pre["x"][:rows].float().cpu().numpy()
    Wq = pre["Wq"].cpu().numpy()
    Ws = pre["Ws"].cpu().numpy()
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=None)
    except Exception:
        pass
    t0 = time.perf_counter()
    aq, As = oq.per_token_group(x, blk, EPS, -448.0, 448.0, False, "e4m3")
    og.blockwise_scaled_mm(aq, As, Wq, Ws, blk, blk)
    dt = time.perf_counter() - t0
    _ = np
    return {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"prefill rows 0..{rows - 1} of {M} (quant + block GEMM, N={N}, K={K}), {dt:.2f} s of CPU time"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--clock-ramp-ms", type=float, default=150.0,
                    help="untimed prefill steps for this long before the warm-up steps (clock settling)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="prefill rows for the oracle baseline")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run prefill GEMM launches and a 256 MiB device copy (for HBM counters)")
    ap.add_argument("--skip-secondary", action="store_true", help="headline prefill only")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2

    import torch

    import int8_quantized_gemm_amd as q8
    import synth

    torch.cuda.init()
    log(f"device {torch.cuda.get_device_name(0)}")
    if args.traffic_probe:
        return traffic_probe(torch, q8, synth)
    pre = bench_prefill(torch, q8, synth, args.steps, args.warmup, args.clock_ramp_ms)
    log(f"prefill: {pre['ms_per_step']:.3f} ms/step, GEMM {pre['gemm_us']['mean']:.1f} us "
        f"= {pre['gemm_tflops']:.0f} TFLOP/s")
    M, N, K, blk = pre["shape"]
    sha = tile_kernel_sha()
    roof = {"bound": "mfma", "achieved": round(pre["gemm_tflops"], 1), "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": round(pre["gemm_tflops"] / PEAK_FP8_TFLOPS, 4),
            "traffic": measured_traffic("gemm_tile", "prefill_4096x7168x7168", sha),
            "kernel": "gemm_tile (block-FP8, [128,128])",
            "kernel_us": {k: round(v, 2) for k, v in pre["gemm_us"].items()}}
    paths = {"prefill_quant_us": {k: round(v, 2) for k, v in pre["quant_us"].items()}}
    if not args.skip_secondary:
        reps = max(args.steps, 50)
        paths["prefill_gemm"] = bench_prefill_variants(torch, q8, synth, pre, reps)
        log(f"prefill variants: {json.dumps(paths['prefill_gemm'])}")
        paths["decode_block32"] = bench_decode(torch, q8, synth, 30)
        log(f"decode: {json.dumps(paths['decode_block32'])}")
        paths["quant_4096x7168"] = bench_quant(torch, q8, synth, 30)
        log(f"quant: {json.dumps(paths['quant_4096x7168'])}")
        paths["silu_quant"] = bench_silu_quant(torch, q8, synth, 30)
        log(f"silu quant: {json.dumps(paths['silu_quant'])}")
        paths["e8m0_block32"] = bench_e8m0(torch, q8, synth, reps)
        log(f"e8m0: {json.dumps(paths['e8m0_block32'])}")
        paths["int8_2048x8192x8192"] = bench_int8(torch, q8, synth, reps)
        log(f"int8: {json.dumps(paths['int8_2048x8192x8192'])}")
        paths["fp8_per_token_x_channel_4096x7168x7168"] = bench_fp8_scaled(torch, q8, synth, reps)
        log(f"fp8 scaled: {json.dumps(paths['fp8_per_token_x_channel_4096x7168x7168'])}")
        paths["moe_4096tok_e64_top8"] = bench_moe(torch, q8, synth, reps)
        log(f"moe: {json.dumps(paths['moe_4096tok_e64_top8'])}")
    cpu = cpu_baseline(pre, args.cpu_rows) if args.cpu_rows > 0 else None
    line = {
        "metric": "TFLOP/s & % fp8 MFMA peak (prefill), GB/s & % HBM (decode M≤16)",
        "value": round(pre["tflops_step"], 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp": pre["clock_ramp"],
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "prefill: group-128 FP8 activation quant + [128,128]-block-scaled FP8 GEMM, bf16 out",
                   "M": M, "N": N, "K": K, "block": [blk, blk], "activation": "bf16 N(0,1)",
                   "weight": "N(0,0.02) quantized per [128,128] tile", "bias": None},
        "roofline": roof,
        "cpu_baseline": cpu,
        "paths": paths,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
