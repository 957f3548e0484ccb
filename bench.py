#!/usr/bin/env python3
"""Benchmark of the NVFP4 MoE layer on one MI355X.

One step = one forward of the whole hot path on one batch: route + permute and
NVFP4 quantisation of the activations (one call whose kernels share launches),
gate_up grouped GEMM with the fused
SwiGLU + re-quantisation and down grouped GEMM (bf16 rows) through
moe_expert_ffn (one persistent launch from 48 rows per expert, the default
workload's 64), weighted gather combine to bf16 token order.  Default workload: the decode MoE at
16-64 tokens per expert (T=2048, H=6144, I=256, E=256, top-8, Zipf-skewed
routing), seeded synthetic inputs, weights drawn N(0, 0.02) and quantised to
NVFP4 on the GPU and repacked into the streaming tile layout (untimed).  Two
weight copies alternate between steps so the
256 MB last-level cache cannot serve a step's weights from the previous step.

Prints ONE JSON line: value = touched expert weight bytes (codes + scales of
both GEMMs, experts that received tokens) per second of layer step, plus the
layer's TFLOPS, per-stage times, the roofline of the dominant kernel (the
gate_up GEMM), and the CPU oracle timed on a sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload 2]
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16/BF16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4/FP6 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2,
                    help="workload index: 0..3 MoE layers (2 is the reported one), 4 the dense 8192^3 GEMM")
    ap.add_argument("--tokens", type=int, default=0,
                    help="MoE workloads: T tokens instead of the workload's own, same recipe otherwise (a sweep "
                         "over tokens per expert; not the reported line)")
    ap.add_argument("--ffn", choices=["one_launch", "two_launch"], default="one_launch",
                    help="gate_up + down through moe_expert_ffn (one persistent launch at decode sizes) or the two "
                         "grouped-GEMM calls")
    ap.add_argument("--format", choices=["nvfp4", "mxfp4", "fp8"], default="nvfp4",
                    help="number format: NVFP4 (the reported one), the MXFP4 variant (E8M0 scale per 32, "
                         "gfx950's block-scaled FP4 MFMA) or the FP8 block-scaled grouped GEMMs (E4M3, float32 "
                         "scales per 1x128 / 128x128 block)")
    ap.add_argument("--launch", choices=["eager", "graph"], default="eager",
                    help="launch each timed step's kernels one by one, or replay it as one HIP graph of its kernels "
                         "(recorded once per weight copy; measured slower on MI355X: 0.355 against 0.329 ms)")
    ap.add_argument("--swiglu", choices=["fused", "separate"], default="fused",
                    help="SwiGLU + requant in the gate_up epilogue, or a separate call")
    ap.add_argument("--combine", choices=["gather", "atomic", "fused"], default="gather",
                    help="bf16 down output + gather combine, float32 atomic scatter-add epilogue, or the combine "
                         "fused into the expert-FFN call (one-launch regime: inside the persistent launch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the CPU-oracle sample")
    ap.add_argument("--oracle-only", action="store_true",
                    help="time only the CPU oracle on the workload (no GPU) and print one JSON line")
    ap.add_argument("--oracle-threads", type=int, default=0, help="BLAS threads of the oracle (0: all)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB 5 times (to scale HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}), flush=True)


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("grouped_gemm.hip", "gemm_device.h", "moe_ffn.hip", "nvfp4_device.h"):
        with open(os.path.join(ROOT, "block_scaled_fp4_permute_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    ent = d.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_hash") != gemm_source_hash():
        return None
    return ent.get("bytes_per_launch")


def host_cpu():
    """Host CPU model (from /proc/cpuinfo, as lscpu reports it) and logical CPU count."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"host_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline(cfg, logits_np, x_np, expert_weights, g_h, budget_s=15.0, pool=8, threads=None):
    """The CPU oracle, as it stands, on a bounded sample of the same workload.

    Timed: whole layer steps, repeated - routing, permutation and activation
    quantisation over all T tokens, then expert by expert (in id order, experts
    with tokens only) the gate_up GEMM of the expert's routed rows, SwiGLU +
    re-quantisation, the down GEMM and the weighted combine of its rows - until
    ``budget_s`` seconds have passed (checked after each expert).  Expert
    weights are quantised by the oracle outside the timed region; to keep that
    preparation short, ``pool`` experts' weights are quantised and expert e
    computes with pool[e % pool] (same shapes, so the same arithmetic volume).
    Returns the throughput in the benchmark's unit: weight bytes of the experts
    done per second."""
    import contextlib

    import numpy as np
    from oracle import moe as OM
    from oracle import quant as OQ
    from threadpoolctl import threadpool_info, threadpool_limits
    wq = [tuple(OQ.quantize(w) for w in expert_weights(e)) for e in range(min(pool, cfg.E))]
    limit = threadpool_limits(limits=threads) if threads else contextlib.nullcontext()
    with limit:
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        res = _cpu_baseline_timed(cfg, logits_np, x_np, wq, g_h, budget_s)
    res["cores"] = int(used)
    res.update(host_cpu())
    return res


def _cpu_baseline_timed(cfg, logits_np, x_np, wq, g_h, budget_s):
    import numpy as np
    from oracle import moe as OM
    from oracle import quant as OQ
    done = rows_done = passes = 0
    n_touched = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        ids, w = OM.route(logits_np, cfg.k)
        counts, offsets, src, perm_of, pw = OM.permute(ids, w, cfg.E)
        xq = OQ.quantize(x_np)
        out = np.zeros((cfg.T, cfg.H), np.float64)
        touched = [e for e in range(cfg.E) if counts[e] > 0]
        n_touched = len(touched)
        for e in touched:
            (gc, gs, gg), (dc, ds, dg) = wq[e % len(wq)]
            p0, p1 = int(offsets[e]), int(offsets[e + 1])
            rows = src[p0:p1]
            off = np.array([0, p1 - p0])
            y1, _ = OM.grouped_gemm(*xq, gc[None], gs[None], np.array([gg]), off, a_rows=rows, want_absdot=False)
            hc, hs, hg, _ = OM.swiglu_quantize(y1, g_h)
            y2, _ = OM.grouped_gemm(hc, hs, hg, dc[None], ds[None], np.array([dg]), off, want_absdot=False)
            np.add.at(out, rows, pw[p0:p1, None].astype(np.float64) * y2)
            done += 1
            rows_done += p1 - p0
            if time.perf_counter() - t0 >= budget_s:
                break
        passes += 1
    dt = time.perf_counter() - t0
    per_expert = 3 * cfg.I * cfg.H * 9 // 16
    return {"value": round(done * per_expert / dt / 1e9, 6), "unit": "GB/s",
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{passes} pass(es) of the layer step, {done} expert GEMM pairs in all ({n_touched} touched "
                      f"experts per step; {rows_done} routed rows; weights from a pool of {len(wq)} "
                      f"oracle-quantised experts): gate_up, SwiGLU+requant, down, weighted combine, with routing, "
                      f"permutation and activation quantisation over all {cfg.T} tokens each pass; numpy, float64; "
                      f"stopped after {budget_s:g} s"}


def dense_gemm(cfg, args):
    """The single dense NVFP4 GEMM (E=1, no routing, bf16 out): A [M, K] and
    B [N, K] drawn N(0, 1) on the GPU, quantised to NVFP4 (B repacked) untimed;
    K steps of the GEMM alone, timed with events on the launch stream.  A
    secondary measurement of the MFMA-bound regime; not the reported metric."""
    import numpy as np
    import torch

    from block_scaled_fp4_permute_amd import EPI_BF16, lib, nvfp4_grouped_gemm, nvfp4_quantize, nvfp4_weight_repack

    lib()
    dev = torch.device("cuda:0")
    M, N, K = cfg.T, cfg.H, cfg.I
    a32, b32 = workloads_mod().torch_dense_operands(cfg, dev)
    aq = nvfp4_quantize(a32)
    bq = nvfp4_quantize(b32)
    del a32, b32
    b_codes, b_scales = bq.codes.view(1, N, K // 2), bq.scales.view(1, N, K // 16)
    packed = nvfp4_weight_repack(b_codes, b_scales)
    offsets = torch.tensor([0, M], dtype=torch.int32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def run():
        nvfp4_grouped_gemm(aq, b_codes, b_scales, bq.g, offsets, m_total=M, epilogue=EPI_BF16, out=out,
                           max_rows_per_expert_hint=M, b_packed=packed)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s_, e_ in evs:
        s_.record()
        run()
        e_.record()
    torch.cuda.synchronize()
    ms = float(np.mean([s_.elapsed_time(e_) for s_, e_ in evs]))
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "dense NVFP4 GEMM TFLOP/s (secondary: the MFMA-bound regime)", "value": round(tflops, 1),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "vs_baseline": None, "dtype": "nvfp4 operands, f16 mfma, f32 accumulate",
        "data": "synthetic", "config": {"workload": f"dense_gemm_M{M}_N{N}_K{K}", "out": "bf16"},
        "roofline": {"kernel": "nvfp4 grouped GEMM, large-M tile", "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "frac_fp8_peak": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None}}), flush=True)


def oracle_only(args):
    """The CPU oracle alone on a MoE workload (weights drawn on the host from
    the seeded recipe; g_h from the workload's static calibration), with a
    chosen number of BLAS threads: the single- and all-thread oracle timings."""
    import numpy as np

    wl = workloads_mod()
    cfg = wl.CONFIGS[args.workload]
    g_h = float(np.float32(np.float32(wl.H_CALIBRATION_AMAX[cfg.index]) / np.float32(2688.0)))
    res = cpu_baseline(cfg, wl.logits(cfg), wl.activations(cfg),
                       lambda e: (wl.gate_up_weight(cfg, e), wl.down_weight(cfg, e)), g_h,
                       budget_s=args.cpu_seconds, pool=min(8, cfg.E), threads=args.oracle_threads or None)
    print(json.dumps({"oracle_only": True, "workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                      "top_k": cfg.k, "threads_requested": args.oracle_threads or "all", **res}), flush=True)


def mx_bench(cfg, args):
    """The MXFP4 variant (secondary measurements, not the reported metric):
    the MoE layer step on the MoE workloads (route + permute, MXFP4 quantise
    of x, gate_up with fused SwiGLU + MXFP4 requant, down, combine), or the
    dense GEMM.  Roofline of the gate_up kernel against HBM (MoE below 256
    rows per expert) or against the dense FP4 MFMA peak (MoE from 256 rows per
    expert, and the dense GEMM), with the FP8 peak fraction beside it."""
    import numpy as np
    import torch

    from block_scaled_fp4_permute_amd import EPI_BF16, lib, mxfp4_grouped_gemm, mxfp4_quantize
    from block_scaled_fp4_permute_amd.layer import MXMoELayer, quantize_expert_weights_mx

    lib()
    dev = torch.device("cuda:0")
    wl = workloads_mod()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    if cfg.dense:
        M, N, K = cfg.T, cfg.H, cfg.I
        a32, b32 = wl.torch_dense_operands(cfg, dev)
        aq, bq = mxfp4_quantize(a32), mxfp4_quantize(b32)
        del a32, b32
        from block_scaled_fp4_permute_amd import MXFP4Tensor
        from block_scaled_fp4_permute_amd import mxfp4_weight_repack
        b3 = MXFP4Tensor(bq.codes.view(1, N, K // 2), bq.scales.view(1, N, K // 32))
        b3p = mxfp4_weight_repack(b3)
        offsets = torch.tensor([0, M], dtype=torch.int32, device=dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def run():
            mxfp4_grouped_gemm(aq, b3, offsets, m_total=M, epilogue=EPI_BF16, out=out, max_rows_per_expert_hint=M,
                               b_packed=b3p)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0, t1 = ev(), ev()
        t0.record()
        for _ in range(args.steps):
            run()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "dense MXFP4 GEMM TFLOP/s (secondary: gfx950 block-scaled FP4 MFMA)", "value": round(tflops, 1),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "vs_baseline": None, "dtype": "mxfp4 operands, fp4 scaled mfma, f32 accumulate",
            "data": "synthetic", "config": {"workload": f"dense_gemm_M{M}_N{N}_K{K}", "format": "mxfp4", "out": "bf16"},
            "roofline": {"kernel": "k_mx_gemm_l (256 x 256 tile, both operands staged in LDS)", "bound": "mfma",
                         "achieved": round(tflops, 1), "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_FP4_PEAK_TFLOPS, 4),
                         "frac_fp8_peak": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None}}), flush=True)
        return

    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    logits = torch.from_numpy(wl.logits(cfg)).to(dev)
    x = torch.from_numpy(wl.activations(cfg)).to(dev).to(torch.bfloat16)
    copies = []
    for c in range(2):
        w_gu, w_dn = wl.torch_expert_weights(cfg, dev, copy=c)
        copies.append(quantize_expert_weights_mx(w_gu, w_dn))
        del w_gu, w_dn
    layer = MXMoELayer(T, H, I, E, k, dev)
    for i in range(args.warmup):
        layer.forward(logits, x, copies[i % 2])
    torch.cuda.synchronize()
    counts = layer.routing.counts.cpu().numpy()
    t_start, t_end = ev(), ev()
    gu_marks = [[None, None, ev(), ev(), None, None] for _ in range(args.steps)]
    t_start.record()
    for i in range(args.steps):
        layer.forward(logits, x, copies[i % 2], marks=gu_marks[i])
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    gu_ms = float(np.mean([m_[2].elapsed_time(m_[3]) for m_ in gu_marks]))
    marks = [[ev() for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        layer.forward(logits, x, copies[i % 2], marks=marks[i])
    torch.cuda.synchronize()
    names = ["route_permute", "quantize_x", "gate_up_swiglu", "down", "combine"]
    stage_ms = {n: round(float(np.mean([m_[j].elapsed_time(m_[j + 1]) for m_ in marks])), 5)
                for j, n in enumerate(names)}
    touched = int((counts > 0).sum())
    bpe = 17 / 32                         # bytes per element: 4-bit code + one byte per 32
    gu_w = 2 * I * H * bpe
    dn_w = H * I * bpe
    weight_bytes = touched * (gu_w + dn_w)
    gu_alg = touched * gu_w + T * H * bpe + T * k * I * bpe
    # from 256 rows per expert gate_up runs the 256 x 256 tile and is bound by
    # the matrix cores: its roofline is then the dense FP4 MFMA peak
    large = (T * k) // E >= 256
    gu_flops = 2.0 * T * k * 2 * I * H
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    gu_gbs = gu_alg / (gu_ms * 1e-3) / 1e9
    if large:
        roof = {"kernel": "k_mx_gemm_l gate_up + SwiGLU/MXFP4 requant epilogue (256 x 256 tile)", "bound": "mfma",
                "achieved": round(gu_tflops, 1), "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tflops / MFMA_FP4_PEAK_TFLOPS, 4),
                "frac_fp8_peak": round(gu_tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None,
                "flops_per_launch": gu_flops, "avg_launch_ms": round(gu_ms, 5), "hbm_gbs": round(gu_gbs, 2)}
    else:
        roof = {"kernel": "k_mx_gemm gate_up + SwiGLU/MXFP4 requant epilogue", "bound": "hbm",
                "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "alg_bytes_per_launch": int(gu_alg), "avg_launch_ms": round(gu_ms, 5)}
    print(json.dumps({
        "metric": "MXFP4 MoE layer weight GB/s (secondary: the block format gfx950's scaled FP4 MFMA takes natively)",
        "value": round(weight_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "vs_baseline": None,
        "dtype": "mxfp4 operands, fp4 scaled mfma, f32 accumulate", "data": "synthetic",
        "tflops": round(2.0 * T * k * 3 * I * H / (ms * 1e-3) / 1e12, 3), "weight_bytes": int(weight_bytes),
        "stage_ms": stage_ms,
        "config": {"workload": f"{'decode' if T <= 2048 else 'prefill'}_moe_T{T}_H{H}_I{I}_E{E}_top{k}_{cfg.routing}",
                   "format": "mxfp4", "weight_copies": 2},
        "roofline": roof}), flush=True)


def fp8_bench(cfg, args):
    """The FP8 block-scaled variant (secondary measurements, not the reported
    metric).  MoE workloads: the FP8 layer step (route + permute, FP8
    quantisation of x, gate_up grouped GEMM with SwiGLU + FP8 requant in its
    epilogue below 256 rows per expert (--swiglu separate, or from 256 rows:
    float32 rows and the separate SwiGLU kernel), down grouped GEMM with bf16
    rows, combine), weights quantised with
    128 x 128 blocks and repacked (untimed), two weight copies alternating;
    roofline of gate_up against HBM.  Dense workload: the GEMM against the
    dense FP8 MFMA peak."""
    import numpy as np
    import torch

    from block_scaled_fp4_permute_amd import EPI_BF16, fp8_grouped_gemm, fp8_quantize, fp8_weight_repack, lib

    lib()
    dev = torch.device("cuda:0")
    wl = workloads_mod()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed(run, steps):
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
        t0, t1 = ev(), ev()
        t0.record()
        for i in range(steps):
            run(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    if cfg.dense:
        M, N, K = cfg.T, cfg.H, cfg.I
        a32, b32 = wl.torch_dense_operands(cfg, dev)
        aq, bq = fp8_quantize(a32, 1), fp8_quantize(b32.view(1, N, K), 128)
        del a32, b32
        bp = fp8_weight_repack(bq.codes)
        offsets = torch.tensor([0, M], dtype=torch.int32, device=dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda i: fp8_grouped_gemm(aq, bp, bq.scales, offsets, N=N, m_total=M, epilogue=EPI_BF16, out=out,
                                              max_rows_per_expert_hint=M), args.steps)
        tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "dense FP8 block-scaled GEMM TFLOP/s (secondary: gfx950 FP8 MFMA)", "value": round(tflops, 1),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "vs_baseline": None,
            "dtype": "e4m3 operands, f32 block scales, fp8 mfma, f32 accumulate", "data": "synthetic",
            "config": {"workload": f"dense_gemm_M{M}_N{N}_K{K}", "format": "fp8_block128", "out": "bf16"},
            "roofline": {"kernel": "k_fp8_gemm_l (256 x 256 tile, both operands staged in LDS)", "bound": "mfma",
                         "achieved": round(tflops, 1), "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None}}), flush=True)
        return

    from block_scaled_fp4_permute_amd.layer import FP8MoELayer, quantize_expert_weights_fp8
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    M = T * k
    logits = torch.from_numpy(wl.logits(cfg)).to(dev)
    x = torch.from_numpy(wl.activations(cfg)).to(dev).to(torch.bfloat16)
    copies = []
    for c in range(2):
        w_gu, w_dn = wl.torch_expert_weights(cfg, dev, copy=c)
        copies.append(quantize_expert_weights_fp8(w_gu, w_dn))
        del w_gu, w_dn
    layer = FP8MoELayer(T, H, I, E, k, dev, swiglu=args.swiglu)
    ms = timed(lambda i: layer.forward(logits, x, copies[i % 2]), args.steps)
    marks = [[ev() for _ in range(7)] for _ in range(args.steps)]
    for i in range(args.steps):
        layer.forward(logits, x, copies[i % 2], marks=marks[i])
    torch.cuda.synchronize()
    # fused SwiGLU: marks 3 and 4 both follow gate_up, whose stage includes it
    names = ["route_permute", "quantize_x", "gate_up_swiglu" if layer.fused else "gate_up",
             None if layer.fused else "swiglu_quantize", "down", "combine"]
    stage_ms = {n: round(float(np.mean([m_[j].elapsed_time(m_[j + 1]) for m_ in marks])), 5)
                for j, n in enumerate(names) if n}
    gu_ms = stage_ms["gate_up_swiglu" if layer.fused else "gate_up"]
    counts = layer.routing.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    gu_w = 2 * I * H * (1 + 4 / (128 * 128))        # E4M3 codes + one float32 per 128 x 128 block
    dn_w = H * I * (1 + 4 / (128 * 128))
    weight_bytes = touched * (gu_w + dn_w)
    # gate_up writes float32 rows, or (fused SwiGLU) h in FP8 with one float32 per 128 values
    gu_out = M * I * (1 + 4 / 128) if layer.fused else M * 2 * I * 4
    gu_alg = touched * gu_w + T * H * (1 + 4 / 128) + gu_out
    gu_gbs = gu_alg / (gu_ms * 1e-3) / 1e9
    # from 256 rows per expert gate_up runs the 256 x 256 tile, bound by the
    # matrix cores: its roofline is then the dense FP8 MFMA peak
    if M // E >= 256:
        gu_flops = 2.0 * M * 2 * I * H
        gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"kernel": "k_fp8_gemm_l gate_up (float32 rows, 256 x 256 tile)", "bound": "mfma",
                "achieved": round(gu_tflops, 1), "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None,
                "flops_per_launch": gu_flops, "avg_launch_ms": round(gu_ms, 5), "hbm_gbs": round(gu_gbs, 2)}
    else:
        roof = {"kernel": "k_fp8_gemm gate_up + SwiGLU/FP8 requant epilogue" if layer.fused
                else "k_fp8_gemm gate_up (float32 rows)", "bound": "hbm", "achieved": round(gu_gbs, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "alg_bytes_per_launch": int(gu_alg), "avg_launch_ms": round(gu_ms, 5)}
    print(json.dumps({
        "metric": "FP8 block-scaled MoE layer weight GB/s (secondary: E4M3 with float32 scales per 1x128 / 128x128 "
                  "block on the FP8 MFMA)",
        "value": round(weight_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "vs_baseline": None,
        "dtype": "e4m3 operands, f32 block scales, fp8 mfma, f32 accumulate", "data": "synthetic",
        "tflops": round(2.0 * M * 3 * I * H / (ms * 1e-3) / 1e12, 3), "weight_bytes": int(weight_bytes),
        "stage_ms": stage_ms,
        "config": {"workload": f"{'decode' if T <= 2048 else 'prefill'}_moe_T{T}_H{H}_I{I}_E{E}_top{k}_{cfg.routing}",
                   "format": "fp8_block128", "swiglu": "fused" if layer.fused else "separate", "weight_copies": 2},
        "roofline": roof}), flush=True)


def workloads_mod():
    import workloads
    return workloads


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the layer runs "
              "unsharded on a single MI355X and multi-GPU runs are not part of this benchmark", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.oracle_only:
        oracle_only(args)
        return

    import numpy as np
    import torch

    import workloads
    from block_scaled_fp4_permute_amd import EPI_F32, lib, moe_route_permute, moe_swiglu, nvfp4_grouped_gemm, \
        nvfp4_quantize
    from block_scaled_fp4_permute_amd.layer import MoELayer, capture_step, quantize_expert_weights

    lib()
    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS[args.workload]
    if args.tokens > 0 and not cfg.dense:
        cfg = workloads.small_variant(cfg, T=args.tokens)
    if args.format == "fp8":
        fp8_bench(cfg, args)
        return
    if args.format == "mxfp4":
        mx_bench(cfg, args)
        return
    if cfg.dense:
        dense_gemm(cfg, args)
        return
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k

    logits_np = workloads.logits(cfg)
    x_np = workloads.activations(cfg)
    logits = torch.from_numpy(logits_np).to(dev)
    x = torch.from_numpy(x_np).to(dev).to(torch.bfloat16)
    copies = []
    w_gu0 = w_dn0 = None
    for c in range(2):
        w_gu, w_dn = workloads.torch_expert_weights(cfg, dev, copy=c)
        copies.append(quantize_expert_weights(w_gu, w_dn).pack())
        if c == 0:
            w_gu0, w_dn0 = w_gu, w_dn
        else:
            del w_gu, w_dn
    torch.cuda.synchronize()

    # static calibration of the intermediate's per-tensor scale from one
    # unfused pass (amax of h computed on the device)
    r = moe_route_permute(logits, k)
    xq = nvfp4_quantize(x)
    y1 = nvfp4_grouped_gemm(xq, copies[0].gu_codes, copies[0].gu_scales, copies[0].gu_g, r.offsets, m_total=T * k,
                            a_rows=r.perm_src_token, epilogue=EPI_F32)
    g_h = moe_swiglu(y1).g.clone()
    counts = r.counts.cpu().numpy()
    del y1
    torch.cuda.synchronize()

    layer = MoELayer(T, H, I, E, k, dev, swiglu=args.swiglu, combine=args.combine, ffn=args.ffn)
    one_call = layer.ffn == "one_launch"
    # moe_expert_ffn's tile table: one persistent launch from 48 rows per
    # expert, the two grouped-GEMM launches below
    one_launch = one_call and (T * k) // E >= 48
    for i in range(args.warmup):
        layer.forward(logits, x, copies[i % 2], g_h)
    torch.cuda.synchronize()

    # routing and the quantisation of x share launches (one call): one stage
    fused_combine = one_call and layer.combine == "fused"
    if one_call:
        ffn_name = "expert_ffn_one_launch" if one_launch else "expert_ffn_two_launches"
        names = ["route_permute+quantize_x", None, ffn_name + ("+combine" if fused_combine else ""), None,
                 None if fused_combine else "combine"]
    else:
        names = ["route_permute+quantize_x", None, "gate_up_swiglu",
                 "down" if args.combine == "gather" else "down_scatter_add",
                 "combine" if args.combine == "gather" else "to_bf16"]

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---- timed region: exactly K steps.  Eager: two events per step bracket
    # the FFN call on the launch stream (its live average duration).  Graph:
    # each step is one replay of the step's recorded kernels (one graph per
    # weight copy), and the FFN call's duration comes from the instrumented
    # eager steps below.
    graphs = None
    if args.launch == "graph":
        graphs = [capture_step(layer, logits, x, copies[c], g_h) for c in range(2)]
        for i in range(args.warmup):
            graphs[i % 2].replay()
        torch.cuda.synchronize()
    t_start, t_end = ev(), ev()
    gu_marks = [[None, None, ev(), ev(), None, None] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        if graphs is not None:
            graphs[i % 2].replay()
        else:
            layer.forward(logits, x, copies[i % 2], g_h, marks=gu_marks[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    eager_ms = None
    if graphs is not None:
        # the same K steps launched kernel by kernel, for reference
        e0, e1 = ev(), ev()
        e0.record()
        for i in range(args.steps):
            layer.forward(logits, x, copies[i % 2], g_h, marks=gu_marks[i])
        e1.record()
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / args.steps
    gu_ms = float(np.mean([m[2].elapsed_time(m[3]) for m in gu_marks]))

    # ---- per-stage breakdown (after the timed region; events between all stages)
    marks = [[ev() for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        layer.forward(logits, x, copies[i % 2], g_h, marks=marks[i])
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([m[j].elapsed_time(m[j + 1]) for m in marks])) for j, n in enumerate(names) if n}

    touched = int((counts > 0).sum())
    gu_bytes_e = 2 * I * H * 9 // 16
    dn_bytes_e = H * I * 9 // 16
    weight_bytes = touched * (gu_bytes_e + dn_bytes_e)
    flops = 2.0 * T * k * 3 * I * H
    gbs = weight_bytes / (ms_per_step * 1e-3) / 1e9
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel.  Algorithmic bytes per launch: gate_up = touched gate_up
    # weights + the NVFP4 activations read once + the NVFP4 h written; down =
    # touched down weights + h read + the bf16 rows written.  The one-launch
    # FFN kernel does both; its bracket also holds the small planning kernel
    # launched with it (so the rate is, if anything, understated).
    gu_alg = touched * gu_bytes_e + T * H * 9 // 16 + T * k * I * 9 // 16
    dn_alg = touched * dn_bytes_e + T * k * I * 9 // 16 + T * k * H * 2
    alg = gu_alg + dn_alg if one_call else gu_alg
    # with the combine fused into the call: + the bf16 rows read back and the
    # bf16 output written (the combine's own algorithmic bytes)
    if fused_combine:
        alg += T * k * H * 2 + T * H * 2
    achieved = alg / (gu_ms * 1e-3) / 1e9
    # from 128 rows per expert the FFN is bound by the matrix cores, not HBM: its roofline is the dense FP16 MFMA
    # peak (the exact NVFP4 path decodes to FP16), with the FP8 peak beside it
    mfma_bound = one_call and (T * k) // E >= 128
    ffn_flops = 2.0 * T * k * 3 * I * H if one_call else 2.0 * T * k * 2 * I * H
    ffn_tflops = ffn_flops / (gu_ms * 1e-3) / 1e12
    wl_name = f"{'decode' if T <= 2048 else 'prefill'}_moe_T{T}_H{H}_I{I}_E{E}_top{k}_{cfg.routing}"
    tkey = ("expert_ffn_one_launch" + ("_fused_combine" if fused_combine else "") if one_launch
            else "expert_ffn_two_launches" if one_call else "gate_up_swiglu")
    traffic = measured_traffic(tkey, wl_name) if args.swiglu == "fused" else None

    res = {
        "metric": "NVFP4 MoE grouped-GEMM TFLOPS & weight GB/s at 16-64 tok/expert, 1 MI355X",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "eager_ms_per_step": None if eager_ms is None else round(eager_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands, f16 mfma, f32 accumulate",
        "data": "synthetic",
        "tflops": round(tflops, 3),
        "gemm_weight_gbs": round(weight_bytes / (sum(stage_ms[n] for n in names[2:4] if n) * 1e-3) / 1e9, 2),
        "tflops_frac_f16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "weight_bytes": weight_bytes,
        "layer_flops": flops,
        "stage_ms": {k_: round(v, 5) for k_, v in stage_ms.items()},
        "tokens_per_expert": {"min": int(counts.min()), "median": float(np.median(counts)),
                              "max": int(counts.max()), "touched_experts": touched},
        "config": {"workload": wl_name, "T": T, "H": H, "I": I, "E": E, "top_k": k, "routing": cfg.routing,
                   "ffn": layer.ffn, "swiglu": args.swiglu, "combine": args.combine, "weight_layout": "packed tiles",
                   "launch": "hip_graph" if graphs is not None else "eager",
                   "weight_copies": 2},
        "roofline": ({"kernel": "k_moe_ffn: gate_up + SwiGLU/requant + down grouped GEMMs"
                      + (" + weighted top-k combine" if fused_combine else "") + ", one persistent launch",
                      "bound": "mfma", "achieved": round(ffn_tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(ffn_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                      "frac_fp8_peak": round(ffn_tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                      "flops_per_launch": ffn_flops, "avg_launch_ms": round(gu_ms, 5),
                      "hbm_gbs": round(achieved, 2)} if mfma_bound else
                     {"kernel": ("k_moe_ffn: gate_up + SwiGLU/requant + down grouped GEMMs"
                                 + (" + weighted top-k combine" if fused_combine else "") + ", one persistent launch"
                                 if one_launch else
                                 "moe_expert_ffn: gate_up + SwiGLU/requant and down grouped GEMMs, two launches"
                                 if one_call else "nvfp4 grouped GEMM gate_up + SwiGLU/requant epilogue"),
                      "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                      "alg_bytes_per_launch": alg, "avg_launch_ms": round(gu_ms, 5)}),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        gh = float(g_h.cpu().numpy()[0])
        res["cpu_baseline"] = cpu_baseline(
            cfg, logits_np, x_np, lambda e: (w_gu0[e].float().cpu().numpy(), w_dn0[e].float().cpu().numpy()), gh,
            budget_s=args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
