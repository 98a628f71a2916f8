#!/usr/bin/env python3
"""Benchmark: BSR block-sparse attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one forward (bsr_attn_fwd) plus one backward (bsr_attn_bwd) over the
configured batch, inputs resident in HBM. At least W untimed steps, and more
until --min-warmup-ms of wall time has passed (clocks ramp up under load), then
K steps timed with HIP events on the stream the library launches on,
bracketed by device synchronisation. Prints one JSON line.

value      effective TFLOP/s counted over stored blocks only:
           14 * B * H * nnzb * 128^2 * D FLOPs per step (forward Q K^T and P V;
           backward Q K^T recomputed, dO V^T, P^T dO, dS K, dS^T Q) / step time.
roofline   the kernel with the largest share of the step, against the bound
           that limits it at peak: its algorithmic FLOPs per launch over its
           average launch duration against the dense MFMA peak of the operand
           dtype ("mfma"), or, when its compulsory HBM bytes take longer at
           8 TB/s than its FLOPs at the MFMA peak (sparse workloads), those
           bytes over the duration against 8 TB/s ("hbm"). Durations come from
           HIP events recorded by the library around each launch during a
           second pass of K steps run right after the timed ones. `traffic`
           comes from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary for
           that kernel when it was taken on the current kernel source, else
           null.
measured_mfma_peak  TFLOP/s of the library's MFMA-loop probe (products on
           random register operands, two waves per SIMD on every CU), timed
           after the other passes: the ceiling that clocks and power allow on
           this device. pct_of_measured_mfma_peak and the roofline's
           frac_of_measured_peak are taken against it.
cpu_baseline  the fp64 CPU oracle on a bounded sample (whole heads of the same
           workload, until --cpu-seconds), in the same effective-FLOP unit.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "fwd+bwd effective TFLOP/s (stored blocks) at seq 8192, % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}  # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0
B128 = 128
# Algorithmic FLOPs per stored block, in units of 128^2 * D, for each kernel:
# fwd: Q K^T, P V; dq: Q K^T, dO V^T, dS K; dkdv: Q K^T, dO V^T, P^T dO, dS^T Q;
# the two-pass forward's passes (head_dim 512's forward): fwd_stats Q K^T,
# fwd_out Q K^T, P V; head_dim 512's backward score blocks: Q K^T, dO V^T.
KERNEL_FLOP_UNITS = {"fwd": 4, "dq": 6, "dkdv": 8, "fwd_stats": 2, "fwd_out": 4, "sddmm_bwd": 4}


def compulsory_bytes(role: str, rows: int, D: int, e: int, blocks: int = 0):
    """Bytes one launch must move through HBM at least (every operand read once,
    every output written once), for rows = batch * heads * seq_len and
    blocks = batch * heads * stored blocks per head:
    fwd reads Q, K, V and writes O, row_max, row_denom; dq reads Q, K, V, O, dO,
    row_max, row_denom and writes dQ, delta, lse2; dkdv reads Q, K, V, dO,
    delta, lse2 and writes dK, dV; fwd_stats reads Q, K and writes the two
    statistics; fwd_out reads Q, K, V and the statistics and writes O;
    sddmm_bwd reads Q, K, V, dO, lse2 and delta and writes the P and dS
    blocks."""
    per_row = {"fwd": 4 * D * e + 8, "dq": 6 * D * e + 16, "dkdv": 6 * D * e + 8, "fwd_stats": 2 * D * e + 8,
               "fwd_out": 4 * D * e + 8, "sddmm_bwd": 4 * D * e + 8}.get(role)
    per_block = 2 * B128 * B128 * e if role == "sddmm_bwd" else 0
    return None if per_row is None else rows * per_row + blocks * per_block
KERNEL_SOURCE = ROOT / "block_sparse_attention_bsr_amd" / "csrc" / "kernels.hip"


def kernel_source_hash() -> str:
    return hashlib.sha256(KERNEL_SOURCE.read_bytes()).hexdigest()[:16]


def read_traffic(kernel_role: str, workload: str):
    """HBM bytes per launch from profiles/<role>_<workload>_traffic.txt, if that
    summary was taken on the current kernel source; else None."""
    path = ROOT / "profiles" / f"{kernel_role}_{workload}_traffic.txt"
    if not path.exists():
        return None
    text = path.read_text()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def roofline_of(kernels: dict, BH: int, nnzb: int, S: int, D: int, dtype: str, workload: str):
    """Roofline object of the kernel with the largest share of the step: its
    algorithmic FLOPs (or compulsory bytes, whichever takes longer at peak)
    per launch over its average launch duration, against the dtype's MFMA
    peak (or 8 TB/s)."""
    if not kernels:
        return None
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
    role = dom.split("<")[0]
    units = KERNEL_FLOP_UNITS.get(role)
    if units is None:
        return {"kernel": dom, "bound": None}
    peak = PEAK_TFLOPS[dtype]
    flops_launch = units * BH * nnzb * B128 * B128 * D
    bytes_launch = compulsory_bytes(role, BH * S, D, 4 if dtype == "fp32" else 2, BH * nnzb)
    sec = kernels[dom]["avg_ms"] * 1e-3
    hbm = bytes_launch / (HBM_PEAK_GBS * 1e9) > flops_launch / (peak * 1e12)
    if hbm:
        achieved, ceiling, unit = bytes_launch / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, ceiling, unit = flops_launch / sec / 1e12, peak, "TFLOP/s"
    return {"bound": "hbm" if hbm else "mfma", "kernel": dom, "achieved": round(achieved, 2),
            "peak": ceiling, "unit": unit, "frac": round(achieved / ceiling, 4),
            "traffic": read_traffic(role, workload),
            "algorithmic_flops_per_launch": flops_launch,
            "compulsory_bytes_per_launch": bytes_launch,
            "mfma_tflops": round(flops_launch / sec / 1e12, 2),
            "hbm_gbs": round(bytes_launch / sec / 1e9, 1)}


def measure_config(bsr, W, torch, name: str, steps: int, min_warmup_ms: float, dev):
    """One workload end to end on its own inputs: time-based warm-up, `steps`
    timed fwd+bwd steps (HIP events on the launch stream), then the same
    steps again under the library's per-launch events. Returns the summary
    the benchmark line carries for every workload."""
    dtype, batch, heads, S, D, kind, dens = W.CONFIGS[name]
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    rp, ci = W.bsr_from_block_mask(W.config_mask(name))
    nnzb = int(len(ci))
    s = bsr.bsr_attn_build_structure(rp, ci)
    q, k, v, do = (t.to(dev, tdt).contiguous() for t in W.make_inputs(batch, heads, S, D, dtype, seed=0))

    def step():
        o, m, l_ = bsr.bsr_attn_fwd(s, q, k, v)
        return bsr.bsr_attn_bwd(s, q, k, v, o, do, m, l_)

    t0, n = time.perf_counter(), 0
    while n < 3 or (time.perf_counter() - t0) * 1e3 < min_warmup_ms:
        step()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    bsr.timing_begin()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kernels = {kn: {"launches": c, "avg_ms": tot / c, "ms_per_step": tot / steps}
               for kn, (c, tot) in bsr.timing_end().items()}
    BH = batch * heads
    flops = 14.0 * BH * nnzb * B128 * B128 * D
    tf = flops / (ms * 1e-3) / 1e12
    return {"dtype": dtype, "shape": [batch, heads, S, D], "mask": kind, "density_target": dens,
            "nnzb_per_head": nnzb, "split_threshold": s.info["split_threshold"], "ms_per_step": round(ms, 4),
            "tflops": round(tf, 2), "pct_of_peak": round(100.0 * tf / PEAK_TFLOPS[dtype], 2),
            "kernels_us": {kn: round(v["avg_ms"] * 1e3, 1) for kn, v in kernels.items()},
            "roofline": roofline_of(kernels, BH, nnzb, S, D, dtype, name)}


DETAIL_CONFIGS = ["c1_fp32_local", "c2_bf16_dilated", "c4_bf16_rand10_d256"] + [
    f"c5_{dt}_rand{d:02d}" for d in (1, 5, 10, 25, 50) for dt in ("bf16", "fp32")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warmup-ms", type=float, default=300.0,
                    help="keep running untimed warm-up steps until this much wall time has passed (the GPU "
                         "raises its clocks only after tens of milliseconds of continuous work)")
    ap.add_argument("--config", default="c3_bf16_global")
    ap.add_argument("--split", type=int, default=0, help="split threshold (0 = automatic)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample: whole heads of the workload, one after another, until this much "
                         "time has passed or every head is done")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip detail.configs (the other workloads, each timed the same way)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain copy kernel (fp32 negation) that reads and writes this many MiB "
                         "before timing: a known-size dispatch for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the "
              "(batch, head) slices would be dealt to GPUs, each computing its own with no "
              "communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_bsr_amd as bsr
    import workloads as W

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    dtype, batch, heads, S, D, kind, dens = W.CONFIGS[args.config]
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    bm = W.config_mask(args.config)
    rp, ci = W.bsr_from_block_mask(bm)
    nnzb = int(len(ci))
    nb = bm.shape[0]

    t_build = time.perf_counter()
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=args.split)
    s.device_plan(dev)
    t_build = time.perf_counter() - t_build

    q, k, v, do = W.make_inputs(batch, heads, S, D, dtype, seed=0)
    qd, kd, vd, dod = (t.to(dev, tdt).contiguous() for t in (q, k, v, do))
    del q, k, v, do

    def step():
        o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
        return bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_)

    if args.calibration_copy_mib > 0:
        # One elementwise dispatch that reads n bytes and writes n bytes.
        n = (args.calibration_copy_mib << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    t_warm = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or (time.perf_counter() - t_warm) * 1e3 < args.min_warmup_ms:
        step()
        n_warm += 1
        if n_warm % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps

    BH = batch * heads
    flops_step = 14.0 * BH * nnzb * B128 * B128 * D
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    workload = args.config

    # Per-kernel durations: the same K steps again, straight after the timed
    # ones, with the library's timing events around every launch (events inside
    # the timed steps would add their own gaps to the step time).
    roofline = None
    kernels = {}
    if not args.no_roofline:
        bsr.timing_begin()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        times = bsr.timing_end()
        kernels = {name: {"launches": n, "avg_ms": tot / n, "ms_per_step": tot / args.steps}
                   for name, (n, tot) in times.items()}
        roofline = roofline_of(kernels, BH, nnzb, S, D, dtype, workload)

    # Forward-only and backward-only times (events around each call).
    fw, bw = [], []
    for _ in range(max(3, min(args.steps, 10))):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
        e[1].record(stream)
        bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_)
        e[2].record(stream)
        torch.cuda.synchronize()
        fw.append(e[0].elapsed_time(e[1]))
        bw.append(e[1].elapsed_time(e[2]))

    # A/B: the pages' two-pass forward (statistics pass, then output pass).
    for _ in range(3):
        bsr.bsr_attn_fwd_two_pass(s, qd, kd, vd)
    torch.cuda.synchronize()
    t2 = []
    for _ in range(max(3, min(args.steps, 10))):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        bsr.bsr_attn_fwd_two_pass(s, qd, kd, vd)
        e[1].record(stream)
        torch.cuda.synchronize()
        t2.append(e[0].elapsed_time(e[1]))

    # A/B: the backward that stores dS in the dK/dV pass and reads it for dQ
    # (16-bit operands), on the same inputs; its per-kernel durations too.
    bwd_ds = None
    if dtype != "fp32":
        o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
        for _ in range(3):
            bsr.bsr_attn_bwd_ds(s, qd, kd, vd, o, dod, m, l_)
        torch.cuda.synchronize()
        td = []
        for _ in range(max(3, min(args.steps, 10))):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            bsr.bsr_attn_bwd_ds(s, qd, kd, vd, o, dod, m, l_)
            e[1].record(stream)
            torch.cuda.synchronize()
            td.append(e[0].elapsed_time(e[1]))
        bsr.timing_begin()
        for _ in range(args.steps):
            bsr.bsr_attn_bwd_ds(s, qd, kd, vd, o, dod, m, l_)
        torch.cuda.synchronize()
        bwd_ds = {"ms_median": round(statistics.median(td), 4),
                  "kernels_us": {n: round(tot / c * 1e3, 1) for n, (c, tot) in bsr.timing_end().items()}}

    # Block-sparse times dense on the same machinery: the pages' SpMM shape
    # (n = 8192, width 512), random blocks + diagonal at 1 % and 10 %, in the
    # configuration's dtype; effective TFLOP/s over stored blocks.
    spmm = {}
    if S == 8192:
        for sp_dens in (0.01, 0.10):
            bm_s = W.block_mask("random", 64, density=sp_dens, seed=0)
            rps, cis = W.bsr_from_block_mask(bm_s)
            ss = bsr.bsr_attn_build_structure(rps, cis)
            gs = torch.Generator().manual_seed(0)
            blocks = torch.randn((len(cis), B128, B128), generator=gs).to(dev, tdt)
            bmat = torch.randn((8192, 512), generator=gs).to(dev, tdt)
            for _ in range(5):
                bsr.bsr_spmm(ss, blocks, bmat)
            torch.cuda.synchronize()
            e0s, e1s = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0s.record(stream)
            for _ in range(args.steps):
                bsr.bsr_spmm(ss, blocks, bmat)
            e1s.record(stream)
            torch.cuda.synchronize()
            ms_s = e0s.elapsed_time(e1s) / args.steps
            fl = 2.0 * len(cis) * B128 * B128 * 512
            hbm = len(cis) * B128 * B128 * bmat.element_size() + 2 * bmat.numel() * bmat.element_size()
            spmm[f"rand{int(sp_dens * 100):02d}_w512"] = {
                "nnzb": len(cis), "ms": round(ms_s, 4), "tflops": round(fl / ms_s / 1e9, 2),
                "compulsory_hbm_gbs": round(hbm / ms_s / 1e6, 1)}
            del blocks, bmat

    # The same step through the autograd wrapper (forward saves the statistics,
    # backward reuses them): wrapper overhead on top of the direct calls.
    ql, kl, vl = (t.detach().clone().requires_grad_() for t in (qd, kd, vd))

    def autograd_step():
        for t in (ql, kl, vl):
            t.grad = None
        bsr.block_sparse_attention(ql, kl, vl, s).backward(dod)

    # the same time-based warm-up as the timed steps: the clocks drop during
    # the synchronised measurements above
    t_ag = time.perf_counter()
    n_ag = 0
    while n_ag < 3 or (time.perf_counter() - t_ag) * 1e3 < args.min_warmup_ms:
        autograd_step()
        n_ag += 1
        if n_ag % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for _ in range(args.steps):
        autograd_step()
    eb.record(stream)
    torch.cuda.synchronize()
    autograd_ms = ea.elapsed_time(eb) / args.steps
    del ql, kl, vl


    # Every other workload, timed the same way (after the main one, so that
    # the clocks are warm); no CPU baseline for these.
    configs = {}
    if not args.no_configs:
        for name in DETAIL_CONFIGS:
            if name == workload:
                continue
            configs[name] = measure_config(bsr, W, torch, name, max(5, min(args.steps, 20)), 150.0, dev)
            torch.cuda.empty_cache()

    # The measured MFMA-loop peak of this device (products on random register
    # operands, two waves per SIMD on every CU): the ceiling the clocks and
    # power limit allow, next to the spec peak. ~0.3 s of probes first, so
    # that it is taken in the same clock state as the steps.
    sink = torch.zeros(1, device=dev)
    probe_iters = 4096
    t_probe = time.perf_counter()
    while time.perf_counter() - t_probe < 0.3:
        bsr.mfma_probe(tdt, probe_iters, sink)
        torch.cuda.synchronize()
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record(stream)
    probe_flops = sum(bsr.mfma_probe(tdt, probe_iters, sink) for _ in range(20))
    pe1.record(stream)
    torch.cuda.synchronize()
    measured_peak = probe_flops / (pe0.elapsed_time(pe1) * 1e-3) / 1e12
    if roofline is not None and roofline.get("bound") == "mfma":
        roofline["measured_peak"] = round(measured_peak, 1)
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / measured_peak, 4)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        # The same inputs the GPU ran on (same generator, same shape); whole
        # (batch, head) slices, forward then backward, until the time budget.
        qc, kc, vc, doc = (t.reshape(BH, 1, S, D) for t in W.make_inputs(batch, heads, S, D, dtype, seed=0))
        hs, tc = 0, 0.0
        while hs < BH and tc < args.cpu_seconds:
            q1, k1, v1, do1 = (t[hs:hs + 1].double().numpy() for t in (qc, kc, vc, doc))
            t0 = time.perf_counter()
            oracle.fwd(q1, k1, v1, rp, ci)
            oracle.bwd(q1, k1, v1, do1, rp, ci)
            tc += time.perf_counter() - t0
            hs += 1
        cpu_flops = 14.0 * hs * nnzb * B128 * B128 * D
        cpu = {"value": round(cpu_flops / tc / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.threads(),
               "kind": "oracle",
               "sample": f"{hs} of {BH} (batch, head) slices of the same workload and inputs, forward + "
                         f"backward in fp64, {tc:.1f} s"}

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": workload, "mask": kind, "density_target": dens, "batch": batch, "heads": heads,
                   "seq_len": S, "head_dim": D, "block": B128, "nnzb_per_head": nnzb,
                   "block_density": round(nnzb / (nb * nb), 4), "split_threshold": s.info["split_threshold"],
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "measured_mfma_peak": round(measured_peak, 1),
        "pct_of_measured_mfma_peak": round(100.0 * value / measured_peak, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {
            "fwd_ms_median": round(statistics.median(fw), 4), "bwd_ms_median": round(statistics.median(bw), 4),
            "fwd_two_pass_ms_median": round(statistics.median(t2), 4),
            "bwd_ds": bwd_ds,
            "wall_s_timed": round(wall, 4), "structure_build_ms": round(t_build * 1e3, 3),
            "warmup_steps_run": n_warm, "autograd_ms_per_step": round(autograd_ms, 4), "spmm": spmm,
            "flops_per_step": flops_step, "kernels": kernels, "configs": configs,
            "context_trn2": "pages: ~4 ms fwd+bwd, 1 head, fp32, seq 8192, global mask (trn2.3xlarge)",
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
