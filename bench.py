#!/usr/bin/env python3
"""Throughput of the SSD layer forward on one MI355X.

Default workload: the 2.7B-layer shape (batch 4, L 4096, H 80, P 64, N 128,
one B/C group, chunk 256, bfloat16 inputs, float32 accumulation), seeded
synthetic inputs already resident in device memory.  A step is one full
``ssd_forward`` call (all kernels of the chunked algorithm).  Before each
timed step a 512 MiB buffer is overwritten so the 256 MB Infinity Cache does
not hold the inputs; HIP events on the launch stream bracket the forward call
alone.  Prints one JSON line.

Other modes: ``--workload backward`` (the gradient of the same layer at the
same shape: ``ssd_backward`` with dy drawn N(0, 1), D present, no initial or
final state, as in training), ``--workload decode`` (512 single-token steps
on a [256, 80, 64, 128] float32 state), ``--workload gated_norm`` (the
normalisation after the gate on the forward's output), ``--workload scan``
(the selective Mamba-1 scan on the 2.8B-layer shape: batch 4, L 4096, 5120
channels, N 16) and ``--workload copy`` (a plain device-to-device copy used
to calibrate hardware byte counters).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F32_PEAK_TFLOPS = 157.3
METRIC = "SSD fwd tokens/s at H=80,P=64,N=128,L=4096; % of MFMA/HBM roofline"
# forward workloads: --shape -> index into ssd_inputs.WORKLOADS, description
FORWARD_SHAPES = {
    "tiny": (0, "tiny SSD forward (float32)"),
    "370M-layer": (1, "370M-layer-shaped SSD forward"),
    "2.7B-layer": (2, "2.7B-layer-shaped SSD forward"),
    "long-fp32": (3, "long-sequence SSD forward with carried state"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["forward", "backward", "decode", "gated_norm", "scan", "copy"],
                    default="forward")
    ap.add_argument("--shape", choices=list(FORWARD_SHAPES), default="2.7B-layer",
                    help="forward: the workload (tiny: batch 1, L 256, H 4, P 16, N 16, float32; "
                         "370M-layer: batch 8, L 2048, H 32; 2.7B-layer: batch 4, L 4096, H 80; "
                         "long-fp32: batch 1, L 65536, H 32, float32, carried state)")
    ap.add_argument("--ngroups", type=int, default=0,
                    help="forward: B/C groups (0 = the workload's own, 1)")
    ap.add_argument("--path", choices=["fused", "staged"], default="fused")
    ap.add_argument("--options", choices=["none", "mamba2", "zoh"], default="none",
                    help="forward step-size options: mamba2 = dt_bias + softplus + Euler input "
                         "scale; zoh = zero-order-hold input scale (ssd_forward_ex)")
    ap.add_argument("--scan-algo", choices=["auto", "segments", "rows"], default="auto",
                    help="scan: the arrangement (ssd_scan_dims.algo)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    return ap.parse_args()


def forward_bytes(w) -> int:
    """Compulsory bytes of one forward: read x, dt, B, C, A, D (+ init) once,
    write y (+ final state) once."""
    e = 2 if w.dtype == "bf16" else 4
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    n = 2 * b * L * H * P * e + b * L * H * e + 2 * b * L * G * N * e + 2 * H * 4
    n += b * H * P * N * 4 * (2 if w.init_mode == "normal" else 1)
    return n


def chunk_scan_flops(w) -> int:
    """Algorithmic flops of the output step: the masked intra-chunk product
    over lower-triangular pairs and the state term C h."""
    b, L, H, P, N, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk
    tri = sum(min(Q, L - c * Q) * (min(Q, L - c * Q) + 1) // 2 for c in range((L + Q - 1) // Q))
    return b * H * 2 * (P * tri + L * N * P)


def forward_flops(w) -> int:
    """Algorithmic flops of the chunked algorithm (lower-triangular blocks)."""
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    tri = 0
    for c in range((L + Q - 1) // Q):
        q = min(Q, L - c * Q)
        tri += q * (q + 1) // 2
    nc = (L + Q - 1) // Q
    per_bh = 2 * (P * tri + L * N * P + L * N * P) + 2 * nc * N * P
    per_bg = 2 * N * tri
    return b * H * per_bh + b * G * per_bg


def kernel_bytes(w) -> dict:
    """Algorithmic bytes of each kernel of the staged sequence, per launch
    (what its own inputs and outputs must move at least once)."""
    e = 2 if w.dtype == "bf16" else 4
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = (L + Q - 1) // Q
    T16 = Q // 16
    cs = b * H * nc * Q * 4
    cb = b * nc * G * (T16 * (T16 + 1) // 2) * 256 * e
    S = b * nc * H * P * N * 4
    x = b * L * H * P * e
    BC = b * L * G * N * e
    st = b * H * P * N * 4
    init_b = st if w.init_mode == "normal" else 0
    Bt = b * nc * G * N * ((Q + 31) // 32 * 32) * e
    return {
        # single-pass arrangement: the compulsory bytes of the forward split
        # between its two launches (their sum is forward_bytes); the
        # per-chunk fragments and decay records the preparation writes and
        # the walk reads are intermediates and count for neither
        "forward_prep": b * L * H * e + 2 * BC + H * 4,
        "forward_main": 2 * x + H * 4 + init_b + st,
        "chunk_cumsum": b * L * H * e + H * 4 + cs,
        "chunk_cb": 2 * BC + cb,
        "chunk_state": x + BC + cs + S,
        "state_passing": 2 * S + b * H * nc * 4 + st * (2 if w.init_mode == "normal" else 1),
        "chunk_scan": x + BC + cb + cs + S + H * 4 + x,
    }


def kernel_flops(w) -> dict:
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    tri = sum(min(Q, L - c * Q) * (min(Q, L - c * Q) + 1) // 2 for c in range((L + Q - 1) // Q))
    return {"chunk_cb": 2 * N * tri * b * G, "chunk_state": 2 * L * N * P * b * H,
            "chunk_scan": (2 * P * tri + 2 * L * N * P) * b * H}


def backward_bytes(w) -> int:
    """Compulsory bytes of one gradient call without initial or final state:
    read x, dy, dt, B, C, A, D once, write dx, ddt, dB, dC, dA, dD once."""
    e = 2 if w.dtype == "bf16" else 4
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    return 3 * b * L * H * P * e + 2 * b * L * H * e + 4 * b * L * G * N * e + 4 * H * 4


def backward_flops(w) -> int:
    """Matrix flops of the gradient as computed here (lower-triangular blocks):
    per (b, h) the transposed intra-chunk product and the state term of dx,
    the masked dy x^T of dCB, the state terms of dC and dB, the forward and
    reverse chunk states, and the forward output again for the decay
    gradients; per (b, g) C B^T and the two dCB products."""
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    tri = sum(min(Q, L - c * Q) * (min(Q, L - c * Q) + 1) // 2 for c in range((L + Q - 1) // Q))
    per_bh = 3 * 2 * P * tri + 6 * 2 * L * N * P
    per_bg = 3 * 2 * N * tri
    return b * H * per_bh + b * G * per_bg


def backward_kernel_bytes(w) -> dict:
    """Algorithmic bytes of each launch of the gradient (its own inputs and
    outputs once; workspace intermediates count where a kernel reads or
    writes them)."""
    e = 2 if w.dtype == "bf16" else 4
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = (L + Q - 1) // Q
    T16 = Q // 16
    cs = b * H * nc * Q * 4
    cb = b * nc * G * (T16 * (T16 + 1) // 2) * 256 * e
    S = b * nc * H * P * N * 4
    x = b * L * H * P * e
    BC = b * L * G * N * e
    dtb = b * L * H * e
    dcb = b * nc * G * (T16 * (T16 + 1) // 2) * 256 * 4
    gst = b * L * G * N * 4
    part = b * nc * H * 8
    frags = w.dtype == "bf16" and Q <= 256
    if frags:
        # bfloat16: the prep writes C B^T as the 16 x 16 tiles the chunk backward reads
        # (row tiles 0 .. 2 (I / 2) + 1 of row tile I, and the transposed column blocks),
        # C and B in fragment order and the float32 diagonal; the chunk backward reads them
        ntile = sum(min(2 * (I // 2) + 2, T16) for I in range(T16))
        cb = b * nc * G * ntile * 256 * e
        rows = 2 * BC
        diag = b * nc * G * Q * 4
    else:
        rows, diag = 0, 0
    return {
        "chunk_cumsum": dtb + H * 4 + cs,
        "chunk_cumsum64": dtb + H * 4 + 2 * cs if w.dtype == "f32" else 0,
        "chunk_cb": 2 * BC + 2 * cb + rows + diag,
        "chunk_state": x + BC + cs + S,
        "state_passing": 2 * S + b * H * nc * 4,
        "chunk_state_rev": x + BC + cs + S,
        "state_passing_rev": 2 * S + b * H * nc * 4,
        "chunk_bwd": 3 * x + 2 * dtb + 2 * BC + 2 * cb + diag + cs + 2 * S + 2 * H * 4 + part,
        "group_bwd": 2 * x + cs + 2 * S + 2 * dcb + 2 * gst,
        "group_combine": 2 * BC + 2 * dcb + 2 * gst + 2 * BC,
        "head_reduce": part + 2 * H * 4,
    }


def run_backward_bench(args):
    import ctypes

    import torch

    import selective_state_space_04_amd as ssd
    import ssd_inputs as si

    w = si.WORKLOADS[2]
    dev = torch.device("cuda:0")
    inp = si.make_forward_inputs(w)
    grads = si.make_output_grads(w, with_final=False)
    g = lambda t: None if t is None else t.to(dev)
    x, dt, A, B, C, D, init = (g(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init"))
    dy = g(grads["dy"])
    dims = ssd.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk,
                         ssd.BF16 if w.dtype == "bf16" else ssd.F32)
    ws = torch.empty(max(ssd.backward_workspace_bytes(dims), 1), dtype=torch.uint8, device=dev)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "dB": torch.empty_like(B),
           "dC": torch.empty_like(C), "dA": torch.empty_like(A), "dD": torch.empty_like(D)}
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def step():
        ssd.backward(x, dt, A, B, C, dy, D=D, init_state=init, chunk=w.chunk, out=out, workspace=ws,
                     want_dinit=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(k & 0xFF)
        starts[k].record()
        step()
        ends[k].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b_) for a, b_ in zip(starts, ends)]
    ms_per_step = statistics.mean(ms)
    tokens = w.batch * w.seqlen
    t_hbm = backward_bytes(w) / (HBM_PEAK_GBS * 1e3)
    t_mfma = backward_flops(w) / (BF16_PEAK_TFLOPS * 1e6)
    t_roof_us = max(t_hbm, t_mfma)
    result = {
        "metric": "SSD bwd tokens/s at H=80,P=64,N=128,L=4096; % of MFMA/HBM roofline",
        "value": tokens / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded; distributions of the workload)",
        "config": {"workload": "2.7B-layer-shaped SSD backward", "batch": w.batch, "seqlen": w.seqlen,
                   "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk": w.chunk, "inputs": "bf16", "accumulate": "fp32",
                   "grads": "dx, ddt, dA, dB, dC, dD (no initial or final state)",
                   "mall_flushed": flush is not None},
        "backward_roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma", "t_roof_us": t_roof_us,
                              "t_hbm_us": t_hbm, "t_mfma_us": t_mfma,
                              "frac": t_roof_us / (ms_per_step * 1e3), "alg_bytes": backward_bytes(w),
                              "alg_flops": backward_flops(w)},
        "ms_min": min(ms), "ms_median": statistics.median(ms), "wall_s": wall,
    }
    if not args.no_kernel_timing:
        # per-launch durations: hipEvents recorded by the library between its launches
        hip = ctypes.CDLL("libamdhip64.so")
        dp = ctypes.byref(dims)
        n = ssd.lib.ssd_backward_launch_count(dp)
        names = [ssd.lib.ssd_backward_launch_name(dp, i).decode() for i in range(n)]
        evs = (ctypes.c_void_p * (n + 1))()
        for i in range(n + 1):
            if hip.hipEventCreate(ctypes.byref(evs, i * ctypes.sizeof(ctypes.c_void_p))) != 0:
                raise RuntimeError("hipEventCreate failed")
        p = ssd._p
        times = {nm: [] for nm in names}
        reps = max(args.steps, 5)
        for rep in range(reps + 2):
            if flush is not None:
                flush.fill_(rep & 0xFF)
            st = ssd.lib.ssd_backward_timed(dp, p(x), p(dt), p(A), p(B), p(C), p(D), p(init), p(dy), None,
                                            p(out["dx"]), p(out["ddt"]), p(out["dA"]), p(out["dB"]),
                                            p(out["dC"]), p(out["dD"]), None, p(ws), ws.numel(), ssd._stream(),
                                            evs, n + 1)
            if st != 0:
                raise RuntimeError(f"ssd_backward_timed: status {st}")
            torch.cuda.synchronize()
            if rep >= 2:
                for i, nm in enumerate(names):
                    f = ctypes.c_float()
                    hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(evs[i]), ctypes.c_void_p(evs[i + 1]))
                    times[nm].append(f.value * 1e3)
        for i in range(n + 1):
            hip.hipEventDestroy(ctypes.c_void_p(evs[i]))
        avg = {nm: statistics.mean(v) for nm, v in times.items()}
        dom = max(avg, key=avg.get)
        kb = backward_kernel_bytes(w)[dom]
        achieved = kb / (avg[dom] * 1e-6) / 1e9
        result["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                              "traffic": measured_traffic("bwd_" + dom), "alg_bytes_per_launch": kb,
                              "avg_launch_us": avg[dom]}
        result["kernels_us"] = avg
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_backward(w, inp, grads)
    return result


def cpu_baseline_backward(w, inp, grads):
    """The float64 adjoint oracle on a bounded sample: the first two batch rows
    at full length and all heads (half the workload's (batch, head)
    sequences; every sequence costs the same, so tokens/s is that of the
    sample)."""
    import oracle

    nb = 2
    f = oracle._f64
    t0 = time.perf_counter()
    oracle.backward(f(inp["x"][:nb]), f(inp["dt"][:nb]), f(inp["A"]), f(inp["B"][:nb]), f(inp["C"][:nb]),
                    f(inp["D"]), None, f(grads["dy"][:nb]), None)
    t = time.perf_counter() - t0
    return {"value": nb * w.seqlen / t, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"batch rows 0-{nb - 1} of {w.batch} at full length, all {w.nheads} heads, float64 "
            f"reverse-mode recurrence, {t:.2f} s"}


def run_forward_bench(args):
    import torch

    import selective_state_space_04_amd as ssd
    import ssd_inputs as si

    long32 = args.shape == "long-fp32"
    widx, wdesc = FORWARD_SHAPES[args.shape]
    w = si.WORKLOADS[widx]
    if args.ngroups:
        w = w.with_(ngroups=args.ngroups)
    dev = torch.device("cuda:0")
    inp = si.make_forward_inputs(w)
    g = lambda t: None if t is None else t.to(dev)
    x, dt, A, B, C, D, init = (g(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init"))
    dims = ssd.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk,
                         ssd.BF16 if w.dtype == "bf16" else ssd.F32)
    ws = torch.empty(max(ssd.workspace_bytes(dims), 1), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    staged = args.path == "staged"
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    okw = {}
    if args.options == "mamba2":
        # raw step = inverse softplus of the workload's dt minus the bias, so the
        # preprocessed step keeps the workload's magnitudes
        gen = torch.Generator().manual_seed(903)
        bias = (torch.randn(w.nheads, generator=gen) * 0.5).float()
        dt = (torch.log(torch.expm1(inp["dt"].float())) - bias).to(inp["dt"].dtype).to(dev)
        okw = dict(dt_bias=bias.to(dev), dt_softplus=True, input_scale="euler")
    elif args.options == "zoh":
        okw = dict(input_scale="zoh")

    def step():
        ssd.forward(x, dt, A, B, C, D, init, chunk=w.chunk, staged=staged, y=y, final_state=fin,
                    workspace=ws, **okw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(k & 0xFF)
        starts[k].record()
        step()
        ends[k].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = statistics.mean(ms)
    tokens = w.batch * w.seqlen
    value = tokens / (ms_per_step * 1e-3)
    t_hbm = forward_bytes(w) / (HBM_PEAK_GBS * 1e3)
    t_mfma = forward_flops(w) / ((F32_PEAK_TFLOPS if long32 else BF16_PEAK_TFLOPS) * 1e6)
    t_roof_us = max(t_hbm, t_mfma)

    metric = METRIC if args.shape == "2.7B-layer" else (
        f"SSD fwd tokens/s at H={w.nheads},P={w.headdim},N={w.dstate},L={w.seqlen} {w.dtype}; "
        "% of MFMA/HBM roofline")
    result = {
        "metric": metric,
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic (seeded; distributions of the workload)",
        "config": {"workload": wdesc, "batch": w.batch, "seqlen": w.seqlen,
                   "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk": w.chunk, "inputs": w.dtype, "accumulate": "fp32", "path": args.path,
                   "dt_options": args.options, "mall_flushed": flush is not None, "seed": w.seed},
        "forward_roofline": {"bound": "mfma" if t_mfma > t_hbm else "hbm", "t_roof_us": t_roof_us,
                             "frac": t_roof_us / (ms_per_step * 1e3),
                             "alg_bytes": forward_bytes(w), "alg_flops": forward_flops(w)},
        "ms_min": min(ms), "ms_median": statistics.median(ms), "wall_s": wall,
    }

    if not args.no_kernel_timing and args.options == "none":
        result["roofline"], result["kernels_us"] = kernel_roofline(ssd, w, x, dt, A, B, C, D, init, ws,
                                                                  y, fin, flush, args)
    result["env"] = environment(torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"], ref = cpu_baseline(w, inp)
        if args.options == "none":
            result["parity"] = parity(w, y, fin, ref)
    return result


def environment(torch) -> dict:
    """The machine the line was measured on: GPU, ROCm/HIP and host CPU."""
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip": getattr(torch.version, "hip", None),
            "torch": torch.__version__, "cpu_model": cpu, "host_cpus": os.cpu_count()}


def parity(w, y, fin, ref) -> dict:
    """Relative L2 error of the timed forward's y and final state against the
    float64 oracle on the same inputs: the worst (batch, head) slice, the
    bound the workload's dtype sets."""
    import numpy as np

    y_ref, f_ref = ref
    yg = y.detach().float().cpu().double().numpy()
    fg = fin.detach().cpu().double().numpy()

    def worst(a, r, kind):
        if kind == "y":
            b, L, H, P = r.shape
            a = a.transpose(0, 2, 1, 3).reshape(b * H, -1)
            r = r.transpose(0, 2, 1, 3).reshape(b * H, -1)
        else:
            a = a.reshape(-1, a.shape[-2] * a.shape[-1])
            r = r.reshape(-1, r.shape[-2] * r.shape[-1])
        return float(np.max(np.linalg.norm(a - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)))

    tol = 2e-2 if w.dtype == "bf16" else 1e-5
    ey, ef = worst(yg, y_ref, "y"), worst(fg, f_ref, "state")
    return {"y_rel_l2_worst_slice": ey, "final_rel_l2_worst_slice": ef, "tol": tol,
            "ok": bool(ey <= tol and ef <= tol)}


def kernel_roofline(ssd, w, x, dt, A, B, C, D, init, ws, y, fin, flush, args):
    """Average duration of each kernel launch of the forward, measured with
    HIP events on the launch stream around the same launches the forward
    makes (through the per-launch entry points), and the roofline of the
    slowest one."""
    import ctypes

    import torch

    Q, L = w.chunk, w.seqlen
    nc = (L + Q - 1) // Q
    e = 2 if w.dtype == "bf16" else 4
    stream = ssd._stream()
    dims = ssd.make_dims(w.batch, L, w.nheads, w.headdim, w.dstate, w.ngroups, Q,
                         ssd.BF16 if w.dtype == "bf16" else ssd.F32)
    dp = ctypes.byref(dims)
    p = ssd._p
    nbytes = ws.numel()
    single = args.path == "fused" and ssd.lib.ssd_forward_is_single_pass(dp)
    if single:
        seq = [
            ("forward_prep", lambda: ssd.lib.ssd_forward_prep(dp, p(dt), p(A), p(B), p(C), p(ws), nbytes, stream)),
            ("forward_main", lambda: ssd.lib.ssd_forward_main(dp, p(x), p(dt), p(A), p(B), p(C), p(D), p(init),
                                                             p(y), p(fin), p(ws), nbytes, stream)),
        ]
    else:
        # carve the workspace exactly as the staged arrangement does
        al = lambda v: (v + 255) // 256 * 256
        cs_b = w.batch * w.nheads * nc * Q * 4
        cb_b = w.batch * nc * w.ngroups * Q * Q * e
        S_b = w.batch * nc * w.nheads * w.headdim * w.dstate * 4
        cs = ws[:cs_b]
        cb = ws[al(cs_b): al(cs_b) + cb_b]
        S = ws[al(al(cs_b) + cb_b):]
        seq = [
            ("chunk_cumsum", lambda: ssd.lib.ssd_chunk_cumsum(dp, p(dt), p(A), p(cs), stream)),
            ("chunk_cb", lambda: ssd.lib.ssd_chunk_cb(dp, p(B), p(C), p(cb), stream)),
            ("chunk_state", lambda: ssd.lib.ssd_chunk_state(dp, p(x), p(B), p(cs), p(S), stream)),
            ("state_passing", lambda: ssd.lib.ssd_state_passing(dp, p(S), p(cs), p(init), p(fin), stream)),
            ("chunk_scan", lambda: ssd.lib.ssd_chunk_scan(dp, p(x), p(C), p(cb), p(cs), p(S), p(D), p(y),
                                                          stream)),
        ]
    reps = max(args.steps, 5)
    times = {n: [] for n, _ in seq}
    for rep in range(reps + 2):
        if flush is not None:
            flush.fill_(rep & 0xFF)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)]
        evs[0].record()
        for i, (n, fn) in enumerate(seq):
            st = fn()
            if st != 0:
                raise RuntimeError(f"{n}: status {st}")
            evs[i + 1].record()
        torch.cuda.synchronize()
        if rep >= 2:
            for i, (n, _) in enumerate(seq):
                times[n].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)
    avg = {n: statistics.mean(v) for n, v in times.items()}
    dom = max(avg, key=avg.get)
    if w.dtype == "f32" and dom == "chunk_scan":
        # float32: the output kernel is bound by the fp32 MFMA rate
        fl = chunk_scan_flops(w)
        achieved = fl / (avg[dom] * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / F32_PEAK_TFLOPS, "traffic": None,
                "alg_flops_per_launch": fl, "avg_launch_us": avg[dom]}
        return roof, avg
    kb = kernel_bytes(w)[dom]
    achieved = kb / (avg[dom] * 1e-6) / 1e9
    tag = f"{args.shape}/G{w.ngroups}/{args.options}"
    roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(dom, tag), "alg_bytes_per_launch": kb,
            "avg_launch_us": avg[dom]}
    return roof, avg


def measured_traffic(key: str, tag: str = ""):
    """HBM bytes per launch from the committed rocprofv3 counters
    (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE, scaled by the copy
    calibration) for this kernel on this workload (`tag`: shape, groups and
    options, "" for the kernels with one workload), or None when no entry
    matches or the kernel source has changed since they were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{key}@{tag}" if tag else key)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return rec["bytes"]


def cpu_baseline(w, inp):
    """The float64 oracle on the same inputs, timed on the host cores; also
    returns its (y, final_state) for the parity entry."""
    import oracle

    args = [inp[k] for k in ("x", "dt", "A", "B", "C", "D", "init")]
    f = [oracle._f64(a) for a in args]
    t0 = time.perf_counter()
    ref = oracle.forward(*f)
    t = time.perf_counter() - t0
    return {"value": w.batch * w.seqlen / t, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"the full workload ({w.batch}x{w.seqlen} tokens, {w.nheads} heads), "
            f"float64 sequential recurrence, {t:.2f} s"}, ref


def run_gated_norm_bench(args):
    """The normalisation after the gate on the 2.7B-layer output
    ([4, 4096, 80, 64] bf16): reads y and z, writes out, once each."""
    import torch

    import selective_state_space_04_amd as ssd

    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(1005)
    b, L, H, P = 4, 4096, 80, 64
    y = torch.randn((b, L, H, P), generator=gen).to(torch.bfloat16).to(dev)
    z = torch.randn((b, L, H, P), generator=gen).to(torch.bfloat16).to(dev)
    wt = torch.randn(H * P, generator=gen).to(dev)
    out = torch.empty_like(y)
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        ssd.gated_rmsnorm(y, z, wt, out=out)
    torch.cuda.synchronize()
    ms = []
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(k & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ssd.gated_rmsnorm(y, z, wt, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    avg = statistics.mean(ms)
    nbytes = 3 * b * L * H * P * 2 + H * P * 4
    achieved = nbytes / (avg * 1e-3) / 1e9
    res = {"metric": "gated RMSNorm tokens/s, [4,4096,80,64] bf16", "value": b * L / (avg * 1e-3),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": avg,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": "gated RMSNorm after the SSD output", "batch": b,
                                           "seqlen": L, "nheads": H, "headdim": P, "norm_groups": 1,
                                           "mall_flushed": flush is not None},
           "roofline": {"kernel": "gated_rmsnorm", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("gated_norm"),
                        "alg_bytes_per_launch": nbytes, "avg_launch_us": avg * 1e3}}
    if not args.no_cpu_baseline:
        import oracle
        rows = 2048
        yc = y.reshape(-1, H, P)[:rows].cpu()
        zc = z.reshape(-1, H, P)[:rows].cpu()
        t0 = time.perf_counter()
        oracle.gated_rmsnorm(yc, zc, wt.cpu())
        t = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": rows / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{rows} of {b * L} token rows, numpy float64, {t:.2f} s"}
    return res

# Vector-ALU issue rate of the chip: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz,
# one full-rate fp32 operation per lane per clock (packed fp32 is not used),
# the exponential (v_exp_f32) at half that rate (measured on gfx950: 19.0 T
# exp/s against 38.1 T fma/s on the whole chip).
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
EXP_RATE = 0.5
SCAN_FLOPS_PER_UPDATE = 7      # dt*A, exp, (dt x)*B, fma into h, fma C.h into y (fma = 2)
SCAN_SLOTS_PER_UPDATE = 4 + 1 / EXP_RATE  # issue slots of those five operations
SCAN_PEAK_TFLOPS = SCAN_FLOPS_PER_UPDATE * VALU_LANE_OPS / SCAN_SLOTS_PER_UPDATE / 1e12


def scan_inputs(b, L, Dch, N, seed=4077):
    """Seeded inputs of the Mamba-1 layer shape: x, z ~ N(0, 1); B, C ~
    N(0, 1)/sqrt(N) (one group); A = -U(1, 16) per (channel, state); the
    step log-uniform in [1e-3, 1e-1], given raw (inverse softplus minus the
    bias, bias ~ N(0, 0.25)); D ~ N(0, 1)."""
    import math

    import torch

    g = torch.Generator().manual_seed(seed)
    x = torch.randn((b, L, Dch), generator=g)
    Bm = torch.randn((b, L, 1, N), generator=g) / math.sqrt(N)
    Cm = torch.randn((b, L, 1, N), generator=g) / math.sqrt(N)
    A = -(torch.rand((Dch, N), generator=g) * 15 + 1)
    step = torch.exp(torch.rand((b, L, Dch), generator=g) * (math.log(1e-1) - math.log(1e-3)) + math.log(1e-3))
    bias = torch.randn(Dch, generator=g) * 0.5
    delta = torch.log(torch.expm1(step)) - bias
    D = torch.randn(Dch, generator=g)
    z = torch.randn((b, L, Dch), generator=g)
    bf = torch.bfloat16
    return dict(x=x.to(bf), delta=delta.to(bf), A=A, B=Bm.to(bf), C=Cm.to(bf), D=D, z=z.to(bf), delta_bias=bias)


def run_scan_bench(args):
    """The selective scan on the Mamba-2.8B layer shape (batch 4, L 4096,
    5120 channels, N 16, bf16 inputs, softplus step with bias, D and the
    SiLU gate, no initial state, final state written)."""
    import ctypes

    import torch

    import selective_state_space_04_amd as ssd

    b, L, Dch, N = 4, 4096, 5120, 16
    dev = torch.device("cuda:0")
    host = scan_inputs(b, L, Dch, N)
    c = {k: v.to(dev) for k, v in host.items()}
    y = torch.empty_like(c["x"])
    fin = torch.empty((b, Dch, N), dtype=torch.float32, device=dev)
    dims = ssd.ScanDims(b, L, Dch, N, 1, ssd.BF16, ssd.SCAN_ALGOS[args.scan_algo])
    dp = ctypes.byref(dims)
    ws = torch.empty(max(int(ssd.lib.ssd_selective_scan_workspace_bytes(dp)), 1), dtype=torch.uint8, device=dev)
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    p = ssd._p
    args_abi = lambda: (dp, p(c["x"]), p(c["delta"]), p(c["A"]), p(c["B"]), p(c["C"]), p(c["D"]), p(c["z"]),
                        p(c["delta_bias"]), 1, None, p(y), p(fin), p(ws), ws.numel(), ssd._stream())

    def step():
        st = ssd.lib.ssd_selective_scan(*args_abi())
        if st != 0:
            raise RuntimeError(f"ssd_selective_scan: status {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(k & 0xFF)
        starts[k].record()
        step()
        ends[k].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(e) for a, e in zip(starts, ends)]
    ms_per_step = statistics.mean(ms)
    updates = b * L * Dch * N
    alg_bytes = 4 * b * L * Dch * 2 + 2 * b * L * N * 2 + Dch * N * 4 + 2 * Dch * 4 + b * Dch * N * 4
    t_alu = updates * SCAN_SLOTS_PER_UPDATE / VALU_LANE_OPS * 1e6
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e3)
    res = {
        "metric": "selective scan tokens/s at D=5120,N=16,L=4096; % of ALU roofline", "value": b * L /
        (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; distributions of the layer)",
        "config": {"workload": "Mamba-2.8B-layer-shaped selective scan", "batch": b, "seqlen": L,
                   "channels": Dch, "dstate": N, "ngroups": 1, "inputs": "bf16", "accumulate": "fp32",
                   "step": "softplus(delta + bias)", "D": True, "gate": True, "mall_flushed": flush is not None},
        "scan_roofline": {"bound": "alu" if t_alu >= t_hbm else "hbm", "t_alu_us": t_alu, "t_hbm_us": t_hbm,
                          "frac": max(t_alu, t_hbm) / (ms_per_step * 1e3), "updates": updates,
                          "alg_bytes": alg_bytes},
        "ms_min": min(ms), "ms_median": statistics.median(ms), "wall_s": wall,
    }
    if not args.no_kernel_timing:
        hip = ctypes.CDLL("libamdhip64.so")
        algo = ssd.lib.ssd_selective_scan_algo(dp)
        names = ["scan_seg_state", "scan_pass", "scan_seg_out"] if algo == 1 else ["scan_bc_transpose", "scan_rows"]
        res["config"]["algo"] = "segments" if algo == 1 else "rows"
        nev = len(names) + 1
        evs = (ctypes.c_void_p * nev)()
        for i in range(nev):
            if hip.hipEventCreate(ctypes.byref(evs, i * ctypes.sizeof(ctypes.c_void_p))) != 0:
                raise RuntimeError("hipEventCreate failed")
        times = {nm: [] for nm in names}
        for rep in range(max(args.steps, 5) + 2):
            if flush is not None:
                flush.fill_(rep & 0xFF)
            st = ssd.lib.ssd_selective_scan_timed(*args_abi(), evs, nev)
            if st != 0:
                raise RuntimeError(f"ssd_selective_scan_timed: status {st}")
            torch.cuda.synchronize()
            if rep >= 2:
                for i, nm in enumerate(names):
                    f = ctypes.c_float()
                    hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(evs[i]), ctypes.c_void_p(evs[i + 1]))
                    times[nm].append(f.value * 1e3)
        for i in range(nev):
            hip.hipEventDestroy(ctypes.c_void_p(evs[i]))
        avg = {nm: statistics.mean(v) for nm, v in times.items()}
        # the dominant kernel runs every update once (rows: the whole scan;
        # segments: the output pass, which rescans from the entering states)
        dom = names[-1]
        us = avg[dom]
        achieved = updates * SCAN_FLOPS_PER_UPDATE / (us * 1e-6) / 1e12
        res["roofline"] = {"kernel": dom, "bound": "alu", "achieved": achieved,
                           "peak": SCAN_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / SCAN_PEAK_TFLOPS,
                           "traffic": measured_traffic(dom),
                           "alg_flops_per_launch": updates * SCAN_FLOPS_PER_UPDATE, "avg_launch_us": us}
        res["kernels_us"] = avg
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        oracle.selective_scan(host["x"], host["delta"], host["A"], host["B"], host["C"], host["D"], host["z"],
                              host["delta_bias"], True)
        t = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": b * L / t, "unit": "tokens/s", "cores": oracle.num_threads(),
                               "kind": "oracle", "sample": f"the full workload ({b}x{L} tokens, {Dch} channels), "
                               f"float64 sequential recurrence, {t:.2f} s"}
    return res



def run_decode_bench(args):
    import torch

    import selective_state_space_04_amd as ssd
    import ssd_inputs as si

    w = si.WORKLOADS[4]
    dev = torch.device("cuda:0")
    par = si.make_decode_params(w)
    state = par["state"].to(dev)
    A, D = par["A"].to(dev), par["D"].to(dev)
    nsteps = w.steps
    steps = [si.make_decode_step_inputs(w, s) for s in range(nsteps)]
    xs = torch.stack([s["x"] for s in steps]).to(dev)
    dts = torch.stack([s["dt"] for s in steps]).to(dev)
    Bs = torch.stack([s["B"] for s in steps]).to(dev)
    Cs = torch.stack([s["C"] for s in steps]).to(dev)
    ys = torch.empty_like(xs)
    for s in range(min(args.warmup, nsteps)):
        ssd.decode_step(state, xs[s], dts[s], A, Bs[s], Cs[s], D, y=ys[s])
    state.copy_(par["state"].to(dev))
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for s in range(nsteps):
        ssd.decode_step(state, xs[s], dts[s], A, Bs[s], Cs[s], D, y=ys[s])
        ev[s + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[s].elapsed_time(ev[s + 1]) * 1e3 for s in range(nsteps)]
    total_ms = ev[0].elapsed_time(ev[-1])
    bytes_step = 2 * w.batch * w.nheads * w.headdim * w.dstate * 4 + 2 * w.batch * w.nheads * w.headdim * 2 \
        + w.batch * w.nheads * 2 + 2 * w.batch * w.ngroups * w.dstate * 2 + 2 * w.nheads * 4
    avg_us = statistics.mean(per)
    achieved = bytes_step / (avg_us * 1e-6) / 1e9
    return {"metric": "SSD decode tokens/s, state [256,80,64,128] fp32, 512 steps", "value": w.batch * nsteps /
            (total_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": nsteps, "warmup": args.warmup,
            "ms_per_step": total_ms / nsteps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic", "config": {"workload": "decode step", "batch": w.batch,
                                                              "nheads": w.nheads, "headdim": w.headdim,
                                                              "dstate": w.dstate, "steps": nsteps},
            "roofline": {"kernel": "decode", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("decode"),
                         "alg_bytes_per_launch": bytes_step, "avg_launch_us": avg_us},
            "wall_s": wall}


def run_copy(args):
    """Device-to-device copy of 1 GiB, repeated: reference for byte counters."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"metric": "device copy GB/s (1 GiB read + 1 GiB write)", "value": 2 * n / (ms * 1e-3) / 1e9,
            "unit": "GB/s", "ms_per_step": ms, "steps": args.steps, "bytes_read_per_copy": n}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(each (batch, head) sequence is independent, so multi-GPU runs would shard batch/heads "
              "with no communication -- not part of this build)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "forward":
        res = run_forward_bench(args)
    elif args.workload == "backward":
        res = run_backward_bench(args)
    elif args.workload == "gated_norm":
        res = run_gated_norm_bench(args)
    elif args.workload == "decode":
        res = run_decode_bench(args)
    elif args.workload == "scan":
        res = run_scan_bench(args)
    else:
        res = run_copy(args)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
