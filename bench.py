#!/usr/bin/env python3
"""Benchmark of the emulated FP4 linear layer on one MI355X.

One step = the whole hot path on the FFN up-projection shape
(X 16384x4096 bf16, W 14336x4096 bf16, dY 16384x14336 bf16), as a refresh
step of sample-and-hold tensor scaling, in training order:
  amax(X), then quantize X  ROW16 + COL16 RNE (fwd operand; wgrad operand
              along tokens), one pass
  amax(W), then quantize W  TILE16x16 RNE + transposed copy (fwd and dgrad
              operand)
  Y  = Xq Wq^T     (bf16 out)    fwd
  amax(dY)
  quantize dY ROW16 + COL16 SR  (dgrad operand; wgrad operand along tokens), one
              pass, one Philox word per element for both
  dX = dYq Wq      (bf16 out)    dgrad
  dW = dYq^T Xq    (fp32 out)    wgrad
Quantized operands use the K64 packing (--pack rows: row-major).
value = 3 * 2 M N K flops / step time (TFLOP/s); inputs are resident in HBM
before timing starts. Also measured in the same run: each kernel's average
duration inside the step (HIP events on the launch stream), the quantize-only workload
(8192x4096 bf16 ROW16 RNE, rotating over >256 MiB of inputs and outputs so
the Infinity Cache cannot serve it) in GB/s, the 8192-token linear layer
(forward: X 8192x4096, W 4096x4096; backward: dY 8192x4096 with SR, dgrad
and wgrad over 8192 tokens) launch by launch with each GEMM's fraction of
the dense MFMA peak and the SR quantize's fractions of the HBM and VALU
peaks, and the CPU oracle on a bounded sample. Prints one JSON line.
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

HBM_PEAK_GBS = 8000.0
MFMA16_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 MFMA, MI355X
# VALU issue peak in wave64 instructions per second: 256 CUs x 4 SIMDs at
# 2.4 GHz, one wave64 instruction per SIMD every 2 cycles (32 lanes per
# cycle: the fp32 vector peak of 157.3 TFLOP/s is 1024 SIMDs x 32 lanes x 2
# FLOP per FMA x 2.4 GHz). Several integer and conversion instructions
# (v_bitop3, v_mad_u64_u32, v_cvt_*, v_fract, v_ldexp, v_med3) issue at half
# that rate.
VALU_PEAK_WAVE_INSTR = 256 * 4 * 2.4e9 / 2
METRIC = "FP4-emulated linear TFLOP/s (fwd+dgrad+wgrad) and quantize GB/s, % of roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--profile-op", default=None,
                    help="profiling mode: run only this launch of the step (e.g. gemm_fwd, "
                         "quant_x_row16, quantize_only, copy) --reps times and exit")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--pack", choices=("k64", "rows"), default="k64",
                    help="memory packing of the step's quantized operands")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from fp4_block_scaled_fp4q_amd import api, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = inputs.make("ffn_up_step")
    M, N, K = wl.dims["M"], wl.dims["N"], wl.dims["K"]
    X = wl.tensors["X"].t.to(dev)
    W = wl.tensors["W"].t.to(dev)
    dY = wl.tensors["dY"].t.to(dev)
    host = wl
    log(args, f"inputs ready in {time.time() - t0:.1f}s: M={M} N={N} K={K}")

    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    amax = {k: torch.empty(1, **f32) for k in ("X", "W", "dY")}
    S = {k: torch.empty(1, **f32) for k in ("x", "w", "dy")}
    pack = api.PACK_K64 if args.pack == "k64" else api.PACK_ROWS

    def operand(rows, cols, tile, s):
        codes, scales = api.operand_buffers(rows, cols, tile, 16, pack, dev)
        return api.QTensor(codes, scales, s, rows, cols, api.TILE16x16 if tile else api.ROW16, 16, api.UE5M3,
                           pack)
    xq, xqt = operand(M, K, False, S["x"]), operand(K, M, False, S["x"])
    wq, wqt = operand(N, K, True, S["w"]), operand(K, N, True, S["w"])
    dyq, dyqt = operand(M, N, False, S["dy"]), operand(N, M, False, S["dy"])
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), **f32)
    T = 448.0
    seed = 0

    # every launch of one step, in the order of a training step (forward,
    # then the backward once dY exists), as (kernel family, callable)
    # each operand's amax is followed by its own quantization (which then
    # re-reads a tensor that the amax has just streamed through the cache)
    ops = [
        ("amax", lambda: api.fp4q_amax(X, amax["X"])),
        # X: ROW16 (fwd) and COL16 (wgrad) in one pass
        ("quant_x_row_col", lambda: api.fp4q_quantize_fmt(X, amax["X"], T, api.ROW16, 16, api.UE5M3, pack,
                                                          api.RNE, 0, 0, xq.codes, xq.scales, S["x"],
                                                          xqt.codes, xqt.scales)),
        ("amax", lambda: api.fp4q_amax(W, amax["W"])),
        ("quant_w_tile", lambda: api.fp4q_quantize_fmt(W, amax["W"], T, api.TILE16x16, 16, api.UE5M3, pack,
                                                       api.RNE, 0, 0, wq.codes, wq.scales, S["w"],
                                                       wqt.codes, wqt.scales)),
        ("gemm_fwd", lambda: api.fp4q_linear_fwd(xq, wq, Y)),
        ("amax", lambda: api.fp4q_amax(dY, amax["dY"])),
        # dY: ROW16 (dgrad) and COL16 (wgrad) in one pass, one Philox word per element
        ("quant_dy_row_col_sr", lambda: api.fp4q_quantize_fmt(dY, amax["dY"], T, api.ROW16, 16, api.UE5M3,
                                                              pack, api.SR, seed, 0, dyq.codes, dyq.scales,
                                                              S["dy"], dyqt.codes, dyqt.scales)),
        ("gemm_dgrad", lambda: api.fp4q_linear_dgrad(dyq, wqt, dX)),
        ("gemm_wgrad", lambda: api.fp4q_linear_wgrad(dyqt, xqt, dW)),
    ]

    def step():
        for _, fn in ops:
            fn()

    if args.profile_op:
        extra = {"gemm_probe_fwd": lambda: api.fp4q_linear_probe(xq, wq, Y, 10)}
        if any(n.startswith("lin_") for n in args.profile_op.split(",")):
            for k, f in linear_layer(args, api, inputs, torch, dev, pack, T):
                extra["lin_" + k] = f
        profile_only(args, ops, X, dev, api, inputs, torch, extra)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(args, "warmup done")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    flops_step = 3 * 2.0 * M * N * K
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    log(args, f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s")

    # per-kernel durations inside the step: a second pass of the same steps with
    # a HIP event recorded on the launch stream between consecutive launches
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s_ev in evs:
        s_ev[0].record()
        for i, (_, fn) in enumerate(ops):
            fn()
            s_ev[i + 1].record()
    torch.cuda.synchronize()
    fam_us, fam_calls = {}, {}
    for s_ev in evs:
        for i, (name, _) in enumerate(ops):
            fam_us[name] = fam_us.get(name, 0.0) + s_ev[i].elapsed_time(s_ev[i + 1]) * 1e3
            fam_calls[name] = fam_calls.get(name, 0) + 1
    kern = {k: fam_us[k] / fam_calls[k] for k in fam_us}  # us per call
    log(args, "per-call us in the step: " + ", ".join(f"{k}={v:.1f}" for k, v in kern.items()))

    gemm_us = (kern["gemm_fwd"] + kern["gemm_dgrad"] + kern["gemm_wgrad"]) / 3.0
    gemm_tflops = 2.0 * M * N * K / (gemm_us * 1e-6) / 1e12

    # algorithmic bytes of each codec launch family per step (each input read
    # once, each output written once)
    def qbytes(rows, cols, es, transposed=False):
        b = rows * cols * es + rows * cols / 2 + rows * cols / 16
        if transposed:
            b += rows * cols / 2 + rows * cols / 256
        return b
    codec_bytes = {
        "amax": (M * K + N * K + M * N) * 2,  # the three launches together
        "quant_x_row_col": qbytes(M, K, 2) + M * K * (0.5 + 1 / 16),
        "quant_w_tile": qbytes(N, K, 2, True) - N * K / 16 + N * K / 256,
        "quant_dy_row_col_sr": qbytes(M, N, 2) + M * N * (0.5 + 1 / 16),
    }
    codec_gbs = {k: codec_bytes[k] * args.steps / (fam_us[k] * 1e-6) / 1e9 for k in codec_bytes}

    # the FP4Linear module (autograd over the same C ABI) on the same shape:
    # steps 1..steps of its sample-and-hold schedule (D = 50), so no refresh
    from fp4_block_scaled_fp4q_amd.recipe import Fp4Recipe, FP4Linear
    layer = FP4Linear(K, N, Fp4Recipe(refresh_period=50), device=dev)
    with torch.no_grad():
        layer.weight.copy_(W.float())
    xin = X.detach().clone().requires_grad_(True)

    def module_step():
        xin.grad = None
        layer.weight.grad = None
        layer(xin).backward(dY)

    module_step()  # step 0: the refresh step
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        module_step()
    b.record()
    torch.cuda.synchronize()
    module_ms = a.elapsed_time(b) / args.steps
    module_tflops = 3 * 2.0 * M * N * K / (module_ms * 1e-3) / 1e12
    log(args, f"FP4Linear fwd+bwd (held amax): {module_ms:.3f} ms/step, {module_tflops:.1f} TFLOP/s")
    del layer, xin

    # the probe-matched accumulation mode on the forward GEMM (same operands)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    api.fp4q_linear_probe(xq, wq, Y, 10)
    a.record()
    for _ in range(3):
        api.fp4q_linear_probe(xq, wq, Y, 10)
    b.record()
    torch.cuda.synchronize()
    probe_us = a.elapsed_time(b) / 3 * 1e3
    probe_tflops = 2.0 * M * N * K / (probe_us * 1e-6) / 1e12
    log(args, f"probe-mode fwd GEMM: {probe_us:.1f} us, {probe_tflops:.1f} TFLOP/s")

    # the 8192-token linear layer, forward and backward, launch by launch
    lin = linear_layer(args, api, inputs, torch, dev, pack, T)

    # quantize-only workload: 8192x4096 bf16 ROW16 RNE, held amax; inputs and
    # outputs rotate over 6 sets (6 x 82 MiB > the 256 MiB Infinity Cache)
    qw = inputs.make("quantize", with_held=True)
    Mq, Kq = qw.dims["M"], qw.dims["K"]
    Xq0 = qw.tensors["X"].t.to(dev)
    held = api.amax(qw.tensors["X"].held_from.to(dev))
    nrot = 6
    Xrot = [Xq0] + [Xq0.clone() for _ in range(nrot - 1)]
    qcr = [torch.empty((Mq, Kq // 2), **u8) for _ in range(nrot)]
    qsr = [torch.empty((Mq, Kq // 16), **u8) for _ in range(nrot)]
    qS = torch.empty(1, **f32)
    for i in range(nrot):
        api.fp4q_quantize(Xrot[i], held, T, api.ROW16, api.RNE, 0, 0, qcr[i], qsr[i], qS)
    reps = 5 * nrot
    # The launches are replayed from a HIP graph: a kernel this short would
    # otherwise wait on the Python-side launch of the next one.
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(reps):
            api.fp4q_quantize(Xrot[i % nrot], held, T, api.ROW16, api.RNE, 0, 0, qcr[i % nrot], qsr[i % nrot],
                              qS)
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    q_us = a.elapsed_time(b) / reps * 1e3
    # every replayed result equals an eager call on the same input
    ec, es_ = torch.empty_like(qcr[0]), torch.empty_like(qsr[0])
    for i in range(nrot):
        api.fp4q_quantize(Xrot[i], held, T, api.ROW16, api.RNE, 0, 0, ec, es_, qS)
        torch.cuda.synchronize()
        if not (torch.equal(ec, qcr[i]) and torch.equal(es_, qsr[i])):
            raise RuntimeError("quantize replayed from a graph differs from the eager call")
    qc, qs = qcr[0], qsr[0]
    del qcr, qsr
    q_bytes = Mq * Kq * (2 + 0.5 + 1 / 16)
    q_gbs = q_bytes / (q_us * 1e-6) / 1e9
    log(args, f"quantize-only 8192x4096: {q_us:.2f} us, {q_gbs:.0f} GB/s")

    # the block-32 and E4M3-scale variants: quantize-only (same workload,
    # graph replay) and the forward GEMM on the FFN shape with variant operands
    variants = {}
    for block, fmt, tag in ((32, api.UE5M3, "block32_ue5m3"), (16, api.E4M3, "block16_e4m3"),
                            (32, api.E4M3, "block32_e4m3")):
        vc = torch.empty((Mq, Kq // 2), **u8)
        vs = torch.empty((Mq, Kq // block), **u8)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(reps):
                api.fp4q_quantize_fmt(Xrot[i % nrot], held, T, api.ROW16, block, fmt, api.PACK_ROWS, api.RNE,
                                      0, 0, vc, vs, qS)
        g.replay()
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        v_us = a.elapsed_time(b) / reps * 1e3
        v_bytes = Mq * Kq * (2 + 0.5 + 1 / block)
        xv, _, _ = api.quantize(X, amax["X"], T, api.ROW16, block=block, scale_fmt=fmt, pack=pack)
        wv, _, _ = api.quantize(W, amax["W"], T, api.TILE16x16, block=block, scale_fmt=fmt, pack=pack)
        api.fp4q_linear_fwd(xv, wv, Y)
        a.record()
        for _ in range(3):
            api.fp4q_linear_fwd(xv, wv, Y)
        b.record()
        torch.cuda.synchronize()
        f_us = a.elapsed_time(b) / 3 * 1e3
        variants[tag] = {"quantize_only_us": round(v_us, 2),
                         "quantize_only_GB/s": round(v_bytes / (v_us * 1e-6) / 1e9, 1),
                         "gemm_fwd_us": round(f_us, 1),
                         "gemm_fwd_TFLOP/s": round(2.0 * M * N * K / (f_us * 1e-6) / 1e12, 1)}
        del xv, wv, g
        log(args, f"variant {tag}: quantize-only {v_us:.2f} us, fwd GEMM {f_us:.1f} us")
    del Xrot

    # traffic from committed rocprofv3 counters, valid only for this GEMM
    # source built with these flags
    rec = _record("gemm_ffn_up_traffic.json", {"gemm_hip_sha256": "csrc/gemm.hip", "codec_h_sha256": "csrc/codec.h"})
    traffic = rec.get("bytes_per_launch") if rec else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, host, M, N, K)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "ffn_up_step: fwd+dgrad+wgrad refresh step, X 16384x4096 bf16 "
                               "(t3 outlier channels), W 14336x4096 bf16 N(0,0.02) 16x16 blocks, "
                               "dY 16384x14336 bf16 log-uniform with SR",
                   "M": M, "N": N, "K": K, "target": T, "pack": args.pack,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel (fwd/dgrad/wgrad average)",
                     "achieved": round(gemm_tflops, 2), "peak": MFMA16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / MFMA16_PEAK_TFLOPS, 4), "traffic": traffic},
        "kernels_us": {k: round(v, 2) for k, v in kern.items()},
        # each GEMM's achieved rate as a fraction of the dense fp16/bf16 MFMA peak
        "gemm_frac": {g: round(2.0 * M * N * K / (kern["gemm_" + g] * 1e-6) / 1e12 / MFMA16_PEAK_TFLOPS, 4)
                      for g in ("fwd", "dgrad", "wgrad")},
        "codec_gbs": {k: round(v, 1) for k, v in codec_gbs.items()},
        "sr_quantize_valu": valu_line(kern["quant_dy_row_col_sr"], "quant_dy_row_col_sr"),
        "linear_8192": lin,
        "quantize_only": {"workload": "8192x4096 bf16 ROW16 RNE, held amax; inputs and outputs rotated "
                                      "over 6 sets (492 MiB)", "us": round(q_us, 2),
                          "GB/s": round(q_gbs, 1), "frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu,
        "next_rows": {
            "probe_gemm_fwd": {"what": "fwd GEMM with the probe-matched accumulation (64-wide slices, "
                                       "toward-zero slice additions, 1/1024 snap)",
                               "us": round(probe_us, 1), "TFLOP/s": round(probe_tflops, 1),
                               "frac_bf16_peak": round(probe_tflops / MFMA16_PEAK_TFLOPS, 4)},
            "variants": variants,
            "fp4linear_step": {"what": "FP4Linear module fwd+bwd through torch autograd on the same "
                                       "shapes, held-amax steps of a D = 50 schedule (no amax "
                                       "kernels), fp32 master weight quantized directly",
                               "ms_per_step": round(module_ms, 4), "TFLOP/s": round(module_tflops, 1)},
        },
    }
    print(json.dumps(out), flush=True)


def _record(name: str, files: dict):
    """A committed rocprofv3 record under profiles/, used only while every
    source it was taken from (and the build flags) is unchanged: files maps
    the record's *_sha256 keys to paths under the package."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        pkg = os.path.join(ROOT, "fp4_block_scaled_fp4q_amd")
        for key, rel in dict(files, build_py_sha256="build.py").items():
            if rec.get(key) != hashlib.sha256(open(os.path.join(pkg, rel), "rb").read()).hexdigest():
                return None
        return rec
    except Exception:
        return None


def valu_line(us: float, launch: str):
    """VALU roofline of a stochastic-rounding quantize launch: its wave64
    VALU instructions per launch (rocprofv3 SQ_INSTS_VALU, committed in
    profiles/codec_valu_counts.json for the current quantize source) over
    its measured duration, against VALU_PEAK_WAVE_INSTR."""
    rec = _record("codec_valu_counts.json", {"source_sha256": "csrc/quantize.hip", "codec_h_sha256": "csrc/codec.h"})
    if rec is None or launch not in rec.get("per_launch", {}):
        return None
    n = rec["per_launch"][launch]["sq_insts_valu"]
    achieved = n / (us * 1e-6)
    return {"bound": "alu", "achieved": round(achieved / 1e9, 2), "peak": round(VALU_PEAK_WAVE_INSTR / 1e9, 2),
            "unit": "G wave64 VALU instr/s", "frac": round(achieved / VALU_PEAK_WAVE_INSTR, 4),
            "valu_instr_per_element": rec["per_launch"][launch].get("valu_lane_instr_per_element")}


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def linear_layer(args, api, inputs, torch, dev, pack, T):
    """The 8192-token linear layer (X 8192x4096, W 4096x4096, dY 8192x4096),
    with held tensor maxima from the companion draws. Forward: quantize X
    ROW16, quantize W TILE16x16, Y = Xq Wq^T (bf16). Backward: quantize dY
    ROW16 + COL16 with SR in one pass, quantize X COL16 (along the 8192
    tokens), dX = dYq Wq (bf16, W's transposed copy prepared beforehand),
    dW = dYq^T Xq (fp32, contraction over the tokens). Each sequence runs
    --steps times after --warmup runs: once timed as a whole, once with an
    event between launches. Returns the per-launch durations, each GEMM's
    TFLOP/s and fraction of the dense MFMA peak, the SR quantize's GB/s and
    fractions of the HBM and VALU peaks, and both sequences end to end."""
    wl = inputs.make("linear_bwd")
    M, N, K = wl.dims["M"], wl.dims["N"], wl.dims["K"]
    X, W, dY = (wl.tensors[k].t.to(dev) for k in ("X", "W", "dY"))
    held = {k: api.amax(wl.tensors[k].held_from.to(dev)) for k in ("X", "W", "dY")}
    del wl
    f32 = dict(dtype=torch.float32, device=dev)
    S = {k: torch.empty(1, **f32) for k in ("x", "w", "dy")}

    def operand(rows, cols, tile, s):
        codes, scales = api.operand_buffers(rows, cols, tile, 16, pack, dev)
        return api.QTensor(codes, scales, s, rows, cols, api.TILE16x16 if tile else api.ROW16, 16, api.UE5M3,
                           pack)
    xq, xqt = operand(M, K, False, S["x"]), operand(K, M, False, S["x"])
    wq, wqt = operand(N, K, True, S["w"]), operand(K, N, True, S["w"])
    dyq, dyqt = operand(M, N, False, S["dy"]), operand(N, M, False, S["dy"])
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), **f32)
    # W's transposed copy for dgrad (an input of the backward sequence)
    api.fp4q_quantize_fmt(W, held["W"], T, api.TILE16x16, 16, api.UE5M3, pack, api.RNE, 0, 0, wq.codes, wq.scales,
                          S["w"], wqt.codes, wqt.scales)
    fwd = [
        ("quant_x_row16", lambda: api.fp4q_quantize_fmt(X, held["X"], T, api.ROW16, 16, api.UE5M3, pack, api.RNE,
                                                        0, 0, xq.codes, xq.scales, S["x"])),
        ("quant_w_tile", lambda: api.fp4q_quantize_fmt(W, held["W"], T, api.TILE16x16, 16, api.UE5M3, pack,
                                                       api.RNE, 0, 0, wq.codes, wq.scales, S["w"])),
        ("gemm_fwd", lambda: api.fp4q_linear_fwd(xq, wq, Y)),
    ]
    bwd = [
        ("quant_dy_row_col_sr", lambda: api.fp4q_quantize_fmt(dY, held["dY"], T, api.ROW16, 16, api.UE5M3, pack,
                                                              api.SR, 0, 0, dyq.codes, dyq.scales, S["dy"],
                                                              dyqt.codes, dyqt.scales)),
        ("quant_x_col16", lambda: api.fp4q_quantize_fmt(X, held["X"], T, api.COL16, 16, api.UE5M3, pack, api.RNE,
                                                        0, 0, xqt.codes, xqt.scales, S["x"])),
        ("gemm_dgrad", lambda: api.fp4q_linear_dgrad(dyq, wqt, dX)),
        ("gemm_wgrad", lambda: api.fp4q_linear_wgrad(dyqt, xqt, dW)),
    ]
    if args.profile_op:
        return fwd + bwd
    out = {"workload": "X 8192x4096 bf16 (t3 outlier channels), W 4096x4096 bf16 N(0,0.02) 16x16 blocks, "
                       "dY 8192x4096 bf16 log-uniform with SR; held tensor maxima; K64 packing",
           "M": M, "N": N, "K": K}
    flops = 2.0 * M * N * K
    for tag, seq in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(args.warmup):
            for _, fn in seq:
                fn()
        torch.cuda.synchronize()
        a, b = _events(torch, 2)
        a.record()
        for _ in range(args.steps):
            for _, fn in seq:
                fn()
        b.record()
        torch.cuda.synchronize()
        seq_us = a.elapsed_time(b) / args.steps * 1e3
        evs = [_events(torch, len(seq) + 1) for _ in range(args.steps)]
        for ev in evs:
            ev[0].record()
            for i, (_, fn) in enumerate(seq):
                fn()
                ev[i + 1].record()
        torch.cuda.synchronize()
        us = {name: sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / args.steps * 1e3
              for i, (name, _) in enumerate(seq)}
        ngemm = 1 if tag == "fwd" else 2
        out[tag] = {"sequence_us": round(seq_us, 2), "sequence_TFLOP/s": round(ngemm * flops / (seq_us * 1e-6) / 1e12, 1),
                    "launch_us": {k: round(v, 2) for k, v in us.items()}}
        for name, v in us.items():
            if name.startswith("gemm_"):
                tf = flops / (v * 1e-6) / 1e12
                out[tag][name] = {"us": round(v, 2), "TFLOP/s": round(tf, 1),
                                  "frac_mfma": round(tf / MFMA16_PEAK_TFLOPS, 4)}
        log(args, f"linear 8192 {tag}: " + ", ".join(f"{k}={v:.1f}" for k, v in us.items())
            + f"; sequence {seq_us:.1f} us")
    # the SR quantize of dY: reads 2 B and writes 2 x (0.5 + 1/16) B per element
    sr_us = out["bwd"]["launch_us"]["quant_dy_row_col_sr"]
    sr_bytes = M * N * (2 + 2 * (0.5 + 1 / 16))
    gbs = sr_bytes / (sr_us * 1e-6) / 1e9
    out["sr_quantize"] = {"us": round(sr_us, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                          "valu": valu_line(sr_us, "lin_quant_dy_row_col_sr")}
    return out


def profile_only(args, ops, X, dev, api, inputs, torch, extra):
    """Run each launch kind of a comma-separated --profile-op list --reps
    times (after one untimed call), for counter collection and tuning.
    'quantize_only' is the 8192x4096 ROW16 RNE workload; 'copy' is a plain
    device copy of 256 MiB, the reference for scaling FETCH_SIZE and
    WRITE_SIZE to bytes; 'lin_<launch>' names a launch of the 8192-token
    linear layer (lin_gemm_fwd, lin_quant_dy_row_col_sr, ...)."""
    prepared = False
    for k, f in extra.items():
        if k.startswith("lin_") and not k.startswith("lin_gemm"):
            f()  # the linear layer's operands, before any of its launches is measured
    for name in args.profile_op.split(","):
        if name == "copy":
            src = torch.empty(256 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            src.fill_(1.0)
            fn = lambda: dst.copy_(src)  # noqa: E731
        elif name == "quantize_only":
            qw = inputs.make("quantize", with_held=False)
            Xq = qw.tensors["X"].t.to(dev)
            held = api.amax(Xq)
            u8 = dict(dtype=torch.uint8, device=dev)
            qc = torch.empty((Xq.shape[0], Xq.shape[1] // 2), **u8)
            qs = torch.empty((Xq.shape[0], Xq.shape[1] // 16), **u8)
            qS = torch.empty(1, dtype=torch.float32, device=dev)
            fn = lambda: api.fp4q_quantize(Xq, held, 448.0, api.ROW16, api.RNE, 0, 0, qc, qs, qS)  # noqa: E731
        else:
            if not prepared:
                for k, f in ops:
                    if not k.startswith("gemm"):
                        f()  # the operands the measured launches read
                prepared = True
            fn = extra[name] if name in extra else dict(ops)[name]
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        print(json.dumps({"profile_op": name, "reps": args.reps,
                          "us_per_call": round(a.elapsed_time(b) / args.reps * 1e3, 2)}), flush=True)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, wl, M, N, K):
    """The oracle, as it stands, on a bounded sample of one step: the first
    Ms token rows of X and dY (their amax, ROW16/COL16 quantizations, fwd
    and dgrad on those rows, wgrad contracting over those tokens) plus the
    full weight quantization; value scaled to the step's FLOPs per second.

    The codec runs twice: once as single calls (one thread), once as
    independent row (ROW16, TILE) or column (COL16) chunks on all host cores
    (the oracle's C calls release the GIL; chunk results equal the single
    calls, SR taking each chunk's origin). The GEMMs run in fp64 numpy BLAS
    on its own thread pool. value uses the all-cores codec time."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_info

    Ms = 2048
    Xs = np.ascontiguousarray(wl.tensors["X"].oracle_view[:Ms])
    dYs = np.ascontiguousarray(wl.tensors["dY"].oracle_view[:Ms])
    Wv = wl.tensors["W"].oracle_view
    # the host cores this process may use, at most 16 (one GPU's share of the host)
    ncpu = max(1, min(16, len(os.sched_getaffinity(0))))

    def codec_single():
        ax, aw, ady = oracle.amax(Xs), oracle.amax(Wv), oracle.amax(dYs)
        xq = oracle.quantize(Xs, ax).q
        w = oracle.quantize(Wv, aw, layout=oracle.TILE16, transposed=True)
        dyq = oracle.quantize(dYs, ady, rnd=oracle.SR).q
        dyqt = oracle.quantize(dYs, ady, layout=oracle.COL16, rnd=oracle.SR).q
        xqt = oracle.quantize(Xs, ax, layout=oracle.COL16).q
        return xq, w, dyq, dyqt, xqt

    def codec_par(ex):
        def amax_par(x):
            parts = list(ex.map(lambda r: oracle.amax(np.ascontiguousarray(x[r:r + 256])),
                                range(0, x.shape[0], 256)))
            return max(parts)

        def q_par(x, amax, layout, rnd=oracle.RNE, transposed=False):
            rows, cols = x.shape
            col = layout == oracle.COL16
            n = cols if col else rows
            ch = 256

            def one(c0):
                part = np.ascontiguousarray(x[:, c0:c0 + ch] if col else x[c0:c0 + ch])
                return oracle.quantize(part, amax, layout=layout, rnd=rnd, transposed=transposed,
                                       origin=(0, c0, cols) if col else (c0, 0, cols))
            return list(ex.map(one, range(0, n, ch)))
        ax, aw, ady = amax_par(Xs), amax_par(Wv), amax_par(dYs)
        parts = [q_par(Xs, ax, oracle.ROW16), q_par(Wv, aw, oracle.TILE16, transposed=True),
                 q_par(dYs, ady, oracle.ROW16, oracle.SR), q_par(dYs, ady, oracle.COL16, oracle.SR),
                 q_par(Xs, ax, oracle.COL16)]
        return parts

    t0 = time.perf_counter()
    xq, w, dyq, dyqt, xqt = codec_single()
    t_codec1 = time.perf_counter() - t0
    with ThreadPoolExecutor(ncpu) as ex:
        t0 = time.perf_counter()
        parts = codec_par(ex)
        t_codecn = time.perf_counter() - t0
    # the chunked run is the same computation: its codes equal the single calls'
    cat = np.concatenate([p.q.codes for p in parts[2]], axis=0)
    if not np.array_equal(cat, dyq.codes):
        raise RuntimeError("chunked oracle quantize differs from the single call")
    del parts
    t0 = time.perf_counter()
    oracle.gemm(xq, w.q)
    oracle.gemm(dyq, w.qt)
    oracle.gemm(dyqt, xqt)
    t_gemm = time.perf_counter() - t0
    flops = 3 * 2.0 * Ms * N * K
    dt = t_codecn + t_gemm
    blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    log(args, f"cpu oracle sample: codec {t_codec1:.1f}s on 1 thread, {t_codecn:.1f}s on {ncpu}; "
              f"GEMMs {t_gemm:.1f}s on {blas_threads} BLAS threads; {flops / dt / 1e12:.4f} TFLOP/s")
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(max(ncpu, blas_threads)),
            "kind": "oracle",
            "sample": f"first {Ms} of {M} token rows of the ffn_up_step (amax + ROW16/COL16 "
                      f"quantize of X and dY rows, full W TILE quantize, fwd/dgrad/wgrad on those "
                      f"rows in fp64 BLAS); codec in row/column chunks on {ncpu} threads "
                      f"({t_codecn:.1f} s; {t_codec1:.1f} s on one thread), GEMMs on {blas_threads} "
                      f"BLAS threads ({t_gemm:.1f} s)",
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(), "codec_threads": ncpu, "blas_threads": int(blas_threads),
            "codec_s_1_thread": round(t_codec1, 2), "codec_s_all_cores": round(t_codecn, 2),
            "gemm_s": round(t_gemm, 2), "seconds": round(dt, 2),
            "value_1_thread_codec": round(flops / (t_codec1 + t_gemm) / 1e12, 5)}


if __name__ == "__main__":
    main()
