#!/usr/bin/env python3
"""Benchmark of the selective scan (S6) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one ssm_scan_fwd over the Mamba-2.8B-shaped layer (batch 16,
D 5120, N 16, L 2048; bf16 inputs and output, fp32 state and arithmetic) with
every input already resident in HBM.  The line also reports the decode
workload (ssm_state_update, batch 256, D 5120, N 16, 64 steps) as a second
object, the roofline of the dominant kernel, and the fp64 CPU oracle timed on
a bounded sample of the same workload on this host.

HBM traffic is read from the GPU's counters in the same run: before this
process touches the GPU it starts three child processes under rocprofv3
(FETCH_SIZE, then WRITE_SIZE, each with a plain device copy of known size as
the calibration, then a kernel trace), each running the same scan step
(`bench.py --counters-child`), and parses their CSV output.

Every timed workload first runs its warm-up calls and then a settle phase of
back-to-back calls lasting at least --settle-ms, so that the timed calls see
the GPU's sustained clock whatever --warmup is.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan elements/s (batch·D·L) + achieved HBM GB/s vs peak, 1×MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, public spec
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, public spec
# One fp32 VALU instruction per lane per clock: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz (the non-packed issue rate; packed fp32 doubles it to 157.3 TFLOP/s
# of FMA, but packed fp32 is not used here).
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Algorithmic VALU work of the scan per (element, state): Delta*A, exp2,
# Delta*u*B, the state FMA and the readout FMA.
OPS_PER_ELEMENT_STATE = 5
# With the zero-order-hold input term, counted as the plain formula needs it:
# Delta*A, exp2, u*B, times 1/A, the fma forming (Abar - 1)*w, the state FMA
# and the readout FMA.  The kernel executes more (13): it also evaluates the
# Taylor series that keeps small |Delta A| accurate, and selects between the
# two forms.
OPS_PER_ELEMENT_STATE_ZOH = 7
OPS_EXECUTED_PER_ELEMENT_STATE_ZOH = 13
# The convolution prologue per element: K taps (FMAs) and silu (exp2, add,
# reciprocal, multiply), at the width the benchmark uses.
CONV_WIDTH = 4
OPS_PER_ELEMENT_CONV = CONV_WIDTH + 4
# Backward by recomputation, per (element, state): the forward recurrence
# and readout again (Delta*A, exp2, Delta*u*B, state FMA, C*h FMA), then the
# reverse step (lambda FMA, lambda*h*Abar: 2, dA FMA, dDelta FMA, lambda*B
# FMA, dB and dC terms, the carry Abar*lambda) and one add each for the
# channel sums of dB and dC.
OPS_PER_ELEMENT_STATE_BWD = 16
KERNEL_NAME = "ssm::scan_kernel<unsigned short, 4, 4, 16, 0, 0, true>"
KERNEL_NAME_ZOH = "ssm::scan_kernel<unsigned short, 4, 4, 16, 0, 1, true>"
KERNEL_NAME_CONV = "ssm::scan_kernel<unsigned short, 4, 4, 16, 0, 2, true>"
PACK_KERNEL_NAME = "ssm::pack_bc_kernel<unsigned short, 4, 4>"
# VALU counters of the scan kernel (one rocprofv3 pass): waves, VALU
# instructions, and VALU-active quad-cycles summed over the waves
VALU_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU")
NUM_SIMDS = 256 * 4
# the plain device copy that calibrates the byte counters: 1 GiB, three times
CALIB_BYTES = 1 << 30
CALIB_COPIES = 3


def scan_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one scan: every input read once, y written
    once, parameters once; the state never goes to HBM."""
    s = 2 if cfg.dtype == "bf16" else 4
    el = cfg.batch * cfg.dim * cfg.seqlen
    tok = el * s * (2 + (1 if cfg.gate else 0))          # u, delta (, z)
    bc = 2 * cfg.batch * cfg.dstate * cfg.seqlen * s      # B, C
    params = cfg.dim * cfg.dstate * 4 + cfg.dim * 4 * (2 if cfg.dskip else 1)
    return tok + bc + params + el * s                    # + y


def ssd_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one SSD call: x, z read and y written once
    per element, dt once per (batch, head, step), B and C once, parameters."""
    s = 2 if cfg.dtype == "bf16" else 4
    el = cfg.batch * cfg.dim * cfg.seqlen
    tok = el * s * (2 + (1 if cfg.gate else 0))               # x, y (, z)
    dt = cfg.batch * cfg.nheads * cfg.seqlen * s
    bc = 2 * cfg.batch * cfg.dstate * cfg.seqlen * s
    params = cfg.nheads * 4 * 2 + (cfg.dim * 4 if cfg.dskip else 0)
    return tok + dt + bc + params


def ssd_flops(cfg, chunk=64) -> int:
    """Matrix work of the chunked evaluation, per chunk and head: the causal
    half of C^T B (Q^2 N) and of M X^T (Q^2 P), C^T H and the state update
    (2 Q N P each), as multiply-adds times two."""
    Q, N, P = chunk, cfg.dstate, cfg.headdim
    per = Q * Q * N + Q * Q * P + 4 * Q * N * P
    nchunks = (cfg.seqlen + Q - 1) // Q
    return cfg.batch * cfg.nheads * nchunks * per


def decode_bytes(cfg) -> int:
    s = 2 if cfg.dtype == "bf16" else 4
    rows = cfg.batch * cfg.dim
    state = rows * cfg.dstate * 4 * 2                     # read + write
    tok = rows * s * (2 + (1 if cfg.gate else 0)) + rows * s   # u, delta, z in; y out
    bc = 2 * cfg.batch * cfg.dstate * s
    params = cfg.dim * cfg.dstate * 4 + cfg.dim * 4 * (2 if cfg.dskip else 1)
    return state + tok + bc + params


def _to_dev(a, dt, dev):
    import torch
    if a is None:
        return None
    if dt == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def settle(step, dev, min_ms):
    """Back-to-back calls until at least min_ms of wall time has passed (the
    GPU's clock ramps up over the first tens of milliseconds of sustained
    load after idling).  Returns (calls, ms)."""
    import torch
    if min_ms <= 0:
        return 0, 0.0
    t0 = time.perf_counter()
    calls = 0
    while True:
        for _ in range(8):
            step()
        calls += 8
        torch.cuda.synchronize(dev)
        ms = (time.perf_counter() - t0) * 1e3
        if ms >= min_ms:
            return calls, round(ms, 1)


def timed(step, dev, stream, steps):
    """Milliseconds per call over `steps` back-to-back calls: one pair of HIP
    events recorded on the stream the kernels run on brackets all of them
    (so no event sits between two calls), with a device synchronisation
    before and after.  Also returns the host wall time per call."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize(dev)
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return float(start.elapsed_time(end)) / steps, wall


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    # The GPU's clock ramps up over the first ~35 ms of sustained load after
    # idling (c3 step: about 0.70 ms for the first calls, 0.58 ms once
    # settled), and the ramp repeats after about two seconds of idle; every
    # workload therefore runs a settle phase of this length before its timed
    # calls, whatever --warmup is.
    ap.add_argument("--settle-ms", type=float, default=300.0)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--no-counters", action="store_true",
                    help="skip the rocprofv3 child runs (counters and kernel trace)")
    ap.add_argument("--prof-dir", default=None,
                    help="keep the child runs' rocprofv3 output in this directory")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the long-sequence workloads (c1, c2) that split the sequence")
    ap.add_argument("--split-only", action="store_true",
                    help="run only the long-sequence workloads (c1, c2) and print their objects")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--counters-child", action="store_true",
                    help="(internal) the program the rocprofv3 child runs execute")
    ap.add_argument("--child-steps", type=int, default=3)
    ap.add_argument("--child-calibrate", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scan is data-parallel over channels and batch rows, so shards would need "
              "no communication, but no multi-GPU path is built).", file=sys.stderr)
        return 2
    if args.counters_child:
        return counters_child(args)

    # counters and kernel trace first, in child processes, before this
    # process touches the GPU
    prof = None
    if not args.no_counters and not args.split_only:
        prof = collect_profiles(args)

    import torch
    import selective_state_space_28_amd as ssm
    import synth

    dev = torch.device("cuda:0")
    ssm.load()
    if args.split_only:
        print(json.dumps({f"split_{name}": bench_split(dev, name, args.steps, args.warmup,
                                                       args.settle_ms)
                          for name in ("c1", "c2")}), flush=True)
        return 0
    cfg = synth.SCAN_CONFIGS["c3"]
    t_gen = time.time()
    inp = synth.make_scan_inputs(cfg)
    gen_s = time.time() - t_gen

    dt = cfg.dtype
    u, delta, B, C, z = (_to_dev(inp[k], dt, dev) for k in ("u", "delta", "B", "C", "z"))
    A, D, bias = (_to_dev(inp[k], "f32", dev) for k in ("A", "D", "delta_bias"))
    y = torch.empty_like(u)
    need = ssm.ssm_scan_fwd_workspace_bytes(cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, u.dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssm.ssm_scan_fwd(u, delta, A, B, C, D, z, bias, out=y, workspace=ws)

    for _ in range(args.warmup):
        step()
    settle_calls, settle_ms = settle(step, dev, args.settle_ms)
    ms, wall_ms = timed(step, dev, stream, args.steps)
    elements = cfg.batch * cfg.dim * cfg.seqlen
    value = elements / (ms * 1e-3)
    alg_bytes = scan_bytes(cfg)
    alg_gbps = alg_bytes / (ms * 1e-3) / 1e9
    ops = elements * cfg.dstate * OPS_PER_ELEMENT_STATE
    alu_tops = ops / (ms * 1e-3) / 1e12
    scan_prof = (prof or {}).get("kernels", {}).get(KERNEL_NAME, {})
    traffic = scan_prof.get("hbm_bytes_per_launch")
    trace_ns = scan_prof.get("trace_avg_ns")
    hbm_view = {"achieved": round(alg_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(alg_gbps / HBM_PEAK_GBPS, 4),
                "note": "algorithmic bytes per launch / timed step (the timed calls between one HIP event pair, over their number)"}
    if traffic:
        hbm_view["measured_GBps"] = round(traffic / (ms * 1e-3) / 1e9, 1)
        hbm_view["measured_frac"] = round(traffic / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    # The binding roof is the one whose lower-bound time is larger: here the
    # VALU (5 fp32 instructions per (element, state) at one per lane per
    # clock) rather than HBM.
    t_hbm = alg_bytes / (HBM_PEAK_GBPS * 1e9)
    t_alu = ops / (VALU_PEAK_TOPS * 1e12)
    roof = {"bound": "alu" if t_alu >= t_hbm else "hbm",
            "achieved": round(alu_tops, 3), "peak": round(VALU_PEAK_TOPS, 3), "unit": "TOP/s",
            "frac": round(alu_tops / VALU_PEAK_TOPS, 4), "traffic": traffic,
            "kernel": KERNEL_NAME,
            "work_per_launch": {"ops": ops, "bytes": alg_bytes},
            "lower_bound_us": {"alu": round(t_alu * 1e6, 1), "hbm": round(t_hbm * 1e6, 1)},
            "hbm": hbm_view,
            "kernel_trace_avg_ms": (round(trace_ns / 1e6, 4) if trace_ns else None)}
    if t_alu < t_hbm:
        roof.update({"achieved": round(alg_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(alg_gbps / HBM_PEAK_GBPS, 4)})
    vc = scan_prof.get("valu_counters")
    if vc and vc.get("SQ_WAVES"):
        tiles = (cfg.seqlen + 15) // 16
        active = vc["SQ_ACTIVE_INST_VALU"] * 4 / NUM_SIMDS  # VALU-busy cycles per SIMD
        roof["valu"] = {
            "wave_insts_per_element": round(vc["SQ_INSTS_VALU"] / elements, 3),
            "lane_ops_per_element": round(vc["SQ_INSTS_VALU"] * 64 / elements, 1),
            "insts_per_wave_tile": round(vc["SQ_INSTS_VALU"] / (vc["SQ_WAVES"] * tiles), 1),
            "active_cycles_per_simd": round(active),
            "busy_frac": (round(active / (trace_ns * 1e-9 * 2.4e9), 4) if trace_ns else None),
            "note": "SQ_INSTS_VALU and SQ_ACTIVE_INST_VALU (quad-cycles) per dispatch, measured in this run; a wave "
                    "instruction covers 64 lanes (lane_ops = 64 x wave instructions; the recurrence alone is 5 x 16 "
                    "states = 80 per element); a wave-tile is one wave's 16 steps of its 64 channels; busy_frac = "
                    "VALU-active cycles per SIMD over the traced kernel time at the 2.4 GHz peak clock"}

    out = {
        "metric": METRIC, "value": value, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "mamba-2.8b-shaped layer scan: batch 16, D 5120, N 16, L 2048, "
                               "bf16 inputs/output, fp32 state, silu gate, D-skip, A jittered",
                   "batch": cfg.batch, "dim": cfg.dim, "dstate": cfg.dstate,
                   "seqlen": cfg.seqlen, "io_dtype": "bf16", "state_dtype": "f32", "seed": cfg.seed},
        "settle": {"calls": settle_calls, "ms": settle_ms, "min_ms": args.settle_ms},
        "hbm": {"algorithmic_bytes": alg_bytes, "algorithmic_GBps": round(alg_gbps, 1),
                "frac_of_peak": round(alg_gbps / HBM_PEAK_GBPS, 4),
                "measured_bytes_per_launch": traffic,
                "measured_GBps": hbm_view.get("measured_GBps"),
                "copy_GBps": copy_rate(dev, stream),
                "copy_note": "practical roof: torch device-to-device copy of 1 GiB buffers (bytes read + written)"},
        "wall_ms_per_step": wall_ms,
        "roofline": roof,
    }
    if prof is not None:
        out["counters"] = prof

    # the same workload with the zero-order-hold input term (flag of the same
    # entry point), timed the same way
    def step_zoh():
        ssm.ssm_scan_fwd(u, delta, A, B, C, D, z, bias, out=y, workspace=ws, bbar="zoh")

    for _ in range(args.warmup):
        step_zoh()
    settle(step_zoh, dev, args.settle_ms)
    ms_z, _ = timed(step_zoh, dev, stream, args.steps)
    ops_z = elements * cfg.dstate * OPS_PER_ELEMENT_STATE_ZOH
    tops_z = ops_z / (ms_z * 1e-3) / 1e12
    out["zoh"] = {"workload": "the same scan with the zero-order-hold input term (bbar='zoh')",
                  "ms_per_step": ms_z, "value": elements / (ms_z * 1e-3), "unit": "elements/s",
                  "roofline": {"bound": "alu", "achieved": round(tops_z, 3),
                               "peak": round(VALU_PEAK_TOPS, 3), "unit": "TOP/s",
                               "frac": round(tops_z / VALU_PEAK_TOPS, 4),
                               "kernel": KERNEL_NAME_ZOH,
                               "ops_per_launch": ops_z,
                               "ops_executed_per_element_state": OPS_EXECUTED_PER_ELEMENT_STATE_ZOH,
                               "hbm_frac": round(alg_bytes / (ms_z * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}}

    # the same workload with the width-4 convolution prologue fused in (x is
    # the u draw; taps and bias from the generator)
    cp = synth.make_conv_params(cfg.dim, CONV_WIDTH, cfg.seed)
    cw = torch.from_numpy(cp["conv_w"]).to(dev)
    cb = torch.from_numpy(cp["conv_b"]).to(dev)

    def step_conv():
        ssm.ssm_conv_scan_fwd(u, cw, cb, delta, A, B, C, D, z, bias, out=y, workspace=ws)

    for _ in range(args.warmup):
        step_conv()
    settle(step_conv, dev, args.settle_ms)
    ms_c, _ = timed(step_conv, dev, stream, args.steps)
    ops_c = elements * (cfg.dstate * OPS_PER_ELEMENT_STATE + OPS_PER_ELEMENT_CONV)
    tops_c = ops_c / (ms_c * 1e-3) / 1e12
    conv_prof = (prof or {}).get("kernels", {}).get(KERNEL_NAME_CONV, {})
    out["conv"] = {"workload": f"the same scan with the causal depthwise conv1d + silu prologue "
                               f"fused in (width {CONV_WIDTH}, ssm_conv_scan_fwd)",
                   "ms_per_step": ms_c, "value": elements / (ms_c * 1e-3), "unit": "elements/s",
                   "roofline": {"bound": "alu", "achieved": round(tops_c, 3),
                                "peak": round(VALU_PEAK_TOPS, 3), "unit": "TOP/s",
                                "frac": round(tops_c / VALU_PEAK_TOPS, 4),
                                "kernel": KERNEL_NAME_CONV,
                                "ops_per_launch": ops_c,
                                "traffic": conv_prof.get("hbm_bytes_per_launch"),
                                "hbm_frac": round(alg_bytes / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}}

    if not args.no_bwd:
        # the backward pass of the same workload (dy ~ N(0, 1), bf16)
        gy = torch.randn(u.shape, generator=torch.Generator(device=dev).manual_seed(5), device=dev,
                         dtype=torch.float32).to(u.dtype)
        bws = torch.empty(ssm.ssm_scan_bwd_workspace_bytes(cfg.batch, cfg.dim, cfg.dstate,
                                                           cfg.seqlen, u.dtype),
                          dtype=torch.uint8, device=dev)

        def step_bwd():
            ssm.ssm_scan_bwd(u, delta, A, B, C, D, z, bias, dy=gy, workspace=bws)

        step_bwd()
        settle(step_bwd, dev, args.settle_ms)
        nb = max(1, args.steps // 5)
        ms_b, _ = timed(step_bwd, dev, stream, nb)
        ops_b = elements * cfg.dstate * OPS_PER_ELEMENT_STATE_BWD
        tops_b = ops_b / (ms_b * 1e-3) / 1e12
        out["bwd"] = {"workload": "ssm_scan_bwd of the same scan (all gradients, states recomputed)",
                      "steps": nb, "ms_per_step": ms_b, "value": elements / (ms_b * 1e-3),
                      "unit": "elements/s",
                      "roofline": {"bound": "alu", "achieved": round(tops_b, 3),
                                   "peak": round(VALU_PEAK_TOPS, 3), "unit": "TOP/s",
                                   "frac": round(tops_b / VALU_PEAK_TOPS, 4),
                                   "kernel": "ssm::bwd_kernel<unsigned short, 4, 4, 16, false, 4> (+ "
                                             "checkpoint pass and sums)",
                                   "ops_per_launch": ops_b}}

        # the same backward with the zero-order-hold input term
        def step_bwd_zoh():
            ssm.ssm_scan_bwd(u, delta, A, B, C, D, z, bias, dy=gy, bbar="zoh", workspace=bws)

        step_bwd_zoh()
        settle(step_bwd_zoh, dev, args.settle_ms)
        ms_bz, _ = timed(step_bwd_zoh, dev, stream, nb)
        out["bwd_zoh"] = {"workload": "ssm_scan_bwd of the same scan with the zero-order-hold input term",
                          "steps": nb, "ms_per_step": ms_bz, "value": elements / (ms_bz * 1e-3),
                          "unit": "elements/s"}
        del bws

        # the training pair: the forward writes the tile checkpoints beside y
        # and the backward starts from them (no checkpoint pass of its own)
        ck = torch.empty((cfg.batch, (cfg.seqlen + 15) // 16, cfg.dstate, cfg.dim), dtype=torch.float32,
                         device=dev)
        cws = torch.empty(max(1, ssm.ssm_scan_bwd_ckpt_workspace_bytes(cfg.batch, cfg.dim, cfg.dstate,
                                                                       cfg.seqlen, u.dtype)),
                          dtype=torch.uint8, device=dev)
        train = {"workload": "one training step of the same scan: forward then backward "
                             "(Euler input term unless named)", "steps": nb}
        for bbar in ("euler", "zoh"):
            sfx = "" if bbar == "euler" else "_zoh"

            def step_fwd_ckpt():
                ssm.ssm_scan_fwd_ckpt(u, delta, A, B, C, D, z, bias, out=y, ckpt=ck, workspace=ws,
                                      bbar=bbar)

            def step_bwd_ckpt():
                ssm.ssm_scan_bwd_ckpt(u, delta, A, B, C, D, z, bias, ckpt=ck, dy=gy, workspace=cws,
                                      bbar=bbar)

            def step_train():
                step_fwd_ckpt()
                step_bwd_ckpt()

            for name, fn, n in (("fwd_ckpt", step_fwd_ckpt, args.steps), ("bwd_ckpt", step_bwd_ckpt, nb),
                                ("fwd_plus_bwd_ckpt", step_train, nb)):
                fn()
                settle(fn, dev, args.settle_ms)
                ms_t, _ = timed(fn, dev, stream, n)
                train[name + sfx + "_ms"] = ms_t
            fwd_ms = ms if bbar == "euler" else ms_z
            bwd_ms = ms_b if bbar == "euler" else ms_bz
            train["fwd_plus_bwd_plain" + sfx + "_ms"] = fwd_ms + bwd_ms
        train["note"] = ("fwd_ckpt: ssm_scan_fwd_ckpt (y, last_state and the tile checkpoints); bwd_ckpt: "
                         "ssm_scan_bwd_ckpt from them; fwd_plus_bwd_ckpt: the two timed back to back; "
                         "fwd_plus_bwd_plain: ssm_scan_fwd + ssm_scan_bwd (the latter running its own "
                         "checkpoint pass), the sum of their timings above")
        out["train"] = train
        del gy, ck, cws
    del u, delta, B, C, z, y, ws

    if not args.no_split:
        for name in ("c1", "c2"):
            out[f"split_{name}"] = bench_split(dev, name, args.steps, args.warmup, args.settle_ms)
    if not args.no_decode:
        out["decode"] = bench_decode(dev, args.decode_steps)
    if not args.no_ssd:
        out["ssd"] = bench_ssd(dev, args.steps, args.warmup, args.settle_ms)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    out["input_generation_s"] = round(gen_s, 2)
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------- rocprofv3 children
def counters_child(args):
    """The program each rocprofv3 child run executes: the c3 scan step
    (warm-up, settle, then --child-steps calls) and, with --child-calibrate,
    afterwards CALIB_COPIES plain device copies of CALIB_BYTES (the known
    size that calibrates the byte counters).  Prints one JSON line."""
    import torch
    import selective_state_space_28_amd as ssm
    import synth
    dev = torch.device("cuda:0")
    ssm.load()
    cfg = synth.SCAN_CONFIGS["c3"]
    inp = synth.make_scan_inputs(cfg)
    u, delta, B, C, z = (_to_dev(inp[k], cfg.dtype, dev) for k in ("u", "delta", "B", "C", "z"))
    A, D, bias = (_to_dev(inp[k], "f32", dev) for k in ("A", "D", "delta_bias"))
    y = torch.empty_like(u)
    ws = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(cfg.batch, cfg.dim, cfg.dstate,
                                                             cfg.seqlen, u.dtype)),
                     dtype=torch.uint8, device=dev)
    cp = synth.make_conv_params(cfg.dim, CONV_WIDTH, cfg.seed)
    cw, cb = torch.from_numpy(cp["conv_w"]).to(dev), torch.from_numpy(cp["conv_b"]).to(dev)

    def step():
        ssm.ssm_scan_fwd(u, delta, A, B, C, D, z, bias, out=y, workspace=ws)

    def step_conv():
        ssm.ssm_conv_scan_fwd(u, cw, cb, delta, A, B, C, D, z, bias, out=y, workspace=ws)

    for fn in (step, step_conv):
        fn()
        settle(fn, dev, args.settle_ms if args.child_steps > 3 else 0.0)
        for _ in range(args.child_steps):
            fn()
        torch.cuda.synchronize(dev)
    del u, delta, B, C, z, y, ws
    if args.child_calibrate:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        for _ in range(CALIB_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
    print(json.dumps({"counters_child": "ok", "steps": args.child_steps}), flush=True)
    return 0


def _csv_rows(directory, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _field(row, *names):
    for n in names:
        if n in row and row[n] not in (None, ""):
            return row[n]
    low = {k.lower(): v for k, v in row.items() if k}
    for n in names:
        v = low.get(n.lower())
        if v not in (None, ""):
            return v
    return None


def _kname(row):
    name = _field(row, "Kernel_Name", "KernelName", "Kernel-Name") or ""
    return name[5:] if name.startswith("void ") else name


def _counter_per_dispatch(rows, counter):
    """{dispatch id: (kernel name, summed value)} of one counter."""
    out = {}
    for r in rows:
        if (_field(r, "Counter_Name", "Counter-Name") or "") != counter:
            continue
        did = int(float(_field(r, "Dispatch_Id", "Dispatch_ID", "Dispatch-Id") or -1))
        val = float(_field(r, "Counter_Value", "Counter-Value") or 0.0)
        name, acc = out.get(did, (_kname(r), 0.0))
        out[did] = (name, acc + val)
    return out


def _starts(name, prefix):
    return name == prefix or name.startswith(prefix + "(") or name.startswith(prefix + " ")


def parse_profile_dirs(dirs, steps):
    """Bytes per launch and traced durations from the child runs' CSV files.

    dirs: {"fetch": dir, "write": dir, "valu": dir, "trace": dir} (any may be
    missing).
    In the fetch and write runs, the copies after the last scan dispatch are
    the calibration: CALIB_COPIES x CALIB_BYTES read and written, so
    scale = known bytes / counted bytes turns a counter reading into bytes.
    Returns (calibration, {kernel: figures}, first error or None)."""
    kernels, calib, err = {}, {}, None
    for tag, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        if tag not in dirs:
            continue
        per = _counter_per_dispatch(_csv_rows(dirs[tag], "counter_collection.csv"), counter)
        if not per:
            err = err or f"no {counter} rows in the '{tag}' run's output"
            continue
        last_scan = max((i for i, (n, _) in per.items() if _starts(n, KERNEL_NAME)), default=-1)
        copy_kib = sum(v for i, (n, v) in per.items() if i > last_scan and "copy" in n.lower())
        if copy_kib <= 0:
            err = err or f"no calibration copy found in the '{tag}' run"
            continue
        scale = CALIB_COPIES * CALIB_BYTES / (copy_kib * 1024.0)
        calib[counter] = {"copy_KiB": round(copy_kib, 1), "scale": round(scale, 4)}
        for name in (KERNEL_NAME, KERNEL_NAME_CONV, PACK_KERNEL_NAME):
            vals = [v for i, (n, v) in per.items() if _starts(n, name)]
            if vals:
                k = kernels.setdefault(name, {})
                k[f"{counter}_KiB"] = round(float(np.mean(vals)), 1)
                k["read_bytes" if counter == "FETCH_SIZE" else "write_bytes"] = \
                    round(float(np.mean(vals)) * 1024.0 * scale)
                k[f"{counter}_dispatches"] = len(vals)
    for name, k in kernels.items():
        if "read_bytes" in k and "write_bytes" in k:
            k["hbm_bytes_per_launch"] = k["read_bytes"] + k["write_bytes"]
    if "valu" in dirs:
        # VALU instructions and VALU-active quad-cycles (summed over the
        # device's SIMDs) per dispatch, and the waves that ran them
        rows = _csv_rows(dirs["valu"], "counter_collection.csv")
        for name in (KERNEL_NAME, KERNEL_NAME_CONV):
            got = {}
            for counter in VALU_COUNTERS:
                vals = [v for i, (n, v) in _counter_per_dispatch(rows, counter).items() if _starts(n, name)]
                if vals:
                    got[counter] = float(np.mean(vals))
            if len(got) == len(VALU_COUNTERS):
                kernels.setdefault(name, {})["valu_counters"] = {c: round(v) for c, v in got.items()}
            elif name == KERNEL_NAME:
                err = err or "no VALU counter rows for the scan kernel in the 'valu' run"
    if "trace" in dirs:
        rows = _csv_rows(dirs["trace"], "kernel_trace.csv")
        for name in (KERNEL_NAME, KERNEL_NAME_CONV, PACK_KERNEL_NAME):
            durs = []
            for r in rows:
                if not _starts(_kname(r), name):
                    continue
                t0 = float(_field(r, "Start_Timestamp", "Start-Timestamp", "BeginNs") or 0)
                t1 = float(_field(r, "End_Timestamp", "End-Timestamp", "EndNs") or 0)
                durs.append((t0, t1 - t0))
            durs.sort()
            if durs:
                last = [d for _, d in durs[-steps:]]
                k = kernels.setdefault(name, {})
                k["trace_avg_ns"] = round(float(np.mean(last)), 1)
                k["trace_dispatches_averaged"] = len(last)
    return calib, kernels, err


def collect_profiles(args):
    """Four child runs of this program under rocprofv3, before this process
    touches the GPU: FETCH_SIZE and WRITE_SIZE per dispatch (each run ends
    with plain copies of known size, whose counter reading gives the factor
    that turns the counter into bytes), the VALU instruction counters, then a
    kernel trace of the same step after a settle phase.  Returns per-kernel bytes per launch and the traced
    mean duration of the last --steps dispatches; or an 'error' entry."""
    exe = shutil.which("rocprofv3")
    if exe is None:
        return {"error": "rocprofv3 not found: traffic not measured"}
    keep = args.prof_dir is not None
    base = os.path.abspath(args.prof_dir) if keep else tempfile.mkdtemp(prefix="ssm_bench_prof_")
    os.makedirs(base, exist_ok=True)
    env = dict(os.environ)
    env.setdefault("TMPDIR", "/tmp")
    me = os.path.abspath(__file__)
    runs = [("fetch", ["--kernel-trace", "--pmc", "FETCH_SIZE"], ["--child-calibrate"], 3),
            ("write", ["--kernel-trace", "--pmc", "WRITE_SIZE"], ["--child-calibrate"], 3),
            ("valu", ["--kernel-trace", "--pmc", *VALU_COUNTERS], [], 3),
            ("trace", ["--kernel-trace", "--stats"], [], args.steps)]
    res = {"commands": [], "note": "child runs of this program under rocprofv3, in this bench run"}
    dirs = {}
    for tag, popts, copts, nsteps in runs:
        d = os.path.join(base, tag)
        cmd = ["timeout", "-s", "KILL", "240", exe, *popts, "-f", "csv", "-d", d, "-o", tag, "--",
               sys.executable, me, "--counters-child", "--child-steps", str(nsteps),
               "--settle-ms", str(args.settle_ms), *copts]
        res["commands"].append(" ".join(["rocprofv3", *popts, "-f", "csv", "-d", "<dir>", "-o", tag,
                                         "--", "python3", "bench.py", "--counters-child",
                                         "--child-steps", str(nsteps), *copts]))
        print(f"[bench] rocprofv3 child run '{tag}' ...", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        try:
            r = subprocess.run(cmd, cwd=base, env=env, capture_output=True, text=True, timeout=270)
        except subprocess.TimeoutExpired:
            res["error"] = f"child run '{tag}' timed out"
            break
        ok = '"counters_child": "ok"' in r.stdout
        print(f"[bench]   rc {r.returncode}, {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
        if not ok:
            res["error"] = (f"child run '{tag}' failed (rc {r.returncode}): "
                            + (r.stderr or r.stdout)[-400:])
            break
        dirs[tag] = d
    try:
        calib, kernels, err = parse_profile_dirs(dirs, args.steps)
        if err:
            res.setdefault("error", err)
        res["calibration"] = calib
        res["kernels"] = kernels
    except Exception as e:  # a malformed profiler output must not lose the bench line
        res["error"] = f"parsing the rocprofv3 output failed: {type(e).__name__}: {e}"
    if not keep:
        shutil.rmtree(base, ignore_errors=True)
    else:
        res["dir"] = base
    return res


def copy_rate(dev, stream, nbytes=1 << 30, reps=10):
    """GB/s (read + written) of a plain device copy over three rotating
    1 GiB buffer pairs, as the practical HBM roof of a streaming kernel."""
    import torch
    src = [torch.ones(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(3)]
    dst = [torch.empty_like(t) for t in src]
    for i in range(3):
        dst[i].copy_(src[i])
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        dst[i % 3].copy_(src[i % 3])
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def bench_split(dev, name, steps, warmup, settle_ms):
    """A workload whose channels alone do not fill the GPU, so the library
    splits the sequence into segments and composes their aggregates (an
    aggregate launch, then the main launch): c1 (batch 8, D 1536, L 2048,
    fp32) or c2 (batch 1, D 2048, L 65536, bf16), N 16, timed like the main
    step."""
    import torch
    import selective_state_space_28_amd as ssm
    import synth
    cfg = synth.SCAN_CONFIGS[name]
    inp = synth.make_scan_inputs(cfg)
    u, delta, B, C, z = (_to_dev(inp.get(k), cfg.dtype, dev) for k in ("u", "delta", "B", "C", "z"))
    A, D, bias = (_to_dev(inp.get(k), "f32", dev) for k in ("A", "D", "delta_bias"))
    y = torch.empty_like(u)
    ws = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen,
                                                            u.dtype)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssm.ssm_scan_fwd(u, delta, A, B, C, D, z, bias, out=y, workspace=ws)

    for _ in range(warmup):
        step()
    settle(step, dev, settle_ms)
    ms, _ = timed(step, dev, stream, steps)
    elements = cfg.batch * cfg.dim * cfg.seqlen
    ops = elements * cfg.dstate * OPS_PER_ELEMENT_STATE
    tops = ops / (ms * 1e-3) / 1e12
    nbytes = scan_bytes(cfg)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{cfg.batch}x{cfg.dim}x{cfg.seqlen}, N {cfg.dstate}, {cfg.dtype} I/O, "
                        f"gate {'on' if cfg.gate else 'off'}, D-skip {'on' if cfg.dskip else 'off'}; "
                        "the sequence split into segments (aggregate launch + main launch)",
            "steps": steps, "ms_per_step": ms, "value": elements / (ms * 1e-3), "unit": "elements/s",
            "hbm": {"algorithmic_bytes": nbytes, "algorithmic_GBps": round(gbps, 1),
                    "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)},
            "roofline": {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 3),
                         "unit": "TOP/s", "frac": round(tops / VALU_PEAK_TOPS, 4),
                         "ops_per_launch": ops,
                         "note": "ops count the result pass only; the aggregate pass is extra work"}}


def bench_decode(dev, steps):
    """The decode workload: 64 successive one-token steps on a persistent
    fp32 state (batch 256, D 5120, N 16), token inputs resident in HBM."""
    import torch
    import selective_state_space_28_amd as ssm
    import synth
    cfg = synth.DECODE_CONFIG
    p = synth.make_decode_params(cfg)
    st = torch.from_numpy(p["h0"]).to(dev)
    A = torch.from_numpy(p["A"]).to(dev)
    D = torch.from_numpy(p["D"]).to(dev)
    bias = torch.from_numpy(p["delta_bias"]).to(dev)
    toks = []
    for s in range(steps):
        t = synth.make_decode_step(cfg, s)
        toks.append({k: torch.from_numpy(t[k].view(np.int16)).view(torch.bfloat16).to(dev)
                     for k in ("u", "delta", "B", "C", "z")})
    ys = [torch.empty_like(toks[0]["u"]) for _ in range(steps)]
    stream = torch.cuda.current_stream(dev)

    def run():
        for s in range(steps):
            t = toks[s]
            ssm.ssm_state_update(st, t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias, out=ys[s])

    run()  # warm-up (the state keeps evolving; the work per step is the same)
    settle(run, dev, 300.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    nbytes = decode_bytes(cfg)
    gbps = nbytes / (ms * 1e-3) / 1e9

    # Reference: a plain in-place update of a state-sized fp32 buffer (torch's
    # elementwise kernel), rotating over six buffers so that, as in the decode
    # loop with fresh tokens each step, the state is not held in the 256 MB
    # last-level cache.  This is the practical HBM rate of the access pattern.
    bufs = [torch.zeros_like(st) for _ in range(6)]
    for b_ in bufs:
        b_.mul_(0.999)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for i in range(steps):
        bufs[i % 6].mul_(0.999)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ref_ms = e0.elapsed_time(e1) / steps
    ref_gbps = 2 * st.numel() * 4 / (ref_ms * 1e-3) / 1e9
    del bufs
    return {"workload": "decode ssm_state_update: batch 256, D 5120, N 16, bf16 tokens, fp32 state",
            "steps": steps, "ms_per_token_step": ms,
            "channels_per_s": cfg.batch * cfg.dim / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "bytes_per_launch": nbytes,
                         "inplace_update_reference_GBps": round(ref_gbps, 1),
                         "note": "reference = torch in-place update of a state-sized buffer "
                                 "over six rotating buffers (the practical HBM rate of an "
                                 "in-place read-modify-write)"}}


def bench_ssd(dev, steps, warmup, settle_ms):
    """The SSD (scalar A per head) workload: the 2.8B token grid (batch 16,
    L 2048, 5120 channels) as 80 heads of 64 with 128 states, bf16."""
    import torch
    import selective_state_space_28_amd as ssm
    import synth
    cfg = synth.SSD_CONFIG
    inp = synth.make_ssd_inputs(cfg)

    def dev_t(a, f32=False):
        if a is None:
            return None
        if not f32 and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    x, dt, B, C, z = (dev_t(inp[k]) for k in ("x", "dt", "B", "C", "z"))
    A, D, bias = (dev_t(inp[k], True) for k in ("A", "D", "dt_bias"))
    y = torch.empty_like(x)
    ws = torch.empty(ssm.ssm_ssd_scan_fwd_workspace_bytes(cfg.batch, cfg.dstate, cfg.seqlen, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssm.ssm_ssd_scan_fwd(x, dt, A, B, C, D, z, bias, out=y, workspace=ws)

    for _ in range(warmup):
        step()
    settle(step, dev, settle_ms)
    ms, _ = timed(step, dev, stream, steps)
    nbytes = ssd_bytes(cfg)
    flops = ssd_flops(cfg)
    gbps = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof.update({"kernel": f"ssm::ssd_kernel<unsigned short, {cfg.dstate}, true>",
                 "bytes_per_launch": nbytes, "flops_per_launch": flops,
                 "mfma_TFLOPs": round(tflops, 2)})
    del x, dt, B, C, z, y, ws
    return {"workload": f"SSD (scalar A per head) scan: batch {cfg.batch}, {cfg.nheads} heads x "
                        f"{cfg.headdim}, N {cfg.dstate}, L {cfg.seqlen}, bf16, chunks of 64 on the "
                        "matrix cores", "ms_per_step": ms, "value": cfg.elements / (ms * 1e-3),
            "unit": "elements/s", "roofline": roof}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, inp, min_core_seconds=12.0):
    """The fp64 oracle as it stands, timed on this host over a bounded sample
    of the same workload: whole batch rows (all channels, whole sequences),
    four at a time, until about `min_core_seconds` of CPU time (threads x
    wall) is spent or the whole batch is done.  Threads: every CPU this
    process may run on, capped by OMP_NUM_THREADS when that is set (on a
    shared GPU host it states the CPU share of one GPU)."""
    import oracle
    import synth
    host = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = host
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = max(1, min(usable, omp) if omp > 0 else usable)
    sec, nb, chunk = 0.0, 0, 4
    while nb < cfg.batch and sec * threads < min_core_seconds:
        sl = slice(nb, min(nb + chunk, cfg.batch))
        w = {k: synth.widen(inp[k][sl], cfg.dtype) for k in ("u", "delta", "B", "C", "z")}
        t0 = time.perf_counter()
        oracle.scan_fwd(w["u"], w["delta"], inp["A"], w["B"], w["C"], inp["D"], w["z"],
                        inp["delta_bias"], True, None, nthreads=threads)
        sec += time.perf_counter() - t0
        nb = sl.stop
        del w
    el = nb * cfg.dim * cfg.seqlen
    return {"value": el / sec, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "host_cpus": host, "usable_cpus": usable, "omp_num_threads": omp or None,
            "cpu_model": _cpu_model(),
            "sample": f"batch rows 0..{nb - 1} of the same workload ({nb}x{cfg.dim}x{cfg.seqlen} "
                      f"elements, N {cfg.dstate}), fp64, {threads} threads, {sec:.1f} s wall, "
                      f"{sec * threads:.0f} core-s"}


if __name__ == "__main__":
    sys.exit(main())
