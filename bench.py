"""Benchmark of the selective scan on one MI355X.

One step = one forward scan over the Mamba-2.8B layer workload (B=4, L=4096,
D=5120, N=16; bfloat16 u/delta/z/Bm/Cm, float32 A/Dskip/dt_bias/state,
float32 arithmetic), inputs resident in HBM.  Prints one JSON line:

* value: algorithmic GB/s of the forward (bytes the method must move: u,
  delta, z, y, Bm, Cm, A, Dskip, dt_bias and h_final; the (B,L,D,N) state
  expansion is never moved) per wall time of a step;
* roofline: the forward kernel's average launch duration from HIP events
  recorded around every timed launch on the launch stream, against the VALU
  bound of the chip (its published fp32 vector rate, 157.3 TFLOP/s: 32 FMA
  lanes per SIMD per clock, which non-packed code reaches with two or more
  waves issuing on a SIMD): the scan does 4 VALU instructions and one
  v_exp_f32 per (b, t, d, n), the transcendental priced at half the FMA rate,
  and moves only O(B L D) bytes, so at these shapes the VALU, not HBM,
  bounds it.  Also the median and minimum
  launch, a cold launch (after overwriting the 256 MB last-level cache with a
  512 MB scratch write, untimed) and the bandwidth of a plain 1 GiB device
  copy measured in the same run;
* configs: the other workloads, each timed the same way -- Tiny (per call,
  and per call inside a replayed HIP graph, which leaves out the host's launch
  cost), the 130M-layer and 1M-step forwards (GB/s, fractions of the HBM and
  VALU bounds) and the training workload's forward + backward;
* cpu_baseline: the float64 oracle timed on this host on a bounded channel
  sample of the same workload (host CPU model and core count stated).

``--gpus N`` with N > 1 exits: this benchmark and the library run on one GPU.
``--extra`` adds the 2.8B-layer forward behind the fused causal conv1d + SiLU
front end (x in place of u, d_conv = 4) and that front end's backward, the
recurrent step at the 2.8B layer's width (B=4, D=5120, N=16: one decode step
per call from Python, so the host's launch overhead, not the kernel, sets this
rate; the kernel's own duration is in the kernel trace; also over buffers
bound once, per call and per step inside a replayed graph), the same step at
B = 64 and 256 (batched decode, where the state's read and write set the
rate), the step behind the conv front end at B = 256, a 4-token forward at
B = 256 (the short-sequence path) and the Mamba-2 (SSD) layers.
``--no-configs`` leaves out the other workloads (the headline alone).
``--ssd`` times only the Mamba-2 (SSD) layers of ``--extra`` and prints them
as their own JSON line (no headline).
``--copy-probe`` runs a plain device copy of 1 GiB first (counter calibration).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0                     # MI355X HBM3E, published
# HBM traffic of the forward kernel, from two rocprofv3 --pmc runs (FETCH_SIZE,
# WRITE_SIZE) calibrated against a copy of known size; valid only for the
# kernel sources it was measured on (their SHA-256 is recorded beside it).
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "scan_fwd_2p8b_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_mssm_amd", "csrc", f)
                  for f in ("scan_fwd.hip", "scan_fwd_kernels.h", "balanced_plan.h", "device_common.h", "launch.h")]
# FMA-lane slots per second: CUs x SIMDs x 32 lanes per clock x clock = 78.6 T (157.3 TFLOP/s)
VALU_PEAK_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
SLOTS_PER_ELEM_STATE = 6                  # 4 VALU + 1 v_exp_f32 priced at half the FMA rate (2 slots)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_bytes(w: workloads.Workload) -> int:
    act = 2 if w.dtype == "bf16" else 4
    return (w.B * w.L * w.D * 4 * act + w.B * w.L * w.N * 2 * act
            + 4 * w.D * w.N + 8 * w.D + 4 * w.B * w.D * w.N)


def conv_fwd_bytes(w: workloads.Workload, d_conv: int = 4) -> int:
    """The forward behind the fused conv front end: x in place of u, plus the
    taps and bias (u itself never moves)."""
    return fwd_bytes(w) + 4 * w.D * d_conv + 4 * w.D


def conv_bwd_bytes(w: workloads.Workload, d_conv: int = 4) -> int:
    """Backward of the conv front end: reads x and du, writes dx; the taps,
    bias and their gradients."""
    act = 2 if w.dtype == "bf16" else 4
    return 3 * w.B * w.L * w.D * act + 2 * 4 * w.D * (d_conv + 1)


def time_conv_bwd(mssm, torch, w, reps=20, warmup=3):
    """Median time of one mssm_conv_bwd call (both of its kernels), HIP events."""
    inp = workloads.make_inputs(w)
    inp.update(workloads.conv_front_end(w, 4))
    t = workloads.to_torch(inp, "cuda", keys=("u", "conv_w", "conv_b", "x_prev"))
    du = workloads.to_torch(dict(inp, u=inp["z"]), "cuda", keys=("u",))["u"]  # any (B, L, D) activations
    del inp

    def run():
        mssm.conv_bwd(t["u"], t["conv_w"], du, conv_b=t["conv_b"], x_prev=t["x_prev"])

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3


def bwd_bytes(w: workloads.Workload) -> int:
    act = 2 if w.dtype == "bf16" else 4
    # reads u, delta, z, dy, Bm, Cm, A, Dskip, dt_bias; writes du, ddelta, dz, dB, dC, dA, dD, ddt_bias
    return (w.B * w.L * w.D * 7 * act + w.B * w.L * w.N * 4 * act
            + 2 * 4 * w.D * w.N + 4 * 4 * w.D)


def kernel_sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the forward kernel recorded in the traffic
    summary, or None when it is missing or was measured on other sources."""
    try:
        with open(TRAFFIC_SUMMARY, encoding="utf-8") as fh:
            text = fh.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    try:
        if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_fwd(mssm, torch, w, steps, warmup, cold_reps=0, conv=False):
    """Forward kernel time per call (HIP events on the launch stream); with
    `conv`, the forward behind the fused causal conv1d + SiLU front end
    (d_conv = 4), the workload's u serving as the conv input x."""
    inp = workloads.make_inputs(w)
    if conv:
        inp.update(workloads.conv_front_end(w, 4))
    t = workloads.to_torch(inp, "cuda")
    del inp
    y = torch.empty_like(t["u"])
    hf = torch.empty((w.B, w.D, w.N), dtype=torch.float32, device="cuda")
    ws_n = mssm.fwd_workspace_bytes(w.B, w.L, w.D, w.N, t["u"].dtype)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def run():
        if conv:
            mssm.conv_scan_fwd(t["u"], t["conv_w"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"],
                               t["dt_bias"], None, conv_b=t["conv_b"], y=y, h_final=hf, workspace=ws)
        else:
            mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"],
                          None, y=y, h_final=hf, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    cold_ms = []
    if cold_reps:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        for _ in range(cold_reps):
            scratch.fill_(1)  # untimed: evicts the inputs from the last-level cache
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            b.record(stream)
            torch.cuda.synchronize()
            cold_ms.append(a.elapsed_time(b))
        del scratch
    return wall, launch_ms, cold_ms


def time_fwd_graph(mssm, torch, w, calls=200, reps=5):
    """Forward time per call with `calls` calls captured in one HIP graph and
    the graph replayed (launch-bound workloads: no host cost between calls).
    Median over `reps` replays, HIP events around each replay."""
    inp = workloads.make_inputs(w)
    t = workloads.to_torch(inp, "cuda")
    y = torch.empty_like(t["u"])
    hf = torch.empty((w.B, w.D, w.N), dtype=torch.float32, device="cuda")
    ws_n = mssm.fwd_workspace_bytes(w.B, w.L, w.D, w.N, t["u"].dtype)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def run():
        mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"],
                      None, y=y, h_final=hf, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return float(np.median(ms)) * 1e3 / calls


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def fwd_entry(w, kern_s):
    """GB/s of algorithmic bytes and the fractions of the HBM and VALU bounds
    at kernel time `kern_s` seconds per forward."""
    return {"GBs": round(fwd_bytes(w) / kern_s / 1e9, 1),
            "hbm_frac": round(fwd_bytes(w) / kern_s / 1e9 / HBM_PEAK_GBS, 4),
            "valu_frac": round(SLOTS_PER_ELEM_STATE * w.elem_states / kern_s / 1e12 / VALU_PEAK_TOPS, 4),
            "elem_state_per_s": float(f"{w.elem_states / kern_s:.4e}")}


def copy_bandwidth(torch, reps=5):
    """Read + write bytes per second of a plain 1 GiB device-to-device copy."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return 2 * n / (float(np.median(ms)) / 1e3) / 1e9


def time_bwd(mssm, torch, w, steps, warmup):
    inp = workloads.make_inputs(w, with_dy=True)
    t = workloads.to_torch(inp, "cuda")
    del inp
    ws = torch.empty(mssm.bwd_workspace_bytes(w.B, w.L, w.D, w.N, t["u"].dtype), dtype=torch.uint8, device="cuda")

    def run():
        mssm.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["z"],
                      t["dt_bias"], None, None, want_dh0=False, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3


def time_train_pair(mssm, torch, w, steps, warmup):
    """The training pair: mssm_scan_fwd_train (the forward saving its context)
    and mssm_scan_bwd_saved (the backward from it).  Median seconds of each,
    HIP events on the launch stream, buffers allocated once."""
    inp = workloads.make_inputs(w, with_dy=True)
    t = workloads.to_torch(inp, "cuda")
    del inp
    act = t["u"].dtype
    y = torch.empty_like(t["u"])
    hf = torch.empty((w.B, w.D, w.N), dtype=torch.float32, device="cuda")
    ctx = torch.empty(mssm.ctx_bytes(w.B, w.L, w.D, w.N, act), dtype=torch.uint8, device="cuda")
    fws = torch.empty(max(1, mssm.fwd_workspace_bytes(w.B, w.L, w.D, w.N, act)), dtype=torch.uint8, device="cuda")
    prob = mssm.problem(w.B, w.L, w.D, w.N, act)
    bws = torch.empty(int(mssm.lib.mssm_scan_bwd_saved_workspace_bytes(ctypes.byref(prob))),
                      dtype=torch.uint8, device="cuda")

    def fwd():
        mssm.scan_fwd_train(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"],
                            y=y, h_final=hf, ctx=ctx, workspace=fws)

    def bwd():
        mssm.scan_bwd_saved(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, t["Dskip"], t["z"],
                            t["dt_bias"], want_dh0=False, workspace=bws)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for a, b, c in ev:
        a.record(stream)
        fwd()
        b.record(stream)
        bwd()
        c.record(stream)
    torch.cuda.synchronize()
    kf = float(np.median([a.elapsed_time(b) for a, b, _ in ev])) / 1e3
    kb = float(np.median([b.elapsed_time(c) for _, b, c in ev])) / 1e3
    return kf, kb


def time_conv_step(mssm, torch, w, batch, reps=100):
    """mssm_conv_step (conv front end + recurrent step, d_conv = 4) at batch
    `batch`, the workload's width: median us per call (HIP events)."""
    ww = workloads.custom(batch, 1, w.D, w.N, w.dtype, seed=w.seed)
    inp = workloads.make_inputs(ww)
    inp.update(workloads.conv_front_end(ww, 4))
    t = workloads.to_torch(inp, "cuda")
    state = torch.zeros((ww.B, ww.D, ww.N), dtype=torch.float32, device="cuda")
    cst = t["x_prev"].clone()
    args = [t["u"][:, 0].contiguous(), t["conv_w"], cst, t["delta"][:, 0].contiguous(), t["A"],
            t["Bm"][:, 0].contiguous(), t["Cm"][:, 0].contiguous(), state, t["Dskip"], t["z"][:, 0].contiguous(),
            t["dt_bias"]]
    y_t = torch.empty_like(args[0])
    for _ in range(10):
        mssm.conv_step(*args, conv_b=t["conv_b"], y_t=y_t)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        mssm.conv_step(*args, conv_b=t["conv_b"], y_t=y_t)
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3


def time_ssd(mssm, torch, B, L, H, N, reps=20, backward=False):
    """Mamba-2 (SSD) forward (or backward), head dim 64, float32: median us per
    call (HIP events), and the dense flops of the forward's chunked dual form at
    64-step chunks (C B^T, C S^T, M X, and the state update, as full 64 x 64
    products)."""
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=11)
    t = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    del inp
    y = torch.empty_like(t["x"])
    hf = torch.empty((B, H, 64, N), dtype=torch.float32, device="cuda")
    if backward:
        t["dy"] = torch.randn_like(t["x"])
        prob = mssm.binding.SsdProblem(B, L, H, 64, N, 0, 1)
        ws = torch.empty(int(mssm.lib.mssm_ssd_bwd_workspace_bytes(ctypes.byref(prob))), dtype=torch.uint8,
                         device="cuda")

    def run():
        if backward:
            mssm.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["dt_bias"], workspace=ws)
        else:
            mssm.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"], y=y, h_final=hf)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    Q, P = 64, 64
    flops = B * H * (-(-L // Q)) * 2 * (Q * Q * N + Q * P * N + Q * Q * P + Q * P * N)
    return us, flops


def time_ssd_train_pair(mssm, torch, B, L, H, N, reps=5):
    """The SSD training pair (mssm_ssd_fwd_train, then mssm_ssd_bwd_saved), head
    dim 64, float32: median us of the forward and of the backward."""
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=11)
    t = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    del inp
    t["dy"] = torch.randn_like(t["x"])
    y = torch.empty_like(t["x"])
    hf = torch.empty((B, H, 64, N), dtype=torch.float32, device="cuda")
    prob = mssm.binding.SsdProblem(B, L, H, 64, N, 0, 1)
    ctx = torch.empty(int(mssm.lib.mssm_ssd_ctx_bytes(ctypes.byref(prob))), dtype=torch.uint8, device="cuda")
    fws = torch.empty(max(1, int(mssm.lib.mssm_ssd_fwd_train_workspace_bytes(ctypes.byref(prob)))),
                      dtype=torch.uint8, device="cuda")
    bws = torch.empty(int(mssm.lib.mssm_ssd_bwd_saved_workspace_bytes(ctypes.byref(prob))), dtype=torch.uint8,
                      device="cuda")

    def fwd():
        mssm.ssd_fwd_train(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"], y=y, h_final=hf,
                           ctx=ctx, workspace=fws)

    def bwd():
        mssm.ssd_bwd_saved(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, t["Dskip"], t["dt_bias"],
                           workspace=bws)

    for _ in range(2):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for a, b, c in ev:
        a.record()
        fwd()
        b.record()
        bwd()
        c.record()
    torch.cuda.synchronize()
    return (float(np.median([a.elapsed_time(b) for a, b, _ in ev])) * 1e3,
            float(np.median([b.elapsed_time(c) for _, b, c in ev])) * 1e3)


def ssd_layers(mssm, torch):
    """The Mamba-2 (SSD) layers, float32 on the matrix cores: the 2.7B shape
    (80 heads of 64, d_state 128, B = 8, L = 2048) and the batch-1 prefill of
    a 24-head layer (time segments scanned in parallel), forward and backward
    (all eight gradients): median us per call."""
    r = {}
    ssd_us, ssd_flops = time_ssd(mssm, torch, 8, 2048, 80, 128)
    r["ssd_fwd_H80_N128_B8_L2048_us"] = round(ssd_us, 1)
    r["ssd_fwd_dense_TFLOPs"] = round(ssd_flops / ssd_us / 1e6, 1)
    r["ssd_fwd_H24_N128_B1_L2048_us"] = round(time_ssd(mssm, torch, 1, 2048, 24, 128)[0], 1)
    r["ssd_bwd_H80_N128_B8_L2048_us"] = round(time_ssd(mssm, torch, 8, 2048, 80, 128, 5, True)[0], 1)
    r["ssd_bwd_H24_N128_B1_L2048_us"] = round(time_ssd(mssm, torch, 1, 2048, 24, 128, 10, True)[0], 1)
    # the training pair: the forward keeps the chunk states, the backward skips its first pass over the chunks
    tf, tb = time_ssd_train_pair(mssm, torch, 8, 2048, 80, 128)
    r["ssd_fwd_train_H80_N128_B8_L2048_us"] = round(tf, 1)
    r["ssd_bwd_saved_H80_N128_B8_L2048_us"] = round(tb, 1)
    tf, tb = time_ssd_train_pair(mssm, torch, 1, 2048, 24, 128, 10)  # time segments in both
    r["ssd_fwd_train_H24_N128_B1_L2048_us"] = round(tf, 1)
    r["ssd_bwd_saved_H24_N128_B1_L2048_us"] = round(tb, 1)
    return r


def time_step(mssm, torch, w, reps=200, batch=None):
    """One recurrent step (decode) at the workload's width: (B, D) inputs, the
    (B, D, N) float32 state updated in place; `batch` overrides B (batched
    decode).  Returns (us per call, GB/s of algorithmic bytes: state read +
    write, inputs, y, A, Dskip, dt_bias)."""
    if batch is not None:
        w = workloads.custom(batch, 1, w.D, w.N, w.dtype, seed=w.seed)
    inp = workloads.make_inputs(workloads.custom(w.B, 1, w.D, w.N, w.dtype, seed=w.seed))
    t = workloads.to_torch(inp, "cuda")
    args = [t["u"][:, 0].contiguous(), t["delta"][:, 0].contiguous(), t["A"], t["Bm"][:, 0].contiguous(),
            t["Cm"][:, 0].contiguous()]
    z_t = t["z"][:, 0].contiguous()
    state = torch.zeros((w.B, w.D, w.N), dtype=torch.float32, device="cuda")
    y_t = torch.empty_like(z_t)
    for _ in range(10):
        mssm.step(*args, state, t["Dskip"], z_t, t["dt_bias"], y_t=y_t)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        mssm.step(*args, state, t["Dskip"], z_t, t["dt_bias"], y_t=y_t)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    act = 2 if w.dtype == "bf16" else 4
    nbytes = 8 * w.B * w.D * w.N + 4 * w.B * w.D * act + 2 * w.B * w.N * act + 4 * w.D * w.N + 8 * w.D
    return us, nbytes / (us * 1e-6) / 1e9


def time_step_bound(mssm, torch, w, reps=200, graph_steps=32):
    """The decode step over buffers bound once (binding.Stepper): us per call
    from Python, and us per step inside a replayed graph of `graph_steps`
    steps (no host work per step)."""
    inp = workloads.make_inputs(workloads.custom(w.B, 1, w.D, w.N, w.dtype, seed=w.seed))
    t = workloads.to_torch(inp, "cuda")
    b = {k: t[k][:, 0].contiguous() for k in ("u", "delta", "Bm", "Cm", "z")}
    state = torch.zeros((w.B, w.D, w.N), dtype=torch.float32, device="cuda")

    def bound():
        return mssm.Stepper(b["u"], b["delta"], t["A"], b["Bm"], b["Cm"], state, t["Dskip"], b["z"], t["dt_bias"])

    st = bound()
    for _ in range(10):
        st()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        st()
    e1.record()
    torch.cuda.synchronize()
    per_call = e0.elapsed_time(e1) / reps * 1e3
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        gs = bound()
        for _ in range(graph_steps):
            gs()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    n = 20
    e0.record()
    for _ in range(n):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return per_call, e0.elapsed_time(e1) / (n * graph_steps) * 1e3


def cpu_baseline(w: workloads.Workload, target_s: float = 12.0):
    """Oracle (float64 C, OpenMP) on a channel sample of the workload."""
    import oracle

    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(0)

    def run(ch):
        sub = workloads.as_float32(workloads.select_channels(inp, ch))
        t0 = time.perf_counter()
        oracle.scan_fwd(sub["u"], sub["delta"], sub["A"], sub["Bm"], sub["Cm"], sub["Dskip"], sub["z"],
                        sub["dt_bias"], None)
        return time.perf_counter() - t0

    probe = np.sort(rng.choice(w.D, 64, replace=False))
    tp = run(probe)
    nch = int(min(w.D, max(64, 64 * target_s / max(tp, 1e-3))))
    nch = max(64, nch // 64 * 64)
    ch = np.sort(rng.choice(w.D, nch, replace=False))
    # when the sample is the whole workload and still short, repeat it (median of the runs)
    times = [run(ch)]
    while sum(times) < target_s and len(times) < 30:
        times.append(run(ch))
    dt = float(np.median(times))
    frac = nch / w.D
    gbs = fwd_bytes(w) * frac / dt / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "sample": f"{nch} of {w.D} channels of the {w.name} workload (B={w.B}, L={w.L}, full sequence), "
                      f"median of {len(times)} runs of {dt:.2f} s ({sum(times):.1f} s in all); "
                      f"elem_state_per_s={w.B * w.L * nch * w.N / dt:.3e}"}


def other_configs(mssm, torch):
    """The other workloads, timed with HIP events on the launch stream (median
    launch; cold = after a 512 MB scratch write)."""
    cfg = {}
    tw = workloads.WORKLOADS["tiny"]
    _, tl, _ = time_fwd(mssm, torch, tw, 200, 20)
    cfg["tiny"] = {"fwd_us_per_call": round(float(np.median(tl)) * 1e3, 2)}
    try:
        cfg["tiny"]["fwd_us_in_graph"] = round(time_fwd_graph(mssm, torch, tw), 2)
    except RuntimeError as e:  # graph capture unavailable: the per-call figure stands alone
        log(f"tiny: graph timing skipped ({e})")
    log("configs: tiny timed")
    w = workloads.WORKLOADS["130m"]
    _, ml, cl = time_fwd(mssm, torch, w, 20, 3, cold_reps=3)
    k = float(np.median(ml)) / 1e3
    cfg["130m"] = dict(fwd_us=round(k * 1e6, 1), fwd_us_cold=round(float(np.median(cl)) * 1e3, 1), **fwd_entry(w, k))
    log("configs: 130m timed")
    w = workloads.WORKLOADS["long"]
    _, ml, _ = time_fwd(mssm, torch, w, 3, 1)
    k = float(np.median(ml)) / 1e3
    cfg["long"] = dict(fwd_us=round(k * 1e6, 1), **fwd_entry(w, k))
    log("configs: long timed")
    w = workloads.WORKLOADS["train"]
    _, ml, _ = time_fwd(mssm, torch, w, 20, 3)
    kf = float(np.median(ml)) / 1e3
    kb = time_bwd(mssm, torch, w, 10, 2)
    cfg["train"] = {"fwd_us": round(kf * 1e6, 1), "bwd_us": round(kb * 1e6, 1),
                    "fwd_bwd_us": round((kf + kb) * 1e6, 1),
                    "bwd_GBs": round(bwd_bytes(w) / kb / 1e9, 1),
                    "fwd_bwd_GBs": round((fwd_bytes(w) + bwd_bytes(w)) / (kf + kb) / 1e9, 1),
                    "fwd_bwd_hbm_frac": round((fwd_bytes(w) + bwd_bytes(w)) / (kf + kb) / 1e9 / HBM_PEAK_GBS, 4)}
    # the training pair: the forward saves the tile states and the pre-gate readout, the backward starts from them
    tf, tb = time_train_pair(mssm, torch, w, 10, 2)
    cfg["train"].update({"fwd_train_us": round(tf * 1e6, 1), "bwd_saved_us": round(tb * 1e6, 1),
                         "fwd_bwd_saved_us": round((tf + tb) * 1e6, 1),
                         "fwd_bwd_saved_GBs": round((fwd_bytes(w) + bwd_bytes(w)) / (tf + tb) / 1e9, 1),
                         "fwd_bwd_saved_hbm_frac": round((fwd_bytes(w) + bwd_bytes(w)) / (tf + tb) / 1e9
                                                         / HBM_PEAK_GBS, 4)})
    log("configs: train fwd + bwd timed")
    return cfg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="2.8b", choices=["2.8b", "130m", "long", "tiny", "train"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="only the headline workload")
    ap.add_argument("--extra", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--ssd", action="store_true", help="only the Mamba-2 (SSD) layers (their own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the selective-scan library has no multi-GPU path; "
              "it would shard by channel (and by time for long sequences) with one GPU's share "
              "being exactly this single-GPU workload.", file=sys.stderr)
        sys.exit(2)

    import torch

    import selective_state_space_mssm_amd as mssm

    if args.ssd:
        print(json.dumps({"ssd": ssd_layers(mssm, torch)}), flush=True)
        return
    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 3 x 1 GiB device copies done")

    w = workloads.WORKLOADS[args.workload]
    log(f"workload {workloads.DESCRIPTIONS[w.name]}; steps {args.steps}, warmup {args.warmup}")
    wall, launch_ms, cold_ms = time_fwd(mssm, torch, w, args.steps, args.warmup, cold_reps=5)
    log(f"forward timed: {wall * 1e6:.1f} us per step")
    copy_gbs = copy_bandwidth(torch)
    nbytes = fwd_bytes(w)
    gbs = nbytes / wall / 1e9
    kern_s = float(np.mean(launch_ms)) / 1e3
    cold_s = float(np.median(cold_ms)) / 1e3
    slots = SLOTS_PER_ELEM_STATE * w.elem_states
    achieved = slots / kern_s / 1e12
    out = {
        "metric": "selective-scan fwd/bwd GB/s & % HBM peak (B·L·D·N elem/s) on 1 MI355X",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "act_dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": workloads.DESCRIPTIONS[w.name], "B": w.B, "L": w.L, "D": w.D, "N": w.N,
                   "act_storage": w.dtype, "direction": "fwd"},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "elem_state_per_s": float(f"{w.elem_states / wall:.4e}"),
        "roofline": {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": round(VALU_PEAK_TOPS, 3),
            "unit": "T FMA-lane slots/s",
            "frac": round(achieved / VALU_PEAK_TOPS, 4),
            "traffic": measured_traffic() if w.name == "2.8b" else None,
            "kernel": "scan_fwd_kernel",
            "kernel_us": round(kern_s * 1e6, 2),
            "work_per_launch": f"{SLOTS_PER_ELEM_STATE} VALU slots x {w.elem_states} (b,t,d,n)",
            "kernel_us_median": round(float(np.median(launch_ms)) * 1e3, 2),
            "kernel_us_min": round(float(np.min(launch_ms)) * 1e3, 2),
            "kernel_us_cold": round(float(np.median(cold_ms)) * 1e3, 2),
            "hbm_achieved_GBs": round(nbytes / kern_s / 1e9, 1),
            "hbm_peak_GBs": HBM_PEAK_GBS,
            "copy_GBs": round(copy_gbs, 1),
            "frac_of_copy": round(nbytes / kern_s / 1e9 / copy_gbs, 4),
            "hbm_frac": round(nbytes / kern_s / 1e9 / HBM_PEAK_GBS, 4),
            "note": "frac is against the fp32 VALU bound, 157.3 TFLOP/s (the binding one); hbm_frac against 8 TB/s",
        },
        # cold: each launch after a 512 MB scratch write has evicted the inputs from the last-level cache
        "cold": {"kernel_us": round(cold_s * 1e6, 2), "GBs": round(nbytes / cold_s / 1e9, 1),
                 "hbm_frac": round(nbytes / cold_s / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_configs:
        out["configs"] = other_configs(mssm, torch)
    if args.extra:
        _, cl, _ = time_fwd(mssm, torch, w, 20, 3, conv=True)
        conv_us = float(np.median(cl)) * 1e3
        out.setdefault("extra", {})["conv_fwd_us"] = round(conv_us, 1)   # median kernel time, fused front end
        out["extra"]["conv_fwd_GBs"] = round(conv_fwd_bytes(w) / conv_us / 1e3, 1)
        out["extra"]["conv_fwd_vs_plain_median"] = round(conv_us / (float(np.median(launch_ms)) * 1e3), 3)
        log("extra: fused conv forward timed")
        cb_us = time_conv_bwd(mssm, torch, w)
        out["extra"]["conv_bwd_us"] = round(cb_us, 1)   # median, backward of the conv front end
        out["extra"]["conv_bwd_GBs"] = round(conv_bwd_bytes(w) / cb_us / 1e3, 1)
        st_us, st_gbs = time_step(mssm, torch, w)
        out.setdefault("extra", {})["step_us_per_call"] = round(st_us, 2)
        out["extra"]["step_GBs_per_call"] = round(st_gbs, 1)
        bound_us, graph_us = time_step_bound(mssm, torch, w)  # bound buffers; and inside a replayed graph
        out["extra"]["step_us_per_call_bound"] = round(bound_us, 2)
        out["extra"]["step_us_in_graph"] = round(graph_us, 2)
        for bb in (64, 256):  # batched decode: the state read and write dominate
            st_us, st_gbs = time_step(mssm, torch, w, reps=100, batch=bb)
            out["extra"][f"step_B{bb}_us_per_call"] = round(st_us, 2)
            out["extra"][f"step_B{bb}_GBs"] = round(st_gbs, 1)
        out["extra"]["conv_step_B256_us"] = round(time_conv_step(mssm, torch, w, 256), 2)  # conv front end + step
        # a few tokens over many rows (the forward's short-sequence path): B = 256, 4 tokens
        sw = workloads.custom(256, 4, w.D, w.N, w.dtype, seed=w.seed)
        _, sl, _ = time_fwd(mssm, torch, sw, 30, 3)
        out["extra"]["short_fwd_B256_L4_us"] = round(float(np.median(sl)) * 1e3, 1)
        log("extra: conv backward, decode steps and short-sequence forward timed")
        out["extra"].update(ssd_layers(mssm, torch))
        log("extra: SSD forwards and backwards timed")
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
