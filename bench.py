#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full layer call (router logits, top-k + gates, permutation with
counts and LIS, grouped gate/up GEMM, grouped down GEMM, shared experts when
the layer has them, combine) on one batch of seeded synthetic input that is
already resident in HBM.  The primary line is the Mixtral-8x7B-shaped prefill
(T=4096, d=4096, E=8, top-2, SwiGLU d_ff=14336, bf16); the Mixtral decode
(T=16) and the INT4-expert decode (T=64) are reported alongside in the same
JSON line.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import ctypes as C
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 157.3
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_wavefront_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_hbm_traffic.md")
# sources whose text fixes each dominant kernel; a counter record taken from other text is void
KERNEL_SOURCES = {"grouped_gemm": ("grouped_ffn.hip", "moe_internal.h"),
                  "stream_ffn": ("stream_ffn.hip", "moe_internal.h")}
COPY_CAL_BYTES = 1 << 30


def _hip():
    h = C.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
    h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    h.hipEventSynchronize.argtypes = [C.c_void_p]
    h.hipEventDestroy.argtypes = [C.c_void_p]
    return h


def work(cfg, counts):
    """Algorithmic FLOPs and bytes of the layer and of its two GEMM kernels.

    Counts only active experts' weights; excludes the H and y_rows round trips
    (implementation traffic, reported by the counters instead)."""
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F
    rows = T * k
    active = int(np.count_nonzero(counts))
    swiglu = cfg.act == "swiglu"
    esz = 4 if cfg.dtype == "f32" else 2
    wsz = (0.5 + 2 * 2 / 128) if cfg.int4 else esz     # INT4: nibble + fp16 s,z per 128
    gu_mats = 2 if swiglu else 1
    gu_flops = 2.0 * rows * d * F * gu_mats
    dn_flops = 2.0 * rows * d * F
    gu_bytes = active * gu_mats * F * d * wsz + T * d * esz
    dn_bytes = active * F * d * wsz + rows * d * 4
    flops = gu_flops + dn_flops + 2.0 * T * d * E
    wbytes = active * (gu_mats + 1) * F * d * wsz
    if cfg.n_shared:
        Fs = cfg.n_shared * cfg.F_shared
        flops += 2.0 * T * d * Fs * 3
        wbytes += 3.0 * Fs * d * esz
    total_bytes = wbytes + E * d * esz + T * d * esz + T * d * 4
    return dict(flops=flops, bytes=total_bytes, gu_flops=gu_flops, dn_flops=dn_flops,
                gu_bytes=gu_bytes, dn_bytes=dn_bytes, active=active)


def work_mwq(cfg, counts3):
    """Algorithmic bytes of the nested-expert layer: per active expert, the 2-bit
    codes with s2, z2, plus each residual plane (1 bit, fp16 magnitude per 128)
    that one of its rows' widths needs; token rows and gate-scaled outputs as in
    work()."""
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F
    c = np.asarray(counts3).reshape(E, 3)
    gu_mats = 2 if cfg.act == "swiglu" else 1
    per_w = np.zeros(E)
    for e in range(E):
        if c[e].sum() == 0:
            continue
        per_w[e] = 0.25 + 4.0 / 128                      # codes, s2, z2
        if c[e, 1] + c[e, 2] > 0:
            per_w[e] += 0.125 + 2.0 / 128                # plane 3, a3
        if c[e, 2] > 0:
            per_w[e] += 0.125 + 2.0 / 128                # plane 4, a4
    wsum = float(per_w.sum())
    gu_bytes = wsum * gu_mats * F * d + T * d * 2
    dn_bytes = wsum * F * d + T * k * d * 4
    widths = {str(b): int(c[:, b - 2].sum()) for b in (2, 3, 4)}
    return dict(gu_bytes=gu_bytes, dn_bytes=dn_bytes, widths=widths,
                active=int(np.count_nonzero(c.sum(axis=1))),
                bytes=wsum * (gu_mats + 1) * F * d + E * d * 2 + T * d * 2 + T * d * 4)


def work_floe(cfg, counts, nnz):
    """Algorithmic bytes of the sparse-down layer: per active expert the INT2 up
    projection (2 bits + fp16 s2, z2 per 128) and, for the channels some row
    keeps, the gate rows and down columns in bf16."""
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F
    active = np.asarray(counts) > 0
    nz = np.asarray(nnz, np.float64) * active
    up = float(active.sum()) * F * d * (0.25 + 4.0 / 128)
    gate = float(nz.sum()) * d * 2
    down = float(nz.sum()) * d * 2
    return dict(gu_bytes=up + gate + T * d * 2, dn_bytes=down + T * k * d * 4,
                bytes=up + gate + down + E * d * 2 + T * d * 2 + T * d * 4,
                kept_channels=[int(v) for v in np.asarray(nnz)],
                dense_bf16_bytes=float(active.sum()) * 3 * F * d * 2)


FLUSH_BYTES = 512 << 20   # read before each cold step: more than the 256 MB MALL
# (read, not written: a written flush leaves dirty lines behind whose write-back
# the first kernel of the step would pay for)


def run_gpu(name, steps, warmup, cold=False, flags=0):
    """Warm wall-clock timing of `steps` back-to-back layer calls, then one
    event-timed pass per step (per-stage HIP events).  With cold=True a 512 MB
    buffer is read before each event-timed step, outside its events, so the
    weights start from HBM rather than the MALL."""
    import torch
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd.device_inputs import (floe_to_device, mwq_to_device,
                                                                    to_device)
    from workloads import make_workload
    wl = make_workload(name)
    cfg = wl.cfg
    layer, x = to_device(wl)
    if cfg.mwq:
        ex, widths = mwq_to_device(wl)
        runner = moe.LayerRunner(layer, cfg.T, mwq=ex)

        def call():
            return runner(x, widths=widths)
    elif cfg.floe:
        runner = moe.LayerRunner(layer, cfg.T, floe=floe_to_device(wl))

        def call():
            return runner(x)
    else:
        runner = moe.LayerRunner(layer, cfg.T)

        def call():
            return runner(x, flags)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1000.0 / steps
    counts = runner.aux_t["counts"].cpu().numpy()
    lis = float(runner.aux_t["lis"].cpu().numpy()[0])

    # Per-stage durations from HIP events that the library records on the stream it
    # launches on (torch's current stream).  One event set per step, no host sync
    # inside the loop, so the stages run back to back as in the timed loop above.
    hip = _hip()
    sets = []
    for _ in range(steps):
        hs = []
        for i in range(7):
            h = C.c_void_p()
            assert hip.hipEventCreate(C.byref(h)) == 0
            hs.append(h.value)
        sets.append((C.c_void_p * 7)(*hs))
    B = moe.lib()
    per = np.zeros((steps, 7))
    flush = None
    if cold:
        flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=x.device)
        flush.sum()
        torch.cuda.synchronize()
    try:
        for n, evs in enumerate(sets):
            if cold:
                flush.sum()
            B.moe_set_stage_events(C.cast(evs, C.POINTER(C.c_void_p)), 7)
            call()
        B.moe_set_stage_events(None, 0)
        torch.cuda.synchronize()
        for n, evs in enumerate(sets):
            for i in range(6):
                f = C.c_float(0)
                assert hip.hipEventElapsedTime(C.byref(f), evs[i], evs[i + 1]) == 0
                per[n, i] = f.value
            f = C.c_float(0)
            assert hip.hipEventElapsedTime(C.byref(f), evs[0], evs[6]) == 0
            per[n, 6] = f.value
    finally:
        B.moe_set_stage_events(None, 0)
        for evs in sets:
            for i in range(7):
                hip.hipEventDestroy(evs[i])
    st = per[:, :6].mean(axis=0)
    layer_ms = per[:, 6]
    if cold:
        # the cold layer time from two events per step only (the stage events
        # above add their own overhead between the stages)
        ev = []
        for _ in range(steps):
            pair = []
            for _ in range(2):
                h = C.c_void_p()
                assert hip.hipEventCreate(C.byref(h)) == 0
                pair.append(h.value)
            ev.append(pair)
        hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        try:
            for n, (a, b) in enumerate(ev):
                flush.sum()
                assert hip.hipEventRecord(C.c_void_p(a), stream) == 0
                call()
                assert hip.hipEventRecord(C.c_void_p(b), stream) == 0
            torch.cuda.synchronize()
            cold_ms = []
            for a, b in ev:
                f = C.c_float(0)
                assert hip.hipEventElapsedTime(C.byref(f), C.c_void_p(a), C.c_void_p(b)) == 0
                cold_ms.append(f.value)
        finally:
            for a, b in ev:
                hip.hipEventDestroy(C.c_void_p(a))
                hip.hipEventDestroy(C.c_void_p(b))
        layer_ms = np.asarray(cold_ms)
    w = work(cfg, counts)
    if cfg.mwq:
        w.update(work_mwq(cfg, runner.aux_t["mwq_counts"].cpu().numpy()))
    if cfg.floe:
        w.update(work_floe(cfg, counts, runner.aux_t["floe_nnz"].cpu().numpy()))
    stages = dict(zip(["route_topk", "permute", "gate_up_gemm", "down_gemm", "shared_experts",
                       "combine"], [round(v * 1000.0, 2) for v in st]))
    timing = dict(event_ms_p10=round(float(np.percentile(layer_ms, 10)), 4),
                  event_ms_p50=round(float(np.percentile(layer_ms, 50)), 4),
                  event_ms_p90=round(float(np.percentile(layer_ms, 90)), 4))
    del flush
    return wl, dict(ms=ms, counts=counts, lis=lis, stages_us=stages, work=w, timing=timing,
                    cold=cold, event_ms=float(layer_ms.mean()))


def sources_sha256(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of the gate/up kernel from committed rocprofv3 counter runs.

    Records are lines 'traffic_record {json}' in the profile summary; each holds
    FETCH_SIZE and WRITE_SIZE per dispatch already scaled by the copy-kernel factor,
    and the sha256 of the kernel's sources when the counters were taken.  A record
    whose hash differs from the current sources is stale and gives None."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    cur = sources_sha256(kernel)
    for ln in lines:
        if not ln.startswith("traffic_record "):
            continue
        rec = json.loads(ln[len("traffic_record "):])
        if rec.get("workload") == workload and rec.get("kernel") == kernel:
            if rec.get("sources_sha256") != cur:
                return None
            return round(float(rec["read_bytes"]) + float(rec["write_bytes"]))
    return None


_ATOMIC_WL = {}


def run_atomic(spec, steps, warmup):
    """The atomic-expert layer (router grid, exact top-K, expert grouping, then
    the schedule's input and output sides, shared MLP, combine), per-stage HIP
    events as in run_gpu.  `spec` is a workload name, optionally ':' and a
    schedule (auto, dense, expert_centric)."""
    import torch
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd.device_inputs import atomic_to_device
    from workloads import make_workload
    name, _, schedule = spec.partition(":")
    schedule = schedule or "auto"
    if name not in _ATOMIC_WL:
        _ATOMIC_WL.clear()
        _ATOMIC_WL[name] = make_workload(name)
    wl = _ATOMIC_WL[name]
    cfg = wl.cfg
    layer, x = atomic_to_device(wl, schedule=schedule)
    runner = moe.AtomicRunner(layer, cfg.T)
    resolved = runner.schedule_used()
    for _ in range(warmup):
        runner(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        runner(x)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    hip = _hip()
    B = moe.lib()
    per = np.zeros((steps, 7))
    sets = []
    try:
        for _ in range(steps):
            hs = []
            for i in range(7):
                h = C.c_void_p()
                assert hip.hipEventCreate(C.byref(h)) == 0
                hs.append(h.value)
            sets.append((C.c_void_p * 7)(*hs))
        for evs in sets:
            B.moe_set_stage_events(C.cast(evs, C.POINTER(C.c_void_p)), 7)
            runner(x)
        B.moe_set_stage_events(None, 0)
        torch.cuda.synchronize()
        for n, evs in enumerate(sets):
            for i in range(6):
                f = C.c_float(0)
                assert hip.hipEventElapsedTime(C.byref(f), evs[i], evs[i + 1]) == 0
                per[n, i] = f.value
            f = C.c_float(0)
            assert hip.hipEventElapsedTime(C.byref(f), evs[0], evs[6]) == 0
            per[n, 6] = f.value
    finally:
        B.moe_set_stage_events(None, 0)
        for evs in sets:
            for i in range(7):
                hip.hipEventDestroy(evs[i])
    st = per[:, :6].mean(axis=0)
    ec = resolved == "expert_centric"
    stages = dict(zip(["route_grid_topk", "permute",
                       "input_expert_centric" if ec else "input_gemm_masked",
                       "output_expert_centric" if ec else "output_gemm",
                       "shared_mlp", "reduce" if ec else "combine"],
                      [round(v * 1000.0, 2) for v in st]))
    T, d, N, K = cfg.T, cfg.d, cfg.nr * cfg.nc, cfg.k
    counts = runner.aux_t["counts"].cpu().numpy()
    active = int(np.count_nonzero(counts))
    dense_flops = 2.0 * T * N * d
    method_flops = 2.0 * T * K * d     # per side: each kept (token, unit) pair, one d-long dot
    t_in = st[2] * 1e-3
    line = {"workload": name, "schedule": resolved, "T": T, "d_model": d, "experts": N,
            "top_k": K, "active_experts": active,
            "tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
            "lis": float(runner.aux_t["lis"].cpu().numpy()[0]),
            "useful_fraction_of_dense_gemm": round(K / N, 4),
            "stages_us": stages,
            "timing": dict(event_ms_p50=round(float(np.percentile(per[:, 6], 50)), 4))}
    if ec:
        # expert-centric input side: the input vectors of the experts some token
        # kept, each read once, plus x
        in_bytes = active * d * 2.0 + T * d * 2.0
        ach = in_bytes / t_in / 1e9
        line["roofline"] = dict(kernel="atomic_ec_in (kept experts' w_in read once, v_dot2)",
                                bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS,
                                unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4), traffic=None,
                                per_launch=dict(bytes=in_bytes, us=round(t_in * 1e6, 2)),
                                method_flops_rate=dict(
                                    flops=method_flops,
                                    tflops=round(method_flops / t_in / 1e12, 2)))
    else:
        ach = method_flops / t_in / 1e12
        line["roofline"] = dict(
            kernel="grouped_gemm_tile<kAtomIn> (dense x . W_in^T, masked epilogue)",
            bound="mfma", achieved=round(ach, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
            frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4), traffic=None,
            per_launch=dict(flops=method_flops, us=round(t_in * 1e6, 2)),
            dense_gemm_rate=dict(flops=dense_flops, tflops=round(dense_flops / t_in / 1e12, 1),
                                 note="all T x N cells computed; only the K kept per token "
                                      "are used"))
    return line


def run_replica(name, steps, warmup):
    """The layer with an INT4 replica of its heaviest expert (chosen by a
    calibration call on the same batch) against the plain layer."""
    import torch
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd.device_inputs import replica_to_device, to_device
    from workloads import make_replica, make_workload
    wl = make_workload(name)
    cfg = wl.cfg
    layer, x = to_device(wl)

    def timed(runner):
        for _ in range(warmup):
            runner(x)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            runner(x)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / steps
    plain = moe.LayerRunner(layer, cfg.T)
    ms_plain = timed(plain)
    counts = plain.aux_t["counts"].cpu().numpy()
    heavy = int(np.flatnonzero(counts == counts.max())[0])
    rep = replica_to_device(make_replica(wl, heavy))
    split = moe.LayerRunner(layer, cfg.T, replica=rep)
    ms_rep = timed(split)
    c2 = split.aux_t["counts"].cpu().numpy()
    return {"workload": name, "T": cfg.T, "E": cfg.E, "top_k": cfg.k, "heavy_expert": heavy,
            "heavy_rows": int(counts[heavy]), "rows_after": [int(c2[heavy]), int(c2[-1])],
            "lis_before": float(split.lis_base.cpu().numpy()[0]),
            "lis_after": float(split.aux_t["lis"].cpu().numpy()[0]),
            "tokens_per_s_plain": round(cfg.T / (ms_plain / 1e3), 1),
            "tokens_per_s_replica": round(cfg.T / (ms_rep / 1e3), 1),
            "ms_plain": round(ms_plain, 4), "ms_replica": round(ms_rep, 4)}


def roofline(cfg, r):
    w = r["work"]
    t = r["stages_us"]["gate_up_gemm"] * 1e-6
    if cfg.floe:
        ach = w["gu_bytes"] / t / 1e9
        return dict(kernel="sparse-down up+gate (INT2 up, kept gate rows)", bound="hbm",
                    achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4), traffic=None,
                    per_launch=dict(bytes=w["gu_bytes"], us=round(t * 1e6, 2)))
    if cfg.mwq:
        ach = w["gu_bytes"] / t / 1e9
        return dict(kernel="mwq_stream gate/up (nested 2/3/4-bit table decode)", bound="hbm",
                    achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4), traffic=None,
                    per_launch=dict(bytes=w["gu_bytes"], us=round(t * 1e6, 2)))
    if cfg.dtype == "f32":             # fp32 layers run on the vector ALUs
        ach = w["gu_flops"] / t / 1e12
        return dict(kernel="ffn_f32_up (fp32 VALU gate/up)", bound="alu",
                    achieved=round(ach, 3), peak=FP32_VALU_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / FP32_VALU_PEAK_TFLOPS, 5), traffic=None,
                    per_launch=dict(flops=w["gu_flops"], us=round(t * 1e6, 2)))
    if cfg.T * cfg.k >= 1024:          # many rows per expert: the GEMM is MFMA-bound
        ach = w["gu_flops"] / t / 1e12
        return dict(kernel="grouped_gemm gate/up (SwiGLU epilogue)", bound="mfma",
                    achieved=round(ach, 1), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                    traffic=measured_traffic(cfg.name, "grouped_gemm"),
                    per_launch=dict(flops=w["gu_flops"], us=round(t * 1e6, 2)))
    ach = w["gu_bytes"] / t / 1e9
    return dict(kernel="grouped_gemm gate/up (weight streaming)", bound="hbm",
                achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4),
                traffic=measured_traffic(cfg.name, "stream_ffn"),
                per_launch=dict(bytes=w["gu_bytes"], us=round(t * 1e6, 2)))


def host_cpu_model():
    """The host CPU's model name (lscpu's "Model name", read from /proc/cpuinfo)."""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, target_s=15.0):
    """The oracle (as it stands) on a bounded sample: the first S tokens as a batch."""
    import oracle
    cfg = wl.cfg
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))

    def sample(S):
        c = dataclasses.replace(cfg, T=S)
        return dataclasses.replace(wl, cfg=c, x=wl.x[:S].copy())
    S = min(cfg.T, 8)
    t0 = time.perf_counter()
    oracle.layer_forward(sample(S))
    dt = time.perf_counter() - t0
    S2 = int(min(cfg.T, max(S, S * target_s / max(dt, 1e-3))))
    if S2 > S:
        S = S2
        t0 = time.perf_counter()
        oracle.layer_forward(sample(S))
        dt = time.perf_counter() - t0
    return dict(value=round(S / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                host=host_cpu_model(),
                sample="first %d of %d tokens as one batch, whole layer (router, top-k, "
                       "permutation, FFN, combine), fp64 C oracle, %.1f s" % (S, cfg.T, dt))


# HBM-bound workloads are timed from a cold cache (a 512 MB read before each
# step); the Switch-shaped layer, whose 75 MB of weights fit in the MALL, is
# reported both warm and cold
COLD = {"mixtral_decode_bf16": ("cold",), "mixtral_int4_decode": ("cold",),
        "mixtral_mwq_decode": ("cold",), "mixtral_floe_decode": ("cold",),
        "mixtral_floe_decode_t1": ("cold",), "switch_bf16": ("warm", "cold")}


def secondary_lines(name, steps, warmup, oracle_s):
    """One line per cache state of a workload: tokens/s, stage times and the
    gate/up roofline from the event-timed pass (cold) or the wall clock
    (warm), plus the oracle timed on the host beside it."""
    modes = COLD.get(name, ("warm",))
    wl, r = run_gpu(name, steps, warmup, cold="cold" in modes)
    rw = None
    if "warm" in modes and "cold" in modes:
        _, rw = run_gpu(name, steps, warmup, cold=False)
    c = wl.cfg
    lines = []
    for mode in modes:
        rr = rw if (mode == "warm" and rw is not None) else r
        ms = rr["event_ms"] if mode == "cold" else rr["ms"]
        gbs = rr["work"]["bytes"] / (ms * 1e-3) / 1e9
        lines.append({"workload": name, "cache": mode, "T": c.T,
                      "tokens_per_s": round(c.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
                      "lis": rr["lis"], "active_experts": rr["work"]["active"],
                      "layer_tflops": round(rr["work"]["flops"] / (ms * 1e-3) / 1e12, 2),
                      "layer_GBps": round(gbs, 1), "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "stages_us": rr["stages_us"], "timing": rr["timing"],
                      "roofline": roofline(c, rr)})
    if oracle_s > 0:
        base = cpu_baseline(wl, target_s=oracle_s)
        for ln in lines:
            ln["cpu_baseline"] = base
    del wl
    return lines


def vendor_gate_up(name, steps, warmup, lib_gate_up_us=None):
    """The same gate/up work through the vendor GEMM library, for comparison.

    torch's bf16 F.linear (hipBLASLt) on the rows the library's own routing
    gives: one GEMM per expert with its gate and up rows concatenated ([2F][d],
    built once, not timed), alone, and as a pipeline doing the step's whole
    work -- gather of the expert-major rows, the GEMMs, silu(g) * u to bf16.
    Beside them the library's fused gate/up launch (stage events of the same
    layer), all warm wall-clock means on the same box."""
    import torch
    import torch.nn.functional as Fn
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd.device_inputs import to_device
    from workloads import make_workload
    wl = make_workload(name)
    cfg = wl.cfg
    if cfg.act != "swiglu" or cfg.dtype != "bf16" or cfg.int4:
        return None
    layer, x = to_device(wl)
    runner = moe.LayerRunner(layer, cfg.T)
    runner(x)
    torch.cuda.synchronize()
    offs = runner.aux_t["offsets"].cpu().tolist()
    tok = (runner.aux_t["row_assign"][:cfg.T * cfg.k].long() // cfg.k).contiguous()
    wg, wu = layer.routed.w_gate, layer.routed.w_up
    wc = [torch.cat([wg[e], wu[e]], 0).contiguous() for e in range(cfg.E)]
    F = cfg.F

    def gemms():
        for e in range(cfg.E):
            a, b = offs[e], offs[e + 1]
            if b > a:
                Fn.linear(x[:b - a], wc[e])

    def pipeline():
        xs = x.index_select(0, tok)
        for e in range(cfg.E):
            a, b = offs[e], offs[e + 1]
            if b > a:
                gu = Fn.linear(xs[a:b], wc[e])
                Fn.silu(gu[:, :F]) * gu[:, F:]

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / steps

    g_ms, p_ms = timed(gemms), timed(pipeline)
    del wc
    if lib_gate_up_us is None:  # not the headline workload: time the library's launch here
        lib_gate_up_us = run_gpu(name, steps, warmup)[1]["stages_us"]["gate_up_gemm"]
    return {"workload": name, "vendor_gemms_ms": round(g_ms, 4), "vendor_pipeline_ms": round(p_ms, 4),
            "library_gate_up_ms": round(lib_gate_up_us / 1000.0, 4),
            "note": "torch F.linear (hipBLASLt) per expert, gate and up rows concatenated; "
                    "pipeline = gather + GEMMs + silu(g)*u; library = the fused gate/up launch"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill_bf16")
    ap.add_argument("--secondary",
                    default="mixtral_decode_bf16,mixtral_int4_decode,deepseek_v2_lite_bf16,"
                            "switch_bf16,tiny_fp32",
                    help="comma-separated extra workloads reported in the same line ('' for none)")
    ap.add_argument("--oracle-seconds", type=float, default=4.0,
                    help="CPU seconds of oracle work timed beside each secondary workload "
                         "(0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bf16-rows", default="deepseek_v2_lite_bf16",
                    help="comma-separated workloads also run with MOE_F_BF16_ROWS (warm; '' for "
                         "none)")
    ap.add_argument("--replica", default="switch_bf16,deepseek_v2_lite_bf16",
                    help="comma-separated workloads also run with an INT4 replica of their "
                         "heaviest expert ('' for none)")
    ap.add_argument("--mwq", default="mixtral_mwq_decode",
                    help="comma-separated nested low-bit expert workloads reported in the "
                         "same line ('' for none)")
    ap.add_argument("--floe", default="mixtral_floe_decode,mixtral_floe_decode_t1",
                    help="comma-separated sparse-down workloads reported in the same line "
                         "('' for none)")
    ap.add_argument("--atomic",
                    default="omni_atomic,omni_atomic:expert_centric,omni_atomic_decode,"
                            "omni_atomic_decode:dense",
                    help="comma-separated atomic-expert workloads, each optionally with "
                         "':schedule' (auto, dense, expert_centric), reported in the same line "
                         "('' for none)")
    ap.add_argument("--vendor", default="mixtral_prefill_bf16",
                    help="workloads whose gate/up step is also timed through the vendor GEMM "
                         "library (comma-separated; '' for none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 5 times (the known-size kernel "
                         "that scales the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        import torch as _t
        a = _t.empty(COPY_CAL_BYTES, dtype=_t.uint8, device="cuda").fill_(1)
        b = _t.empty_like(a)
        _t.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        _t.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_CAL_BYTES, "copies": 5}), flush=True)
        return

    wl, r = run_gpu(args.workload, args.steps, args.warmup)
    cfg = wl.cfg
    value = cfg.T / (r["ms"] / 1000.0)
    out = {
        "metric": "MoE-layer tokens/sec at Mixtral shape; % MFMA peak (prefill) / % HBM BW (decode)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) random-init weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "n_experts": cfg.E,
                   "top_k": cfg.k, "d_ff": cfg.F, "act": cfg.act, "int4": cfg.int4,
                   "n_shared": cfg.n_shared, "parallelism": "none (1 GPU)"},
        "lis": r["lis"], "active_experts": r["work"]["active"],
        "layer_tflops": round(r["work"]["flops"] / (r["ms"] * 1e-3) / 1e12, 2),
        "stages_us": r["stages_us"],
        "timing": r["timing"],
        "roofline": roofline(cfg, r),
    }
    sec = []
    for name in [s for s in args.secondary.split(",") if s]:
        sec.extend(secondary_lines(name, args.steps, args.warmup, args.oracle_seconds))
    if sec:
        out["secondary"] = sec
    mw = []
    for name in [s for s in args.mwq.split(",") if s]:
        wl3, r3 = run_gpu(name, args.steps, args.warmup)
        c3 = wl3.cfg
        mw.append({"workload": name, "T": c3.T, "tokens_per_s": round(c3.T / (r3["ms"] / 1e3), 1),
                   "ms_per_step": round(r3["ms"], 4), "lis": r3["lis"],
                   "widths": r3["work"]["widths"], "active_experts": r3["work"]["active"],
                   "layer_GBps": round(r3["work"]["bytes"] / (r3["ms"] * 1e-3) / 1e9, 1),
                   "stages_us": r3["stages_us"], "timing": r3["timing"],
                   "roofline": roofline(c3, r3)})
        del wl3
    if mw:
        out["mwq"] = mw
    fl = []
    for name in [s for s in args.floe.split(",") if s]:
        wl4, r4 = run_gpu(name, args.steps, args.warmup)
        c4 = wl4.cfg
        w4 = r4["work"]
        fl.append({"workload": name, "T": c4.T, "tokens_per_s": round(c4.T / (r4["ms"] / 1e3), 1),
                   "ms_per_step": round(r4["ms"], 4), "lis": r4["lis"],
                   "kept_channels": w4["kept_channels"],
                   "bytes_vs_dense_bf16": round(w4["bytes"] / w4["dense_bf16_bytes"], 4),
                   "layer_GBps": round(w4["bytes"] / (r4["ms"] * 1e-3) / 1e9, 1),
                   "stages_us": r4["stages_us"], "timing": r4["timing"],
                   "roofline": roofline(c4, r4)})
        del wl4
    if fl:
        out["floe"] = fl
    atoms = [run_atomic(n, args.steps, args.warmup) for n in args.atomic.split(",") if n]
    _ATOMIC_WL.clear()
    if atoms:
        out["atomic"] = atoms
    reps = [run_replica(n, args.steps, args.warmup) for n in args.replica.split(",") if n]
    if reps:
        out["replica"] = reps
    rows16 = []
    for n in [n for n in args.bf16_rows.split(",") if n]:
        import sparse_mixture_experts_wavefront_amd as moe
        w32, r32 = run_gpu(n, args.steps, args.warmup)
        w16, r16 = run_gpu(n, args.steps, args.warmup, flags=moe.MOE_F_BF16_ROWS)
        rows16.append({"workload": n, "cache": "warm", "ms_fp32_rows": round(r32["ms"], 4),
                       "ms_bf16_rows": round(r16["ms"], 4),
                       "tokens_per_s_bf16_rows": round(w16.cfg.T / (r16["ms"] / 1000.0), 1),
                       "stages_us_fp32_rows": r32["stages_us"],
                       "stages_us_bf16_rows": r16["stages_us"]})
    if rows16:
        out["bf16_rows"] = rows16
    vend = [v for v in (vendor_gate_up(n, args.steps, args.warmup,
                                       r["stages_us"]["gate_up_gemm"] if n == args.workload else None)
                        for n in args.vendor.split(",") if n) if v]
    if vend:
        out["vendor_gate_up"] = vend
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
