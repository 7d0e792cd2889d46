#!/usr/bin/env python3
"""Throughput of the routed MoE layer on one MI355X.

Headline (``value``): decode, T = 1 token row per step, on the
Qwen3.5-35B-A3B-shaped layer (H=2048, 256 experts, top-8, I=512, a shared
expert of I=512; Q4_K gate/up, Q5_K down; seeded synthetic weights and tokens).
One step = one moe_layer_forward call (router + top-k + gate/up/SwiGLU + down +
slot-order combine).  Steps cycle through a pool of 64 token rows and through
16 copies of the weights at different addresses, so that neither a step's
routed experts nor a copy's router matrix and shared expert are served from
the 256 MB last-level cache left warm by earlier steps.  Exactly `--steps`
steps are captured in one HIP graph; after one untimed replay, one replay is
timed with stream events.

The other workloads of the layer, each its own JSON object, timed the same way
(one graph of exactly the stated number of steps):
  sharded_decode   T = 1, router_topk + the two 256/256 shards + the reduce;
  batched_decode   T = 32 rows, automatic path;
  zipf_prefill     T = 512 rows with Zipf-like expert load;
  prefill          T = 4096 rows, uniform router;
  sharded_prefill  T = 4096 rows in the two-shard mode;
  mxfp4            decode and prefill with MXFP4 expert weights;
  edges            RMSNorm before the layer and the partial reduce plus
                   residual after it, at T = 4096.
Per-kernel durations come from start/stop HIP events that the library attaches
to each kernel launch (moe_opts.kernel_events, hipExtLaunchKernel) in an eager
pass over the same workload.  The CPU-baseline leg times the oracle on the
host and compares each workload's GPU output with it (max|err|/RMS over a
stated sample of rows).

Run: python bench.py [--steps K] [--warmup W] [--gpus 1]
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

METRIC = ("MoE-layer tokens/s at T=1 and T=4096; % peak HBM BW (decode) / % MFMA (prefill)")
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak (fp8 x fp4 runs at the fp8 rate)
MX_TERMS = 3                    # MX-FP8 terms per token / h value on the MXFP4 MFMA path


# HBM bytes per launch of the roofline kernels, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, averaged over the bench's
# dispatches of that kernel), each multiplied by the calibration factor that the
# same counter gives for a plain device copy of known size (bench.py
# --copy-probe).  Keyed by the SHA-256 of the kernel's sources: when they change,
# the counters no longer describe the kernel and traffic is reported as null.
TRAFFIC = {
    # decode T=1, 280 dispatches: FETCH 5347.0 KiB x 1.99980, WRITE 18.1 KiB x 1.0
    "gemv_gateup": {"sources_sha256": "a0156ea4c49fe8856b2acbbfad167349df54fdecc42435744e4987386e9269e3",
                    "fetch_bytes": 10949472, "write_bytes": 18505},
    # prefill T=4096, 18 dispatches: FETCH 226176.6 KiB x 1.99980, WRITE 36864.0 KiB x 1.0
    "gemm_gateup": {"sources_sha256": "38c44c264ee3711088101b5964188bfb0a068286c3bf8ee0d684227a24fcfa10",
                    "fetch_bytes": 463163407, "write_bytes": 37748736},
    # MXFP4 decode T=1, 280 dispatches: FETCH 5365.6 KiB x 1.99980, WRITE 18.1 KiB x 1.0
    "gemv_gateup_mx": {"sources_sha256": "a0156ea4c49fe8856b2acbbfad167349df54fdecc42435744e4987386e9269e3",
                    "fetch_bytes": 10987668, "write_bytes": 18496},
    # MXFP4 prefill T=4096, 18 dispatches: FETCH 269652.6 KiB x 1.99980, WRITE 59906.3 KiB x 1.0
    "gemm_gateup_mx": {"sources_sha256": "a23e786497430292dc59f05cc49339feebce277ef6f4fb50273feff6ae084548",
                    "fetch_bytes": 552193244, "write_bytes": 61344089},
}
FETCH_SIZE_FACTOR = 1.99980   # plain 256 MiB copy: true bytes read / FETCH_SIZE bytes
WRITE_SIZE_FACTOR = 1.0
TRAFFIC_SOURCES = {
    "gemv_gateup": ["gemv.hip", "topk.h", "moe_internal.h"],
    "gemm_gateup": ["gemm.hip", "moe_internal.h"],
}
TRAFFIC_SOURCES["gemv_gateup_mx"] = TRAFFIC_SOURCES["gemv_gateup"]
TRAFFIC_SOURCES["gemm_gateup_mx"] = ["gemm_mx.hip", "moe_internal.h"]


def sources_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kernel]:
        with open(os.path.join(ROOT, "quantized_moe_transformer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# Matrix-core counters of the prefill gate/up GEMMs (profiles/gemm_*_prefill_T4096.md,
# rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_* GRBM_GUI_ACTIVE),
# keyed like TRAFFIC: mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x
# GRBM_GUI_ACTIVE / 8 XCDs); executed_flops = MOPS x 512 (padded rows included).
MFMA_COUNTERS = {
    "gemm_gateup": {"sources_sha256": "38c44c264ee3711088101b5964188bfb0a068286c3bf8ee0d684227a24fcfa10",
                    "mfma_busy": 0.3374, "executed_flops": 1.71262e+11},
    "gemm_gateup_mx": {"sources_sha256": "a23e786497430292dc59f05cc49339feebce277ef6f4fb50273feff6ae084548",
                    "mfma_busy": 0.3852, "executed_flops": 5.11772e+11},
}


def counters_for(kernel):
    t = MFMA_COUNTERS.get(kernel)
    if t is None or t["sources_sha256"] != sources_sha(kernel):
        return None
    return {k: v for k, v in t.items() if k != "sources_sha256"}


def traffic_for(kernel):
    t = TRAFFIC.get(kernel)
    if t is None or t["sources_sha256"] != sources_sha(kernel):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def copy_probe(torch, mib):
    """A plain device-to-device copy of known size, for calibrating the
    FETCH_SIZE / WRITE_SIZE counters (one torch copy kernel per call)."""
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "dispatches": 5}), flush=True)


class HipEvents:
    """hipEvent_t handles from libamdhip64 (torch's events only see torch's own
    stream bookkeeping; these are passed into the library call)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def array(self, i0, n):
        return (ctypes.c_void_p * n)(*self.ev[i0:i0 + n])

    def ms(self, a, b):
        f = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(self.ev[a]),
                                        ctypes.c_void_p(self.ev[b])) != 0:
            self.hip.hipGetLastError()   # clear the error it left for later launch checks
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_profile(torch, qm, call, n_steps, names, stats=None):
    """Average duration (ms) of each named kernel over n_steps eager calls, from
    start/stop events the library attaches to those launches (hipExtLaunchKernel
    records the dispatch's own begin/end).  `stats` (a dict, optional) receives
    each kernel's median and minimum as well."""
    from quantized_moe_transformer_amd._lib import KERNEL_IDS, N_KERNEL_IDS
    per_step = 2 * N_KERNEL_IDS
    ev = HipEvents(n_steps * per_step)
    for i in range(n_steps):
        call(i, ev.array(i * per_step, per_step))
    torch.cuda.synchronize()
    out = {}
    for n in names:
        kid = KERNEL_IDS[n]
        try:
            d = [ev.ms(i * per_step + 2 * kid, i * per_step + 2 * kid + 1) for i in range(n_steps)]
        except RuntimeError:
            continue   # a kernel this path does not launch (its events were never recorded)
        out[n] = float(np.mean(d))
        if stats is not None:
            stats[n] = {"median_ms": float(np.median(d)), "min_ms": float(np.min(d))}
    ev.close()
    return out


def time_steps(torch, run_step, K):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run_step(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def graph_time(torch, step, K):
    """Exactly K consecutive steps captured in ONE HIP graph; one untimed replay
    (graph upload), then one timed replay bracketed by synchronisations, timed
    by events on the replaying stream.  Returns (device s/step, host s/step)."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    host = time.perf_counter() - t0
    dev = a.elapsed_time(b) * 1e-3
    del g
    return dev / K, host / K


def kernel_profile_calls(torch, call, n_steps, n_calls, names, stats=None):
    """Like kernel_profile for a step made of n_calls library calls: call(i,
    evs) passes evs[c] to call c.  Returns {(c, name): average ms}."""
    from quantized_moe_transformer_amd._lib import KERNEL_IDS, N_KERNEL_IDS
    per = 2 * N_KERNEL_IDS
    ev = HipEvents(n_steps * n_calls * per)
    for i in range(n_steps):
        call(i, [ev.array((i * n_calls + c) * per, per) for c in range(n_calls)])
    torch.cuda.synchronize()
    out = {}
    for c in range(n_calls):
        for n in names:
            kid = KERNEL_IDS[n]
            d = [ev.ms((i * n_calls + c) * per + 2 * kid, (i * n_calls + c) * per + 2 * kid + 1)
                 for i in range(n_steps)]
            out[(c, n)] = float(np.mean(d))
            if stats is not None:
                stats[(c, n)] = {"median_ms": float(np.median(d)), "min_ms": float(np.min(d))}
    ev.close()
    return out


def down_sb_bytes(mi, shp):
    return mi.MXFP4_SB_BYTES if shp.fmt == 1 else mi.Q5K_SB_BYTES


def expert_bytes(mi, shp):
    """(gate + up bytes, down bytes) of one expert."""
    return (2 * (shp.I * shp.H // 256) * mi.Q4K_SB_BYTES,
            (shp.H * shp.I // 256) * down_sb_bytes(mi, shp))


def weight_copies(base, n):
    return [base] + [base.clone_weights() for _ in range(n - 1)]


def roofline(kernel, bound, work, ms, unit, peak, traffic=None, extra=None):
    per_s = work / (ms * 1e-3)
    achieved = per_s / (1e9 if unit == "GB/s" else 1e12)
    r = {"kernel": kernel, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
         "frac": achieved / peak, "traffic": traffic,
         ("algorithmic_bytes_per_launch" if unit == "GB/s" else "algorithmic_flops_per_launch"): work,
         "avg_launch_ms": ms}
    if extra:
        r.update(extra)
    return r


def bench_decode(args, torch, qm, mi, DeviceLayer, name="decode"):
    """Decode, T = 1 row per step, one moe_layer_forward per step."""
    w = mi.WORKLOADS[name]
    shp = w.shape
    layer = mi.make_layer(shp, w.seed)
    base = DeviceLayer.from_shape(layer, shp)
    copies = weight_copies(base, args.copies)
    pool = torch.from_numpy(mi.make_tokens(shp, w.seed, 64, stream=101)).cuda()
    T = 1
    ws = base.workspace(T)
    out = torch.empty((T, shp.H), device="cuda")
    used = []

    def step(i, events=None):
        c = copies[i % len(copies)]
        used.append(qm.moe_layer_forward(c.desc, pool[i % 64:i % 64 + 1], T, out, ws,
                                         events=events))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert set(used) == {qm.MOE_PATH_GEMV}, used
    eager_s = time_steps(torch, step, args.steps)
    dev_s, host_s = graph_time(torch, step, args.steps)

    nprof = min(args.steps, 256)
    kst = {}
    kms = kernel_profile(torch, qm, lambda i, e: step(i, e), nprof,
                         ["gemv_front", "gateup_gemv", "down_gemv"], kst)
    gu, dn = expert_bytes(mi, shp)
    # the gate/up kernel streams the k routed experts and the shared one
    gateup_bytes = (shp.k + 1) * gu + shp.H * 4 + (shp.k + 1) * shp.I * 4
    layer_bytes = (shp.k + 1) * (gu + dn) + shp.H * shp.E * 4   # K-quant: 19,202,048 B
    res = {
        "value": T / dev_s,
        "ms_per_step": dev_s * 1e3,
        "host_ms_per_step": host_s * 1e3,
        "eager_tokens_per_s": T * args.steps / eager_s,
        "eager_ms_per_step": eager_s / args.steps * 1e3,
        "weight_copies": len(copies),
        "kernel_ms": kms,
        "layer_algorithmic_bytes": layer_bytes,
        "layer_hbm_frac_graph": layer_bytes / dev_s / (HBM_PEAK_GBS * 1e9),
        "layer_hbm_frac_kernels": layer_bytes / (sum(kms.values()) * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "roofline": roofline(
            "gemv_gateup_kernel<%s,64,1,true> (8 routed experts and the shared one)"
            % ("MXFP4" if shp.fmt else "K-quant"),
            "hbm", gateup_bytes, kms["gateup_gemv"], "GB/s", HBM_PEAK_GBS,
            traffic_for("gemv_gateup_mx" if shp.fmt else "gemv_gateup"),
            {"median_launch_ms": kst["gateup_gemv"]["median_ms"],
             "min_launch_ms": kst["gateup_gemv"]["min_ms"], "launches": nprof}),
    }
    # outputs of 8 pool tokens (one T = 1 call each) for the oracle check
    xs, outs = [], []
    for i in range(8):
        qm.moe_layer_forward(base.desc, pool[i:i + 1], T, out, ws)
        torch.cuda.synchronize()
        xs.append(pool[i:i + 1].cpu().numpy())
        outs.append(out.cpu().numpy().copy())
    check = {"name": name, "layer": layer, "shape": shp, "x": np.concatenate(xs),
             "out": np.concatenate(outs), "tol": 1e-4}
    return res, check


def bench_layer_batches(args, torch, qm, mi, DeviceLayer, name, T, n_copies, K, W,
                        label, x_stream=None):
    """T rows per step through moe_layer_forward (automatic path), cycling
    weight copies and 4 token batches; HIP graph of exactly K steps."""
    w = mi.WORKLOADS[name]
    shp = w.shape
    layer = mi.make_layer(shp, w.seed, zipf=w.zipf)
    base = DeviceLayer.from_shape(layer, shp)
    copies = weight_copies(base, n_copies)
    xs = mi.make_tokens(shp, w.seed, 4 * T, stream=w.x_stream if x_stream is None else x_stream,
                        zipf=w.zipf)
    xd = torch.from_numpy(xs).cuda().view(4, T, shp.H)
    ws = base.workspace(T)
    out = torch.empty((T, shp.H), device="cuda")
    used = []

    def step(i, events=None):
        used.append(qm.moe_layer_forward(copies[i % len(copies)].desc, xd[(i // len(copies)) % 4],
                                         T, out, ws, events=events))

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    path = used[-1]
    dev_s, host_s = graph_time(torch, step, K)
    # distinct experts each batch touches (the library's own routing)
    idx = torch.empty((T, shp.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, shp.k), dtype=torch.float32, device="cuda")
    distinct = []
    for bi in range(4):
        qm.router_topk(base.desc, xd[bi], T, idx, wts, ws)
        distinct.append(int(torch.unique(idx).numel()))
    d_avg = float(np.mean(distinct))
    gu, dn = expert_bytes(mi, shp)
    alg_bytes = (d_avg + 1) * (gu + dn) + shp.H * shp.E * 4 + 2 * T * shp.H * 4
    flops = T * (shp.k + 1) * 6.0 * shp.H * shp.I + 2.0 * T * shp.H * shp.E
    if path == qm.MOE_PATH_MFMA:
        names = ["gemm_gateup", "gemm_down", "combine"]
        kms = kernel_profile(torch, qm, lambda i, e: step(i, e), min(K, 32), names)
        gu_bytes = (d_avg + 1) * gu + T * shp.H * 2 + T * (shp.k + 1) * shp.I * 2
        rl = roofline("gemm_grouped_kernel<0> (gate/up + SwiGLU)", "hbm", gu_bytes,
                      kms["gemm_gateup"], "GB/s", HBM_PEAK_GBS)
    else:
        names = ["gemv_front", "gateup_gemv", "down_gemv"]
        kms = kernel_profile(torch, qm, lambda i, e: step(i, e), min(K, 32), names)
        gu_bytes = (d_avg + 1) * gu + shp.H * 4 * T + T * (shp.k + 1) * shp.I * 4
        rl = roofline("gemv_gateup_kernel", "hbm", gu_bytes, kms["gateup_gemv"], "GB/s",
                      HBM_PEAK_GBS)
    qm.moe_layer_forward(base.desc, xd[0], T, out, ws)
    qm.router_topk(base.desc, xd[0], T, idx, wts, ws)
    torch.cuda.synchronize()
    res = {
        "workload": label,
        "value": T / dev_s, "unit": "tokens/s", "T": T,
        "ms_per_step": dev_s * 1e3, "host_ms_per_step": host_s * 1e3, "steps": K, "warmup": W,
        "path": "gemv" if path == qm.MOE_PATH_GEMV else "mfma",
        "weight_copies": len(copies), "distinct_experts": d_avg,
        "layer_algorithmic_bytes": alg_bytes, "layer_gflop": flops / 1e9,
        "layer_hbm_frac": alg_bytes / dev_s / (HBM_PEAK_GBS * 1e9),
        "kernel_ms": kms, "roofline": rl,
    }
    check = {"name": name, "layer": layer, "shape": shp, "x": xs[:T], "out": out.cpu().numpy(),
             "idx": idx.cpu().numpy(), "tol": 1e-4 if path == qm.MOE_PATH_GEMV else 1e-2}
    return res, check


def bench_sharded(args, torch, qm, mi, DeviceLayer, name, T, n_copies, n_batches, K, W, label,
                  check_rows, two_streams):
    """The 256/256 shard mode as one step: router_topk once (the synchronised
    decision), moe_layer_forward_shard(0, 2) and (1, 2), moe_reduce_partials.
    two_streams: shard 1 runs on a second stream, forked after the router and
    joined before the reduce (the shard calls are independent, as on two
    devices); else both run in order on one stream."""
    w = mi.WORKLOADS[name]
    shp = w.shape
    layer = mi.make_layer(shp, w.seed, zipf=w.zipf)
    base = DeviceLayer.from_shape(layer, shp)
    copies = weight_copies(base, n_copies)
    xs = mi.make_tokens(shp, w.seed, n_batches * T, stream=101 if T == 1 else w.x_stream,
                        zipf=w.zipf)
    xd = torch.from_numpy(xs).cuda().view(n_batches, T, shp.H)
    ws_r = base.workspace(T)
    ws = [base.workspace(T, 2) for _ in range(2)]
    idx = torch.empty((T, shp.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, shp.k), dtype=torch.float32, device="cuda")
    parts = [torch.empty((T, shp.H), device="cuda") for _ in range(2)]
    out = torch.empty((T, shp.H), device="cuda")
    used = []

    side = torch.cuda.Stream() if two_streams else None

    def step(i, evs=None):
        c = copies[i % len(copies)]
        x = xd[(i // len(copies)) % n_batches]
        qm.router_topk(c.desc, x, T, idx, wts, ws_r)
        main = torch.cuda.current_stream()
        if side is not None:
            side.wait_stream(main)
        for s in range(2):
            with torch.cuda.stream(main if s == 0 or side is None else side):
                used.append(qm.moe_layer_forward_shard(c.desc, x, T, idx, wts, s, 2, parts[s],
                                                       ws[s], events=None if evs is None else evs[s]))
        if side is not None:
            main.wait_stream(side)
        qm.moe_reduce_partials(parts, T * shp.H, out)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    path = used[-1]
    dev_s, host_s = graph_time(torch, step, K)
    gu, dn = expert_bytes(mi, shp)
    if path == qm.MOE_PATH_MFMA:
        names = ["gemm_gateup", "gemm_down", "combine"]
    else:
        # with the routing given, a shard call is two kernels (the gate/up
        # kernel also runs the shared expert; no front kernel)
        names = ["gateup_gemv", "down_gemv"]
    kst = {}
    kms = kernel_profile_calls(torch, lambda i, e: step(i, e), min(K, 16), 2, names, kst)
    kms_flat = {f"shard{c}.{n}": v for (c, n), v in kms.items()}
    if path == qm.MOE_PATH_MFMA:
        slots = T * shp.k + T
        flops_gu = 2.0 * 2 * shp.H * (shp.I // 2) * slots
        flops = 3.0 * 2 * shp.H * shp.I * slots
        if two_streams:
            # the shards' kernels overlap, so no single launch's duration is
            # its own: the whole step carries the figure (a lower bound for
            # the GEMMs, since the step also holds the router and the reduce)
            rl = roofline("whole two-shard step (both shards' grouped GEMMs, concurrent)", "mfma",
                          flops, dev_s * 1e3, "TFLOP/s", FP16_MFMA_PEAK_TFLOPS)
        else:
            rl = roofline("gemm_grouped_kernel<0> of shard 0 (gate/up + SwiGLU, I/2 = %d)"
                          % (shp.I // 2), "mfma", flops_gu, kms[(0, "gemm_gateup")], "TFLOP/s",
                          FP16_MFMA_PEAK_TFLOPS,
                          extra={"median_launch_ms": kst[(0, "gemm_gateup")]["median_ms"],
                                 "min_launch_ms": kst[(0, "gemm_gateup")]["min_ms"]})
        gemm_ms = sum(v for (c, n), v in kms.items() if n.startswith("gemm"))
        whole = {"expert_gflop": flops / 1e9,
                 "expert_mfma_frac": flops / (gemm_ms * 1e-3) / (FP16_MFMA_PEAK_TFLOPS * 1e12),
                 "step_mfma_frac": flops / dev_s / (FP16_MFMA_PEAK_TFLOPS * 1e12)}
    else:
        # the whole step (router_topk, two shards of two kernels, the reduce):
        # eager per-kernel events of these many small calls run slow (the GPU
        # idles between the host's calls), so the step's own graph time is
        # the basis
        layer_bytes = (shp.k + 1) * (gu + dn) + shp.H * shp.E * 4 + 3 * T * shp.H * 4
        rl = roofline("whole sharded step (router_topk + 2 x 2 shard kernels + reduce)", "hbm",
                      layer_bytes, dev_s * 1e3, "GB/s", HBM_PEAK_GBS)
        whole = {"layer_algorithmic_bytes": layer_bytes,
                 "layer_hbm_frac": layer_bytes / dev_s / (HBM_PEAK_GBS * 1e9)}
    x0 = xd[0]
    qm.router_topk(base.desc, x0, T, idx, wts, ws_r)
    for s in range(2):
        qm.moe_layer_forward_shard(base.desc, x0, T, idx, wts, s, 2, parts[s], ws[s])
    qm.moe_reduce_partials(parts, T * shp.H, out)
    torch.cuda.synchronize()
    res = {"workload": label, "value": T / dev_s, "unit": "tokens/s", "T": T,
           "ms_per_step": dev_s * 1e3, "host_ms_per_step": host_s * 1e3, "steps": K, "warmup": W,
           "path": "gemv" if path == qm.MOE_PATH_GEMV else "mfma", "weight_copies": len(copies),
           "kernel_ms": kms_flat, "roofline": rl, **whole}
    r = min(T, check_rows)
    check = {"name": name, "layer": layer, "shape": shp, "x": xs[:r], "out": out.cpu().numpy()[:r],
             "idx": idx.cpu().numpy()[:r], "tol": 1e-4 if path == qm.MOE_PATH_GEMV else 1e-2,
             "rows_note": f"first {r} of {T} rows"}
    return res, check


def bench_prefill(args, torch, qm, mi, DeviceLayer, name="prefill4096", check_rows=256):
    w = mi.WORKLOADS[name]
    shp = w.shape
    layer = mi.make_layer(shp, w.seed)
    base = DeviceLayer.from_shape(layer, shp)
    copies = [base, base.clone_weights()]
    T = w.T
    x_host = mi.make_tokens(shp, w.seed, T)
    x = torch.from_numpy(x_host).cuda()
    ws = base.workspace(T)
    out = torch.empty((T, shp.H), device="cuda")
    used = []

    def step(i, events=None):
        c = copies[i % len(copies)]
        used.append(qm.moe_layer_forward(c.desc, x, T, out, ws, events=events))

    K, W = args.prefill_steps, args.prefill_warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    assert set(used) == {qm.MOE_PATH_MFMA}, used
    eager_secs = time_steps(torch, step, K)
    dev_s, host_s = graph_time(torch, step, K)
    names = ["x_f16", "x_mx", "router_mfma", "router_topk", "bucket_hist",
             "bucket_scatter", "gemm_gateup", "gemm_down", "combine"]
    kst = {}
    kms = kernel_profile(torch, qm, lambda i, e: step(i, e), K, names, kst)
    slots = T * shp.k + T
    flops_gu = 2.0 * 2 * shp.H * shp.I * slots
    flops_d = 2.0 * shp.I * shp.H * slots
    gu_ms = kms["gemm_gateup"]
    d_ms = kms["gemm_down"]
    mx = shp.fmt == 1
    # the contraction's own dtype: fp16 x fp16 (K-quant), fp8 x fp4 block-scaled (MXFP4)
    peak = FP8_MFMA_PEAK_TFLOPS if mx else FP16_MFMA_PEAK_TFLOPS
    res = {
        "workload": ("prefill T=4096: same layer shape, %s weights, seed %d, uniform router, "
                     "grouped %s path, 2 rotating weight copies, HIP graph of exactly "
                     "`steps` steps" % ("MXFP4" if mx else "Q4_K/Q5_K", w.seed,
                                        "block-scaled fp8 x fp4 MFMA" if mx else "fp16-MFMA")),
        "value": T / dev_s,
        "unit": "tokens/s",
        "ms_per_step": dev_s * 1e3,
        "host_ms_per_step": host_s * 1e3,
        "eager_tokens_per_s": T * K / eager_secs,
        "eager_ms_per_step": eager_secs / K * 1e3,
        "steps": K,
        "warmup": W,
        "dtype": ("fp4 E2M1 weights x fp8 e4m3 tokens and h (%d MX-FP8 terms per value), "
                  "block-scaled MFMA, fp32 accumulate (router fp32)" % MX_TERMS if mx else
                  "fp16 operands, fp32 accumulate (router fp32)"),
        "kernel_ms": kms,
        "expert_gflop": (flops_gu + flops_d) / 1e9,
        "expert_mfma_frac": (flops_gu + flops_d) / ((gu_ms + d_ms) * 1e-3) / (peak * 1e12),
        "step_mfma_frac": (flops_gu + flops_d) / dev_s / (peak * 1e12),
        "roofline": roofline("gemm_mx_kernel<0>" if mx else "gemm_grouped_kernel<0>", "mfma",
                             flops_gu, gu_ms, "TFLOP/s", peak,
                             traffic_for("gemm_gateup_mx" if mx else "gemm_gateup"),
                             {"counters": counters_for("gemm_gateup_mx" if mx else "gemm_gateup"),
                              "median_launch_ms": kst["gemm_gateup"]["median_ms"],
                              "min_launch_ms": kst["gemm_gateup"]["min_ms"], "launches": K}),
    }
    if mx:
        # every product runs as MX_TERMS block-scaled MFMAs: executed matrix work
        res["roofline"]["executed_flops_per_launch"] = MX_TERMS * flops_gu
        res["roofline"]["executed_frac"] = MX_TERMS * res["roofline"]["frac"]
    qm.moe_layer_forward(base.desc, x, T, out, ws)
    idx = torch.empty((T, shp.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, shp.k), dtype=torch.float32, device="cuda")
    qm.router_topk(base.desc, x, T, idx, wts, ws)
    torch.cuda.synchronize()
    check = {"name": name, "layer": layer, "shape": shp, "x": x_host[:check_rows],
             "out": out.cpu().numpy()[:check_rows], "idx": idx.cpu().numpy()[:check_rows],
             "tol": 1e-2, "rows_note": f"first {check_rows} of {T} rows"}
    return res, check, layer, x_host


CONTINUUM_T = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)


def bench_continuum(args, torch, qm, mi, DeviceLayer):
    """Both paths at T = 1 .. 512 rows on the decode-shaped layer (seed 2,
    uniform router), each forced through moe_opts.path, replayed from HIP
    graphs over 4 weight copies and 4 token batches.  One JSON line per (T,
    path) on stdout: step time, tokens/s, algorithmic bytes (every distinct
    touched expert once, the shared expert, the router matrix, x and out) and
    FLOPs, GB/s and GFLOP/s, and the path the automatic rule takes at that T.
    --continuum-fmt 1 runs the same with MXFP4 expert weights."""
    shp = mi.QWEN35_MOE_MX if args.continuum_fmt == 1 else mi.QWEN35_MOE
    seed = 2
    layer = mi.make_layer(shp, seed)
    base = DeviceLayer.from_shape(layer, shp)
    copies = [base] + [base.clone_weights() for _ in range(3)]
    E_bytes = sum(expert_bytes(mi, shp))
    G = 8   # steps per graph: two rounds over the weight copies
    rows = []
    for T in args.continuum_t:
        xs = torch.from_numpy(mi.make_tokens(shp, seed, 4 * T, stream=7)).cuda().view(4, T, shp.H)
        out = torch.empty((T, shp.H), device="cuda")
        ws = base.workspace(T)
        # distinct experts the routing touches, per batch (the library's own top-k)
        idx = torch.empty((T, shp.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, shp.k), dtype=torch.float32, device="cuda")
        distinct = []
        for b in range(4):
            qm.router_topk(base.desc, xs[b], T, idx, wts, ws)
            distinct.append(int(torch.unique(idx).numel()))
        torch.cuda.synchronize()
        d_avg = float(np.mean(distinct))
        alg_bytes = (d_avg + 1) * E_bytes + shp.H * shp.E * 4 + 2 * T * shp.H * 4
        flops = T * (shp.k + 1) * 6.0 * shp.H * shp.I + 2.0 * T * shp.H * shp.E
        auto_used = []
        qm.moe_layer_forward(base.desc, xs[0], T, out, ws, path=qm.MOE_PATH_AUTO)
        auto_used.append(qm.moe_layer_forward(base.desc, xs[0], T, out, ws))
        for path, pname in ((qm.MOE_PATH_GEMV, "gemv"), (qm.MOE_PATH_MFMA, "mfma")):
            def step(i, path=path):
                return qm.moe_layer_forward(copies[i % 4].desc, xs[(i // 4 + i) % 4], T, out,
                                            ws, path=path)
            for i in range(2 * G):
                assert step(i) == path
            eager_n = max(G, min(256, int(4096 // T)))
            eager_s = time_steps(torch, step, eager_n)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(G):
                    step(i)
            g.replay()
            torch.cuda.synchronize()
            n_rep = max(2, min(64, int(2048 // (G * T)) + 2))
            t0 = time.perf_counter()
            for _ in range(n_rep):
                g.replay()
            torch.cuda.synchronize()
            secs = (time.perf_counter() - t0) / (n_rep * G)
            del g
            rows.append({
                "T": T, "fmt": "mxfp4" if shp.fmt == 1 else "kquant", "path": pname,
                "ms_per_step": secs * 1e3,
                "tokens_per_s": T / secs,
                "eager_ms_per_step": eager_s / eager_n * 1e3,
                "distinct_experts": d_avg,
                "algorithmic_bytes": alg_bytes, "gflop": flops / 1e9,
                "gb_per_s": alg_bytes / secs / 1e9, "gflop_per_s": flops / secs / 1e9,
                "hbm_frac": alg_bytes / secs / 1e9 / HBM_PEAK_GBS,
                "auto_path": "gemv" if auto_used[0] == qm.MOE_PATH_GEMV else "mfma",
                "steps_timed": n_rep * G,
            })
            print(json.dumps(rows[-1]), flush=True)
    return rows


def bench_edges(torch, qm, T=4096, H=2048, reps=20):
    """The steps either side of the layer at the prefill size: RMSNorm of the
    input rows, and the reduce of two shard partials plus the residual.  Both
    are HBM-bound; algorithmic bytes are one read of every input and one write
    of the output."""
    g = torch.Generator(device="cuda").manual_seed(9)
    x = torch.randn((T, H), device="cuda", generator=g)
    w = torch.randn(H, device="cuda", generator=g)
    y = torch.empty_like(x)
    parts = [torch.randn((T, H), device="cuda", generator=g) for _ in range(2)]
    r = torch.randn((T, H), device="cuda", generator=g)
    out = torch.empty_like(r)
    res = {}
    for name, fn, nbytes in (
            ("rmsnorm", lambda: qm.moe_rmsnorm(x, w, 1e-6, y), 2 * T * H * 4 + H * 4),
            ("reduce_residual_2", lambda: qm.moe_reduce_residual(parts, T * H, r, out),
             4 * T * H * 4)):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        res[name] = {"T": T, "H": H, "us": us, "algorithmic_bytes": nbytes,
                     "gb_per_s": nbytes / (us * 1e-6) / 1e9,
                     "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    return res


def split_rows(fracs, I, q=64):
    """Intermediate rows per lane for the given fractions, in multiples of q
    (the kernels' column quantum), by largest remainder; every lane gets at
    least q rows."""
    units = I // q
    raw = [f / sum(fracs) * units for f in fracs]
    rows = [max(1, int(r)) for r in raw]
    while sum(rows) > units:
        rows[rows.index(max(rows))] -= 1
    order = sorted(range(len(raw)), key=lambda i: raw[i] - int(raw[i]), reverse=True)
    for i in order[:units - sum(rows)]:
        rows[i] += 1
    return [r * q for r in rows]


def lane_times(torch, qm, dl, xd, idx, wts, T, rows, reps):
    """Each lane's shard alone (moe_layer_forward_range, routing given), replayed
    from a HIP graph of `reps` calls: microseconds per call."""
    out, a = [], 0
    for r in rows:
        b = a + r
        part = torch.empty((T, dl.H), device="cuda")
        ws = dl.workspace(T)

        def call(a=a, b=b, part=part, ws=ws):
            qm.moe_layer_forward_range(dl.desc, xd, T, idx, wts, a, b, part, ws)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(3):
                call()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                call()
        g.replay()
        torch.cuda.synchronize()
        n_rep = 5
        t0 = time.perf_counter()
        for _ in range(n_rep):
            g.replay()
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) / (n_rep * reps) * 1e6)
        del g
        a = b
    return out


def lane_report(rows, us):
    region = max(us)
    return {"rows": rows, "fractions": [r / sum(rows) for r in rows],
            "lane_us": [round(v, 2) for v in us], "region_us": round(region, 2),
            "idle_us_at_barrier": round(sum(region - v for v in us), 2)}


def bench_balance(args, torch, qm, mi, DeviceLayer):
    """Lane-time balance of shards sized by fraction (page "Distributed CPU:
    Zip Fusion Beyond Tensor Parallelism", "Heterogeneous Topology": shards in
    proportion to each lane's measured throughput; the region ends with the
    slowest lane).  Every lane here is the same GPU, timed alone: a lane's
    throughput is its rows per microsecond, and the rebalanced split gives each
    lane rows in proportion to it."""
    shp = mi.QWEN35_MOE
    report = {}
    for label, wname, T, reps in (("decode_T1", "decode", 1, 32),
                                  ("prefill_T4096", "prefill4096", 4096, 4)):
        w = mi.WORKLOADS[wname]
        layer = mi.make_layer(shp, w.seed)
        dl = DeviceLayer.from_shape(layer, shp)
        xd = torch.from_numpy(mi.make_tokens(shp, w.seed, T)).cuda()
        idx = torch.empty((T, shp.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, shp.k), dtype=torch.float32, device="cuda")
        qm.router_topk(dl.desc, xd, T, idx, wts, dl.workspace(T))   # the synchronised decision
        torch.cuda.synchronize()
        cases = {}
        for name, fracs in (("equal_2", (1, 1)), ("equal_4", (1, 1, 1, 1)), ("30_70", (0.3, 0.7))):
            rows = split_rows(fracs, shp.I)
            us = lane_times(torch, qm, dl, xd, idx, wts, T, rows, reps)
            cases[name] = lane_report(rows, us)
            print(f"[balance] {label} {name} rows={rows} lane_us={[round(v, 1) for v in us]}",
                  file=sys.stderr, flush=True)
        # one rebalancing step of the 30/70 split: rows in proportion to each
        # lane's measured rows per microsecond
        c = cases["30_70"]
        rates = [r / t for r, t in zip(c["rows"], c["lane_us"])]
        rows = split_rows(rates, shp.I)
        us = lane_times(torch, qm, dl, xd, idx, wts, T, rows, reps)
        cases["30_70_rebalanced"] = lane_report(rows, us)
        cases["30_70_rebalanced"]["from_rates_rows_per_us"] = [round(v, 3) for v in rates]
        full = lane_times(torch, qm, dl, xd, idx, wts, T, [shp.I], reps)[0]
        report[label] = {"T": T, "whole_layer_us": round(full, 2), "splits": cases}
    return report


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_decode(layer, shape, pool, budget_s):
    import oracle
    ol = oracle.Layer.from_shape(layer, shape)
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) < budget_s:
        i = n % pool.shape[0]
        oracle.forward(ol, pool[i:i + 1])
        n += 1
    dt = time.perf_counter() - t0
    # the same calls on one thread (a token's arithmetic is the same either way)
    n1 = 0
    t1 = time.perf_counter()
    while (time.perf_counter() - t1) < budget_s / 3:
        i = n1 % pool.shape[0]
        oracle.forward(ol, pool[i:i + 1], nthreads=1)
        n1 += 1
    dt1 = time.perf_counter() - t1
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n} decode tokens (cycling {pool.shape[0]} pool tokens), one T=1 oracle call each "
                      f"(routing, decode of the 9 touched experts, fp64 FFN), {dt:.1f} s",
            "single_thread": {"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{n1} decode tokens, {dt1:.1f} s"}}


def cpu_baseline_prefill(layer, shape, x, rows):
    import oracle
    ol = oracle.Layer.from_shape(layer, shape)
    t0 = time.perf_counter()
    oracle.forward(ol, x[:rows])
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {rows} of the 4096 prefill rows in one oracle call (routing, decode "
                      f"of every touched expert, fp64 FFN), {dt:.1f} s"}


def oracle_check(chk):
    """max|gpu - oracle| / RMS(oracle) over the rows of a config's sample whose
    GPU routing equals the oracle's (rows that differ are near-ties, counted)."""
    import oracle
    shp = chk["shape"]
    ol = oracle.Layer.from_shape(chk["layer"], shp)
    x = np.ascontiguousarray(chk["x"])
    oi, _, _, _ = oracle.router(x, chk["layer"]["router_w"], shp.k)
    same = np.ones(x.shape[0], bool) if "idx" not in chk else np.all(chk["idx"] == oi, axis=1)
    ref = oracle.forward(ol, x).astype(np.float64)[same]
    got = np.asarray(chk["out"], np.float64)[same]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.abs(got - ref).max() / rms) if ref.size else None
    return {"max_err_over_rms": err, "tolerance": chk["tol"],
            "within_tolerance": err is not None and err <= chk["tol"],
            "rows_compared": int(same.sum()), "rows_near_tie_routing": int((~same).sum()),
            "rows": chk.get("rows_note", f"{x.shape[0]} rows")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--copies", type=int, default=16,
                    help="weight copies cycled by decode steps (16 x 19 MB between reuses of a "
                         "copy's router and shared expert exceeds the 256 MB last-level cache)")
    ap.add_argument("--mid-steps", type=int, default=64,
                    help="steps timed at T = 32 and T = 512")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the decode and prefill runs of the MXFP4-weight layer")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle decode work")
    ap.add_argument("--cpu-prefill-rows", type=int, default=2048)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB device copy five times (counter calibration)")
    ap.add_argument("--continuum", action="store_true",
                    help="only time both paths at T = 1 .. 512 (one JSON line per point)")
    ap.add_argument("--continuum-t", type=int, nargs="+", default=list(CONTINUUM_T))
    ap.add_argument("--sharded-decode-streams", type=int, default=1, choices=[1, 2],
                    help="C2 sharded decode: the two shard calls in order on one stream (1) or "
                         "on two streams (2)")
    ap.add_argument("--continuum-fmt", type=int, default=0, choices=[0, 1],
                    help="expert weight format of the continuum: 0 K-quant, 1 MXFP4")
    ap.add_argument("--only", nargs="+", default=None, metavar="WORKLOAD",
                    choices=["decode", "sharded_decode", "batched_decode", "zipf_prefill",
                             "prefill", "sharded_prefill", "edges", "mxfp4_decode",
                             "mxfp4_prefill"],
                    help="run only these workloads (profiler runs); the JSON line then holds "
                         "only them")
    ap.add_argument("--balance", action="store_true",
                    help="only report lane times of shards sized by fraction (one JSON object)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the library has no multi-GPU path; the layer's shards run on one device.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import quantized_moe_transformer_amd as qm
    from quantized_moe_transformer_amd.layer import DeviceLayer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
        return
    if args.continuum:
        bench_continuum(args, torch, qm, mi, DeviceLayer)
        return
    if args.balance:
        print(json.dumps(bench_balance(args, torch, qm, mi, DeviceLayer)), flush=True)
        return

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def want(name):
        return args.only is None or name in args.only

    checks = {}
    dec = c2s = c2b = pre = c3 = c4s = edges = mx = None
    if want("decode"):
        say("C1 decode T=1 ...")
        dec, checks["C1_decode_T1"] = bench_decode(args, torch, qm, mi, DeviceLayer)
    if want("sharded_decode"):
        say("C2 sharded decode T=1 ...")
        c2s, checks["C2_sharded_T1"] = bench_sharded(
        args, torch, qm, mi, DeviceLayer, "decode_sharded", 1, args.copies, 64, args.steps,
        args.warmup, "sharded decode T=1: the same layer (seed 2), router_topk once, the 256/256 "
        "shards as two moe_layer_forward_shard calls "
        + ("in order on one stream (two streams measured slower at T=1)"
           if args.sharded_decode_streams == 1 else "on two streams")
        + ", moe_reduce_partials; 64-token pool, "
        f"{args.copies} rotating weight copies, HIP graph of exactly `steps` steps", 64,
        two_streams=args.sharded_decode_streams == 2)
    if want("batched_decode"):
        say("C2 batched decode T=32 ...")
        c2b, checks["C2_batched_T32"] = bench_layer_batches(
            args, torch, qm, mi, DeviceLayer, "decode_batched", 32, args.copies, args.mid_steps,
            args.prefill_warmup, "batched decode T=32: the same layer (seed 2), rows N(0,1), "
            f"automatic path, 4 token batches, {args.copies} rotating weight copies, HIP graph of "
            "exactly `steps` steps")
    if not args.no_prefill and want("zipf_prefill"):
        say("C3 prefill T=512 (Zipf-like expert load) ...")
        c3, checks["C3_zipf_T512"] = bench_layer_batches(
            args, torch, qm, mi, DeviceLayer, "prefill512_zipf", 512, 2, args.mid_steps,
            args.prefill_warmup, "prefill T=512: the same layer (seed 3) with Zipf-like expert "
            "load (slope -1), automatic path, 4 token batches, 2 rotating weight copies, HIP "
            "graph of exactly `steps` steps")
    if not args.no_prefill and want("prefill"):
        say("C4 prefill T=4096 ...")
        pre, checks["C4_prefill_T4096"], pre_layer, x_pre = bench_prefill(
            args, torch, qm, mi, DeviceLayer)
    if not args.no_prefill and want("sharded_prefill"):
        say("C4 two-shard prefill T=4096 ...")
        c4s, checks["C4_sharded_T4096"] = bench_sharded(
            args, torch, qm, mi, DeviceLayer, "prefill4096", 4096, 2, 1, args.prefill_steps,
            args.prefill_warmup, "two-shard prefill T=4096: the same layer (seed 4), router_topk "
            "once, the 256/256 shards as two moe_layer_forward_shard calls on two streams, "
            "moe_reduce_partials; 2 rotating weight copies, HIP graph of exactly `steps` steps", 256,
            two_streams=True)
    if not args.no_prefill and want("edges"):
        say("RMSNorm / residual at T=4096 ...")
        edges = bench_edges(torch, qm)
    if not args.no_mxfp4 and want("mxfp4_decode"):
        say("MXFP4 weights: decode T=1 ...")
        mdec, checks["mxfp4_decode_T1"] = bench_decode(args, torch, qm, mi, DeviceLayer,
                                                       "decode_mx")
        mx = {"decode": {
            "workload": ("decode T=1: the same layer shape with MXFP4 gate/up/down weights "
                         "(144-byte superblocks), seed 6, 64-token pool, "
                         f"{args.copies} rotating weight copies, HIP graph of exactly `steps` "
                         "steps"),
            "value": mdec["value"], "unit": "tokens/s", **{k: v for k, v in mdec.items()
                                                          if k != "value"}}}
    if not args.no_prefill and not args.no_mxfp4 and want("mxfp4_prefill"):
        say("MXFP4 weights: prefill T=4096 ...")
        mx = mx or {}
        mx["prefill"], checks["mxfp4_prefill_T4096"], _, _ = bench_prefill(
            args, torch, qm, mi, DeviceLayer, "prefill4096_mx")
    if args.only is not None:
        print(json.dumps({"only": args.only, "decode": dec, "sharded_decode": c2s,
                          "batched_decode": c2b, "zipf_prefill": c3, "prefill": pre,
                          "sharded_prefill": c4s, "mxfp4": mx, "edges": edges}), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        say("oracle on the host: baseline and per-config max|err|/RMS ...")
        cpu = cpu_baseline_decode(checks["C1_decode_T1"]["layer"], checks["C1_decode_T1"]["shape"],
                                  checks["C1_decode_T1"]["x"], args.cpu_budget)
        if pre is not None:
            pre["cpu_baseline"] = cpu_baseline_prefill(pre_layer, mi.QWEN35_MOE, x_pre,
                                                       args.cpu_prefill_rows)
        cpu["parity"] = {k: oracle_check(c) for k, c in checks.items()}
        for key, obj in (("C1_decode_T1", dec), ("C2_sharded_T1", c2s), ("C2_batched_T32", c2b),
                         ("C3_zipf_T512", c3), ("C4_prefill_T4096", pre),
                         ("C4_sharded_T4096", c4s)):
            if obj is not None:
                obj["parity"] = cpu["parity"][key]
        if mx is not None:
            mx["decode"]["parity"] = cpu["parity"]["mxfp4_decode_T1"]
            if mx.get("prefill"):
                mx["prefill"]["parity"] = cpu["parity"]["mxfp4_prefill_T4096"]

    line = {
        "metric": METRIC,
        "value": dec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 (Q4_K/Q5_K weights decoded in registers, fp32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": ("decode T=1: Qwen3.5-35B-A3B-shaped routed MoE layer, H=2048, 256 "
                         "experts, top-8, I=512, shared expert I=512, Q4_K gate/up, Q5_K down, "
                         f"seed 1, 64-token pool, {args.copies} rotating weight copies, one HIP "
                         "graph of exactly `steps` steps"),
            "T": 1,
            "path": "gemv",
            "parallelism": "single GPU",
        },
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode": {k: v for k, v in dec.items() if k not in ("value", "ms_per_step", "roofline")},
        "sharded_decode": c2s,
        "batched_decode": c2b,
        "zipf_prefill": c3,
        "prefill": pre,
        "sharded_prefill": c4s,
        "mxfp4": mx,
        "edges": edges,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
