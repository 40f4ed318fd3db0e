#!/usr/bin/env python3
"""Benchmark of the selective state-space scan on one MI355X.

One step = one chunked SSD prefill call (the fused bf16 prefill kernel: Δ cumsum,
state passing, intra-chunk and state-to-output products in one launch) over the
Mamba-2-2.7B-like layer shape: batch 8, seqlen 2048, 80 heads of
headdim 64, dstate 128, one B/C group, chunk 256, bf16 inputs with float32
accumulation and state.  Inputs are seeded synthetic tensors resident in HBM
before the timed region.

Timing: W untimed warm-up calls, then K calls.  Before each timed call a 1 GiB
buffer is read, outside the timed region, so that the 256 MB last-level
cache (MALL) holds none of the call's inputs.  Each call is bracketed by HIP
events on its stream, and every kernel launch inside it by the library's own
launch events; ms_per_step and the per-kernel times are medians over the K
calls (the mean of K back-to-back calls without the flush is reported beside
them).  GPU clocks are read with rocm-smi before and after the timed region.

The same run also times, as separate legs of the JSON line: the single-token
decode step at batch 256 (state cache of a 2.7B-layer prefill; each of the 64
steps timed, median per step, and the 64-step chain back to back), the
64K-token long-context prefill with eight groups, the 2.7B-layer prefill with
float8 e4m3fn x, B and C (bf16 dt and y), the Mamba-1 selective scan
(batch 8, seqlen 4096, 5120 channels, dstate 16), a packed variable-length
prefill (8 sequences of mixed lengths, 16384 tokens), the causal conv1d (width
4 over 5376 channels) and the gated RMSNorm (5120 channels) of the same layer,
the chunked backward at the prefill shape; and the CPU float64 oracle on the
prefill workload (the `cpu_baseline`, timed on this host's cores).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs ...]
       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # dense bf16 flop/s
VALU_F32_PEAK = 78.6e12    # non-packed fp32 FMA flop/s (256 CU x 64 lanes x 2 x 2.4 GHz)
VALU_LANE_OPS = 39.3e12    # non-packed vector lane-ops/s (256 CU x 4 SIMD x 16 lanes x 2.4 GHz)
METRIC = "SSD prefill tokens/s and decode tokens/s at 2.7B-layer shape; % MFMA/HBM roofline"

# kernels of one bf16 prefill call: the fused kernel alone, or, when the call is
# cut into sequence segments (few (batch, head) pairs, long sequence), the
# segment-state pass and the segment combine before it
FUSED_KERNELS = ["ssd_fused"]
SEGMENTED_KERNELS = ["segment_states", "segment_combine", "ssd_fused"]
# with a short segment 0 run whole beside the state walks of segments 1 .. S-2
LEAD_KERNELS = ["lead_segment_and_states", "segment_combine", "ssd_fused"]
# the sources of each kernel family: counter records in profiles/ apply while they match
_C = "selective_state_space_13_amd/csrc/"
FUSED_SOURCES = [_C + f for f in ("ssd_fused.hip", "ssd_fused_pair.h", "ssd_fused_walk.h", "mfma_tile.h",
                                  "ssd_kernels.h")]
DECODE_SOURCES = [_C + f for f in ("decode.hip", "ssd_kernels.h")]
BWD_SOURCES = [_C + f for f in ("ssd_bwd.hip", "ssd_fused_walk.h", "mfma_tile.h", "ssd_kernels.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(t):
    import numpy as np
    import torch
    if t is None:
        return None
    if t.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t.data)).cuda()
    if t.dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(t.data)).cuda().view(torch.float8_e4m3fn)
    return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).cuda()


class LaunchTimer:
    """HIP events around every kernel launch of the library calls in a region."""

    def __init__(self, nkernels, ncalls):
        import torch
        self.nk, self.nc = nkernels, ncalls
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nkernels * ncalls)]
        s = torch.cuda.current_stream()
        for e in self.ev:  # materialise the underlying hipEvent_t handles
            e.record(s)
        torch.cuda.synchronize()
        self.handles = [(ctypes.c_void_p * (2 * nkernels))(
            *[self.ev[2 * nkernels * c + j].cuda_event for j in range(2 * nkernels)])
            for c in range(ncalls)]

    def arm(self, lib, call):
        lib.ssd_set_launch_events(self.handles[call], 2 * self.nk)

    @staticmethod
    def disarm(lib):
        lib.ssd_set_launch_events(None, 0)

    def per_kernel_ms(self, reduce=None):
        out = []
        for k in range(self.nk):
            ts = [self.ev[2 * self.nk * c + 2 * k].elapsed_time(self.ev[2 * self.nk * c + 2 * k + 1])
                  for c in range(self.nc)]
            out.append(reduce(ts) if reduce else sum(ts) / len(ts))
        return out


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


_FLUSH = []


def flush_mall():
    """Read a 1 GiB device buffer (a sum into one value): afterwards the 256 MB
    last-level cache holds none of the benchmark's inputs, and no dirty lines that
    the next kernel would have to write back.  Enqueued on the current stream,
    outside any timed region."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.ones(1 << 28, dtype=torch.int32, device="cuda"))
        _FLUSH.append(torch.empty((), dtype=torch.int64, device="cuda"))
    torch.sum(_FLUSH[0], dim=0, dtype=torch.int64, out=_FLUSH[1])


def time_calls(fn, nkernels, steps, warmup, flush=True):
    """Warm-up, then `steps` calls, each bracketed by events, with the MALL
    flushed before each when `flush`; then `steps` more calls, flushed the same
    way, with the library's launch events around each kernel for the per-kernel
    times (kept apart so that the step time carries no event records between
    kernels).  Returns (median ms per call, median ms per kernel, mean ms per
    call back to back without the flush)."""
    import torch
    import selective_state_space_13_amd as ssd
    lib = ssd.lib()
    for _ in range(warmup):
        fn()
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush:
            flush_mall()
        calls[i][0].record()
        fn()
        calls[i][1].record()
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) for a, b in calls]
    timer = LaunchTimer(nkernels, steps)
    torch.cuda.synchronize()
    for i in range(steps):
        if flush:
            flush_mall()
        timer.arm(lib, i)
        fn()
    LaunchTimer.disarm(lib)
    torch.cuda.synchronize()
    per_kernel = timer.per_kernel_ms(median)
    # the same calls back to back (MALL warm), wall clock
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    b2b = (time.perf_counter() - t0) * 1e3 / steps
    return median(per_call), per_kernel, b2b


def gpu_clocks():
    """Current GPU clocks from rocm-smi (None when it is unavailable, or under a
    profiler, whose preloaded library would initialise the GPU in the child
    before rocm-smi's interpreter starts)."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=30)
        d = json.loads(r.stdout)
    except Exception:  # noqa: BLE001 - any failure just means no clock record
        return None
    out = {}
    for card, v in d.items():
        if isinstance(v, dict):
            out[card] = {k: v[k] for k in v if "clock" in k.lower() or "sclk" in k.lower()
                         or "mclk" in k.lower() or "fclk" in k.lower()}
    return out or None


def source_digest(paths):
    """Digest of the code of the kernel's source files: comments and trailing blanks
    are left out, so that a comment edit does not retire counters taken on the
    same code."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(text.encode("utf-8"))
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(f"{kernel}@{workload}")
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("bytes_per_launch")


def counter_rates(kernel_ms, workload, sources):
    """For each timed kernel with a counter record taken on its current sources:
    the measured HBM bytes per launch and those bytes over the kernel's time."""
    dg = source_digest(sources)
    out = {}
    for k, ms in kernel_ms.items():
        b = measured_traffic(k, workload, dg)
        if b:
            out[k] = {"bytes": b, "achieved_gbps": round(b / (ms * 1e-3) / 1e9, 1),
                      "frac": round(b / (ms * 1e-3) / HBM_PEAK, 4)}
    return out or None


def prefill_work(c):
    """Algorithmic bytes and flops of a prefill call (inputs read once, outputs
    written once; causal flops of the block decomposition at the workload's
    chunk size)."""
    b, L, H, P, N, G, Q = (c[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate",
                                          "ngroups", "chunk"))
    K = (L + Q - 1) // Q
    es = {"fp8": 1, "bf16": 2, "f32": 4}[c["dtype"]]   # x, B, C
    ea = 2 if c["dtype"] == "fp8" else es              # dt, y (bf16 beside float8 inputs)
    x_bytes = b * L * H * P * es         # x
    y_bytes = b * L * H * P * ea         # y
    bc_bytes = b * L * G * N * es        # B, and likewise C
    dt_bytes = b * L * H * ea
    final = b * H * N * P * 4 if c.get("final_state") else 0
    units_h = b * K * H
    units_g = b * K * G
    # the same causal count at the 64-token blocking the bf16 kernel uses
    K64 = (L + 63) // 64
    flops_q64 = b * K64 * H * (4 * 64 * N * P + 64 * 65 * P) + b * K64 * G * 64 * 65 * N
    total = dict(bytes=x_bytes + y_bytes + 2 * bc_bytes + dt_bytes + final,
                 flops=units_h * (4 * Q * N * P + Q * (Q + 1) * P) + units_g * Q * (Q + 1) * N,
                 flops_q64=flops_q64)
    # the fused kernel does all of it (a cut last round included: its halves
    # hand the state at the cut over within the launch); the segment passes
    # re-read x, B and dt
    return {"ssd_fused": total, "total": total,
            "segment_states": dict(bytes=x_bytes + bc_bytes + dt_bytes, flops=units_h * 2 * Q * N * P),
            "segment_combine": dict(bytes=0, flops=0)}


def bench_prefill(cfg, steps, warmup, seed=0):
    import torch
    import selective_state_space_13_amd as ssd
    from workloads import gen
    log(f"[bench] prefill {cfg['name']}: generating inputs")
    d = gen.ssd_inputs(cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"],
                       cfg["ngroups"], cfg["dtype"], seed=seed, config_id=cfg["id"])
    x, dt, B, C, A, D = (to_dev(d[k]) for k in ("x", "dt", "B", "C", "A", "D"))
    del d
    code = {"bf16": ssd.SSD_BF16, "f32": ssd.SSD_F32, "fp8": ssd.SSD_FP8}[cfg["dtype"]]
    ws = torch.empty(ssd.chunk_scan_workspace_size(cfg["batch"], cfg["seqlen"], cfg["nheads"],
                                                   cfg["headdim"], cfg["dstate"], cfg["ngroups"],
                                                   cfg["chunk"], code), dtype=torch.uint8, device="cuda")
    y = torch.empty(x.shape, dtype=dt.dtype, device="cuda")  # bf16 beside float8 inputs
    fs = torch.empty(cfg["batch"], cfg["nheads"], cfg["dstate"], cfg["headdim"], device="cuda") \
        if cfg.get("final_state") else None
    launches, _, _, lead = ssd.chunk_scan_plan(cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"],
                                         cfg["dstate"], cfg["ngroups"], cfg["chunk"], code)
    names = {3: LEAD_KERNELS if lead else SEGMENTED_KERNELS}.get(launches, FUSED_KERNELS)

    def step():
        ssd.ssd_chunk_scan(x, dt, A, B, C, D, chunk=cfg["chunk"], workspace=ws, out=y,
                           return_final_state=fs is not None, final_state=fs)

    log(f"[bench] prefill {cfg['name']}: timing {steps} steps after {warmup} warm-up")
    ms, per, b2b = time_calls(step, len(names), steps, warmup)
    tokens = cfg["batch"] * cfg["seqlen"]
    return dict(ms=ms, b2b_ms=b2b, per_kernel_ms=dict(zip(names, per)), tokens=tokens,
                work=prefill_work(cfg), final_state=fs, y=y)


def measured_mfma_flops(kernel, workload, digest):
    """Issued MFMA flops per launch (rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)
    from the committed counter summary, if taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(f"{kernel}@{workload}")
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("mfma_flops_per_launch")


def roofline_entry(kernel, ms, work, workload, digest):
    t = ms * 1e-3
    byte_frac = work["bytes"] / t / HBM_PEAK
    flop_frac = work["flops"] / t / MFMA_BF16_PEAK
    if byte_frac >= flop_frac:
        bound, achieved, peak, unit = "hbm", work["bytes"] / t / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", work["flops"] / t / 1e12, MFMA_BF16_PEAK / 1e12, "TFLOP/s"
    traffic = measured_traffic(kernel, workload, digest)
    issued = measured_mfma_flops(kernel, workload, digest)
    return {"kernel": kernel, "bound": bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": traffic, "hbm_frac": round(byte_frac, 4),
            "mfma_frac": round(flop_frac, 4),
            "mfma_frac_q64": round(work["flops_q64"] / t / MFMA_BF16_PEAK, 4) if "flops_q64" in work else None,
            "mfma_frac_issued": round(issued / t / MFMA_BF16_PEAK, 4) if issued else None,
            "median_launch_ms": round(ms, 5)}


def bench_decode(steps, warmup, prefill_state, bf16_state=False):
    import torch
    import selective_state_space_13_amd as ssd
    from workloads import configs, gen
    c = configs.DECODE_STATE_CACHE
    c2 = configs.MAMBA2_LAYER_PREFILL
    reps = c["batch"] // c2["batch"]
    state = prefill_state.repeat(reps, 1, 1, 1).contiguous()  # state cache of the 2.7B-layer prefill
    if bf16_state:
        state = state.to(torch.bfloat16)
    A, D = (to_dev(t) for t in gen.ssd_params(c["nheads"], config_id=c2["id"]))
    log("[bench] decode: generating per-step inputs")
    steps_in = []
    for k in range(c["steps"]):
        s = gen.decode_inputs(c["batch"], c["nheads"], c["headdim"], c["dstate"], c["ngroups"],
                              c["dtype"], step=k, config_id=c["id"])
        steps_in.append(tuple(to_dev(s[n]) for n in ("x", "dt", "B", "C")))
    y = torch.empty_like(steps_in[0][0])
    it = [0]
    step_fn = ssd.ssd_decode_step_bf16_state if bf16_state else ssd.ssd_decode_step

    def one():
        x, dt, B, C = steps_in[it[0] % len(steps_in)]
        it[0] += 1
        step_fn(x, dt, A, B, C, D, state, out=y)

    ms, per, b2b = time_calls(one, 1, c["steps"], warmup)
    state_bytes = c["batch"] * c["nheads"] * c["dstate"] * c["headdim"] * (2 if bf16_state else 4)
    io = c["batch"] * (c["nheads"] * c["headdim"] * 2 * 2 + c["nheads"] * 2 + 2 * c["ngroups"] * c["dstate"] * 2)
    return dict(ms=ms, b2b_ms=b2b, kernel_ms=per[0], tokens=c["batch"], bytes=2 * state_bytes + io,
                flops=c["batch"] * c["nheads"] * c["dstate"] * c["headdim"] * 5, steps=c["steps"])


def bench_mamba1(steps, warmup, general_A=False):
    """The Mamba-1 workload, with its A = -[1..N] per channel, or (general_A) with an
    A of per-(channel, state) random rates, which takes one exponential per state."""
    import numpy as np
    import torch
    import selective_state_space_13_amd as ssd
    from workloads import configs, gen
    c = configs.MAMBA1_SELECTIVE_SCAN
    log("[bench] mamba1: generating inputs")
    d = gen.mamba1_inputs(c["batch"], c["seqlen"], c["dim"], c["dstate"], c["dtype"], config_id=c["id"])
    if general_A:
        rng = np.random.default_rng([0, c["id"], 99])
        d["A"] = gen.Tensor(-np.exp(rng.uniform(0.0, np.log(16.0), (c["dim"], c["dstate"]))).astype(np.float32), "f32")
    u, dl, A, B, C, D, z = (to_dev(d[k]) for k in ("u", "delta", "A", "B", "C", "D", "z"))
    del d
    out = torch.empty_like(u)
    segmented = ssd.lib().selective_scan_workspace_size(c["batch"], c["seqlen"], c["dim"], c["dstate"],
                                                        ssd.SSD_BF16) > 0
    names = ["segment_states", "segment_combine", "selective_scan"] if segmented else ["selective_scan"]

    def one():
        ssd.selective_scan(u, dl, A, B, C, D, z, out=out)

    ms, per, _ = time_calls(one, len(names), steps, warmup)
    n_el = c["batch"] * c["seqlen"] * c["dim"]
    return dict(ms=ms, kernel_ms=sum(per), per_kernel_ms=dict(zip(names, per)),
                tokens=c["batch"] * c["seqlen"],
                bytes=4 * n_el * 2 + 2 * c["batch"] * c["seqlen"] * c["dstate"] * 2,
                exps=n_el * c["dstate"])


def bench_varlen(steps, warmup):
    import torch
    import selective_state_space_13_amd as ssd
    from workloads import configs, gen
    c = configs.VARLEN_PREFILL
    log("[bench] varlen: generating inputs")
    d = gen.ssd_varlen_inputs(c["lengths"], c["nheads"], c["headdim"], c["dstate"], c["ngroups"],
                              c["dtype"], config_id=c["id"])
    x, dt, A, B, C, D = (to_dev(d[k]) for k in ("x", "dt", "A", "B", "C", "D"))
    cu = torch.from_numpy(d["cu_seqlens"]).cuda()
    del d
    y = torch.empty_like(x)

    def one():
        ssd.ssd_chunk_scan_varlen(x, dt, A, B, C, D, cu_seqlens=cu, out=y)

    ms, per, _ = time_calls(one, 1, steps, warmup)
    T = sum(c["lengths"])
    nbytes = 2 * T * c["nheads"] * c["headdim"] * 2 + 2 * T * c["ngroups"] * c["dstate"] * 2 \
        + T * c["nheads"] * 2
    return dict(ms=ms, kernel_ms=per[0], tokens=T, bytes=nbytes)


BWD_KERNELS = ["state_and_adjoint_walks", "chunk_gradients", "dA_dD_reduce"]
BWD_SEGMENTED = ["segment_states", "segment_combine"] + BWD_KERNELS


def bench_backward(cfg, steps, warmup, seed=0):
    """The chunked backward at the prefill workload's shape (dL/dy random, dL/dh_final = 0)."""
    import torch
    import selective_state_space_13_amd as ssd
    from workloads import gen
    log(f"[bench] backward {cfg['name']}: generating inputs")
    d = gen.ssd_inputs(cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"],
                       cfg["ngroups"], cfg["dtype"], seed=seed, config_id=cfg["id"])
    gr = gen.ssd_grad_inputs(cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"],
                             cfg["dtype"], seed=seed, config_id=cfg["id"], with_dfinal=False)
    x, dt, B, C, A, D = (to_dev(d[k]) for k in ("x", "dt", "B", "C", "A", "D"))
    dy = to_dev(gr["dy"])
    del d, gr
    b, L, H, P, N, G = (cfg[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups"))
    ws = torch.empty(ssd.lib().ssd_chunk_scan_bwd_workspace_size(b, L, H, P, N, G, ssd.SSD_BF16),
                     dtype=torch.uint8, device="cuda")
    nchunks = (L + 63) // 64
    # the forward state pass is cut into segments exactly when the forward's is
    _, nseg, _, _ = ssd.chunk_scan_plan(b, L, H, P, N, G, cfg["chunk"], ssd.SSD_BF16)
    names = BWD_SEGMENTED if nseg > 1 else BWD_KERNELS

    def step():
        ssd.ssd_chunk_scan_bwd(x, dt, A, B, C, dy, D, workspace=ws)

    log(f"[bench] backward: timing {steps} steps after {warmup} warm-up")
    ms, per, _ = time_calls(step, len(names), steps, warmup)
    alg = 3 * b * L * H * P * 2 + 2 * b * L * H * 2 + 4 * b * L * G * N * 2
    states = 2 * b * H * nchunks * N * P * 4
    return dict(ms=ms, per_kernel_ms=dict(zip(names, per)), tokens=b * L, alg_bytes=alg,
                state_bytes=states)


def bench_convnorm(steps, warmup):
    """The causal conv1d and the gated RMSNorm at the 2.7B-layer shape."""
    import torch
    import selective_state_space_13_amd as ssd
    from workloads import configs, gen
    c = configs.CONV1D_LAYER
    log("[bench] conv1d: generating inputs")
    d = gen.conv1d_inputs(c["batch"], c["seqlen"], c["channels"], c["width"], c["dtype"],
                          config_id=c["id"])
    x, w, bias, s0 = (to_dev(d[k]) for k in ("x", "weight", "bias", "state"))
    del d
    y = torch.empty_like(x)
    fs = torch.empty_like(s0)

    def conv():
        ssd.causal_conv1d(x, w, bias, initial_state=s0, return_final_state=True, out=y, final_state=fs)

    ms_c, per_c, _ = time_calls(conv, 1, steps, warmup)
    n = c["batch"] * c["seqlen"] * c["channels"]
    conv_bytes = 2 * n * 2 + 2 * s0.numel() * 4 + w.numel() * 4 + bias.numel() * 4
    del x, y
    r = configs.GATED_RMSNORM_LAYER
    log("[bench] rmsnorm: generating inputs")
    d = gen.rmsnorm_inputs(r["rows"], r["channels"], r["dtype"], config_id=r["id"])
    yy, z, wn = (to_dev(d[k]) for k in ("y", "z", "weight"))
    del d
    out = torch.empty_like(yy)

    def norm():
        ssd.gated_rmsnorm(yy, z, wn, ngroups=r["ngroups"], out=out)

    ms_n, per_n, _ = time_calls(norm, 1, steps, warmup)
    norm_bytes = 3 * r["rows"] * r["channels"] * 2 + wn.numel() * 4
    return dict(conv_ms=per_c[0], conv_bytes=conv_bytes, norm_ms=per_n[0], norm_bytes=norm_bytes,
                conv_tokens=c["batch"] * c["seqlen"], norm_rows=r["rows"])


def cpu_baseline(cfg, seed=0, min_seconds=10.0):
    """The float64 oracle on the prefill workload, on this host's cores."""
    import oracle
    from workloads import gen
    d = gen.ssd_inputs(cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"],
                       cfg["ngroups"], cfg["dtype"], seed=seed, config_id=cfg["id"])
    args = [d[k].f64() for k in ("x", "dt", "A", "B", "C")]
    D = d["D"].f64()
    del d
    total, calls = 0.0, 0
    while total < min_seconds and calls < 64:
        oracle.ssd_scan(*args, D=D)
        total += oracle.last_seconds
        calls += 1
        log(f"[bench] cpu oracle call {calls}: {oracle.last_seconds:.2f} s")
    tokens = cfg["batch"] * cfg["seqlen"] * calls
    return {"value": round(tokens / total, 1), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{calls} x the full prefill workload (b{cfg['batch']} L{cfg['seqlen']} "
                      f"H{cfg['nheads']} P{cfg['headdim']} N{cfg['dstate']}), float64 sequential "
                      f"recurrence, {total:.1f} s of compute"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="decode,long,fp8,mamba1,varlen,convnorm,backward",
                    help="extra legs to time besides the prefill step (comma list or 'none')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy a MIB-mebibyte device buffer 3 times: a plain copy kernel of "
                         "known size, against which HBM byte counters are scaled")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the library has no "
                                   "multi-GPU path (how the scan would shard is described, not "
                                   "implemented)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import selective_state_space_13_amd as ssd
    from workloads import configs
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible: this benchmark needs an MI355X")
    ssd.lib()

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 device copies of {nbytes} bytes")
        del src, dst

    # practical reference for the HBM fractions: a device copy of 1 GiB (read + write bytes)
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_tbs = 2 * 5 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del src, dst

    legs = [] if args.legs == "none" else [s for s in args.legs.split(",") if s]
    cfg = configs.MAMBA2_LAYER_PREFILL
    workload = f"{cfg['name']}:b{cfg['batch']}L{cfg['seqlen']}H{cfg['nheads']}P{cfg['headdim']}" \
               f"N{cfg['dstate']}G{cfg['ngroups']}Q{cfg['chunk']}"
    digest = source_digest(FUSED_SOURCES)
    clocks_before = gpu_clocks()
    pf = bench_prefill(cfg, args.steps, args.warmup)
    clocks_after = gpu_clocks()
    per = pf["per_kernel_ms"]
    dom = max(per, key=lambda k: per[k])
    roof = roofline_entry(dom, per[dom], pf["work"][dom], workload, digest)
    total_work = pf["work"]["total"]
    t_step = pf["ms"] * 1e-3
    result = {
        "metric": METRIC,
        "value": round(pf["tokens"] / t_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms"], 5),
        "ms_per_step_back_to_back": round(pf["b2b_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "batch": cfg["batch"], "seqlen": cfg["seqlen"],
                   "nheads": cfg["nheads"], "headdim": cfg["headdim"], "dstate": cfg["dstate"],
                   "ngroups": cfg["ngroups"], "chunk": cfg["chunk"], "parallelism": "single-gpu"},
        "roofline": roof,
        "step_roofline": {"hbm_frac": round(total_work["bytes"] / t_step / HBM_PEAK, 4),
                          "mfma_frac": round(total_work["flops"] / t_step / MFMA_BF16_PEAK, 4),
                          "alg_bytes": total_work["bytes"], "alg_flops": total_work["flops"]},
        "per_kernel_ms": {k: round(v, 5) for k, v in per.items()},
        "per_kernel_measured_hbm": counter_rates(per, workload, FUSED_SOURCES),
        "timing": "median over the timed calls of HIP events around each call, with a 1 GiB buffer "
                  "read before every call so the 256 MB MALL holds no input; per-kernel times from as "
                  "many calls again with events around each kernel; ms_per_step_back_to_back: mean of "
                  "the same calls back to back without the flush",
        "gpu_clocks": {"before": clocks_before, "after": clocks_after},
        "hbm_copy_reference": {"value": round(copy_tbs, 3), "unit": "TB/s",
                               "what": "torch device copy of a 1 GiB buffer, read + write bytes, 5 copies; "
                                       "context for the HBM fractions, which are against the 8 TB/s peak"},
    }
    del pf
    extra = {}
    if "decode" in legs:
        # state cache left by the 2.7B-layer prefill (its 8 final states, tiled over the batch)
        from workloads import gen
        d = gen.ssd_inputs(cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"],
                           cfg["ngroups"], cfg["dtype"], config_id=cfg["id"])
        x, dt, B, C, A, D = (to_dev(d[k]) for k in ("x", "dt", "B", "C", "A", "D"))
        del d
        _, fs8 = ssd.ssd_chunk_scan(x, dt, A, B, C, D, chunk=cfg["chunk"], return_final_state=True)
        del x, dt, B, C
        for key, lp in (("decode", False), ("decode_bf16_state", True)):
            dec = bench_decode(args.steps, args.warmup, fs8, bf16_state=lp)
            t = dec["kernel_ms"] * 1e-3
            extra[key] = {"workload": "decode_state_cache:b256H80P64N128G1, 64 single-token steps, "
                                      + ("bf16" if lp else "float32") + " state cache",
                          "tokens_per_s": round(dec["tokens"] / (dec["ms"] * 1e-3), 1),
                          "ms_per_step": round(dec["ms"], 5), "kernel_ms": round(dec["kernel_ms"], 5),
                          "chain_ms_back_to_back": round(dec["b2b_ms"] * dec["steps"], 5),
                          "measured_hbm": counter_rates(
                              {"decode_step_" + ("bf16" if lp else "f32") + "_state": dec["kernel_ms"]},
                              "decode_state_cache:b256H80P64N128G1", DECODE_SOURCES),
                          "roofline": {"bound": "hbm", "achieved": round(dec["bytes"] / t / 1e9, 2),
                                       "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                                       "frac": round(dec["bytes"] / t / HBM_PEAK, 4)}}
    if "long" in legs:
        c3 = configs.LONG_CONTEXT_PREFILL
        lp = bench_prefill(c3, max(3, args.steps // 4), 2)
        t = lp["ms"] * 1e-3
        w = lp["work"]["total"]
        extra["long_prefill"] = {"workload": "long_context_prefill:b1L65536H80P64N128G8Q256",
                                 "tokens_per_s": round(lp["tokens"] / t, 1), "ms": round(lp["ms"], 5),
                                 "per_kernel_ms": {k: round(v, 5) for k, v in lp["per_kernel_ms"].items()},
                                 "per_kernel_measured_hbm": counter_rates(
                                     lp["per_kernel_ms"], "long_context_prefill:b1L65536H80P64N128G8Q256",
                                     FUSED_SOURCES),
                                 "hbm_frac": round(w["bytes"] / t / HBM_PEAK, 4),
                                 "mfma_frac": round(w["flops"] / t / MFMA_BF16_PEAK, 4)}
        del lp
    for key in ("mamba1", "mamba1_general_A"):
        if "mamba1" not in legs:
            break
        m1 = bench_mamba1(max(3, args.steps // 4), 1, general_A=key.endswith("general_A"))
        t = m1["kernel_ms"] * 1e-3
        # the state update's minimal ALU work per (token, channel, state): Δ·A (or, with
        # A = -[1..N], one product of the power tree), B·(Δu), the update FMA and the
        # output FMA on the vector ALU, and one exponential per state (or per (token,
        # channel)) on the transcendental unit, at the chip's unit counts: 256 CUs x 4
        # SIMDs x 16 lanes x 2.4 GHz = 39.3e12 lane-ops/s, exponentials at a quarter
        gen_A = key.endswith("general_A")
        n_exp = m1["exps"] if gen_A else m1["exps"] // 16
        alu_roof_s = m1["exps"] * 4 / VALU_LANE_OPS + n_exp / (VALU_LANE_OPS / 4)
        extra[key] = {"workload": "mamba1_selective_scan:b8L4096D5120N16"
                                  + (", A random per (channel, state) in [-16, -1]" if key.endswith("general_A")
                                     else ", A = -[1..16] per channel (one exponential per step, then powers)"),
                           "tokens_per_s": round(m1["tokens"] / (m1["ms"] * 1e-3), 1),
                           "ms": round(m1["ms"], 5),
                           "per_kernel_ms": {k: round(v, 5) for k, v in m1["per_kernel_ms"].items()},
                           "roofline": {"bound": "alu", "roof_ms": round(alu_roof_s * 1e3, 5),
                                        "frac": round(alu_roof_s / t, 4),
                                        "what": "4 VALU lane-ops per (token, channel, state) and 1 exp per "
                                                + ("(token, channel, state)" if gen_A else "(token, channel)")
                                                + " at 39.3e12 lane-ops/s and 9.8e12 exp/s"},
                           "hbm_frac": round(m1["bytes"] / t / HBM_PEAK, 4),
                           "exp_per_s": round(n_exp / t, 1)}
    if "fp8" in legs:
        # the 2.7B-layer prefill with float8 e4m3fn x, B, C (bf16 dt and y)
        c8 = dict(cfg, dtype="fp8", name=cfg["name"] + "_fp8")
        f8 = bench_prefill(c8, args.steps, args.warmup)
        per8 = f8["per_kernel_ms"]
        w8 = f8["work"]["ssd_fused"]
        t8 = per8["ssd_fused"] * 1e-3
        extra["fp8_prefill"] = {
            "workload": workload + ", x B C float8 e4m3fn, dt and y bf16",
            "tokens_per_s": round(f8["tokens"] / (f8["ms"] * 1e-3), 1), "ms": round(f8["ms"], 5),
            "per_kernel_ms": {k: round(v, 5) for k, v in per8.items()},
            "alg_bytes": w8["bytes"],
            "roofline": {"kernel": "ssd_fused", "bound": "hbm",
                         "achieved": round(w8["bytes"] / t8 / 1e9, 3), "peak": HBM_PEAK / 1e9,
                         "unit": "GB/s", "frac": round(w8["bytes"] / t8 / HBM_PEAK, 4),
                         "mfma_frac_q64": round(w8["flops_q64"] / t8 / MFMA_BF16_PEAK, 4)}}
        del f8
    if "varlen" in legs:
        vl = bench_varlen(args.steps, args.warmup)
        t = vl["kernel_ms"] * 1e-3
        extra["varlen"] = {"workload": "varlen_packed_prefill:8 sequences, 16384 tokens, H80P64N128G1",
                           "tokens_per_s": round(vl["tokens"] / (vl["ms"] * 1e-3), 1),
                           "ms": round(vl["ms"], 5), "kernel_ms": round(vl["kernel_ms"], 5),
                           "hbm_frac": round(vl["bytes"] / t / HBM_PEAK, 4)}
    if "backward" in legs:
        bw = bench_backward(cfg, max(3, args.steps // 2), 2)
        t = bw["ms"] * 1e-3
        extra["backward"] = {
            "workload": workload + " (dL/dy random; dx, ddt, dA, dB, dC, dD)",
            "tokens_per_s": round(bw["tokens"] / t, 1), "ms": round(bw["ms"], 5),
            "per_kernel_ms": {k: round(v, 5) for k, v in bw["per_kernel_ms"].items()},
            "per_kernel_measured_hbm": counter_rates(bw["per_kernel_ms"], workload, BWD_SOURCES),
            "alg_bytes": bw["alg_bytes"], "state_bytes_written_and_read": bw["state_bytes"],
            "hbm_frac_algorithmic": round(bw["alg_bytes"] / t / HBM_PEAK, 4),
            "hbm_frac_with_states": round((bw["alg_bytes"] + 2 * bw["state_bytes"]) / t / HBM_PEAK, 4)}
    if "convnorm" in legs:
        cn = bench_convnorm(args.steps, args.warmup)
        for key, wl in (("conv", "conv1d_layer:b8L2048C5376W4"), ("norm", "gated_rmsnorm_layer:rows16384C5120G1")):
            t = cn[key + "_ms"] * 1e-3
            extra[{"conv": "conv1d", "norm": "gated_rmsnorm"}[key]] = {
                "workload": wl, "kernel_ms": round(cn[key + "_ms"], 5),
                "roofline": {"bound": "hbm", "achieved": round(cn[key + "_bytes"] / t / 1e9, 2),
                             "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                             "frac": round(cn[key + "_bytes"] / t / HBM_PEAK, 4)}}
    if extra:
        result["legs"] = extra
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on the prefill workload")
        result["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
