#!/usr/bin/env python3
"""Benchmark of the gfx950 selective scan.

Headline: the long-context scan, the largest single-GPU workload (batch 1,
d_inner 1536, L 1,048,576, d_state 16, bf16 IO with fp32 state, silu gate,
last_state returned).  One step = one full prefill scan of the sequence with
inputs already resident in HBM: all four launches of the segmented scan
(pass 1 over every segment, the plan and the work lists, pass 2 over the
head windows of the segments while the incoming state still counts).  Throughput is algorithmic bytes per second (every input
element read once, B and C once per (batch, token), every output written
once, the state never touching HBM) and channel*tokens per second; the HBM
fraction is against MI355X's 8 TB/s.  The scan is bound by vector
arithmetic (one exp and four fp32 operations per token and state, plus the
per-token softplus and silu), so the line also reports the fraction of the
chip's vector issue rate and of the measured arithmetic ceiling (a
register-only kernel with the same instruction mix, libssm_micro.so), and
names the binding one.

Before timing, every workload runs untimed launches for at least 200 ms
beyond the requested warm-up steps, so that the clocks have settled; kernel
durations are medians of per-launch HIP events on the launching stream.

Also measured (secondary, same JSON line): the Mamba-130m-like fp32 layer
scan, the bf16 2.8b-like layer scan, the 1000-step decode update, the
130m-like scan with the width-4 causal conv of the block's conv branch fused
in front, with d_state 64 and with per-channel B/C, the Mamba-2 SSD layer
and its long-context form (segmented and as one segment), the scan backward
on the two layer shapes and the long-context workload, a length sweep, and
the oracle's rate on the other workloads.

Prints ONE JSON line on stdout.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "selective-scan GB/s and channel·tokens/s (1 GPU); % of HBM roofline"
SCAN_KERNEL_SRC = ["selective_state_space_74_amd/csrc/scan_fwd.hip",
                   "selective_state_space_74_amd/csrc/scan_fwd_kernel.h",
                   "selective_state_space_74_amd/csrc/scan_fwd_seg_s1.hip",
                   "selective_state_space_74_amd/csrc/ssm_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_fwd_long_context_bf16_traffic.json")
# Vector issue rate of MI355X from its unit counts and clock: 256 CUs x 4
# SIMDs x 16 lanes x 2.4 GHz = one fp32 VALU lane-instruction per lane per
# clock (the 157.3 TFLOP/s fp32 figure counts packed FMAs, 2 lanes x 2 flops,
# which this build does not generate).
ALU_PEAK_T = 256 * 64 * 2.4e9 / 1e12     # T lane-instructions / s
# Algorithmic lane-instructions per (token, state) step: 2 multiplies, 1 exp,
# 2 FMAs (state, readout), plus per token the delta bias add, softplus
# (4 VALU + 2 transcendentals), silu (3 + 2), Delta*u, D*u, the gate, and one
# per loaded input (u, delta, z), spread over the token's 16 states.
ALU_OPS_PER_STEP = 5 + (11 + 4) / 16
WARM_MS = 200.0                # untimed launches before any timing, at least


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scan_bytes(batch, dim, L, N, esz, last_state=True, h0=False, gate=True, ngroups=0):
    """Algorithmic bytes of one prefill scan."""
    io = batch * dim * L * esz * (3 + (1 if gate else 0))   # u, delta, out (+ z)
    bc = 2 * batch * max(ngroups, 1) * N * L * esz          # B, C once per (batch, group, token)
    params = dim * N * 4 + 2 * dim * 4                      # A, D, bias
    st = batch * dim * N * 4 * ((1 if last_state else 0) + (1 if h0 else 0))
    return io + bc + params + st


def decode_bytes(batch, dim, N, esz):
    """Algorithmic bytes of one decode step."""
    state = 2 * batch * dim * N * 4                         # read + write
    io = 4 * batch * dim * esz                              # x, dt, z, out
    bc = 2 * batch * N * esz
    params = dim * N * 4 + 2 * dim * 4
    return state + io + bc + params


def kernel_source_sha():
    h = hashlib.sha256()
    for rel in SCAN_KERNEL_SRC:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the scan kernel from the committed rocprofv3
    counter runs, or None when the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def timed_launches(fn, iters, torch):
    """Per-launch durations (ms) with HIP events on the launching stream:
    (median, min, mean)."""
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return float(np.median(ms)), float(np.min(ms)), float(np.mean(ms))


def warm(fn, n, torch, min_ms=WARM_MS):
    """n untimed launches, then more until at least min_ms have elapsed (the
    clocks settle under sustained load).  Returns (launches, ms)."""
    t0 = time.perf_counter()
    i = 0
    while i < n or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn(i)
        i += 1
        if i >= n:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i, (time.perf_counter() - t0) * 1e3


def bench_scan(cfg, steps, warmup, torch, ssm, si, rotate=2, conv=0, graph=False):
    """Times `steps` full scans; returns a dict of measurements.  With graph,
    the `steps` launches are captured once into a HIP graph (torch.cuda.graph,
    a private stream at default priority) and the timed region is one replay
    of it, after an untimed one: back-to-back launches without the host's
    per-call dispatch between them."""
    dev = "cuda"
    sets = []
    for r in range(rotate):
        if cfg.seqlen * cfg.batch * (cfg.dim + 2 * max(cfg.ngroups, 1) * cfg.dstate) > 200_000_000:
            t = si.scan_inputs_device(cfg, dev)
        else:
            t = si.to_torch(si.scan_inputs_for(cfg), dev)
        sets.append(t)
        if r == 0 and rotate > 1 and cfg.seqlen * cfg.dim * cfg.batch > 1_000_000_000:
            break   # the long config alone exceeds every cache; one set is enough
    io = sets[0]["u"].dtype
    outs = [torch.empty_like(s["u"]) for s in sets]
    lasts = [torch.empty((cfg.batch, cfg.dim, cfg.dstate), device=dev) for _ in sets]
    # the segment workspace, allocated once outside the timed region
    a = ssm.ScanArgs()
    a.batch, a.dim, a.seqlen, a.dstate = cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate
    nws = ssm.scan_workspace_size(a)
    ws = torch.empty(max(1, nws), dtype=torch.uint8, device=dev) if nws else False

    ckw = {}
    if conv:
        # the fused conv branch: u is the conv input, weights (dim, conv)
        g = torch.Generator(device=dev)
        g.manual_seed(cfg.seed)
        ckw = dict(conv_weight=torch.randn(cfg.dim, conv, device=dev, generator=g) / conv ** 0.5,
                   conv_bias=torch.zeros(cfg.dim, device=dev))

    def step(i):
        k = i % len(sets)
        s = sets[k]
        ssm.selective_scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                               delta_bias=s["delta_bias"], out=outs[k], last_state=lasts[k],
                               workspace=ws, **ckw)

    wl, wms = warm(step, warmup, torch)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    kern_ms, kern_min, kern_mean = timed_launches(step, max(10, min(steps, 200)), torch)
    esz = 2 if io == torch.bfloat16 else 4
    nbytes = scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, esz, ngroups=cfg.ngroups)
    if conv:
        nbytes += cfg.dim * conv * 4 + cfg.dim * 4              # conv weights and bias
    ms_step = wall / steps * 1e3
    res = dict(ms_per_step=ms_step, kernel_ms=kern_ms, kernel_ms_min=kern_min,
               kernel_ms_mean=kern_mean, bytes=nbytes,
               gbps=nbytes / (ms_step * 1e-3) / 1e9,
               kernel_gbps=nbytes / (kern_ms * 1e-3) / 1e9,
               channel_tokens_per_s=cfg.batch * cfg.dim * cfg.seqlen / (ms_step * 1e-3),
               io_dtype="bf16" if esz == 2 else "f32",
               launch="one HIP graph of the timed steps" if graph else "eager launches",
               warmup_launches=wl, warmup_ms=round(wms, 1),
               segment_workspace_bytes=nws)
    res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBS
    del sets, outs, lasts, ws
    torch.cuda.empty_cache()
    return res


def scan_bwd_bytes(batch, dim, L, N, esz, gate=True):
    """Algorithmic bytes of one scan backward: u, delta, dout (+ z) and B, C
    read once, the forward's checkpoints read once, du, ddelta (+ dz) written
    once, dB, dC (fp32) written once, parameters and their gradients."""
    io = batch * dim * L * esz * (5 + (2 if gate else 0))   # u, delta, dout, du, ddelta (+ z, dz)
    bc = 2 * batch * N * L * esz + 2 * batch * N * L * 4    # B, C in; dB, dC out
    ck = batch * dim * ((L + 15) // 16) * N * 4
    params = 2 * (dim * N * 4 + 2 * dim * 4)                # A, D, bias and their gradients
    return io + bc + ck + params


def bench_bwd(cfg, steps, torch, ssm, si):
    """Times the scan backward (from the forward's checkpoints); long
    sequences with few channels run segmented (the workspace holds the
    segments' adjoint aggregates)."""
    dev = "cuda"
    big = cfg.seqlen * cfg.batch * cfg.dim > 200_000_000
    t = si.scan_inputs_device(cfg, dev) if big else si.to_torch(si.scan_inputs_for(cfg), dev)
    ck = torch.empty(ssm.checkpoint_shape(cfg.batch, cfg.dim, cfg.seqlen), dtype=torch.float32,
                     device=dev)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"])
    ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], checkpoints=ck, **kw)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    dout = torch.randn(t["u"].shape, generator=gen, device=dev).to(t["u"].dtype)
    # the dB/dC partial-sum workspace, allocated once outside the timed region
    a = ssm.ScanBwdArgs()
    a.batch, a.dim, a.seqlen, a.dstate = cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate
    ws = torch.empty(max(1, ssm.scan_bwd_workspace_size(a)), dtype=torch.uint8, device=dev)

    def step(i):
        ssm.selective_scan_bwd(dout, t["u"], t["delta"], t["A"], t["B"], t["C"], ck, workspace=ws,
                               **kw)

    wl, wms = warm(step, 5, torch)
    kern_ms, kern_min, kern_mean = timed_launches(step, steps, torch)
    esz = 2 if t["u"].dtype == torch.bfloat16 else 4
    nbytes = scan_bwd_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, esz)
    res = dict(kernel_ms=kern_ms, kernel_ms_min=kern_min, kernel_ms_mean=kern_mean, bytes=nbytes,
               gbps=nbytes / (kern_ms * 1e-3) / 1e9,
               channel_tokens_per_s=cfg.batch * cfg.dim * cfg.seqlen / (kern_ms * 1e-3),
               warmup_launches=wl, warmup_ms=round(wms, 1))
    res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBS
    res["dBdC"] = "per-block partial sums" if ws.numel() > 1 else "device atomics"
    del t, ck, dout, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(cfg, torch, ssm, si, warmup=20, conv=0, state_sets=1):
    """1000 consecutive decode steps with per-step inputs pre-resident (with
    conv > 0 the conv branch's state update of that width is fused in).
    With state_sets > 1, step s updates state set s % state_sets: the sets
    together (84 MB each here) exceed the 256 MB Infinity Cache, so every
    step's state comes from HBM (the cold cross-check)."""
    dev = "cuda"
    d = si.decode_inputs_device(cfg, device=dev)
    states = [torch.zeros((cfg.batch, cfg.dim, cfg.dstate), device=dev) for _ in range(state_sets)]
    out = torch.empty((cfg.steps, cfg.batch, cfg.dim), dtype=d["x"].dtype, device=dev)
    ckw = {}
    if conv:
        ckw = dict(conv_state=torch.zeros((cfg.batch, cfg.dim, conv), device=dev),
                   conv_weight=torch.full((cfg.dim, conv), 1.0 / conv, device=dev),
                   conv_bias=torch.zeros(cfg.dim, device=dev))

    def step(i):
        s = i % cfg.steps
        ssm.selective_state_update(states[i % state_sets], d["x"][s], d["dt"][s], d["A"], d["B"][s],
                                   d["C"][s], D=d["D"], z=d["z"][s], dt_bias=d["dt_bias"],
                                   out=out[s], **ckw)

    wl, wms = warm(step, warmup, torch)
    for st in states:
        st.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(cfg.steps):
        step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms, kern_min, kern_mean = timed_launches(step, 200, torch)
    esz = 2 if d["x"].dtype == torch.bfloat16 else 4
    nbytes = decode_bytes(cfg.batch, cfg.dim, cfg.dstate, esz)
    if conv:
        nbytes += 2 * cfg.batch * cfg.dim * conv * 4 + cfg.dim * (conv + 1) * 4
    ms_step = wall / cfg.steps * 1e3
    res = dict(steps=cfg.steps, ms_total=wall * 1e3, ms_per_step=ms_step, kernel_ms=kern_ms,
               kernel_ms_min=kern_min, kernel_ms_mean=kern_mean, bytes_per_step=nbytes,
               warmup_launches=wl, warmup_ms=round(wms, 1),
               gbps=nbytes / (ms_step * 1e-3) / 1e9,
               kernel_gbps=nbytes / (kern_ms * 1e-3) / 1e9,
               channel_tokens_per_s=cfg.batch * cfg.dim / (ms_step * 1e-3))
    res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBS
    res["state_sets"] = state_sets
    del d, out, states
    torch.cuda.empty_cache()
    return res


def ssd_bytes(batch, L, H, P, G, N, esz, gate=True, last_state=True):
    """Algorithmic bytes of one Mamba-2 SSM prefill: x, out (+ z) and dt read
    or written once, B and C once per (batch, token, group), the per-head
    parameters, and the final state."""
    io = batch * L * H * P * esz * (2 + (1 if gate else 0))
    dt = batch * L * H * esz
    bc = 2 * batch * L * G * N * esz
    params = 3 * H * 4
    st = batch * H * P * N * 4 if last_state else 0
    return io + dt + bc + params + st


def bench_ssd(cfg, steps, torch, ssm, si, segmented=True):
    """Times the Mamba-2 SSM prefill on device-drawn inputs (two input sets
    in rotation; one for sequences of 1M tokens and more).  With
    `segmented`, the library's workspace is allocated once outside the timed
    region (long sequences with few heads then run as segments); without it
    each sequence runs as one segment."""
    sets = [si.ssd_inputs_device(cfg, "cuda")]
    if cfg.batch * cfg.seqlen < (1 << 20):
        sets.append({k: v.clone() for k, v in sets[0].items()})
    outs = [torch.empty_like(s["x"]) for s in sets]
    lasts = [torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), device="cuda")
             for _ in sets]
    a = ssm.SsdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.ngroups, a.dstate = (
        cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate)
    a.io_dtype = ssm.SSM_BF16 if cfg.io_dtype == "bf16" else ssm.SSM_F32
    nws = ssm.ssd_workspace_size(a) if segmented else 0
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else False

    def step(i):
        k = i % len(sets)
        s = sets[k]
        ssm.ssd_scan_fwd(s["x"], s["dt"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                         dt_bias=s["dt_bias"], out=outs[k], last_state=lasts[k], workspace=ws)

    wl, wms = warm(step, 5, torch)
    kern_ms, kern_min, kern_mean = timed_launches(step, steps, torch)
    esz = 2 if cfg.io_dtype == "bf16" else 4
    nbytes = ssd_bytes(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, esz)
    # matrix-core work of the chunked form: per (batch, head, 64-token chunk),
    # the causal half of the Q x Q scores (k = N), the intra-chunk product,
    # the state product and the state update (k = Q), each 2 flops per MAC
    Q = 64
    chunks = cfg.batch * cfg.nheads * ((cfg.seqlen + Q - 1) // Q)
    macs = chunks * (Q * (Q + 16) // 2 * cfg.dstate + Q * (Q + 16) // 2 * cfg.headdim
                     + 2 * Q * cfg.dstate * cfg.headdim)
    res = dict(kernel_ms=kern_ms, kernel_ms_min=kern_min, kernel_ms_mean=kern_mean, bytes=nbytes,
               gbps=nbytes / (kern_ms * 1e-3) / 1e9, mfma_tflops=2 * macs / (kern_ms * 1e-3) / 1e12,
               token_heads_per_s=cfg.batch * cfg.seqlen * cfg.nheads / (kern_ms * 1e-3),
               warmup_launches=wl, warmup_ms=round(wms, 1), segment_workspace_bytes=nws)
    res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBS
    del sets, outs, lasts, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, si, max_s=30.0):
    """The fp64 oracle, as it stands, on the host cores, over a layer workload
    (whole batch rows at full length).  It runs batch row 0 first and adds
    further batch rows while the projected total stays under max_s; when the
    whole workload takes under 2 s it is repeated (up to 5 s in all) and the
    median run is reported."""
    import oracle
    inp = si.scan_inputs_for(cfg)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1

    def run(k):
        t0 = time.perf_counter()
        oracle.selective_scan(inp["u"][:k], inp["delta"][:k], inp["A"], inp["B"][:k],
                              inp["C"][:k], D=inp["D"], z=inp["z"][:k],
                              delta_bias=inp["delta_bias"], nthreads=threads,
                              return_last_state=True)
        return time.perf_counter() - t0

    t1 = run(1)
    k = int(max(1, min(cfg.batch, max_s / max(t1, 1e-9))))
    dt = run(k) if k > 1 else t1
    reps = 1
    if dt < 2.0:
        reps = int(min(20, max(1, 5.0 / max(dt, 1e-9))))
        dt = float(np.median([dt] + [run(k) for _ in range(reps - 1)]))
    used = oracle.selective_scan.last_threads
    rows = k * cfg.dim
    esz = 2 if cfg.io_dtype == "bf16" else 4
    nbytes = scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, esz) * k / cfg.batch
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "channel_tokens_per_s": rows * cfg.seqlen / dt, "seconds": round(dt, 3),
            "sample": f"{k} of {cfg.batch} batch rows ({rows} channel rows) of {cfg.name} "
                      f"at full L={cfg.seqlen}; fp64 oracle with {used} OpenMP threads; "
                      f"median of {reps} run(s)"}


def cpu_baseline_channels(cfg, si, torch, channels=128, target_s=10.0):
    """The fp64 oracle, as it stands, on the host cores, over a seeded sample
    of `channels` channels of a single-sequence workload at its full length
    (the device-drawn inputs of those channels, read back).  The sample is
    run repeatedly until about target_s seconds of CPU work have been done;
    the median run is reported, scaled to the workload's bytes per
    channel-token."""
    import oracle
    t = si.scan_inputs_device(cfg, "cuda")
    ch = np.sort(np.random.default_rng(cfg.seed).choice(cfg.dim, channels, replace=False))
    idx = torch.from_numpy(ch).to("cuda")
    host = lambda x: x.float().cpu().numpy()
    sel = lambda x: host(x.index_select(1, idx))
    u, dl, z = sel(t["u"]), sel(t["delta"]), sel(t["z"])
    B, C = host(t["B"]), host(t["C"])
    A, D, bias = host(t["A"])[ch], host(t["D"])[ch], host(t["delta_bias"])[ch]
    del t
    torch.cuda.empty_cache()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1

    def run():
        t0 = time.perf_counter()
        oracle.selective_scan(u, dl, A, B, C, D=D, z=z, delta_bias=bias, nthreads=threads,
                              return_last_state=True)
        return time.perf_counter() - t0

    runs = [run()]
    while sum(runs) < target_s and len(runs) < 50:
        runs.append(run())
    dt = float(np.median(runs))
    used = oracle.selective_scan.last_threads
    ct = cfg.batch * channels * cfg.seqlen
    esz = 2 if cfg.io_dtype == "bf16" else 4
    nbytes = scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, esz) * channels / cfg.dim
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "channel_tokens_per_s": ct / dt, "seconds": round(dt, 3),
            "sample": f"{channels} of {cfg.dim} channels (seeded choice) of {cfg.name} at its full "
                      f"L={cfg.seqlen}, bytes scaled by {channels}/{cfg.dim}; fp64 oracle with "
                      f"{used} OpenMP threads; median of {len(runs)} run(s), "
                      f"{sum(runs):.1f} s of CPU work"}


def oracle_timings(si, torch):
    """The fp64 oracle on the other workloads, as it stands: the tiny and the
    130m-like configs single-threaded (one batch row of the latter), the
    long-context config's 16-channel parity sample at its full length, and
    the decode workload on every channel for its first 100 steps."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1
    res = {}

    def timed(fn, min_s=1.0):
        runs = []
        while not runs or (sum(runs) < min_s and len(runs) < 20):
            t0 = time.perf_counter()
            fn()
            runs.append(time.perf_counter() - t0)
        return float(np.median(runs)), len(runs)

    for cfg, rows in ((si.TINY, None), (si.LAYER_130M, 1)):
        inp = si.scan_inputs_for(cfg)
        k = cfg.batch if rows is None else rows
        sl = lambda x: x[:k]
        dt, n = timed(lambda: oracle.selective_scan(sl(inp["u"]), sl(inp["delta"]), inp["A"],
                                                    sl(inp["B"]), sl(inp["C"]), D=inp["D"],
                                                    z=sl(inp["z"]), delta_bias=inp["delta_bias"],
                                                    nthreads=1, return_last_state=True))
        ct = k * cfg.dim * cfg.seqlen
        res[f"{cfg.name}-1-thread"] = {"channel_tokens_per_s": ct / dt, "seconds": round(dt, 4),
                                       "sample": f"{k} of {cfg.batch} batch rows, median of {n}"}
    c3 = si.LONG_CONTEXT
    t = si.scan_inputs_device(c3, "cuda")
    ch = np.sort(np.random.default_rng(3).choice(c3.dim, 16, replace=False))
    idx = torch.from_numpy(ch).to("cuda")
    host = lambda x: x.float().cpu().numpy()
    sel = lambda x: host(x.index_select(1, idx))
    u, dl, z, B, C = sel(t["u"]), sel(t["delta"]), sel(t["z"]), host(t["B"]), host(t["C"])
    A, D, bias = host(t["A"])[ch], host(t["D"])[ch], host(t["delta_bias"])[ch]
    del t
    torch.cuda.empty_cache()
    dt, n = timed(lambda: oracle.selective_scan(u, dl, A, B, C, D=D, z=z, delta_bias=bias,
                                                nthreads=threads, return_last_state=True))
    res[f"{c3.name}-16-channel-sample"] = {
        "channel_tokens_per_s": 16 * c3.seqlen / dt, "seconds": round(dt, 4),
        "threads": oracle.selective_scan.last_threads,
        "sample": f"the 16 parity channels over L={c3.seqlen}, median of {n}"}
    del u, dl, z, B, C
    dc = si.DECODE_CONFIG
    d = si.decode_inputs_device(dc, steps=100, device="cuda")
    steps = [{k: host(d[k][s]) for k in ("x", "dt", "z", "B", "C")} for s in range(100)]
    A, D, bias = host(d["A"]), host(d["D"]), host(d["dt_bias"])
    del d
    torch.cuda.empty_cache()

    def dec():
        st = np.zeros((dc.batch, dc.dim, dc.dstate))
        for v in steps:
            _, st = oracle.state_update(st, v["x"], v["dt"], A, v["B"], v["C"], D=D, z=v["z"],
                                        dt_bias=bias, nthreads=threads)
    dt, n = timed(dec, min_s=0.1)
    res[f"{dc.name}-100-steps"] = {
        "channel_tokens_per_s": 100 * dc.batch * dc.dim / dt, "seconds": round(dt, 4),
        "ms_per_step": round(dt * 10, 3),
        "sample": f"every channel, the first 100 steps, {threads} threads, median of {n}"}
    return res


def length_sweep(torch, ssm, si, lengths=(1024, 2048, 4096, 8192, 16384)):
    """The scan of the pages' length sweep shape: one sequence of the
    Mamba(d_model=1024, d_state=16, expand=2) block, d_inner 2048, fp32, at
    doubling lengths; kernel medians after the >= 200 ms warm-up."""
    out = {}
    for L in lengths:
        cfg = si.ScanConfig(f"sweep-L{L}", 1, 2048, L, 16, "f32", 10 + L)
        r = bench_scan(cfg, 50, 5, torch, ssm, si, rotate=1)
        out[str(L)] = round(r["kernel_ms"] * 1e3, 2)
    ls = sorted(out, key=int)
    return {"what": "batch 1, d_inner 2048, d_state 16, fp32: kernel median us per length",
            "kernel_us": out,
            "ratio_per_doubling": [round(out[b] / out[a], 3) for a, b in zip(ls, ls[1:])]}


def valu_ceiling(torch, lanes=2048 * 256, blocks=4096, reps=10):
    """(token, state) steps per second of the register-only kernel that
    executes the scan's unavoidable instruction mix (libssm_micro.so), median
    of `reps` timed launches after a >= 200 ms warm-up."""
    import ctypes
    path = os.path.join(ROOT, "selective_state_space_74_amd", "libssm_micro.so")
    lib = ctypes.CDLL(path)
    lib.ssm_micro_valu_mix.restype = ctypes.c_int
    lib.ssm_micro_valu_mix.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_void_p]
    out = torch.empty(lanes, device="cuda")

    def step(i):
        st = lib.ssm_micro_valu_mix(ctypes.c_void_p(out.data_ptr()), lanes, blocks,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"ssm_micro_valu_mix: hip error {st}")

    warm(step, 3, torch)
    ms, mn, _ = timed_launches(step, reps, torch)
    steps = lanes * blocks * 16
    del out
    return {"steps_per_s": steps / (ms * 1e-3), "kernel_ms": round(ms, 4),
            "steps": steps, "what": "register-only kernel, per 16 (token, state) steps of a lane: "
                                    "16 x (2 mul, exp, 2 fma) + the per-token softplus, silu, "
                                    "Delta*u, D*u, gate and input operations; 8 waves per SIMD"}


def mfma_rate(torch, k, lanes=2048 * 256, iters=4096, reps=10):
    """Dense bf16 matrix throughput of v_mfma_f32_16x16x{k}_bf16 (k 16 or
    32) from a register-only kernel (libssm_micro.so; eight independent
    accumulator chains per wavefront, 8 wavefronts per SIMD), median of
    `reps` timed launches after a >= 200 ms warm-up."""
    import ctypes
    path = os.path.join(ROOT, "selective_state_space_74_amd", "libssm_micro.so")
    lib = ctypes.CDLL(path)
    lib.ssm_micro_mfma_rate.restype = ctypes.c_int
    lib.ssm_micro_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p]
    out = torch.empty(lanes, device="cuda")

    def step(i):
        st = lib.ssm_micro_mfma_rate(ctypes.c_void_p(out.data_ptr()), lanes, iters, k,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"ssm_micro_mfma_rate: hip error {st}")

    warm(step, 3, torch)
    ms, _, _ = timed_launches(step, reps, torch)
    instrs = lanes // 64 * iters * 8
    flops = instrs * 2 * 16 * 16 * k
    del out
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return {"k": k, "kernel_ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "instr_per_clk_per_cu_at_2p4ghz": round(instrs / (ms * 1e-3) / 2.4e9 / cus, 3)}


def stream_copy(torch, reps=10):
    """Measured streaming bandwidth of the device: a plain 1 GiB -> 1 GiB
    device copy, timed with HIP events (the practical ceiling that a
    read-once, write-once kernel can reach, beside the 8 TB/s spec)."""
    n = 1 << 28                      # 2^28 fp32 = 1 GiB
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * 4 * n / (ms * 1e-3) / 1e9


def calibration_copy(torch, launches):
    """A plain copy kernel of known size (reads 1 GiB, writes 1 GiB) so that
    the FETCH_SIZE / WRITE_SIZE counters can be scaled to bytes."""
    n = (1 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for i in range(launches):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def profile_long(cfg, torch, ssm, si, launches=5):
    """The headline scan (all its launches) after a >= 200 ms warm-up, then the
    calibration copy; for rocprofv3."""
    t = si.scan_inputs_device(cfg, "cuda")
    out = torch.empty_like(t["u"])
    last = torch.empty((cfg.batch, cfg.dim, cfg.dstate), device="cuda")
    a = ssm.ScanArgs()
    a.batch, a.dim, a.seqlen, a.dstate = cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate
    ws = torch.empty(max(1, ssm.scan_workspace_size(a)), dtype=torch.uint8, device="cuda")

    def step(i):
        ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               delta_bias=t["delta_bias"], out=out, last_state=last, workspace=ws)

    wl, _ = warm(step, 1, torch)
    kern_ms, _, _ = timed_launches(step, launches, torch)
    del t, out, last, ws
    torch.cuda.empty_cache()
    calibration_copy(torch, launches)
    esz = 2 if cfg.io_dtype == "bf16" else 4
    log(f"[profile] {wl} warm-up + {launches} timed scans of {cfg.name} "
        f"({scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, esz)} algorithmic bytes each; "
        f"HIP events median {kern_ms:.3f} ms per scan, all launches), {launches} copy launches "
        f"(1 GiB read + 1 GiB write)")


def profile_layer(cfg, torch, ssm, si, launches=10, cfg2=None):
    """Layer scan launches (and, with cfg2, as many of a second layer
    afterwards), decode steps on the decode workload, and the calibration
    copy; for rocprofv3."""
    for c in (cfg,) + ((cfg2,) if cfg2 is not None else ()):
        t = si.to_torch(si.scan_inputs_for(c), "cuda")
        out = torch.empty_like(t["u"])
        last = torch.empty((c.batch, c.dim, c.dstate), device="cuda")
        for i in range(launches):
            ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                   delta_bias=t["delta_bias"], out=out, last_state=last)
        torch.cuda.synchronize()
        del t, out, last
    dc = si.DECODE_CONFIG
    d = si.decode_inputs_device(dc, steps=launches, device="cuda")
    state = torch.zeros((dc.batch, dc.dim, dc.dstate), device="cuda")
    dout = torch.empty((dc.batch, dc.dim), dtype=d["x"].dtype, device="cuda")
    for s in range(launches):
        ssm.selective_state_update(state, d["x"][s], d["dt"][s], d["A"], d["B"][s], d["C"][s],
                                   D=d["D"], z=d["z"][s], dt_bias=d["dt_bias"], out=dout)
    torch.cuda.synchronize()
    del d, state, dout
    calibration_copy(torch, launches)
    extra = ""
    if cfg2 is not None:
        extra = (f", then {launches} of {cfg2.name} "
                 f"({scan_bytes(cfg2.batch, cfg2.dim, cfg2.seqlen, cfg2.dstate, 2)} bytes each)")
    log(f"[profile] {launches} scan launches ({scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, 4)}"
        f" algorithmic bytes each){extra}, {launches} decode steps "
        f"({decode_bytes(dc.batch, dc.dim, dc.dstate, 2)} bytes each), {launches} copy launches "
        f"(1 GiB read + 1 GiB write)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only the headline scan (warm-up, then 5 scans) and a 1 GiB copy kernel "
                         "(5 launches) that calibrates the HBM byte counters; for rocprofv3")
    ap.add_argument("--profile-layer", action="store_true",
                    help="only the 130m-like and the 2.8b-like layer scans (10 launches each), "
                         "10 decode steps and the calibration copy; for rocprofv3")
    ap.add_argument("--profile-general", action="store_true",
                    help="only the 130m-like layer with the width-4 conv fused, with 64 states "
                         "and with per-channel B/C (10 launches each); for rocprofv3")
    ap.add_argument("--profile-ssd", action="store_true",
                    help="only the Mamba-2 SSD layer (10 launches) and the long-context SSD "
                         "layer (3 segmented launches); for rocprofv3")
    ap.add_argument("--micro-mfma", action="store_true",
                    help="only the bf16 matrix-instruction rate micro-benchmark (k = 16 and k = 32); "
                         "prints one JSON line")
    ap.add_argument("--profile-bwd", action="store_true",
                    help="only the scan backward of the 130m-like and the 2.8b-like layer "
                         "(10 launches each), then the calibration copy; for rocprofv3")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the scan would shard by batch rows and channel blocks, with no communication between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_74_amd as ssm
    import synth_inputs as si

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    ssm.lib()
    torch.cuda.init()

    head = si.LONG_CONTEXT           # the long-context scan: the largest single-GPU workload
    layer = si.LAYER_130M
    if args.profile:
        profile_long(head, torch, ssm, si)
        return
    if args.profile_layer:
        profile_layer(layer, torch, ssm, si, cfg2=si.LAYER_2P8B)
        return
    if args.profile_general:
        # the 130m-like layer with the width-4 conv fused, with 64 states, and
        # with per-channel B/C (10 launches each)
        g = torch.Generator(device="cuda")
        g.manual_seed(layer.seed)
        for name, cg, conv in (("conv4", layer, 4),
                               ("dstate64", dataclasses.replace(layer, dstate=64), 0),
                               ("bc-per-channel", dataclasses.replace(layer, ngroups=layer.dim), 0)):
            t = si.to_torch(si.scan_inputs_for(cg), "cuda")
            kw = {}
            if conv:
                kw = dict(conv_weight=torch.randn(cg.dim, conv, device="cuda", generator=g) / conv ** 0.5,
                          conv_bias=torch.zeros(cg.dim, device="cuda"))
            out = torch.empty_like(t["u"])
            for _ in range(10):
                ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                       delta_bias=t["delta_bias"], out=out, **kw)
            torch.cuda.synchronize()
            del t, out
            log(f"[profile] 10 launches of {layer.name} ({name})")
        return
    if args.profile_ssd:
        cs = si.SSD_CONFIG
        t = si.ssd_inputs_device(cs, "cuda")
        out = torch.empty_like(t["x"])
        for _ in range(10):
            ssm.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             dt_bias=t["dt_bias"], out=out)
        torch.cuda.synchronize()
        del t, out
        cl = si.SSD_LONG_CONFIG
        t = si.ssd_inputs_device(cl, "cuda")
        out = torch.empty_like(t["x"])
        for _ in range(3):   # segmented (the binding allocates the workspace)
            ssm.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             dt_bias=t["dt_bias"], out=out)
        torch.cuda.synchronize()
        log(f"[profile] 10 launches of the SSD layer {cs.name}, 3 of {cl.name} (segmented)")
        return
    if args.micro_mfma:
        print(json.dumps({"mfma_bf16_16x16": [mfma_rate(torch, k) for k in (16, 32)]}), flush=True)
        return
    if args.profile_bwd:
        for cb in (layer, si.LAYER_2P8B):
            t = si.to_torch(si.scan_inputs_for(cb), "cuda")
            ck = torch.empty(ssm.checkpoint_shape(cb.batch, cb.dim, cb.seqlen),
                             dtype=torch.float32, device="cuda")
            kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"])
            ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], checkpoints=ck, **kw)
            dout = torch.randn_like(t["u"])
            for _ in range(10):
                ssm.selective_scan_bwd(dout, t["u"], t["delta"], t["A"], t["B"], t["C"], ck, **kw)
            torch.cuda.synchronize()
            del t, ck, dout
            log(f"[profile] 10 launches of the scan backward on {cb.name} "
                f"({scan_bwd_bytes(cb.batch, cb.dim, cb.seqlen, cb.dstate, 4 if cb.io_dtype == 'f32' else 2)}"
                f" algorithmic bytes each)")
        calibration_copy(torch, 10)
        log("[profile] 10 copy launches (1 GiB read + 1 GiB write)")
        return
    log(f"[bench] headline {head.name}: warmup {args.warmup} (+ >= {WARM_MS:.0f} ms), "
        f"steps {args.steps}")
    r = bench_scan(head, args.steps, args.warmup, torch, ssm, si, rotate=1)
    log(f"[bench] headline {r['gbps']:.1f} GB/s, kernel median {r['kernel_ms']:.3f} ms")
    ceiling = valu_ceiling(torch)
    log(f"[bench] measured arithmetic ceiling {ceiling['steps_per_s'] / 1e12:.3f} T steps/s")

    secondary = {}
    if not args.no_secondary:
        log(f"[bench] secondary {layer.name}")
        secondary[layer.name] = bench_scan(layer, max(20, args.steps), args.warmup, torch, ssm, si)
        log(f"[bench] {layer.name} {secondary[layer.name]['gbps']:.1f} GB/s, "
            f"kernel median {secondary[layer.name]['kernel_ms'] * 1e3:.1f} us")
        c2 = si.LAYER_2P8B
        log(f"[bench] secondary {c2.name}")
        secondary[c2.name] = bench_scan(c2, max(20, args.steps), 5, torch, ssm, si)
        log(f"[bench] {c2.name} {secondary[c2.name]['gbps']:.1f} GB/s, "
            f"kernel median {secondary[c2.name]['kernel_ms'] * 1e3:.1f} us")
        log(f"[bench] secondary {si.DECODE_CONFIG.name}")
        secondary[si.DECODE_CONFIG.name] = bench_decode(si.DECODE_CONFIG, torch, ssm, si)
        log(f"[bench] decode {secondary[si.DECODE_CONFIG.name]['gbps']:.1f} GB/s")
        key = f"{si.DECODE_CONFIG.name}-cold-4-state-sets"
        log(f"[bench] secondary {key}")
        secondary[key] = bench_decode(si.DECODE_CONFIG, torch, ssm, si, state_sets=4)
        log(f"[bench] {key} {secondary[key]['gbps']:.1f} GB/s")
        key = f"{si.DECODE_CONFIG.name}-conv4-fused"
        log(f"[bench] secondary {key}")
        secondary[key] = bench_decode(si.DECODE_CONFIG, torch, ssm, si, conv=4)
        log(f"[bench] {key} {secondary[key]['gbps']:.1f} GB/s")
        key = f"{layer.name}-conv4-fused"
        log(f"[bench] secondary {key}")
        secondary[key] = bench_scan(layer, max(20, args.steps), 5, torch, ssm, si, conv=4)
        log(f"[bench] {key} {secondary[key]['gbps']:.1f} GB/s, "
            f"kernel {secondary[key]['kernel_ms'] * 1e3:.1f} us")
        # the generalised kernel: 64 states (four slots per lane), and B/C of
        # its own per channel (lane mode)
        for cg in (dataclasses.replace(layer, name=f"{layer.name}-dstate64", dstate=64),
                   dataclasses.replace(layer, name=f"{layer.name}-bc-per-channel", ngroups=layer.dim)):
            log(f"[bench] secondary {cg.name}")
            secondary[cg.name] = bench_scan(cg, 20, 5, torch, ssm, si)
            log(f"[bench] {cg.name} {secondary[cg.name]['gbps']:.1f} GB/s, "
                f"kernel {secondary[cg.name]['kernel_ms'] * 1e3:.1f} us")
        cs = si.SSD_CONFIG
        log(f"[bench] secondary {cs.name}")
        secondary[cs.name] = bench_ssd(cs, 100, torch, ssm, si)
        log(f"[bench] {cs.name} {secondary[cs.name]['gbps']:.1f} GB/s, "
            f"{secondary[cs.name]['kernel_ms'] * 1e3:.1f} us, "
            f"{secondary[cs.name]['mfma_tflops']:.1f} TFLOP/s on the matrix cores")
        cl = si.SSD_LONG_CONFIG
        for seg in (True, False):
            key = cl.name if seg else f"{cl.name}-one-segment"
            log(f"[bench] secondary {key}")
            secondary[key] = bench_ssd(cl, 10, torch, ssm, si, segmented=seg)
            log(f"[bench] {key} {secondary[key]['gbps']:.1f} GB/s, "
                f"{secondary[key]['kernel_ms']:.2f} ms")
        for cb in (si.LAYER_130M, si.LAYER_2P8B, si.LONG_CONTEXT):
            key = f"{cb.name}-backward"
            log(f"[bench] secondary {key}")
            secondary[key] = bench_bwd(cb, 20, torch, ssm, si)
            log(f"[bench] {key} {secondary[key]['gbps']:.1f} GB/s, "
                f"{secondary[key]['kernel_ms'] * 1e3:.1f} us")

    if not args.no_secondary:
        log("[bench] length sweep")
        secondary["length-sweep-d2048-f32"] = length_sweep(torch, ssm, si)
        log(f"[bench] length sweep {secondary['length-sweep-d2048-f32']['kernel_us']}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline_channels(head, si, torch)
        log(f"[bench] cpu baseline {cpu['value']:.3f} GB/s on {cpu['cores']} threads")
        if not args.no_secondary:
            log("[bench] oracle on the other workloads")
            secondary["oracle"] = oracle_timings(si, torch)

    traffic = measured_traffic()
    steps_tn = head.batch * head.dim * head.seqlen * head.dstate
    ksec = r["kernel_ms"] * 1e-3
    hbm_ach = r["bytes"] / ksec / 1e9
    alu_ach = steps_tn * ALU_OPS_PER_STEP / ksec / 1e12
    hbm_frac, alu_frac = hbm_ach / HBM_PEAK_GBS, alu_ach / ALU_PEAK_T
    valu_frac = (steps_tn / ceiling["steps_per_s"]) / ksec
    copy_gbps = stream_copy(torch)
    log(f"[bench] device copy {copy_gbps:.1f} GB/s")
    alu = {"achieved": round(alu_ach, 3), "peak": round(ALU_PEAK_T, 3),
           "unit": "T lane-instructions/s", "frac": round(alu_frac, 4),
           "ops_per_token_state": ALU_OPS_PER_STEP,
           "what": "algorithmic fp32 VALU lane-instructions (each exp or log counted once) "
                   "against 256 CUs x 64 lanes x 2.4 GHz"}
    hbm = {"achieved": round(hbm_ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(hbm_frac, 4)}
    bound = "alu" if alu_frac >= hbm_frac else "hbm"
    main_ = alu if bound == "alu" else hbm
    line = {
        "metric": METRIC,
        "value": round(r["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded torch Philox on the device: u,z~N(0,1), dt~0.1N(0,1), "
                "B,C~N(0,1), rounded to bf16; numpy PCG64 parameters: "
                "bias=inv-softplus(logU[1e-3,1e-1]), A=-(n+1), D=1)",
        "config": {"workload": "selective scan fwd, long context: batch 1, d_inner 1536, "
                               "L 1048576, d_state 16, bf16 IO, fp32 state and arithmetic, "
                               "silu gate, last_state; all launches of the segmented scan",
                   "batch": head.batch, "dim": head.dim, "seqlen": head.seqlen,
                   "dstate": head.dstate, "io_dtype": "bf16"},
        "channel_tokens_per_s": r["channel_tokens_per_s"],
        "hbm_frac": round(r["hbm_frac"], 4),
        "launch": r["launch"],
        "warmup_launches": r["warmup_launches"],
        "warmup_ms": r["warmup_ms"],
        "roofline": {"bound": bound, "achieved": main_["achieved"], "peak": main_["peak"],
                     "unit": main_["unit"], "frac": main_["frac"], "traffic": traffic,
                     "kernel": "scan_fwd_kernel<bf16> pass 1 (kSeg) + seg_plan_kernel + seg_list_kernel + pass 2 (kFix)",
                     "kernel_ms": round(r["kernel_ms"], 5),
                     "kernel_ms_min": round(r["kernel_ms_min"], 5),
                     "kernel_ms_mean": round(r["kernel_ms_mean"], 5),
                     "timing": "median of per-step HIP events around all four launches",
                     "algorithmic_bytes_per_launch": r["bytes"],
                     "token_state_steps_per_launch": steps_tn,
                     "hbm": hbm, "alu": alu,
                     "valu_frac_of_measured_ceiling": round(valu_frac, 4),
                     "measured_ceiling": ceiling},
        "cpu_baseline": cpu,
        "stream": {"copy_gbps": round(copy_gbps, 1),
                   "frac_of_copy": round(hbm_ach / copy_gbps, 4),
                   "what": "device copy, 1 GiB read + 1 GiB written, HIP events"},
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
