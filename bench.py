#!/usr/bin/env python3
"""Benchmark of the gfx950 selective scan.

Headline: the Mamba-130m-like layer scan (batch 8, d_inner 1536, L 2048,
d_state 16, fp32 IO, silu gate, last_state returned).  One step = one full
prefill scan over the batch with inputs already resident in HBM.  Throughput is
algorithmic bytes per second (every input element read once, B and C once per
(batch, token), every output written once, the state never touching HBM) and
channel*tokens per second; the HBM fraction is against MI355X's 8 TB/s.

Also measured (secondary, same JSON line): the bf16 2.8b-like layer scan, the
1000-step decode update, the headline scan with the width-4 causal conv of the
block's conv branch fused in front, and the scan backward on the two layer
shapes; with --all also the 1M-token scan.

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
                   "selective_state_space_74_amd/csrc/scan_fwd_s1.hip",
                   "selective_state_space_74_amd/csrc/ssm_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_fwd_mamba130m_f32_traffic.json")


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
    """Average kernel duration with HIP events on the launching stream."""
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return float(np.mean(ms)), float(np.min(ms))


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
                               **ckw)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
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
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    kern_ms, kern_min = timed_launches(step, max(10, min(steps, 200)), torch)
    esz = 2 if io == torch.bfloat16 else 4
    nbytes = scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, esz, ngroups=cfg.ngroups)
    if conv:
        nbytes += cfg.dim * conv * 4 + cfg.dim * 4              # conv weights and bias
    ms_step = wall / steps * 1e3
    res = dict(ms_per_step=ms_step, kernel_ms=kern_ms, kernel_ms_min=kern_min, bytes=nbytes,
               gbps=nbytes / (ms_step * 1e-3) / 1e9,
               kernel_gbps=nbytes / (kern_ms * 1e-3) / 1e9,
               channel_tokens_per_s=cfg.batch * cfg.dim * cfg.seqlen / (ms_step * 1e-3),
               io_dtype="bf16" if esz == 2 else "f32",
               launch="one HIP graph of the timed steps" if graph else "eager launches")
    res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBS
    del sets, outs, lasts
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
    """Times the scan backward (from the forward's checkpoints)."""
    dev = "cuda"
    t = si.to_torch(si.scan_inputs_for(cfg), dev)
    ck = torch.empty(ssm.checkpoint_shape(cfg.batch, cfg.dim, cfg.seqlen), dtype=torch.float32,
                     device=dev)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"])
    ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], checkpoints=ck, **kw)
    dout = torch.randn_like(t["u"], dtype=torch.float32).to(t["u"].dtype)
    # the dB/dC partial-sum workspace, allocated once outside the timed region
    a = ssm.ScanBwdArgs()
    a.batch, a.dim, a.seqlen, a.dstate = cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate
    ws = torch.empty(max(1, ssm.scan_bwd_workspace_size(a)), dtype=torch.uint8, device=dev)

    def step(i):
        ssm.selective_scan_bwd(dout, t["u"], t["delta"], t["A"], t["B"], t["C"], ck, workspace=ws,
                               **kw)

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    kern_ms, kern_min = timed_launches(step, steps, torch)
    esz = 2 if t["u"].dtype == torch.bfloat16 else 4
    nbytes = scan_bwd_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, esz)
    res = dict(kernel_ms=kern_ms, kernel_ms_min=kern_min, bytes=nbytes,
               gbps=nbytes / (kern_ms * 1e-3) / 1e9,
               channel_tokens_per_s=cfg.batch * cfg.dim * cfg.seqlen / (kern_ms * 1e-3))
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

    def step(s):
        ssm.selective_state_update(states[s % state_sets], d["x"][s], d["dt"][s], d["A"], d["B"][s],
                                   d["C"][s], D=d["D"], z=d["z"][s], dt_bias=d["dt_bias"],
                                   out=out[s], **ckw)

    for s in range(warmup):
        step(s)
    for st in states:
        st.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(cfg.steps):
        step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms, kern_min = timed_launches(step, 200, torch)
    esz = 2 if d["x"].dtype == torch.bfloat16 else 4
    nbytes = decode_bytes(cfg.batch, cfg.dim, cfg.dstate, esz)
    if conv:
        nbytes += 2 * cfg.batch * cfg.dim * conv * 4 + cfg.dim * (conv + 1) * 4
    ms_step = wall / cfg.steps * 1e3
    res = dict(steps=cfg.steps, ms_total=wall * 1e3, ms_per_step=ms_step, kernel_ms=kern_ms,
               kernel_ms_min=kern_min, bytes_per_step=nbytes,
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


def bench_ssd(cfg, steps, torch, ssm, si):
    """Times the Mamba-2 SSM prefill on device-drawn inputs (two input sets
    in rotation)."""
    sets = [si.ssd_inputs_device(cfg, "cuda")]
    sets.append({k: v.clone() for k, v in sets[0].items()})
    outs = [torch.empty_like(s["x"]) for s in sets]
    lasts = [torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), device="cuda")
             for _ in sets]

    def step(i):
        k = i % 2
        s = sets[k]
        ssm.ssd_scan_fwd(s["x"], s["dt"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                         dt_bias=s["dt_bias"], out=outs[k], last_state=lasts[k])

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    kern_ms, kern_min = timed_launches(step, steps, torch)
    esz = 2 if cfg.io_dtype == "bf16" else 4
    nbytes = ssd_bytes(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, esz)
    # matrix-core work of the chunked form: per (batch, head, 64-token chunk),
    # the causal half of the Q x Q scores (k = N), the intra-chunk product,
    # the state product and the state update (k = Q), each 2 flops per MAC
    Q = 64
    chunks = cfg.batch * cfg.nheads * ((cfg.seqlen + Q - 1) // Q)
    macs = chunks * (Q * (Q + 16) // 2 * cfg.dstate + Q * (Q + 16) // 2 * cfg.headdim
                     + 2 * Q * cfg.dstate * cfg.headdim)
    res = dict(kernel_ms=kern_ms, kernel_ms_min=kern_min, bytes=nbytes,
               gbps=nbytes / (kern_ms * 1e-3) / 1e9, mfma_tflops=2 * macs / (kern_ms * 1e-3) / 1e12,
               token_heads_per_s=cfg.batch * cfg.seqlen * cfg.nheads / (kern_ms * 1e-3))
    res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBS
    del sets, outs, lasts
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, si, max_s=30.0):
    """The fp64 oracle, as it stands, on the host cores, over the headline
    workload (whole batch rows at full length).  It runs batch row 0 first and
    adds further batch rows while the projected total stays under max_s; when
    the whole workload takes under 2 s it is repeated (up to 5 s in all) and
    the median run is reported."""
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
    nbytes = scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, 4) * k / cfg.batch
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "channel_tokens_per_s": rows * cfg.seqlen / dt, "seconds": round(dt, 3),
            "sample": f"{k} of {cfg.batch} batch rows ({rows} channel rows) of the headline "
                      f"workload at full L={cfg.seqlen}; fp64 oracle with {used} OpenMP threads; "
                      f"median of {reps} run(s)"}


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


def profile_run(cfg, torch, ssm, si, launches=10):
    """Headline scan launches, decode steps on the decode workload, and a plain
    copy kernel of known size (reads 1 GiB, writes 1 GiB) so that the
    FETCH_SIZE / WRITE_SIZE counters can be scaled to bytes."""
    t = si.to_torch(si.scan_inputs_for(cfg), "cuda")
    out = torch.empty_like(t["u"])
    last = torch.empty((cfg.batch, cfg.dim, cfg.dstate), device="cuda")
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
    n = (1 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for i in range(launches):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"[profile] {launches} scan launches ({scan_bytes(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, 4)}"
        f" algorithmic bytes each), {launches} decode steps "
        f"({decode_bytes(dc.batch, dc.dim, dc.dstate, 2)} bytes each), {launches} copy launches "
        f"(1 GiB read + 1 GiB write)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--all", action="store_true", help="also time the 1M-token scan")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the headline's steps as eager launches, not one HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only the headline scan (10 launches) and a 1 GiB copy kernel "
                         "(10 launches) that calibrates the HBM byte counters; for rocprofv3")
    ap.add_argument("--profile-ssd", action="store_true",
                    help="only the Mamba-2 SSD layer (10 launches); for rocprofv3")
    ap.add_argument("--profile-bwd", action="store_true",
                    help="only the scan backward of the 130m-like layer (10 launches); for rocprofv3")
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

    head = si.SCAN_CONFIGS[1]
    if args.profile:
        profile_run(head, torch, ssm, si)
        return
    if args.profile_ssd:
        cs = si.SSD_CONFIG
        t = si.ssd_inputs_device(cs, "cuda")
        out = torch.empty_like(t["x"])
        for _ in range(10):
            ssm.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             dt_bias=t["dt_bias"], out=out)
        torch.cuda.synchronize()
        log(f"[profile] 10 launches of the SSD layer {cs.name}")
        return
    if args.profile_bwd:
        t = si.to_torch(si.scan_inputs_for(head), "cuda")
        ck = torch.empty(ssm.checkpoint_shape(head.batch, head.dim, head.seqlen),
                         dtype=torch.float32, device="cuda")
        kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"])
        ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], checkpoints=ck, **kw)
        dout = torch.randn_like(t["u"])
        for _ in range(10):
            ssm.selective_scan_bwd(dout, t["u"], t["delta"], t["A"], t["B"], t["C"], ck, **kw)
        torch.cuda.synchronize()
        log(f"[profile] 10 launches of the scan backward on {head.name}")
        return
    log(f"[bench] headline {head.name}: warmup {args.warmup}, steps {args.steps}")
    r = bench_scan(head, args.steps, args.warmup, torch, ssm, si, graph=not args.no_graph)
    log(f"[bench] headline {r['gbps']:.1f} GB/s, kernel {r['kernel_ms'] * 1e3:.1f} us")

    secondary = {}
    if not args.no_secondary:
        c2 = si.SCAN_CONFIGS[2]
        log(f"[bench] secondary {c2.name}")
        secondary[c2.name] = bench_scan(c2, max(20, args.steps // 4), 5, torch, ssm, si)
        log(f"[bench] {c2.name} {secondary[c2.name]['gbps']:.1f} GB/s")
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
        c1 = si.SCAN_CONFIGS[1]
        key = f"{c1.name}-conv4-fused"
        log(f"[bench] secondary {key}")
        secondary[key] = bench_scan(c1, max(20, args.steps // 4), 5, torch, ssm, si, conv=4)
        log(f"[bench] {key} {secondary[key]['gbps']:.1f} GB/s, "
            f"kernel {secondary[key]['kernel_ms'] * 1e3:.1f} us")
        # the generalised kernel: 64 states (four slots per lane), and B/C of
        # its own per channel (lane mode)
        for cg in (dataclasses.replace(c1, name=f"{c1.name}-dstate64", dstate=64),
                   dataclasses.replace(c1, name=f"{c1.name}-bc-per-channel", ngroups=c1.dim)):
            log(f"[bench] secondary {cg.name}")
            secondary[cg.name] = bench_scan(cg, max(20, args.steps // 10), 5, torch, ssm, si)
            log(f"[bench] {cg.name} {secondary[cg.name]['gbps']:.1f} GB/s, "
                f"kernel {secondary[cg.name]['kernel_ms'] * 1e3:.1f} us")
        cs = si.SSD_CONFIG
        log(f"[bench] secondary {cs.name}")
        secondary[cs.name] = bench_ssd(cs, 100, torch, ssm, si)
        log(f"[bench] {cs.name} {secondary[cs.name]['gbps']:.1f} GB/s, "
            f"{secondary[cs.name]['kernel_ms'] * 1e3:.1f} us, "
            f"{secondary[cs.name]['mfma_tflops']:.1f} TFLOP/s on the matrix cores")
        for cid in (1, 2):
            cb = si.SCAN_CONFIGS[cid]
            key = f"{cb.name}-backward"
            log(f"[bench] secondary {key}")
            secondary[key] = bench_bwd(cb, 20, torch, ssm, si)
            log(f"[bench] {key} {secondary[key]['gbps']:.1f} GB/s, "
                f"{secondary[key]['kernel_ms'] * 1e3:.1f} us")
        if args.all:
            c3 = si.SCAN_CONFIGS[3]
            log(f"[bench] secondary {c3.name}")
            secondary[c3.name] = bench_scan(c3, 3, 1, torch, ssm, si, rotate=1)
            log(f"[bench] {c3.name} {secondary[c3.name]['gbps']:.1f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(head, si)
        log(f"[bench] cpu baseline {cpu['value']:.3f} GB/s on {cpu['cores']} threads")

    traffic = measured_traffic()
    achieved = r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
    copy_gbps = stream_copy(torch)
    log(f"[bench] device copy {copy_gbps:.1f} GB/s")
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
        "data": "synthetic (seeded numpy PCG64: u,z~N(0,1), dt~0.1N(0,1), B,C~N(0,1), "
                "bias=inv-softplus(logU[1e-3,1e-1]), A=-(n+1), D=1)",
        "config": {"workload": "selective scan fwd, mamba-130m-like layer: batch 8, d_inner 1536, "
                               "L 2048, d_state 16, fp32 IO, silu gate, last_state",
                   "batch": head.batch, "dim": head.dim, "seqlen": head.seqlen,
                   "dstate": head.dstate},
        "channel_tokens_per_s": r["channel_tokens_per_s"],
        "hbm_frac": round(r["hbm_frac"], 4),
        "launch": r["launch"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "scan_fwd_kernel<float>",
                     "kernel_ms": round(r["kernel_ms"], 5),
                     "algorithmic_bytes_per_launch": r["bytes"]},
        "cpu_baseline": cpu,
        "stream": {"copy_gbps": round(copy_gbps, 1),
                   "frac_of_copy": round(achieved / copy_gbps, 4),
                   "what": "device copy, 1 GiB read + 1 GiB written, HIP events"},
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
