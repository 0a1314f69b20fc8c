"""Seeded synthetic inputs for the selective scan and the decode update.

This module only draws random numbers and rounds them to the IO dtype; it holds
none of the scan's arithmetic.  Both the HIP path (through the tests and the
bench) and the fp64 oracle consume the arrays it returns.

Input recipe (the pages use trained language models, which are out of reach, so
seeded data with the layer shapes stands in for them):
  u, z ~ N(0, 1);  dt ~ 0.1 * N(0, 1);  B, C ~ N(0, 1) of shape (batch, N, L),
  shared by every channel of a batch row;
  per-channel bias = inverse softplus of Delta0, Delta0 log-uniform in
  [1e-3, 1e-1] (the Mamba training/inference guide, FAQ item 2: the projection
  bias is initialised so that Delta starts in a target range);
  A[d, n] = -(n + 1), a real diagonal structured initialisation (Mamba model
  notes, section 3.3: A is given a special structure so the state keeps long
  history);  D = 1.
Draw order for one seed: u, z, dt, B, C, then the per-channel Delta0.
bf16 inputs are the fp32 draws rounded to nearest-even.

Small and mid-size configs are drawn with numpy PCG64 (deterministic on every
machine).  The two configs whose inputs run to gigabytes (the 1M-token scan and
the 1000-step decode) are drawn on the device with torch's Philox generator;
the oracle then reads the sampled rows back from those same tensors.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DSTATE = 16


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    dim: int
    seqlen: int
    dstate: int
    io_dtype: str  # "f32" or "bf16"
    seed: int
    last_state: bool = True
    ngroups: int = 0   # B/C groups: 0 = (batch, N, L), else (batch, ngroups, N, L)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    io_dtype: str
    steps: int
    seed: int


# The five workloads: four prefill scans and one decode run.
SCAN_CONFIGS = {
    0: ScanConfig("tiny-f32", 2, 32, 64, DSTATE, "f32", 0),
    1: ScanConfig("mamba130m-layer-f32", 8, 1536, 2048, DSTATE, "f32", 1),
    2: ScanConfig("mamba2.8b-layer-bf16", 4, 5120, 4096, DSTATE, "bf16", 2),
    3: ScanConfig("long-context-bf16", 1, 1536, 1 << 20, DSTATE, "bf16", 3),
}
DECODE_CONFIG = DecodeConfig("decode-b256-d5120-bf16", 256, 5120, DSTATE, "bf16", 1000, 4)
TINY = SCAN_CONFIGS[0]          # batch 2, d_inner 32, L 64, fp32
LAYER_130M = SCAN_CONFIGS[1]    # batch 8, d_inner 1536, L 2048, fp32
LAYER_2P8B = SCAN_CONFIGS[2]    # batch 4, d_inner 5120, L 4096, bf16
LONG_CONTEXT = SCAN_CONFIGS[3]  # batch 1, d_inner 1536, L 1,048,576, bf16


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest-even) and return them as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.float32(np.nan)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _to_io(x: np.ndarray, io_dtype: str) -> np.ndarray:
    return bf16_round(x) if io_dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def delta_bias_from_delta0(delta0: np.ndarray) -> np.ndarray:
    """Bias b with softplus(b) = delta0 (recipe input, computed in fp64)."""
    d0 = np.asarray(delta0, dtype=np.float64)
    return (d0 + np.log(-np.expm1(-d0))).astype(np.float32)


def channel_params(dim: int, dstate: int, rng: np.random.Generator):
    """A (dim, dstate), D (dim), bias (dim) in fp32."""
    lo, hi = math.log(1e-3), math.log(1e-1)
    delta0 = np.exp(rng.uniform(lo, hi, size=dim))
    A = -np.tile(np.arange(1, dstate + 1, dtype=np.float32), (dim, 1))
    D = np.ones(dim, dtype=np.float32)
    return A, D, delta_bias_from_delta0(delta0)


def scan_inputs(batch: int, dim: int, seqlen: int, dstate: int = DSTATE,
                io_dtype: str = "f32", seed: int = 0, ngroups: int = 0) -> dict:
    """Host (numpy) inputs for one prefill scan; IO tensors are fp32 arrays
    whose values are exact in io_dtype.  B and C are (batch, dstate, L), or
    (batch, ngroups, dstate, L) when ngroups >= 1."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((batch, dim, seqlen), dtype=np.float32)
    z = rng.standard_normal((batch, dim, seqlen), dtype=np.float32)
    dt = np.float32(0.1) * rng.standard_normal((batch, dim, seqlen), dtype=np.float32)
    bc = (batch, ngroups, dstate, seqlen) if ngroups else (batch, dstate, seqlen)
    B = rng.standard_normal(bc, dtype=np.float32)
    C = rng.standard_normal(bc, dtype=np.float32)
    A, D, bias = channel_params(dim, dstate, rng)
    return dict(u=_to_io(u, io_dtype), z=_to_io(z, io_dtype), delta=_to_io(dt, io_dtype),
                B=_to_io(B, io_dtype), C=_to_io(C, io_dtype), A=A, D=D, delta_bias=bias,
                io_dtype=io_dtype)


def scan_inputs_for(cfg: ScanConfig) -> dict:
    return scan_inputs(cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate, cfg.io_dtype, cfg.seed,
                       cfg.ngroups)


def torch_io_dtype(io_dtype: str):
    import torch
    return torch.bfloat16 if io_dtype == "bf16" else torch.float32


def to_torch(inputs: dict, device="cpu") -> dict:
    """numpy inputs -> torch tensors: IO arrays in the IO dtype, parameters fp32."""
    import torch
    io = torch_io_dtype(inputs["io_dtype"])
    out = {}
    for k, v in inputs.items():
        if k == "io_dtype":
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("u", "z", "delta", "B", "C", "x", "dt", "h0", "state"):
            if k in ("h0", "state"):
                t = t.to(torch.float32)
            else:
                t = t.to(io)
        out[k] = t.to(device)
    return out


def scan_inputs_device(cfg: ScanConfig, device="cuda", chunk: int = 1 << 22) -> dict:
    """Device-drawn inputs (torch Philox) for configs too large for host numpy.

    Parameters (A, D, bias) still come from numpy so that they are identical
    on every machine.  IO tensors are drawn in fp32 chunks of the flattened
    (batch, dim, L) index space and rounded to the IO dtype.
    """
    import torch
    io = torch_io_dtype(cfg.io_dtype)
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)

    def draw(shape, scale=1.0):
        t = torch.empty(shape, dtype=io, device=device)
        flat = t.view(-1)
        for s in range(0, flat.numel(), chunk):
            e = min(flat.numel(), s + chunk)
            x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
            if scale != 1.0:
                x.mul_(scale)
            flat[s:e].copy_(x)
        return t

    shp = (cfg.batch, cfg.dim, cfg.seqlen)
    u = draw(shp)
    z = draw(shp)
    dt = draw(shp, 0.1)
    bc = ((cfg.batch, cfg.ngroups, cfg.dstate, cfg.seqlen) if cfg.ngroups
          else (cfg.batch, cfg.dstate, cfg.seqlen))
    B = draw(bc)
    C = draw(bc)
    rng = np.random.default_rng(cfg.seed)
    A, D, bias = channel_params(cfg.dim, cfg.dstate, rng)
    return dict(u=u, z=z, delta=dt, B=B, C=C, A=torch.from_numpy(A).to(device),
                D=torch.from_numpy(D).to(device), delta_bias=torch.from_numpy(bias).to(device))


def decode_inputs_device(cfg: DecodeConfig, steps: int | None = None, device="cuda") -> dict:
    """Per-step decode inputs for `steps` consecutive tokens, drawn on device.

    x, dt, z: (steps, batch, dim); B, C: (steps, batch, dstate); io dtype.
    The fp32 state starts at zero (the pages: the state is zero right after
    initialisation)."""
    import torch
    steps = cfg.steps if steps is None else steps
    io = torch_io_dtype(cfg.io_dtype)
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)

    def draw(shape, scale=1.0):
        out = torch.empty(shape, dtype=io, device=device)
        for s in range(shape[0]):
            x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
            if scale != 1.0:
                x.mul_(scale)
            out[s].copy_(x)
        return out

    x = draw((steps, cfg.batch, cfg.dim))
    z = draw((steps, cfg.batch, cfg.dim))
    dt = draw((steps, cfg.batch, cfg.dim), 0.1)
    B = draw((steps, cfg.batch, cfg.dstate))
    C = draw((steps, cfg.batch, cfg.dstate))
    rng = np.random.default_rng(cfg.seed)
    A, D, bias = channel_params(cfg.dim, cfg.dstate, rng)
    return dict(x=x, z=z, dt=dt, B=B, C=C, A=torch.from_numpy(A).to(device),
                D=torch.from_numpy(D).to(device), dt_bias=torch.from_numpy(bias).to(device))


def decode_inputs_host(batch: int, dim: int, dstate: int = DSTATE, io_dtype: str = "bf16",
                       steps: int = 1, seed: int = 0, random_state: bool = False,
                       ngroups: int = 0) -> dict:
    """Small host-drawn decode inputs (numpy), for parity tests.

    x, dt, z: (steps, batch, dim); B, C: (steps, batch, dstate), or (steps,
    batch, ngroups, dstate) when ngroups >= 1.  With random_state the initial
    state is N(0, 1), else zero."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((steps, batch, dim), dtype=np.float32)
    z = rng.standard_normal((steps, batch, dim), dtype=np.float32)
    dt = np.float32(0.1) * rng.standard_normal((steps, batch, dim), dtype=np.float32)
    bc = (steps, batch, ngroups, dstate) if ngroups else (steps, batch, dstate)
    B = rng.standard_normal(bc, dtype=np.float32)
    C = rng.standard_normal(bc, dtype=np.float32)
    A, D, bias = channel_params(dim, dstate, rng)
    state = (rng.standard_normal((batch, dim, dstate), dtype=np.float32) if random_state
             else np.zeros((batch, dim, dstate), dtype=np.float32))
    return dict(x=_to_io(x, io_dtype), z=_to_io(z, io_dtype), dt=_to_io(dt, io_dtype),
                B=_to_io(B, io_dtype), C=_to_io(C, io_dtype), A=A, D=D, dt_bias=bias,
                state=state, io_dtype=io_dtype)


# ---------------------------------------------------------------------------
# Mamba-2 (SSD layer) inputs.  Same distributions as above, per head: x, z ~
# N(0, 1); dt ~ 0.1 N(0, 1); B, C ~ N(0, 1); per-head step bias = inverse
# softplus of Delta0 log-uniform in [1e-3, 1e-1]; A[h] = -exp(U(0, ln 16)),
# i.e. decays spread over [-16, -1] like the Mamba-1 recipe's -(n+1); D = 1.
# Draw order: x, z, dt, B, C, then per head Delta0 and A.

@dataclasses.dataclass(frozen=True)
class SsdConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    io_dtype: str
    seed: int


# The page's Mamba2(d_model=1024, d_state=64, expand=2, headdim 64) block:
# d_inner 2048 = 32 heads of 64, at the 130m-like layer's batch and length.
SSD_CONFIG = SsdConfig("mamba2-d1024-layer-bf16", 8, 2048, 32, 64, 1, 64, "bf16", 5)
# a long-context Mamba-2 layer: one sequence of 1M tokens, 32 heads of 64
SSD_LONG_CONFIG = SsdConfig("mamba2-long-context-bf16", 1, 1 << 20, 32, 64, 1, 64, "bf16", 6)


def head_params(nheads: int, rng: np.random.Generator):
    lo, hi = math.log(1e-3), math.log(1e-1)
    delta0 = np.exp(rng.uniform(lo, hi, size=nheads))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=nheads)).astype(np.float32)
    D = np.ones(nheads, dtype=np.float32)
    return A, D, delta_bias_from_delta0(delta0)


def ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, ngroups: int, dstate: int,
               io_dtype: str = "f32", seed: int = 0) -> dict:
    """Host (numpy) inputs of one Mamba-2 SSM prefill: x, z (batch, L, H, P);
    dt (batch, L, H); B, C (batch, L, G, N); A, D, dt_bias (H)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32)
    z = rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32)
    dt = np.float32(0.1) * rng.standard_normal((batch, seqlen, nheads), dtype=np.float32)
    B = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32)
    C = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32)
    A, D, bias = head_params(nheads, rng)
    return dict(x=_to_io(x, io_dtype), z=_to_io(z, io_dtype), dt=_to_io(dt, io_dtype),
                B=_to_io(B, io_dtype), C=_to_io(C, io_dtype), A=A, D=D, dt_bias=bias,
                io_dtype=io_dtype)


def ssd_inputs_device(cfg: SsdConfig, device="cuda", chunk: int = 1 << 22) -> dict:
    """Device-drawn (torch Philox) inputs of the Mamba-2 layer config."""
    import torch
    io = torch_io_dtype(cfg.io_dtype)
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)

    def draw(shape, scale=1.0):
        t = torch.empty(shape, dtype=io, device=device)
        flat = t.view(-1)
        for s in range(0, flat.numel(), chunk):
            e = min(flat.numel(), s + chunk)
            v = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
            if scale != 1.0:
                v.mul_(scale)
            flat[s:e].copy_(v)
        return t

    xs = (cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim)
    x = draw(xs)
    z = draw(xs)
    dt = draw((cfg.batch, cfg.seqlen, cfg.nheads), 0.1)
    B = draw((cfg.batch, cfg.seqlen, cfg.ngroups, cfg.dstate))
    C = draw((cfg.batch, cfg.seqlen, cfg.ngroups, cfg.dstate))
    A, D, bias = head_params(cfg.nheads, np.random.default_rng(cfg.seed))
    return dict(x=x, z=z, dt=dt, B=B, C=C, A=torch.from_numpy(A).to(device),
                D=torch.from_numpy(D).to(device), dt_bias=torch.from_numpy(bias).to(device))
