"""GPU parity of the Mamba-2 SSM (SSD layer) prefill, through the C ABI,
against the fp64 oracle (oracle.ssd_scan) on the same seeded inputs.

Bars (row-normwise max relative error; a row is one (batch, head, channel)
sequence over t, or one state vector over n): 1e-4 for fp32 IO and 2e-2 for
bf16 IO.  With bf16 IO the kernel rounds the masked chunk scores and the
decay-weighted x to bf16 where they enter a matrix product (fp32
accumulation; the chunk-entry state enters as a bf16 value plus its bf16
remainder), so its error is of the order of bf16 rounding; the printed
errors show the margin."""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from parity import TOL, row_rel_err, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines only to be skipped
    pytest.skip("no GPU", allow_module_level=True)

import selective_state_space_74_amd as ssm  # noqa: E402

DEV = "cuda"


def to_dev(inp, io):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        if v is None or k == "io_dtype":
            continue
        t = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
        out[k] = t.to(dt) if k in ("x", "z", "dt", "B", "C") else t.float()
    return out


def run_gpu(inp, io, gate=True, skip=True, bias=True, softplus=True, h0=None):
    t = to_dev(inp, io)
    h0t = None if h0 is None else torch.from_numpy(h0).to(DEV).float()
    out, last = ssm.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"] if skip else None,
                                 z=t["z"] if gate else None, dt_bias=t["dt_bias"] if bias else None,
                                 dt_softplus=softplus, h0=h0t, return_last_state=True)
    torch.cuda.synchronize()
    return to_np(out), to_np(last)


def run_oracle(inp, gate=True, skip=True, bias=True, softplus=True, h0=None):
    return oracle.ssd_scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                           D=inp["D"] if skip else None, z=inp["z"] if gate else None,
                           dt_bias=inp["dt_bias"] if bias else None, dt_softplus=softplus,
                           h0=h0, return_last_state=True)


def errors(got, ref, glast, rlast):
    # rows: (b, h, p) over t; states: (b, h, p) over n
    e = row_rel_err(np.moveaxis(got, 1, -1), np.moveaxis(ref, 1, -1))
    el = row_rel_err(glast, rlast)
    return e, el


def check(inp, io, label, **kw):
    got, glast = run_gpu(inp, io, **kw)
    ref, rlast = run_oracle(inp, **kw)
    e, el = errors(got, ref, glast, rlast)
    print(f"[ssd {label}] err_out={e:.3e} err_last={el:.3e}", flush=True)
    assert e <= TOL[io] and el <= TOL[io], (e, el)


@pytest.mark.parametrize("batch,L,H,P,G,N,io", [
    (2, 64, 4, 16, 2, 16, "f32"),     # one full chunk
    (2, 200, 4, 64, 1, 64, "f32"),    # ragged last chunk
    (1, 130, 6, 20, 3, 40, "f32"),    # head and state sizes off the 16 grid
    (3, 1, 2, 16, 1, 64, "f32"),      # one token
    (2, 129, 4, 64, 1, 64, "bf16"),
    (2, 300, 8, 64, 2, 128, "bf16"),
    (1, 77, 6, 24, 6, 96, "bf16"),    # a group per head
    (2, 64, 2, 64, 1, 16, "bf16"),
])
def test_ssd_matches_oracle(batch, L, H, P, G, N, io):
    inp = si.ssd_inputs(batch, L, H, P, G, N, io_dtype=io, seed=batch * 1000 + L + N)
    h0 = np.random.default_rng(L).standard_normal((batch, H, P, N)).astype(np.float32)
    check(inp, io, f"b{batch} L{L} H{H} P{P} G{G} N{N} {io}", h0=h0)
    check(inp, io, f"b{batch} L{L} H{H} P{P} G{G} N{N} {io} no h0")


@pytest.mark.parametrize("batch,L,H,P,G,N,io", [
    (2, 100, 256, 48, 4, 64, "bf16"),   # four blocks, the last one masked
    (2, 70, 256, 64, 2, 128, "bf16"),   # two blocks, 128 states
    (2, 90, 256, 40, 1, 64, "f32"),     # two blocks, the second ragged
    (2, 66, 256, 32, 4, 40, "f32"),     # two blocks, element-wise staging
])
def test_ssd_channel_blocks_per_workgroup(batch, L, H, P, G, N, io):
    """Enough (batch, head) pairs (512) that a workgroup takes several blocks
    of 16 head channels (sharing the chunk's scores and B/C staging), with
    head sizes that leave channel blocks partly or wholly past headdim."""
    inp = si.ssd_inputs(batch, L, H, P, G, N, io_dtype=io, seed=L + P + N)
    h0 = np.random.default_rng(P).standard_normal((batch, H, P, N)).astype(np.float32)
    check(inp, io, f"blocks b{batch} L{L} H{H} P{P} G{G} N{N} {io}", h0=h0)


@pytest.mark.parametrize("gate,skip,bias,softplus", [
    (False, False, False, True), (True, True, True, False), (False, True, False, True)])
def test_ssd_optional_inputs(gate, skip, bias, softplus):
    inp = si.ssd_inputs(2, 150, 4, 32, 2, 64, io_dtype="f32", seed=3)
    if not softplus:   # a positive step taken as is
        inp["dt"] = np.abs(inp["dt"]) + np.float32(0.01)
        inp["dt_bias"] = np.abs(inp["dt_bias"]) * np.float32(0.01)
    check(inp, "f32", f"gate{gate} skip{skip} bias{bias} sp{softplus}", gate=gate, skip=skip,
          bias=bias, softplus=softplus)


def test_ssd_split_sequence_carries_the_state():
    inp = si.ssd_inputs(2, 256, 4, 64, 1, 64, io_dtype="f32", seed=5)
    ref, rlast = run_oracle(inp)
    cut = 100
    a = {k: (v[:, :cut] if k in ("x", "z", "dt", "B", "C") else v) for k, v in inp.items()}
    b = {k: (v[:, cut:] if k in ("x", "z", "dt", "B", "C") else v) for k, v in inp.items()}
    o1, l1 = run_gpu(a, "f32")
    o2, l2 = run_gpu(b, "f32", h0=l1.astype(np.float32))
    e, el = errors(np.concatenate([o1, o2], axis=1), ref, l2, rlast)
    print(f"[ssd split] err_out={e:.2e} err_last={el:.2e}", flush=True)
    assert e <= 1e-4 and el <= 1e-4


def _ssd_args(batch, L, H, P, G, N):
    a = ssm.SsdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.ngroups, a.dstate = batch, L, H, P, G, N
    return a


@pytest.mark.parametrize("H,P,N,io", [(2, 64, 64, "f32"), (3, 40, 128, "bf16"), (2, 64, 64, "bf16")])
def test_ssd_segmented_long_sequence(H, P, N, io):
    """Few (batch, head) slices and a long sequence: with the workspace the
    sequence is cut into segments (pass 1 from zero states, pass 2 rescanning
    each segment's head from its folded incoming state).  Checked against the
    oracle, with and without h0, next to the one-segment run (no workspace)."""
    batch, L, G = 1, 3 * 32768 + 100, 1
    assert ssm.ssd_workspace_size(_ssd_args(batch, L, H, P, G, N)) > 0
    inp = si.ssd_inputs(batch, L, H, P, G, N, io_dtype=io, seed=H * 100 + N)
    h0 = np.random.default_rng(N).standard_normal((batch, H, P, N)).astype(np.float32)
    ref, rlast = run_oracle(inp, h0=h0)
    t = to_dev(inp, io)
    kw = dict(D=t["D"], z=t["z"], dt_bias=t["dt_bias"], h0=torch.from_numpy(h0).to(DEV),
              return_last_state=True)
    for ws in (None, False):
        out, last = ssm.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], workspace=ws, **kw)
        torch.cuda.synchronize()
        e, el = errors(to_np(out), ref, to_np(last), rlast)
        print(f"[ssd segmented={ws is None} H{H} P{P} N{N} {io}] err_out={e:.3e} err_last={el:.3e}",
              flush=True)
        assert e <= TOL[io] and el <= TOL[io], (e, el)
    check(inp, io, f"segmented H{H} P{P} N{N} {io} no h0")


def test_ssd_segmented_in_place_carry_and_no_decay():
    """Segmented: the final state written over h0 (pass 1 reads h0 before
    pass 2 writes it), and a head with A = 0 whose incoming state never
    decays (pass 2 then rescans its whole segments)."""
    batch, L, H, P, G, N = 1, 2 * 32768 + 640, 2, 32, 1, 64
    assert ssm.ssd_workspace_size(_ssd_args(batch, L, H, P, G, N)) > 0
    inp = si.ssd_inputs(batch, L, H, P, G, N, io_dtype="f32", seed=21)
    inp["A"] = inp["A"].copy()
    inp["A"][1] = 0.0
    h0 = np.random.default_rng(21).standard_normal((batch, H, P, N)).astype(np.float32)
    ref, rlast = run_oracle(inp, h0=h0)
    t = to_dev(inp, "f32")
    state = torch.from_numpy(h0).to(DEV)
    out = ssm.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           dt_bias=t["dt_bias"], h0=state, last_state=state)
    torch.cuda.synchronize()
    e, el = errors(to_np(out), ref, to_np(state), rlast)
    print(f"[ssd segmented in-place, A=0 head] err_out={e:.3e} err_last={el:.3e}", flush=True)
    assert e <= 1e-4 and el <= 1e-4


def test_ssd_zero_length_copies_initial_state():
    H, P, N = 4, 16, 32
    x = torch.zeros((2, 0, H, P), device=DEV)
    dt = torch.zeros((2, 0, H), device=DEV)
    Bm = torch.zeros((2, 0, 1, N), device=DEV)
    A = -torch.ones(H, device=DEV)
    h0 = torch.randn((2, H, P, N), device=DEV)
    out, last = ssm.ssd_scan_fwd(x, dt, A, Bm, Bm, h0=h0, return_last_state=True)
    torch.cuda.synchronize()
    assert out.shape == x.shape and torch.equal(last, h0)


def test_ssd_strided_views_and_in_place_state():
    """x, z, out as head-dim slices of wider tensors; B/C as views; the final
    state written over h0."""
    batch, L, H, P, G, N = 2, 140, 4, 32, 2, 48
    inp = si.ssd_inputs(batch, L, H, P, G, N, io_dtype="f32", seed=8)
    h0 = np.random.default_rng(8).standard_normal((batch, H, P, N)).astype(np.float32)
    ref, rlast = run_oracle(inp, h0=h0)
    t = to_dev(inp, "f32")
    xw = torch.zeros((batch, L, H, P + 8), device=DEV)
    xw[..., 3:3 + P] = t["x"]
    zw = torch.zeros((batch, L, H, P + 8), device=DEV)
    zw[..., 1:1 + P] = t["z"]
    Bw = torch.zeros((batch, L, G + 1, N), device=DEV)
    Bw[:, :, 1:] = t["B"]
    ow = torch.full((batch, L, H, P + 4), 5.0, device=DEV)
    state = torch.from_numpy(h0).to(DEV)
    out, last = ssm.ssd_scan_fwd(xw[..., 3:3 + P], t["dt"], t["A"], Bw[:, :, 1:], t["C"], D=t["D"],
                                 z=zw[..., 1:1 + P], dt_bias=t["dt_bias"], h0=state,
                                 last_state=state, out=ow[..., 2:2 + P], return_last_state=True)
    torch.cuda.synchronize()
    e, el = errors(to_np(out), ref, to_np(state), rlast)
    print(f"[ssd views] err_out={e:.2e} err_last={el:.2e}", flush=True)
    assert e <= 1e-4 and el <= 1e-4
    assert torch.all(ow[..., :2] == 5.0) and torch.all(ow[..., 2 + P:] == 5.0)


def test_ssd_layer_bf16_sampled_heads():
    """The benchmarked Mamba-2 layer shape (batch 8, L 2048, 32 heads of 64,
    d_state 64, one group, bf16): every output computed on the GPU, 16
    distinct (batch, head) pairs checked against the oracle."""
    cfg = si.SSD_CONFIG
    t = si.ssd_inputs_device(cfg, DEV)
    out, last = ssm.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                 dt_bias=t["dt_bias"], return_last_state=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(0)
    pairs = rng.choice(cfg.batch * cfg.nheads, 16, replace=False)
    for b, h in zip(pairs // cfg.nheads, pairs % cfg.nheads):
        sel = lambda v: to_np(v[b:b + 1])
        inp = dict(x=sel(t["x"])[:, :, h:h + 1], z=sel(t["z"])[:, :, h:h + 1],
                   dt=sel(t["dt"])[:, :, h:h + 1], B=sel(t["B"]), C=sel(t["C"]),
                   A=to_np(t["A"])[h:h + 1], D=to_np(t["D"])[h:h + 1],
                   dt_bias=to_np(t["dt_bias"])[h:h + 1])
        ref, rlast = run_oracle(inp)
        got = to_np(out[b:b + 1, :, h:h + 1])
        e, el = errors(got, ref, to_np(last[b:b + 1, h:h + 1]), rlast)
        print(f"[ssd layer b{b} h{h}] err_out={e:.2e} err_last={el:.2e}", flush=True)
        assert e <= TOL["bf16"] and el <= TOL["bf16"]


def test_ssd_deterministic():
    inp = si.ssd_inputs(2, 200, 4, 64, 1, 64, io_dtype="bf16", seed=13)
    a, la = run_gpu(inp, "bf16")
    b, lb = run_gpu(inp, "bf16")
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_ssd_rejects_unsupported_state_size():
    x = torch.zeros((1, 8, 2, 16), device=DEV)
    dt = torch.zeros((1, 8, 2), device=DEV)
    Bm = torch.zeros((1, 8, 1, 72), device=DEV)      # fp32 supports up to 64 states
    with pytest.raises(ssm.SSMError) as ei:
        ssm.ssd_scan_fwd(x, dt, -torch.ones(2, device=DEV), Bm, Bm)
    assert ei.value.status == 7


def test_mamba2_decode_is_the_mamba1_step_with_head_broadcast():
    """A Mamba-2 decode step through ssm_selective_state_update: channel
    d = h * P + p, A[d, n] = A[h] for every n, the head's step and bias
    repeated over its P channels, D repeated, B/C in G groups (channel d reads
    group d / (H P / G) = h / (H / G)).  Checked against the SSD oracle one
    token at a time, starting from a random state."""
    batch, H, P, G, N, steps = 2, 4, 16, 2, 64, 5
    inp = si.ssd_inputs(batch, steps, H, P, G, N, io_dtype="f32", seed=44)
    state0 = np.random.default_rng(44).standard_normal((batch, H, P, N)).astype(np.float32)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in inp.items()
           if k != "io_dtype"}
    A1 = dev["A"].repeat_interleave(P)[:, None].expand(H * P, N).contiguous()
    D1 = dev["D"].repeat_interleave(P)
    bias1 = dev["dt_bias"].repeat_interleave(P)
    state = torch.from_numpy(state0.reshape(batch, H * P, N)).to(DEV)
    ref_state = state0.astype(np.float64)
    for t in range(steps):
        x = dev["x"][:, t].reshape(batch, H * P).contiguous()
        z = dev["z"][:, t].reshape(batch, H * P).contiguous()
        dt = dev["dt"][:, t].repeat_interleave(P, dim=1).contiguous()
        out = ssm.selective_state_update(state, x, dt, A1, dev["B"][:, t].contiguous(),
                                         dev["C"][:, t].contiguous(), D=D1, z=z, dt_bias=bias1)
        torch.cuda.synchronize()
        one = {k: (v[:, t:t + 1] if k in ("x", "z", "dt", "B", "C") else v) for k, v in inp.items()}
        ref, ref_state = oracle.ssd_scan(one["x"], one["dt"], one["A"], one["B"], one["C"], D=one["D"],
                                         z=one["z"], dt_bias=one["dt_bias"], h0=ref_state,
                                         return_last_state=True)
        e = row_rel_err(to_np(out).reshape(batch, H, P), ref[:, 0])
        es = row_rel_err(to_np(state).reshape(batch, H, P, N), ref_state)
        print(f"[mamba2 decode step {t}] err_out={e:.2e} err_state={es:.2e}", flush=True)
        assert e <= 1e-4 and es <= 1e-4
