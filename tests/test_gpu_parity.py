"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Bars: row-normwise max relative error <= 1e-4 for fp32 IO
and <= 2e-2 for bf16 IO (see tests/parity.py)."""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from parity import TOL, gpu_scan, oracle_scan, row_rel_err, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines only to be skipped
    pytest.skip("no GPU", allow_module_level=True)

import selective_state_space_74_amd as ssm  # noqa: E402

DEV = "cuda"


def check_scan(inp, io, rows=None, twin=True, h0=None, label=""):
    """out + last_state (+ the SSM-only twin: no D, no gate) against the oracle."""
    out, last = gpu_scan(inp, h0=h0)
    ref, rlast = oracle_scan(inp, h0=h0, rows=rows)
    got, glast = to_np(out), to_np(last)
    if rows is not None:
        got, glast = got[np.ix_(*rows)], glast[np.ix_(*rows)]
    e_out, e_last = row_rel_err(got, ref), row_rel_err(glast, rlast)
    print(f"[{label}] err_out={e_out:.3e} err_last={e_last:.3e}", flush=True)
    assert e_out <= TOL[io], e_out
    assert e_last <= TOL[io], e_last
    if twin:
        out2, _ = gpu_scan(inp, D=False, z=False, h0=h0)
        ref2, _ = oracle_scan(inp, D=False, z=False, h0=h0, rows=rows)
        g2 = to_np(out2)
        if rows is not None:
            g2 = g2[np.ix_(*rows)]
        e2 = row_rel_err(g2, ref2)
        print(f"[{label}] err_ssm_only={e2:.3e}", flush=True)
        assert e2 <= TOL[io], e2


def test_config0_tiny_f32():
    cfg = si.TINY
    check_scan(si.scan_inputs_for(cfg), "f32", label="tiny")


@pytest.mark.parametrize("batch,dim,L,io", [
    (1, 37, 37, "f32"), (3, 20, 1, "f32"), (2, 5, 129, "f32"), (1, 16, 1000, "f32"),
    (2, 16, 1000, "bf16"), (1, 48, 17, "bf16"), (2, 33, 300, "bf16"),
])
def test_ragged_shapes(batch, dim, L, io):
    inp = si.scan_inputs(batch, dim, L, io_dtype=io, seed=100 + L + dim)
    check_scan(inp, io, label=f"ragged b{batch} d{dim} L{L} {io}")


@pytest.mark.parametrize("batch,dim,L,io", [(1, 37, 50, "f32"), (2, 13, 3 * 32768 + 5, "bf16")])
def test_ragged_channels_with_initial_state(batch, dim, L, io):
    """Channel counts that leave a partial last channel group, with h0 and
    last_state (the second case is also cut into segments)."""
    inp = si.scan_inputs(batch, dim, L, io_dtype=io, seed=dim + L)
    h0 = np.random.default_rng(dim).standard_normal((batch, dim, 16)).astype(np.float32)
    check_scan(inp, io, h0=h0, label=f"ragged h0 b{batch} d{dim} L{L} {io}")


def test_initial_state_and_split_sequence():
    inp = si.scan_inputs(2, 32, 200, io_dtype="f32", seed=7)
    rng = np.random.default_rng(7)
    h0 = rng.standard_normal((2, 32, 16)).astype(np.float32)
    check_scan(inp, "f32", h0=h0, label="h0")
    ref, rlast = oracle_scan(inp, h0=h0)
    for cut in (1, 37, 100, 199):
        a = {k: (np.ascontiguousarray(v[..., :cut]) if k in ("u", "delta", "z", "B", "C") else v)
             for k, v in inp.items()}
        b = {k: (np.ascontiguousarray(v[..., cut:]) if k in ("u", "delta", "z", "B", "C") else v)
             for k, v in inp.items()}
        o1, l1 = gpu_scan(a, h0=h0)
        o2, l2 = gpu_scan(b, h0=to_np(l1).astype(np.float32))
        got = np.concatenate([to_np(o1), to_np(o2)], axis=2)
        e = row_rel_err(got, ref)
        el = row_rel_err(to_np(l2), rlast)
        print(f"[split {cut}] err_out={e:.3e} err_last={el:.3e}", flush=True)
        assert e <= TOL["f32"] and el <= TOL["f32"]


def test_config1_full_f32():
    cfg = si.LAYER_130M
    check_scan(si.scan_inputs_for(cfg), "f32", label="130m-like layer")


def test_config2_bf16_full():
    """The 2.8b-like layer (batch 4, d_inner 5120, L 4096, bf16 IO) on every
    channel: out, last_state and the SSM-only twin."""
    cfg = si.LAYER_2P8B
    check_scan(si.scan_inputs_for(cfg), "bf16", label="2.8b-like layer, all channels")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("blocks", [768, 769])
def test_readout_forms_either_side_of_the_grid_switch(blocks, io):
    """Up to 768 workgroups (3 wavefronts per SIMD) the one-slot scan defers
    each block's readout to the next block; above, it reads out at the end of
    the block.  One batch row of `blocks` 16-channel blocks, ragged length."""
    inp = si.scan_inputs(1, 16 * blocks, 45, io_dtype=io, seed=blocks)
    check_scan(inp, io, label=f"{blocks} workgroups {io}")


def test_config3_long_context_16_channels():
    cfg = si.LONG_CONTEXT
    t = si.scan_inputs_device(cfg, DEV)
    out, last = ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],
                                       z=t["z"], delta_bias=t["delta_bias"],
                                       return_last_state=True)
    torch.cuda.synchronize()
    ch = np.sort(np.random.default_rng(3).choice(cfg.dim, 16, replace=False))
    idx = torch.from_numpy(ch).to(DEV)
    sel = lambda x: to_np(x.index_select(1, idx))
    ref, rlast = oracle.selective_scan(sel(t["u"]), sel(t["delta"]), to_np(t["A"])[ch],
                                       to_np(t["B"]), to_np(t["C"]), D=to_np(t["D"])[ch],
                                       z=sel(t["z"]), delta_bias=to_np(t["delta_bias"])[ch],
                                       return_last_state=True)
    e = row_rel_err(sel(out), ref)
    el = row_rel_err(to_np(last)[:, ch], rlast)
    print(f"[1M tokens] err_out={e:.3e} err_last={el:.3e}", flush=True)
    assert e <= TOL["bf16"] and el <= TOL["bf16"]
    del t, out, last
    torch.cuda.empty_cache()


def test_segmented_wide_fp32_gathers_windows_by_chunk():
    """fp32, d_inner 1100, L 2^20 + 37: a B/C group's rows span 1100 rows of
    4 MiB, more than a 32-bit buffer window can reach, so the segmented
    scan's second pass gathers each window's channels from chunks of the
    group (1023 channels, then 77) whose rows fit.  Checked against the
    oracle on 24 channels taken from both chunks, with h0."""
    cfg = si.ScanConfig("wide-fp32-long", 1, 1100, (1 << 20) + 37, 16, "f32", 9)
    a = ssm.ScanArgs()
    a.batch, a.dim, a.seqlen, a.dstate = cfg.batch, cfg.dim, cfg.seqlen, cfg.dstate
    assert ssm.scan_workspace_size(a) > 0          # segmented
    t = si.scan_inputs_device(cfg, DEV)
    rng = np.random.default_rng(9)
    h0 = torch.from_numpy(rng.standard_normal((1, cfg.dim, 16)).astype(np.float32)).to(DEV)
    out, last = ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],
                                       z=t["z"], delta_bias=t["delta_bias"], h0=h0,
                                       return_last_state=True)
    torch.cuda.synchronize()
    ch = np.sort(np.concatenate([rng.choice(1023, 12, replace=False),
                                 1023 + rng.choice(77, 12, replace=False)]))
    idx = torch.from_numpy(ch).to(DEV)
    sel = lambda x: to_np(x.index_select(1, idx))
    ref, rlast = oracle.selective_scan(sel(t["u"]), sel(t["delta"]), to_np(t["A"])[ch],
                                       to_np(t["B"]), to_np(t["C"]), D=to_np(t["D"])[ch],
                                       z=sel(t["z"]), delta_bias=to_np(t["delta_bias"])[ch],
                                       h0=sel(h0), return_last_state=True)
    e = row_rel_err(sel(out), ref)
    el = row_rel_err(to_np(last)[:, ch], rlast)
    print(f"[wide fp32 1M tokens, chunked windows] err_out={e:.3e} err_last={el:.3e}", flush=True)
    assert e <= TOL["f32"] and el <= TOL["f32"]
    del t, out, last
    torch.cuda.empty_cache()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_segmented_long_sequence(io):
    """Few channels and a long sequence: the library cuts the sequence into
    segments (aggregate pass + scan pass).  Checked against the oracle on all
    channels, and against the same call run as one segment."""
    L = 3 * 32768 + 100
    inp = si.scan_inputs(1, 16, L, io_dtype=io, seed=77)
    t = si.to_torch(inp, DEV)
    rng = np.random.default_rng(77)
    h0 = rng.standard_normal((1, 16, 16)).astype(np.float32)
    h0t = torch.from_numpy(h0).to(DEV)
    args = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], h0=h0t, return_last_state=True)
    a = ssm.ScanArgs()
    a.batch, a.dim, a.seqlen, a.dstate = 1, 16, L, 16
    assert ssm.scan_workspace_size(a) > 0          # this shape is segmented
    out, last = ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **args)
    out1, last1 = ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                         workspace=False, **args)
    torch.cuda.synchronize()
    ref, rlast = oracle_scan(inp, h0=h0)
    e, el = row_rel_err(to_np(out), ref), row_rel_err(to_np(last), rlast)
    e1 = row_rel_err(to_np(out1), ref)
    print(f"[segmented {io}] err_out={e:.3e} err_last={el:.3e} single-segment err_out={e1:.3e}",
          flush=True)
    assert e <= TOL[io] and el <= TOL[io] and e1 <= TOL[io]
    assert row_rel_err(to_np(out), to_np(out1)) <= TOL[io]


def test_deterministic_bitwise():
    inp = si.scan_inputs(4, 256, 777, io_dtype="f32", seed=11)
    o1, l1 = gpu_scan(inp)
    o2, l2 = gpu_scan(inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_graph_replay_matches_eager(io):
    """The scan captured in a HIP graph (as bench.py times it): three launches
    over two input sets, replayed several times with eager scans and
    synchronisations between the replays; every replay equals the eager
    result bit for bit (outputs cleared before each replay)."""
    sets = [si.to_torch(si.scan_inputs(2, 96, 300, io_dtype=io, seed=s), DEV) for s in (5, 6)]
    outs = [torch.empty_like(t["u"]) for t in sets]
    lasts = [torch.empty((2, 96, 16), device=DEV) for _ in sets]

    def step(i):
        t = sets[i % 2]
        ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               delta_bias=t["delta_bias"], out=outs[i % 2], last_state=lasts[i % 2])

    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in zip(outs, lasts)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(3):
            step(i)
    for r in range(4):
        for o, l in zip(outs, lasts):
            o.zero_()
            l.zero_()
        g.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(zip(outs, lasts), ref):
            assert torch.equal(o, ro) and torch.equal(l, rl), r
        eager = gpu_scan(si.scan_inputs(1, 20, 50, io_dtype=io, seed=r))   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(eager[0].float()).all()


def test_strided_views():
    batch, dim, L = 2, 40, 96
    inp = si.scan_inputs(batch, dim, L, io_dtype="bf16", seed=5)
    t = si.to_torch(inp, DEV)
    # every IO tensor is a view into a wider buffer (dim and batch strides != contiguous)
    def widen(x, extra_dim=3, extra_t=5):
        big = torch.zeros((x.shape[0], x.shape[1] + extra_dim, x.shape[2] + extra_t),
                          dtype=x.dtype, device=DEV)
        big[:, : x.shape[1], : x.shape[2]] = x
        return big[:, : x.shape[1], : x.shape[2]]
    u, dl, z, B, C = (widen(t[k]) for k in ("u", "delta", "z", "B", "C"))
    outbuf = torch.zeros((batch, dim + 2, L + 7), dtype=torch.bfloat16, device=DEV)
    out = outbuf[:, :dim, :L]
    ssm.selective_scan_fwd(u, dl, t["A"], B, C, D=t["D"], z=z, delta_bias=t["delta_bias"],
                           out=out)
    torch.cuda.synchronize()
    ref = oracle_scan(inp, last=False)
    e = row_rel_err(to_np(out), ref)
    print(f"[strided] err_out={e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    assert torch.count_nonzero(outbuf[:, dim:, :]) == 0 and torch.count_nonzero(outbuf[:, :, L:]) == 0


def test_seqlen_zero_copies_initial_state():
    batch, dim = 2, 24
    h0 = torch.randn((batch, dim, 16), device=DEV)
    e = torch.empty((batch, dim, 0), device=DEV)
    A = -torch.ones((dim, 16), device=DEV)
    Bz = torch.empty((batch, 16, 0), device=DEV)
    out, last = ssm.selective_scan_fwd(e, e, A, Bz, Bz, h0=h0, return_last_state=True)
    torch.cuda.synchronize()
    assert out.shape == (batch, dim, 0) and torch.equal(last, h0)
    _, last0 = ssm.selective_scan_fwd(e, e, A, Bz, Bz, return_last_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(last0) == 0


def test_nan_propagates_within_its_row():
    inp = si.scan_inputs(2, 16, 64, io_dtype="f32", seed=13)
    inp["u"] = inp["u"].copy()
    inp["u"][0, 1, 5] = np.nan
    out, _ = gpu_scan(inp)
    o = to_np(out)
    assert np.all(np.isnan(o[0, 1, 5:])) and not np.any(np.isnan(o[0, 1, :5]))
    mask = np.ones(o.shape, bool)
    mask[0, 1, 5:] = False
    assert not np.any(np.isnan(o[mask]))


def test_binding_raises_on_unsupported_state_size():
    u = torch.zeros((1, 16, 8), device=DEV)
    A = -torch.ones((16, 65), device=DEV)
    Bm = torch.zeros((1, 65, 8), device=DEV)
    with pytest.raises(ssm.SSMError) as ei:
        ssm.selective_scan_fwd(u, u, A, Bm, Bm)
    assert ei.value.status == 7


# ----------------------------------------------------------------------------- decode

def gpu_decode_steps(d, steps, state):
    outs = []
    for s in range(steps):
        outs.append(ssm.selective_state_update(state, d["x"][s], d["dt"][s], d["A"], d["B"][s],
                                               d["C"][s], D=d["D"], z=d["z"][s],
                                               dt_bias=d["dt_bias"]))
    torch.cuda.synchronize()
    return torch.stack(outs)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_single_step_random_state(io):
    h = si.decode_inputs_host(8, 200, io_dtype=io, steps=1, seed=21, random_state=True)
    d = si.to_torch(h, DEV)
    state = d["state"].clone()
    out = gpu_decode_steps(d, 1, state)[0]
    ref, rstate = oracle.state_update(h["state"], h["x"][0], h["dt"][0], h["A"], h["B"][0],
                                      h["C"][0], D=h["D"], z=h["z"][0], dt_bias=h["dt_bias"])
    e = row_rel_err(to_np(out), ref, axis=1)          # rows: batch entries over channels
    es = row_rel_err(to_np(state), rstate)            # rows: state vectors
    print(f"[decode 1 step {io}] err_out={e:.3e} err_state={es:.3e}", flush=True)
    assert e <= TOL[io] and es <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_batch_rows_per_thread_ragged(io):
    """A grid large enough that each thread takes two batch rows (odd batch:
    the last pair has one row; dim not a multiple of the 64-channel block),
    two steps from a random state."""
    h = si.decode_inputs_host(51, 5100, io_dtype=io, steps=2, seed=23, random_state=True)
    d = si.to_torch(h, DEV)
    state = d["state"].clone()
    outs = gpu_decode_steps(d, 2, state)
    rstate = h["state"]
    for s in range(2):
        ref, rstate = oracle.state_update(rstate, h["x"][s], h["dt"][s], h["A"], h["B"][s],
                                          h["C"][s], D=h["D"], z=h["z"][s], dt_bias=h["dt_bias"])
        e = row_rel_err(to_np(outs[s]), ref, axis=1)
        print(f"[decode rows {io} step {s}] err_out={e:.3e}", flush=True)
        assert e <= TOL[io]
    es = row_rel_err(to_np(state), rstate)
    print(f"[decode rows {io}] err_state={es:.3e}", flush=True)
    assert es <= TOL[io]


def test_decode_equals_scan_on_gpu():
    """L decode steps reproduce the scan's outputs and final state (both HIP)."""
    inp = si.scan_inputs(2, 48, 64, io_dtype="f32", seed=31)
    out, last = gpu_scan(inp)
    t = si.to_torch(inp, DEV)
    state = torch.zeros((2, 48, 16), device=DEV)
    d = dict(x=t["u"].permute(2, 0, 1).contiguous(), dt=t["delta"].permute(2, 0, 1).contiguous(),
             z=t["z"].permute(2, 0, 1).contiguous(), B=t["B"].permute(2, 0, 1).contiguous(),
             C=t["C"].permute(2, 0, 1).contiguous(), A=t["A"], D=t["D"], dt_bias=t["delta_bias"])
    steps = gpu_decode_steps(d, 64, state)           # (L, batch, dim)
    e = row_rel_err(to_np(steps.permute(1, 2, 0)), to_np(out))
    es = row_rel_err(to_np(state), to_np(last))
    print(f"[decode==scan] err_out={e:.3e} err_state={es:.3e}", flush=True)
    assert e <= TOL["f32"] and es <= TOL["f32"]


def test_decode_b256_d5120_1000_steps_sampled():
    cfg = si.DECODE_CONFIG
    d = si.decode_inputs_device(cfg, device=DEV)
    state = torch.zeros((cfg.batch, cfg.dim, cfg.dstate), device=DEV)
    outs = gpu_decode_steps(d, cfg.steps, state)      # (steps, batch, dim)
    rng = np.random.default_rng(4)
    bi = np.sort(rng.choice(cfg.batch, 4, replace=False))
    di = np.sort(rng.choice(cfg.dim, 64, replace=False))
    tb, td = torch.from_numpy(bi).to(DEV), torch.from_numpy(di).to(DEV)
    x = to_np(d["x"].index_select(1, tb).index_select(2, td))
    dt = to_np(d["dt"].index_select(1, tb).index_select(2, td))
    z = to_np(d["z"].index_select(1, tb).index_select(2, td))
    B = to_np(d["B"].index_select(1, tb))
    C = to_np(d["C"].index_select(1, tb))
    A, D, bias = to_np(d["A"])[di], to_np(d["D"])[di], to_np(d["dt_bias"])[di]
    rstate = np.zeros((4, 64, cfg.dstate))
    ref = np.empty((cfg.steps, 4, 64))
    for s in range(cfg.steps):
        ref[s], rstate = oracle.state_update(rstate, x[s], dt[s], A, B[s], C[s], D=D, z=z[s],
                                             dt_bias=bias)
    got = to_np(outs.index_select(1, tb).index_select(2, td))
    e = row_rel_err(np.moveaxis(got, 0, -1), np.moveaxis(ref, 0, -1))
    es = row_rel_err(to_np(state)[np.ix_(bi, di)], rstate)
    print(f"[decode b256 d5120, 1000 steps] err_out={e:.3e} err_state={es:.3e}", flush=True)
    assert e <= TOL["bf16"] and es <= TOL["bf16"]
    del d, outs
    torch.cuda.empty_cache()


def test_decode_b256_d5120_all_channels_100_steps():
    """The decode workload on every (batch, channel) for its first 100 steps:
    each step's output and the state after the last one against the oracle
    stepped on the same inputs."""
    cfg = si.DECODE_CONFIG
    steps = 100
    d = si.decode_inputs_device(cfg, device=DEV)        # the workload's 1000 steps of inputs
    state = torch.zeros((cfg.batch, cfg.dim, cfg.dstate), device=DEV)
    outs = gpu_decode_steps(d, steps, state)          # (steps, batch, dim)
    A, D, bias = to_np(d["A"]), to_np(d["D"]), to_np(d["dt_bias"])
    rstate = np.zeros((cfg.batch, cfg.dim, cfg.dstate))
    worst = 0.0
    ref = np.empty((steps, cfg.batch, cfg.dim))
    for s in range(steps):
        ref[s], rstate = oracle.state_update(rstate, to_np(d["x"][s]), to_np(d["dt"][s]), A,
                                             to_np(d["B"][s]), to_np(d["C"][s]), D=D,
                                             z=to_np(d["z"][s]), dt_bias=bias)
    got = to_np(outs)
    e = row_rel_err(np.moveaxis(got, 0, -1), np.moveaxis(ref, 0, -1))   # rows: (b, d) over steps
    es = row_rel_err(to_np(state), rstate)
    for s in (0, steps - 1):
        worst = max(worst, row_rel_err(got[s], ref[s]))                  # rows: batch over channels
    print(f"[decode b256 d5120, all channels, {steps} steps] err_out={e:.3e} "
          f"err_step_rows={worst:.3e} err_state={es:.3e}", flush=True)
    assert e <= TOL["bf16"] and es <= TOL["bf16"] and worst <= TOL["bf16"]
    del d, outs
    torch.cuda.empty_cache()


def test_decode_strided_state_and_batch_views():
    h = si.decode_inputs_host(6, 64, io_dtype="bf16", steps=1, seed=41, random_state=True)
    d = si.to_torch(h, DEV)
    big = torch.zeros((6, 64 + 3, 16), device=DEV)        # state rows not 16-byte aligned per batch
    big[:, :64] = d["state"]
    state = big[:, :64]
    xbig = torch.zeros((6, 80), dtype=torch.bfloat16, device=DEV)
    xbig[:, :64] = d["x"][0]
    out = ssm.selective_state_update(state, xbig[:, :64], d["dt"][0], d["A"], d["B"][0], d["C"][0],
                                     D=d["D"], z=d["z"][0], dt_bias=d["dt_bias"])
    torch.cuda.synchronize()
    ref, rstate = oracle.state_update(h["state"], h["x"][0], h["dt"][0], h["A"], h["B"][0],
                                      h["C"][0], D=h["D"], z=h["z"][0], dt_bias=h["dt_bias"])
    assert row_rel_err(to_np(out), ref, axis=1) <= TOL["bf16"]
    assert row_rel_err(to_np(state), rstate) <= TOL["bf16"]
    assert torch.count_nonzero(big[:, 64:]) == 0
