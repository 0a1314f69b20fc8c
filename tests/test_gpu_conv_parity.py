"""GPU parity of the fused conv branch (causal depthwise conv + SiLU in front
of the scan, and the conv-state update fused into decode) against the fp64
oracle's conv followed by its scan, on the same seeded inputs.  Bars as for
the scan: row-normwise 1e-4 (fp32 IO), 2e-2 (bf16 IO); the returned conv
states are copies of inputs and must match exactly."""
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


def conv_params(dim, K, seed, batch):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((dim, K)) / np.sqrt(K)).astype(np.float32)
    b = (0.1 * rng.standard_normal(dim)).astype(np.float32)
    st = rng.standard_normal((batch, dim, K)).astype(np.float32)
    return w, b, st


def as_io(a, io):
    return si.bf16_round(a) if io == "bf16" else a.astype(np.float32)


def gpu_conv_scan(inp, w, b, st, silu=True, h0=None, want_conv_out=True, workspace=None):
    t = si.to_torch(inp, DEV)
    batch, dim, L = t["u"].shape
    K = w.shape[1]
    wt, bt = torch.from_numpy(w).to(DEV), torch.from_numpy(b).to(DEV)
    st_in = None if st is None else torch.from_numpy(st).to(DEV)
    st_out = torch.empty((batch, dim, K), device=DEV)
    cout = torch.empty_like(t["u"]) if want_conv_out else None
    h0t = None if h0 is None else torch.from_numpy(np.asarray(h0, np.float32)).to(DEV)
    out, last = ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],
                                       z=t["z"], delta_bias=t["delta_bias"], h0=h0t,
                                       return_last_state=True, conv_weight=wt, conv_bias=bt,
                                       conv_state_in=st_in, conv_state_out=st_out,
                                       conv_out=cout, conv_silu=silu, workspace=workspace)
    torch.cuda.synchronize()
    return out, last, st_out, cout


def oracle_conv_scan(inp, w, b, st, silu=True, h0=None):
    u, st_out = oracle.causal_conv1d(inp["u"], w, bias=b, state=st, silu=silu, return_state=True)
    out, last = oracle.selective_scan(u, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                                      z=inp["z"], delta_bias=inp["delta_bias"], h0=h0,
                                      return_last_state=True)
    return out, last, st_out, u


def check(inp, io, K, seed, silu=True, st=True, label=""):
    batch, dim, L = inp["u"].shape
    w, b, s = conv_params(dim, K, seed, batch)
    s = as_io(s, io) if st else None            # conv state holds x values (exact in io)
    got = gpu_conv_scan(inp, w, b, s, silu=silu)
    ref = oracle_conv_scan(inp, w, b, s, silu=silu)
    e_out = row_rel_err(to_np(got[0]), ref[0])
    e_last = row_rel_err(to_np(got[1]), ref[1])
    e_u = row_rel_err(to_np(got[3]), ref[3])
    print(f"[conv {label}] err_out={e_out:.2e} err_last={e_last:.2e} err_u={e_u:.2e}", flush=True)
    assert e_out <= TOL[io] and e_last <= TOL[io] and e_u <= TOL[io]
    assert np.array_equal(to_np(got[2]), ref[2])


@pytest.mark.parametrize("blocks", [768, 769])
def test_conv4_readout_forms_either_side_of_the_grid_switch(blocks):
    """The width-4 conv scan on both sides of the 768-workgroup switch (the
    conv path keeps the end-of-block readout on both; the plain scan changes
    form there)."""
    inp = si.scan_inputs(1, 16 * blocks, 37, io_dtype="f32", seed=blocks)
    check(inp, "f32", 4, seed=blocks, label=f"{blocks} workgroups")


@pytest.mark.parametrize("batch,dim,L,io,K", [
    (2, 32, 64, "f32", 4), (1, 37, 37, "f32", 4), (2, 13, 100, "bf16", 3), (2, 16, 1000, "f32", 4),
    (1, 20, 50, "f32", 1), (1, 20, 50, "f32", 2), (2, 24, 70, "f32", 5), (2, 24, 70, "bf16", 8),
    (3, 8, 3, "f32", 4), (2, 8, 2, "bf16", 7),
])
def test_fused_conv_scan_matches_oracle(batch, dim, L, io, K):
    inp = si.scan_inputs(batch, dim, L, io_dtype=io, seed=L + dim + K)
    check(inp, io, K, seed=K, label=f"b{batch} d{dim} L{L} {io} K{K}")


def test_fused_conv_without_silu_and_without_state():
    inp = si.scan_inputs(2, 16, 80, seed=5)
    check(inp, "f32", 4, seed=5, silu=False, st=False, label="no silu, zero state")


def test_fused_conv_config1_layer():
    cfg = si.LAYER_130M
    inp = si.scan_inputs_for(cfg)
    check(inp, "f32", 4, seed=1, label="130m-like layer")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fused_conv_segmented_long_sequence(io):
    L = 3 * 32768 + 100
    inp = si.scan_inputs(1, 16, L, io_dtype=io, seed=88)
    check(inp, io, 4, seed=88, label=f"segmented {io}")


def test_chunked_prefill_hands_over_both_states():
    batch, dim, L, K, cut = 2, 20, 150, 4, 57
    inp = si.scan_inputs(batch, dim, L, seed=9)
    w, b, s = conv_params(dim, K, 9, batch)
    ref_out, ref_last, ref_st, _ = oracle_conv_scan(inp, w, b, s)
    first = {k: (np.ascontiguousarray(v[..., :cut]) if k in ("u", "delta", "z", "B", "C") else v)
             for k, v in inp.items()}
    second = {k: (np.ascontiguousarray(v[..., cut:]) if k in ("u", "delta", "z", "B", "C") else v)
              for k, v in inp.items()}
    o1, l1, s1, _ = gpu_conv_scan(first, w, b, s)
    o2, l2, s2, _ = gpu_conv_scan(second, w, b, to_np(s1).astype(np.float32), h0=to_np(l1))
    got = np.concatenate([to_np(o1), to_np(o2)], axis=2)
    e = row_rel_err(got, ref_out)
    el = row_rel_err(to_np(l2), ref_last)
    print(f"[conv chunked] err_out={e:.2e} err_last={el:.2e}", flush=True)
    assert e <= TOL["f32"] and el <= TOL["f32"]
    assert np.array_equal(to_np(s2), ref_st)


@pytest.mark.parametrize("io,K,batch,dim,L,S", [
    ("f32", 4, 3, 40, 48, 6), ("bf16", 4, 3, 40, 48, 6), ("f32", 2, 3, 40, 48, 6),
    ("bf16", 7, 3, 40, 48, 6),
    # a grid large enough that each decode thread takes two batch rows (odd
    # batch, a partial last channel block)
    ("bf16", 4, 51, 5100, 8, 3), ("f32", 3, 51, 5100, 8, 3)])
def test_decode_with_conv_continues_the_prefill(io, K, batch, dim, L, S):
    """Prefill L tokens, then decode S tokens one at a time from the returned
    SSM and conv states: the decode outputs equal the last S outputs of one
    prefill over L + S tokens."""
    inp = si.scan_inputs(batch, dim, L + S, io_dtype=io, seed=31 + K)
    w, b, st = conv_params(dim, K, 31, batch)
    st = as_io(st, io)
    ref_out, ref_last, ref_st, _ = oracle_conv_scan(inp, w, b, st)
    pre = {k: (np.ascontiguousarray(v[..., :L]) if k in ("u", "delta", "z", "B", "C") else v)
           for k, v in inp.items()}
    _, last, cst, _ = gpu_conv_scan(pre, w, b, st, want_conv_out=False)
    t = si.to_torch(inp, DEV)
    wt, bt = torch.from_numpy(w).to(DEV), torch.from_numpy(b).to(DEV)
    state = last.contiguous()
    outs = []
    for s in range(S):
        tt = L + s
        out = ssm.selective_state_update(state, t["u"][..., tt].contiguous(),
                                         t["delta"][..., tt].contiguous(), t["A"],
                                         t["B"][..., tt].contiguous(), t["C"][..., tt].contiguous(),
                                         D=t["D"], z=t["z"][..., tt].contiguous(),
                                         dt_bias=t["delta_bias"], conv_state=cst,
                                         conv_weight=wt, conv_bias=bt)
        outs.append(to_np(out))
    torch.cuda.synchronize()
    got = np.stack(outs, axis=2)
    e = row_rel_err(got, ref_out[..., L:])
    es = row_rel_err(to_np(state), ref_last)
    print(f"[conv decode {io} K{K}] err_out={e:.2e} err_state={es:.2e}", flush=True)
    assert e <= TOL[io] and es <= TOL[io]
    assert np.array_equal(to_np(cst), ref_st)
