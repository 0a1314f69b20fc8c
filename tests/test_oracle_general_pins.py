"""Pins of the oracle beyond the 16-state, one-group layout: the state size
over the pages' range (Mamba training/inference guide, parameter table:
d_state typically 8 to 64; Mamba-2 section of the mamba_ssm notes: 64 or
128), B/C in groups of channels (one group is the pages' layout, B_t and C_t
shared by every channel; dim groups is one B/C per channel), and A of either
sign.

As in test_oracle_pins.py, every check is against the mathematics, not the
oracle's loop: the unrolled closed form of the recurrence evaluated directly
(written here with its own group lookup), the LTI convolution for a growing
(A > 0) mode, decode == scan, exact Jacobian-vector products of the forward
for the backward's linear inputs, central differences for A, and the
decomposition of a grouped problem into one-group problems on each group's
channel slice."""
import numpy as np
import pytest
import scipy.special as sps

import oracle


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def grouped_inputs(seed, batch=2, dim=4, L=12, N=8, G=2, a_lo=-2.0, a_hi=0.5):
    r = np.random.default_rng(seed)
    return dict(u=r.standard_normal((batch, dim, L)), z=r.standard_normal((batch, dim, L)),
                delta=0.3 * r.standard_normal((batch, dim, L)),
                B=r.standard_normal((batch, G, N, L)), C=r.standard_normal((batch, G, N, L)),
                A=r.uniform(a_lo, a_hi, (dim, N)), D=r.standard_normal(dim),
                delta_bias=r.uniform(-3, 0, dim), h0=r.standard_normal((batch, dim, N)))


def unrolled_grouped(inp):
    """h_t[n] = exp(A_n S(0..t)) h0[n] + sum_{s<=t} exp(A_n S(s+1..t)) Delta_s B_s[n] u_s
    with B_s, C_t those of the channel's group (channels split into G equal,
    consecutive slices); y = C_t . h_t + D u_t; out = y silu(z)."""
    u, z, dt, B, C, A, D, bias, h0 = (inp[k] for k in ("u", "z", "delta", "B", "C", "A", "D",
                                                        "delta_bias", "h0"))
    batch, dim, L = u.shape
    G = B.shape[1]
    per = dim // G
    dl = np.logaddexp(0.0, dt + bias[None, :, None])
    S = np.cumsum(dl, axis=2)
    out = np.empty_like(u)
    last = np.empty_like(h0)
    for b in range(batch):
        for d in range(dim):
            g = d // per
            for t in range(L):
                h = np.exp(A[d] * S[b, d, t]) * h0[b, d]
                for s in range(t + 1):
                    h = h + np.exp(A[d] * (S[b, d, t] - S[b, d, s])) * dl[b, d, s] * B[b, g, :, s] * u[b, d, s]
                y = np.dot(C[b, g, :, t], h) + D[d] * u[b, d, t]
                out[b, d, t] = y * z[b, d, t] * sps.expit(z[b, d, t])
            last[b, d] = h
    return out, last


def run(inp, **kw):
    return oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                                 z=inp["z"], delta_bias=inp["delta_bias"], h0=inp["h0"],
                                 return_last_state=True, **kw)


@pytest.mark.parametrize("N", [1, 8, 33, 64])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_unrolled_sum_any_dstate_groups_and_sign(N, G):
    inp = grouped_inputs(100 + N + G, N=N, G=G)
    got, last = run(inp)
    want, wlast = unrolled_grouped(inp)
    assert rel(got, want) < 1e-11
    assert rel(last, wlast) < 1e-11


def test_one_group_4d_equals_3d_layout():
    inp = grouped_inputs(7, G=1)
    got, last = run(inp)
    flat = dict(inp, B=inp["B"][:, 0], C=inp["C"][:, 0])
    got3, last3 = run(flat)
    assert np.array_equal(got, got3) and np.array_equal(last, last3)


def test_group_decomposition_bit_exact():
    """A G-group scan is G independent one-group scans over the channel slices."""
    inp = grouped_inputs(8, dim=6, G=3, N=16)
    got, last = run(inp)
    for g in range(3):
        sl = slice(2 * g, 2 * g + 2)
        part = dict(u=inp["u"][:, sl], z=inp["z"][:, sl], delta=inp["delta"][:, sl],
                    B=inp["B"][:, g], C=inp["C"][:, g], A=inp["A"][sl], D=inp["D"][sl],
                    delta_bias=inp["delta_bias"][sl], h0=inp["h0"][:, sl])
        o, s = run(part)
        assert np.array_equal(o, got[:, sl]) and np.array_equal(s, last[:, sl])


def test_lti_convolution_growing_modes():
    """A > 0 (a growing mode) with constant Delta, B, C: still the causal
    convolution with K_k = sum_n C_n exp(k Delta A_n) Delta B_n (Mamba model
    notes, section 3.2)."""
    r = np.random.default_rng(21)
    batch, dim, L, N = 1, 3, 20, 64
    u = r.standard_normal((batch, dim, L))
    dl = r.uniform(0.01, 0.2, dim)
    Bn, Cn = r.standard_normal((batch, N)), r.standard_normal((batch, N))
    A = r.uniform(-1.0, 1.0, (dim, N))
    delta = np.broadcast_to(dl[None, :, None], (batch, dim, L)).copy()
    B = np.broadcast_to(Bn[:, :, None], (batch, N, L)).copy()
    C = np.broadcast_to(Cn[:, :, None], (batch, N, L)).copy()
    got = oracle.selective_scan(u, delta, A, B, C, delta_softplus=False)
    k = np.arange(L)
    decay = np.exp(k[None, None, :] * (dl[:, None] * A)[:, :, None])
    K = np.einsum("bn,dnk,bn->bdk", Cn, decay, Bn) * dl[None, :, None]
    want = np.zeros_like(u)
    for t in range(L):
        want[:, :, t] = np.einsum("bdk,bdk->bd", K[:, :, : t + 1], u[:, :, t::-1])
    assert rel(got, want) < 1e-12


@pytest.mark.parametrize("N,G", [(8, 2), (64, 4), (33, 1)])
def test_decode_equals_scan_grouped(N, G):
    inp = grouped_inputs(30 + N, L=9, N=N, G=G)
    want, wlast = run(inp)
    state = inp["h0"].copy()
    for t in range(inp["u"].shape[2]):
        o, state = oracle.state_update(state, inp["u"][:, :, t], inp["delta"][:, :, t], inp["A"],
                                       inp["B"][..., t], inp["C"][..., t], D=inp["D"],
                                       z=inp["z"][:, :, t], dt_bias=inp["delta_bias"])
        assert np.array_equal(o, want[:, :, t])
    assert np.array_equal(state, wlast)


# ---- backward with groups, any N, A of either sign -------------------------------------

def objective(p, dout, dlast):
    out, last = run(p)
    return float(np.sum(dout * out) + np.sum(dlast * last))


def grads(p, dout, dlast):
    return oracle.selective_scan_bwd(dout, p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"],
                                     z=p["z"], delta_bias=p["delta_bias"], h0=p["h0"], dlast=dlast)


@pytest.mark.parametrize("N,G", [(8, 2), (33, 4), (64, 1)])
@pytest.mark.parametrize("name", ["B", "C", "u", "h0"])
def test_grouped_backward_exact_jvp(name, N, G):
    p = grouped_inputs(40 + N + G, L=7, N=N, G=G)
    r = np.random.default_rng(41)
    dout, dlast = r.standard_normal(p["u"].shape), r.standard_normal(p["h0"].shape)
    key = {"B": "dB", "C": "dC", "u": "du", "h0": "dh0"}[name]
    g = grads(p, dout, dlast)[key]
    assert g.shape == p[name].shape
    f0 = objective(p, dout, dlast)
    for _ in range(2):
        V = r.standard_normal(p[name].shape)
        q = dict(p)
        q[name] = p[name] + V
        jvp = objective(q, dout, dlast) - f0
        assert abs(jvp - float(np.sum(g * V))) <= 1e-10 * max(1.0, abs(jvp))


@pytest.mark.parametrize("N,G", [(8, 2), (64, 4)])
def test_grouped_backward_dA_central_difference(N, G):
    p = grouped_inputs(50 + N, L=7, N=N, G=G)
    r = np.random.default_rng(51)
    dout, dlast = r.standard_normal(p["u"].shape), r.standard_normal(p["h0"].shape)
    g = grads(p, dout, dlast)["dA"]
    V = r.standard_normal(p["A"].shape)
    eps = 1e-6
    qp, qm = dict(p), dict(p)
    qp["A"], qm["A"] = p["A"] + eps * V, p["A"] - eps * V
    fd = (objective(qp, dout, dlast) - objective(qm, dout, dlast)) / (2 * eps)
    assert abs(fd - float(np.sum(g * V))) <= 1e-6 * max(1.0, abs(fd))


def test_grouped_backward_decomposes_by_group():
    p = grouped_inputs(60, dim=6, G=3, N=16, L=8)
    r = np.random.default_rng(61)
    dout, dlast = r.standard_normal(p["u"].shape), r.standard_normal(p["h0"].shape)
    g = grads(p, dout, dlast)
    for gi in range(3):
        sl = slice(2 * gi, 2 * gi + 2)
        part = {k: (v[:, sl] if k in ("u", "z", "delta", "h0") else v[sl] if k in ("A", "D", "delta_bias")
                    else v[:, gi]) for k, v in p.items()}
        gp = grads(part, dout[:, sl], dlast[:, sl])
        assert np.array_equal(gp["dB"], g["dB"][:, gi]) and np.array_equal(gp["dC"], g["dC"][:, gi])
        assert np.array_equal(gp["du"], g["du"][:, sl]) and np.array_equal(gp["dA"], g["dA"][sl])
