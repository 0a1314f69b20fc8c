"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, none of which re-types the oracle's own loop.

Each test names the passage it rests on (page title and section).  A
plausible mistake in the oracle (a dropped term, a wrong sign, B and C
swapped, a missing softplus, the gate before the skip term, an off-by-one in
the recurrence) fails at least one of them:
  * LTI convolution (constant Delta, B, C)  -> recurrence + readout + h0 path
  * unrolled-sum brute force, fp64 and 40-digit decimal -> time-varying case,
    B/C time indices, softplus, gate order
  * Delta -> 0, reset (exp underflow), A = 0 prefix sum, L = 1 closed form
  * split sequence and decode == scan (bit-exact), linearity
  * softplus identities and the page's printed Mamba parameter count.
"""
import decimal
import os

import numpy as np
import pytest
import scipy.special as sps

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def tiny_inputs(seed, batch=2, dim=3, L=24, N=5, softplus=True):
    r = rng(seed)
    d = dict(u=r.standard_normal((batch, dim, L)), z=r.standard_normal((batch, dim, L)),
             delta=0.3 * r.standard_normal((batch, dim, L)),
             B=r.standard_normal((batch, N, L)), C=r.standard_normal((batch, N, L)),
             A=-r.uniform(0.2, 3.0, (dim, N)), D=r.standard_normal(dim),
             delta_bias=r.uniform(-3, 0, dim), h0=r.standard_normal((batch, dim, N)))
    return d


# --------------------------------------------------------------------------------------
# P1: LTI special case is a causal convolution.
# Mamba model notes, section 3.2 and Mamba paper notes, section 2.2: with parameters
# that do not depend on the token, the recurrence equals a convolution with a fixed
# kernel K_k = C . Abar^k . Bbar.
@pytest.mark.parametrize("with_h0", [False, True])
def test_lti_convolution(with_h0):
    r = rng(1)
    batch, dim, L, N = 2, 4, 48, 16
    u = r.standard_normal((batch, dim, L))
    dl = r.uniform(0.01, 0.5, dim)                       # constant step per channel
    Bn = r.standard_normal((batch, N))
    Cn = r.standard_normal((batch, N))
    A = -r.uniform(0.1, 4.0, (dim, N))
    D = r.standard_normal(dim)
    h0 = r.standard_normal((batch, dim, N)) if with_h0 else None
    delta = np.broadcast_to(dl[None, :, None], (batch, dim, L)).copy()
    B = np.broadcast_to(Bn[:, :, None], (batch, N, L)).copy()
    C = np.broadcast_to(Cn[:, :, None], (batch, N, L)).copy()
    got = oracle.selective_scan(u, delta, A, B, C, D=D, delta_softplus=False, h0=h0)

    k = np.arange(L)
    # K[b, d, k] = sum_n C[b,n] exp(k dl_d A[d,n]) dl_d B[b,n]
    decay = np.exp(k[None, None, :] * (dl[:, None] * A)[:, :, None])          # (dim, N, L)
    K = np.einsum("bn,dnk,bn->bdk", Cn, decay, Bn) * dl[None, :, None]
    want = np.zeros_like(u)
    for t in range(L):
        want[:, :, t] = np.einsum("bdk,bdk->bd", K[:, :, : t + 1], u[:, :, t::-1])
    want += D[None, :, None] * u
    if with_h0:
        # free response of the initial state: sum_n C_n exp((t+1) dl A_n) h0_n
        dec1 = np.exp((k + 1)[None, None, :] * (dl[:, None] * A)[:, :, None])  # (dim, N, L)
        want += np.einsum("bn,dnt,bdn->bdt", Cn, dec1, h0)
    assert rel(got, want) < 1e-12


# --------------------------------------------------------------------------------------
# P9: unrolled sum of the time-varying recurrence (Mamba model notes section 2.2 with
# the selection of section 4.1 and the discretisation of the paper notes section 2.3):
#   h_t[n] = exp(A_n S(0..t)) h0[n] + sum_{s<=t} exp(A_n S(s+1..t)) Delta_s B_s[n] u_s
#   S(i..j) = sum of Delta over i..j;  y_t = sum_n C_t[n] h_t[n] + D u_t;  out = y silu(z).
def unrolled_fp64(inp, softplus=True):
    u, z, dt, B, C, A, D, bias, h0 = (inp[k] for k in ("u", "z", "delta", "B", "C", "A", "D",
                                                        "delta_bias", "h0"))
    batch, dim, L = u.shape
    x = dt + bias[None, :, None]
    dl = np.logaddexp(0.0, x) if softplus else x              # library softplus
    S = np.cumsum(dl, axis=2)                                  # S(0..t)
    out = np.empty_like(u)
    last = np.empty_like(h0)
    for b in range(batch):
        for d in range(dim):
            for t in range(L):
                free = np.exp(A[d] * S[b, d, t]) * h0[b, d]
                forced = np.zeros_like(A[d])
                for s in range(t + 1):
                    seg = S[b, d, t] - S[b, d, s]              # S(s+1..t)
                    forced += np.exp(A[d] * seg) * dl[b, d, s] * B[b, :, s] * u[b, d, s]
                h = free + forced
                y = np.dot(C[b, :, t], h) + D[d] * u[b, d, t]
                out[b, d, t] = y * z[b, d, t] * sps.expit(z[b, d, t])
            last[b, d] = h
    return out, last


def test_unrolled_sum_fp64():
    inp = tiny_inputs(2, batch=2, dim=3, L=24, N=5)
    got, last = oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                      D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                      h0=inp["h0"], return_last_state=True)
    want, wlast = unrolled_fp64(inp)
    assert rel(got, want) < 1e-11
    assert rel(last, wlast) < 1e-11


def test_unrolled_sum_decimal40():
    """Same closed form evaluated with 40-digit decimal arithmetic (stdlib exp/ln);
    bounds the oracle's own fp64 error."""
    ctx = decimal.Context(prec=40)
    Dm = lambda v: ctx.create_decimal(repr(float(v)))  # exact binary64 value, as decimal
    inp = tiny_inputs(3, batch=1, dim=2, L=10, N=4)
    got, last = oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                      D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                      h0=inp["h0"], return_last_state=True)
    u, z, dt, B, C, A, Dv, bias, h0 = (inp[k] for k in ("u", "z", "delta", "B", "C", "A", "D",
                                                         "delta_bias", "h0"))
    _, dim, L = u.shape
    N = A.shape[1]
    one = ctx.create_decimal(1)
    for d in range(dim):
        dl = []
        for t in range(L):
            x = ctx.add(Dm(dt[0, d, t]), Dm(bias[d]))
            dl.append(ctx.ln(ctx.add(one, ctx.exp(x))))          # softplus
        S = [sum(dl[: t + 1], ctx.create_decimal(0)) for t in range(L)]
        for t in range(L):
            y = ctx.create_decimal(0)
            hs = []
            for n in range(N):
                a = Dm(A[d, n])
                h = ctx.exp(a * S[t]) * Dm(h0[0, d, n])
                for s in range(t + 1):
                    h += ctx.exp(a * (S[t] - S[s])) * dl[s] * Dm(B[0, n, s]) * Dm(u[0, d, s])
                hs.append(h)
                y += Dm(C[0, n, t]) * h
            y += Dm(Dv[d]) * Dm(u[0, d, t])
            zz = Dm(z[0, d, t])
            y = y * zz / (one + ctx.exp(-zz))
            assert abs(float(y) - got[0, d, t]) <= 1e-13 * max(1.0, abs(float(y)))
        for n in range(N):
            assert abs(float(hs[n]) - last[0, d, n]) <= 1e-13 * max(1.0, abs(float(hs[n])))


# --------------------------------------------------------------------------------------
# P2: Delta -> 0 keeps the state (Mamba model notes section 4.1: small Delta keeps the
# memory; paper notes section 2.3: a small step leaves the state almost unchanged).
def test_delta_zero_keeps_state_exactly():
    inp = tiny_inputs(4, L=30)
    zeros = np.zeros_like(inp["delta"])
    out, last = oracle.selective_scan(inp["u"], zeros, inp["A"], inp["B"], inp["C"], D=inp["D"],
                                      delta_softplus=False, h0=inp["h0"], return_last_state=True)
    assert np.array_equal(last, inp["h0"])                     # bit-exact
    want = np.einsum("bnt,bdn->bdt", inp["C"], inp["h0"]) + inp["D"][None, :, None] * inp["u"]
    assert rel(out, want) < 1e-14


def test_delta_tiny_with_softplus_bounded_drift():
    inp = tiny_inputs(5, L=30)
    dt = np.full_like(inp["delta"], -40.0)                    # softplus(-40) ~ 4.2e-18
    _, last = oracle.selective_scan(inp["u"], dt, inp["A"], inp["B"], inp["C"],
                                    h0=inp["h0"], return_last_state=True)
    L = dt.shape[2]
    dl = np.logaddexp(0.0, -40.0)
    bound = L * dl * (np.max(np.abs(inp["B"])) * np.max(np.abs(inp["u"]))
                      + np.max(np.abs(inp["A"])) * np.max(np.abs(inp["h0"])) * 2)
    assert np.max(np.abs(last - inp["h0"])) <= bound


# --------------------------------------------------------------------------------------
# P3: L = 1 closed form (every term appears once).
def test_single_token_closed_form():
    inp = tiny_inputs(6, L=1, N=16)
    out, last = oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                      D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                      h0=inp["h0"], return_last_state=True)
    dl = np.logaddexp(0.0, inp["delta"][..., 0] + inp["delta_bias"][None, :])   # (b, d)
    u = inp["u"][..., 0]
    h = (np.exp(dl[..., None] * inp["A"][None]) * inp["h0"]
         + dl[..., None] * inp["B"][:, None, :, 0] * u[..., None])
    y = np.einsum("bdn,bn->bd", h, inp["C"][..., 0]) + inp["D"][None] * u
    zz = inp["z"][..., 0]
    want = y * zz * sps.expit(zz)
    assert rel(out[..., 0], want) < 1e-14
    assert rel(last, h) < 1e-14


def test_single_token_zero_state():
    """h0 = 0, no gate: y = Delta u sum_n B_n C_n + D u."""
    inp = tiny_inputs(7, L=1, N=16)
    out = oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                                delta_bias=inp["delta_bias"])
    dl = np.logaddexp(0.0, inp["delta"][..., 0] + inp["delta_bias"][None, :])
    u = inp["u"][..., 0]
    bc = np.einsum("bn,bn->b", inp["B"][..., 0], inp["C"][..., 0])
    want = dl * u * bc[:, None] + inp["D"][None] * u
    assert rel(out[..., 0], want) < 1e-14


# --------------------------------------------------------------------------------------
# P4: split sequence with the carried state equals the full run (paper notes, section
# 5.3/5.4: long inputs are cut into chunks and the state is handed from one to the next).
@pytest.mark.parametrize("cut", [1, 13, 20, 39])
def test_split_sequence_bit_exact(cut):
    inp = tiny_inputs(8, L=40)
    full, flast = oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                        D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                        h0=inp["h0"], return_last_state=True)
    sl = lambda k, a, b: np.ascontiguousarray(inp[k][..., a:b])
    o1, l1 = oracle.selective_scan(sl("u", 0, cut), sl("delta", 0, cut), inp["A"],
                                   sl("B", 0, cut), sl("C", 0, cut), D=inp["D"],
                                   z=sl("z", 0, cut), delta_bias=inp["delta_bias"], h0=inp["h0"],
                                   return_last_state=True)
    o2, l2 = oracle.selective_scan(sl("u", cut, 40), sl("delta", cut, 40), inp["A"],
                                   sl("B", cut, 40), sl("C", cut, 40), D=inp["D"],
                                   z=sl("z", cut, 40), delta_bias=inp["delta_bias"], h0=l1,
                                   return_last_state=True)
    assert np.array_equal(np.concatenate([o1, o2], axis=2), full)
    assert np.array_equal(l2, flast)


# --------------------------------------------------------------------------------------
# P5: decode == scan (paper notes, section 4.3: the step form and the scan share the
# parameters and compute the same thing).  Separate code paths, bit-exact.
def test_decode_equals_scan_bit_exact():
    inp = tiny_inputs(9, L=25, N=16)
    full, flast = oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                        D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                        h0=inp["h0"], return_last_state=True)
    state = inp["h0"].copy()
    for t in range(25):
        o, state = oracle.state_update(state, inp["u"][..., t], inp["delta"][..., t], inp["A"],
                                       inp["B"][..., t], inp["C"][..., t], D=inp["D"],
                                       z=inp["z"][..., t], dt_bias=inp["delta_bias"])
        assert np.array_equal(o, full[..., t])
    assert np.array_equal(state, flast)


# --------------------------------------------------------------------------------------
# P6: reset.  Mamba model notes section 4.1: a large Delta rewrites the state.  When
# exp(Delta A) underflows to zero, h_t = Delta_t B_t u_t exactly (memoryless).
def test_reset_when_decay_underflows():
    inp = tiny_inputs(10, L=20, N=8)
    A = np.full_like(inp["A"], -1e5)
    dl = np.abs(inp["delta"]) + 0.05                          # Delta*A <= -5000 -> exp == 0
    out, last = oracle.selective_scan(inp["u"], dl, A, inp["B"], inp["C"], D=None,
                                      delta_softplus=False, h0=inp["h0"], return_last_state=True)
    h = dl[:, :, None, :] * inp["B"][:, None, :, :] * inp["u"][:, :, None, :]   # (b,d,n,t)
    want = np.einsum("bdnt,bnt->bdt", h, inp["C"])
    assert rel(out, want) < 1e-14
    assert rel(last, h[..., -1]) < 1e-14


# --------------------------------------------------------------------------------------
# P7: A = 0 -> Abar = 1 and the state is a prefix sum of Delta B u.
def test_zero_A_is_prefix_sum():
    inp = tiny_inputs(11, L=32, N=6)
    A = np.zeros_like(inp["A"])
    out, last = oracle.selective_scan(inp["u"], inp["delta"], A, inp["B"], inp["C"],
                                      delta_bias=inp["delta_bias"], h0=inp["h0"],
                                      return_last_state=True)
    dl = np.logaddexp(0.0, inp["delta"] + inp["delta_bias"][None, :, None])
    inc = dl[:, :, None, :] * inp["B"][:, None, :, :] * inp["u"][:, :, None, :]
    h = inp["h0"][..., None] + np.cumsum(inc, axis=3)
    want = np.einsum("bdnt,bnt->bdt", h, inp["C"])
    assert rel(out, want) < 1e-13
    assert rel(last, h[..., -1]) < 1e-13


# --------------------------------------------------------------------------------------
# P8: with Delta, B, C fixed and no gate the output is linear in (u, h0)
# (Mamba model notes section 2.2: the discrete system is linear in input and state).
def test_linearity_in_input_and_state():
    a, b = 0.7, -1.9
    i1, i2 = tiny_inputs(12, L=30), tiny_inputs(13, L=30)
    common = dict(A=i1["A"], B=i1["B"], C=i1["C"], D=i1["D"], delta_bias=i1["delta_bias"])

    def run(u, h0):
        return oracle.selective_scan(u, i1["delta"], common["A"], common["B"], common["C"],
                                     D=common["D"], delta_bias=common["delta_bias"], h0=h0)

    y1, y2 = run(i1["u"], i1["h0"]), run(i2["u"], i2["h0"])
    y = run(a * i1["u"] + b * i2["u"], a * i1["h0"] + b * i2["h0"])
    assert rel(y, a * y1 + b * y2) < 1e-12


# --------------------------------------------------------------------------------------
# P10: softplus (paper notes section 2.3 and 5.5: Delta goes through a softplus with a
# bias) and the data generator's bias.
def test_softplus_identities_and_bias():
    for x in [-50.0, -7.3, -1e-3, 0.0, 0.5, 3.0, 25.0, 700.0]:
        assert abs(oracle.softplus(x) - oracle.softplus(-x) - x) <= 1e-15 * max(1.0, abs(x))
        assert abs(oracle.softplus(x) - float(np.logaddexp(0.0, x))) <= 1e-15 * max(1.0, abs(x))
    assert oracle.softplus(-745.0) > 0.0
    assert abs(oracle.softplus(-30.0) / np.exp(-30.0) - 1.0) < 1e-12
    assert abs(oracle.silu(2.5) - 2.5 * sps.expit(2.5)) < 1e-15
    r = rng(0)
    delta0 = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), 64))
    bias = si.delta_bias_from_delta0(delta0)
    back = np.array([oracle.softplus(float(b)) for b in bias])
    assert np.max(np.abs(back / delta0 - 1.0)) < 1e-5      # bias is stored as fp32


# --------------------------------------------------------------------------------------
# NaN propagation (IEEE): a NaN input poisons its own row from that token on, and
# nothing else.
def test_nan_propagates_within_row_only():
    inp = tiny_inputs(14, L=16)
    u = inp["u"].copy()
    u[0, 1, 5] = np.nan
    out = oracle.selective_scan(u, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                                z=inp["z"], delta_bias=inp["delta_bias"])
    assert np.all(np.isnan(out[0, 1, 5:])) and not np.any(np.isnan(out[0, 1, :5]))
    mask = np.ones(out.shape, bool)
    mask[0, 1, 5:] = False
    assert not np.any(np.isnan(out[mask]))


def test_empty_sequence_returns_initial_state():
    inp = tiny_inputs(15, L=1)
    e = lambda k: np.zeros(inp[k].shape[:-1] + (0,))
    out, last = oracle.selective_scan(e("u"), e("delta"), inp["A"], e("B"), e("C"),
                                      h0=inp["h0"], return_last_state=True)
    assert out.shape[-1] == 0 and np.array_equal(last, inp["h0"])


# --------------------------------------------------------------------------------------
# P11: layout conventions.  Mamba model notes section 8.1 prints the parameter count of
# Mamba(d_model=16, d_state=64, d_conv=4, expand=2).  It decomposes only if A is
# (d_inner x d_state), D and the Delta bias are per channel, and each token carries
# 2*d_state numbers (B_t, C_t) shared by all channels -- the layouts used here.
def test_page_parameter_count_pins_layouts():
    golden = {}
    with open(os.path.join(GOLDEN, "mamba_block_param_count.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                golden[k.strip()] = int(v)
    d_model, d_state, d_conv, expand = (golden[k] for k in ("d_model", "d_state", "d_conv",
                                                             "expand"))
    d_inner = expand * d_model
    dt_rank = -(-d_model // 16)
    A_shape = (d_inner, d_state)              # one diagonal A per channel
    D_shape = (d_inner,)                      # skip weight per channel
    bias_shape = (d_inner,)                   # Delta bias per channel
    per_token_BC = 2 * d_state                # B_t and C_t, shared across channels
    count = (d_model * 2 * d_inner                       # in_proj (x and gate z), no bias
             + d_inner * d_conv + d_inner                # depthwise conv + bias
             + d_inner * (dt_rank + per_token_BC)        # x_proj -> (dt, B, C)
             + dt_rank * d_inner + bias_shape[0]         # dt_proj weight + Delta bias
             + int(np.prod(A_shape)) + D_shape[0]        # A, D
             + d_inner * d_model)                        # out_proj
    assert count == golden["params"]
