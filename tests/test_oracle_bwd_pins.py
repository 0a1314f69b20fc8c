"""Pins of the oracle's backward (the reverse-mode derivative of the prefill
scan).  Every gradient is checked against the forward oracle alone:

* out and last_state are linear in u, B, C, D and h0 (Delta depends on delta
  and the bias only), so for any direction V the forward difference
  f(X + V) - f(X) equals the Jacobian-vector product exactly, up to fp64
  rounding; <dout, J V> must equal <grad_X, V>;
* for delta, A, z and the bias, central differences of the forward along
  random directions agree with <grad, V> to the truncation error;
* closed forms: the gradient of last_state with respect to h0 is the decay
  exp(A * sum of Delta) alone, and at L = 1 with no state the gradient of out
  with respect to u is Delta * sum_n C_n B_n + D.

A mistake in the backward (a dropped term, a wrong sign, a missing chain-rule
factor, a wrong time index) changes <grad, V> and fails one of these; the
planted mistakes in test_oracle_mutants.py show it."""
import numpy as np
import pytest

import oracle
import synth_inputs as si

LINEAR = ["u", "B", "C", "D", "h0"]
NONLINEAR = ["delta", "A", "z", "delta_bias"]


def make(batch=2, dim=3, L=9, N=4, seed=5, h0=True):
    inp = si.scan_inputs(batch, dim, L, dstate=N, seed=seed)
    rng = np.random.default_rng(seed + 1)
    p = {k: np.asarray(inp[k], dtype=np.float64) for k in
         ("u", "delta", "z", "B", "C", "A", "D", "delta_bias")}
    p["A"] = p["A"] * rng.uniform(0.5, 2.0, p["A"].shape)   # a less regular A
    p["delta"] = p["delta"] * 5.0                            # Delta over a wider range
    p["h0"] = rng.standard_normal((batch, dim, N)) if h0 else None
    dout = rng.standard_normal(p["u"].shape)
    dlast = rng.standard_normal((batch, dim, N))
    return p, dout, dlast


def forward(p, softplus=True):
    return oracle.selective_scan(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                                 delta_bias=p["delta_bias"], delta_softplus=softplus,
                                 h0=p["h0"], return_last_state=True)


def objective(p, dout, dlast, softplus=True):
    out, last = forward(p, softplus)
    return float(np.sum(dout * out) + (np.sum(dlast * last) if dlast is not None else 0.0))


def grads(p, dout, dlast, softplus=True):
    return oracle.selective_scan_bwd(dout, p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"],
                                     z=p["z"], delta_bias=p["delta_bias"],
                                     delta_softplus=softplus, h0=p["h0"], dlast=dlast)


GRAD_KEY = {"u": "du", "delta": "ddelta", "z": "dz", "B": "dB", "C": "dC", "A": "dA",
            "D": "dD", "delta_bias": "ddelta_bias", "h0": "dh0"}


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("name", LINEAR)
def test_linear_inputs_exact_jvp(name, softplus):
    p, dout, dlast = make()
    if not softplus:                                           # keep Delta positive
        p["delta"] = np.abs(p["delta"]) + 0.05
        p["delta_bias"] = np.abs(p["delta_bias"]) * 0.01
    g = grads(p, dout, dlast, softplus)[GRAD_KEY[name]]
    f0 = objective(p, dout, dlast, softplus)
    rng = np.random.default_rng(11)
    for _ in range(3):
        V = rng.standard_normal(p[name].shape)
        q = dict(p)
        q[name] = p[name] + V
        jvp = objective(q, dout, dlast, softplus) - f0
        est = float(np.sum(g * V))
        assert abs(jvp - est) <= 1e-10 * max(1.0, abs(jvp)), (name, jvp, est)


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("name", NONLINEAR)
def test_nonlinear_inputs_central_difference(name, softplus):
    p, dout, dlast = make()
    if not softplus:                                           # keep Delta positive
        p["delta"] = np.abs(p["delta"]) + 0.05
        p["delta_bias"] = np.abs(p["delta_bias"]) * 0.01
    g = grads(p, dout, dlast, softplus)[GRAD_KEY[name]]
    rng = np.random.default_rng(12)
    for _ in range(3):
        V = rng.standard_normal(p[name].shape)
        eps = 1e-6
        qp, qm = dict(p), dict(p)
        qp[name] = p[name] + eps * V
        qm[name] = p[name] - eps * V
        fd = (objective(qp, dout, dlast, softplus) - objective(qm, dout, dlast, softplus)) / (2 * eps)
        est = float(np.sum(g * V))
        assert abs(fd - est) <= 1e-6 * max(1.0, abs(fd)), (name, fd, est)


def test_every_element_of_du_by_unit_directions():
    """Element by element for u on a tiny case: with unit directions the exact
    forward difference is one column of the Jacobian, so the whole du array is
    pinned, not only its projections."""
    p, dout, dlast = make(batch=1, dim=2, L=5, N=3)
    g = grads(p, dout, dlast)["du"]
    f0 = objective(p, dout, dlast)
    for idx in np.ndindex(p["u"].shape):
        q = dict(p)
        q["u"] = p["u"].copy()
        q["u"][idx] += 1.0
        assert abs((objective(q, dout, dlast) - f0) - g[idx]) <= 1e-12 * max(1.0, abs(g[idx]))


def test_last_state_gradient_wrt_h0_is_the_total_decay():
    p, _, dlast = make()
    dout = np.zeros_like(p["u"])
    g = grads(p, dout, dlast)
    x = p["delta"] + p["delta_bias"][None, :, None]
    S = np.logaddexp(0.0, x).sum(axis=2)                     # sum of softplus over t
    expect = dlast * np.exp(p["A"][None, :, :] * S[:, :, None])
    np.testing.assert_allclose(g["dh0"], expect, rtol=1e-12, atol=1e-15)


def test_single_token_du_closed_form():
    p, dout, _ = make(L=1, h0=False)
    p["z"] = None
    g = grads(p, dout, None)
    x = p["delta"][..., 0] + p["delta_bias"][None, :]
    dl = np.logaddexp(0.0, x)                                # (batch, dim)
    cb = np.einsum("bn,bn->b", p["C"][..., 0], p["B"][..., 0])
    expect = dout[..., 0] * (dl * cb[:, None] + p["D"][None, :])
    np.testing.assert_allclose(g["du"][..., 0], expect, rtol=1e-12)


def test_backward_is_linear_in_the_upstream_gradient():
    p, dout, dlast = make()
    g1 = grads(p, dout, dlast)
    g2 = grads(p, 2.5 * dout, 2.5 * dlast)
    for k in g1:
        np.testing.assert_allclose(g2[k], 2.5 * g1[k], rtol=1e-12, atol=1e-14)


def test_thread_count_does_not_change_the_result():
    p, dout, dlast = make(batch=3, dim=8, L=33)
    g1 = oracle.selective_scan_bwd(dout, p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"],
                                   z=p["z"], delta_bias=p["delta_bias"], h0=p["h0"],
                                   dlast=dlast, nthreads=1)
    g4 = oracle.selective_scan_bwd(dout, p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"],
                                   z=p["z"], delta_bias=p["delta_bias"], h0=p["h0"],
                                   dlast=dlast, nthreads=4)
    for k in g1:
        assert np.array_equal(g1[k], g4[k]), k
