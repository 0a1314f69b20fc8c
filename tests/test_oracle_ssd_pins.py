"""Pins for the Mamba-2 (SSD layer) oracle, oracle.ssd_scan.

Each check rests on something other than the oracle's own loop:
  * the page's printed Mamba-2 parameter count decomposes only with one A,
    one D and one step bias per head and 2 * ngroups * d_state B/C numbers
    per token (Mamba model notes, section 8.2);
  * a Mamba-2 head of P channels is P Mamba-1 channels that share one step
    size, one scalar A (broadcast over the states) and one D: the Mamba-1
    oracle (pinned in test_oracle_pins.py) must give the same numbers bit
    for bit after the layout change;
  * the structured-matrix ("state space duality") form y = M x with
    M[t, s] = C_t . B_s exp(A (S_t - S_s)) Delta_s for s <= t, plus the
    initial state's free response C_t exp(A S_t) h0, evaluated directly in
    O(L^2) with numpy (the SSD view of the Mamba-2 section: the SSM as a
    structured matrix akin to masked attention);
  * split sequences carry the state bit-exactly; L = 1 and zero-input closed
    forms."""
import os

import numpy as np
import pytest
import scipy.special as sps

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def inputs(seed, batch=2, L=20, H=4, P=3, G=2, N=5, a_lo=-2.0, a_hi=-0.1):
    r = np.random.default_rng(seed)
    return dict(x=r.standard_normal((batch, L, H, P)), z=r.standard_normal((batch, L, H, P)),
                dt=0.4 * r.standard_normal((batch, L, H)),
                B=r.standard_normal((batch, L, G, N)), C=r.standard_normal((batch, L, G, N)),
                A=r.uniform(a_lo, a_hi, H), D=r.standard_normal(H),
                dt_bias=r.uniform(-3, 0, H), h0=r.standard_normal((batch, H, P, N)))


def run(p, **kw):
    return oracle.ssd_scan(p["x"], p["dt"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                           dt_bias=p["dt_bias"], h0=p["h0"], return_last_state=True, **kw)


def test_page_parameter_count_pins_head_layout():
    g = {}
    with open(os.path.join(GOLDEN, "mamba2_block_param_count.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                g[k.strip()] = int(v)
    d_inner = g["expand"] * g["d_model"]
    H = d_inner // g["headdim"]
    bc_per_token = 2 * g["ngroups"] * g["d_state"]     # B_t, C_t per group
    per_head = 3 * H                                    # A, D, step bias: one per head
    conv_ch = d_inner + bc_per_token                    # the conv runs over x, B and C
    count = (g["d_model"] * (2 * d_inner + bc_per_token + H)   # in_proj: z, x, B, C, dt
             + conv_ch * g["d_conv"] + conv_ch                 # depthwise conv + bias
             + per_head
             + d_inner                                         # gated RMSNorm weight
             + d_inner * g["d_model"])                         # out_proj
    assert count == g["params"]
    # an A per (head, state) or per channel would not add up
    assert count - H + H * g["d_state"] != g["params"]
    assert count - H + d_inner != g["params"]


@pytest.mark.parametrize("H,P,G,N", [(4, 3, 2, 5), (6, 1, 3, 8), (2, 8, 1, 16), (4, 4, 4, 2)])
def test_equals_mamba1_oracle_with_shared_head_parameters_bit_exact(H, P, G, N):
    p = inputs(H * 10 + N, H=H, P=P, G=G, N=N)
    out, last = run(p)
    batch, L = p["x"].shape[:2]
    # Mamba-1 view: channel d = h * P + p; (batch, d, L) layouts
    u = p["x"].reshape(batch, L, H * P).transpose(0, 2, 1).copy()
    z = p["z"].reshape(batch, L, H * P).transpose(0, 2, 1).copy()
    delta = np.repeat(p["dt"], P, axis=2).transpose(0, 2, 1).copy()
    A1 = np.repeat(np.repeat(p["A"][:, None], N, axis=1), P, axis=0)     # (H*P, N)
    D1 = np.repeat(p["D"], P)
    bias1 = np.repeat(p["dt_bias"], P)
    B1 = p["B"].transpose(0, 2, 3, 1).copy()                              # (batch, G, N, L)
    C1 = p["C"].transpose(0, 2, 3, 1).copy()
    h01 = p["h0"].reshape(batch, H * P, N)
    ref, rlast = oracle.selective_scan(u, delta, A1, B1, C1, D=D1, z=z, delta_bias=bias1,
                                       h0=h01, return_last_state=True)
    assert np.array_equal(out, ref.transpose(0, 2, 1).reshape(out.shape))
    assert np.array_equal(last, rlast.reshape(last.shape))


def structured_matrix_form(p, softplus=True):
    x, dt, B, C, A, D, bias, h0, z = (p[k] for k in ("x", "dt", "B", "C", "A", "D", "dt_bias",
                                                     "h0", "z"))
    batch, L, H, P = x.shape
    G = B.shape[2]
    xd = dt + bias[None, None, :]
    step = np.logaddexp(0.0, xd) if softplus else xd                  # (batch, L, H)
    S = np.cumsum(step, axis=1)
    out = np.empty_like(x)
    last = np.empty_like(h0)
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            CB = C[b, :, g, :] @ B[b, :, g, :].T                          # (t, s)
            seg = S[b, :, h][:, None] - S[b, :, h][None, :]              # S_t - S_s
            M = np.where(np.tril(np.ones((L, L), bool)), CB * np.exp(A[h] * seg), 0.0)
            M = M * step[b, :, h][None, :]
            y = M @ x[b, :, h, :]                                         # (L, P)
            free = np.exp(A[h] * S[b, :, h])                              # (L,)
            y += free[:, None] * (C[b, :, g, :] @ h0[b, h].T)             # C_t exp(A S_t) h0
            y += D[h] * x[b, :, h, :]
            out[b, :, h, :] = y * z[b, :, h, :] * sps.expit(z[b, :, h, :])
            # final state: exp(A S_L) h0 + sum_s exp(A (S_L - S_s)) Delta_s x_s B_s^T
            w = np.exp(A[h] * (S[b, -1, h] - S[b, :, h])) * step[b, :, h]
            last[b, h] = np.exp(A[h] * S[b, -1, h]) * h0[b, h] + (x[b, :, h, :] * w[:, None]).T @ B[b, :, g, :]
    return out, last


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("H,P,G,N,L", [(4, 3, 2, 5, 20), (2, 6, 1, 16, 33), (3, 2, 3, 4, 7)])
def test_structured_matrix_form(H, P, G, N, L, softplus):
    p = inputs(L + N, L=L, H=H, P=P, G=G, N=N)
    if not softplus:
        p["dt"] = np.abs(p["dt"]) * 0.2
        p["dt_bias"] = np.abs(p["dt_bias"]) * 0.01
    out, last = run(p, dt_softplus=softplus)
    want, wlast = structured_matrix_form(p, softplus)
    assert rel(out, want) < 1e-11
    assert rel(last, wlast) < 1e-11


def test_growing_modes_in_the_matrix_form():
    p = inputs(5, L=16, a_lo=-0.5, a_hi=0.5)
    out, last = run(p)
    want, wlast = structured_matrix_form(p)
    assert rel(out, want) < 1e-11 and rel(last, wlast) < 1e-11


@pytest.mark.parametrize("cut", [1, 7, 19])
def test_split_sequence_bit_exact(cut):
    p = inputs(9, L=20)
    out, last = run(p)
    a = dict(p, x=p["x"][:, :cut].copy(), z=p["z"][:, :cut].copy(), dt=p["dt"][:, :cut].copy(),
             B=p["B"][:, :cut].copy(), C=p["C"][:, :cut].copy())
    o1, l1 = run(a)
    b = dict(p, x=p["x"][:, cut:].copy(), z=p["z"][:, cut:].copy(), dt=p["dt"][:, cut:].copy(),
             B=p["B"][:, cut:].copy(), C=p["C"][:, cut:].copy(), h0=l1)
    o2, l2 = run(b)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), out)
    assert np.array_equal(l2, last)


def test_single_token_closed_form():
    p = inputs(11, L=1)
    out, last = run(p)
    step = np.logaddexp(0.0, p["dt"][:, 0] + p["dt_bias"])                     # (batch, H)
    H, G = p["A"].shape[0], p["B"].shape[2]
    for b in range(out.shape[0]):
        for h in range(H):
            g = h // (H // G)
            Sn = (np.exp(step[b, h] * p["A"][h]) * p["h0"][b, h]
                  + step[b, h] * np.outer(p["x"][b, 0, h], p["B"][b, 0, g]))
            y = Sn @ p["C"][b, 0, g] + p["D"][h] * p["x"][b, 0, h]
            zz = p["z"][b, 0, h]
            assert rel(out[b, 0, h], y * zz * sps.expit(zz)) < 1e-13
            assert rel(last[b, h], Sn) < 1e-13


def test_zero_input_decays_every_state_by_the_head_scalar():
    p = inputs(12, L=15)
    p["x"] = np.zeros_like(p["x"])
    _, last = run(p)
    S = np.logaddexp(0.0, p["dt"] + p["dt_bias"]).sum(axis=1)                 # (batch, H)
    want = np.exp(p["A"][None, :, None, None] * S[:, :, None, None]) * p["h0"]
    assert rel(last, want) < 1e-13
