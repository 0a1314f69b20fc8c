"""Pins of the oracle's causal depthwise conv (the Mamba block's conv branch).

* Zero initial state, no activation: each row is a plain full convolution of
  x with the reversed kernel, cut to the first L outputs (numpy.convolve).
* A unit impulse at t0 reads the kernel back: pre[t0 + m] = w[K-1-m].
* Causality: changing x at t' leaves every output before t' unchanged.
* Splitting the sequence and handing the returned state to the second half
  reproduces the whole run bit for bit; so do L decode steps.
* K = 1 is pointwise: u = silu(w x + b)."""
import numpy as np
import pytest

import oracle


def silu(v):
    return v / (1.0 + np.exp(-v))


def data(batch=2, dim=3, L=23, K=4, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((batch, dim, L)), rng.standard_normal((dim, K)),
            rng.standard_normal(dim), rng.standard_normal((batch, dim, K)))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 7])
def test_zero_state_is_a_truncated_full_convolution(K):
    x, w, b, _ = data(K=K)
    u = oracle.causal_conv1d(x, w, bias=b, silu=False)
    for bi in range(x.shape[0]):
        for d in range(x.shape[1]):
            ref = np.convolve(x[bi, d], w[d][::-1])[: x.shape[2]] + b[d]
            np.testing.assert_allclose(u[bi, d], ref, rtol=1e-13, atol=1e-13)
    us = oracle.causal_conv1d(x, w, bias=b, silu=True)
    np.testing.assert_allclose(us, silu(u), rtol=1e-13, atol=1e-15)


def test_impulse_reads_the_kernel_back():
    K, L, t0 = 4, 12, 5
    w = np.arange(1.0, 1.0 + K)[None, :] * np.array([[1.0], [-0.5]])
    x = np.zeros((1, 2, L))
    x[..., t0] = 1.0
    u = oracle.causal_conv1d(x, w, silu=False)
    for d in range(2):
        expect = np.zeros(L)
        for m in range(K):
            expect[t0 + m] = w[d, K - 1 - m]
        assert np.array_equal(u[0, d], expect)


def test_causality():
    x, w, b, st = data(L=30)
    u1 = oracle.causal_conv1d(x, w, bias=b, state=st)
    x2 = x.copy()
    x2[..., 17:] += 3.0
    u2 = oracle.causal_conv1d(x2, w, bias=b, state=st)
    assert np.array_equal(u1[..., :17], u2[..., :17])
    assert not np.array_equal(u1[..., 17:], u2[..., 17:])


@pytest.mark.parametrize("cut", [1, 2, 3, 9, 22])
def test_split_with_state_is_bit_exact(cut):
    x, w, b, st = data(L=23)
    u, s_end = oracle.causal_conv1d(x, w, bias=b, state=st, return_state=True)
    u1, s1 = oracle.causal_conv1d(np.ascontiguousarray(x[..., :cut]), w, bias=b, state=st,
                                  return_state=True)
    u2, s2 = oracle.causal_conv1d(np.ascontiguousarray(x[..., cut:]), w, bias=b, state=s1,
                                  return_state=True)
    assert np.array_equal(np.concatenate([u1, u2], axis=2), u)
    assert np.array_equal(s2, s_end)


def test_returned_state_is_the_last_inputs():
    x, w, b, st = data(L=23, K=4)
    _, s = oracle.causal_conv1d(x, w, bias=b, state=st, return_state=True)
    assert np.array_equal(s, x[..., -4:])
    xs = np.ascontiguousarray(x[..., :2])                 # shorter than K: state fills in
    _, s = oracle.causal_conv1d(xs, w, bias=b, state=st, return_state=True)
    assert np.array_equal(s, np.concatenate([st[..., 2:], xs], axis=2))


def test_decode_steps_equal_prefill_bit_exact():
    x, w, b, st = data(L=11)
    u, s_end = oracle.causal_conv1d(x, w, bias=b, state=st, return_state=True)
    s = st
    for t in range(x.shape[2]):
        ut, s = oracle.conv_state_update(s, x[..., t], w, bias=b)
        assert np.array_equal(ut, u[..., t])
    assert np.array_equal(s, s_end)


def test_width_one_is_pointwise():
    x, w, b, _ = data(K=1)
    u = oracle.causal_conv1d(x, w, bias=b)
    np.testing.assert_allclose(u, silu(w[None, :, 0:1] * x + b[None, :, None]), rtol=1e-14)
