"""fp64 CPU oracle for the selective scan (TEST INFRASTRUCTURE).

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The product path (the HIP library and its Python
binding) never does, and the two share no code: the oracle is the plain C file
ssm_oracle.c next to this file, compiled with gcc, wrapped here with ctypes.

Functions take numpy arrays of any float dtype (bf16 values arrive widened to
fp32 by the caller) and compute in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ssm_oracle.c into liboracle.so (gcc -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_selective_scan_f64.restype = ctypes.c_int
        lib.oracle_selective_scan_f64.argtypes = [I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P,
                                                  ctypes.c_int, P, P, P, ctypes.c_int]
        lib.oracle_state_update_f64.restype = ctypes.c_int
        lib.oracle_state_update_f64.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P, P,
                                                ctypes.c_int, P, ctypes.c_int]
        lib.oracle_selective_scan_bwd_f64.restype = ctypes.c_int
        lib.oracle_selective_scan_bwd_f64.argtypes = [I64, I64, I64, I64, I64] + [P] * 8 + [
            ctypes.c_int] + [P] * 12 + [ctypes.c_int]
        lib.oracle_causal_conv1d_f64.restype = ctypes.c_int
        lib.oracle_causal_conv1d_f64.argtypes = [I64, I64, I64, I64, P, P, P, P, ctypes.c_int,
                                                 P, P, ctypes.c_int]
        lib.oracle_conv_state_update_f64.restype = ctypes.c_int
        lib.oracle_conv_state_update_f64.argtypes = [I64, I64, I64, P, P, P, P, ctypes.c_int, P]
        lib.oracle_ssd_scan_f64.restype = ctypes.c_int
        lib.oracle_ssd_scan_f64.argtypes = [I64] * 6 + [P] * 8 + [ctypes.c_int, P, P, P,
                                                                  ctypes.c_int]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        _lib = lib
    return _lib


class use_library:
    """Context manager: run the oracle functions against another build of
    ssm_oracle.c (used by the test that plants mistakes in the oracle)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = None
        lib = ctypes.CDLL(self.path)
        for name in ("oracle_selective_scan_f64", "oracle_state_update_f64",
                     "oracle_selective_scan_bwd_f64", "oracle_causal_conv1d_f64",
                     "oracle_conv_state_update_f64", "oracle_ssd_scan_f64", "oracle_softplus",
                     "oracle_silu"):
            src = getattr(self.saved, name)
            dst = getattr(lib, name)
            dst.restype, dst.argtypes = src.restype, src.argtypes
        _lib = lib
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _groups(B, C, batch, dim, N, tail):
    """Number of B/C groups from the shape of B: (batch, N, *tail) is one
    group, (batch, G, N, *tail) is G groups of dim // G channels."""
    assert B.shape == C.shape
    if B.shape == (batch, N) + tail:
        return 1
    G = B.shape[1]
    assert B.shape == (batch, G, N) + tail and G >= 1 and dim % G == 0
    return G


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def silu(x: float) -> float:
    return _load().oracle_silu(float(x))


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                   h0=None, return_last_state=False, nthreads=0):
    """out[b,d,t] (and last_state[b,d,n]) in fp64.

    u, delta, z: (batch, dim, L); B, C: (batch, N, L), or (batch, G, N, L)
    with channel d reading group d // (dim // G); A: (dim, N); D, delta_bias:
    (dim,); h0: (batch, dim, N)."""
    lib = _load()
    u, delta, z, B, C, A, D, delta_bias, h0 = map(_f64, (u, delta, z, B, C, A, D, delta_bias, h0))
    batch, dim, L = u.shape
    N = A.shape[1]
    assert N <= 1024
    assert delta.shape == u.shape and (z is None or z.shape == u.shape)
    G = _groups(B, C, batch, dim, N, (L,))
    assert A.shape == (dim, N)
    out = np.empty_like(u)
    last = np.empty((batch, dim, N)) if return_last_state else None
    used = lib.oracle_selective_scan_f64(batch, dim, L, N, G, _ptr(u), _ptr(delta), _ptr(z),
                                         _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(delta_bias),
                                         int(bool(delta_softplus)), _ptr(h0), _ptr(out),
                                         _ptr(last), int(nthreads))
    selective_scan.last_threads = used
    return (out, last) if return_last_state else out


def state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
                 nthreads=0):
    """One decode token.  Returns (out (batch, dim), new_state (batch, dim, N));
    the input state is not modified."""
    lib = _load()
    s = np.array(state, dtype=np.float64, copy=True, order="C")
    x, dt, z, B, C, A, D, dt_bias = map(_f64, (x, dt, z, B, C, A, D, dt_bias))
    batch, dim, N = s.shape
    assert x.shape == (batch, dim) and dt.shape == (batch, dim)
    G = _groups(B, C, batch, dim, N, ())
    assert A.shape == (dim, N)
    out = np.empty((batch, dim))
    used = lib.oracle_state_update_f64(batch, dim, N, G, _ptr(s), _ptr(x), _ptr(dt), _ptr(z),
                                       _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(dt_bias),
                                       int(bool(dt_softplus)), _ptr(out), int(nthreads))
    state_update.last_threads = used
    return out, s


def selective_scan_bwd(dout, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, dlast=None, nthreads=0):
    """Gradients of the prefill scan in fp64 for the upstream gradient dout
    (batch, dim, L) on out and, optionally, dlast (batch, dim, N) on
    last_state.  Returns a dict with du, ddelta, dB, dC, dA and, when the
    matching input is given, dz, dD, ddelta_bias, dh0."""
    lib = _load()
    dout, dlast = _f64(dout), _f64(dlast)
    u, delta, z, B, C, A, D, delta_bias, h0 = map(_f64, (u, delta, z, B, C, A, D, delta_bias, h0))
    batch, dim, L = u.shape
    N = A.shape[1]
    assert dout.shape == u.shape and (dlast is None or dlast.shape == (batch, dim, N))
    G = _groups(B, C, batch, dim, N, (L,))
    assert A.shape == (dim, N)
    g = dict(du=np.empty_like(u), ddelta=np.empty_like(u), dB=np.empty(B.shape),
             dC=np.empty(B.shape), dA=np.empty((dim, N)))
    g["dz"] = np.empty_like(u) if z is not None else None
    g["dD"] = np.empty(dim) if D is not None else None
    g["ddelta_bias"] = np.empty(dim) if delta_bias is not None else None
    g["dh0"] = np.empty((batch, dim, N)) if h0 is not None else None
    used = lib.oracle_selective_scan_bwd_f64(
        batch, dim, L, N, G, _ptr(u), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), _ptr(dout), _ptr(dlast),
        _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dz"]), _ptr(g["dB"]), _ptr(g["dC"]),
        _ptr(g["dA"]), _ptr(g["dD"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), int(nthreads))
    selective_scan_bwd.last_threads = used
    return {k: v for k, v in g.items() if v is not None}


def causal_conv1d(x, weight, bias=None, state=None, silu=True, return_state=False, nthreads=0):
    """Causal depthwise conv of the block's conv branch, in fp64.
    x: (batch, dim, L); weight: (dim, K); bias: (dim,); state: (batch, dim,
    K) holding x[-K .. -1] (zeros when None).  Returns u (batch, dim, L) and,
    with return_state, the last K inputs (batch, dim, K)."""
    lib = _load()
    x, weight, bias, state = map(_f64, (x, weight, bias, state))
    batch, dim, L = x.shape
    K = weight.shape[1]
    assert weight.shape == (dim, K) and (state is None or state.shape == (batch, dim, K))
    u = np.empty_like(x)
    st = np.empty((batch, dim, K)) if return_state else None
    used = lib.oracle_causal_conv1d_f64(batch, dim, L, K, _ptr(x), _ptr(weight), _ptr(bias),
                                        _ptr(state), int(bool(silu)), _ptr(u), _ptr(st),
                                        int(nthreads))
    causal_conv1d.last_threads = used
    return (u, st) if return_state else u


def conv_state_update(state, x, weight, bias=None, silu=True):
    """One decode token of the conv branch.  Returns (u (batch, dim),
    new_state (batch, dim, K)); the input state is not modified."""
    lib = _load()
    s = np.array(state, dtype=np.float64, copy=True, order="C")
    x, weight, bias = map(_f64, (x, weight, bias))
    batch, dim, K = s.shape
    assert x.shape == (batch, dim) and weight.shape == (dim, K)
    u = np.empty((batch, dim))
    lib.oracle_conv_state_update_f64(batch, dim, K, _ptr(s), _ptr(x), _ptr(weight), _ptr(bias),
                                     int(bool(silu)), _ptr(u))
    return u, s


def ssd_scan(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
             return_last_state=False, nthreads=0):
    """Mamba-2 SSM (SSD layer) in fp64, recurrent form.

    x, z: (batch, L, H, P); dt: (batch, L, H); B, C: (batch, L, G, N) with
    head h reading group h // (H // G); A, D, dt_bias: (H,); h0: (batch, H,
    P, N).  Returns out (batch, L, H, P) and, with return_last_state, the
    final state (batch, H, P, N)."""
    lib = _load()
    x, dt, z, B, C, A, D, dt_bias, h0 = map(_f64, (x, dt, z, B, C, A, D, dt_bias, h0))
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (batch, L, H) and (z is None or z.shape == x.shape)
    assert B.shape == (batch, L, G, N) and C.shape == B.shape and H % G == 0
    assert A.shape == (H,) and (h0 is None or h0.shape == (batch, H, P, N))
    out = np.empty_like(x)
    last = np.empty((batch, H, P, N)) if return_last_state else None
    used = lib.oracle_ssd_scan_f64(batch, L, H, P, G, N, _ptr(x), _ptr(dt), _ptr(z), _ptr(B),
                                   _ptr(C), _ptr(A), _ptr(D), _ptr(dt_bias), int(bool(dt_softplus)),
                                   _ptr(h0), _ptr(out), _ptr(last), int(nthreads))
    ssd_scan.last_threads = used
    return (out, last) if return_last_state else out
