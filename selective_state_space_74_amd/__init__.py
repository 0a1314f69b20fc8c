"""MI355X (gfx950) selective scan: Python binding over libssm.so.

This module only marshals arguments: it checks tensor placement and dtypes,
allocates outputs through torch, fills the C argument blocks declared in
include/ssm.h and calls the library on torch's current HIP stream.  Every step
of the computation runs in the HIP kernels of libssm.so; there is no Python or
CPU fallback, and importing a missing library raises.

    selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, return_last_state=False,
                       checkpoints=None)
        -> out, or (out, last_state)
    selective_scan_bwd(dout, u, delta, A, B, C, checkpoints, D=None, z=None,
                       delta_bias=None, delta_softplus=True, h0=None, dlast=None)
        -> dict of gradients (du, ddelta, dB, dC, dA and dz, dD,
           ddelta_bias, dh0 for the inputs that were given)
    selective_state_update(state, x, dt, A, B, C, D=None, z=None,
                           dt_bias=None, dt_softplus=True) -> out  (state updated in place)

Shapes (N = dstate, 1..64): u, delta, z (batch, dim, L) with time stride 1;
B, C (batch, N, L), or (batch, G, N, L) for G groups of dim // G channels,
with time stride 1; A (dim, N) fp32; D, delta_bias (dim,) fp32; h0 and
last_state (batch, dim, N) fp32.  Decode: state (batch, dim, N) fp32 with
state stride 1; x, dt, z (batch, dim); B, C (batch, N) or (batch, G, N).
IO tensors are float32 or bfloat16 (all of one dtype).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssm.so")

SSM_ABI_VERSION = 8
CHECKPOINT_TOKENS = 16
MAX_CONV = 8
SSM_F32, SSM_BF16 = 0, 1
STATUS = {0: "SSM_OK", 1: "SSM_ERR_NULL", 2: "SSM_ERR_SHAPE", 3: "SSM_ERR_STRIDE",
          4: "SSM_ERR_DTYPE", 5: "SSM_ERR_ALIGN", 6: "SSM_ERR_ALIAS", 7: "SSM_ERR_UNSUPPORTED",
          8: "SSM_ERR_HIP", 9: "SSM_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


class ScanArgs(ctypes.Structure):
    """Mirror of ssm_scan_args."""
    _fields_ = [("batch", _I64), ("dim", _I64), ("seqlen", _I64), ("dstate", _I64),
                ("io_dtype", _I32), ("delta_softplus", _I32),
                ("u", _P), ("u_batch_stride", _I64), ("u_dim_stride", _I64),
                ("delta", _P), ("delta_batch_stride", _I64), ("delta_dim_stride", _I64),
                ("z", _P), ("z_batch_stride", _I64), ("z_dim_stride", _I64),
                ("B", _P), ("B_batch_stride", _I64), ("B_state_stride", _I64),
                ("C", _P), ("C_batch_stride", _I64), ("C_state_stride", _I64),
                ("A", _P), ("A_dim_stride", _I64), ("A_state_stride", _I64),
                ("D", _P), ("delta_bias", _P), ("h0", _P), ("last_state", _P),
                ("out", _P), ("out_batch_stride", _I64), ("out_dim_stride", _I64),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
                ("checkpoints", _P),
                ("conv_weight", _P), ("conv_bias", _P), ("conv_state_in", _P),
                ("conv_state_out", _P),
                ("conv_out", _P), ("conv_out_batch_stride", _I64), ("conv_out_dim_stride", _I64),
                ("d_conv", _I32), ("conv_silu", _I32),
                ("ngroups", _I64), ("B_group_stride", _I64), ("C_group_stride", _I64)]


class ScanBwdArgs(ctypes.Structure):
    """Mirror of ssm_scan_bwd_args."""
    _fields_ = [("batch", _I64), ("dim", _I64), ("seqlen", _I64), ("dstate", _I64),
                ("io_dtype", _I32), ("delta_softplus", _I32),
                ("u", _P), ("u_batch_stride", _I64), ("u_dim_stride", _I64),
                ("delta", _P), ("delta_batch_stride", _I64), ("delta_dim_stride", _I64),
                ("z", _P), ("z_batch_stride", _I64), ("z_dim_stride", _I64),
                ("B", _P), ("B_batch_stride", _I64), ("B_state_stride", _I64),
                ("C", _P), ("C_batch_stride", _I64), ("C_state_stride", _I64),
                ("A", _P), ("A_dim_stride", _I64), ("A_state_stride", _I64),
                ("D", _P), ("delta_bias", _P), ("h0", _P), ("checkpoints", _P),
                ("dout", _P), ("dout_batch_stride", _I64), ("dout_dim_stride", _I64),
                ("dlast", _P),
                ("du", _P), ("du_batch_stride", _I64), ("du_dim_stride", _I64),
                ("ddelta", _P), ("ddelta_batch_stride", _I64), ("ddelta_dim_stride", _I64),
                ("dz", _P), ("dz_batch_stride", _I64), ("dz_dim_stride", _I64),
                ("dB", _P), ("dC", _P), ("dA", _P), ("dD", _P), ("ddelta_bias", _P),
                ("dh0", _P),
                ("ngroups", _I64), ("B_group_stride", _I64), ("C_group_stride", _I64),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class UpdateArgs(ctypes.Structure):
    """Mirror of ssm_update_args."""
    _fields_ = [("batch", _I64), ("dim", _I64), ("dstate", _I64),
                ("io_dtype", _I32), ("dt_softplus", _I32),
                ("state", _P), ("state_batch_stride", _I64), ("state_dim_stride", _I64),
                ("x", _P), ("x_batch_stride", _I64),
                ("dt", _P), ("dt_batch_stride", _I64),
                ("z", _P), ("z_batch_stride", _I64),
                ("B", _P), ("B_batch_stride", _I64),
                ("C", _P), ("C_batch_stride", _I64),
                ("A", _P), ("A_dim_stride", _I64),
                ("D", _P), ("dt_bias", _P),
                ("out", _P), ("out_batch_stride", _I64),
                ("conv_state", _P), ("conv_weight", _P), ("conv_bias", _P),
                ("d_conv", _I32), ("conv_silu", _I32),
                ("ngroups", _I64), ("B_group_stride", _I64), ("C_group_stride", _I64)]


class SsdArgs(ctypes.Structure):
    """Mirror of ssm_ssd_args."""
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("nheads", _I64), ("headdim", _I64),
                ("ngroups", _I64), ("dstate", _I64),
                ("io_dtype", _I32), ("dt_softplus", _I32),
                ("x", _P), ("x_batch_stride", _I64), ("x_seq_stride", _I64), ("x_head_stride", _I64),
                ("dt", _P), ("dt_batch_stride", _I64), ("dt_seq_stride", _I64),
                ("z", _P), ("z_batch_stride", _I64), ("z_seq_stride", _I64), ("z_head_stride", _I64),
                ("B", _P), ("B_batch_stride", _I64), ("B_seq_stride", _I64), ("B_group_stride", _I64),
                ("C", _P), ("C_batch_stride", _I64), ("C_seq_stride", _I64), ("C_group_stride", _I64),
                ("A", _P), ("D", _P), ("dt_bias", _P), ("h0", _P), ("last_state", _P),
                ("out", _P), ("out_batch_stride", _I64), ("out_seq_stride", _I64),
                ("out_head_stride", _I64), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class SSMError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def lib():
    """The loaded libssm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libssm.so not found at {LIB_PATH}; build it with "
                              "`python -m selective_state_space_74_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        L.ssm_abi_version.restype = ctypes.c_int
        L.ssm_scan_args_size.restype = ctypes.c_size_t
        L.ssm_scan_bwd_args_size.restype = ctypes.c_size_t
        L.ssm_update_args_size.restype = ctypes.c_size_t
        L.ssm_ssd_args_size.restype = ctypes.c_size_t
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_status_string.argtypes = [ctypes.c_int]
        for name, T in (("ssm_validate_scan", ScanArgs), ("ssm_validate_update", UpdateArgs),
                        ("ssm_validate_scan_bwd", ScanBwdArgs), ("ssm_validate_ssd", SsdArgs)):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.POINTER(T)]
        L.ssm_scan_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_workspace_size.argtypes = [ctypes.POINTER(ScanArgs)]
        L.ssm_scan_bwd_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ScanBwdArgs)]
        L.ssm_ssd_workspace_size.restype = ctypes.c_size_t
        L.ssm_ssd_workspace_size.argtypes = [ctypes.POINTER(SsdArgs)]
        L.ssm_selective_scan_fwd.restype = ctypes.c_int
        L.ssm_selective_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), _P]
        L.ssm_selective_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_selective_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), _P]
        L.ssm_selective_scan_bwd.restype = ctypes.c_int
        L.ssm_selective_scan_bwd.argtypes = [ctypes.POINTER(ScanBwdArgs), _P]
        L.ssm_selective_state_update.restype = ctypes.c_int
        L.ssm_selective_state_update.argtypes = [ctypes.POINTER(UpdateArgs), _P]
        L.ssm_ssd_scan_fwd.restype = ctypes.c_int
        L.ssm_ssd_scan_fwd.argtypes = [ctypes.POINTER(SsdArgs), _P]
        if L.ssm_abi_version() != SSM_ABI_VERSION:
            raise ImportError(f"libssm.so ABI {L.ssm_abi_version()} != {SSM_ABI_VERSION}")
        if (L.ssm_scan_args_size() != ctypes.sizeof(ScanArgs)
                or L.ssm_scan_bwd_args_size() != ctypes.sizeof(ScanBwdArgs)
                or L.ssm_update_args_size() != ctypes.sizeof(UpdateArgs)
                or L.ssm_ssd_args_size() != ctypes.sizeof(SsdArgs)):
            raise ImportError("libssm.so argument struct layout differs from the binding")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ssm_status_string(int(status)).decode()


def validate_scan(args: ScanArgs) -> int:
    return lib().ssm_validate_scan(ctypes.byref(args))


def validate_scan_bwd(args: ScanBwdArgs) -> int:
    return lib().ssm_validate_scan_bwd(ctypes.byref(args))


def validate_update(args: UpdateArgs) -> int:
    return lib().ssm_validate_update(ctypes.byref(args))


def scan_workspace_size(args: ScanArgs) -> int:
    return lib().ssm_scan_workspace_size(ctypes.byref(args))


def scan_bwd_workspace_size(args: "ScanBwdArgs") -> int:
    return lib().ssm_scan_bwd_workspace_size(ctypes.byref(args))


def scan_fwd_raw(args: ScanArgs, stream: int = 0) -> int:
    return lib().ssm_selective_scan_fwd(ctypes.byref(args), _P(stream or None))


def scan_fwd_noalloc_raw(args: ScanArgs, stream: int = 0) -> int:
    return lib().ssm_selective_scan_fwd_noalloc(ctypes.byref(args), _P(stream or None))


def validate_ssd(args: SsdArgs) -> int:
    return lib().ssm_validate_ssd(ctypes.byref(args))


def ssd_workspace_size(args: SsdArgs) -> int:
    return lib().ssm_ssd_workspace_size(ctypes.byref(args))


def ssd_fwd_raw(args: SsdArgs, stream: int = 0) -> int:
    return lib().ssm_ssd_scan_fwd(ctypes.byref(args), ctypes.c_void_p(stream))


def scan_bwd_raw(args: ScanBwdArgs, stream: int = 0) -> int:
    return lib().ssm_selective_scan_bwd(ctypes.byref(args), _P(stream or None))


def checkpoint_shape(batch: int, dim: int, seqlen: int, dstate: int = 16):
    """Shape of the fp32 state checkpoints the forward writes for the backward."""
    return (batch, dim, (seqlen + CHECKPOINT_TOKENS - 1) // CHECKPOINT_TOKENS, dstate)


def state_update_raw(args: UpdateArgs, stream: int = 0) -> int:
    return lib().ssm_selective_state_update(ctypes.byref(args), _P(stream or None))


# ---------------------------------------------------------------------------
# torch-level wrappers

def _torch():
    import torch
    return torch


def _io_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"IO tensors must be float32 or bfloat16, got {t.dtype}")


def _check_dev(name, t, device, dtype=None):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _contig_f32(name, t, shape):
    if t is None:
        return None
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _bc_groups(B, C, batch, dim, N, tail):
    """B/C groups from the shape of B: (batch, N, *tail) is one group shared
    by every channel, (batch, G, N, *tail) is G groups of dim // G channels."""
    if tuple(B.shape) != tuple(C.shape):
        raise ValueError("B and C must have the same shape")
    if tuple(B.shape) == (batch, N) + tuple(tail):
        return 0
    if B.dim() == 3 + len(tail) and tuple(B.shape[2:]) == (N,) + tuple(tail) \
            and B.shape[0] == batch and B.shape[1] >= 1 and dim % B.shape[1] == 0:
        return int(B.shape[1])
    raise ValueError("B and C must be (batch, dstate%s) or (batch, ngroups, dstate%s) with "
                     "ngroups dividing dim" % ((", L",) * 2 if tail else ("", "")))


def _set_bc(a, B, C, G, time):
    """B/C pointers and strides into an argument block (0 groups: 3-D B/C)."""
    a.B, a.C, a.ngroups = _ptr(B), _ptr(C), G
    if time:
        if G:
            a.B_batch_stride, a.B_group_stride, a.B_state_stride = B.stride()[:3]
            a.C_batch_stride, a.C_group_stride, a.C_state_stride = C.stride()[:3]
        else:
            a.B_batch_stride, a.B_state_stride = B.stride()[:2]
            a.C_batch_stride, a.C_state_stride = C.stride()[:2]
    else:
        a.B_batch_stride, a.C_batch_stride = B.stride(0), C.stride(0)
        if G:
            a.B_group_stride, a.C_group_stride = B.stride(1), C.stride(1)


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                       h0=None, return_last_state=False, out=None, last_state=None, stream=None,
                       workspace=None, checkpoints=None, conv_weight=None, conv_bias=None,
                       conv_state_in=None, conv_state_out=None, conv_out=None, conv_silu=True,
                       noalloc=False):
    """Prefill selective scan on the GPU (see the module docstring).

    `workspace` (optional): a device tensor reused across calls; when None,
    one of the size the library asks for is allocated through torch; False
    passes no workspace (the scan then runs each sequence as one segment).
    `checkpoints` (optional): an fp32 tensor of checkpoint_shape(...) that
    receives the state entering every 16-token block, for the backward.
    Fused conv branch: with conv_weight (dim, d_conv) fp32, `u` is the conv
    input x and the SSM input is silu(conv_bias + causal depthwise conv of
    x) (no SiLU with conv_silu=False).  conv_state_in (batch, dim, d_conv)
    fp32 holds the inputs before the sequence; conv_state_out (same shape,
    filled with the last d_conv inputs) and conv_out (like u, the SSM
    input) are optional output tensors.
    `noalloc=True` calls ssm_selective_scan_fwd_noalloc, which keeps the
    segment aggregates in the library's static device scratch (no workspace
    is passed or allocated; pass `out` and `last_state` to allocate
    nothing at all)."""
    torch = _torch()
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    dev = u.device
    io = u.dtype
    code = _io_code(u)
    for name, t in (("delta", delta), ("z", z), ("B", B), ("C", C)):
        _check_dev(name, t, dev, io)
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("h0", h0),
                    ("last_state", last_state)):
        _check_dev(name, t, dev, torch.float32)
    if tuple(delta.shape) != (batch, dim, L) or (z is not None and tuple(z.shape) != (batch, dim, L)):
        raise ValueError("delta and z must match u's shape")
    G = _bc_groups(B, C, batch, dim, N, (L,))
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, dstate)")
    for name, t in (("u", u), ("delta", delta), ("z", z), ("B", B), ("C", C)):
        if t is not None and L > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have time stride 1")
    _contig_f32("D", D, (dim,))
    _contig_f32("delta_bias", delta_bias, (dim,))
    _contig_f32("h0", h0, (batch, dim, N))
    if out is None:
        out = torch.empty((batch, dim, L), dtype=io, device=dev)
    _check_dev("out", out, dev, io)
    if tuple(out.shape) != (batch, dim, L) or (L > 1 and out.stride(2) != 1):
        raise ValueError("out must be (batch, dim, L) with time stride 1")
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    if last_state is not None:
        _contig_f32("last_state", last_state, (batch, dim, N))
    a = ScanArgs()
    a.batch, a.dim, a.seqlen, a.dstate = batch, dim, L, N
    a.io_dtype, a.delta_softplus = code, int(bool(delta_softplus))
    a.u, (a.u_batch_stride, a.u_dim_stride) = _ptr(u), u.stride()[:2]
    a.delta, (a.delta_batch_stride, a.delta_dim_stride) = _ptr(delta), delta.stride()[:2]
    if z is not None:
        a.z, (a.z_batch_stride, a.z_dim_stride) = _ptr(z), z.stride()[:2]
    _set_bc(a, B, C, G, time=True)
    a.A, (a.A_dim_stride, a.A_state_stride) = _ptr(A), A.stride()
    a.D, a.delta_bias, a.h0 = _ptr(D), _ptr(delta_bias), _ptr(h0)
    a.last_state = _ptr(last_state)
    a.out, (a.out_batch_stride, a.out_dim_stride) = _ptr(out), out.stride()[:2]
    if checkpoints is not None:
        _contig_f32("checkpoints", checkpoints, checkpoint_shape(batch, dim, L, N))
        _check_dev("checkpoints", checkpoints, dev, torch.float32)
        a.checkpoints = _ptr(checkpoints)
    if conv_weight is not None:
        if conv_weight.dim() != 2 or conv_weight.shape[0] != dim:
            raise ValueError("conv_weight must be (dim, d_conv)")
        K = conv_weight.shape[1]
        _check_dev("conv_weight", conv_weight, dev, torch.float32)
        _contig_f32("conv_weight", conv_weight, (dim, K))
        for name, t, shp in (("conv_bias", conv_bias, (dim,)),
                             ("conv_state_in", conv_state_in, (batch, dim, K)),
                             ("conv_state_out", conv_state_out, (batch, dim, K))):
            _check_dev(name, t, dev, torch.float32)
            _contig_f32(name, t, shp)
        a.conv_weight, a.conv_bias = _ptr(conv_weight), _ptr(conv_bias)
        a.conv_state_in, a.conv_state_out = _ptr(conv_state_in), _ptr(conv_state_out)
        a.d_conv, a.conv_silu = K, int(bool(conv_silu))
        if conv_out is not None:
            _check_dev("conv_out", conv_out, dev, io)
            if tuple(conv_out.shape) != (batch, dim, L) or (L > 1 and conv_out.stride(2) != 1):
                raise ValueError("conv_out must be (batch, dim, L) with time stride 1")
            a.conv_out = _ptr(conv_out)
            a.conv_out_batch_stride, a.conv_out_dim_stride = conv_out.stride()[:2]
    if noalloc:
        st = scan_fwd_noalloc_raw(a, _stream(stream))
        if st != 0:
            raise SSMError(st, "ssm_selective_scan_fwd_noalloc")
        return (out, last_state) if return_last_state else out
    need = scan_workspace_size(a) if workspace is not False else 0
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check_dev("workspace", workspace, dev)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = scan_fwd_raw(a, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_selective_scan_fwd")
    return (out, last_state) if return_last_state else out


def selective_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
                           out=None, stream=None, conv_state=None, conv_weight=None,
                           conv_bias=None, conv_silu=True):
    """Single-token decode update on the GPU; `state` is updated in place.
    With conv_weight (dim, d_conv), x is the conv input and conv_state
    (batch, dim, d_conv) fp32 is shifted in place (the fused conv branch)."""
    torch = _torch()
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, dstate)")
    batch, dim, N = state.shape
    dev = state.device
    io = x.dtype
    code = _io_code(x)
    _check_dev("state", state, dev, torch.float32)
    for name, t in (("x", x), ("dt", dt), ("z", z), ("B", B), ("C", C)):
        _check_dev(name, t, dev, io)
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        _check_dev(name, t, dev, torch.float32)
    for name, t in (("x", x), ("dt", dt), ("z", z)):
        if t is not None and (tuple(t.shape) != (batch, dim) or (dim > 1 and t.stride(1) != 1)):
            raise ValueError(f"{name} must be (batch, dim) with dim stride 1")
    G = _bc_groups(B, C, batch, dim, N, ())
    for name, t in (("B", B), ("C", C)):
        if N > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have state stride 1")
    if tuple(A.shape) != (dim, N) or (N > 1 and A.stride(1) != 1):
        raise ValueError("A must be (dim, dstate) with state stride 1")
    if N > 1 and state.stride(2) != 1:
        raise ValueError("state must have state stride 1")
    _contig_f32("D", D, (dim,))
    _contig_f32("dt_bias", dt_bias, (dim,))
    if out is None:
        out = torch.empty((batch, dim), dtype=io, device=dev)
    _check_dev("out", out, dev, io)
    if tuple(out.shape) != (batch, dim) or (dim > 1 and out.stride(1) != 1):
        raise ValueError("out must be (batch, dim) with dim stride 1")
    a = UpdateArgs()
    a.batch, a.dim, a.dstate = batch, dim, N
    a.io_dtype, a.dt_softplus = code, int(bool(dt_softplus))
    a.state, (a.state_batch_stride, a.state_dim_stride) = _ptr(state), state.stride()[:2]
    a.x, a.x_batch_stride = _ptr(x), x.stride(0)
    a.dt, a.dt_batch_stride = _ptr(dt), dt.stride(0)
    if z is not None:
        a.z, a.z_batch_stride = _ptr(z), z.stride(0)
    _set_bc(a, B, C, G, time=False)
    a.A, a.A_dim_stride = _ptr(A), A.stride(0)
    a.D, a.dt_bias = _ptr(D), _ptr(dt_bias)
    a.out, a.out_batch_stride = _ptr(out), out.stride(0)
    if conv_weight is not None:
        if conv_weight.dim() != 2 or conv_weight.shape[0] != dim:
            raise ValueError("conv_weight must be (dim, d_conv)")
        K = conv_weight.shape[1]
        if conv_state is None:
            raise ValueError("conv_state is required with conv_weight")
        for name, t, shp in (("conv_weight", conv_weight, (dim, K)), ("conv_bias", conv_bias, (dim,)),
                             ("conv_state", conv_state, (batch, dim, K))):
            _check_dev(name, t, dev, torch.float32)
            _contig_f32(name, t, shp)
        a.conv_state, a.conv_weight, a.conv_bias = _ptr(conv_state), _ptr(conv_weight), _ptr(conv_bias)
        a.d_conv, a.conv_silu = K, int(bool(conv_silu))
    st = state_update_raw(a, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_selective_state_update")
    return out


# the backward's workspace is allocated automatically only up to this size
BWD_WORKSPACE_AUTO_MAX = 2 << 30


def selective_scan_bwd(dout, u, delta, A, B, C, checkpoints, D=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, dlast=None, stream=None, workspace=None):
    """Gradients of selective_scan_fwd for the upstream gradient dout on out
    (and dlast on last_state), from the checkpoints that forward wrote.
    Returns a dict: du, ddelta (IO dtype, shaped like u), dB, dC (fp32, like
    B), dA (fp32, like A) and, for the inputs that were given, dz, dD,
    ddelta_bias, dh0 (fp32).  The sums over channels (dB, dC) and batch rows
    (dA, dD, ddelta_bias) are formed from partials in a workspace, in fixed
    order (deterministic), or with device atomics without one (their last
    bits may then vary between runs).
    `workspace`: a device tensor reused across calls; None allocates one of
    the size the library asks for (up to BWD_WORKSPACE_AUTO_MAX bytes);
    False passes none (dB/dC then always by atomics)."""
    torch = _torch()
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    dev, io = u.device, u.dtype
    code = _io_code(u)
    for name, t in (("delta", delta), ("z", z), ("B", B), ("C", C), ("dout", dout)):
        _check_dev(name, t, dev, io)
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("h0", h0),
                    ("checkpoints", checkpoints), ("dlast", dlast)):
        _check_dev(name, t, dev, torch.float32)
    for name, t in (("delta", delta), ("z", z), ("dout", dout)):
        if t is not None and tuple(t.shape) != (batch, dim, L):
            raise ValueError(f"{name} must match u's shape")
    G = _bc_groups(B, C, batch, dim, N, (L,))
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, dstate)")
    for name, t in (("u", u), ("delta", delta), ("z", z), ("B", B), ("C", C), ("dout", dout)):
        if t is not None and L > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have time stride 1")
    _contig_f32("D", D, (dim,))
    _contig_f32("delta_bias", delta_bias, (dim,))
    _contig_f32("h0", h0, (batch, dim, N))
    _contig_f32("dlast", dlast, (batch, dim, N))
    _contig_f32("checkpoints", checkpoints, checkpoint_shape(batch, dim, L, N))
    g = dict(du=torch.empty((batch, dim, L), dtype=io, device=dev),
             ddelta=torch.empty((batch, dim, L), dtype=io, device=dev),
             dB=torch.empty(tuple(B.shape), dtype=torch.float32, device=dev),
             dC=torch.empty(tuple(C.shape), dtype=torch.float32, device=dev),
             dA=torch.empty((dim, N), dtype=torch.float32, device=dev))
    if z is not None:
        g["dz"] = torch.empty((batch, dim, L), dtype=io, device=dev)
    if D is not None:
        g["dD"] = torch.empty(dim, dtype=torch.float32, device=dev)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty(dim, dtype=torch.float32, device=dev)
    if h0 is not None:
        g["dh0"] = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    a = ScanBwdArgs()
    a.batch, a.dim, a.seqlen, a.dstate = batch, dim, L, N
    a.io_dtype, a.delta_softplus = code, int(bool(delta_softplus))
    a.u, (a.u_batch_stride, a.u_dim_stride) = _ptr(u), u.stride()[:2]
    a.delta, (a.delta_batch_stride, a.delta_dim_stride) = _ptr(delta), delta.stride()[:2]
    if z is not None:
        a.z, (a.z_batch_stride, a.z_dim_stride) = _ptr(z), z.stride()[:2]
        a.dz, (a.dz_batch_stride, a.dz_dim_stride) = _ptr(g["dz"]), g["dz"].stride()[:2]
    _set_bc(a, B, C, G, time=True)
    a.A, (a.A_dim_stride, a.A_state_stride) = _ptr(A), A.stride()
    a.D, a.delta_bias, a.h0 = _ptr(D), _ptr(delta_bias), _ptr(h0)
    a.checkpoints, a.dlast = _ptr(checkpoints), _ptr(dlast)
    a.dout, (a.dout_batch_stride, a.dout_dim_stride) = _ptr(dout), dout.stride()[:2]
    a.du, (a.du_batch_stride, a.du_dim_stride) = _ptr(g["du"]), g["du"].stride()[:2]
    a.ddelta, (a.ddelta_batch_stride, a.ddelta_dim_stride) = _ptr(g["ddelta"]), g["ddelta"].stride()[:2]
    a.dB, a.dC, a.dA = _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dA"])
    a.dD, a.ddelta_bias, a.dh0 = _ptr(g.get("dD")), _ptr(g.get("ddelta_bias")), _ptr(g.get("dh0"))
    need = scan_bwd_workspace_size(a) if workspace is not False else 0
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = (torch.empty(need, dtype=torch.uint8, device=dev)
                         if need <= BWD_WORKSPACE_AUTO_MAX else None)
        if workspace is not None:
            _check_dev("workspace", workspace, dev)
            a.workspace = _ptr(workspace)
            a.workspace_bytes = workspace.numel() * workspace.element_size()
    st = scan_bwd_raw(a, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_selective_scan_bwd")
    return g


def ssd_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
                 return_last_state=False, out=None, last_state=None, stream=None, workspace=None):
    """Mamba-2 SSM (SSD layer) prefill on the GPU.

    x, z: (batch, L, nheads, headdim) with headdim stride 1; dt: (batch, L,
    nheads) with head stride 1 (IO dtype); B, C: (batch, L, ngroups, dstate)
    with state stride 1; A, D, dt_bias: (nheads,) fp32; h0: (batch, nheads,
    headdim, dstate) fp32.  Returns out (like x) or (out, last_state).
    `workspace`: as for selective_scan_fwd (None allocates what the library
    asks for, False passes none: each sequence then runs as one segment)."""
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be (batch, L, nheads, headdim)")
    batch, L, H, P = x.shape
    dev, io = x.device, x.dtype
    code = _io_code(x)
    for name, t in (("dt", dt), ("z", z), ("B", B), ("C", C)):
        _check_dev(name, t, dev, io)
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias), ("h0", h0),
                    ("last_state", last_state)):
        _check_dev(name, t, dev, torch.float32)
    if B.dim() != 4 or tuple(B.shape) != tuple(C.shape) or tuple(B.shape[:2]) != (batch, L):
        raise ValueError("B and C must be (batch, L, ngroups, dstate)")
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (batch, L, H) or (z is not None and tuple(z.shape) != tuple(x.shape)):
        raise ValueError("dt must be (batch, L, nheads) and z shaped like x")
    for name, t in (("x", x), ("z", z), ("dt", dt), ("B", B), ("C", C)):
        if t is not None and t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have a unit innermost stride")
    _contig_f32("A", A, (H,))
    _contig_f32("D", D, (H,))
    _contig_f32("dt_bias", dt_bias, (H,))
    _contig_f32("h0", h0, (batch, H, P, N))
    if out is None:
        out = torch.empty_like(x)
    _check_dev("out", out, dev, io)
    if tuple(out.shape) != tuple(x.shape) or (P > 1 and out.stride(-1) != 1):
        raise ValueError("out must be shaped like x with headdim stride 1")
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    if last_state is not None:
        _contig_f32("last_state", last_state, (batch, H, P, N))
    a = SsdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.ngroups, a.dstate = batch, L, H, P, G, N
    a.io_dtype, a.dt_softplus = code, int(bool(dt_softplus))
    a.x, (a.x_batch_stride, a.x_seq_stride, a.x_head_stride) = _ptr(x), x.stride()[:3]
    a.dt, (a.dt_batch_stride, a.dt_seq_stride) = _ptr(dt), dt.stride()[:2]
    if z is not None:
        a.z, (a.z_batch_stride, a.z_seq_stride, a.z_head_stride) = _ptr(z), z.stride()[:3]
    a.B, (a.B_batch_stride, a.B_seq_stride, a.B_group_stride) = _ptr(B), B.stride()[:3]
    a.C, (a.C_batch_stride, a.C_seq_stride, a.C_group_stride) = _ptr(C), C.stride()[:3]
    a.A, a.D, a.dt_bias, a.h0 = _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(h0)
    a.last_state = _ptr(last_state)
    a.out, (a.out_batch_stride, a.out_seq_stride, a.out_head_stride) = _ptr(out), out.stride()[:3]
    need = ssd_workspace_size(a) if workspace is not False else 0
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check_dev("workspace", workspace, dev)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = ssd_fwd_raw(a, _stream(stream))
    if st != 0:
        raise SSMError(st, "ssm_ssd_scan_fwd")
    return (out, last_state) if return_last_state else out


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True):
    """selective_scan_fwd as a differentiable torch op: the forward keeps the
    state checkpoints and the backward runs ssm_selective_scan_bwd on them.
    Gradients flow to u, delta, A, B, C and, when given, D, z and delta_bias
    (d_state 1..64; B/C shared or in groups that keep 16-channel blocks whole)."""
    torch = _torch()

    class _Scan(torch.autograd.Function):
        @staticmethod
        def forward(ctx, u, delta, A, B, C, D, z, delta_bias):
            batch, dim, L = u.shape
            ck = torch.empty(checkpoint_shape(batch, dim, L, A.shape[1]), dtype=torch.float32,
                             device=u.device)
            out = selective_scan_fwd(u, delta, A, B, C, D=D, z=z, delta_bias=delta_bias,
                                     delta_softplus=delta_softplus, checkpoints=ck)
            ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, ck)
            return out

        @staticmethod
        def backward(ctx, dout):
            u, delta, A, B, C, D, z, delta_bias, ck = ctx.saved_tensors
            g = selective_scan_bwd(dout.contiguous(), u, delta, A, B, C, ck, D=D, z=z,
                                   delta_bias=delta_bias, delta_softplus=delta_softplus)
            return (g["du"], g["ddelta"], g["dA"], g["dB"].to(B.dtype), g["dC"].to(C.dtype),
                    g.get("dD"), g.get("dz"), g.get("ddelta_bias"))

    return _Scan.apply(u, delta, A, B, C, D, z, delta_bias)
