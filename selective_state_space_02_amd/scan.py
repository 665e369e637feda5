"""ctypes binding of libssm_scan.so (include/ssm_scan.h).

Argument marshalling only: every step of the scan runs in the HIP kernels of the
library.  PyTorch allocates and owns device memory (inputs, outputs, workspace)
and supplies the stream.  There is no fallback: if the library is missing the
call raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssm_scan.so")

SSM_LAYOUT_BDL = 0
SSM_LAYOUT_BLHP = 1
SSM_F32 = 0
SSM_BF16 = 1
SSM_DISC_DELTA_B = 0
SSM_DISC_ZOH = 1
DISCRETIZATIONS = {"delta_b": SSM_DISC_DELTA_B, "zoh": SSM_DISC_ZOH}

SSM_OK = 0
SSM_ERR_NULL_ARG = -1
SSM_ERR_BAD_DIMS = -2
SSM_ERR_UNSUPPORTED = -3
SSM_ERR_ALIGN = -4
SSM_ERR_ALIAS = -5
SSM_ERR_WORKSPACE = -6
SSM_ERR_HIP = -7
SSM_ERR_SCRATCH = -8

EXPORTED = ("ssm_scan_fwd", "ssm_scan_workspace_size", "ssm_strerror", "ssm_scan_describe", "ssm_scan_version",
            "ssm_state_update", "ssm_conv_scan_fwd", "ssm_scan_fwd_noalloc", "ssm_scan_scratch_capacity")


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("ngroups", ctypes.c_int64),
        ("layout", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("discretization", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class Conv(ctypes.Structure):
    _fields_ = [
        ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("state_in", ctypes.c_void_p),
        ("state_out", ctypes.c_void_p),
        ("width", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Open libssm_scan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m selective_state_space_02_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp = ctypes.c_void_p
        lib.ssm_scan_fwd.restype = ctypes.c_int
        lib.ssm_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                     ctypes.POINTER(Dims), vp]
        lib.ssm_scan_workspace_size.restype = ctypes.c_size_t
        lib.ssm_scan_workspace_size.argtypes = [ctypes.POINTER(Dims)]
        lib.ssm_strerror.restype = ctypes.c_char_p
        lib.ssm_strerror.argtypes = [ctypes.c_int]
        lib.ssm_scan_describe.restype = ctypes.c_int
        lib.ssm_scan_describe.argtypes = [ctypes.POINTER(Dims), ctypes.c_char_p, ctypes.c_size_t]
        lib.ssm_scan_version.restype = ctypes.c_int
        lib.ssm_scan_version.argtypes = []
        lib.ssm_conv_scan_fwd.restype = ctypes.c_int
        lib.ssm_conv_scan_fwd.argtypes = [vp, ctypes.POINTER(Conv), vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                          vp, vp, ctypes.POINTER(Dims), vp]
        lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
        lib.ssm_scan_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                             ctypes.POINTER(Dims), vp]
        lib.ssm_scan_scratch_capacity.restype = ctypes.c_size_t
        lib.ssm_scan_scratch_capacity.argtypes = []
        lib.ssm_state_update.restype = ctypes.c_int
        lib.ssm_state_update.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                         ctypes.POINTER(Dims), vp]
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().ssm_strerror(int(code)).decode()


def make_dims(layout: str, io_dtype: str, batch: int, seqlen: int, dim: int, dstate: int,
              nheads: int = 0, headdim: int = 0, ngroups: int = 1, discretization: str = "delta_b") -> Dims:
    return Dims(batch, seqlen, dim, dstate, nheads, headdim, ngroups,
                SSM_LAYOUT_BDL if layout == "bdl" else SSM_LAYOUT_BLHP,
                SSM_BF16 if io_dtype == "bf16" else SSM_F32, None, 0, DISCRETIZATIONS[discretization], 0)


def workspace_size(dims: Dims) -> int:
    return int(load_library().ssm_scan_workspace_size(ctypes.byref(dims)))


def describe(dims: Dims) -> str:
    buf = ctypes.create_string_buffer(256)
    rc = load_library().ssm_scan_describe(ctypes.byref(dims), buf, 256)
    if rc != SSM_OK:
        raise ValueError(strerror(rc))
    return buf.value.decode()


def call_raw(u, delta, A, B, C, D, z, delta_bias, softplus, h0, y, h_last, dims: Dims, stream=None) -> int:
    """Direct ABI call with integer addresses (None = NULL).  Returns the status code."""
    return int(load_library().ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, int(bool(softplus)), h0, y,
                                          h_last, ctypes.byref(dims), stream))


def call_noalloc_raw(u, delta, A, B, C, D, z, delta_bias, softplus, h0, y, h_last, dims: Dims, stream=None) -> int:
    """Direct ABI call of ssm_scan_fwd_noalloc (the library's static device scratch, no
    allocation) with integer addresses (None = NULL).  Returns the status code."""
    return int(load_library().ssm_scan_fwd_noalloc(u, delta, A, B, C, D, z, delta_bias, int(bool(softplus)), h0, y,
                                                  h_last, ctypes.byref(dims), stream))


def scratch_capacity() -> int:
    """Bytes of the static device scratch ssm_scan_fwd_noalloc uses on each GPU."""
    return int(load_library().ssm_scan_scratch_capacity())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(t: Optional[torch.Tensor], name: str, dtype, shape, device):
    if t is None:
        return
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_stream(fn):
    """With stream= given, allocate the outputs and the internal workspace under that stream, so
    torch's caching allocator reuses their memory only in that stream's order."""
    @functools.wraps(fn)
    def run(*args, stream: Optional[torch.cuda.Stream] = None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return run


@_on_stream
def ssm_scan_fwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                 D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 delta_bias: Optional[torch.Tensor] = None, softplus: bool = True,
                 h0: Optional[torch.Tensor] = None, *, layout: str = "bdl", ngroups: int = 1,
                 y: Optional[torch.Tensor] = None, h_last: Optional[torch.Tensor] = None,
                 want_h_last: bool = True, workspace: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None,
                 discretization: str = "delta_b") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Selective scan on the GPU.  Shapes as in include/ssm_scan.h; returns (y, h_last).
    discretization: "delta_b" (B̄ = Δ·B) or "zoh" (exact zero-order hold)."""
    lib = load_library()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("ssm_scan_fwd runs on the GPU: tensors must be on a cuda device")
    io = u.dtype
    if io not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    if layout == "bdl":
        Bsz, Dm, L = u.shape
        G, N = B.shape[1], B.shape[2]
        H, P = 0, 0
        shapes = dict(delta=(Bsz, Dm, L), A=(Dm, N), B=(Bsz, G, N, L), bias=(Dm,), x=(Bsz, Dm, L))
    elif layout == "blhp":
        Bsz, L, H, P = u.shape
        Dm = H * P
        G, N = B.shape[2], B.shape[3]
        shapes = dict(delta=(Bsz, L, H), A=(H,), B=(Bsz, L, G, N), bias=(H,), x=(Bsz, L, H, P))
    else:
        raise ValueError(layout)
    if G != ngroups:
        ngroups = G
    f32 = torch.float32
    _check(delta, "delta", io, shapes["delta"], dev)
    _check(A, "A", f32, shapes["A"], dev)
    _check(B, "B", io, shapes["B"], dev)
    _check(C, "C", io, shapes["B"], dev)
    _check(D, "D", f32, (Dm,), dev)
    _check(z, "z", io, shapes["x"], dev)
    _check(delta_bias, "delta_bias", f32, shapes["bias"], dev)
    _check(h0, "h0", f32, (Bsz, Dm, N), dev)
    if y is None:
        y = torch.empty(shapes["x"], dtype=io, device=dev)
    _check(y, "y", io, shapes["x"], dev)
    if h_last is None and want_h_last:
        h_last = torch.empty((Bsz, Dm, N), dtype=f32, device=dev)
    _check(h_last, "h_last", f32, (Bsz, Dm, N), dev)
    dims = make_dims(layout, "bf16" if io == torch.bfloat16 else "f32", Bsz, L, Dm, N, H, P, ngroups, discretization)
    need = int(lib.ssm_scan_workspace_size(ctypes.byref(dims)))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        dims.workspace = workspace.data_ptr()
        dims.workspace_bytes = workspace.numel() * workspace.element_size()
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = lib.ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                          int(bool(softplus)), _ptr(h0), _ptr(y), _ptr(h_last), ctypes.byref(dims),
                          ctypes.c_void_p(st.cuda_stream))
    if rc != SSM_OK:
        raise RuntimeError(f"ssm_scan_fwd failed ({rc}): {strerror(rc)}")
    return y, h_last


def ssm_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, h0=None, **kw):
    """Convenience wrapper: returns (y, h_last)."""
    return ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, softplus, h0, **kw)


def call_update_raw(x, delta, A, B, C, D, z, delta_bias, softplus, h_in, h_out, y, dims: Dims, stream=None) -> int:
    """Direct ABI call of ssm_state_update with integer addresses (None = NULL).  Returns the status code."""
    return int(load_library().ssm_state_update(x, delta, A, B, C, D, z, delta_bias, int(bool(softplus)), h_in, h_out,
                                              y, ctypes.byref(dims), stream))


@_on_stream
def ssm_state_update(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                     D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                     delta_bias: Optional[torch.Tensor] = None, softplus: bool = True,
                     h_in: Optional[torch.Tensor] = None, *, layout: str = "bdl",
                     h_out: Optional[torch.Tensor] = None, inplace: bool = False, y: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None,
                     discretization: str = "delta_b") -> Tuple[torch.Tensor, torch.Tensor]:
    """One decode step on the GPU.  BDL: x, delta (B, D); BLHP: x (B, H, P), delta (B, H); B, C (B, G, N);
    state (B, D, N) float32.  Returns (y, new state); with inplace=True the new state overwrites h_in."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssm_state_update runs on the GPU: tensors must be on a cuda device")
    io = x.dtype
    if io not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    if layout == "bdl":
        Bsz, Dm = x.shape
        H, P = 0, 0
        shapes = dict(delta=(Bsz, Dm), A=(Dm, B.shape[2]), bias=(Dm,))
    elif layout == "blhp":
        Bsz, H, P = x.shape
        Dm = H * P
        shapes = dict(delta=(Bsz, H), A=(H,), bias=(H,))
    else:
        raise ValueError(layout)
    G, N = B.shape[1], B.shape[2]
    f32 = torch.float32
    _check(delta, "delta", io, shapes["delta"], dev)
    _check(A, "A", f32, shapes["A"], dev)
    _check(B, "B", io, (Bsz, G, N), dev)
    _check(C, "C", io, (Bsz, G, N), dev)
    _check(D, "D", f32, (Dm,), dev)
    _check(z, "z", io, tuple(x.shape), dev)
    _check(delta_bias, "delta_bias", f32, shapes["bias"], dev)
    _check(h_in, "h_in", f32, (Bsz, Dm, N), dev)
    if inplace:
        if h_in is None:
            raise ValueError("inplace=True needs h_in")
        h_out = h_in
    elif h_out is None:
        h_out = torch.empty((Bsz, Dm, N), dtype=f32, device=dev)
    _check(h_out, "h_out", f32, (Bsz, Dm, N), dev)
    if y is None:
        y = torch.empty(tuple(x.shape), dtype=io, device=dev)
    _check(y, "y", io, tuple(x.shape), dev)
    dims = make_dims(layout, "bf16" if io == torch.bfloat16 else "f32", Bsz, 1, Dm, N, H, P, G, discretization)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = lib.ssm_state_update(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                              int(bool(softplus)), _ptr(h_in), _ptr(h_out), _ptr(y), ctypes.byref(dims),
                              ctypes.c_void_p(st.cuda_stream))
    if rc != SSM_OK:
        raise RuntimeError(f"ssm_state_update failed ({rc}): {strerror(rc)}")
    return y, h_out


def call_conv_raw(x, conv: Conv, delta, A, B, C, D, z, delta_bias, softplus, h0, y, h_last, dims: Dims,
                  stream=None) -> int:
    """Direct ABI call of ssm_conv_scan_fwd with integer addresses (None = NULL)."""
    return int(load_library().ssm_conv_scan_fwd(x, None if conv is None else ctypes.byref(conv), delta, A, B, C, D,
                                               z, delta_bias, int(bool(softplus)), h0, y, h_last, ctypes.byref(dims),
                                               stream))


@_on_stream
def ssm_conv_scan_fwd(x: torch.Tensor, conv_weight: torch.Tensor, conv_bias: Optional[torch.Tensor],
                      delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                      D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                      delta_bias: Optional[torch.Tensor] = None, softplus: bool = True,
                      h0: Optional[torch.Tensor] = None, *, conv_state_in: Optional[torch.Tensor] = None,
                      want_conv_state: bool = False, discretization: str = "delta_b", layout: str = "bdl",
                      stream: Optional[torch.cuda.Stream] = None):
    """Causal depthwise conv1d + SiLU on x along time, then the scan.  layout "bdl": x (B, D, L);
    "blhp": x (B, L, H, P), channel d = h*P + p.  conv_weight (D, K) float32, K in 1..4.
    Returns (y, h_last, conv_state_out or None)."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssm_conv_scan_fwd runs on the GPU: tensors must be on a cuda device")
    f32 = torch.float32
    io = x.dtype
    if layout == "bdl":
        Bsz, Dm, L = x.shape
        G, N = B.shape[1], B.shape[2]
        H, P = 0, 0
        shapes = dict(delta=(Bsz, Dm, L), A=(Dm, N), B=(Bsz, G, N, L), bias=(Dm,))
    elif layout == "blhp":
        Bsz, L, H, P = x.shape
        Dm = H * P
        G, N = B.shape[2], B.shape[3]
        shapes = dict(delta=(Bsz, L, H), A=(H,), B=(Bsz, L, G, N), bias=(H,))
    else:
        raise ValueError(layout)
    K = conv_weight.shape[1]
    _check(conv_weight, "conv_weight", f32, (Dm, K), dev)
    _check(conv_bias, "conv_bias", f32, (Dm,), dev)
    _check(conv_state_in, "conv_state_in", f32, (Bsz, Dm, K - 1), dev)
    for t, name, dt, shp in ((delta, "delta", io, shapes["delta"]), (A, "A", f32, shapes["A"]),
                             (B, "B", io, shapes["B"]), (C, "C", io, shapes["B"]), (D, "D", f32, (Dm,)),
                             (z, "z", io, tuple(x.shape)), (delta_bias, "delta_bias", f32, shapes["bias"]),
                             (h0, "h0", f32, (Bsz, Dm, N))):
        _check(t, name, dt, shp, dev)
    y = torch.empty_like(x)
    h_last = torch.empty((Bsz, Dm, N), dtype=f32, device=dev)
    state_out = torch.empty((Bsz, Dm, max(K - 1, 1)), dtype=f32, device=dev) if want_conv_state else None
    dims = make_dims(layout, "bf16" if io == torch.bfloat16 else "f32", Bsz, L, Dm, N, H, P, G, discretization)
    need = int(lib.ssm_scan_workspace_size(ctypes.byref(dims)))
    ws = None
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        dims.workspace = ws.data_ptr()
        dims.workspace_bytes = need
    conv = Conv(conv_weight.data_ptr(), _ptr(conv_bias), _ptr(conv_state_in),
                None if state_out is None else state_out.data_ptr(), K, 0)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = lib.ssm_conv_scan_fwd(_ptr(x), ctypes.byref(conv), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(z), _ptr(delta_bias), int(bool(softplus)), _ptr(h0), _ptr(y), _ptr(h_last),
                               ctypes.byref(dims), ctypes.c_void_p(st.cuda_stream))
    if rc != SSM_OK:
        raise RuntimeError(f"ssm_conv_scan_fwd failed ({rc}): {strerror(rc)}")
    if state_out is not None and K == 1:
        state_out = state_out[:, :, :0]
    return y, h_last, state_out
