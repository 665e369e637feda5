"""ctypes wrapper around the C oracle plus an independent numpy twin.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Array conventions (all host, C-contiguous):
  layout "bdl"  (Mamba-1): u, delta, z, y: (B, D, L); B, C: (B, G, N, L);
                A: (D, N); delta_bias: (D,); D: (D,); h0, h_last: (B, D, N)
  layout "blhp" (multi-head): u, z, y: (B, L, H, P); delta: (B, L, H);
                B, C: (B, L, G, N); A: (H,); delta_bias: (H,); D: (H*P,);
                h0, h_last: (B, H*P, N)
Floating inputs are either float32 arrays or bfloat16 bit patterns carried in
uint16 arrays (``io_dtype="bf16"``); the oracle upcasts the stored values to
float64, so it sees exactly what the GPU sees.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

LAYOUT_BDL = 0
LAYOUT_BLHP = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")


def lib_path() -> str:
    return _LIB


def default_threads() -> int:
    """Host threads for the oracle: the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build(verbose: bool = False) -> str:
    """Compile ssm_oracle.c with gcc (plain -O2, IEEE fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Dims(ctypes.Structure):
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
        ("discretization", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        lib.oracle_scan_f64.restype = ctypes.c_int
        lib.oracle_scan_f64.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                        ctypes.POINTER(_Dims), vp, ctypes.c_int64, vp, vp, ctypes.c_int]
        lib.oracle_conv_scan_f64.restype = ctypes.c_int
        lib.oracle_conv_scan_f64.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.c_int, vp, ctypes.POINTER(_Dims), vp, ctypes.c_int64, vp, vp,
                                             ctypes.c_int]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        _lib = lib
    return _lib


def softplus_f64(r: float) -> float:
    return _load().oracle_softplus(float(r))


def silu_f64(z: float) -> float:
    return _load().oracle_silu(float(z))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _io(a, io_dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    want = np.uint16 if io_dtype == 1 else np.float32
    if a.dtype != want:
        raise TypeError(f"expected {want} storage, got {a.dtype}")
    return a


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def scan_f64(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, h0=None, *,
             layout="bdl", io_dtype="f32", ngroups=1, nheads=None, headdim=None,
             t_out=None, nthreads=None, want_h_last=True, discretization="euler",
             conv_w=None, conv_b=None, conv_state_in=None, want_conv_state=False):
    """Run the C oracle.  Returns (y float64, h_last float64 or None), plus the final
    convolution state when want_conv_state.

    discretization: "euler" (B̄ = Δ·B) or "zoh" (exact zero-order hold, B̄ = expm1(ΔA)/A·B).
    conv_w (D, K) [, conv_b (D,), conv_state_in (B, D, K-1)]: u is the raw input of a causal
    depthwise convolution along time followed by SiLU, per channel d (d = h*P + p in the
    multi-head layout).
    """
    lay = LAYOUT_BDL if layout == "bdl" else LAYOUT_BLHP
    iod = 1 if io_dtype == "bf16" else 0
    u, delta, B, C, z = (_io(x, iod) for x in (u, delta, B, C, z))
    A, D, delta_bias, h0 = (_f32(x) for x in (A, D, delta_bias, h0))
    if lay == LAYOUT_BDL:
        Bsz, Dm, L = u.shape
        N = B.shape[2]
        H, P = Dm, 1
    else:
        Bsz, L, H, P = u.shape
        Dm = H * P
        N = B.shape[3]
    if discretization not in ("euler", "zoh"):
        raise ValueError(discretization)
    dims = _Dims(Bsz, L, Dm, N, H if lay else 0, P if lay else 0, ngroups, lay, iod,
                 1 if discretization == "zoh" else 0, 0)
    if t_out is not None:
        t_out = np.ascontiguousarray(np.asarray(t_out, dtype=np.int64))
        T = len(t_out)
    else:
        T = L
    y = np.empty((Bsz, Dm, T) if lay == LAYOUT_BDL else (Bsz, T, H, P), dtype=np.float64)
    h_last = np.empty((Bsz, Dm, N), dtype=np.float64) if want_h_last else None
    if nthreads is None:
        nthreads = default_threads()
    K = 0
    conv_out = None
    if conv_w is not None:
        conv_w = _f32(conv_w)
        K = conv_w.shape[1]
        conv_b, conv_state_in = _f32(conv_b), _f32(conv_state_in)
        conv_out = np.zeros((Bsz, Dm, max(K - 1, 0)), dtype=np.float64)
    rc = _load().oracle_conv_scan_f64(_ptr(u), _ptr(conv_w), _ptr(conv_b), int(K), _ptr(conv_state_in),
                                      _ptr(conv_out), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(delta_bias), int(bool(softplus)), _ptr(h0), ctypes.byref(dims),
                                      _ptr(t_out), ctypes.c_int64(0 if t_out is None else T), _ptr(y),
                                      _ptr(h_last), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_scan_f64 rejected its arguments")
    if want_conv_state:
        return y, h_last, conv_out
    return y, h_last


# ----------------------------------------------------------------------------
# Independent numpy twin (vectorised over rows, python loop over time).
# ----------------------------------------------------------------------------

def _to_f64(a, io_dtype):
    if a is None:
        return None
    a = np.asarray(a)
    if io_dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def scan_numpy_f64(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, h0=None, *,
                   layout="bdl", io_dtype="f32", ngroups=1, discretization="euler", conv_w=None, conv_b=None,
                   conv_state_in=None):
    """Same recurrence as scan_f64, written with numpy on (rows, N) arrays.

    Intended for small inputs (it loops over time in Python).
    """
    u, delta, B, C, z = (_to_f64(x, io_dtype) for x in (u, delta, B, C, z))
    if conv_w is not None:                                            # causal depthwise conv + SiLU on u
        w = np.asarray(conv_w, np.float64)                            # (D, K)
        K = w.shape[1]
        if layout == "bdl":
            xs = u                                                    # (B, D, L)
        else:                                                         # (B, L, H, P) -> (B, D, L), d = h*P + p
            xs = u.reshape(u.shape[0], u.shape[1], -1).transpose(0, 2, 1)
        Bsz_, Dm_, L_ = xs.shape
        left = np.zeros((Bsz_, Dm_, K - 1)) if conv_state_in is None else np.asarray(conv_state_in, np.float64)
        xp = np.concatenate([left, xs], axis=2)                       # (B, D, K-1+L)
        c = np.zeros_like(xs) + (0.0 if conv_b is None else np.asarray(conv_b, np.float64)[None, :, None])
        for k in range(K):
            c = c + w[None, :, k:k + 1] * xp[:, :, k:k + L_]
        xs = c / (1.0 + np.exp(-c))
        u = xs if layout == "bdl" else np.ascontiguousarray(xs.transpose(0, 2, 1)).reshape(u.shape)
    A = np.asarray(A, np.float64)
    if layout == "bdl":
        Bsz, Dm, L = u.shape
        N = B.shape[2]
        G = ngroups
        g_of_d = np.arange(Dm) // (Dm // G)
        x_t = lambda t: u[:, :, t]                                   # (B, D)
        r_t = lambda t: delta[:, :, t] + (0.0 if delta_bias is None else np.asarray(delta_bias, np.float64)[None, :])
        B_t = lambda t: B[:, :, :, t][:, g_of_d, :]                  # (B, D, N)
        C_t = lambda t: C[:, :, :, t][:, g_of_d, :]
        A_dn = A[None, :, :]                                         # (1, D, N)
        z_t = (lambda t: z[:, :, t]) if z is not None else None
        y = np.empty((Bsz, Dm, L))
        put = lambda t, v: y.__setitem__((slice(None), slice(None), t), v)
    else:
        Bsz, L, H, P = u.shape
        Dm = H * P
        N = B.shape[3]
        G = ngroups
        head_of_d = np.arange(Dm) // P
        g_of_d = head_of_d // (H // G)
        x_t = lambda t: u[:, t].reshape(Bsz, Dm)
        bias_h = 0.0 if delta_bias is None else np.asarray(delta_bias, np.float64)
        r_t = lambda t: (delta[:, t, :] + bias_h)[:, head_of_d]
        B_t = lambda t: B[:, t][:, g_of_d, :]
        C_t = lambda t: C[:, t][:, g_of_d, :]
        A_dn = np.repeat(A[head_of_d][:, None], N, axis=1)[None]
        z_t = (lambda t: z[:, t].reshape(Bsz, Dm)) if z is not None else None
        y = np.empty((Bsz, L, H, P))
        put = lambda t, v: y.__setitem__((slice(None), t), v.reshape(Bsz, H, P))
    Dv = np.zeros(Dm) if D is None else np.asarray(D, np.float64)
    h = np.zeros((Bsz, Dm, N)) if h0 is None else np.asarray(h0, np.float64).copy()
    for t in range(L):
        r = r_t(t)
        dt = np.logaddexp(0.0, r) if softplus else r                  # log(1 + e^r)
        x = x_t(t)
        if discretization == "zoh":                                   # expm1(ΔA)/A, Δ where A = 0
            with np.errstate(divide="ignore", invalid="ignore"):
                bbar = np.where(A_dn != 0.0, np.expm1(dt[..., None] * A_dn) / A_dn, dt[..., None])
        else:
            bbar = dt[..., None]
        h = np.exp(dt[..., None] * A_dn) * h + (bbar * x[..., None]) * B_t(t)
        yt = np.einsum("bdn,bdn->bd", C_t(t), h) + Dv[None, :] * x
        if z_t is not None:
            zz = z_t(t)
            yt = yt * (zz / (1.0 + np.exp(-zz)))
        put(t, yt)
    return y, h
