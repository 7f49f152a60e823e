"""ctypes wrapper around the fp64 oracle (``ssm_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Arguments are numpy
arrays in the layouts of the C functions; everything is widened to float64
(exactly: fp32 and bf16 values are representable in fp64) before the call.
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


def lib_path() -> str:
    return _LIB


def build() -> str:
    """Compile ``ssm_oracle.c`` into ``liboracle.so`` with gcc (plain IEEE
    double arithmetic: no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    """Load liboracle.so (building it if absent).  SSM_ORACLE_LIB names
    another build of the same source to load instead (the sanitizer build
    of the CPU tests)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SSM_ORACLE_LIB") or _LIB
    if path == _LIB and not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.oracle_scan_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                    dp, dp, dp, L, L, L, L, ctypes.c_int]
    lib.oracle_scan_fwd.restype = ctypes.c_int
    lib.oracle_state_update.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int,
                                        ctypes.c_int, dp, L, L, L]
    lib.oracle_state_update.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                    dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, L, L, L, L,
                                    ctypes.c_int]
    lib.oracle_scan_bwd.restype = ctypes.c_int
    lib.oracle_causal_conv1d_silu.argtypes = [dp, dp, dp, L, dp, dp, dp, L, L, L]
    lib.oracle_causal_conv1d_silu.restype = ctypes.c_int
    lib.oracle_conv_step.argtypes = [dp, dp, dp, dp, L, dp, L, L]
    lib.oracle_conv_step.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _zoh(bbar):
    if bbar not in ("euler", "zoh"):
        raise ValueError(f"bbar must be 'euler' or 'zoh', not {bbar!r}")
    return int(bbar == "zoh")


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, nthreads=1, bbar="euler"):
    """Sequential fp64 scan.  bbar selects the input term: 'euler'
    (Delta*B*u) or 'zoh' ((exp(Delta*A) - 1)/A * B*u).

    u, delta, z: (batch, dim, L); A: (dim, N); B, C: (batch, N, L);
    D, delta_bias: (dim,); h0: (batch, dim, N).  Returns (y, last_state) as
    float64 arrays of shapes (batch, dim, L) and (batch, dim, N).
    """
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
    batch, dim, L = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (dim, N)
    assert B.shape == (batch, N, L) and C.shape == (batch, N, L)
    assert z is None or z.shape == u.shape
    assert D is None or D.shape == (dim,)
    assert delta_bias is None or delta_bias.shape == (dim,)
    assert h0 is None or h0.shape == (batch, dim, N)
    y = np.empty((batch, dim, L), dtype=np.float64)
    last = np.empty((batch, dim, N), dtype=np.float64)
    rc = _load().oracle_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                 _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _zoh(bbar),
                                 _ptr(h0),
                                 _ptr(y), _ptr(last), batch, dim, N, L, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_scan_fwd failed with {rc}")
    return y, last


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=True, bbar="euler"):
    """One fp64 decode step.  ``state`` (batch, dim, N) is taken as a new
    float64 copy, updated and returned together with y (batch, dim)."""
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias = map(_f64, (D, z, delta_bias))
    batch, dim, N = st.shape
    assert u.shape == (batch, dim) and delta.shape == (batch, dim)
    assert A.shape == (dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
    y = np.empty((batch, dim), dtype=np.float64)
    rc = _load().oracle_state_update(_ptr(st), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                     _ptr(D), _ptr(z), _ptr(delta_bias),
                                     int(bool(delta_softplus)), _zoh(bbar), _ptr(y), batch, dim, N)
    if rc != 0:
        raise RuntimeError(f"oracle_state_update failed with {rc}")
    return y, st


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             dy=None, dlast=None, nthreads=1, bbar="euler"):
    """Gradients of L = sum(dy * y) + sum(dlast * last_state) for scan_fwd
    with the same arguments.  Returns a dict of float64 arrays: du, ddelta,
    dA, dB, dC, dD, dz (None without a gate), ddelta_bias, dh0."""
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias, h0, dy, dlast = map(_f64, (D, z, delta_bias, h0, dy, dlast))
    batch, dim, L = u.shape
    N = A.shape[1]
    assert dy is not None and dy.shape == u.shape
    assert dlast is None or dlast.shape == (batch, dim, N)
    out = dict(du=np.empty_like(u), ddelta=np.empty_like(u), dA=np.empty((dim, N)),
               dB=np.empty((batch, N, L)), dC=np.empty((batch, N, L)), dD=np.empty(dim),
               dz=np.empty_like(u) if z is not None else None, ddelta_bias=np.empty(dim),
               dh0=np.empty((batch, dim, N)))
    rc = _load().oracle_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                 _ptr(delta_bias), int(bool(delta_softplus)), _zoh(bbar), _ptr(h0),
                                 _ptr(dy), _ptr(dlast), _ptr(out["du"]), _ptr(out["ddelta"]),
                                 _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                                 _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dh0"]),
                                 batch, dim, N, L, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_scan_bwd failed with {rc}")
    return out


def causal_conv1d_silu(x, w, cb=None, state_in=None):
    """u = silu(causal depthwise conv of x with w (dim, K), + cb).  x:
    (batch, dim, L); state_in: (batch, dim, K-1), the inputs before t = 0
    (zeros if None).  Returns (u, state_out), state_out the K-1 last
    inputs."""
    x, w, cb, state_in = map(_f64, (x, w, cb, state_in))
    batch, dim, L = x.shape
    K = w.shape[1]
    assert w.shape == (dim, K) and K >= 1
    assert cb is None or cb.shape == (dim,)
    assert state_in is None or state_in.shape == (batch, dim, K - 1)
    u = np.empty_like(x)
    st = np.empty((batch, dim, K - 1), dtype=np.float64)
    rc = _load().oracle_causal_conv1d_silu(_ptr(x), _ptr(w), _ptr(cb), K, _ptr(state_in), _ptr(u),
                                           _ptr(st) if K > 1 else None, batch, dim, L)
    if rc != 0:
        raise RuntimeError(f"oracle_causal_conv1d_silu failed with {rc}")
    return u, st


def conv_step(conv_state, x, w, cb=None):
    """One decode token of the convolution: returns (u, new conv_state)."""
    cs = np.array(conv_state, dtype=np.float64, order="C", copy=True)
    x, w, cb = map(_f64, (x, w, cb))
    batch, dim = x.shape
    K = w.shape[1]
    assert cs.shape == (batch, dim, K - 1)
    u = np.empty_like(x)
    rc = _load().oracle_conv_step(_ptr(cs) if K > 1 else None, _ptr(x), _ptr(w), _ptr(cb), K,
                                  _ptr(u), batch, dim)
    if rc != 0:
        raise RuntimeError(f"oracle_conv_step failed with {rc}")
    return u, cs


def conv_scan_fwd(x, conv_w, conv_b, conv_state_in, delta, A, B, C, D=None, z=None,
                  delta_bias=None, delta_softplus=True, h0=None, nthreads=1, bbar="euler"):
    """The convolution prologue, then the scan on its output (two separate
    steps, in that order).  Returns (y, last_state, conv_state_out)."""
    u, cst = causal_conv1d_silu(x, conv_w, conv_b, conv_state_in)
    y, last = scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, nthreads, bbar)
    return y, last, cst


def ssd_scan_fwd(x, dt, A_head, B, C, D=None, z=None, dt_bias=None, delta_softplus=True, h0=None,
                 nthreads=1, bbar="euler"):
    """The SSD (Mamba-2) layer with scalar A per head, as the selective scan
    it is: channel d belongs to head d // P, and every channel of head h
    uses A[d, n] = A_head[h] for all n and Delta[b, d, t] = Delta_head[b, h, t].

    x, z: (batch, dim, L) with dim = H * P; dt: (batch, H, L) (raw, before
    bias and softplus); A_head, dt_bias: (H,); B, C: (batch, N, L) shared by
    all heads; D: (dim,); h0: (batch, dim, N).  Returns (y, last_state)."""
    x, dt, A_head = map(_f64, (x, dt, A_head))
    batch, dim, L = x.shape
    H = A_head.shape[0]
    assert dim % H == 0, "dim must be a multiple of the number of heads"
    P = dim // H
    assert dt.shape == (batch, H, L)
    N = np.asarray(B).shape[1]
    A_full = np.repeat(A_head, P)[:, None] * np.ones((1, N))
    delta_full = np.repeat(dt, P, axis=1)
    bias_full = None if dt_bias is None else np.repeat(_f64(dt_bias), P)
    return scan_fwd(x, delta_full, A_full, B, C, D, z, bias_full, delta_softplus, h0, nthreads, bbar)
