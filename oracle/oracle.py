"""fp64 CPU oracle of the selective scan (S6) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It wraps ``oracle.c`` (plain sequential C,
fp64, built with gcc) through ctypes and shares nothing with the HIP library.

Every function takes numpy arrays (any float dtype; they are converted exactly to
float64) in the shapes the pages give (u, delta, z: (B,L,D); A: (D,N);
B, C: (B,L,N); D_skip, delta_bias: (D,)).  See ``oracle.c`` for the equations
and the page sections each step follows.

Pins: every routine here is checked by ``tests/test_oracle_pins.py`` against
closed forms, brute-force convolution / quadratic forms, ODE integration,
finite differences and library routines; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

ZOH, EULER = 0, 1
_DISC = {"zoh": ZOH, "euler": EULER, ZOH: ZOH, EULER: EULER}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_discretize.argtypes = [ctypes.c_double, ctypes.c_double, I, P, P]
        lib.oracle_discretize.restype = None
        lib.oracle_fwd.argtypes = [I64, I64, I64, I64, I, I] + [P] * 11 + [I]
        lib.oracle_fwd.restype = I
        lib.oracle_bwd.argtypes = [I64, I64, I64, I64, I, I] + [P] * 19
        lib.oracle_bwd.restype = I
        lib.oracle_conv1d_fwd.argtypes = [I64, I64, I64, I64, I] + [P] * 4
        lib.oracle_conv1d_fwd.restype = I
        lib.oracle_conv1d_bwd.argtypes = [I64, I64, I64, I64, I] + [P] * 7
        lib.oracle_conv1d_bwd.restype = I
        lib.oracle_conv1d_step.argtypes = [I64, I64, I64, I] + [P] * 5
        lib.oracle_conv1d_step.restype = I
        lib.oracle_ssd_fwd.argtypes = [I64] * 6 + [I] + [P] * 10 + [I]
        lib.oracle_ssd_fwd.restype = I
        lib.oracle_fwd_complex.argtypes = [I64, I64, I64, I64, I, I] + [P] * 11 + [I]
        lib.oracle_fwd_complex.restype = I
        lib.oracle_step.argtypes = [I64, I64, I64, I, I] + [P] * 10
        lib.oracle_step.restype = I
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def discretize(dt: float, a: float, disc="zoh"):
    """(A_bar, B_bar/B) for one step size dt and diagonal entry a."""
    ab = ctypes.c_double()
    bc = ctypes.c_double()
    _load().oracle_discretize(float(dt), float(a), _DISC[disc], ctypes.byref(ab), ctypes.byref(bc))
    return ab.value, bc.value


def _shapes(u, A):
    Bt, L, D = u.shape
    D2, N = A.shape
    assert D2 == D, "A must be (D, N)"
    return Bt, L, D, N


def fwd(u, delta, A, B, C, D=None, delta_bias=None, z=None, h0=None,
        disc="zoh", softplus=True, nthreads=1):
    """Forward scan. Returns (out (B,L,D) float64, h_last (B,D,N) float64)."""
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, delta_bias, z, h0 = map(_f64, (D, delta_bias, z, h0))
    Bt, L, Dd, N = _shapes(u, A)
    out = np.empty((Bt, L, Dd), dtype=np.float64)
    h_last = np.empty((Bt, Dd, N), dtype=np.float64)
    rc = _load().oracle_fwd(Bt, L, Dd, N, _DISC[disc], int(bool(softplus)),
                            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                            _ptr(delta_bias), _ptr(z), _ptr(h0), _ptr(out), _ptr(h_last),
                            int(nthreads))
    if rc != 0:
        raise ValueError("oracle_fwd failed: %d" % rc)
    return out, h_last


def _pairs(x):
    """Complex arrays (any complex dtype, or real with a last axis of 2) as
    float64 (..., 2) (re, im) pairs."""
    if x is None:
        return None
    x = np.asarray(x)
    if np.iscomplexobj(x):
        x = np.stack([x.real, x.imag], axis=-1)
    return np.ascontiguousarray(x, dtype=np.float64)


def fwd_complex(u, delta, A, B, C, D=None, delta_bias=None, z=None, h0=None,
                disc="zoh", softplus=True, nthreads=1):
    """Forward scan with complex diagonal A: A (D,N), B and C (B,L,N), h0 (B,D,N)
    complex (numpy complex or real with a last axis of 2).  Returns
    (out (B,L,D) float64, h_last (B,D,N) complex128).  See oracle.c."""
    u, delta = _f64(u), _f64(delta)
    A, B, C, h0 = _pairs(A), _pairs(B), _pairs(C), _pairs(h0)
    D, delta_bias, z = map(_f64, (D, delta_bias, z))
    Bt, L, Dd = u.shape
    N = A.shape[1]
    out = np.empty((Bt, L, Dd), dtype=np.float64)
    h_last = np.empty((Bt, Dd, N, 2), dtype=np.float64)
    rc = _load().oracle_fwd_complex(Bt, L, Dd, N, _DISC[disc], int(bool(softplus)),
                                    _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(delta_bias), _ptr(z), _ptr(h0), _ptr(out), _ptr(h_last),
                                    int(nthreads))
    if rc != 0:
        raise ValueError("oracle_fwd_complex failed: %d" % rc)
    return out, h_last[..., 0] + 1j * h_last[..., 1]


def _flip_t(x):
    return None if x is None else np.ascontiguousarray(np.asarray(x)[:, ::-1])


def fwd_reverse(u, delta, A, B, C, D=None, delta_bias=None, z=None, h0=None,
                disc="zoh", softplus=True, nthreads=1):
    """The same system run backwards in time ("A Survey of Mamba" summary, scan
    modes: scanning the token sequence the other way), by definition the forward
    scan of the time-reversed sequence, reversed back:
    h_t = abar_t h_{t+1} + bbar_t u_t for t = L-1 .. 0; h0 enters at t = L-1 and
    h_last is the state after t = 0.  Returns (out, h_last)."""
    out, h_last = fwd(_flip_t(u), _flip_t(delta), A, _flip_t(B), _flip_t(C), D=D,
                      delta_bias=delta_bias, z=_flip_t(z), h0=h0, disc=disc,
                      softplus=softplus, nthreads=nthreads)
    return np.ascontiguousarray(out[:, ::-1]), h_last


def bwd(u, delta, A, B, C, D=None, delta_bias=None, z=None, h0=None, g=None,
        disc="zoh", softplus=True):
    """Backward scan. Returns a dict of float64 gradients
    (du, ddelta, dA, dB, dC, dD, ddelta_bias, dz, dh0)."""
    u, delta, A, B, C, g = map(_f64, (u, delta, A, B, C, g))
    D, delta_bias, z, h0 = map(_f64, (D, delta_bias, z, h0))
    Bt, L, Dd, N = _shapes(u, A)
    r = {
        "du": np.empty((Bt, L, Dd)), "ddelta": np.empty((Bt, L, Dd)),
        "dA": np.empty((Dd, N)), "dB": np.empty((Bt, L, N)), "dC": np.empty((Bt, L, N)),
        "dD": np.empty((Dd,)), "ddelta_bias": np.empty((Dd,)),
        "dz": np.empty((Bt, L, Dd)) if z is not None else None,
        "dh0": np.empty((Bt, Dd, N)),
    }
    rc = _load().oracle_bwd(Bt, L, Dd, N, _DISC[disc], int(bool(softplus)),
                            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                            _ptr(delta_bias), _ptr(z), _ptr(h0), _ptr(g),
                            _ptr(r["du"]), _ptr(r["ddelta"]), _ptr(r["dA"]), _ptr(r["dB"]),
                            _ptr(r["dC"]), _ptr(r["dD"]), _ptr(r["ddelta_bias"]),
                            _ptr(r["dz"]), _ptr(r["dh0"]))
    if rc != 0:
        raise ValueError("oracle_bwd failed: %d" % rc)
    return r


def step(h, u, delta, A, B, C, D=None, delta_bias=None, z=None, disc="zoh", softplus=True):
    """One recurrent step. h: (B,D,N); u, delta, z: (B,D); B, C: (B,N).
    Returns (out (B,D), h_new (B,D,N)); the input h is not modified."""
    h = np.array(h, dtype=np.float64, copy=True, order="C")
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, delta_bias, z = map(_f64, (D, delta_bias, z))
    Bt, Dd = u.shape
    N = A.shape[1]
    out = np.empty((Bt, Dd), dtype=np.float64)
    rc = _load().oracle_step(Bt, Dd, N, _DISC[disc], int(bool(softplus)), _ptr(h), _ptr(u),
                             _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(delta_bias), _ptr(z), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_step failed: %d" % rc)
    return out, h


# ---------------------------------------------------------------- conv1d + SiLU
def conv1d_fwd(x, w, bias=None, silu=True):
    """Causal depthwise conv of width K = w.shape[1] along time, then SiLU.
    x: (B, L, D); w: (D, K); bias: (D,) or None.  Returns u (B, L, D) float64."""
    x = _f64(x); w = _f64(w); bias = None if bias is None else _f64(bias)
    Bt, L, D = x.shape
    K = w.shape[1]
    u = np.empty((Bt, L, D))
    rc = _load().oracle_conv1d_fwd(Bt, L, D, K, int(bool(silu)), _ptr(x), _ptr(w), _ptr(bias),
                                   _ptr(u))
    assert rc == 0
    return u


def conv1d_bwd(x, w, g, bias=None, silu=True):
    """Gradients of sum(g * conv1d_fwd(x, w, bias)): dict dx, dw, dbias."""
    x = _f64(x); w = _f64(w); g = _f64(g); bias = None if bias is None else _f64(bias)
    Bt, L, D = x.shape
    K = w.shape[1]
    dx = np.empty((Bt, L, D)); dw = np.empty((D, K)); db = np.empty(D)
    rc = _load().oracle_conv1d_bwd(Bt, L, D, K, int(bool(silu)), _ptr(x), _ptr(w), _ptr(bias),
                                   _ptr(g), _ptr(dx), _ptr(dw), _ptr(db))
    assert rc == 0
    return {"dx": dx, "dw": dw, "dbias": db if bias is not None else None}


def conv1d_step(state, x, w, bias=None, silu=True):
    """One decode step: state (B, D, K-1) (copied, not modified), x (B, D).
    Returns (u (B, D), new state)."""
    st = _f64(state).copy(); x = _f64(x); w = _f64(w)
    bias = None if bias is None else _f64(bias)
    Bt, D = x.shape
    K = w.shape[1]
    u = np.empty((Bt, D))
    rc = _load().oracle_conv1d_step(Bt, D, K, int(bool(silu)), _ptr(st), _ptr(x), _ptr(w),
                                    _ptr(bias), _ptr(u))
    assert rc == 0
    return u, st


# ---------------------------------------------------------------- SSD (Mamba-2)
def ssd_fwd(x, dt, A, B, C, D=None, dt_bias=None, softplus=True, nthreads=None, h0=None,
            return_last=False):
    """Sequential SSD layer: x (Bt, L, H, P), dt (Bt, L, H), A (H,), B and C
    (Bt, L, G, N), D and dt_bias (H,), h0 (Bt, H, N, P) or None.  Returns y
    (Bt, L, H, P) float64, and the state after the last step (Bt, H, N, P) when
    return_last."""
    x = _f64(x); dt = _f64(dt); A = _f64(A); B = _f64(B); C = _f64(C)
    D = None if D is None else _f64(D)
    dt_bias = None if dt_bias is None else _f64(dt_bias)
    h0 = None if h0 is None else _f64(h0)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.empty((Bt, L, H, P))
    hl = np.empty((Bt, H, N, P)) if return_last else None
    th = nthreads if nthreads else min(16, os.cpu_count() or 1)
    rc = _load().oracle_ssd_fwd(Bt, L, H, P, N, G, int(bool(softplus)), _ptr(x), _ptr(dt),
                                _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(h0),
                                _ptr(y), _ptr(hl), th)
    assert rc == 0
    return (y, hl) if return_last else y
