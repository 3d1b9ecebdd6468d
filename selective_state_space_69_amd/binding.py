"""Thin ctypes binding of libssscan.so (C ABI declared in include/ss_scan.h,
include/ss_conv.h and include/ss_ssd.h).

The functions named like the C entry points (ss_scan_fwd, ss_scan_fwd_noalloc, ss_scan_fwd_dir,
ss_scan_fwd_complex, ss_scan_fwd_complex_ws, ss_scan_bwd, ss_scan_step, ss_scan_step_complex, ss_scan_workspace_bytes, ss_scan_strerror, ss_scan_version,
ss_conv1d_fwd, ss_conv1d_bwd, ss_conv1d_step, ss_conv1d_workspace_bytes, ss_ssd_fwd,
ss_ssd_fwd_state, ss_ssd_step) only
marshal arguments: torch tensors become device pointers, None becomes NULL and
the stream defaults to torch's current HIP stream.  Every step runs in the HIP
kernels; there is no fallback.  The convenience wrappers scan_fwd, scan_bwd,
scan_bidir, scan_fwd_complex, scan_step, scan_step_complex, conv1d_fwd, conv1d_bwd, conv1d_step, ssd_fwd and ssd_step additionally allocate
outputs and workspace with torch.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssscan.so")

SS_OK, SS_ERR_INVALID_ARG, SS_ERR_UNSUPPORTED, SS_ERR_WORKSPACE, SS_ERR_HIP = 0, -1, -2, -3, -4
SS_ERR_SCRATCH_LIMIT = -5
SS_SCAN_STATIC_SCRATCH_BYTES = 32 << 20
SS_F32, SS_BF16 = 0, 1
SS_ZOH, SS_EULER = 0, 1
SS_OP_FWD, SS_OP_BWD, SS_OP_FWD_COMPLEX = 0, 1, 2
SS_DIR_FORWARD, SS_DIR_REVERSE = 0, 1

_DTYPE = {torch.float32: SS_F32, torch.bfloat16: SS_BF16}
_DISC = {"zoh": SS_ZOH, "euler": SS_EULER}


class ss_desc_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("disc", ctypes.c_int32),
                ("delta_softplus", ctypes.c_int32), ("bc_stride", ctypes.c_int64)]


class ss_conv_desc_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("width", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("silu", ctypes.c_int32)]


class ss_ssd_desc_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("dt_softplus", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ScanError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %d (%s)" % (where, status, ss_scan_strerror(status)))
        self.status = status


_lib = None


def load_library():
    """Load libssscan.so from the package directory; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libssscan.so is not built (%s); run "
                              "`python -m selective_state_space_69_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        D = ctypes.POINTER(ss_desc_t)
        lib.ss_scan_workspace_bytes.argtypes = [D, I]
        lib.ss_scan_workspace_bytes.restype = SZ
        lib.ss_scan_fwd.argtypes = [D] + [P] * 11 + [P, SZ, P]
        lib.ss_scan_fwd.restype = I
        lib.ss_scan_fwd_noalloc.argtypes = [D] + [P] * 11 + [P]
        lib.ss_scan_fwd_noalloc.restype = I
        lib.ss_scan_fwd_dir.argtypes = [D, I, I] + [P] * 11 + [P, SZ, P]
        lib.ss_scan_fwd_dir.restype = I
        lib.ss_scan_fwd_complex.argtypes = [D] + [P] * 11 + [P]
        lib.ss_scan_fwd_complex.restype = I
        lib.ss_scan_fwd_complex_ws.argtypes = [D] + [P] * 11 + [P, SZ, P]
        lib.ss_scan_fwd_complex_ws.restype = I
        lib.ss_scan_bwd.argtypes = [D] + [P] * 19 + [P, SZ, P]
        lib.ss_scan_bwd.restype = I
        lib.ss_scan_step.argtypes = [D] + [P] * 10 + [P]
        lib.ss_scan_step.restype = I
        lib.ss_scan_step_complex.argtypes = [D] + [P] * 10 + [P]
        lib.ss_scan_step_complex.restype = I
        C = ctypes.POINTER(ss_conv_desc_t)
        lib.ss_conv1d_workspace_bytes.argtypes = [C]
        lib.ss_conv1d_workspace_bytes.restype = SZ
        lib.ss_conv1d_fwd.argtypes = [C] + [P] * 4 + [P]
        lib.ss_conv1d_fwd.restype = I
        lib.ss_conv1d_bwd.argtypes = [C] + [P] * 7 + [P, SZ, P]
        lib.ss_conv1d_bwd.restype = I
        lib.ss_conv1d_step.argtypes = [C] + [P] * 5 + [P]
        lib.ss_conv1d_step.restype = I
        lib.ss_ssd_fwd.argtypes = [ctypes.POINTER(ss_ssd_desc_t)] + [P] * 8 + [P]
        lib.ss_ssd_fwd.restype = I
        lib.ss_ssd_fwd_state.argtypes = [ctypes.POINTER(ss_ssd_desc_t)] + [P] * 10 + [P]
        lib.ss_ssd_fwd_state.restype = I
        lib.ss_ssd_step.argtypes = [ctypes.POINTER(ss_ssd_desc_t)] + [P] * 9 + [P]
        lib.ss_ssd_step.restype = I
        lib.ss_scan_strerror.argtypes = [I]
        lib.ss_scan_strerror.restype = ctypes.c_char_p
        lib.ss_scan_version.argtypes = []
        lib.ss_scan_version.restype = I
        lib.ss_scan_arch_supported.argtypes = [ctypes.c_char_p]
        lib.ss_scan_arch_supported.restype = I
        _lib = lib
    return _lib


def make_desc(batch, seqlen, dim, dstate, in_dtype=SS_BF16, out_dtype=SS_F32, disc=SS_ZOH,
              delta_softplus=True, bc_stride=0) -> ss_desc_t:
    return ss_desc_t(int(batch), int(seqlen), int(dim), int(dstate), int(in_dtype),
                     int(out_dtype), int(disc), int(bool(delta_softplus)), int(bc_stride))


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- C-named entry points
def ss_scan_version() -> int:
    return load_library().ss_scan_version()


def ss_scan_arch_supported(arch_name) -> int:
    return load_library().ss_scan_arch_supported(
        None if arch_name is None else arch_name.encode())


def ss_scan_strerror(status: int) -> str:
    return load_library().ss_scan_strerror(int(status)).decode()


def ss_scan_workspace_bytes(desc: ss_desc_t, op: int) -> int:
    return int(load_library().ss_scan_workspace_bytes(ctypes.byref(desc), int(op)))


def ss_scan_fwd(desc, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y, h_last,
                workspace, ws_bytes, stream=None) -> int:
    return load_library().ss_scan_fwd(ctypes.byref(desc), _p(u), _p(delta), _p(A), _p(Bm), _p(Cm),
                                      _p(D_skip), _p(delta_bias), _p(z), _p(h0), _p(y), _p(h_last),
                                      _p(workspace), int(ws_bytes), _stream(stream))


def ss_scan_fwd_noalloc(desc, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y, h_last,
                        stream=None) -> int:
    return load_library().ss_scan_fwd_noalloc(ctypes.byref(desc), _p(u), _p(delta), _p(A), _p(Bm),
                                              _p(Cm), _p(D_skip), _p(delta_bias), _p(z), _p(h0),
                                              _p(y), _p(h_last), _stream(stream))


def ss_scan_fwd_dir(desc, direction, accumulate, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0,
                    y, h_last, workspace, ws_bytes, stream=None) -> int:
    return load_library().ss_scan_fwd_dir(ctypes.byref(desc), int(direction), int(accumulate),
                                          _p(u), _p(delta), _p(A), _p(Bm), _p(Cm), _p(D_skip),
                                          _p(delta_bias), _p(z), _p(h0), _p(y), _p(h_last),
                                          _p(workspace), int(ws_bytes), _stream(stream))


def ss_scan_fwd_complex(desc, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y, h_last,
                        stream=None) -> int:
    return load_library().ss_scan_fwd_complex(ctypes.byref(desc), _p(u), _p(delta), _p(A), _p(Bm),
                                              _p(Cm), _p(D_skip), _p(delta_bias), _p(z), _p(h0),
                                              _p(y), _p(h_last), _stream(stream))


def ss_scan_fwd_complex_ws(desc, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, y, h_last,
                           workspace, ws_bytes, stream=None) -> int:
    return load_library().ss_scan_fwd_complex_ws(ctypes.byref(desc), _p(u), _p(delta), _p(A),
                                                 _p(Bm), _p(Cm), _p(D_skip), _p(delta_bias), _p(z),
                                                 _p(h0), _p(y), _p(h_last), _p(workspace),
                                                 int(ws_bytes), _stream(stream))


def ss_scan_bwd(desc, u, delta, A, Bm, Cm, D_skip, delta_bias, z, h0, dy, du, ddelta, dA, dB, dC,
                dD_skip, ddelta_bias, dz, dh0, workspace, ws_bytes, stream=None) -> int:
    return load_library().ss_scan_bwd(ctypes.byref(desc), _p(u), _p(delta), _p(A), _p(Bm), _p(Cm),
                                      _p(D_skip), _p(delta_bias), _p(z), _p(h0), _p(dy), _p(du),
                                      _p(ddelta), _p(dA), _p(dB), _p(dC), _p(dD_skip),
                                      _p(ddelta_bias), _p(dz), _p(dh0), _p(workspace),
                                      int(ws_bytes), _stream(stream))


def ss_scan_step(desc, h, u, delta, A, Bm, Cm, D_skip, delta_bias, z, y, stream=None) -> int:
    return load_library().ss_scan_step(ctypes.byref(desc), _p(h), _p(u), _p(delta), _p(A), _p(Bm),
                                       _p(Cm), _p(D_skip), _p(delta_bias), _p(z), _p(y),
                                       _stream(stream))


def ss_scan_step_complex(desc, h, u, delta, A, Bm, Cm, D_skip, delta_bias, z, y,
                         stream=None) -> int:
    return load_library().ss_scan_step_complex(ctypes.byref(desc), _p(h), _p(u), _p(delta),
                                               _p(A), _p(Bm), _p(Cm), _p(D_skip),
                                               _p(delta_bias), _p(z), _p(y), _stream(stream))


def make_conv_desc(batch, seqlen, dim, width, in_dtype=SS_F32, out_dtype=SS_F32, silu=True):
    return ss_conv_desc_t(int(batch), int(seqlen), int(dim), int(width), int(in_dtype),
                          int(out_dtype), int(bool(silu)))


def ss_conv1d_workspace_bytes(desc: ss_conv_desc_t) -> int:
    return int(load_library().ss_conv1d_workspace_bytes(ctypes.byref(desc)))


def ss_conv1d_fwd(desc, x, w, bias, u, stream=None) -> int:
    return load_library().ss_conv1d_fwd(ctypes.byref(desc), _p(x), _p(w), _p(bias), _p(u),
                                        _stream(stream))


def ss_conv1d_bwd(desc, x, w, bias, du, dx, dw, dbias, workspace, ws_bytes, stream=None) -> int:
    return load_library().ss_conv1d_bwd(ctypes.byref(desc), _p(x), _p(w), _p(bias), _p(du),
                                        _p(dx), _p(dw), _p(dbias), _p(workspace), int(ws_bytes),
                                        _stream(stream))


def ss_conv1d_step(desc, state, x, w, bias, u, stream=None) -> int:
    return load_library().ss_conv1d_step(ctypes.byref(desc), _p(state), _p(x), _p(w), _p(bias),
                                         _p(u), _stream(stream))


# ---------------------------------------------------------------- allocating wrappers
def make_ssd_desc(batch, seqlen, nheads, headdim, dstate, ngroups=1, in_dtype=SS_BF16,
                  out_dtype=SS_F32, dt_softplus=True) -> ss_ssd_desc_t:
    return ss_ssd_desc_t(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate),
                         int(ngroups), int(in_dtype), int(out_dtype), int(bool(dt_softplus)), 0)


def ss_ssd_fwd(desc, x, dt, A, Bm, Cm, D, dt_bias, y, stream=None) -> int:
    return load_library().ss_ssd_fwd(ctypes.byref(desc), _p(x), _p(dt), _p(A), _p(Bm), _p(Cm),
                                      _p(D), _p(dt_bias), _p(y), _stream(stream))


def ss_ssd_fwd_state(desc, x, dt, A, Bm, Cm, D, dt_bias, h0, y, h_last, stream=None) -> int:
    return load_library().ss_ssd_fwd_state(ctypes.byref(desc), _p(x), _p(dt), _p(A), _p(Bm),
                                            _p(Cm), _p(D), _p(dt_bias), _p(h0), _p(y),
                                            _p(h_last), _stream(stream))


def ss_ssd_step(desc, h, x, dt, A, Bm, Cm, D, dt_bias, y, stream=None) -> int:
    return load_library().ss_ssd_step(ctypes.byref(desc), _p(h), _p(x), _p(dt), _p(A), _p(Bm),
                                       _p(Cm), _p(D), _p(dt_bias), _p(y), _stream(stream))


def _check(rc, where):
    if rc != SS_OK:
        raise ScanError(rc, where)


def _row_stride(t, name):
    """Elements from one row of t to the next, over every leading axis flattened
    ((B, L, N) -> B*L rows of N, (B, N) -> B rows); the last axis must be unit
    stride."""
    shape, stride = t.shape, t.stride()
    if shape[-1] > 1 and stride[-1] != 1:
        raise ValueError(f"{name}: the last axis must have unit stride")
    S = None
    step = None
    for n, st in zip(reversed(shape[:-1]), reversed(stride[:-1])):
        if n == 1:
            continue
        if S is None:
            S, step = st, st * n
        elif st != step:
            raise ValueError(f"{name}: rows must be evenly spaced (one stride over all rows)")
        else:
            step = st * n
    return shape[-1] if S is None else S


def _bc_stride(B, C, N):
    """ss_desc_t.bc_stride for B and C read in place: 0 for dense rows, else the
    common row stride (e.g. B, C sliced from the input projection's output)."""
    sb, sc = _row_stride(B, "B"), _row_stride(C, "C")
    if sb != sc:
        raise ValueError("B and C must share one row stride")
    if sb < N:
        raise ValueError("B, C rows overlap (row stride below dstate)")
    # dense rows are read in place with 16-byte loads; a dense view at another
    # offset goes through the strided path, which needs element alignment only
    dense_ok = B.data_ptr() % 16 == 0 and C.data_ptr() % 16 == 0
    return 0 if sb == N and dense_ok else sb


def _dense(**tensors):
    """The library reads every tensor but strided B, C as dense rows: refuse
    views with other strides instead of reading the wrong elements."""
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous (got strides %s)" % (name, tuple(t.stride())))


def _desc_from(u, A, B, C, disc, softplus, out_dtype):
    Bt, L, D = u.shape
    N = A.shape[1]
    return make_desc(Bt, L, D, N, _DTYPE[u.dtype], _DTYPE[out_dtype], _DISC[disc], softplus,
                     _bc_stride(B, C, N))


def workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def scan_fwd(u, delta, A, B, C, D=None, delta_bias=None, z=None, h0=None, disc="zoh",
             softplus=True, out_dtype=torch.float32, return_last_state=False, stream=None,
             ws=None, reverse=False, y=None):
    """Forward scan on device tensors; returns y (and h_last).  reverse=True runs
    the system from the last step to the first; passing y adds the result to it
    (in place) instead of allocating a new output.  B and C may be views with a
    row stride (column ranges of one projection output); the other tensors are
    dense."""
    _dense(u=u, delta=delta, A=A, D=D, delta_bias=delta_bias, z=z, h0=h0, y=y)
    desc = _desc_from(u, A, B, C, disc, softplus, out_dtype if y is None else y.dtype)
    acc = y is not None
    if y is None:
        y = torch.empty(u.shape, dtype=out_dtype, device=u.device)
    h_last = (torch.empty((u.shape[0], u.shape[2], A.shape[1]), dtype=torch.float32,
                          device=u.device) if return_last_state else None)
    nb = ss_scan_workspace_bytes(desc, SS_OP_FWD)
    if ws is None or ws.numel() < nb:
        ws = workspace(nb, u.device)
    _check(ss_scan_fwd_dir(desc, SS_DIR_REVERSE if reverse else SS_DIR_FORWARD, int(acc), u, delta,
                           A, B, C, D, delta_bias, z, h0, y, h_last, ws, nb, stream),
           "ss_scan_fwd_dir")
    return (y, h_last) if return_last_state else y


def scan_fwd_complex(u, delta, A, B, C, D=None, delta_bias=None, z=None, h0=None, disc="zoh",
                     softplus=True, out_dtype=torch.float32, return_last_state=False,
                     stream=None):
    """Complex-A forward: A (D, N, 2) float32, B and C (B, L, N, 2) in u's dtype,
    h0 (B, D, N, 2) float32 ((re, im) pairs).  Returns y (and h_last (B, D, N, 2)).
    Uses ss_scan_fwd_complex_ws with a torch workspace (time chunks where the
    plan wants them)."""
    _dense(u=u, delta=delta, A=A, B=B, C=C, D=D, delta_bias=delta_bias, z=z, h0=h0)
    Bt, L, Dd = u.shape
    N = A.shape[1]
    desc = make_desc(Bt, L, Dd, N, _DTYPE[u.dtype], _DTYPE[out_dtype], _DISC[disc], softplus)
    y = torch.empty(u.shape, dtype=out_dtype, device=u.device)
    h_last = (torch.empty((Bt, Dd, N, 2), dtype=torch.float32, device=u.device)
              if return_last_state else None)
    nb = ss_scan_workspace_bytes(desc, SS_OP_FWD_COMPLEX)
    ws = workspace(nb, u.device)
    _check(ss_scan_fwd_complex_ws(desc, u, delta, A, B, C, D, delta_bias, z, h0, y, h_last, ws,
                                  nb, stream), "ss_scan_fwd_complex_ws")
    return (y, h_last) if return_last_state else y


def scan_bidir(u, delta, A, B, C, D=None, delta_bias=None, z=None, disc="zoh", softplus=True,
               A_rev=None, D_rev=None, delta_bias_rev=None, out_dtype=torch.float32, stream=None):
    """Bidirectional scan: the forward scan plus the reverse-time scan (with its
    own A, D, delta_bias when given), summed inside the second kernel."""
    y = scan_fwd(u, delta, A, B, C, D=D, delta_bias=delta_bias, z=z, disc=disc,
                 softplus=softplus, out_dtype=out_dtype, stream=stream)
    scan_fwd(u, delta, A if A_rev is None else A_rev, B, C,
             D=D if D_rev is None else D_rev,
             delta_bias=delta_bias if delta_bias_rev is None else delta_bias_rev, z=z, disc=disc,
             softplus=softplus, stream=stream, reverse=True, y=y)
    return y


def scan_bwd(u, delta, A, B, C, dy, D=None, delta_bias=None, z=None, h0=None, disc="zoh",
             softplus=True, want_dh0=False, stream=None):
    """Backward scan; returns a dict of fp32 gradients (dB, dC dense even when B
    and C are strided views)."""
    _dense(u=u, delta=delta, A=A, D=D, delta_bias=delta_bias, z=z, h0=h0, dy=dy)
    desc = _desc_from(u, A, B, C, disc, softplus, torch.float32)
    dev = u.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"du": torch.empty(u.shape, **f32), "ddelta": torch.empty(u.shape, **f32),
         "dA": torch.empty(A.shape, **f32), "dB": torch.empty(B.shape, **f32),
         "dC": torch.empty(C.shape, **f32),
         "dD": torch.empty(D.shape, **f32) if D is not None else None,
         "ddelta_bias": torch.empty(delta_bias.shape, **f32) if delta_bias is not None else None,
         "dz": torch.empty(u.shape, **f32) if z is not None else None,
         "dh0": torch.empty((u.shape[0], u.shape[2], A.shape[1]), **f32) if want_dh0 else None}
    nb = ss_scan_workspace_bytes(desc, SS_OP_BWD)
    ws = workspace(nb, dev)
    _check(ss_scan_bwd(desc, u, delta, A, B, C, D, delta_bias, z, h0, dy, g["du"], g["ddelta"],
                       g["dA"], g["dB"], g["dC"], g["dD"], g["ddelta_bias"], g["dz"], g["dh0"],
                       ws, nb, stream), "ss_scan_bwd")
    return g


def scan_step(h, u, delta, A, B, C, D=None, delta_bias=None, z=None, disc="zoh", softplus=True,
              out_dtype=torch.float32, stream=None):
    """One recurrent step; h (B,D,N) fp32 is updated in place; returns y (B,D).
    B and C (B,N) may be strided views, as in scan_fwd."""
    _dense(h=h, u=u, delta=delta, A=A, D=D, delta_bias=delta_bias, z=z)
    Bt, Dd = u.shape
    desc = make_desc(Bt, 1, Dd, A.shape[1], _DTYPE[u.dtype], _DTYPE[out_dtype], _DISC[disc],
                     softplus, _bc_stride(B, C, A.shape[1]))
    y = torch.empty(u.shape, dtype=out_dtype, device=u.device)
    _check(ss_scan_step(desc, h, u, delta, A, B, C, D, delta_bias, z, y, stream), "ss_scan_step")
    return y


def scan_step_complex(h, u, delta, A, B, C, D=None, delta_bias=None, z=None, disc="zoh",
                      softplus=True, out_dtype=torch.float32, stream=None):
    """One step with complex A: h (B,D,N,2) fp32 updated in place, A (D,N,2),
    B and C (B,N,2); returns y (B,D)."""
    _dense(h=h, u=u, delta=delta, A=A, B=B, C=C, D=D, delta_bias=delta_bias, z=z)
    Bt, Dd = u.shape
    desc = make_desc(Bt, 1, Dd, A.shape[1], _DTYPE[u.dtype], _DTYPE[out_dtype], _DISC[disc],
                     softplus)
    y = torch.empty(u.shape, dtype=out_dtype, device=u.device)
    _check(ss_scan_step_complex(desc, h, u, delta, A, B, C, D, delta_bias, z, y, stream),
           "ss_scan_step_complex")
    return y


def conv1d_fwd(x, w, bias=None, silu=True, out_dtype=None, stream=None):
    """Causal depthwise conv of width w.shape[1] (+ SiLU) over x (B, L, D);
    returns u (B, L, D) in out_dtype (default: x's dtype)."""
    _dense(x=x, w=w, bias=bias)
    Bt, L, Dd = x.shape
    out_dtype = x.dtype if out_dtype is None else out_dtype
    desc = make_conv_desc(Bt, L, Dd, w.shape[1], _DTYPE[x.dtype], _DTYPE[out_dtype], silu)
    u = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _check(ss_conv1d_fwd(desc, x, w, bias, u, stream), "ss_conv1d_fwd")
    return u


def conv1d_bwd(x, w, du, bias=None, silu=True, stream=None):
    """Backward of conv1d_fwd given du (fp32); returns dict dx, dw, dbias (fp32)."""
    _dense(x=x, w=w, du=du, bias=bias)
    Bt, L, Dd = x.shape
    desc = make_conv_desc(Bt, L, Dd, w.shape[1], _DTYPE[x.dtype], SS_F32, silu)
    f32 = dict(dtype=torch.float32, device=x.device)
    g = {"dx": torch.empty(x.shape, **f32), "dw": torch.empty(w.shape, **f32),
         "dbias": torch.empty(bias.shape, **f32) if bias is not None else None}
    nb = ss_conv1d_workspace_bytes(desc)
    ws = workspace(nb, x.device)
    _check(ss_conv1d_bwd(desc, x, w, bias, du, g["dx"], g["dw"], g["dbias"], ws, nb, stream),
           "ss_conv1d_bwd")
    return g


def conv1d_step(state, x, w, bias=None, silu=True, out_dtype=torch.float32, stream=None):
    """One decode step: state (B, D, K-1) fp32 updated in place, x (B, D); returns u."""
    _dense(state=state, x=x, w=w, bias=bias)
    Bt, Dd = x.shape
    desc = make_conv_desc(Bt, 1, Dd, w.shape[1], _DTYPE[x.dtype], _DTYPE[out_dtype], silu)
    u = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _check(ss_conv1d_step(desc, state, x, w, bias, u, stream), "ss_conv1d_step")
    return u


def ssd_fwd(x, dt, A, B, C, D=None, dt_bias=None, softplus=True, out_dtype=torch.float32,
            stream=None, h0=None, return_last=False):
    """SSD (Mamba-2) layer forward: x (Bt, L, H, P), dt (Bt, L, H), B and C
    (Bt, L, G, N) in bf16; A, D, dt_bias (H,) fp32; optional start state h0
    (Bt, H, N, P) fp32.  Returns y (Bt, L, H, P), and with return_last the
    state after the last step as well."""
    _dense(x=x, dt=dt, A=A, B=B, C=C, D=D, dt_bias=dt_bias, h0=h0)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    desc = make_ssd_desc(Bt, L, H, P, N, G, _DTYPE[x.dtype], _DTYPE[out_dtype], softplus)
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    if h0 is None and not return_last:
        _check(ss_ssd_fwd(desc, x, dt, A, B, C, D, dt_bias, y, stream), "ss_ssd_fwd")
        return y
    h_last = (torch.empty((Bt, H, N, P), dtype=torch.float32, device=x.device)
              if return_last else None)
    _check(ss_ssd_fwd_state(desc, x, dt, A, B, C, D, dt_bias, h0, y, h_last, stream),
           "ss_ssd_fwd_state")
    return (y, h_last) if return_last else y


def ssd_step(h, x, dt, A, B, C, D=None, dt_bias=None, softplus=True, out_dtype=torch.float32,
             stream=None):
    """One SSD decode step: h (Bt, H, N, P) fp32 updated in place; x (Bt, H, P),
    dt (Bt, H), B and C (Bt, G, N) bf16.  Returns y (Bt, H, P)."""
    _dense(h=h, x=x, dt=dt, A=A, B=B, C=C, D=D, dt_bias=dt_bias)
    Bt, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    desc = make_ssd_desc(Bt, 1, H, P, N, G, _DTYPE[x.dtype], _DTYPE[out_dtype], softplus)
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _check(ss_ssd_step(desc, h, x, dt, A, B, C, D, dt_bias, y, stream), "ss_ssd_step")
    return y
