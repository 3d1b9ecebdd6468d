"""Helpers shared by the GPU parity tests: upload seeded inputs, call the HIP
library through its C ABI, run the fp64 oracle on the same bits, compare."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from selective_state_space_69_amd import binding as B

TOL_F32 = 1e-4        # |y - y_ref| <= 1e-4 (1 + |y_ref|) elementwise, fp32 inputs
TOL_BF16 = 2e-3       # max |y - y_ref| <= 2e-3 max |y_ref|, bf16 inputs, fp32 state
TOL_GRAD = 5e-3       # max |g - g_ref| <= 5e-3 max |g_ref| per gradient tensor


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(x, dtype, device="cuda"):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=device, dtype=dtype).contiguous()


def upload(inp, device="cuda"):
    """Device copies: in_dtype for u, delta, z, B, C (and dy); fp32 for the rest."""
    it = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    f32 = torch.float32
    return dict(u=dev_tensor(inp.u, it, device), delta=dev_tensor(inp.delta, it, device),
                A=dev_tensor(inp.A, f32, device), B=dev_tensor(inp.B, it, device),
                C=dev_tensor(inp.C, it, device), D=dev_tensor(inp.D, f32, device),
                delta_bias=dev_tensor(inp.delta_bias, f32, device),
                z=dev_tensor(inp.z, it, device), h0=dev_tensor(inp.h0, f32, device),
                dy=dev_tensor(inp.dy, it, device))


def gpu_fwd(d, disc, softplus=True, out_dtype=torch.float32, return_last_state=False, **over):
    args = dict(d)
    args.update(over)
    return B.scan_fwd(args["u"], args["delta"], args["A"], args["B"], args["C"], D=args["D"],
                      delta_bias=args["delta_bias"], z=args["z"], h0=args["h0"], disc=disc,
                      softplus=softplus, out_dtype=out_dtype, return_last_state=return_last_state)


def check_f32(y, ref, what=""):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - ref)
    bound = TOL_F32 * (1.0 + np.abs(ref))
    worst = float((err / bound).max()) if err.size else 0.0
    assert np.all(np.isfinite(y)), what + ": non-finite output"
    assert np.all(err <= bound), "%s: fp32 parity failed, worst err/bound = %.3g (max err %.3g)" % (
        what, worst, float(err.max()))
    return worst


def check_rel_max(y, ref, tol, what=""):
    y = np.asarray(y, dtype=np.float64)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(y - ref).max()) if ref.size else 0.0
    assert np.all(np.isfinite(y)), what + ": non-finite output"
    assert err <= tol * max(scale, 1e-30), "%s: max err %.3g > %.1e * max|ref| (%.3g)" % (
        what, err, tol, scale)
    return err / max(scale, 1e-30)


def oracle_threads():
    """Threads for the oracle's channel-parallel loop: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def full_compare_bf16(oracle, inp, y, disc, reverse=False, block=None, what=""):
    """Whole-tensor comparison of a bf16-input forward y (torch, (B, L, D)) with
    the fp64 oracle on the same bits: max|y - ref| <= 2e-3 max|ref| over every
    element.  block: run the oracle on channel blocks of that width (bounded
    host memory for very long sequences).  Returns max err / max|ref|."""
    Bt, L, D = inp.u.shape
    fn = oracle.fwd_reverse if reverse else oracle.fwd
    th = oracle_threads()
    block = block or D
    err = 0.0
    scale = 0.0
    for d0 in range(0, D, block):
        d1 = min(D, d0 + block)
        sl = (slice(None), slice(None), slice(d0, d1))
        ref, _ = fn(inp.u[sl], inp.delta[sl], inp.A[d0:d1], inp.B, inp.C,
                    D=None if inp.D is None else inp.D[d0:d1],
                    delta_bias=None if inp.delta_bias is None else inp.delta_bias[d0:d1],
                    z=None if inp.z is None else inp.z[sl],
                    h0=None if inp.h0 is None else inp.h0[:, d0:d1],
                    disc=disc, nthreads=th)
        got = y[:, :, d0:d1].double().cpu().numpy()
        assert np.all(np.isfinite(got)), what + ": non-finite output"
        err = max(err, float(np.abs(got - ref).max()))
        scale = max(scale, float(np.abs(ref).max()))
        del ref, got
    assert err <= TOL_BF16 * scale, "%s: max err %.3g > %.1e * max|ref| (%.3g)" % (
        what, err, TOL_BF16, scale)
    return err / scale
