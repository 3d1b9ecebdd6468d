"""Seeded synthetic inputs for the selective scan.

This module only draws random numbers and lays them out; it contains none of the
scan's arithmetic, so both the HIP path and the fp64 oracle can be fed from it.

The value recipe follows the shapes and parameterisation of the pages
("Mamba: S4 epic upgrade", section "TL;DR": u, delta: (B,L,D); B, C: (B,L,N);
A: (D,N)) with the standard selective-scan initialisation:
  * u, z, B, C ~ N(0, 1); raw delta ~ N(0, 0.1) (standard deviation 0.1);
  * a per-channel step bias chosen so that softplus(bias) is log-uniform in a
    range (the bias is the inverse softplus of dt = exp(U(ln lo, ln hi)));
  * D_skip ~ U(0.5, 1.5);
  * A[d, n] = -(n + 1) (the real diagonal "S4D-Real" initialisation), or, for
    tests that must not rely on that structure, other real diagonals.
bf16 workloads are rounded once from the fp32 draws with round-to-nearest-even,
and the same bits are given to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32
    arrays whose low 16 bits are zero (exact bf16 values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    r = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exact bf16 numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    """One named workload: shapes, number type and discretisation."""
    name: str
    B: int
    L: int
    D: int
    N: int
    dtype: str              # "f32" or "bf16" (u, delta, z, B, C)
    disc: str               # "zoh" or "euler"
    dt_range: tuple = (1e-3, 1e-1)
    seed: int = 0
    op: str = "fwd"         # "fwd" or "bwd"
    desc: str = ""

    @property
    def elements(self) -> int:
        return self.B * self.L * self.D * self.N


# The workloads the scan is measured and checked on.  Widths follow Mamba-130M
# (d_model 768 x expand 2 = 1536) and Mamba-2.8B (2560 x 2 = 5120); N = 16.
WORKLOADS = {
    w.name: w for w in [
        Workload("fwd_tiny_f32_b1_l256_d64", 1, 256, 64, 16, "f32", "zoh", seed=1000,
                 desc="tiny fp32 forward, exact ZOH, silu gate"),
        Workload("fwd_130m_bf16_b8_l2048_d1536", 8, 2048, 1536, 16, "bf16", "euler", seed=1001,
                 desc="Mamba-130M-shaped layer forward, Euler B_bar"),
        Workload("fwd_2p8b_bf16_b8_l2048_d5120", 8, 2048, 5120, 16, "bf16", "zoh", seed=1002,
                 desc="Mamba-2.8B-shaped layer forward, exact ZOH"),
        Workload("fwd_2p8b_bf16_b2_l8192_d5120", 2, 8192, 5120, 16, "bf16", "zoh", seed=1012,
                 desc="Mamba-2.8B-shaped layer forward, 8192-long variant"),
        Workload("fwd_long_bf16_b1_l1048576_d256", 1, 1048576, 256, 16, "bf16", "zoh",
                 dt_range=(1e-4, 1e-2), seed=1003,
                 desc="million-step forward through the chunked carry"),
        Workload("bwd_130m_bf16_b8_l2048_d1536", 8, 2048, 1536, 16, "bf16", "euler", seed=1004,
                 op="bwd", desc="backward with recompute at the Mamba-130M shape"),
    ]
}


@dataclass
class Inputs:
    """Host arrays (float32 holding the exact values both sides receive)."""
    u: np.ndarray
    delta: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray | None
    delta_bias: np.ndarray | None
    z: np.ndarray | None
    h0: np.ndarray | None = None
    dy: np.ndarray | None = None
    dtype: str = "f32"
    meta: dict = field(default_factory=dict)


def make_A(D: int, N: int, mode: str = "s4d_real", rng: np.random.Generator | None = None):
    """Diagonal A (D, N), float32.
    s4d_real : A[d, n] = -(n + 1)
    random   : A = -exp(N(0, 1))      (no integer structure)
    mixed    : random, with a few exact zeros and small positive entries
    weak     : random, with about half the entries slowly decaying (|A| log-uniform
               in [1e-4, 1e-2]), an exact zero and a tiny positive entry
    grow     : every |A| >= 0.25, about a quarter of the entries positive in
               [0.25, 1] (growing states; for short sequences)
    """
    if mode == "s4d_real":
        return np.tile(-np.arange(1, N + 1, dtype=np.float32), (D, 1))
    rng = rng or np.random.default_rng(7)
    A = -np.exp(rng.standard_normal((D, N))).astype(np.float32)
    if mode == "mixed":
        A[0, 0] = 0.0
        if D > 1:
            A[1, N - 1] = 0.0
        if D > 2:
            A[2, 0] = np.float32(0.05)   # mildly unstable entry, still finite over short L
    elif mode == "weak":
        slow = rng.random((D, N)) < 0.5
        A = np.where(slow, -(10.0 ** rng.uniform(-4.0, -2.0, (D, N))), A).astype(np.float32)
        A[0, 0] = 0.0
        if D > 1:
            A[1, N - 1] = np.float32(1e-3)
    elif mode == "grow":
        A = (A - np.float32(0.25)).astype(np.float32)
        pos = rng.random((D, N)) < 0.25
        A = np.where(pos, rng.uniform(0.25, 1.0, (D, N)), A).astype(np.float32)
    elif mode != "random":
        raise ValueError(mode)
    return A


def make_inputs(B: int, L: int, D: int, N: int, seed: int, dtype: str = "f32",
                dt_range=(1e-3, 1e-1), a_mode: str = "s4d_real", with_z: bool = True,
                with_bias: bool = True, with_D: bool = True, with_h0: bool = False,
                with_dy: bool = False, delta_std: float = 0.1) -> Inputs:
    """Draw one seeded problem.  Order of draws (float32): u, z, B, C, raw delta,
    U for the log step, D_skip, dy; then h0 (if asked) and A (non-default modes)."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    u = rng.standard_normal((B, L, D), dtype=f32)
    z = rng.standard_normal((B, L, D), dtype=f32)
    Bm = rng.standard_normal((B, L, N), dtype=f32)
    Cm = rng.standard_normal((B, L, N), dtype=f32)
    delta = rng.standard_normal((B, L, D), dtype=f32)
    delta *= f32(delta_std)
    lo, hi = dt_range
    U = rng.random(D)
    dskip = (0.5 + rng.random(D)).astype(f32)
    dy = rng.standard_normal((B, L, D), dtype=f32) if with_dy else None
    h0 = rng.standard_normal((B, D, N)).astype(f32) if with_h0 else None
    A = make_A(D, N, a_mode, rng)
    # step bias: inverse softplus of a log-uniform step (input recipe, fp64)
    dt = np.exp(math.log(lo) + U * (math.log(hi) - math.log(lo)))
    bias = (dt + np.log(-np.expm1(-dt))).astype(f32)
    if dtype == "bf16":
        u, z, Bm, Cm, delta = (round_to_bf16(x) for x in (u, z, Bm, Cm, delta))
        if dy is not None:
            dy = round_to_bf16(dy)
    elif dtype != "f32":
        raise ValueError(dtype)
    return Inputs(u=u, delta=delta, A=A, B=Bm, C=Cm, D=dskip if with_D else None,
                  delta_bias=bias if with_bias else None, z=z if with_z else None,
                  h0=h0, dy=dy, dtype=dtype,
                  meta=dict(B=B, L=L, D=D, N=N, seed=seed, dt_range=tuple(dt_range),
                            a_mode=a_mode))


def make_lti_inputs(B: int, L: int, D: int, N: int, seed: int, dtype: str = "f32",
                    dt_range=(1e-4, 1e-3), a_range=(0.25, 1.0), a_log: bool = False) -> Inputs:
    """A time-invariant problem with one-signed input, the hardest case for
    fp32 state: per channel a constant step (raw delta = 0, the bias the
    inverse softplus of a step log-uniform in dt_range), B and C rows constant
    over time (one N(0,1) row per batch row), u = 0.25 + |N(0, 1)| (never
    negative, so rounding errors do not average out), A = -U(a_range) (or
    log-uniform in a_range when a_log), D_skip ~ U(0.5, 1.5), no gate.
    Order of draws: u, B row, C row, U for the step, A, D_skip."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    u = (0.25 + np.abs(rng.standard_normal((B, L, D)))).astype(f32)
    Brow = rng.standard_normal((B, 1, N)).astype(f32)
    Crow = rng.standard_normal((B, 1, N)).astype(f32)
    U = rng.random(D)
    lo, hi = a_range
    if a_log:
        A = -np.exp(rng.uniform(math.log(lo), math.log(hi), (D, N)))
    else:
        A = -rng.uniform(lo, hi, (D, N))
    A = A.astype(f32)
    dskip = (0.5 + rng.random(D)).astype(f32)
    dlo, dhi = dt_range
    dt = np.exp(math.log(dlo) + U * (math.log(dhi) - math.log(dlo)))
    bias = (dt + np.log(-np.expm1(-dt))).astype(f32)
    Bm = np.ascontiguousarray(np.broadcast_to(Brow, (B, L, N)))
    Cm = np.ascontiguousarray(np.broadcast_to(Crow, (B, L, N)))
    delta = np.zeros((B, L, D), dtype=f32)
    if dtype == "bf16":
        u, Bm, Cm = (round_to_bf16(x) for x in (u, Bm, Cm))
    elif dtype != "f32":
        raise ValueError(dtype)
    return Inputs(u=u, delta=delta, A=A, B=Bm, C=Cm, D=dskip, delta_bias=bias, z=None,
                  dtype=dtype, meta=dict(B=B, L=L, D=D, N=N, seed=seed, dt_range=tuple(dt_range),
                                         a_range=tuple(a_range), lti=True))


def make_workload(name: str, with_dy: bool | None = None) -> Inputs:
    w = WORKLOADS[name]
    if with_dy is None:
        with_dy = w.op == "bwd"
    return make_inputs(w.B, w.L, w.D, w.N, w.seed, w.dtype, w.dt_range, with_dy=with_dy)


# ---------------------------------------------------------------- SSD (Mamba-2) layer
@dataclass
class SsdInputs:
    """Host arrays of one SSD problem (float32 holding the exact values both sides
    receive): x (Bt, L, H, P), dt (Bt, L, H), B and C (Bt, L, G, N) as exact bf16
    values; A, D, dt_bias (H,) float32."""
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray | None
    dt_bias: np.ndarray | None
    meta: dict = field(default_factory=dict)


def make_ssd_inputs(Bt: int, L: int, H: int, P: int, N: int, G: int, seed: int,
                    dt_range=(1e-3, 1e-1), a_range=(1.0, 16.0), dt_std: float = 0.1,
                    with_D: bool = True, with_bias: bool = True) -> SsdInputs:
    """Draw one seeded SSD problem.  Recipe: x, B, C ~ N(0, 1); raw dt ~ N(0, dt_std);
    per head a step bias that is the inverse softplus of a log-uniform step in
    dt_range; A_h = -U(a_range) (one scalar per head); D_h ~ U(0.5, 1.5).  x, dt,
    B, C are rounded once to bf16.  Order of draws: x, B, C, dt, U (step), A, D."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    x = rng.standard_normal((Bt, L, H, P), dtype=f32)
    Bm = rng.standard_normal((Bt, L, G, N), dtype=f32)
    Cm = rng.standard_normal((Bt, L, G, N), dtype=f32)
    dt = rng.standard_normal((Bt, L, H), dtype=f32)
    dt *= f32(dt_std)
    U = rng.random(H)
    a_lo, a_hi = a_range
    A = (-(a_lo + (a_hi - a_lo) * rng.random(H))).astype(f32)
    D = (0.5 + rng.random(H)).astype(f32)
    lo, hi = dt_range
    step = np.exp(math.log(lo) + U * (math.log(hi) - math.log(lo)))
    bias = (step + np.log(-np.expm1(-step))).astype(f32)
    x, Bm, Cm, dt = (round_to_bf16(v) for v in (x, Bm, Cm, dt))
    return SsdInputs(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D if with_D else None,
                     dt_bias=bias if with_bias else None,
                     meta=dict(Bt=Bt, L=L, H=H, P=P, N=N, G=G, seed=seed))


# The SSD workload: 80 heads of 64 channels (width 5120, as the Mamba-2.8B scan
# workload), 64 states, one B/C group.
SSD_WORKLOAD = dict(name="ssd_bf16_b8_l2048_h80_p64_n64_g1", Bt=8, L=2048, H=80, P=64, N=64,
                    G=1, seed=2001)


# ---------------------------------------------------------------- complex diagonal A
def make_A_complex(D: int, N: int, mode: str = "s4d_lin", rng: np.random.Generator | None = None):
    """Complex diagonal A as (D, N, 2) float32 (re, im) pairs.
    s4d_lin : A[d, n] = -1/2 + i pi n   (the S4D-Lin initialisation)
    random  : re = -exp(N(0, 1)), im = pi * N(0, 2)
    mixed   : random, with an exact zero and a purely imaginary entry
    weak    : random, with about half the entries of modulus log-uniform in
              [1e-4, 1e-2] (random phase) and an exact zero"""
    if mode == "s4d_lin":
        re = np.full((D, N), -0.5)
        im = np.tile(np.pi * np.arange(N), (D, 1))
    else:
        rng = rng or np.random.default_rng(8)
        re = -np.exp(rng.standard_normal((D, N)))
        im = np.pi * 2.0 * rng.standard_normal((D, N))
        if mode == "mixed":
            re[0, 0] = im[0, 0] = 0.0
            if D > 1:
                re[1, N - 1] = 0.0
        elif mode == "weak":
            slow = rng.random((D, N)) < 0.5
            mod = 10.0 ** rng.uniform(-4.0, -2.0, (D, N))
            ang = rng.uniform(0.5 * np.pi, 1.5 * np.pi, (D, N))   # Re a <= 0
            re = np.where(slow, mod * np.cos(ang), re)
            im = np.where(slow, mod * np.sin(ang), im)
            re[0, 0] = im[0, 0] = 0.0
        elif mode != "random":
            raise ValueError(mode)
    return np.stack([re, im], axis=-1).astype(np.float32)


def make_complex_inputs(B: int, L: int, D: int, N: int, seed: int, dtype: str = "f32",
                        a_mode: str = "s4d_lin", with_h0: bool = False, with_z: bool = True,
                        dt_range=(1e-3, 1e-1)) -> Inputs:
    """Real-scan inputs of make_inputs with complex B, C (B, L, N, 2) (re and im
    ~ N(0, 1/2), so |B_n| has unit second moment), A (D, N, 2) and h0 (B, D, N, 2)."""
    base = make_inputs(B, L, D, N, seed, dtype="f32", dt_range=dt_range, with_z=with_z)
    rng = np.random.default_rng(seed + 7919)
    s = np.float32(np.sqrt(0.5))
    Bm = rng.standard_normal((B, L, N, 2), dtype=np.float32) * s
    Cm = rng.standard_normal((B, L, N, 2), dtype=np.float32) * s
    h0 = rng.standard_normal((B, D, N, 2), dtype=np.float32) * s if with_h0 else None
    A = make_A_complex(D, N, a_mode, rng)
    u, z, delta = base.u, base.z, base.delta
    if dtype == "bf16":
        u, delta, Bm, Cm = (round_to_bf16(x) for x in (u, delta, Bm, Cm))
        z = round_to_bf16(z) if z is not None else None
    return Inputs(u=u, delta=delta, A=A, B=Bm, C=Cm, D=base.D, delta_bias=base.delta_bias, z=z,
                  h0=h0, dtype=dtype, meta=dict(B=B, L=L, D=D, N=N, seed=seed, a_mode=a_mode,
                                                complex=True))
