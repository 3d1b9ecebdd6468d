"""Pins of the oracle's SSD (Mamba-2) layer (CPU only).

The sequential recurrence is checked against the semiseparable-matrix form the
pages give ("A Survey of Mamba" summary, Mamba-2: y = M x with
M_ji = C_j^T A_{j:i} B_i), written with numpy matrix products, and against
the selective-scan oracle in the special case it reduces to (one channel per
head, every state sharing the head's A, B_bar = dt B)."""
import numpy as np
import pytest


def _inputs(Bt, L, H, P, N, G, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bt, L, H, P))
    dt = rng.standard_normal((Bt, L, H)) * 0.5
    A = -np.exp(rng.standard_normal(H))
    B = rng.standard_normal((Bt, L, G, N))
    C = rng.standard_normal((Bt, L, G, N))
    D = rng.uniform(0.5, 1.5, H)
    bias = rng.standard_normal(H) * 0.3 - 1.0
    return x, dt, A, B, C, D, bias


def _softplus(v):
    return np.logaddexp(0.0, v)


@pytest.mark.parametrize("G", [1, 2])
def test_ssd_equals_semiseparable_matrix(oracle, G):
    Bt, L, H, P, N = 2, 23, 4, 5, 6
    x, dt, A, B, C, D, bias = _inputs(Bt, L, H, P, N, G, seed=3 + G)
    y = oracle.ssd_fwd(x, dt, A, B, C, D=D, dt_bias=bias)
    hpg = H // G
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            d = _softplus(dt[b, :, h] + bias[h])          # (L,)
            la = np.cumsum(d * A[h])                      # log of the running decay
            # M[j, i] = C_j . B_i * exp(sum_{i<r<=j} dt_r A) * dt_i for i <= j
            decay = np.exp(la[:, None] - la[None, :])
            M = (C[b, :, g] @ B[b, :, g].T) * decay * d[None, :]
            M = np.tril(M)
            ref = M @ x[b, :, h] + D[h] * x[b, :, h]
            assert np.max(np.abs(y[b, :, h] - ref)) <= 1e-10 * (1 + np.max(np.abs(ref)))


def test_ssd_reduces_to_selective_scan(oracle):
    """P = 1: each head is one selective-scan channel whose N states share A_h,
    with the Euler input coefficient (B_bar = dt B) and no gate."""
    Bt, L, H, N = 2, 31, 3, 8
    x, dt, A, B, C, D, bias = _inputs(Bt, L, H, 1, N, 1, seed=9)
    y = oracle.ssd_fwd(x, dt, A, B, C, D=D, dt_bias=bias)
    u = x[..., 0]                                         # (Bt, L, H): channels = heads
    Ad = np.repeat(A[:, None], N, axis=1)                 # (H, N)
    ref, _ = oracle.fwd(u, dt, Ad, B[:, :, 0], C[:, :, 0], D=D, delta_bias=bias, z=None,
                        disc="euler")
    assert np.max(np.abs(y[..., 0] - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))


def test_ssd_zero_step_keeps_skip_only(oracle):
    """dt -> 0 (softplus(-60)): no state is ever written, y = D x."""
    Bt, L, H, P, N = 1, 9, 2, 3, 4
    x, dt, A, B, C, D, _ = _inputs(Bt, L, H, P, N, 1, seed=2)
    y = oracle.ssd_fwd(x, np.full_like(dt, -60.0), A, B, C, D=D, dt_bias=None)
    assert np.max(np.abs(y - D[None, None, :, None] * x)) <= 1e-20


def test_ssd_state_in_and_out_closed_form(oracle):
    """With a start state H0 the output gains C_t . (prod_{s<=t} a_s) H0 and the
    final state is (prod_t a_t) H0 + sum_t (prod_{s>t} a_s) dt_t B_t x_t^T, both
    written here as numpy products over the whole sequence."""
    Bt, L, H, P, N, G = 2, 17, 3, 5, 4, 1
    x, dt, A, B, C, D, bias = _inputs(Bt, L, H, P, N, G, seed=21)
    rng = np.random.default_rng(22)
    h0 = rng.standard_normal((Bt, H, N, P))
    y, hl = oracle.ssd_fwd(x, dt, A, B, C, D=D, dt_bias=bias, h0=h0, return_last=True)
    y0 = oracle.ssd_fwd(x, dt, A, B, C, D=D, dt_bias=bias)
    for b in range(Bt):
        for h in range(H):
            d = _softplus(dt[b, :, h] + bias[h])
            la = np.cumsum(d * A[h])                      # log prod_{s<=t} a_s
            # the start state's share of y_t
            extra = np.exp(la)[:, None] * (C[b, :, 0] @ h0[b, h])      # (L, P)
            assert np.max(np.abs(y[b, :, h] - y0[b, :, h] - extra)) <= 1e-10 * (
                1 + np.max(np.abs(extra)))
            w = np.exp(la[-1] - la) * d                   # prod_{s>t} a_s * dt_t
            ref = np.exp(la[-1]) * h0[b, h] + (B[b, :, 0] * w[:, None]).T @ x[b, :, h]
            assert np.max(np.abs(hl[b, h] - ref)) <= 1e-10 * (1 + np.max(np.abs(ref)))


def test_ssd_split_sequence(oracle):
    """Running [0, L1) and then [L1, L) from the state the first part leaves equals
    one run over [0, L) (outputs and final state)."""
    Bt, L, H, P, N, G = 2, 29, 4, 3, 5, 2
    x, dt, A, B, C, D, bias = _inputs(Bt, L, H, P, N, G, seed=23)
    y, hl = oracle.ssd_fwd(x, dt, A, B, C, D=D, dt_bias=bias, return_last=True)
    L1 = 11
    ya, ha = oracle.ssd_fwd(x[:, :L1], dt[:, :L1], A, B[:, :L1], C[:, :L1], D=D, dt_bias=bias,
                            return_last=True)
    yb, hb = oracle.ssd_fwd(x[:, L1:], dt[:, L1:], A, B[:, L1:], C[:, L1:], D=D, dt_bias=bias,
                            h0=ha, return_last=True)
    assert np.max(np.abs(np.concatenate([ya, yb], axis=1) - y)) <= 1e-12 * (1 + np.max(np.abs(y)))
    assert np.max(np.abs(hb - hl)) <= 1e-12 * (1 + np.max(np.abs(hl)))
