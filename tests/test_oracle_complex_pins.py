"""Pins of the oracle's complex-A scan (CPU only).

Checked against: an RK4 integration of the complex ODE over one step (the ZOH
step), the real oracle when every imaginary part is zero, the causal
convolution with the complex kernel of an LTI system, and the same system
written with each state and its conjugate as separate states (which fixes the
factor 2 of the real output)."""
import numpy as np
import pytest


def _softplus(v):
    return np.logaddexp(0.0, v)


def _rk4_step(a, b, u, h0, dt, n=2000):
    """Integrate h' = a h + b u (u held) over [0, dt] with RK4, complex."""
    f = lambda h: a * h + b * u  # noqa
    h, s = h0, dt / n
    for _ in range(n):
        k1 = f(h); k2 = f(h + 0.5 * s * k1); k3 = f(h + 0.5 * s * k2); k4 = f(h + s * k3)
        h = h + s / 6 * (k1 + 2 * k2 + 2 * k3 + k4)
    return h


@pytest.mark.parametrize("a", [-0.7 + 2.0j, -0.5 + 9.42477796j, 0.0 + 1.3j, -1.2 + 0.0j])
def test_zoh_step_is_ode_solution(oracle, a):
    """One exact-ZOH step of a single complex state equals the ODE solution with
    the input held over the step."""
    dt = 0.37
    b, c, u0, h0 = 0.8 - 0.3j, 1.0 + 0.0j, 1.7, 0.4 + 0.9j
    delta = np.array([[[np.log(np.expm1(dt))]]])   # softplus(delta) = dt
    out, hl = oracle.fwd_complex(np.array([[[u0]]]), delta, np.array([[a]]),
                                 np.array([[[b]]]), np.array([[[c]]]), h0=np.array([[[h0]]]))
    ref = _rk4_step(a, b, u0, h0, dt)
    assert abs(hl[0, 0, 0] - ref) < 1e-10
    assert abs(out[0, 0, 0] - 2 * (c * ref).real) < 1e-10


def test_real_limit_matches_real_oracle(oracle):
    """Zero imaginary parts: y = 2 (sum_n C h) + D u, the real system's
    contraction doubled (conjugate pair of a real state = the state twice)."""
    rng = np.random.default_rng(41)
    Bt, L, D, N = 2, 50, 4, 6
    u = rng.standard_normal((Bt, L, D)); delta = 0.1 * rng.standard_normal((Bt, L, D))
    A = -np.exp(rng.standard_normal((D, N)))
    Bm = rng.standard_normal((Bt, L, N)); Cm = rng.standard_normal((Bt, L, N))
    Dk = rng.standard_normal(D); bias = rng.standard_normal(D) - 1.0
    for disc in ("zoh", "euler"):
        yc, _ = oracle.fwd_complex(u, delta, A.astype(complex), Bm.astype(complex),
                                   Cm.astype(complex), D=Dk, delta_bias=bias, disc=disc)
        yr, _ = oracle.fwd(u, delta, A, Bm, 2 * Cm, D=Dk, delta_bias=bias, disc=disc)
        np.testing.assert_allclose(yc, yr, rtol=0, atol=1e-12 * np.abs(yr).max())


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_lti_complex_is_convolution(oracle, disc):
    """Constant dt, B, C: y_t = 2 Re(sum_k K_k u_{t-k}) + D u_t with the complex
    kernel K_k = sum_n C_n abar_n^k bcoef_n B_n (abar = exp(dt a); bcoef from
    the ZOH integral or dt), plus the free response 2 Re(sum_n C_n abar_n^{t+1} h0_n)."""
    rng = np.random.default_rng(42)
    Bt, L, D, N = 1, 80, 3, 5
    A = -0.5 + 1j * np.pi * np.arange(N)[None, :] * (1 + 0.1 * rng.standard_normal((D, 1)))
    u = rng.standard_normal((Bt, L, D))
    dconst = 0.3 * rng.standard_normal((Bt, 1, D))
    delta = np.repeat(dconst, L, axis=1)
    Bc = rng.standard_normal((Bt, 1, N)) + 1j * rng.standard_normal((Bt, 1, N))
    Cc = rng.standard_normal((Bt, 1, N)) + 1j * rng.standard_normal((Bt, 1, N))
    h0 = rng.standard_normal((Bt, D, N)) + 1j * rng.standard_normal((Bt, D, N))
    Dk = rng.standard_normal(D)
    out, _ = oracle.fwd_complex(u, delta, A, np.repeat(Bc, L, 1), np.repeat(Cc, L, 1), D=Dk,
                                h0=h0, disc=disc)
    for d in range(D):
        dt = _softplus(dconst[0, 0, d])
        ab = np.exp(dt * A[d])
        if disc == "zoh":
            # bcoef = integral_0^dt exp(a s) ds, by the trapezoid rule on a fine grid
            s = np.linspace(0.0, dt, 20001)
            e = np.exp(np.outer(s, A[d]))
            bc = (e[1:] + e[:-1]).sum(0) * (s[1] - s[0]) / 2
        else:
            bc = np.full(N, dt)
        K = np.array([np.sum(Cc[0, 0] * ab ** k * bc * Bc[0, 0]) for k in range(L)])
        free = np.array([np.sum(Cc[0, 0] * ab ** (t + 1) * h0[0, d]) for t in range(L)])
        for t in range(L):
            ref = 2 * (np.dot(K[:t + 1], u[0, t::-1, d]) + free[t]).real + Dk[d] * u[0, t, d]
            assert abs(out[0, t, d] - ref) < 1e-7 * (1 + abs(ref)), (d, t)


def test_conjugate_pairs_as_separate_states(oracle):
    """Each complex state stands for itself and its conjugate: the same system
    with 2N explicit states (a_n, conj a_n; B_n, conj B_n; C_n, conj C_n) and a
    plain sum of C h has a real output equal to the oracle's y (Euler input)."""
    rng = np.random.default_rng(43)
    Bt, L, D, N = 1, 40, 2, 4
    u = rng.standard_normal((Bt, L, D)); delta = 0.2 * rng.standard_normal((Bt, L, D))
    A = -np.exp(rng.standard_normal((D, N))) + 1j * 3 * rng.standard_normal((D, N))
    Bm = rng.standard_normal((Bt, L, N)) + 1j * rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N)) + 1j * rng.standard_normal((Bt, L, N))
    out, _ = oracle.fwd_complex(u, delta, A, Bm, Cm, disc="euler")
    for d in range(D):
        a2 = np.concatenate([A[d], A[d].conj()])
        h = np.zeros(2 * N, dtype=complex)
        for t in range(L):
            dt = _softplus(delta[0, t, d])
            b2 = np.concatenate([Bm[0, t], Bm[0, t].conj()])
            c2 = np.concatenate([Cm[0, t], Cm[0, t].conj()])
            h = np.exp(dt * a2) * h + dt * b2 * u[0, t, d]
            y = np.sum(c2 * h)
            assert abs(y.imag) < 1e-12 * (1 + abs(y))
            assert abs(out[0, t, d] - y.real) < 1e-12 * (1 + abs(y))
