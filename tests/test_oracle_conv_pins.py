"""Pins of the oracle's causal depthwise Conv1d + SiLU (CPU only).

The convolution that produces the scan's input u (Gu & Dao wiki note, "Mamba
architecture": Linear -> Conv1d -> SiLU -> SSM) is checked against torch's
grouped conv1d and silu (library routines), its impulse response (closed
form), the width-1 case, finite differences, torch autograd, and the decode
step iterated over time.
"""
import numpy as np
import pytest
import torch


def _inputs(Bt, L, D, K, seed, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bt, L, D))
    w = rng.standard_normal((D, K)) * 0.5
    b = rng.standard_normal(D) * 0.3 if bias else None
    return x, w, b


def _torch_conv(x, w, b, silu):
    """Causal depthwise conv by torch: pad K-1 on both sides, keep the first L."""
    Bt, L, D = x.shape
    K = w.shape[1]
    xt = torch.from_numpy(x).permute(0, 2, 1)                    # (B, D, L)
    wt = torch.from_numpy(w).unsqueeze(1)                        # (D, 1, K)
    bt = None if b is None else torch.from_numpy(b)
    y = torch.nn.functional.conv1d(xt, wt, bt, padding=K - 1, groups=D)[..., :L]
    if silu:
        y = torch.nn.functional.silu(y)
    return y.permute(0, 2, 1).numpy()


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("silu", [True, False])
@pytest.mark.parametrize("bias", [True, False])
def test_conv_matches_torch(oracle, K, silu, bias):
    x, w, b = _inputs(3, 37, 11, K, seed=10 * K + silu, bias=bias)
    got = oracle.conv1d_fwd(x, w, b, silu=silu)
    ref = _torch_conv(x, w, b, silu)
    assert np.max(np.abs(got - ref)) <= 1e-13


def test_conv_impulse_response(oracle):
    """A one-hot input at t0 gives pre-activation w[d, K-1-(t-t0)] for
    t0 <= t <= t0+K-1 and 0 elsewhere (taps in causal order, not reversed)."""
    K, L, D, t0 = 4, 12, 3, 5
    w = np.arange(1, D * K + 1, dtype=np.float64).reshape(D, K)
    x = np.zeros((1, L, D))
    x[0, t0, :] = 1.0
    u = oracle.conv1d_fwd(x, w, None, silu=False)
    for d in range(D):
        for t in range(L):
            want = w[d, K - 1 - (t - t0)] if t0 <= t <= t0 + K - 1 else 0.0
            assert u[0, t, d] == want


def test_conv_width_one_is_pointwise(oracle):
    x, w, b = _inputs(2, 9, 5, 1, seed=3)
    u = oracle.conv1d_fwd(x, w, b, silu=True)
    p = x * w[:, 0] + b
    assert np.max(np.abs(u - p / (1 + np.exp(-p)))) <= 1e-15


@pytest.mark.parametrize("silu", [True, False])
def test_conv_backward_finite_differences(oracle, silu):
    x, w, b = _inputs(2, 7, 3, 4, seed=21)
    g = np.random.default_rng(22).standard_normal(x.shape)
    r = oracle.conv1d_bwd(x, w, g, b, silu=silu)
    loss = lambda xx, ww, bb: float(np.sum(g * oracle.conv1d_fwd(xx, ww, bb, silu=silu)))  # noqa
    h = 1e-6
    for name, arr, grad in (("x", x, r["dx"]), ("w", w, r["dw"]), ("b", b, r["dbias"])):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = {"x": (ap, w, b), "w": (x, ap, b), "b": (x, w, ap)}[name]
            args_m = {"x": (am, w, b), "w": (x, am, b), "b": (x, w, am)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.max(np.abs(fd - grad)) <= 1e-7 * (1 + np.max(np.abs(grad))), name


def test_conv_backward_matches_autograd(oracle):
    x, w, b = _inputs(2, 19, 6, 4, seed=31)
    g = np.random.default_rng(32).standard_normal(x.shape)
    r = oracle.conv1d_bwd(x, w, g, b, silu=True)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    L, K = x.shape[1], w.shape[1]
    y = torch.nn.functional.conv1d(xt.permute(0, 2, 1), wt.unsqueeze(1), bt, padding=K - 1,
                                   groups=x.shape[2])[..., :L]
    (torch.nn.functional.silu(y).permute(0, 2, 1) * torch.from_numpy(g)).sum().backward()
    assert np.max(np.abs(r["dx"] - xt.grad.numpy())) <= 1e-12
    assert np.max(np.abs(r["dw"] - wt.grad.numpy())) <= 1e-12
    assert np.max(np.abs(r["dbias"] - bt.grad.numpy())) <= 1e-12


@pytest.mark.parametrize("K", [1, 2, 4])
def test_conv_step_iterates_to_forward(oracle, K):
    """Decode steps from a zero state reproduce the forward row by row; the state
    ends holding the last K-1 inputs."""
    x, w, b = _inputs(2, 10, 4, K, seed=41)
    full = oracle.conv1d_fwd(x, w, b, silu=True)
    st = np.zeros((2, 4, K - 1))
    for t in range(10):
        u, st = oracle.conv1d_step(st, x[:, t], w, b, silu=True)
        assert np.max(np.abs(u - full[:, t])) <= 1e-15
    if K > 1:
        assert np.array_equal(st, np.transpose(x[:, 10 - (K - 1):], (0, 2, 1)))
