"""Tensors past 2^31 elements: B = 1, L = 2^20, D = 2304 (2.4e9 elements per
(B, L, D) tensor, bf16 inputs, N = 16, exact ZOH), so every element index and
byte offset of a whole tensor needs more than 32 bits.  The forward, the
reverse-time scan accumulated into it, and the backward run on the whole
problem, and the Conv1d + SiLU over the same input; sampled channels (the
first, one inside, the last) are checked against the fp64 oracle on the same
bits, which depends on a channel's own inputs and the shared B, C rows only.
The SSD layer runs on x of 2.7e9 elements (one sampled head checked).  Inputs are drawn on the GPU from a seeded generator
(A = -(n + 1), steps log-uniform in [1e-3, 1e-1] through the step bias).
Marked gpu: run on an MI355X (about 60 GB of device memory)."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from gpu_util import TOL_BF16, TOL_GRAD, check_rel_max, log

pytestmark = pytest.mark.gpu

Bt, L, D, N = 1, 1 << 20, 2304, 16
SAMPLE = [0, 1151, D - 1]


@pytest.fixture(scope="module")
def problem():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    B.load_library()
    assert Bt * L * D > (1 << 31)
    g = torch.Generator(device="cuda").manual_seed(8128)
    bf = torch.bfloat16
    p = {
        "u": torch.randn((Bt, L, D), generator=g, device="cuda").to(bf),
        "z": torch.randn((Bt, L, D), generator=g, device="cuda").to(bf),
        "B": torch.randn((Bt, L, N), generator=g, device="cuda").to(bf),
        "C": torch.randn((Bt, L, N), generator=g, device="cuda").to(bf),
        "delta": (0.1 * torch.randn((Bt, L, D), generator=g, device="cuda")).to(bf),
    }
    lo, hi = np.log(1e-3), np.log(1e-1)
    step = torch.exp(lo + (hi - lo) * torch.rand(D, generator=g, device="cuda"))
    p["bias"] = (step + torch.log(-torch.expm1(-step))).float()
    p["A"] = -torch.arange(1, N + 1, device="cuda", dtype=torch.float32).repeat(D, 1).contiguous()
    p["Dk"] = 0.5 + torch.rand(D, generator=g, device="cuda")
    torch.cuda.synchronize()
    yield p
    p.clear()
    torch.cuda.empty_cache()


def _host(p, ds):
    """The sampled channels' inputs as float64 host arrays (the exact bf16 values)."""
    f = lambda t: t.float().cpu().numpy().astype(np.float64)   # noqa: E731
    idx = torch.tensor(ds, device="cuda")
    return dict(u=f(p["u"].index_select(2, idx)), delta=f(p["delta"].index_select(2, idx)),
                z=f(p["z"].index_select(2, idx)), B=f(p["B"]), C=f(p["C"]),
                A=f(p["A"][ds]), D=f(p["Dk"][ds]), bias=f(p["bias"][ds]))


def test_huge_forward_and_reverse(oracle, problem):
    p = problem
    log("huge forward: B=%d L=%d D=%d (%.2e elements per tensor)" % (Bt, L, D, Bt * L * D))
    y = B.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["Dk"], delta_bias=p["bias"],
                   z=p["z"], disc="zoh")
    torch.cuda.synchronize()
    ys = y[:, :, SAMPLE].cpu().numpy()
    # the reverse-time scan added into the same output (the bidirectional form)
    B.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["Dk"], delta_bias=p["bias"],
               z=p["z"], disc="zoh", reverse=True, y=y)
    torch.cuda.synchronize()
    yb = y[:, :, SAMPLE].cpu().numpy()
    assert bool(torch.isfinite(y).all())
    del y
    torch.cuda.empty_cache()
    h = _host(p, SAMPLE)
    ref, _ = oracle.fwd(h["u"], h["delta"], h["A"], h["B"], h["C"], D=h["D"],
                        delta_bias=h["bias"], z=h["z"])
    check_rel_max(ys, ref, TOL_BF16, "forward")
    rev, _ = oracle.fwd_reverse(h["u"], h["delta"], h["A"], h["B"], h["C"], D=h["D"],
                                delta_bias=h["bias"], z=h["z"])
    check_rel_max(yb, ref + rev, TOL_BF16, "forward + reverse")


def test_huge_backward(oracle, problem):
    p = problem
    log("huge backward")
    g = torch.Generator(device="cuda").manual_seed(8129)
    dy = torch.randn((Bt, L, D), generator=g, device="cuda").to(torch.bfloat16)
    gr = B.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], dy, D=p["Dk"],
                    delta_bias=p["bias"], z=p["z"], disc="zoh")
    torch.cuda.synchronize()
    idx = torch.tensor(SAMPLE, device="cuda")
    got = {k: gr[k].index_select(2, idx).cpu().numpy() for k in ("du", "ddelta", "dz")}
    got["dA"] = gr["dA"][SAMPLE].cpu().numpy()
    got["dD"] = gr["dD"][SAMPLE].cpu().numpy()
    got["ddelta_bias"] = gr["ddelta_bias"][SAMPLE].cpu().numpy()
    for k in ("dB", "dC"):
        assert bool(torch.isfinite(gr[k]).all()), k
    dys = dy.index_select(2, idx).float().cpu().numpy().astype(np.float64)
    del gr, dy
    torch.cuda.empty_cache()
    h = _host(p, SAMPLE)
    ref = oracle.bwd(h["u"], h["delta"], h["A"], h["B"], h["C"], D=h["D"], delta_bias=h["bias"],
                     z=h["z"], g=dys, disc="zoh")
    for k, v in got.items():
        check_rel_max(v, ref[k], TOL_GRAD, k)


def test_huge_conv1d(oracle, problem):
    """The causal Conv1d + SiLU over the same 2.4e9-element input (width 4)."""
    p = problem
    g = torch.Generator(device="cuda").manual_seed(8130)
    w = torch.randn((D, 4), generator=g, device="cuda")
    bias = torch.randn(D, generator=g, device="cuda")
    u = B.conv1d_fwd(p["u"], w, bias, silu=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = u[:, :, SAMPLE].cpu().numpy()
    del u
    torch.cuda.empty_cache()
    idx = torch.tensor(SAMPLE, device="cuda")
    x = p["u"].index_select(2, idx).float().cpu().numpy()
    ref = oracle.conv1d_fwd(x, w[SAMPLE].cpu().numpy(), bias[SAMPLE].cpu().numpy())
    check_rel_max(got, ref, 1e-5, "conv1d")


def test_huge_ssd(oracle, problem):
    """The SSD layer with x of 2.7e9 elements (B = 1, L = 2^20, 40 heads of 64,
    64 states): one sampled head against the oracle's sequential layer."""
    Bs, Ls, H, P, Ns = 1, 1 << 20, 40, 64, 64
    assert Bs * Ls * H * P > (1 << 31)
    g = torch.Generator(device="cuda").manual_seed(8131)
    bf = torch.bfloat16
    x = torch.randn((Bs, Ls, H, P), generator=g, device="cuda").to(bf)
    dt = (0.1 * torch.randn((Bs, Ls, H), generator=g, device="cuda")).to(bf)
    Bm = torch.randn((Bs, Ls, 1, Ns), generator=g, device="cuda").to(bf)
    Cm = torch.randn((Bs, Ls, 1, Ns), generator=g, device="cuda").to(bf)
    A = -(1.0 + 15.0 * torch.rand(H, generator=g, device="cuda"))
    Dh = 0.5 + torch.rand(H, generator=g, device="cuda")
    lo, hi = np.log(1e-3), np.log(1e-1)
    step = torch.exp(lo + (hi - lo) * torch.rand(H, generator=g, device="cuda"))
    bias = (step + torch.log(-torch.expm1(-step))).float()
    y = B.ssd_fwd(x, dt, A, Bm, Cm, D=Dh, dt_bias=bias)
    torch.cuda.synchronize()
    hh = H - 1
    got = y[:, :, hh:hh + 1].cpu().numpy()
    f = lambda t: t.float().cpu().numpy()   # noqa: E731
    xs, dts, Bh, Ch = f(x[:, :, hh:hh + 1]), f(dt[:, :, hh:hh + 1]), f(Bm), f(Cm)
    del y, x, dt, Bm, Cm
    torch.cuda.empty_cache()
    ref = oracle.ssd_fwd(xs, dts, f(A[hh:hh + 1]), Bh, Ch, D=f(Dh[hh:hh + 1]),
                      dt_bias=f(bias[hh:hh + 1]))
    check_rel_max(got, ref, 2e-5, "ssd")
