"""Tensors past 2^31 elements: B = 1, L = 2^20, D = 2304 (2.4e9 elements per
(B, L, D) tensor, bf16 inputs, N = 16, exact ZOH), so every element index and
byte offset of a whole tensor needs more than 32 bits.  The forward, the
reverse-time scan accumulated into it, and the backward run on the whole
problem; sampled channels (the first, one inside, the last) are checked against
the fp64 oracle on the same bits, which depends on a channel's own inputs and
the shared B, C rows only.  Inputs are drawn on the GPU from a seeded generator
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
