"""GPU parity of the backward scan (with recomputation) against the fp64 oracle,
through the C ABI.  Bound: max|g - g_ref| <= 5e-3 max|g_ref| per gradient tensor."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd import synth
from gpu_util import TOL_GRAD, log, upload

pytestmark = pytest.mark.gpu

KEYS = ["du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz", "dh0"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    B.load_library()
    yield
    torch.cuda.synchronize()


def run_gpu(d, disc, softplus=True, want_dh0=True):
    return B.scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dy"], D=d["D"],
                      delta_bias=d["delta_bias"], z=d["z"], h0=d["h0"], disc=disc,
                      softplus=softplus, want_dh0=want_dh0)


def run_oracle(oracle, inp, disc, softplus=True):
    return oracle.bwd(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                      z=inp.z, h0=inp.h0, g=inp.dy, disc=disc, softplus=softplus)


def compare(g, ref, tol=TOL_GRAD, what=""):
    worst = {}
    for k in KEYS:
        if ref.get(k) is None or g.get(k) is None:
            continue
        got = g[k].double().cpu().numpy()
        r = ref[k]
        assert np.all(np.isfinite(got)), "%s %s: non-finite" % (what, k)
        scale = float(np.abs(r).max())
        err = float(np.abs(got - r).max())
        worst[k] = err / max(scale, 1e-30)
        assert err <= tol * max(scale, 1e-30), "%s %s: max err %.3g > %.1e * max|ref| (%.3g)" % (
            what, k, err, tol, scale)
    return worst


CASES = [
    # (B, L, D, N, disc, z, bias, Dskip, h0, softplus, a_mode)
    (1, 64, 64, 16, "zoh", True, True, True, True, True, "s4d_real"),
    (2, 77, 150, 16, "zoh", True, True, True, True, True, "random"),
    (2, 77, 150, 16, "euler", True, True, True, True, True, "random"),
    (2, 200, 70, 16, "zoh", True, True, True, True, True, "mixed"),
    (2, 200, 70, 16, "euler", False, True, False, False, True, "mixed"),
    (1, 333, 64, 16, "zoh", True, False, True, True, True, "random"),
    (3, 19, 5, 16, "zoh", True, True, True, True, False, "s4d_real"),
    (2, 130, 66, 5, "zoh", True, True, True, True, True, "random"),
    (1, 129, 64, 8, "euler", True, True, True, True, True, "random"),
    (2, 1, 64, 16, "zoh", True, True, True, True, True, "random"),
    # slowly decaying states (|A| down to 1e-4): exact ZOH's guarded coefficient
    # and the series of its derivative
    (2, 200, 70, 16, "zoh", True, True, True, True, True, "weak"),
    (1, 333, 64, 13, "zoh", True, True, True, True, False, "weak"),
    (2, 130, 66, 16, "euler", True, True, True, True, True, "weak"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_d%d_n%d_%s_z%d_bias%d_D%d_h0%d_sp%d_%s" % c)
def test_bwd_fp32_parity(oracle, case):
    Bt, L, D, N, disc, z, bias, dsk, h0, sp, amode = case
    log("bwd fp32 case", case)
    inp = synth.make_inputs(Bt, L, D, N, seed=3000 + CASES.index(case), dtype="f32", with_z=z,
                            with_bias=bias, with_D=dsk, with_h0=h0, with_dy=True, a_mode=amode,
                            delta_std=0.1 if sp else 0.02)
    if not sp:
        inp.delta_bias = np.zeros_like(inp.delta_bias) + np.float32(0.05)
    d = upload(inp)
    g = run_gpu(d, disc, softplus=sp, want_dh0=h0)
    torch.cuda.synchronize()
    ref = run_oracle(oracle, inp, disc, softplus=sp)
    if not h0:
        ref["dh0"] = None
    worst = compare(g, ref, what=str(case))
    log("  worst rel err", {k: "%.2e" % v for k, v in worst.items()})


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bwd_many_chunks(oracle, disc):
    """L = 8230: 258 chunks of 32 steps, so the forward and adjoint carries run
    as the lane-parallel scan (five 64-chunk tiles, the last one ragged)."""
    inp = synth.make_inputs(1, 8230, 70, 16, seed=3100, dtype="f32", with_dy=True, with_h0=True,
                            a_mode="random")
    d = upload(inp)
    log("bwd many chunks", disc)
    g = run_gpu(d, disc)
    torch.cuda.synchronize()
    ref = run_oracle(oracle, inp, disc)
    worst = compare(g, ref, what="many chunks " + disc)
    log("  worst rel err", {k: "%.2e" % v for k, v in worst.items()})


@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("amode", ["random", "weak", "s4d_real"])
def test_bwd_long_small_steps(oracle, disc, amode):
    """10,250 fp32 steps with steps of 1e-4 to 1e-2 (long memory), random, weak
    and S4D-real A: the exact-ZOH derivative of the input coefficient w.r.t. A
    cancels strongly where |dt A| is small."""
    seed = 3200 + ["random", "weak", "s4d_real"].index(amode)
    inp = synth.make_inputs(1, 10250, 64, 16, seed=seed, dtype="f32", with_dy=True,
                            with_h0=True, a_mode=amode, dt_range=(1e-4, 1e-2))
    d = upload(inp)
    log("bwd long small steps", disc, amode)
    g = run_gpu(d, disc)
    torch.cuda.synchronize()
    ref = run_oracle(oracle, inp, disc)
    worst = compare(g, ref, what="long small steps %s %s" % (disc, amode))
    log("  worst rel err", {k: "%.2e" % v for k, v in worst.items()})


def test_bwd_deterministic():
    inp = synth.make_inputs(2, 300, 200, 16, seed=31, dtype="bf16", with_dy=True)
    d = upload(inp)
    g1 = run_gpu(d, "zoh")
    g2 = run_gpu(d, "zoh")
    torch.cuda.synchronize()
    for k in KEYS:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


@pytest.mark.parametrize("disc", ["euler", "zoh"])
def test_bwd_full_size(oracle, disc):
    """Backward at the Mamba-130M shape (B=8, L=2048, D=1536, N=16, bf16 inputs,
    fp32 gradients) against the full fp64 oracle."""
    w = synth.WORKLOADS["bwd_130m_bf16_b8_l2048_d1536"]
    log("full-size bwd", disc, "generating inputs")
    inp = synth.make_workload(w.name, with_dy=True)
    d = upload(inp)
    log("  running GPU")
    g = run_gpu(d, disc, want_dh0=False)
    torch.cuda.synchronize()
    log("  running oracle")
    ref = run_oracle(oracle, inp, disc)
    ref["dh0"] = None
    worst = compare(g, ref, what="full " + disc)
    log("  worst rel err", {k: "%.2e" % v for k, v in worst.items()})
