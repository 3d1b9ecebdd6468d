"""GPU parity of the complex-A forward (ss_scan_fwd_complex) against the fp64
oracle on the same bits.  Marked gpu: run on an MI355X."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd import synth
from gpu_util import TOL_BF16, check_f32, check_rel_max, log, oracle_threads

pytestmark = pytest.mark.gpu


def _up(inp):
    it = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    cv = lambda x, dt: None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(dt).contiguous()  # noqa
    f32 = torch.float32
    return dict(u=cv(inp.u, it), delta=cv(inp.delta, it), A=cv(inp.A, f32), B=cv(inp.B, it),
                C=cv(inp.C, it), D=cv(inp.D, f32), delta_bias=cv(inp.delta_bias, f32),
                z=cv(inp.z, it), h0=cv(inp.h0, f32))


def _gpu(d, disc, softplus=True, out_dtype=torch.float32, last=True):
    return B.scan_fwd_complex(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                              delta_bias=d["delta_bias"], z=d["z"], h0=d["h0"], disc=disc,
                              softplus=softplus, out_dtype=out_dtype, return_last_state=last)


def _ref(oracle, inp, disc, softplus=True):
    return oracle.fwd_complex(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D,
                              delta_bias=inp.delta_bias, z=inp.z, h0=inp.h0, disc=disc,
                              softplus=softplus)


CASES = [
    # (B, L, D, N, disc, a_mode, dtype, h0)
    (2, 100, 64, 16, "zoh", "s4d_lin", "f32", True),
    (2, 77, 150, 16, "euler", "random", "f32", True),
    (1, 45, 70, 5, "zoh", "mixed", "f32", False),
    (3, 33, 100, 7, "zoh", "random", "bf16", True),
    (2, 9, 64, 16, "euler", "s4d_lin", "bf16", False),
    (1, 200, 40, 1, "zoh", "random", "f32", True),
    (2, 1, 30, 16, "zoh", "s4d_lin", "f32", True),
    (2, 100, 40, 16, "zoh", "weak", "f32", True),
    (1, 64, 33, 9, "euler", "weak", "f32", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_d%d_n%d_%s_%s_%s_%d" % c)
def test_complex_parity(oracle, case):
    Bt, L, D, N, disc, amode, dt, h0 = case
    log("complex case", case)
    inp = synth.make_complex_inputs(Bt, L, D, N, seed=3000 + CASES.index(case), dtype=dt,
                                    a_mode=amode, with_h0=h0)
    y, hl = _gpu(_up(inp), disc)
    torch.cuda.synchronize()
    ref, href = _ref(oracle, inp, disc)
    w = check_f32(y.cpu().numpy(), ref, "y")
    hg = hl.cpu().numpy().astype(np.float64)
    check_f32(hg[..., 0], href.real, "h_last re")
    check_f32(hg[..., 1], href.imag, "h_last im")
    log("  worst err/bound", w)


def test_complex_no_softplus_no_gate(oracle):
    inp = synth.make_complex_inputs(2, 64, 96, 16, seed=3100, with_z=False)
    inp.delta = np.abs(inp.delta).astype(np.float32) * np.float32(0.3)   # plain steps > 0
    inp.delta_bias = None
    d = _up(inp)
    y = _gpu(d, "zoh", softplus=False, last=False)
    torch.cuda.synchronize()
    ref, _ = _ref(oracle, inp, "zoh", softplus=False)
    check_f32(y.cpu().numpy(), ref, "y")


def test_complex_bf16_output(oracle):
    inp = synth.make_complex_inputs(2, 90, 64, 16, seed=3110, dtype="bf16")
    y = _gpu(_up(inp), "zoh", out_dtype=torch.bfloat16, last=False)
    torch.cuda.synchronize()
    ref, _ = _ref(oracle, inp, "zoh")
    got = y.float().cpu().numpy().astype(np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + TOL_BF16 * np.abs(ref).max()
    assert np.all(np.abs(got - ref) <= bound), float((np.abs(got - ref) / bound).max())


def test_complex_full_size(oracle):
    """Mamba-2.8B-shaped layer (B=8, L=2048, D=5120, N=16, bf16) with the S4D-Lin
    A; every element of y against the oracle."""
    Bt, L, D, N = 8, 2048, 5120, 16
    log("complex full size")
    inp = synth.make_complex_inputs(Bt, L, D, N, seed=3120, dtype="bf16")
    y = _gpu(_up(inp), "zoh", last=False)
    torch.cuda.synchronize()
    ref, _ = oracle.fwd_complex(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D,
                                delta_bias=inp.delta_bias, z=inp.z, nthreads=oracle_threads())
    r = check_rel_max(y.cpu().numpy(), ref, TOL_BF16, "complex full size")
    log("  max err / max|ref| =", r)


# (SS_SCAN_CHUNK): time chunks of the chunked complex plan, and one pass ("100000")
CHUNKED = [
    # (B, L, D, N, disc, a_mode, dtype, h0, chunk)
    (2, 3000, 64, 16, "zoh", "s4d_lin", "f32", True, "256"),
    (1, 3001, 40, 16, "zoh", "random", "f32", True, "128"),
    (2, 2000, 70, 9, "euler", "random", "f32", False, "336"),
    (1, 1500, 96, 16, "zoh", "mixed", "f32", True, "144"),
    (2, 700, 40, 16, "zoh", "weak", "f32", True, "128"),
    (2, 2500, 100, 13, "zoh", "random", "bf16", True, "256"),
    (1, 3000, 64, 16, "zoh", "s4d_lin", "f32", True, "100000"),
]


@pytest.mark.parametrize("case", CHUNKED, ids=lambda c: "b%d_l%d_d%d_n%d_%s_%s_%s_h0%d_chunk%s" % c)
def test_complex_chunked(oracle, monkeypatch, case):
    """The chunked complex plan (summary pass, fp64 step sums, in-order carry
    walk, output pass from each chunk's start state) against the oracle: y and
    the state after the last step, ragged last chunks, with and without h0."""
    Bt, L, D, N, disc, amode, dt, h0, chunk = case
    log("complex chunked", case)
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    inp = synth.make_complex_inputs(Bt, L, D, N, seed=3300 + CHUNKED.index(case), dtype=dt,
                                    a_mode=amode, with_h0=h0)
    y, hl = _gpu(_up(inp), disc)
    torch.cuda.synchronize()
    ref, href = _ref(oracle, inp, disc)
    w = check_f32(y.cpu().numpy(), ref, "y")
    hg = hl.cpu().numpy().astype(np.float64)
    check_f32(hg[..., 0], href.real, "h_last re")
    check_f32(hg[..., 1], href.imag, "h_last im")
    log("  worst err/bound", w)


def test_complex_chunked_equals_one_pass(monkeypatch):
    """Chunked and one-pass complex scans agree on fp32 inputs (the precise step
    on both sides; chunk maps exp(a sum dt) instead of the product of per-step
    factors: fp32 reassociation only)."""
    inp = synth.make_complex_inputs(2, 2500, 64, 16, seed=3350, dtype="f32", a_mode="random",
                                    with_h0=True)
    d = _up(inp)
    monkeypatch.setenv("SS_SCAN_CHUNK", "100000")
    y1, h1 = _gpu(d, "zoh")
    for chunk in ("128", "400", "1000"):
        monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
        y2, h2 = _gpu(d, "zoh")
        torch.cuda.synchronize()
        assert float((y1 - y2).abs().max()) <= 1e-5 * float(y1.abs().max()), chunk
        assert float((h1 - h2).abs().max()) <= 1e-5 * float(h1.abs().max()), chunk


def test_complex_long_full_size(oracle):
    """The million-step shape (B=1, L=2^20, D=256, N=16 complex, bf16, S4D-Lin A,
    steps in [1e-4, 1e-2]) on the planner's chunked layout; every element of y
    against the oracle (max|y - y_ref| <= 2e-3 max|y_ref|)."""
    Bt, L, D, N = 1, 1 << 20, 256, 16
    log("complex long full size")
    inp = synth.make_complex_inputs(Bt, L, D, N, seed=3360, dtype="bf16", dt_range=(1e-4, 1e-2))
    desc = B.make_desc(Bt, L, D, N, B.SS_BF16, B.SS_F32, B.SS_ZOH, True)
    assert B.ss_scan_workspace_bytes(desc, B.SS_OP_FWD_COMPLEX) > 0, "expected a chunked plan"
    y = _gpu(_up(inp), "zoh", last=False)
    torch.cuda.synchronize()
    log("  oracle on every channel")
    ref, _ = oracle.fwd_complex(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D,
                                delta_bias=inp.delta_bias, z=inp.z, nthreads=oracle_threads())
    r = check_rel_max(y.cpu().numpy(), ref, TOL_BF16, "complex long")
    log("  max err / max|ref| =", r)


def test_complex_deterministic():
    inp = synth.make_complex_inputs(2, 300, 200, 16, seed=3130, dtype="bf16")
    d = _up(inp)
    y1 = _gpu(d, "zoh", last=False)
    y2 = _gpu(d, "zoh", last=False)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ---------------------------------------------------------------- decode step
STEP_CASES = [
    # (B, D, N, disc, a_mode, dtype)
    (3, 100, 16, "zoh", "s4d_lin", "f32"),
    (2, 70, 5, "zoh", "mixed", "f32"),
    (2, 64, 16, "euler", "random", "bf16"),
    (1, 33, 9, "zoh", "weak", "bf16"),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "b%d_d%d_n%d_%s_%s_%s" % c)
def test_complex_step_parity(oracle, case):
    """ss_scan_step_complex from a random state against the oracle's complex
    scan over one step from that state: y and the new state."""
    Bt, D, N, disc, amode, dt = case
    log("complex step case", case)
    inp = synth.make_complex_inputs(Bt, 1, D, N, seed=3200 + STEP_CASES.index(case), dtype=dt,
                                    a_mode=amode, with_h0=True)
    d = _up(inp)
    h = d["h0"].clone()
    y = B.scan_step_complex(h, d["u"][:, 0].contiguous(), d["delta"][:, 0].contiguous(), d["A"],
                            d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), D=d["D"],
                            delta_bias=d["delta_bias"], z=d["z"][:, 0].contiguous(), disc=disc)
    torch.cuda.synchronize()
    ref, href = _ref(oracle, inp, disc)
    check_f32(y.cpu().numpy(), ref[:, 0], "complex step y")
    hc = h.cpu().numpy().astype(np.float64)
    check_f32(hc[..., 0], href.real, "complex step h re")
    check_f32(hc[..., 1], href.imag, "complex step h im")


def test_complex_step_continues_scan(oracle):
    """A scan over 60 steps keeping h_last, then 4 decode steps: y of every
    step and the final state against the oracle's scan over all 64."""
    Bt, L, D, N, k = 2, 64, 96, 16, 4
    inp = synth.make_complex_inputs(Bt, L, D, N, seed=3250, dtype="bf16", with_h0=True)
    d = _up(inp)
    pre = {n: (d[n][:, :L - k].contiguous() if n in ("u", "delta", "B", "C", "z") else d[n])
           for n in d}
    y0, h = _gpu(pre, "zoh")
    ys = [y0]
    for t in range(L - k, L):
        ys.append(B.scan_step_complex(h, d["u"][:, t].contiguous(), d["delta"][:, t].contiguous(),
                                      d["A"], d["B"][:, t].contiguous(), d["C"][:, t].contiguous(),
                                      D=d["D"], delta_bias=d["delta_bias"],
                                      z=d["z"][:, t].contiguous())[:, None])
    torch.cuda.synchronize()
    ref, href = _ref(oracle, inp, "zoh")
    check_f32(torch.cat(ys, dim=1).cpu().numpy(), ref, "complex scan + steps y")
    hc = h.cpu().numpy().astype(np.float64)
    check_f32(hc[..., 0], href.real, "complex scan + steps h re")
    check_f32(hc[..., 1], href.imag, "complex scan + steps h im")
