"""GPU parity of the forward scan and the decode step against the fp64 oracle,
through the C ABI (libssscan.so).  Marked gpu: run on an MI355X."""
import os

import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd import synth
from gpu_util import (TOL_BF16, check_f32, check_rel_max, full_compare_bf16, gpu_fwd, log,
                      upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    B.load_library()
    yield
    torch.cuda.synchronize()


def _full_oracle(oracle, inp, disc, softplus=True):
    return oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                      z=inp.z, h0=inp.h0, disc=disc, softplus=softplus)


# ------------------------------------------------------------------ small fp32 cases
CASES = [
    # (B, L, D, N, disc, z, bias, Dskip, h0, softplus, a_mode)
    (1, 256, 64, 16, "zoh", True, True, True, False, True, "s4d_real"),
    (2, 77, 150, 16, "zoh", True, True, True, True, True, "random"),
    (2, 77, 150, 16, "euler", True, True, True, True, True, "random"),
    (3, 45, 64, 16, "zoh", False, True, False, False, True, "s4d_real"),
    (2, 64, 70, 16, "euler", False, False, True, True, True, "s4d_real"),
    (2, 33, 100, 16, "zoh", True, True, True, True, True, "mixed"),
    (2, 33, 100, 16, "euler", True, True, True, True, True, "mixed"),
    (1, 19, 5, 16, "zoh", True, True, True, True, False, "s4d_real"),
    (2, 40, 66, 1, "zoh", True, True, True, True, True, "random"),
    (2, 40, 66, 5, "euler", True, True, True, True, True, "random"),
    (1, 50, 130, 8, "zoh", True, False, True, True, True, "mixed"),
    (1, 1, 64, 16, "zoh", True, True, True, True, True, "random"),
    (2, 1000, 150, 16, "zoh", True, True, True, True, True, "random"),     # chunked plan
    (2, 1000, 150, 16, "euler", True, True, True, True, True, "mixed"),    # chunked, A = 0
    (1, 3001, 64, 16, "zoh", True, True, True, True, True, "s4d_real"),    # chunked, ragged
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_d%d_n%d_%s_z%d_bias%d_D%d_h0%d_sp%d_%s" % c)
def test_fwd_fp32_parity(oracle, case):
    Bt, L, D, N, disc, z, bias, dsk, h0, sp, amode = case
    log("fwd fp32 case", case)
    inp = synth.make_inputs(Bt, L, D, N, seed=1000 + CASES.index(case), dtype="f32", with_z=z,
                            with_bias=bias, with_D=dsk, with_h0=h0, a_mode=amode,
                            delta_std=0.1 if sp else 0.02)
    if not sp:   # keep the raw step positive without the activation
        inp.delta_bias = np.abs(inp.delta_bias) * 0 + np.float32(0.05)
    d = upload(inp)
    y, hl = gpu_fwd(d, disc, softplus=sp, return_last_state=True)
    torch.cuda.synchronize()
    ref, href = _full_oracle(oracle, inp, disc, softplus=sp)
    w = check_f32(y.cpu().numpy(), ref, "y")
    check_f32(hl.cpu().numpy(), href, "h_last")
    log("  worst err/bound", w)


SPLIT_CASES = [
    (2, 150, 150, 16, "zoh", "mixed", "f32"), (2, 150, 150, 16, "euler", "random", "f32"),
    (1, 300, 64, 5, "zoh", "random", "f32"), (3, 61, 130, 16, "zoh", "s4d_real", "f32"),
    (2, 203, 100, 16, "zoh", "random", "bf16"), (1, 77, 40, 7, "euler", "mixed", "bf16"),
    # slowly decaying states (|A| down to 1e-4): exact ZOH's guarded coefficient
    (2, 150, 150, 16, "zoh", "weak", "f32"), (1, 203, 100, 13, "zoh", "weak", "bf16"),
    (2, 77, 70, 16, "euler", "weak", "f32"),
    # every |A| >= 0.25 with positive entries: the scaled exact-ZOH states with A[0] > 0
    (2, 61, 150, 16, "zoh", "grow", "f32"), (1, 77, 100, 16, "zoh", "grow", "bf16"),
]


@pytest.mark.parametrize("nsplit", ["1", "2", "4", "8", "16"])
@pytest.mark.parametrize("chunk", ["0", "48"])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "b%d_l%d_d%d_n%d_%s_%s_%s" % c)
def test_fwd_split_variants(oracle, monkeypatch, nsplit, chunk, case):
    """Every kernel layout (64-channel groups with 1, 2 or 4 waves over the
    states; "8" = 32-channel groups, two states per lane; "16" = 16-channel
    groups, one state per lane), with and without time chunks, against the
    oracle."""
    Bt, L, D, N, disc, amode, dt = case
    log("split case", nsplit, chunk, case)
    monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    inp = synth.make_inputs(Bt, L, D, N, seed=2000 + SPLIT_CASES.index(case), dtype=dt,
                            with_h0=True, a_mode=amode)
    d = upload(inp)
    y, hl = gpu_fwd(d, disc, return_last_state=True)
    torch.cuda.synchronize()
    ref, href = _full_oracle(oracle, inp, disc)
    # bf16 inputs reach both sides as the same bits, so the fp32 bound applies
    check_f32(y.cpu().numpy(), ref, "y")
    check_f32(hl.cpu().numpy(), href, "h_last")


def test_fwd_tiny_workload(oracle):
    """The tiny fp32 workload (B=1, L=256, D=64, N=16, exact ZOH, gate)."""
    inp = synth.make_workload("fwd_tiny_f32_b1_l256_d64")
    d = upload(inp)
    y = gpu_fwd(d, "zoh")
    torch.cuda.synchronize()
    ref, _ = _full_oracle(oracle, inp, "zoh")
    check_f32(y.cpu().numpy(), ref, "y")


def test_chunked_equals_sequential(monkeypatch):
    """The chunked two-level carry reproduces the one-pass result (fp32 reassociation)."""
    inp = synth.make_inputs(2, 1500, 96, 16, seed=5, dtype="f32", with_h0=True, a_mode="random")
    d = upload(inp)
    monkeypatch.setenv("SS_SCAN_CHUNK", "100000")
    y1, h1 = gpu_fwd(d, "zoh", return_last_state=True)
    for chunk in ("64", "256", "333"):
        monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
        y2, h2 = gpu_fwd(d, "zoh", return_last_state=True)
        torch.cuda.synchronize()
        # chunk decays are exp(A * sum dt) instead of a product of per-step exps
        scale = float(y1.abs().max())
        assert float((y1 - y2).abs().max()) <= 1e-4 * scale, chunk
        assert float((h1 - h2).abs().max()) <= 1e-4 * float(h1.abs().max()), chunk


# (SS_SCAN_CHUNK, SS_SCAN_NSPLIT): >= 256 chunks (lane-parallel carries) on the
# 64-, 32- and 16-channel layouts, one pass on each, and the planner's choice
LONG_LAYOUTS = [("16", "4"), ("40", "8"), ("100000", "8"), ("100000", "1"), ("48", "16"),
                ("100000", "16"), ("0", "0")]


@pytest.mark.parametrize("dt_range", [(1e-3, 1e-1), (1e-4, 1e-2)], ids=["dt1e-3", "dt1e-4"])
@pytest.mark.parametrize("amode", ["s4d_real", "random", "weak"])
@pytest.mark.parametrize("layout", LONG_LAYOUTS, ids=lambda v: "chunk%s_split%s" % v)
def test_fwd_long_fp32(oracle, monkeypatch, layout, amode, dt_range):
    """10,250 fp32 steps (memory up to 1 / |dt A| ~ 10^6 steps with weak A and
    small steps) on every layout, with and without >= 256 time chunks, at the
    elementwise fp32 bound."""
    chunk, nsplit = layout
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    if nsplit != "0":
        monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    seed = 14 + 10 * ["s4d_real", "random", "weak"].index(amode) + (dt_range[0] < 5e-4)
    inp = synth.make_inputs(2, 10250, 40, 16, seed=seed, dtype="f32", with_h0=True,
                            a_mode=amode, dt_range=dt_range)
    d = upload(inp)
    log("long fp32", layout, amode, dt_range)
    y, hl = gpu_fwd(d, "zoh", return_last_state=True)
    torch.cuda.synchronize()
    ref, href = _full_oracle(oracle, inp, "zoh")
    w = check_f32(y.cpu().numpy(), ref, "y")
    check_f32(hl.cpu().numpy(), href, "h_last")
    log("  worst err/bound", w)


# (SS_SCAN_CHUNK, SS_SCAN_NSPLIT) for the time-invariant cases
LTI_LAYOUTS = [("0", "8"), ("256", "8"), ("0", "1"), ("0", "2"), ("256", "4"), ("0", "16"),
               ("256", "16"), ("0", "0")]


@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("arange", [(0.25, 1.0, False), (1e-3, 0.25, True)],
                         ids=["A0.25to1", "Aweak"])
@pytest.mark.parametrize("layout", LTI_LAYOUTS, ids=lambda v: "chunk%s_split%s" % v)
def test_fwd_lti_one_signed_fp32(oracle, monkeypatch, layout, arange, disc):
    """Constant step, B and C, input of one sign, steps of 1e-4 to 1e-3 over
    16,384 steps: rounding errors of the decay and of the input coefficient
    cannot average out here, and the memory (1 / |dt A| up to 4e4 steps with
    |A| >= 0.25, 1e6 with weak A) spans the whole run.  Elementwise fp32 bound."""
    chunk, nsplit = layout
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    if nsplit != "0":
        monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    lo, hi, lg = arange
    inp = synth.make_lti_inputs(1, 16384, 64, 16, seed=40 + int(lg), dtype="f32",
                                a_range=(lo, hi), a_log=lg)
    d = upload(inp)
    log("lti fp32", layout, arange, disc)
    y, hl = gpu_fwd(d, disc, return_last_state=True)
    torch.cuda.synchronize()
    ref, href = _full_oracle(oracle, inp, disc)
    w = check_f32(y.cpu().numpy(), ref, "y")
    check_f32(hl.cpu().numpy(), href, "h_last")
    log("  worst err/bound", w)


@pytest.mark.parametrize("reverse", [False, True])
def test_fwd_lti_one_signed_bf16(oracle, reverse):
    """The time-invariant one-signed case with bf16 inputs on the planner's
    layout (both directions): the bf16 bound, max|y - y_ref| <= 2e-3 max|y_ref|."""
    inp = synth.make_lti_inputs(2, 16384, 256, 16, seed=42, dtype="bf16")
    d = upload(inp)
    y = B.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                   delta_bias=d["delta_bias"], disc="zoh", reverse=reverse)
    torch.cuda.synchronize()
    fn = oracle.fwd_reverse if reverse else oracle.fwd
    ref, _ = fn(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                disc="zoh")
    r = check_rel_max(y.cpu().numpy(), ref, TOL_BF16, "lti bf16")
    log("  max err / max|ref| =", r)


@pytest.mark.parametrize("nsplit", ["8", "4", "1", "16"])
def test_fwd_tiny_steps_relative(oracle, monkeypatch, nsplit):
    """Steps of softplus(-20) ~ 2e-9 (and smaller): the state they build from
    a zero start keeps full relative accuracy (elementwise 1e-5 relative on
    h_last, far below any absolute floor).  u and B are made one-signed so
    that the state is a sum without cancellation and a relative bound holds."""
    monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    monkeypatch.setenv("SS_SCAN_CHUNK", "0")
    inp = synth.make_inputs(2, 24, 64, 16, seed=44, dtype="f32", a_mode="random")
    inp.u = np.abs(inp.u)
    inp.B = np.abs(inp.B)
    inp.delta = np.full_like(inp.delta, -20.0) - inp.delta_bias[None, None, :]
    inp.delta[:, ::3] -= 6.0                  # some steps of softplus(-26) ~ 5e-12
    d = upload(inp)
    y, hl = gpu_fwd(d, "zoh", return_last_state=True)
    torch.cuda.synchronize()
    ref, href = _full_oracle(oracle, inp, "zoh")
    got = hl.double().cpu().numpy()
    rel = np.abs(got - href) / np.abs(href)
    assert float(rel.max()) <= 1e-5, float(rel.max())
    check_f32(y.cpu().numpy(), ref, "y")


# "0": the planner's choice; the others force a layout (SS_SCAN_NSPLIT)
LAYOUTS = ["0", "4", "8", "16"]


@pytest.mark.parametrize("nsplit", LAYOUTS)
def test_fwd_deterministic(monkeypatch, nsplit):
    if nsplit != "0":
        monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    inp = synth.make_inputs(4, 512, 320, 16, seed=6, dtype="bf16")
    d = upload(inp)
    y1 = gpu_fwd(d, "zoh")
    y2 = gpu_fwd(d, "zoh")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("nsplit", LAYOUTS)
def test_fwd_split_resume(monkeypatch, nsplit):
    """fwd(L1) -> h_last -> fwd(L2, h0 = h_last) equals fwd(L1 + L2)."""
    if nsplit != "0":
        monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    inp = synth.make_inputs(2, 300, 128, 16, seed=7, dtype="f32", with_h0=True, a_mode="random")
    d = upload(inp)
    y, h = gpu_fwd(d, "zoh", return_last_state=True)
    cut = 123
    part = lambda k, s: d[k][:, s].contiguous()  # noqa: E731
    y1, h1 = gpu_fwd(d, "zoh", return_last_state=True,
                     **{k: part(k, slice(0, cut)) for k in ("u", "delta", "z", "B", "C")})
    y2, h2 = gpu_fwd(d, "zoh", return_last_state=True, h0=h1,
                     **{k: part(k, slice(cut, None)) for k in ("u", "delta", "z", "B", "C")})
    torch.cuda.synchronize()
    yy = torch.cat([y1, y2], dim=1)
    assert float((yy - y).abs().max()) <= 1e-5 * (1 + float(y.abs().max()))
    assert float((h2 - h).abs().max()) <= 1e-5 * (1 + float(h.abs().max()))


@pytest.mark.parametrize("nsplit", LAYOUTS)
def test_fwd_bf16_output(oracle, monkeypatch, nsplit):
    if nsplit != "0":
        monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    inp = synth.make_inputs(2, 200, 192, 16, seed=8, dtype="bf16")
    d = upload(inp)
    y = gpu_fwd(d, "zoh", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, _ = _full_oracle(oracle, inp, "zoh")
    # bf16 storage adds at most 2^-9 relative rounding on top of the fp32 result
    check_rel_max(y.float().cpu().numpy(), ref, TOL_BF16 + 2.0 ** -8, "y bf16")


# (B, L, D, N): a single step, one partial block, a block and a step, ragged D
EDGE_SHAPES = [(1, 1, 1, 16), (2, 5, 17, 16), (1, 17, 16, 16), (2, 33, 33, 7)]


@pytest.mark.parametrize("reverse", [False, True], ids=["fwd", "rev"])
@pytest.mark.parametrize("chunk", ["0", "40", "7"])
@pytest.mark.parametrize("nsplit", ["4", "8", "16"])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda v: "b%d_l%d_d%d_n%d" % v)
def test_fwd_layout_edges(oracle, monkeypatch, shape, nsplit, chunk, reverse):
    """Edge shapes on every forced layout: L shorter than one block, chunk
    lengths that are not a multiple of a block (7: more chunks than blocks),
    D below one channel group, both time directions; fp32 at the elementwise
    bound, y and the final state."""
    Bt, L, D, N = shape
    monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    inp = synth.make_inputs(Bt, L, D, N, seed=4000 + EDGE_SHAPES.index(shape), dtype="f32",
                            with_h0=True, a_mode="random")
    d = upload(inp)
    y, hl = B.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                       delta_bias=d["delta_bias"], z=d["z"], h0=d["h0"], disc="zoh",
                       return_last_state=True, reverse=reverse)
    torch.cuda.synchronize()
    fn = oracle.fwd_reverse if reverse else oracle.fwd
    ref, href = fn(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                   z=inp.z, h0=inp.h0, disc="zoh")
    check_f32(y.cpu().numpy(), ref, "y")
    check_f32(hl.cpu().numpy(), href, "h_last")


# ------------------------------------------------------------------ full-size workloads
# (workload, discretisation): every full-size forward workload in its own
# discretisation, plus the Mamba-2.8B shape with Euler B_bar (also measured)
FULL = [("fwd_130m_bf16_b8_l2048_d1536", None), ("fwd_2p8b_bf16_b8_l2048_d5120", None),
        ("fwd_2p8b_bf16_b8_l2048_d5120", "euler"), ("fwd_2p8b_bf16_b2_l8192_d5120", None),
        ("fwd_long_bf16_b1_l1048576_d256", None)]


@pytest.mark.parametrize("name,disc", FULL, ids=lambda v: str(v))
def test_fwd_full_size(oracle, name, disc):
    """Full-size bf16 workloads in the benchmark's launch configuration, every
    element of y against the fp64 oracle (max|y - y_ref| <= 2e-3 max|y_ref|)."""
    w = synth.WORKLOADS[name]
    disc = disc or w.disc
    log("full-size fwd", name, disc, "generating inputs")
    inp = synth.make_workload(name)
    d = upload(inp)
    log("  running GPU")
    y = gpu_fwd(d, disc)
    torch.cuda.synchronize()
    del d
    log("  oracle on every channel")
    r = full_compare_bf16(oracle, inp, y, disc, block=64 if w.L > 100000 else None, what=name)
    log("  max err / max|ref| =", r)


# ------------------------------------------------------------------ decode step
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("N", [16, 5, 13])
@pytest.mark.parametrize("amode", ["mixed", "weak"])
def test_step_parity(oracle, dtype, disc, N, amode):
    log("step case", dtype, disc, N, amode)
    inp = synth.make_inputs(3, 1, 200, N, seed=9, dtype=dtype, with_h0=True, a_mode=amode)
    d = upload(inp)
    h = d["h0"].clone()
    y = B.scan_step(h, d["u"][:, 0].contiguous(), d["delta"][:, 0].contiguous(), d["A"],
                    d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), D=d["D"],
                    delta_bias=d["delta_bias"], z=d["z"][:, 0].contiguous(), disc=disc)
    torch.cuda.synchronize()
    ref_y, ref_h = oracle.step(inp.h0, inp.u[:, 0], inp.delta[:, 0], inp.A, inp.B[:, 0],
                               inp.C[:, 0], D=inp.D, delta_bias=inp.delta_bias, z=inp.z[:, 0],
                               disc=disc)
    check_f32(y.cpu().numpy(), ref_y, "step y")
    check_f32(h.cpu().numpy(), ref_h, "step h")


def test_step_graph_replay():
    """A decode loop of 4 steps captured in a graph: every replay (state reset by
    an eager copy between replays) equals the eager loop bit for bit."""
    inp = synth.make_inputs(2, 4, 192, 16, seed=12, dtype="bf16", with_h0=True, a_mode="random")
    d = upload(inp)
    steps = [{k: d[k][:, t].contiguous() for k in ("u", "delta", "B", "C", "z")} for t in range(4)]
    desc = B.make_desc(2, 1, 192, 16, B.SS_BF16, B.SS_F32, B.SS_ZOH, True)
    ys = [torch.empty(2, 192, device="cuda") for _ in range(4)]

    def loop(h):
        for t, s in enumerate(steps):
            rc = B.ss_scan_step(desc, h, s["u"], s["delta"], d["A"], s["B"], s["C"], d["D"],
                                d["delta_bias"], s["z"], ys[t])
            assert rc == 0

    h_eager = d["h0"].clone()
    loop(h_eager)
    torch.cuda.synchronize()
    y_eager = [y.clone() for y in ys]
    h = d["h0"].clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop(h)                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        loop(h)
    for rep in range(3):
        h.copy_(d["h0"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_eager), rep
        for t in range(4):
            assert torch.equal(ys[t], y_eager[t]), (rep, t)


def test_step_continues_forward():
    """fwd over L steps, then one decode step, equals the last row of fwd over L+1."""
    inp = synth.make_inputs(2, 65, 128, 16, seed=10, dtype="f32", with_h0=True, a_mode="random")
    d = upload(inp)
    yfull = gpu_fwd(d, "zoh")
    L = 64
    y, h = gpu_fwd(d, "zoh", return_last_state=True,
                   **{k: d[k][:, :L].contiguous() for k in ("u", "delta", "z", "B", "C")})
    ys = B.scan_step(h, d["u"][:, L].contiguous(), d["delta"][:, L].contiguous(), d["A"],
                     d["B"][:, L].contiguous(), d["C"][:, L].contiguous(), D=d["D"],
                     delta_bias=d["delta_bias"], z=d["z"][:, L].contiguous())
    torch.cuda.synchronize()
    assert float((ys - yfull[:, L]).abs().max()) <= 1e-5 * (1 + float(yfull.abs().max()))


def test_errors_do_not_launch():
    """Invalid calls return a status and leave outputs untouched."""
    inp = synth.make_inputs(1, 8, 64, 16, seed=11, dtype="f32")
    d = upload(inp)
    y = torch.full(d["u"].shape, 7.0, device="cuda")
    desc = B.make_desc(1, 8, 64, 17, B.SS_F32, B.SS_F32, B.SS_ZOH)
    rc = B.ss_scan_fwd(desc, d["u"], d["delta"], d["A"], d["B"], d["C"], None, None, None, None,
                       y, None, None, 0)
    assert rc == B.SS_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
