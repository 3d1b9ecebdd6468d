"""GPU parity of the reverse-time scan and of the bidirectional sum (forward
call, then reverse call accumulating into y), through ss_scan_fwd_dir, against
the oracle's reverse scan (the forward scan of the time-reversed sequence,
reversed back).  Marked gpu: run on an MI355X."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd import synth
from gpu_util import TOL_BF16, check_f32, check_rel_max, log, oracle_threads, upload

pytestmark = pytest.mark.gpu


def _rev_oracle(oracle, inp, disc, A=None, D=None, bias=None):
    return oracle.fwd_reverse(inp.u, inp.delta, inp.A if A is None else A, inp.B, inp.C,
                              D=inp.D if D is None else D,
                              delta_bias=inp.delta_bias if bias is None else bias, z=inp.z,
                              h0=inp.h0, disc=disc)


def _gpu(d, disc, reverse, y=None, A=None, D=None, bias=None, h0=True, out_dtype=torch.float32):
    return B.scan_fwd(d["u"], d["delta"], d["A"] if A is None else A, d["B"], d["C"],
                      D=d["D"] if D is None else D,
                      delta_bias=d["delta_bias"] if bias is None else bias, z=d["z"],
                      h0=d["h0"] if h0 else None, disc=disc, return_last_state=y is None,
                      reverse=reverse, y=y, out_dtype=out_dtype)


CASES = [
    (2, 150, 150, 16, "zoh", "mixed", "f32"), (2, 150, 150, 16, "euler", "random", "f32"),
    (1, 300, 64, 5, "zoh", "random", "f32"), (2, 203, 100, 16, "zoh", "random", "bf16"),
    (1, 77, 40, 7, "euler", "mixed", "bf16"), (2, 9, 70, 16, "zoh", "s4d_real", "f32"),
    (2, 120, 70, 16, "zoh", "weak", "f32"),
]


@pytest.mark.parametrize("nsplit", ["1", "4", "8", "16"])
@pytest.mark.parametrize("chunk", ["0", "48"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_d%d_n%d_%s_%s_%s" % c)
def test_reverse_layouts(oracle, monkeypatch, nsplit, chunk, case):
    """Reverse scan on the 32-channel layout ("8"), the 16-channel layout
    ("16") and the 4-wave 64-channel layout (which also serves plans that would
    use 1 or 2 waves forward), with and without time chunks; y and the state
    after t = 0."""
    Bt, L, D, N, disc, amode, dt = case
    log("reverse case", nsplit, chunk, case)
    monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    inp = synth.make_inputs(Bt, L, D, N, seed=2100 + CASES.index(case), dtype=dt, with_h0=True,
                            a_mode=amode)
    d = upload(inp)
    y, hl = _gpu(d, disc, reverse=True)
    torch.cuda.synchronize()
    ref, href = _rev_oracle(oracle, inp, disc)
    check_f32(y.cpu().numpy(), ref, "y")
    check_f32(hl.cpu().numpy(), href, "h_last")


@pytest.mark.parametrize("nsplit", ["4", "8", "16"])
def test_bidirectional_sum(oracle, monkeypatch, nsplit):
    """Forward call, then reverse call with its own A, D and bias accumulating
    into y: equals the oracle's forward + reverse."""
    monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    monkeypatch.setenv("SS_SCAN_CHUNK", "0")
    Bt, L, D, N = 2, 130, 96, 16
    inp = synth.make_inputs(Bt, L, D, N, seed=2150, dtype="f32", a_mode="random")
    rng = np.random.default_rng(2151)
    A2 = (-np.exp(rng.standard_normal((D, N)))).astype(np.float32)
    D2 = (0.5 + rng.random(D)).astype(np.float32)
    b2 = (inp.delta_bias + 0.3 * rng.standard_normal(D)).astype(np.float32)
    d = upload(inp)
    to = lambda a: torch.from_numpy(a).cuda()  # noqa
    y = B.scan_bidir(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                     delta_bias=d["delta_bias"], z=d["z"], disc="zoh", A_rev=to(A2),
                     D_rev=to(D2), delta_bias_rev=to(b2))
    torch.cuda.synchronize()
    yf, _ = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D,
                       delta_bias=inp.delta_bias, z=inp.z, disc="zoh")
    yr, _ = _rev_oracle(oracle, inp, "zoh", A=A2, D=D2, bias=b2)
    check_f32(y.cpu().numpy(), yf + yr, "forward + reverse")


def test_accumulate_bf16_output(oracle):
    """bf16 output: each call rounds once, so per element
    |y - ref| <= 2^-8 (|ref| + 2 |y_f|) + 2e-3 max|ref|."""
    inp = synth.make_inputs(2, 200, 128, 16, seed=2160, dtype="bf16")
    d = upload(inp)
    y = B.scan_bidir(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                     delta_bias=d["delta_bias"], z=d["z"], disc="zoh", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yf, _ = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D,
                       delta_bias=inp.delta_bias, z=inp.z, disc="zoh")
    yr, _ = oracle.fwd_reverse(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D,
                               delta_bias=inp.delta_bias, z=inp.z, disc="zoh")
    ref = yf + yr
    got = y.float().cpu().numpy().astype(np.float64)
    bound = 2.0 ** -8 * (np.abs(ref) + 2 * np.abs(yf)) + TOL_BF16 * np.abs(ref).max()
    assert np.all(np.abs(got - ref) <= bound), float((np.abs(got - ref) / bound).max())


@pytest.mark.parametrize("dt_range", [(1e-3, 1e-1), (1e-4, 1e-2)], ids=["dt1e-3", "dt1e-4"])
@pytest.mark.parametrize("amode", ["s4d_real", "random", "weak"])
@pytest.mark.parametrize("layout", [("16", "4"), ("40", "8"), ("100000", "8"), ("100000", "16")],
                         ids=lambda v: "chunk%s_split%s" % v)
def test_reverse_long_fp32(oracle, monkeypatch, layout, amode, dt_range):
    """10,250 fp32 steps in reverse time, with >= 256 chunks (the chunk carries
    run as the lane-parallel scan in reversed chunk order) and in one pass, for
    S4D-real, random and weak A, at the elementwise fp32 bound."""
    chunk, nsplit = layout
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    seed = 2170 + 10 * ["s4d_real", "random", "weak"].index(amode) + (dt_range[0] < 5e-4)
    inp = synth.make_inputs(2, 10250, 40, 16, seed=seed, dtype="f32", with_h0=True,
                            a_mode=amode, dt_range=dt_range)
    d = upload(inp)
    log("reverse long fp32", layout, amode, dt_range)
    y, hl = _gpu(d, "zoh", reverse=True)
    torch.cuda.synchronize()
    ref, href = _rev_oracle(oracle, inp, "zoh")
    check_f32(y.cpu().numpy(), ref, "y")
    check_f32(hl.cpu().numpy(), href, "h_last")


def test_bidirectional_full_size(oracle):
    """The Mamba-2.8B-shaped workload (B=8, L=2048, D=5120, bf16) in both
    directions, summed; every element against the oracle's forward + reverse."""
    name = "fwd_2p8b_bf16_b8_l2048_d5120"
    w = synth.WORKLOADS[name]
    log("bidirectional full size", name)
    inp = synth.make_workload(name)
    d = upload(inp)
    y = B.scan_bidir(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                     delta_bias=d["delta_bias"], z=d["z"], disc=w.disc)
    torch.cuda.synchronize()
    kw = dict(D=inp.D, delta_bias=inp.delta_bias, z=inp.z, disc=w.disc,
              nthreads=oracle_threads())
    args = (inp.u, inp.delta, inp.A, inp.B, inp.C)
    ref = oracle.fwd(*args, **kw)[0]
    ref += oracle.fwd_reverse(*args, **kw)[0]
    r = check_rel_max(y.cpu().numpy(), ref, TOL_BF16, name)
    log("  max err / max|ref| =", r)


def test_reverse_deterministic():
    inp = synth.make_inputs(2, 300, 200, 16, seed=2180, dtype="bf16")
    d = upload(inp)
    y1 = _gpu(d, "zoh", reverse=True, h0=False)[0]
    y2 = _gpu(d, "zoh", reverse=True, h0=False)[0]
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
