"""GPU parity of the SSD (Mamba-2) forward: ss_ssd_fwd through the C ABI against
the fp64 oracle on the same bf16 inputs.

Bound (fp32 output): the kernel keeps every operand it computes (the masked
block of M, the state H, the scaled x) as a bf16 hi + lo pair, so the products
carry about 16 significant bits per operand with fp32 accumulation; the
remaining error is fp32 rounding and the hardware exp2 (about 1 ulp).  A
simulation of that arithmetic gives max|y - ref| about 3e-6 max|ref|; the test
allows 2e-5 max|ref| and, per element, the fp32 bound 1e-4 (1 + |ref|).  bf16
output adds its own rounding, at most the unit roundoff 2^-8 of |y| (8
significant bits): per element |y - ref| <= 2^-8 |ref| + 2e-5 max|ref|."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd.synth import SSD_WORKLOAD, make_ssd_inputs

from gpu_util import check_f32, log

pytestmark = pytest.mark.gpu

TOL_SSD_MAX = 2e-5
BF16_ROUNDOFF = 2.0 ** -8


def _dev(a, dtype):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", dtype).contiguous()


def _run(inp, softplus=True, out_dtype=torch.float32):
    bf = torch.bfloat16
    y = B.ssd_fwd(_dev(inp.x, bf), _dev(inp.dt, bf), _dev(inp.A, torch.float32),
                  _dev(inp.B, bf), _dev(inp.C, bf), D=_dev(inp.D, torch.float32),
                  dt_bias=_dev(inp.dt_bias, torch.float32), softplus=softplus,
                  out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check(y, ref, what, bf16_out=False):
    assert np.all(np.isfinite(y)), what + ": non-finite output"
    m = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(y - ref)))
    if bf16_out:
        bound = BF16_ROUNDOFF * np.abs(ref) + TOL_SSD_MAX * m
        worst = float(np.max(np.abs(y - ref) / bound))
        assert worst <= 1.0, "%s: bf16 output, worst err/bound %.3g" % (what, worst)
    else:
        assert err <= TOL_SSD_MAX * m, "%s: err %.3g > %.3g (max|ref| %.3g)" % (
            what, err, TOL_SSD_MAX * m, m)
        check_f32(y, ref, what)
    return err / m


CASES = [
    # (Bt, L, H, G, seed, options)
    (1, 64, 1, 1, 11, {}),                     # one full chunk
    (2, 200, 4, 2, 12, {}),                    # ragged tail, 4 chunks, two groups
    (1, 1, 2, 1, 13, {}),                      # a single step
    (2, 333, 3, 1, 14, {}),                    # ragged, odd head count
    (1, 130, 4, 4, 15, {"with_D": False, "with_bias": False}),
    (1, 257, 2, 1, 16, {"softplus": False, "with_bias": False}),
    (2, 190, 2, 1, 17, {"bf16_out": True}),
    (1, 1024, 2, 1, 18, {"dt_range": (1e-2, 1.0)}),   # strong decay: exp underflows inside chunks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_h%d_g%d" % c[:4])
def test_ssd_parity(oracle, case):
    Bt, L, H, G, seed, opt = case
    opt = dict(opt)
    softplus = opt.pop("softplus", True)
    bf16_out = opt.pop("bf16_out", False)
    log("ssd case", case)
    inp = make_ssd_inputs(Bt, L, H, 64, 64, G, seed, **opt)
    if not softplus:
        inp.dt = np.abs(inp.dt) * np.float32(0.5)   # plain steps: positive, still exact bf16
    y = _run(inp, softplus=softplus, out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    ref = oracle.ssd_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, D=inp.D, dt_bias=inp.dt_bias,
                         softplus=softplus)
    r = _check(y, ref, "ssd %s" % (case[:4],), bf16_out)
    log("  err/max|ref| = %.3g" % r)


def test_ssd_full_size(oracle):
    """The benchmark shape (8 x 2048, 80 heads) in its launch configuration;
    every element of y against the oracle on the same inputs."""
    w = SSD_WORKLOAD
    log("ssd full size", w["name"])
    inp = make_ssd_inputs(w["Bt"], w["L"], w["H"], w["P"], w["N"], w["G"], w["seed"])
    y = _run(inp)
    ref = oracle.ssd_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, D=inp.D, dt_bias=inp.dt_bias)
    r = _check(y, ref, "ssd full size")
    log("  err/max|ref| = %.3g" % r)


def test_ssd_deterministic():
    inp = make_ssd_inputs(2, 300, 3, 64, 64, 1, 21)
    y1 = _run(inp)
    y2 = _run(inp)
    assert np.array_equal(y1, y2)


# ---------------------------------------------------------------- start state, final state, step
def _state(Bt, H, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((Bt, H, 64, 64), dtype=np.float32) * np.float32(scale)


def _inputs_dev(inp):
    bf, f32 = torch.bfloat16, torch.float32
    return dict(x=_dev(inp.x, bf), dt=_dev(inp.dt, bf), A=_dev(inp.A, f32), B=_dev(inp.B, bf),
                C=_dev(inp.C, bf), D=_dev(inp.D, f32), dt_bias=_dev(inp.dt_bias, f32))


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


STATE_CASES = [
    # (Bt, L, H, G, seed, options)
    (1, 64, 2, 1, 31, {}),       # one full chunk
    (2, 200, 4, 2, 32, {}),      # ragged tail
    (1, 1, 3, 1, 33, {}),        # a single step
    (2, 129, 2, 2, 34, {}),      # two chunks and one step
    (1, 150, 2, 1, 37, {"softplus": False, "with_bias": False}),
    (2, 100, 2, 1, 38, {"bf16_out": True}),
]


@pytest.mark.parametrize("case", STATE_CASES, ids=lambda c: "b%d_l%d_h%d_g%d_s%d" % c[:5])
def test_ssd_state_in_out(oracle, case):
    """ss_ssd_fwd_state from a random start state: y and the final state
    against the oracle on the same bits (state bound as y's)."""
    Bt, L, H, G, seed, opt = case
    opt = dict(opt)
    softplus = opt.pop("softplus", True)
    bf16_out = opt.pop("bf16_out", False)
    log("ssd state case", case)
    inp = make_ssd_inputs(Bt, L, H, 64, 64, G, seed, **opt)
    if not softplus:
        inp.dt = np.abs(inp.dt) * np.float32(0.5)
    h0 = _state(Bt, H, seed + 100)
    d = _inputs_dev(inp)
    y, hl = B.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"],
                      softplus=softplus, out_dtype=torch.bfloat16 if bf16_out else torch.float32,
                      h0=_dev(h0, torch.float32), return_last=True)
    torch.cuda.synchronize()
    ref, ref_h = oracle.ssd_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, D=inp.D, dt_bias=inp.dt_bias,
                                softplus=softplus, h0=h0, return_last=True)
    _check(_np(y), ref, "ssd state y %s" % (case[:5],), bf16_out)
    _check(_np(hl), ref_h, "ssd state h_last %s" % (case[:5],))


def test_ssd_state_none_matches_plain():
    """No start state and no final state: the same bits as ss_ssd_fwd; with
    return_last alone, y is unchanged."""
    inp = make_ssd_inputs(2, 150, 3, 64, 64, 1, 35)
    d = _inputs_dev(inp)
    y0 = B.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"])
    y1, _ = B.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"],
                      return_last=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_ssd_prefill_in_pieces(oracle):
    """A sequence cut into pieces (64-aligned and not), the state advanced in
    place from piece to piece (h0 and h_last one buffer), equals the oracle's
    single pass."""
    Bt, L, H, G, seed = 2, 300, 2, 1, 36
    log("ssd pieces", (Bt, L, H, G, seed))
    inp = make_ssd_inputs(Bt, L, H, 64, 64, G, seed)
    d = _inputs_dev(inp)
    h = torch.zeros((Bt, H, 64, 64), dtype=torch.float32, device="cuda")
    ys = []
    cuts = [0, 64, 101, 230, 300]
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        sl = lambda t: t[:, t0:t1].contiguous()
        desc = B.make_ssd_desc(Bt, t1 - t0, H, 64, 64, G, B.SS_BF16, B.SS_F32, True)
        y = torch.empty((Bt, t1 - t0, H, 64), dtype=torch.float32, device="cuda")
        rc = B.ss_ssd_fwd_state(desc, sl(d["x"]), sl(d["dt"]), d["A"], sl(d["B"]), sl(d["C"]),
                                d["D"], d["dt_bias"], h, y, h)
        assert rc == B.SS_OK
        ys.append(y)
    torch.cuda.synchronize()
    y = _np(torch.cat(ys, dim=1))
    ref, ref_h = oracle.ssd_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, D=inp.D, dt_bias=inp.dt_bias,
                                return_last=True)
    _check(y, ref, "ssd pieces y")
    _check(_np(h), ref_h, "ssd pieces state")


STEP_CASES = [
    # (Bt, H, G, seed, options)
    (1, 1, 1, 41, {}),
    (3, 8, 2, 42, {}),
    (2, 6, 3, 43, {"with_D": False, "with_bias": False}),
    (4, 4, 1, 44, {"softplus": False, "with_bias": False}),
    (2, 4, 1, 45, {"bf16_out": True}),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "b%d_h%d_g%d_s%d" % c[:4])
def test_ssd_step_parity(oracle, case):
    """ss_ssd_step on a random state against the oracle's layer over one step
    from that state."""
    Bt, H, G, seed, opt = case
    opt = dict(opt)
    softplus = opt.pop("softplus", True)
    bf16_out = opt.pop("bf16_out", False)
    log("ssd step case", case)
    inp = make_ssd_inputs(Bt, 1, H, 64, 64, G, seed, **opt)
    if not softplus:
        inp.dt = np.abs(inp.dt) * np.float32(0.5)
    h0 = _state(Bt, H, seed + 100)
    d = _inputs_dev(inp)
    h = _dev(h0, torch.float32)
    y = B.ssd_step(h, d["x"][:, 0].contiguous(), d["dt"][:, 0].contiguous(), d["A"],
                   d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), D=d["D"],
                   dt_bias=d["dt_bias"], softplus=softplus,
                   out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    ref, ref_h = oracle.ssd_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, D=inp.D, dt_bias=inp.dt_bias,
                                softplus=softplus, h0=h0, return_last=True)
    _check(_np(y), ref[:, 0], "ssd step y %s" % (case[:4],), bf16_out)
    _check(_np(h), ref_h, "ssd step state %s" % (case[:4],))


def test_ssd_step_continues_prefill(oracle):
    """Prefill 100 steps with the chunked kernel, keep the state, decode 5 more
    steps one at a time: y of every step and the final state against the
    oracle's single pass over all 105."""
    Bt, L, H, G, seed, k = 2, 105, 4, 2, 46, 5
    log("ssd prefill + decode", (Bt, L, H, G, seed, k))
    inp = make_ssd_inputs(Bt, L, H, 64, 64, G, seed)
    d = _inputs_dev(inp)
    pre = slice(0, L - k)
    y_pre, h = B.ssd_fwd(*(d[n][:, pre].contiguous() for n in ("x", "dt")), d["A"],
                         *(d[n][:, pre].contiguous() for n in ("B", "C")), D=d["D"],
                         dt_bias=d["dt_bias"], return_last=True)
    ys = [y_pre]
    for t in range(L - k, L):
        ys.append(B.ssd_step(h, d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                             d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), D=d["D"],
                             dt_bias=d["dt_bias"])[:, None])
    torch.cuda.synchronize()
    ref, ref_h = oracle.ssd_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, D=inp.D, dt_bias=inp.dt_bias,
                                return_last=True)
    _check(_np(torch.cat(ys, dim=1)), ref, "ssd prefill + decode y")
    _check(_np(h), ref_h, "ssd prefill + decode state")


def test_ssd_step_full_size(oracle):
    """A decode batch at the layer's width (256 rows x 80 heads) in the launch
    configuration of the step leg of the benchmark; every head of every row
    (y and the state) against the oracle."""
    Bt, H = 256, 80
    log("ssd step full size", (Bt, H))
    inp = make_ssd_inputs(Bt, 1, H, 64, 64, 1, 47)
    h0 = _state(Bt, H, 147)
    d = _inputs_dev(inp)
    h = _dev(h0, torch.float32)
    y = B.ssd_step(h, d["x"][:, 0].contiguous(), d["dt"][:, 0].contiguous(), d["A"],
                   d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), D=d["D"],
                   dt_bias=d["dt_bias"])
    torch.cuda.synchronize()
    ref, ref_h = oracle.ssd_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, D=inp.D,
                                dt_bias=inp.dt_bias, h0=h0, return_last=True)
    _check(_np(y), ref[:, 0], "ssd step full size y")
    _check(_np(h), ref_h, "ssd step full size state")
