"""Seeded random problem shapes against the fp64 oracle: batch, length, width
and state count, input and output types, discretisation, time direction, the
forced layout and chunk length, strided B/C rows and an optional start state
are drawn together, so that combinations no hand-written case names still meet
the parity bound.  The draw is fixed (one seed), so the cases are the same on
every run.  Marked gpu: run on an MI355X."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd import synth
from gpu_util import TOL_BF16, TOL_GRAD, check_f32, check_rel_max, log, upload

pytestmark = pytest.mark.gpu


def _draw(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append(dict(
            Bt=int(rng.integers(1, 4)), L=int(rng.choice([1, 7, 16, 33, 100, 257, 700, 1500])),
            D=int(rng.choice([1, 5, 16, 17, 64, 100, 150, 300])), N=int(rng.integers(1, 17)),
            dtype=str(rng.choice(["f32", "bf16"])), disc=str(rng.choice(["zoh", "euler"])),
            reverse=bool(rng.random() < 0.3), layout=str(rng.choice(["0", "1", "2", "4", "8", "16"])),
            chunk=str(rng.choice(["0", "0", "40", "128"])), strided=bool(rng.random() < 0.4),
            h0=bool(rng.random() < 0.5), a_mode=str(rng.choice(["random", "s4d_real", "mixed", "weak"])),
            bf16_out=bool(rng.random() < 0.25), seed=7000 + i))
    return cases


CASES = _draw(40)


def _ids(c):
    return "b%d_l%d_d%d_n%d_%s_%s%s_s%s_c%s%s" % (
        c["Bt"], c["L"], c["D"], c["N"], c["dtype"], c["disc"], "_rev" if c["reverse"] else "",
        c["layout"], c["chunk"], "_strided" if c["strided"] else "")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    B.load_library()
    yield
    torch.cuda.synchronize()


def _strided_view(t, R, seed):
    """t (b, l, N) as a column range of a wider (b, l, R + N + 3) tensor."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(t.shape[:-1] + (R + t.shape[-1] + 3,), generator=g).to(t.device, t.dtype)
    x[..., R:R + t.shape[-1]] = t
    return x[..., R:R + t.shape[-1]]


@pytest.mark.parametrize("c", CASES, ids=_ids)
def test_fwd_random_shape(oracle, monkeypatch, c):
    monkeypatch.setenv("SS_SCAN_NSPLIT", c["layout"])
    monkeypatch.setenv("SS_SCAN_CHUNK", c["chunk"])
    log("random fwd", _ids(c))
    inp = synth.make_inputs(c["Bt"], c["L"], c["D"], c["N"], seed=c["seed"], dtype=c["dtype"],
                            with_h0=c["h0"], a_mode=c["a_mode"])
    d = upload(inp)
    Bm, Cm = d["B"], d["C"]
    if c["strided"]:
        Bm, Cm = _strided_view(Bm, 5, c["seed"]), _strided_view(Cm, 5, c["seed"] + 1)
    out = torch.bfloat16 if c["bf16_out"] else torch.float32
    y, hl = B.scan_fwd(d["u"], d["delta"], d["A"], Bm, Cm, D=d["D"], delta_bias=d["delta_bias"],
                       z=d["z"], h0=d["h0"], disc=c["disc"], out_dtype=out,
                       return_last_state=True, reverse=c["reverse"])
    torch.cuda.synchronize()
    fn = oracle.fwd_reverse if c["reverse"] else oracle.fwd
    ref, href = fn(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                   z=inp.z, h0=inp.h0, disc=c["disc"])
    yv = y.float().cpu().numpy()
    if c["bf16_out"]:
        # one rounding of y to bf16 on top of the input type's bound
        tol = 2.0 ** -8 * np.abs(ref) + (TOL_BF16 if c["dtype"] == "bf16" else 1e-4) * max(
            float(np.abs(ref).max()), 1e-30)
        assert np.all(np.abs(yv - ref) <= tol), "bf16 output out of bound"
    elif c["dtype"] == "f32":
        check_f32(yv, ref, "y")
    else:
        check_rel_max(yv, ref, TOL_BF16, "y")
    if c["dtype"] == "f32":
        check_f32(hl.cpu().numpy(), href, "h_last")
    else:
        check_rel_max(hl.cpu().numpy(), href, TOL_BF16, "h_last")


BWD_CASES = [c for c in CASES if not c["reverse"] and c["Bt"] * c["L"] * c["D"] * c["N"] <= 600000][:16]


@pytest.mark.parametrize("c", BWD_CASES, ids=_ids)
def test_bwd_random_shape(oracle, c):
    log("random bwd", _ids(c))
    inp = synth.make_inputs(c["Bt"], c["L"], c["D"], c["N"], seed=c["seed"], dtype=c["dtype"],
                            with_h0=c["h0"], with_dy=True, a_mode=c["a_mode"])
    d = upload(inp)
    Bm, Cm = d["B"], d["C"]
    if c["strided"]:
        Bm, Cm = _strided_view(Bm, 3, c["seed"]), _strided_view(Cm, 3, c["seed"] + 1)
    g = B.scan_bwd(d["u"], d["delta"], d["A"], Bm, Cm, d["dy"], D=d["D"],
                   delta_bias=d["delta_bias"], z=d["z"], h0=d["h0"], disc=c["disc"],
                   want_dh0=True)
    torch.cuda.synchronize()
    ref = oracle.bwd(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                     z=inp.z, h0=inp.h0, g=inp.dy, disc=c["disc"])
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz", "dh0"):
        if ref.get(k) is not None and g.get(k) is not None:
            check_rel_max(g[k].double().cpu().numpy(), ref[k], TOL_GRAD, k)
