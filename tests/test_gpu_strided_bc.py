"""B and C read in place as column ranges of one projection output (the Mamba
block's x_proj: (B, L, R + 2N), the low-rank step input, then B, then C), through
ss_desc_t.bc_stride: forward (both time directions, every forced layout, chunked
and one pass), backward, decode step and the non-allocating forward, each against
the fp64 oracle and bit for bit against the same call on dense copies of B and C
(the strided rows are copied into the dense padded layout the scan kernels read,
so the arithmetic is the same).  Marked gpu: run on an MI355X."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd import synth
from gpu_util import TOL_GRAD, check_f32, check_rel_max, TOL_BF16, log, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    B.load_library()
    yield
    torch.cuda.synchronize()


def projection(Bd, Cd, R, seed):
    """(b, t, R + 2N) tensor holding noise in its first R columns, then B, then C
    (same bits as the dense tensors); returns the two column views."""
    shape = Bd.shape[:-1] + (R + 2 * Bd.shape[-1],)
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(shape, generator=g).to(device=Bd.device, dtype=Bd.dtype)
    N = Bd.shape[-1]
    x[..., R:R + N] = Bd
    x[..., R + N:] = Cd
    return x[..., R:R + N], x[..., R + N:]


# (B, L, D, N, dtype, R): R odd puts B, C at addresses that are not 16-byte aligned
FWD_CASES = [(2, 77, 150, 16, "f32", 5), (2, 203, 100, 13, "bf16", 7),
             (1, 300, 64, 16, "bf16", 160), (3, 45, 33, 5, "f32", 1)]


@pytest.mark.parametrize("reverse", [False, True], ids=["fwd", "rev"])
@pytest.mark.parametrize("chunk", ["0", "40"])
@pytest.mark.parametrize("nsplit", ["0", "1", "4", "8", "16"])
@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "b%d_l%d_d%d_n%d_%s_r%d" % c)
def test_fwd_strided_bc(oracle, monkeypatch, case, nsplit, chunk, reverse):
    Bt, L, D, N, dtype, R = case
    monkeypatch.setenv("SS_SCAN_NSPLIT", nsplit)
    monkeypatch.setenv("SS_SCAN_CHUNK", chunk)
    log("strided fwd", case, nsplit, chunk, reverse)
    inp = synth.make_inputs(Bt, L, D, N, seed=5000 + FWD_CASES.index(case), dtype=dtype,
                            with_h0=True, a_mode="random")
    d = upload(inp)
    Bv, Cv = projection(d["B"], d["C"], R, seed=R)
    assert B._bc_stride(Bv, Cv, N) == R + 2 * N
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], z=d["z"], h0=d["h0"], disc="zoh",
              return_last_state=True, reverse=reverse)
    y, hl = B.scan_fwd(d["u"], d["delta"], d["A"], Bv, Cv, **kw)
    y0, hl0 = B.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hl, hl0)
    fn = oracle.fwd_reverse if reverse else oracle.fwd
    ref, href = fn(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                   z=inp.z, h0=inp.h0, disc="zoh")
    if dtype == "f32":
        check_f32(y.cpu().numpy(), ref, "y")
        check_f32(hl.cpu().numpy(), href, "h_last")
    else:
        check_rel_max(y.cpu().numpy(), ref, TOL_BF16, "y")


def test_fwd_strided_bc_full_size():
    """The Mamba-2.8B forward shape (B = 8, L = 2048, D = 5120, N = 16, bf16) with
    B and C as columns of a (B, L, 160 + 32) projection output, in the default
    plan: bit for bit the dense call (which the full-size parity tests check
    against the oracle)."""
    inp = synth.make_workload("fwd_2p8b_bf16_b8_l2048_d5120")
    d = upload(inp)
    Bv, Cv = projection(d["B"], d["C"], 160, seed=3)
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], z=d["z"], disc="zoh")
    y = B.scan_fwd(d["u"], d["delta"], d["A"], Bv, Cv, **kw)
    y0 = B.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


@pytest.mark.parametrize("case", [(2, 77, 150, 16, "zoh", "f32", 5),
                                  (1, 200, 70, 13, "euler", "bf16", 3),
                                  (2, 64, 64, 16, "zoh", "bf16", 160)],
                         ids=lambda c: "b%d_l%d_d%d_n%d_%s_%s_r%d" % c)
def test_bwd_strided_bc(oracle, case):
    """Backward with strided B, C: gradients (dB, dC dense) equal the dense call's
    bit for bit and the oracle's to the gradient bound."""
    Bt, L, D, N, disc, dtype, R = case
    log("strided bwd", case)
    inp = synth.make_inputs(Bt, L, D, N, seed=5100 + R, dtype=dtype, with_h0=True,
                            a_mode="random", with_dy=True)
    d = upload(inp)
    Bv, Cv = projection(d["B"], d["C"], R, seed=R)
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], z=d["z"], h0=d["h0"], disc=disc,
              want_dh0=True)
    g = B.scan_bwd(d["u"], d["delta"], d["A"], Bv, Cv, d["dy"], **kw)
    g0 = B.scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dy"], **kw)
    torch.cuda.synchronize()
    for k, v in g.items():
        if v is not None:
            assert v.is_contiguous() and torch.equal(v, g0[k]), k
    ref = oracle.bwd(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D, delta_bias=inp.delta_bias,
                     z=inp.z, h0=inp.h0, g=inp.dy, disc=disc)
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias", "dz", "dh0"):
        if ref.get(k) is not None and g.get(k) is not None:
            check_rel_max(g[k].double().cpu().numpy(), ref[k], TOL_GRAD, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 13])
def test_step_strided_bc(oracle, dtype, N):
    """Decode step with B, C rows of a (B, R + 2N) projection output (R = 5):
    the state and y equal the dense call's bit for bit (N = 16: the dense call
    takes 16-byte vector loads, the strided one scalar loads) and the oracle's."""
    log("strided step", dtype, N)
    inp = synth.make_inputs(3, 1, 200, N, seed=5200 + N, dtype=dtype, with_h0=True,
                            a_mode="mixed")
    d = upload(inp)
    b0, c0 = d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous()
    Bv, Cv = projection(b0, c0, 5, seed=11)
    assert B._bc_stride(Bv, Cv, N) == 5 + 2 * N
    args = (d["u"][:, 0].contiguous(), d["delta"][:, 0].contiguous(), d["A"])
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], z=d["z"][:, 0].contiguous(), disc="zoh")
    h = d["h0"].clone()
    h0 = d["h0"].clone()
    y = B.scan_step(h, *args, Bv, Cv, **kw)
    y0 = B.scan_step(h0, *args, b0, c0, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(h, h0)
    ref_y, ref_h = oracle.step(inp.h0, inp.u[:, 0], inp.delta[:, 0], inp.A, inp.B[:, 0],
                               inp.C[:, 0], D=inp.D, delta_bias=inp.delta_bias, z=inp.z[:, 0],
                               disc="zoh")
    check_f32(y.cpu().numpy(), ref_y, "step y")
    check_f32(h.cpu().numpy(), ref_h, "step h")


def test_noalloc_strided_bc():
    """ss_scan_fwd_noalloc with strided B, C (rows copied into the static
    scratch) equals ss_scan_fwd with a workspace, bit for bit."""
    Bt, L, D, N, R = 2, 500, 96, 16, 9
    inp = synth.make_inputs(Bt, L, D, N, seed=5300, dtype="bf16", with_h0=True, a_mode="random")
    d = upload(inp)
    Bv, Cv = projection(d["B"], d["C"], R, seed=R)
    desc = B.make_desc(Bt, L, D, N, B.SS_BF16, B.SS_F32, B.SS_ZOH, True, bc_stride=R + 2 * N)
    nb = B.ss_scan_workspace_bytes(desc, B.SS_OP_FWD)
    assert 0 < nb <= B.SS_SCAN_STATIC_SCRATCH_BYTES
    ws = B.workspace(nb, "cuda")
    outs = []
    for noalloc in (False, True):
        y = torch.full((Bt, L, D), float("nan"), device="cuda")
        hl = torch.full((Bt, D, N), float("nan"), device="cuda")
        args = (desc, d["u"], d["delta"], d["A"], Bv, Cv, d["D"], d["delta_bias"], d["z"],
                d["h0"], y, hl)
        rc = B.ss_scan_fwd_noalloc(*args) if noalloc else B.ss_scan_fwd(*args, ws, nb)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
        outs.append((y, hl))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert np.isfinite(outs[0][0].cpu().numpy()).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_rows_at_odd_address(oracle, dtype):
    """Dense B, C rows starting one element into a buffer (not 16-byte aligned):
    the binding passes bc_stride = N, the forward packs the rows and the step
    reads them element by element; both equal the aligned dense call bit for bit."""
    Bt, L, D, N = 2, 130, 96, 16
    inp = synth.make_inputs(Bt, L, D, N, seed=5400, dtype=dtype, with_h0=True, a_mode="random")
    d = upload(inp)

    def odd(t):
        buf = torch.zeros(t.numel() + 8, dtype=t.dtype, device=t.device)
        v = buf[1:1 + t.numel()].view(t.shape)
        v.copy_(t)
        return v

    Bv, Cv = odd(d["B"]), odd(d["C"])
    assert B._bc_stride(Bv, Cv, N) == N
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], z=d["z"], h0=d["h0"], disc="zoh",
              return_last_state=True)
    y, hl = B.scan_fwd(d["u"], d["delta"], d["A"], Bv, Cv, **kw)
    y0, hl0 = B.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], **kw)
    b1, c1 = odd(d["B"][:, 0].contiguous()), odd(d["C"][:, 0].contiguous())
    args = (d["u"][:, 0].contiguous(), d["delta"][:, 0].contiguous(), d["A"])
    skw = dict(D=d["D"], delta_bias=d["delta_bias"], z=d["z"][:, 0].contiguous(), disc="zoh")
    h, h0 = d["h0"].clone(), d["h0"].clone()
    ys = B.scan_step(h, *args, b1, c1, **skw)
    ys0 = B.scan_step(h0, *args, d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), **skw)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hl, hl0)
    assert torch.equal(ys, ys0) and torch.equal(h, h0)
