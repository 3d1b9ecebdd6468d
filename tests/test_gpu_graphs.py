"""Graph capture of the library's entry points: each call is captured in a
HIP graph (through torch.cuda.CUDAGraph) and replayed three times, with eager
work and a NaN fill of the outputs between the replays; every replay must equal
the eager call bit for bit (the kernels are deterministic, and nothing in the
library allocates or clears memory with hipMemsetAsync, so the captured graph
holds kernel nodes only).  Covered: the chunked forward (workspace: start
states and step sums), the one-pass forward with B and C read from a projection
output (workspace: packed rows), the backward, the complex-A forward in time
chunks, the SSD layer from a start state and the Conv1d forward and backward.
Marked gpu: run on an MI355X."""
import numpy as np
import pytest
import torch

from selective_state_space_69_amd import binding as B
from selective_state_space_69_amd import synth
from gpu_util import log, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    B.load_library()
    yield
    torch.cuda.synchronize()


def _replays_equal_eager(run, outs, what):
    """run() issues the call on the current stream, writing outs."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                    # warm-up on a side stream, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        noise = torch.randn(1 << 20, device="cuda")
        noise.mul_(2.0).sum()                    # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), "%s: replay %d, output %d differs" % (what, rep, k)
    log("  %s: 3 replays equal the eager call" % what)


def test_graph_fwd_chunked():
    Bt, L, D, N = 1, 3000, 64, 16
    inp = synth.make_inputs(Bt, L, D, N, seed=6001, dtype="bf16", with_h0=True, a_mode="random")
    d = upload(inp)
    desc = B.make_desc(Bt, L, D, N, B.SS_BF16, B.SS_F32, B.SS_ZOH, True)
    nb = B.ss_scan_workspace_bytes(desc, B.SS_OP_FWD)
    assert nb > 0, "expected a chunked plan"
    ws = B.workspace(nb, "cuda")
    y = torch.empty((Bt, L, D), device="cuda")
    hl = torch.empty((Bt, D, N), device="cuda")

    def run():
        rc = B.ss_scan_fwd(desc, d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                           d["delta_bias"], d["z"], d["h0"], y, hl, ws, nb)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
    _replays_equal_eager(run, [y, hl], "chunked forward")


def test_graph_fwd_strided_bc_bf16_out():
    Bt, L, D, N, R = 8, 256, 1536, 16, 48
    inp = synth.make_inputs(Bt, L, D, N, seed=6002, dtype="bf16", a_mode="random")
    d = upload(inp)
    x = torch.zeros((Bt, L, R + 2 * N), dtype=torch.bfloat16, device="cuda")
    x[..., R:R + N] = d["B"]
    x[..., R + N:] = d["C"]
    Bv, Cv = x[..., R:R + N], x[..., R + N:]
    desc = B.make_desc(Bt, L, D, N, B.SS_BF16, B.SS_BF16, B.SS_ZOH, True, bc_stride=R + 2 * N)
    nb = B.ss_scan_workspace_bytes(desc, B.SS_OP_FWD)
    assert nb > 0, "strided rows are packed into the workspace"
    ws = B.workspace(nb, "cuda")
    y = torch.empty((Bt, L, D), dtype=torch.bfloat16, device="cuda")

    def run():
        rc = B.ss_scan_fwd(desc, d["u"], d["delta"], d["A"], Bv, Cv, d["D"], d["delta_bias"],
                           d["z"], None, y, None, ws, nb)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
    _replays_equal_eager(run, [y], "forward, strided B/C, bf16 y")


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_graph_bwd(disc):
    Bt, L, D, N = 2, 200, 128, 16
    inp = synth.make_inputs(Bt, L, D, N, seed=6003, dtype="bf16", with_h0=True, with_dy=True,
                            a_mode="random")
    d = upload(inp)
    desc = B.make_desc(Bt, L, D, N, B.SS_BF16, B.SS_F32, B._DISC[disc], True)
    nb = B.ss_scan_workspace_bytes(desc, B.SS_OP_BWD)
    ws = B.workspace(nb, "cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    g = [torch.empty((Bt, L, D), **f32), torch.empty((Bt, L, D), **f32), torch.empty((D, N), **f32),
         torch.empty((Bt, L, N), **f32), torch.empty((Bt, L, N), **f32), torch.empty((D,), **f32),
         torch.empty((D,), **f32), torch.empty((Bt, L, D), **f32), torch.empty((Bt, D, N), **f32)]

    def run():
        rc = B.ss_scan_bwd(desc, d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                           d["delta_bias"], d["z"], d["h0"], d["dy"], *g, ws, nb)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
    _replays_equal_eager(run, g, "backward %s" % disc)


def test_graph_fwd_complex_chunked():
    Bt, L, D, N = 1, 3000, 64, 16
    inp = synth.make_complex_inputs(Bt, L, D, N, seed=6004, dtype="bf16", with_h0=True)
    it = torch.bfloat16
    dev = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t).contiguous()  # noqa
    u, dl, z = dev(inp.u, it), dev(inp.delta, it), dev(inp.z, it)
    Bm, Cm = dev(inp.B, it), dev(inp.C, it)
    A, Dk, bias, h0 = dev(inp.A), dev(inp.D), dev(inp.delta_bias), dev(inp.h0)
    desc = B.make_desc(Bt, L, D, N, B.SS_BF16, B.SS_F32, B.SS_ZOH, True)
    nb = B.ss_scan_workspace_bytes(desc, B.SS_OP_FWD_COMPLEX)
    assert nb > 0, "expected time chunks"
    ws = B.workspace(nb, "cuda")
    y = torch.empty((Bt, L, D), device="cuda")
    hl = torch.empty((Bt, D, N, 2), device="cuda")

    def run():
        rc = B.ss_scan_fwd_complex_ws(desc, u, dl, A, Bm, Cm, Dk, bias, z, h0, y, hl, ws, nb)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
    _replays_equal_eager(run, [y, hl], "complex forward, time chunks")


def test_graph_ssd_state():
    Bt, L, H, P, N, G = 2, 300, 3, 64, 64, 1
    inp = synth.make_ssd_inputs(Bt, L, H, P, N, G, seed=6005)
    bf = torch.bfloat16
    dev = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t).contiguous()  # noqa
    x, dt, Bm, Cm = dev(inp.x, bf), dev(inp.dt, bf), dev(inp.B, bf), dev(inp.C, bf)
    A, Dk, bias = dev(inp.A), dev(inp.D), dev(inp.dt_bias)
    h0 = torch.randn((Bt, H, N, P), device="cuda")
    desc = B.make_ssd_desc(Bt, L, H, P, N, G, B.SS_BF16, B.SS_F32, True)
    y = torch.empty((Bt, L, H, P), device="cuda")
    hl = torch.empty((Bt, H, N, P), device="cuda")

    def run():
        rc = B.ss_ssd_fwd_state(desc, x, dt, A, Bm, Cm, Dk, bias, h0, y, hl)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
    _replays_equal_eager(run, [y, hl], "SSD from a start state")


def test_graph_conv():
    Bt, L, D, K = 2, 500, 384, 4
    rng = np.random.default_rng(6006)
    x = torch.from_numpy(rng.standard_normal((Bt, L, D), dtype=np.float32)).to("cuda").to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((D, K), dtype=np.float32)).to("cuda")
    bias = torch.from_numpy(rng.standard_normal(D, dtype=np.float32)).to("cuda")
    du = torch.from_numpy(rng.standard_normal((Bt, L, D), dtype=np.float32)).to("cuda")
    fdesc = B.make_conv_desc(Bt, L, D, K, B.SS_BF16, B.SS_F32, True)
    u = torch.empty((Bt, L, D), device="cuda")
    nb = B.ss_conv1d_workspace_bytes(fdesc)
    ws = B.workspace(nb, "cuda")
    dx = torch.empty((Bt, L, D), device="cuda")
    dw = torch.empty((D, K), device="cuda")
    db = torch.empty((D,), device="cuda")

    def run():
        rc = B.ss_conv1d_fwd(fdesc, x, w, bias, u)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
        rc = B.ss_conv1d_bwd(fdesc, x, w, bias, du, dx, dw, db, ws, nb)
        assert rc == B.SS_OK, B.ss_scan_strerror(rc)
    _replays_equal_eager(run, [u, dx, dw, db], "Conv1d forward and backward")
