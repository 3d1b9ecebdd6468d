"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before any HIP call."""
import os
import re

import pytest

from selective_state_space_69_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from selective_state_space_69_amd import build
        build.build(verbose=False)
    return B.load_library()


def declared_functions():
    """Every function declared in include/*.h (comments stripped)."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if not h.endswith(".h"):
            continue
        text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
        names |= set(re.findall(r"\b(ss_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("ss_scan_fwd", "ss_scan_bwd", "ss_scan_step", "ss_scan_workspace_bytes",
              "ss_scan_strerror", "ss_scan_version", "ss_conv1d_fwd", "ss_conv1d_bwd",
              "ss_conv1d_step", "ss_conv1d_workspace_bytes", "ss_ssd_fwd", "ss_ssd_fwd_state",
              "ss_ssd_step", "ss_scan_fwd_dir", "ss_scan_fwd_complex", "ss_scan_step_complex",
              "ss_scan_arch_supported", "ss_scan_fwd_noalloc", "ss_scan_fwd_complex_ws"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_and_version(lib):
    for code in (0, -1, -2, -3, -4, 99):
        assert isinstance(B.ss_scan_strerror(code), str) and B.ss_scan_strerror(code)
    assert B.ss_scan_version() >= 10000


FAKE = 1 << 20   # a 16-byte aligned non-null "device pointer"; never dereferenced


def fwd(desc, **kw):
    args = dict(u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, D_skip=None, delta_bias=None,
                z=None, h0=None, y=FAKE, h_last=None, workspace=None, ws_bytes=0)
    args.update(kw)
    return B.ss_scan_fwd(desc, args["u"], args["delta"], args["A"], args["Bm"], args["Cm"],
                         args["D_skip"], args["delta_bias"], args["z"], args["h0"], args["y"],
                         args["h_last"], args["workspace"], args["ws_bytes"], stream=0)


def desc(**kw):
    base = dict(batch=2, seqlen=64, dim=128, dstate=16, in_dtype=B.SS_BF16, out_dtype=B.SS_F32,
                disc=B.SS_ZOH, delta_softplus=True)
    base.update(kw)
    return B.make_desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), B.SS_ERR_INVALID_ARG), (dict(seqlen=0), B.SS_ERR_INVALID_ARG),
    (dict(dim=0), B.SS_ERR_INVALID_ARG), (dict(dstate=0), B.SS_ERR_INVALID_ARG),
    (dict(dstate=17), B.SS_ERR_INVALID_ARG), (dict(seqlen=-5), B.SS_ERR_INVALID_ARG),
    (dict(seqlen=1 << 31), B.SS_ERR_INVALID_ARG), (dict(in_dtype=7), B.SS_ERR_UNSUPPORTED),
    (dict(out_dtype=3), B.SS_ERR_UNSUPPORTED), (dict(disc=2), B.SS_ERR_UNSUPPORTED),
])
def test_fwd_rejects_bad_descriptor(lib, kw, code):
    assert fwd(desc(**kw)) == code


@pytest.mark.parametrize("field", ["u", "delta", "A", "Bm", "Cm", "y"])
def test_fwd_rejects_null_required(lib, field):
    assert fwd(desc(), **{field: None}) == B.SS_ERR_INVALID_ARG


def test_fwd_rejects_misaligned_and_aliasing(lib):
    assert fwd(desc(), u=FAKE + 2) == B.SS_ERR_INVALID_ARG
    assert fwd(desc(), h0=FAKE + 64, h_last=FAKE + 64) == B.SS_ERR_INVALID_ARG


def test_fwd_workspace_checks(lib):
    d = desc(batch=1, seqlen=1 << 20, dim=256)       # narrow and long: chunked plan
    need = B.ss_scan_workspace_bytes(d, B.SS_OP_FWD)
    assert need > 0
    assert fwd(d, workspace=None, ws_bytes=0) == B.SS_ERR_WORKSPACE
    assert fwd(d, workspace=FAKE, ws_bytes=need - 1) == B.SS_ERR_WORKSPACE
    assert fwd(d, workspace=FAKE + 16, ws_bytes=need) == B.SS_ERR_WORKSPACE   # not 256-aligned


def test_plan_sizes(lib):
    # wide problems run as one pass over time: no workspace
    assert B.ss_scan_workspace_bytes(desc(batch=8, seqlen=2048, dim=5120), B.SS_OP_FWD) == 0
    # N < 16: B and C rows padded to 16 states (B, L, 16) in the input type
    rows = 2 * 8 * 2048 * 16 * 2
    assert B.ss_scan_workspace_bytes(desc(batch=8, seqlen=2048, dim=5120, dstate=8),
                                     B.SS_OP_FWD) == rows
    # Mamba-130M (B = 8, D = 1536: 768 groups of 16 channels) and B = 2 at D = 5120
    # run in one pass on the one-state-per-lane layout
    assert B.ss_scan_workspace_bytes(desc(batch=8, seqlen=2048, dim=1536), B.SS_OP_FWD) == 0
    assert B.ss_scan_workspace_bytes(desc(batch=2, seqlen=8192, dim=5120), B.SS_OP_FWD) == 0
    assert B.ss_scan_workspace_bytes(desc(batch=4, seqlen=2048, dim=1536), B.SS_OP_FWD) == 0
    # narrower ones are chunked: start states (B, chunks, N, D) + step sums (B, chunks, D)
    n = B.ss_scan_workspace_bytes(desc(batch=2, seqlen=2048, dim=1536), B.SS_OP_FWD)
    assert n > 0 and n % 256 == 0
    chunks = n // (2 * 16 * 1536 * 4 + 2 * 1536 * 4)
    assert n == chunks * (2 * 16 * 1536 * 4 + 2 * 1536 * 4) and chunks > 1
    assert B.ss_scan_workspace_bytes(desc(batch=0), B.SS_OP_FWD) == 0
    assert B.ss_scan_workspace_bytes(desc(), 5) == 0


def test_bwd_and_step_validation(lib):
    d = desc()
    P = FAKE
    args = [P, P, P, P, P, None, None, None, None, P, P, P, P, P, P, None, None, None, None, None, 0]
    assert B.ss_scan_bwd(desc(out_dtype=B.SS_BF16), *args, stream=0) == B.SS_ERR_UNSUPPORTED
    bad = list(args)
    bad[9] = None   # dy
    assert B.ss_scan_bwd(d, *bad, stream=0) == B.SS_ERR_INVALID_ARG
    bad = list(args)
    bad[5] = P      # D_skip given without dD_skip
    assert B.ss_scan_bwd(d, *bad, stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_scan_step(desc(dstate=0), P, P, P, P, P, P, None, None, None, P, stream=0) == \
        B.SS_ERR_INVALID_ARG
    assert B.ss_scan_step(d, None, P, P, P, P, P, None, None, None, P, stream=0) == \
        B.SS_ERR_INVALID_ARG


# ---------------------------------------------------------------- conv1d entry points
def cdesc(**kw):
    base = dict(batch=2, seqlen=100, dim=64, width=4, in_dtype=B.SS_BF16, out_dtype=B.SS_BF16,
                silu=True)
    base.update(kw)
    return B.make_conv_desc(**base)


def test_conv_validation(lib):
    P = FAKE
    ok = cdesc()
    for bad in (cdesc(width=0), cdesc(width=5), cdesc(batch=0), cdesc(seqlen=0), cdesc(dim=0)):
        assert B.ss_conv1d_fwd(bad, P, P, None, P + 4096, stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_conv1d_fwd(cdesc(in_dtype=7), P, P, None, P + 4096, stream=0) == B.SS_ERR_UNSUPPORTED
    assert B.ss_conv1d_fwd(ok, None, P, None, P, stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_conv1d_fwd(ok, P, P, None, P, stream=0) == B.SS_ERR_INVALID_ARG      # u aliases x
    assert B.ss_conv1d_fwd(ok, P + 2, P, None, P + 4096, stream=0) == B.SS_ERR_INVALID_ARG
    nb = B.ss_conv1d_workspace_bytes(ok)
    assert nb > 0 and nb % 256 == 0
    args = (P, P, None, P + 8192, P + 4096, P + 12288, None)
    assert B.ss_conv1d_bwd(ok, *args, None, 0, stream=0) == B.SS_ERR_WORKSPACE
    assert B.ss_conv1d_bwd(ok, *args, P, nb - 1, stream=0) == B.SS_ERR_WORKSPACE
    # bias without dbias, dx aliasing du
    assert B.ss_conv1d_bwd(ok, P, P, P, P + 8192, P + 4096, P + 12288, None, P, nb,
                           stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_conv1d_bwd(ok, P, P, None, P + 8192, P + 8192, P + 12288, None, P, nb,
                           stream=0) == B.SS_ERR_INVALID_ARG
    # the decode step needs a state unless the width is 1
    assert B.ss_conv1d_step(ok, None, P, P, None, P + 4096, stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_conv1d_workspace_bytes(cdesc(width=9)) == 0


def test_conv_workspace_size(lib):
    # per-segment (64 steps) partials of dw (B*nseg, D, K) and dbias (B*nseg, D), fp32
    d = cdesc(batch=8, seqlen=2048, dim=5120, width=4)
    parts = 8 * 32
    want = parts * 5120 * 4 * 4 + parts * 5120 * 4
    assert B.ss_conv1d_workspace_bytes(d) == want


# ---------------------------------------------------------------- SSD entry point
def sdesc(**kw):
    base = dict(batch=2, seqlen=100, nheads=4, headdim=64, dstate=64, ngroups=2)
    base.update(kw)
    return B.make_ssd_desc(**base)


def ssd(desc, **kw):
    P = FAKE
    args = dict(x=P, dt=P + 4096, A=P + 8192, Bm=P + 12288, Cm=P + 16384, D=None, dt_bias=None,
                y=P + 20480)
    args.update(kw)
    return B.ss_ssd_fwd(desc, args["x"], args["dt"], args["A"], args["Bm"], args["Cm"], args["D"],
                        args["dt_bias"], args["y"], stream=0)


def test_ssd_validation(lib):
    for bad in (sdesc(batch=0), sdesc(seqlen=0), sdesc(nheads=0), sdesc(ngroups=3),
                sdesc(ngroups=0), sdesc(headdim=0), sdesc(batch=1 << 30, nheads=4)):
        assert ssd(bad) == B.SS_ERR_INVALID_ARG
    d = sdesc()
    d.reserved = 1
    assert ssd(d) == B.SS_ERR_INVALID_ARG
    for uns in (sdesc(headdim=32), sdesc(dstate=128), sdesc(in_dtype=B.SS_F32),
                sdesc(out_dtype=5)):
        assert ssd(uns) == B.SS_ERR_UNSUPPORTED
    ok = sdesc()
    for name in ("x", "dt", "A", "Bm", "Cm", "y"):
        assert ssd(ok, **{name: None}) == B.SS_ERR_INVALID_ARG, name
    assert ssd(ok, y=FAKE) == B.SS_ERR_INVALID_ARG               # y aliases x
    assert ssd(ok, D=FAKE + 2) == B.SS_ERR_INVALID_ARG           # misaligned
    assert ssd(ok, y=FAKE + 20488) == B.SS_ERR_INVALID_ARG
    assert B.load_library().ss_ssd_fwd(None, *([None] * 8), None) == B.SS_ERR_INVALID_ARG


def ssd_state(desc, **kw):
    P = FAKE
    args = dict(x=P, dt=P + 4096, A=P + 8192, Bm=P + 12288, Cm=P + 16384, D=None, dt_bias=None,
                h0=P + 24576, y=P + 20480, h_last=P + 28672)
    args.update(kw)
    return B.ss_ssd_fwd_state(desc, args["x"], args["dt"], args["A"], args["Bm"], args["Cm"],
                              args["D"], args["dt_bias"], args["h0"], args["y"], args["h_last"],
                              stream=0)


def test_ssd_state_validation(lib):
    # the description and the plain forward's pointer rules are shared
    for bad in (sdesc(seqlen=0), sdesc(ngroups=3)):
        assert ssd_state(bad) == B.SS_ERR_INVALID_ARG
    assert ssd_state(sdesc(headdim=32)) == B.SS_ERR_UNSUPPORTED
    ok = sdesc()
    for name in ("x", "dt", "A", "Bm", "Cm", "y"):
        assert ssd_state(ok, **{name: None}) == B.SS_ERR_INVALID_ARG, name
    # the states are optional
    for name in ("h0", "h_last"):
        assert ssd_state(ok, **{name: FAKE + 4}) == B.SS_ERR_INVALID_ARG, name   # misaligned
    # h_last may be h0 but no other argument; h0 may not be y
    for other in ("x", "dt", "A", "Bm", "Cm", "y"):
        target = {"x": FAKE, "dt": FAKE + 4096, "A": FAKE + 8192, "Bm": FAKE + 12288,
                  "Cm": FAKE + 16384, "y": FAKE + 20480}[other]
        assert ssd_state(ok, h_last=target) == B.SS_ERR_INVALID_ARG, other
    assert ssd_state(ok, D=FAKE + 32768, h_last=FAKE + 32768) == B.SS_ERR_INVALID_ARG
    assert ssd_state(ok, h0=FAKE + 20480) == B.SS_ERR_INVALID_ARG
    assert B.load_library().ss_ssd_fwd_state(None, *([None] * 10), None) == B.SS_ERR_INVALID_ARG


def ssd_step(desc, **kw):
    P = FAKE
    args = dict(h=P + 24576, x=P, dt=P + 4096, A=P + 8192, Bm=P + 12288, Cm=P + 16384, D=None,
                dt_bias=None, y=P + 20480)
    args.update(kw)
    return B.ss_ssd_step(desc, args["h"], args["x"], args["dt"], args["A"], args["Bm"],
                         args["Cm"], args["D"], args["dt_bias"], args["y"], stream=0)


def test_ssd_step_validation(lib):
    for bad in (sdesc(batch=0), sdesc(nheads=0), sdesc(ngroups=3), sdesc(batch=1 << 30)):
        assert ssd_step(bad) == B.SS_ERR_INVALID_ARG
    d = sdesc()
    d.reserved = 1
    assert ssd_step(d) == B.SS_ERR_INVALID_ARG
    for uns in (sdesc(headdim=32), sdesc(dstate=16), sdesc(in_dtype=B.SS_F32)):
        assert ssd_step(uns) == B.SS_ERR_UNSUPPORTED
    ok = sdesc()
    for name in ("h", "x", "dt", "A", "Bm", "Cm", "y"):
        assert ssd_step(ok, **{name: None}) == B.SS_ERR_INVALID_ARG, name
    assert ssd_step(ok, y=FAKE) == B.SS_ERR_INVALID_ARG            # y aliases x
    assert ssd_step(ok, y=FAKE + 24576) == B.SS_ERR_INVALID_ARG    # y aliases h
    assert ssd_step(ok, h=FAKE + 8192) == B.SS_ERR_INVALID_ARG     # h aliases A
    assert ssd_step(ok, dt_bias=FAKE + 8) == B.SS_ERR_INVALID_ARG  # misaligned
    assert B.load_library().ss_ssd_step(None, *([None] * 9), None) == B.SS_ERR_INVALID_ARG


def test_fwd_dir_validation(lib):
    d = B.make_desc(2, 64, 32, 16, B.SS_F32, B.SS_F32)
    P = FAKE
    for bad_dir in (-1, 2, 7):
        assert B.ss_scan_fwd_dir(d, bad_dir, 0, P, P, P, P, P, None, None, None, None, P + 4096,
                                 None, None, 0, stream=0) == B.SS_ERR_INVALID_ARG
    # the rest of the validation is shared with ss_scan_fwd
    assert B.ss_scan_fwd_dir(d, B.SS_DIR_REVERSE, 1, None, P, P, P, P, None, None, None, None,
                             P + 4096, None, None, 0, stream=0) == B.SS_ERR_INVALID_ARG


def test_fwd_complex_validation(lib):
    P = FAKE
    ok = B.make_desc(2, 64, 32, 16, B.SS_F32, B.SS_F32)
    args = lambda **kw: [kw.get(k, v) for k, v in dict(u=P, delta=P, A=P, Bm=P, Cm=P, D=None,  # noqa
                         bias=None, z=None, h0=None, y=P + 4096, hl=None).items()]
    assert B.ss_scan_fwd_complex(B.make_desc(2, 64, 32, 17), *args(), stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_scan_fwd_complex(ok, *args(u=None), stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_scan_fwd_complex(ok, *args(A=P + 4), stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_scan_fwd_complex(ok, *args(h0=P + 8192, hl=P + 8192), stream=0) == B.SS_ERR_INVALID_ARG


def test_step_complex_validation(lib):
    P = FAKE
    d = B.make_desc(2, 1, 64, 16, B.SS_BF16, B.SS_F32)
    call = lambda desc, **kw: B.ss_scan_step_complex(  # noqa: E731
        desc, kw.get("h", P + 8192), kw.get("u", P), kw.get("delta", P + 256), kw.get("A", P + 512),
        kw.get("Bm", P + 1024), kw.get("Cm", P + 1536), None, None, kw.get("z", None),
        kw.get("y", P + 4096), stream=0)
    for name in ("h", "u", "delta", "A", "Bm", "Cm", "y"):
        assert call(d, **{name: None}) == B.SS_ERR_INVALID_ARG, name
    assert call(d, y=P) == B.SS_ERR_INVALID_ARG                   # y aliases u
    assert call(d, y=P + 8192) == B.SS_ERR_INVALID_ARG            # y aliases h
    assert call(d, A=P + 516) == B.SS_ERR_INVALID_ARG             # misaligned
    assert call(B.make_desc(2, 1, 64, 17, B.SS_BF16, B.SS_F32)) == B.SS_ERR_INVALID_ARG   # N > 16
    assert B.load_library().ss_scan_step_complex(None, *([None] * 10), None) == B.SS_ERR_INVALID_ARG


def test_step_validation_aliasing_and_grid(lib):
    """y of the decode step must not alias the state or an input (it is written
    while other lanes still read them); batch * dim is bounded by the grid."""
    P = FAKE
    d = B.make_desc(2, 1, 64, 16, B.SS_BF16, B.SS_F32)
    call = lambda desc, **kw: B.ss_scan_step(  # noqa: E731
        desc, kw.get("h", P + 8192), kw.get("u", P), kw.get("delta", P + 256), kw.get("A", P + 512),
        kw.get("Bm", P + 1024), kw.get("Cm", P + 1536), None, None, kw.get("z", P + 2048),
        kw.get("y", P + 4096), stream=0)
    for name in ("h", "u", "delta", "A", "Bm", "Cm", "y"):
        assert call(d, **{name: None}) == B.SS_ERR_INVALID_ARG, name
    for alias in (P + 8192, P, P + 256, P + 1024, P + 1536, P + 2048):   # h, u, delta, B, C, z
        assert call(d, y=alias) == B.SS_ERR_INVALID_ARG, alias
    assert call(d, Cm=P + 1540) == B.SS_ERR_INVALID_ARG                 # misaligned
    huge = B.make_desc(1 << 20, 1, 1 << 14, 16, B.SS_BF16, B.SS_F32)    # 2^34 channels
    assert call(huge) == B.SS_ERR_INVALID_ARG


def test_arch_supported(lib):
    """Only gfx950 devices run the kernels: the name check every launching entry
    point applies to the current device."""
    for name in ("gfx950", "gfx950:sramecc+:xnack-", "gfx950:xnack+"):
        assert B.ss_scan_arch_supported(name) == B.SS_OK, name
    for name in ("gfx942", "gfx942:sramecc+:xnack-", "gfx90a", "gfx9500", "gfx95", "", "sm_90",
                 "gfx1100", " gfx950"):
        assert B.ss_scan_arch_supported(name) == B.SS_ERR_UNSUPPORTED, name
    assert B.ss_scan_arch_supported(None) == B.SS_ERR_INVALID_ARG
    assert "gfx950" in B.ss_scan_strerror(B.SS_ERR_UNSUPPORTED)


def test_noalloc_validation_and_scratch_limit(lib):
    """ss_scan_fwd_noalloc validates like ss_scan_fwd and refuses, before any
    HIP call, a plan that needs more scratch than its static array."""
    P = FAKE
    args = lambda **kw: [kw.get(k, v) for k, v in dict(u=P, delta=P + 256, A=P + 512, Bm=P + 1024,  # noqa
                         Cm=P + 1536, D=None, bias=None, z=None, h0=None, y=P + 4096,
                         hl=None).items()]
    big = B.make_desc(1, 1 << 20, 256, 8, B.SS_BF16, B.SS_F32)     # padded rows: 72 MB
    assert B.ss_scan_workspace_bytes(big, B.SS_OP_FWD) > B.SS_SCAN_STATIC_SCRATCH_BYTES
    assert B.ss_scan_fwd_noalloc(big, *args(), stream=0) == B.SS_ERR_SCRATCH_LIMIT
    assert "static" in B.ss_scan_strerror(B.SS_ERR_SCRATCH_LIMIT)
    ok = B.make_desc(2, 64, 32, 16, B.SS_F32, B.SS_F32)
    assert B.ss_scan_fwd_noalloc(ok, *args(u=None), stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_scan_fwd_noalloc(ok, *args(A=P + 516), stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_scan_fwd_noalloc(ok, *args(h0=P + 8192, hl=P + 8192), stream=0) == \
        B.SS_ERR_INVALID_ARG
    assert B.ss_scan_fwd_noalloc(B.make_desc(2, 64, 32, 17), *args(), stream=0) == \
        B.SS_ERR_INVALID_ARG
    # the binding's size constant is the header's
    text = open(os.path.join(INCLUDE, "ss_scan.h")).read()
    m = re.search(r"#define SS_SCAN_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.SS_SCAN_STATIC_SCRATCH_BYTES


def test_complex_ws_plan_and_validation(lib):
    """The chunked complex forward: long narrow problems get a workspace (chunk
    start states as complex pairs, fp64 step sums), wide ones none; a given but
    short workspace is refused before any HIP call."""
    P = FAKE
    narrow = B.make_desc(1, 1 << 20, 256, 16, B.SS_BF16, B.SS_F32)
    nb = B.ss_scan_workspace_bytes(narrow, B.SS_OP_FWD_COMPLEX)
    # about 1280 workgroups of 32 channels: 160 chunks, the last without a summary slot
    assert nb > 0 and nb % 256 == 0
    assert nb >= 160 * 16 * 256 * 8 + 160 * 256 * 8
    assert B.ss_scan_workspace_bytes(B.make_desc(8, 2048, 5120, 16), B.SS_OP_FWD_COMPLEX) == 0
    assert B.ss_scan_workspace_bytes(B.make_desc(1, 200, 64, 16), B.SS_OP_FWD_COMPLEX) == 0
    args = [P, P + 256, P + 512, P + 1024, P + 1536, None, None, None, None, P + 4096, None]
    assert B.ss_scan_fwd_complex_ws(narrow, *args, P + 8192, nb - 1, stream=0) == B.SS_ERR_WORKSPACE
    assert B.ss_scan_fwd_complex_ws(narrow, *args, P + 8200, nb, stream=0) == B.SS_ERR_WORKSPACE
    bad = list(args)
    bad[0] = None
    assert B.ss_scan_fwd_complex_ws(narrow, *bad, P + 8192, nb, stream=0) == B.SS_ERR_INVALID_ARG


def test_bc_stride_validation_and_plan(lib):
    """Strided B/C rows (column ranges of the input projection's output): the
    stride is bounded, the rows are copied into the workspace (so a strided
    view at a dense N = 16 still needs it), Bm and Cm then need only element
    alignment, and the complex-A entry points refuse a stride.  Every call here
    stops at a host check before any HIP call."""
    P = FAKE
    for bad in (-1, 15, (1 << 20) + 1):
        assert fwd(desc(bc_stride=bad)) == B.SS_ERR_INVALID_ARG, bad
    assert fwd(desc(dstate=8, bc_stride=7)) == B.SS_ERR_INVALID_ARG
    rows = 2 * 8 * 2048 * 16 * 2             # B and C rows, 16 bf16 entries per (b, t)
    for s in (16, 48, 1 << 20):
        d = desc(batch=8, seqlen=2048, dim=5120, bc_stride=s)
        assert B.ss_scan_workspace_bytes(d, B.SS_OP_FWD) == rows, s
    wide = desc(batch=8, seqlen=2048, dim=5120)
    dense_bwd = B.ss_scan_workspace_bytes(wide, B.SS_OP_BWD)
    assert B.ss_scan_workspace_bytes(desc(batch=8, seqlen=2048, dim=5120, bc_stride=48),
                                     B.SS_OP_BWD) == dense_bwd + rows
    # alignment: dense rows need 16 bytes; strided rows their element size.  The
    # workspace check that follows the alignment check tells the two apart.
    d = desc(batch=8, seqlen=2048, dim=5120, bc_stride=48)
    assert fwd(d, Bm=P + 2, Cm=P + 34) == B.SS_ERR_WORKSPACE            # bf16: 2-byte aligned
    assert fwd(d, Bm=P + 1) == B.SS_ERR_INVALID_ARG
    assert fwd(desc(batch=8, seqlen=2048, dim=5120, bc_stride=48, in_dtype=B.SS_F32),
               Bm=P + 2) == B.SS_ERR_INVALID_ARG                         # f32 needs 4
    assert fwd(desc(batch=8, seqlen=2048, dim=5120, bc_stride=48, in_dtype=B.SS_F32),
               Bm=P + 4, Cm=P + 68) == B.SS_ERR_WORKSPACE
    assert fwd(wide, Bm=P + 2) == B.SS_ERR_INVALID_ARG                  # dense: 16 bytes
    bwd_args = [P, P, P, P + 2, P + 34, None, None, None, None, P, P, P, P, P, P, None, None,
                None, None, None, 0]
    assert B.ss_scan_bwd(d, *bwd_args, stream=0) == B.SS_ERR_WORKSPACE
    bwd_args[3] = P + 1
    assert B.ss_scan_bwd(d, *bwd_args, stream=0) == B.SS_ERR_INVALID_ARG
    assert B.ss_scan_bwd(wide, *(bwd_args[:3] + [P + 2] + bwd_args[4:]), stream=0) == \
        B.SS_ERR_INVALID_ARG
    # the step: stride bounds and alignment (acceptance needs a device: GPU tests)
    step = lambda dd, **kw: B.ss_scan_step(  # noqa: E731
        dd, P + 8192, P, P + 256, P + 512, kw.get("Bm", P + 1024), kw.get("Cm", P + 1536), None,
        None, None, P + 4096, stream=0)
    assert step(B.make_desc(2, 1, 64, 16, B.SS_BF16, B.SS_F32, bc_stride=8)) == \
        B.SS_ERR_INVALID_ARG
    assert step(B.make_desc(2, 1, 64, 16, B.SS_BF16, B.SS_F32, bc_stride=40), Bm=P + 1025) == \
        B.SS_ERR_INVALID_ARG
    # complex A: dense rows only
    cd = B.make_desc(2, 64, 32, 16, B.SS_F32, B.SS_F32, bc_stride=48)
    cargs = [P, P + 256, P + 512, P + 1024, P + 1536, None, None, None, None, P + 4096, None]
    assert B.ss_scan_fwd_complex(cd, *cargs, stream=0) == B.SS_ERR_UNSUPPORTED
    assert B.ss_scan_workspace_bytes(cd, B.SS_OP_FWD_COMPLEX) == 0
    assert B.ss_scan_step_complex(B.make_desc(2, 1, 64, 16, B.SS_BF16, B.SS_F32, bc_stride=48),
                                  P + 8192, P, P + 256, P + 512, P + 1024, P + 1536, None, None,
                                  None, P + 4096, stream=0) == B.SS_ERR_UNSUPPORTED
    assert B.ss_scan_version() >= 20000


def test_binding_row_stride():
    """The binding's reading of torch strides into ss_desc_t.bc_stride (host
    only): column ranges of one projection output share a stride; dense rows
    give 0 when 16-byte aligned, else their own stride; uneven rows are refused."""
    import torch
    x = torch.zeros(2, 5, 40)
    assert B._bc_stride(x[:, :, 8:24], x[:, :, 24:40], 16) == 40
    assert B._bc_stride(torch.zeros(2, 5, 16), torch.zeros(2, 5, 16), 16) == 0
    assert B._bc_stride(x[:, :, 9:19], x[:, :, 19:29], 10) == 40
    s = torch.zeros(3, 40)
    assert B._bc_stride(s[:, 8:24], s[:, 24:40], 16) == 40          # step rows (B, N)
    one = torch.zeros(1, 1, 40)
    assert B._bc_stride(one[:, :, 8:24], one[:, :, 24:40], 16) == 0  # one row, aligned
    assert B._bc_stride(one[:, :, 1:17], one[:, :, 17:33], 16) == 16  # one row, misaligned
    t = torch.zeros(2, 5, 16).transpose(0, 1)
    with pytest.raises(ValueError):
        B._bc_stride(t, t, 16)
    with pytest.raises(ValueError):
        B._bc_stride(x[:, :, 8:24], torch.zeros(2, 5, 16), 16)      # different strides
    with pytest.raises(ValueError):
        B._bc_stride(x[:, :, 0:40:2], x[:, :, 1:40:2], 20)          # last axis not unit


def test_binding_refuses_strided_dense_args():
    """The torch-level wrappers refuse non-contiguous views where the library reads
    dense rows (everything but strided B, C), before any library call."""
    import torch
    u = torch.zeros(2, 8, 32)
    A = torch.zeros(32, 16)
    Bm = torch.zeros(2, 8, 16)
    bad = torch.zeros(2, 32, 8).transpose(1, 2)          # (2, 8, 32), not contiguous
    with pytest.raises(ValueError, match="u must be contiguous"):
        B.scan_fwd(bad, u, A, Bm, Bm)
    with pytest.raises(ValueError, match="delta must be contiguous"):
        B.scan_fwd(u, bad, A, Bm, Bm)
    with pytest.raises(ValueError, match="dy must be contiguous"):
        B.scan_bwd(u, u, A, Bm, Bm, bad)
    with pytest.raises(ValueError, match="B must be contiguous"):
        B.scan_fwd_complex(u, u, torch.zeros(32, 16, 2), torch.zeros(2, 16, 8, 2).transpose(1, 2),
                           torch.zeros(2, 8, 16, 2))
    with pytest.raises(ValueError, match="x must be contiguous"):
        B.conv1d_fwd(bad, torch.zeros(32, 4))
    with pytest.raises(ValueError, match="x must be contiguous"):
        B.ssd_fwd(torch.zeros(2, 8, 64, 3).transpose(2, 3), torch.zeros(2, 8, 3),
                  torch.zeros(3), torch.zeros(2, 8, 1, 64), torch.zeros(2, 8, 1, 64))


def test_binding_structs_match_headers(tmp_path):
    """The ctypes descriptors have the C layout: a C program built against the
    headers prints each struct's size and field offsets, which must equal the
    binding's (a mismatch would hand the library shifted fields)."""
    import ctypes
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"ss_desc_t": B.ss_desc_t, "ss_conv_desc_t": B.ss_conv_desc_t,
               "ss_ssd_desc_t": B.ss_ssd_desc_t}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ss_scan.h"',
             '#include "ss_conv.h"', '#include "ss_ssd.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append('  printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for fname, _ in py._fields_:
            lines.append('  printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, fname, cname, fname))
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.check_call([cc, "-std=c99", "-I", INCLUDE, str(src), "-o", str(exe)])
    out = subprocess.check_output([str(exe)]).decode().split("\n")
    got = {}
    for line in out:
        if line.strip():
            parts = line.split()
            got[tuple(parts[:-1])] = int(parts[-1])
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_noalloc_scratch_limit_with_strided_rows(lib):
    """Strided B/C rows are copied into the scratch: a long problem with a row
    stride exceeds the static array where the dense one needs none."""
    P = FAKE
    args = [P, P + 256, P + 512, P + 1026, P + 1538, None, None, None, None, P + 4096, None]
    dense = B.make_desc(1, 1 << 20, 5120, 16, B.SS_BF16, B.SS_F32)
    strided = B.make_desc(1, 1 << 20, 5120, 16, B.SS_BF16, B.SS_F32, bc_stride=48)
    assert B.ss_scan_workspace_bytes(dense, B.SS_OP_FWD) <= B.SS_SCAN_STATIC_SCRATCH_BYTES
    assert B.ss_scan_workspace_bytes(strided, B.SS_OP_FWD) > B.SS_SCAN_STATIC_SCRATCH_BYTES
    assert B.ss_scan_fwd_noalloc(strided, *args, stream=0) == B.SS_ERR_SCRATCH_LIMIT
