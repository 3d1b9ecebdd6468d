"""Selective-scan benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-extra]
                    [--no-cold]

A step is one forward selective scan (steps a1-a8 of the hot path: loads,
softplus, on-the-fly discretisation, recurrence, C contraction, D skip, gate)
over one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the Mamba-2.8B-shaped layer (B=8, L=2048, D=5120, N=16, bf16 inputs,
fp32 state and output, exact ZOH).  The backward and decode-step rows are timed
on their own workloads and reported under "extra".

Prints ONE JSON line.  value = scanned elements (B*L*D*N) per second.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
SIMD_LANES = 256 * 4 * 16      # CUs x SIMDs x lanes
CLOCK_HZ = 2.4e9
VALU_PEAK_TSLOT = SIMD_LANES * CLOCK_HZ / 1e12   # 39.32 T lane-slots/s (non-packed fp32)
# minimal VALU issue slots per scanned element (b, t, d, n): one v_exp_f32 (2 slots,
# half rate on gfx950) + 4 (Euler) or 6 (exact ZOH) single-slot vector ops
SLOTS_PER_ELEM = {"euler": 6.0, "zoh": 8.0}
# complex state (exact ZOH): v_exp_f32, v_sin_f32, v_cos_f32 (2 slots each) and 22
# single-slot ops (dt a_re, dt a_im, fract, |abar| (cos, sin), (abar - 1) / a, B u,
# bcoef B u, abar h + ., Re(C h))
COMPLEX_SLOTS = 28.0


# sources the benchmark's dominant kernel (the 32-channel forward) and its
# launch are built from: a change to the code of any of them voids its stored
# traffic figure (comments and layout do not count)
HEADLINE_SOURCES = ("ss_device.hpp", "ss_fwd_common.hpp", "ss_fwd_hw.hpp", "ss_fwd_hw.hip",
                    "ss_fwd_hw_dispatch.inc", "ss_fwd.hip", "ss_internal.h")


def _code_tokens(text):
    """C++ source without comments, with runs of whitespace collapsed (string
    literals in these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_69_amd", "csrc")
    for f in HEADLINE_SOURCES:
        h.update(_code_tokens(open(os.path.join(csrc, f)).read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def algorithmic_bytes(w, in_bytes=2, out_bytes=4):
    """Each input read once, y written once: u, delta, z (B,L,D), B and C (B,L,N),
    A (D,N), D_skip and bias (D)."""
    bld = w.B * w.L * w.D
    bln = w.B * w.L * w.N
    return bld * (3 * in_bytes + out_bytes) + 2 * bln * in_bytes + w.D * (w.N + 2) * 4


def load_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    e = d.get(name)
    if not e or e.get("kernel_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def upload(inp, torch):
    it = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    cv = lambda x, dt: None if x is None else torch.from_numpy(x).to("cuda").to(dt).contiguous()  # noqa
    return dict(u=cv(inp.u, it), delta=cv(inp.delta, it), A=cv(inp.A, torch.float32),
                B=cv(inp.B, it), C=cv(inp.C, it), D=cv(inp.D, torch.float32),
                delta_bias=cv(inp.delta_bias, torch.float32), z=cv(inp.z, it),
                dy=cv(inp.dy, it))


# The GPU's clocks ramp up over the first ~50 ms of sustained load (a forward at
# the Mamba-2.8B shape takes 0.8 ms per call for the first 20 calls, 0.44 ms from
# about the 100th).  Every timed region is therefore preceded by at least
# `warmup` untimed calls and at least WARM["min_s"] seconds of them.
WARM = {"min_s": 0.3, "last_calls": 0}


def time_calls(fn, steps, warmup, torch):
    """Warm up, then time `steps` calls: total wall (events around the whole region)
    and the mean per-call duration from events around each call (same stream)."""
    n, t0 = 0, time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < WARM["min_s"]:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()   # keep the host clock in step with the GPU
    WARM["last_calls"] = n
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    total_ms = ev[0].elapsed_time(ev[steps])
    return total_ms, sum(per) / len(per), min(per), wall


def time_flushed(fn, torch, runs=20, flush_bytes=512 << 20):
    """Per-call times with the caches flushed: each run writes flush_bytes of scratch
    memory, then times one call (events around the call only), then times a second
    call right after it with nothing in between, as a control taken under the same
    stop-and-go clock conditions.  Returns (flushed median, flushed min, control
    median) in ms."""
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")

    def one():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    cold, ctrl = [], []
    for i in range(runs):
        scratch.fill_(float(i))
        cold.append(one())
        ctrl.append(one())
    del scratch
    cold.sort()
    ctrl.sort()
    return cold[len(cold) // 2], cold[0], ctrl[len(ctrl) // 2]


def stream_gbs(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy bandwidth (bytes read + written per second): the
    achievable streaming rate of this GPU, a second reference beside the 8 TB/s peak."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(inp, w, budget_s=20.0):
    """The fp64 oracle on the same workload: whole batch rows, as many as fit in
    about budget_s seconds (all of them when the estimate allows)."""
    from oracle import oracle
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    # the host's CPU share for one GPU (OMP_NUM_THREADS on the GPU hosts), at
    # most the cores this process may run on
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    threads = max(1, min(share, affinity))

    def run(rows):
        sl = slice(0, rows)
        t0 = time.perf_counter()
        oracle.fwd(inp.u[sl], inp.delta[sl], inp.A, inp.B[sl], inp.C[sl], D=inp.D,
                   delta_bias=inp.delta_bias, z=None if inp.z is None else inp.z[sl],
                   disc=w.disc, nthreads=threads)
        return time.perf_counter() - t0

    if w.L * w.D > 64 * 1024 * 1024:          # one row alone is large: sample channels
        nch = max(1, min(w.D, int(w.D * budget_s / 60.0)))
        sl = (slice(0, 1), slice(None), slice(0, nch))
        t0 = time.perf_counter()
        oracle.fwd(inp.u[sl], inp.delta[sl], inp.A[:nch], inp.B[:1], inp.C[:1], D=inp.D[:nch],
                   delta_bias=inp.delta_bias[:nch], z=inp.z[sl], disc=w.disc, nthreads=threads)
        dt = time.perf_counter() - t0
        elems, what = w.L * nch * w.N, "batch row 0, channels 0..%d of %d" % (nch - 1, w.D)
    else:
        dt1 = run(1)
        rows = int(max(1, min(w.B, budget_s / max(dt1, 1e-3))))
        dt = run(rows) if rows > 1 else dt1
        elems, what = rows * w.L * w.D * w.N, "batch rows 0..%d of %d (all channels)" % (rows - 1, w.B)
    res = {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
           "sample": "%s, full L=%d, N=%d, %s: %.2f s of fp64 C (OpenMP over channels)" % (
               what, w.L, w.N, w.disc, dt)}
    # the same code on one thread, over a smaller sample (4096 channels of batch row 0)
    nch = min(w.D, 4096)
    sl = (slice(0, 1), slice(None), slice(0, nch))
    t0 = time.perf_counter()
    oracle.fwd(inp.u[sl], inp.delta[sl], inp.A[:nch], inp.B[:1], inp.C[:1], D=inp.D[:nch],
               delta_bias=inp.delta_bias[:nch], z=None if inp.z is None else inp.z[sl],
               disc=w.disc, nthreads=1)
    dt1 = time.perf_counter() - t0
    res["single_thread"] = {"value": w.L * nch * w.N / dt1, "unit": "elements/s",
                            "sample": "batch row 0, channels 0..%d, full L=%d: %.2f s" % (
                                nch - 1, w.L, dt1)}
    res["cpu_model"] = cpu_model()
    res["host_cpus"] = {"nproc": os.cpu_count(), "affinity": affinity, "omp_share": share}
    res["other_rows"] = cpu_rows(oracle, threads)
    return res


def cpu_rows(oracle, threads):
    """The oracle beside the other rows: each on a bounded sample drawn with the
    row's own recipe (same L, N and distributions, fewer batch rows, channels or
    heads), repeated for at least 0.5 s, reported in the row's unit."""
    import numpy as np

    def timed(run, min_s=0.5):
        """seconds per call, the call repeated until min_s has passed"""
        n, t0 = 0, time.perf_counter()
        while True:
            run()
            n += 1
            el = time.perf_counter() - t0
            if el >= min_s:
                return el / n

    out = {}
    # backward, Mamba-130M recipe: batch row 0, 192 channels (one thread: the oracle's
    # backward is serial)
    w = synth_mod().WORKLOADS["bwd_130m_bf16_b8_l2048_d1536"]
    nch = 192
    inp = synth_mod().make_inputs(1, w.L, nch, w.N, w.seed, w.dtype, w.dt_range, with_dy=True)
    for disc in ("euler", "zoh"):
        dt = timed(lambda: oracle.bwd(inp.u, inp.delta, inp.A, inp.B, inp.C, D=inp.D,
                                      delta_bias=inp.delta_bias, z=inp.z, g=inp.dy, disc=disc))
        out["bwd_130m:" + disc] = {"value": w.L * nch * w.N / dt, "unit": "elements/s",
                                   "threads": 1, "sample": "1 x %d x %d, N=%d: %.3f s per call" % (
                                       w.L, nch, w.N, dt)}
    # decode step at B=8, D=5120, N=16 (one thread)
    st = synth_mod().make_inputs(8, 1, 5120, 16, 9, "bf16", with_h0=True)
    dt = timed(lambda: oracle.step(st.h0, st.u[:, 0], st.delta[:, 0], st.A, st.B[:, 0],
                                   st.C[:, 0], D=st.D, delta_bias=st.delta_bias, z=st.z[:, 0]))
    out["step_b8_d5120"] = {"value": dt * 1e6, "unit": "us per step", "threads": 1,
                            "sample": "the whole step"}
    # Conv1d (width 4) + SiLU, Mamba-2.8B recipe: batch row 0, 1024 channels, full L
    rng = np.random.default_rng(1002)
    x = synth_mod().round_to_bf16(rng.standard_normal((1, 2048, 1024)).astype(np.float32))
    cw = (rng.standard_normal((1024, 4)) * 0.5).astype(np.float32)
    cb = (rng.standard_normal(1024) * 0.3).astype(np.float32)
    g = rng.standard_normal((1, 2048, 1024)).astype(np.float32)
    dt = timed(lambda: oracle.conv1d_fwd(x, cw, cb))
    out["conv1d_fwd_b8_l2048_d5120"] = {"value": x.size / dt, "unit": "elements/s (b, t, d)",
                                        "threads": 1, "sample": "1 x 2048 x 1024: %.3f s per call" % dt}
    dt = timed(lambda: oracle.conv1d_bwd(x, cw, g, cb))
    out["conv1d_bwd_b8_l2048_d5120"] = {"value": x.size / dt, "unit": "elements/s (b, t, d)",
                                        "threads": 1, "sample": "1 x 2048 x 1024: %.3f s per call" % dt}
    # SSD layer, its workload recipe: one batch row, all heads
    sw = synth_mod().SSD_WORKLOAD
    si = synth_mod().make_ssd_inputs(1, sw["L"], sw["H"], sw["P"], sw["N"], 1, sw["seed"])
    dt = timed(lambda: oracle.ssd_fwd(si.x, si.dt, si.A, si.B, si.C, D=si.D, dt_bias=si.dt_bias,
                                      nthreads=threads))
    out["ssd_bf16_b8_l2048_h80_p64_n64_g1"] = {
        "value": sw["L"] / dt, "unit": "tokens/s", "threads": threads,
        "sample": "1 x %d tokens, %d heads: %.3f s per call" % (sw["L"], sw["H"], dt)}
    # complex A, S4D-Lin recipe: batch row 0, 2048 channels, full L, N=16
    ci = synth_mod().make_complex_inputs(1, 2048, 2048, 16, seed=1002, dtype="bf16")
    dt = timed(lambda: oracle.fwd_complex(ci.u, ci.delta, ci.A, ci.B, ci.C, D=ci.D,
                                          delta_bias=ci.delta_bias, z=ci.z, nthreads=threads))
    out["complex_2p8b_s4dlin"] = {"value": 2048 * 2048 * 16 / dt, "unit": "elements/s",
                                  "threads": threads, "sample": "1 x 2048 x 2048: %.3f s per call" % dt}
    return out


def synth_mod():
    from selective_state_space_69_amd import synth
    return synth


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A plain device copy of known size, to calibrate the FETCH_SIZE / WRITE_SIZE
    counters (run under rocprofv3 --pmc)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warmup-s", type=float, default=WARM["min_s"],
                    help="untimed warm-up lasts at least this long (GPU clock ramp)")
    ap.add_argument("--workload", default="fwd_2p8b_bf16_b8_l2048_d5120")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cache-flushed timing and the copy bandwidth (profiling runs: "
                         "the timed calls are then the last dispatches of the headline kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--only", choices=["bwd", "step", "conv", "ssd", "bidir", "complex"],
                    help="only time the backward (Mamba-130M shape), the decode step or the "
                         "Conv1d + SiLU and print their figures (for profiling runs)")
    args = ap.parse_args()
    WARM["min_s"] = args.min_warmup_s
    if args.gpus != 1:
        print("bench.py measures one GPU only: the selective scan needs no communication "
              "(every (b, d) channel is independent) and the library has no multi-GPU path; "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from selective_state_space_69_amd import binding as Bnd
    from selective_state_space_69_amd import synth

    Bnd.load_library()
    if args.only == "bwd":
        print(json.dumps(time_bwd(torch, Bnd, synth, args.steps, args.warmup)), flush=True)
        return
    if args.only == "step":
        print(json.dumps(time_step(torch, Bnd, synth)), flush=True)
        return
    if args.only == "conv":
        print(json.dumps(time_conv(torch, Bnd, synth, args.steps, args.warmup)), flush=True)
        return
    if args.only == "complex":
        print(json.dumps(time_complex(torch, Bnd, synth, args.steps, args.warmup)), flush=True)
        return
    if args.only == "bidir":
        print(json.dumps(time_bidir(torch, Bnd, synth, args.steps, args.warmup)), flush=True)
        return
    if args.only == "ssd":
        print(json.dumps(time_ssd(torch, Bnd, synth, args.steps, args.warmup)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    inp = synth.make_workload(w.name, with_dy=False)
    d = upload(inp, torch)
    out_dt = torch.float32
    y = torch.empty(d["u"].shape, dtype=out_dt, device="cuda")
    desc = Bnd.make_desc(w.B, w.L, w.D, w.N, Bnd.SS_BF16 if w.dtype == "bf16" else Bnd.SS_F32,
                         Bnd.SS_F32, Bnd.SS_ZOH if w.disc == "zoh" else Bnd.SS_EULER, True)
    nb = Bnd.ss_scan_workspace_bytes(desc, Bnd.SS_OP_FWD)
    ws = Bnd.workspace(nb, "cuda")

    def step():
        rc = Bnd.ss_scan_fwd(desc, d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                             d["delta_bias"], d["z"], None, y, None, ws, nb)
        if rc != 0:
            raise RuntimeError(Bnd.ss_scan_strerror(rc))

    torch.cuda.synchronize()
    total_ms, per_ms, min_ms, wall = time_calls(step, args.steps, args.warmup, torch)
    warm_calls = WARM["last_calls"]
    torch.cuda.synchronize()
    elems = w.elements
    value = elems * args.steps / (total_ms * 1e-3)
    alg = algorithmic_bytes(w, 2 if w.dtype == "bf16" else 4, 4)
    hbm_gbs = alg / (per_ms * 1e-3) / 1e9
    slots = SLOTS_PER_ELEM[w.disc] * elems / (per_ms * 1e-3) / 1e12
    # The roofline is HBM bandwidth: algorithmic bytes (each input read once,
    # y written once) over the mean per-call time, against the 8 TB/s peak.  The
    # VALU lane-slot figure beside it is a model (minimal vector issue slots per
    # element at the published clock), not a measured peak.
    roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic(w.name),
            "algorithmic_bytes": alg,
            "kernel_ms": round(per_ms, 4), "kernel_ms_min": round(min_ms, 4),
            "alu_model": {"achieved": round(slots, 3), "peak": round(VALU_PEAK_TSLOT, 3),
                          "unit": "Tslot/s", "frac": round(slots / VALU_PEAK_TSLOT, 4),
                          "work_per_element": "%s: %d VALU lane-slots (model: 1 v_exp_f32 = 2 "
                                              "slots), 256 CUs x 64 lanes x 2.4 GHz" % (
                                                  w.disc, SLOTS_PER_ELEM[w.disc])}}
    res = {"metric": "selective-scan elements (B*L*D*N)/s, 1 GPU", "value": value,
           "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": warm_calls,
           "warmup_requested": args.warmup, "warmup_min_s": WARM["min_s"],
           "ms_per_step": total_ms / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "L": w.L, "D": w.D, "N": w.N,
                      "in_dtype": w.dtype, "out_dtype": "f32", "disc": w.disc,
                      "plan_workspace_bytes": nb},
           "roofline": roof}
    # the same call with the caches flushed before each run, and the copy bandwidth
    if not args.no_cold:
        cold_med, cold_min, ctrl_med = time_flushed(step, torch)
        sgbs = stream_gbs(torch)
        roof["cold"] = {"median_ms": round(cold_med, 4), "min_ms": round(cold_min, 4),
                        "control_median_ms": round(ctrl_med, 4), "flush_bytes": 512 << 20,
                        "runs": 20}
        roof["stream_gbs"] = round(sgbs, 1)
        roof["frac_of_stream"] = round(hbm_gbs / sgbs, 4)
        roof["graph"] = time_graph(step, torch)
    del d, y, ws
    torch.cuda.empty_cache()

    if not args.no_extra:
        res["extra"] = extras(torch, Bnd, synth, args)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(inp, w)
    print(json.dumps(res), flush=True)


def time_graph(step, torch, calls=20, replays=5):
    """The same call captured 20 times in one graph and replayed: the per-call
    time without the host's launches between calls (informational; value is the
    eagerly launched loop)."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                step()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (calls * replays)
        del g
        return {"ms_per_call": round(ms, 4), "calls_per_replay": calls, "replays": replays}
    except Exception as exc:   # informational: never fail the benchmark over it
        return {"error": str(exc)[:200]}


def extras(torch, Bnd, synth, args):
    """Other rows of the hot path, each on its own workload (not part of value)."""
    out = {}
    steps, warm = max(5, args.steps // 2), 2
    # forward on the other forward workloads
    for name in ("fwd_2p8b_bf16_b8_l2048_d5120:euler", "fwd_130m_bf16_b8_l2048_d1536",
                 "fwd_2p8b_bf16_b2_l8192_d5120", "fwd_long_bf16_b1_l1048576_d256"):
        wname, _, disc = name.partition(":")
        w = synth.WORKLOADS[wname]
        disc = disc or w.disc
        inp = synth.make_workload(wname, with_dy=False)
        d = upload(inp, torch)
        y = torch.empty(d["u"].shape, dtype=torch.float32, device="cuda")
        desc = Bnd.make_desc(w.B, w.L, w.D, w.N, Bnd.SS_BF16, Bnd.SS_F32,
                             Bnd.SS_ZOH if disc == "zoh" else Bnd.SS_EULER, True)
        nb = Bnd.ss_scan_workspace_bytes(desc, Bnd.SS_OP_FWD)
        ws = Bnd.workspace(nb, "cuda")
        f = lambda: Bnd.ss_scan_fwd(desc, d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],  # noqa
                                    d["delta_bias"], d["z"], None, y, None, ws, nb)
        total, per, mn, _ = time_calls(f, steps, warm, torch)
        alg = algorithmic_bytes(w)
        out[name] = {"ms": round(per, 4), "elements_per_s": w.elements / (per * 1e-3),
                     "hbm_gbs": round(alg / (per * 1e-3) / 1e9, 1),
                     "hbm_frac": round(alg / (per * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "alu_model_frac": round(SLOTS_PER_ELEM[disc] * w.elements / (per * 1e-3) / 1e12
                                       / VALU_PEAK_TSLOT, 4),
                     "chunks": "workspace %d B" % nb}
        del d, y, ws, inp
        torch.cuda.empty_cache()
    out.update(time_bwd(torch, Bnd, synth, steps, warm))
    out.update(time_step(torch, Bnd, synth))
    out.update(time_conv(torch, Bnd, synth, steps, warm))
    out.update(time_ssd(torch, Bnd, synth, steps, warm))
    out.update(time_bidir(torch, Bnd, synth, steps, warm))
    out.update(time_complex(torch, Bnd, synth, steps, warm))
    return out


def time_conv(torch, Bnd, synth, steps, warm):
    """Causal depthwise Conv1d (width 4) + SiLU at the Mamba-2.8B shape (B=8,
    L=2048, D=5120): forward bf16 -> bf16, backward (fp32 du and dx), and the
    decode step.  HBM-bound: reported against the algorithmic bytes."""
    import numpy as np
    Bt, L, D, K = 8, 2048, 5120, 4
    rng = np.random.default_rng(1002)
    x = torch.from_numpy(synth.round_to_bf16(rng.standard_normal((Bt, L, D)).astype(np.float32)))
    x = x.to("cuda").to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((D, K)) * 0.5).astype(np.float32)).cuda()
    b = torch.from_numpy((rng.standard_normal(D) * 0.3).astype(np.float32)).cuda()
    du = torch.randn((Bt, L, D), device="cuda")
    u = torch.empty_like(x)
    desc = Bnd.make_conv_desc(Bt, L, D, K, Bnd.SS_BF16, Bnd.SS_BF16, True)
    f = lambda: Bnd.ss_conv1d_fwd(desc, x, w, b, u)  # noqa
    total, per, mn, _ = time_calls(f, steps, warm, torch)
    n = Bt * L * D
    alg_f = n * (2 + 2) + D * (K + 1) * 4
    out = {"conv1d_fwd_b8_l2048_d5120": {"ms": round(per, 4), "ms_min": round(mn, 4),
                                          "hbm_gbs": round(alg_f / (per * 1e-3) / 1e9, 1),
                                          "hbm_frac": round(alg_f / (per * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                          "algorithmic_bytes": alg_f}}
    dx = torch.empty((Bt, L, D), device="cuda")
    dw = torch.empty((D, K), device="cuda")
    db = torch.empty(D, device="cuda")
    bdesc = Bnd.make_conv_desc(Bt, L, D, K, Bnd.SS_BF16, Bnd.SS_F32, True)
    nb = Bnd.ss_conv1d_workspace_bytes(bdesc)
    ws = Bnd.workspace(nb, "cuda")
    f = lambda: Bnd.ss_conv1d_bwd(bdesc, x, w, b, du, dx, dw, db, ws, nb)  # noqa
    total, per, mn, _ = time_calls(f, steps, warm, torch)
    alg_b = n * (2 + 4 + 4) + D * (K + 1) * 4 * 2
    out["conv1d_bwd_b8_l2048_d5120"] = {"ms": round(per, 4), "ms_min": round(mn, 4),
                                         "hbm_gbs": round(alg_b / (per * 1e-3) / 1e9, 1),
                                         "hbm_frac": round(alg_b / (per * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                         "algorithmic_bytes": alg_b}
    del x, u, du, dx, ws
    torch.cuda.empty_cache()
    return out


def time_ssd(torch, Bnd, synth, steps, warm):
    """SSD (Mamba-2) layer forward, 8 x 2048 tokens, 80 heads of 64 channels,
    64 states, one B/C group; fp32 and bf16 output.  Algorithmic bytes: x, dt,
    B, C read once, y written once; algorithmic flops of the chunked form
    (Q = 64): per token and head Q (N + P) for the causal C B^T and M x
    blocks plus 4 N P for C H and the state update."""
    w = synth.SSD_WORKLOAD
    Bt, L, H, P, N, G = (w[k] for k in ("Bt", "L", "H", "P", "N", "G"))
    inp = synth.make_ssd_inputs(Bt, L, H, P, N, G, w["seed"])
    bf, f32 = torch.bfloat16, torch.float32
    dev = lambda a, t: torch.from_numpy(a).to("cuda").to(t).contiguous()  # noqa
    x, dt, Bm, Cm = (dev(a, bf) for a in (inp.x, inp.dt, inp.B, inp.C))
    A, Dh, bias = (dev(a, f32) for a in (inp.A, inp.D, inp.dt_bias))
    out = {}
    toks = Bt * L
    flops = toks * H * (64 * (N + P) + 4 * N * P)
    for od, ob in ((Bnd.SS_F32, 4), (Bnd.SS_BF16, 2)):
        y = torch.empty(x.shape, dtype=f32 if od == Bnd.SS_F32 else bf, device="cuda")
        desc = Bnd.make_ssd_desc(Bt, L, H, P, N, G, Bnd.SS_BF16, od, True)
        f = lambda: Bnd.ss_ssd_fwd(desc, x, dt, A, Bm, Cm, Dh, bias, y)  # noqa
        total, per, mn, _ = time_calls(f, steps, warm, torch)
        alg = toks * H * P * (2 + ob) + toks * H * 2 + 2 * toks * G * N * 2 + 3 * H * 4
        out["%s:y_%s" % (w["name"], "f32" if od == Bnd.SS_F32 else "bf16")] = {
            "ms": round(per, 4), "ms_min": round(mn, 4), "tokens_per_s": toks / (per * 1e-3),
            "hbm_gbs": round(alg / (per * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg / (per * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(flops / (per * 1e-3) / 1e12, 1), "algorithmic_bytes": alg}
        del y
    # from a start state, keeping the final state, in place (a prefill that
    # continues a sequence): the state is read and written once more
    h = torch.zeros((Bt, H, N, P), dtype=f32, device="cuda")
    y = torch.empty(x.shape, dtype=f32, device="cuda")
    desc = Bnd.make_ssd_desc(Bt, L, H, P, N, G, Bnd.SS_BF16, Bnd.SS_F32, True)
    f = lambda: Bnd.ss_ssd_fwd_state(desc, x, dt, A, Bm, Cm, Dh, bias, h, y, h)  # noqa
    total, per, mn, _ = time_calls(f, steps, warm, torch)
    alg = toks * H * P * (2 + 4) + toks * H * 2 + 2 * toks * G * N * 2 + 3 * H * 4
    alg += 2 * Bt * H * N * P * 4
    out["%s:y_f32_state_in_out" % w["name"]] = {
        "ms": round(per, 4), "ms_min": round(mn, 4), "tokens_per_s": toks / (per * 1e-3),
        "hbm_gbs": round(alg / (per * 1e-3) / 1e9, 1),
        "hbm_frac": round(alg / (per * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "tflops": round(flops / (per * 1e-3) / 1e12, 1), "algorithmic_bytes": alg}
    del x, dt, Bm, Cm, h, y
    torch.cuda.empty_cache()
    out.update(time_ssd_step(torch, Bnd, synth))
    return out


def time_ssd_step(torch, Bnd, synth):
    """SSD decode step: 256 rows x 80 heads of 64 channels, 64 states; the
    state (256, 80, 64, 64) fp32 is 336 MB, more than the last-level cache, and
    is read and written once per step.  100 steps captured in one graph."""
    Bt, H, P, N, G = 256, 80, 64, 64, 1
    inp = synth.make_ssd_inputs(Bt, 1, H, P, N, G, seed=2002)
    bf, f32 = torch.bfloat16, torch.float32
    dev = lambda a, t: torch.from_numpy(a).to("cuda").to(t).contiguous()  # noqa
    x, dt, Bm, Cm = (dev(a[:, 0], bf) for a in (inp.x, inp.dt, inp.B, inp.C))
    A, Dh, bias = (dev(a, f32) for a in (inp.A, inp.D, inp.dt_bias))
    h = torch.zeros((Bt, H, N, P), dtype=f32, device="cuda")
    y = torch.empty((Bt, H, P), dtype=f32, device="cuda")
    desc = Bnd.make_ssd_desc(Bt, 1, H, P, N, G, Bnd.SS_BF16, Bnd.SS_F32, True)

    def steps(k):
        for _ in range(k):
            rc = Bnd.ss_ssd_step(desc, h, x, dt, A, Bm, Cm, Dh, bias, y)
            if rc != 0:
                raise RuntimeError(Bnd.ss_scan_strerror(rc))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps(3)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(100)
    total, per, mn, _ = time_calls(g.replay, 10, 2, torch)
    us = per * 10   # 100 steps per replay
    alg = 2 * Bt * H * N * P * 4 + Bt * H * P * (2 + 4) + Bt * H * 2 + 2 * Bt * G * N * 2 + 3 * H * 4
    del g, h, x, dt, Bm, Cm, y
    torch.cuda.empty_cache()
    return {"ssd_step_b256_h80_p64_n64_g1": {
        "us_per_step": round(us, 3), "algorithmic_bytes": alg,
        "hbm_gbs": round(alg / (us * 1e-6) / 1e9, 1),
        "hbm_frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "how": "100 steps captured in one graph, 10 replays"}}


def time_bwd(torch, Bnd, synth, steps, warm):
    """Backward (row a9) at the Mamba-130M shape, both discretisations."""
    out = {}
    w = synth.WORKLOADS["bwd_130m_bf16_b8_l2048_d1536"]
    inp = synth.make_workload(w.name, with_dy=True)
    d = upload(inp, torch)
    for disc in ("euler", "zoh"):
        f = lambda: Bnd.scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dy"],  # noqa
                                 D=d["D"], delta_bias=d["delta_bias"], z=d["z"], disc=disc)
        total, per, mn, _ = time_calls(f, steps, warm, torch)
        bld, bln = w.B * w.L * w.D, w.B * w.L * w.N
        alg = bld * (4 * 2 + 3 * 4) + bln * (2 * 2 + 2 * 4) + w.D * (2 * w.N + 4) * 4
        out["bwd_130m:" + disc] = {"ms": round(per, 4), "elements_per_s": w.elements / (per * 1e-3),
                                   "hbm_gbs": round(alg / (per * 1e-3) / 1e9, 1)}
    del d, inp
    torch.cuda.empty_cache()
    return out


def time_bidir(torch, Bnd, synth, steps, warm):
    """Bidirectional scan at the Mamba-2.8B shape: the forward call, then the
    reverse-time call adding into y (two launches); the reverse call alone too."""
    name = "fwd_2p8b_bf16_b8_l2048_d5120"
    w = synth.WORKLOADS[name]
    inp = synth.make_workload(name)
    d = upload(inp, torch)
    y = torch.empty((w.B, w.L, w.D), dtype=torch.float32, device="cuda")
    desc = Bnd.make_desc(w.B, w.L, w.D, w.N, Bnd.SS_BF16, Bnd.SS_F32, Bnd._DISC[w.disc], True)
    nb = Bnd.ss_scan_workspace_bytes(desc, Bnd.SS_OP_FWD)
    ws = Bnd.workspace(nb, "cuda")
    args = (d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["delta_bias"], d["z"], None, y,
            None, ws, nb)
    rev = lambda acc: Bnd.ss_scan_fwd_dir(desc, Bnd.SS_DIR_REVERSE, acc, *args)  # noqa
    both = lambda: (Bnd.ss_scan_fwd_dir(desc, Bnd.SS_DIR_FORWARD, 0, *args), rev(1))  # noqa
    out = {}
    for key, f, mult in (("bidir_2p8b:fwd+rev_acc", both, 2), ("bidir_2p8b:rev", lambda: rev(0), 1)):
        total, per, mn, _ = time_calls(f, steps, warm, torch)
        out[key] = {"ms": round(per, 4), "ms_min": round(mn, 4),
                    "elements_per_s": mult * w.elements / (per * 1e-3),
                    "alu_model_frac": round(SLOTS_PER_ELEM[w.disc] * mult * w.elements /
                                      (per * 1e-3) / 1e12 / VALU_PEAK_TSLOT, 4)}
    del d, y, ws, inp
    torch.cuda.empty_cache()
    return out


def time_complex(torch, Bnd, synth, steps, warm):
    """Complex-A forward at the Mamba-2.8B shape (B=8, L=2048, D=5120, N=16
    complex states, S4D-Lin A, bf16 in, fp32 out, exact ZOH, gate)."""
    Bt, L, D, N = 8, 2048, 5120, 16
    inp = synth.make_complex_inputs(Bt, L, D, N, seed=1002, dtype="bf16")
    bf, f32 = torch.bfloat16, torch.float32
    cv = lambda x, t: torch.from_numpy(x).to("cuda").to(t).contiguous()  # noqa
    u, dl, Bm, Cm, z = (cv(a, bf) for a in (inp.u, inp.delta, inp.B, inp.C, inp.z))
    A, Dk, bias = (cv(a, f32) for a in (inp.A, inp.D, inp.delta_bias))
    y = torch.empty((Bt, L, D), dtype=f32, device="cuda")
    desc = Bnd.make_desc(Bt, L, D, N, Bnd.SS_BF16, Bnd.SS_F32, Bnd.SS_ZOH, True)
    f = lambda: Bnd.ss_scan_fwd_complex(desc, u, dl, A, Bm, Cm, Dk, bias, z, None, y, None)  # noqa
    total, per, mn, _ = time_calls(f, steps, warm, torch)
    el = Bt * L * D * N
    out = {"complex_2p8b_s4dlin": {"ms": round(per, 4), "ms_min": round(mn, 4),
                                   "elements_per_s": el / (per * 1e-3),
                                   "alu_model_frac": round(COMPLEX_SLOTS * el / (per * 1e-3) / 1e12 /
                                                     VALU_PEAK_TSLOT, 4)}}
    # the same shape with fp32 inputs: every wave on the precise step
    fu, fdl, fB, fC, fz = (cv(a, f32) for a in (inp.u, inp.delta, inp.B, inp.C, inp.z))
    fdesc = Bnd.make_desc(Bt, L, D, N, Bnd.SS_F32, Bnd.SS_F32, Bnd.SS_ZOH, True)
    f = lambda: Bnd.ss_scan_fwd_complex(fdesc, fu, fdl, A, fB, fC, Dk, bias, fz, None, y, None)  # noqa
    total, per, mn, _ = time_calls(f, steps, warm, torch)
    out["complex_2p8b_s4dlin_f32in"] = {"ms": round(per, 4), "ms_min": round(mn, 4),
                                        "elements_per_s": el / (per * 1e-3),
                                        "path": "precise step (fp32 inputs)"}
    del fu, fdl, fB, fC, fz
    torch.cuda.empty_cache()
    # the million-step shape (B=1, L=2^20, D=256): the chunked complex plan
    li = synth.make_complex_inputs(1, 1 << 20, 256, N, seed=1003, dtype="bf16",
                                   dt_range=(1e-4, 1e-2))
    lu, ldl, lB, lC, lz = (cv(a, bf) for a in (li.u, li.delta, li.B, li.C, li.z))
    lA, lD, lbias = (cv(a, f32) for a in (li.A, li.D, li.delta_bias))
    ly = torch.empty((1, 1 << 20, 256), dtype=f32, device="cuda")
    ldesc = Bnd.make_desc(1, 1 << 20, 256, N, Bnd.SS_BF16, Bnd.SS_F32, Bnd.SS_ZOH, True)
    lnb = Bnd.ss_scan_workspace_bytes(ldesc, Bnd.SS_OP_FWD_COMPLEX)
    lws = Bnd.workspace(lnb, "cuda")
    f = lambda: Bnd.ss_scan_fwd_complex_ws(ldesc, lu, ldl, lA, lB, lC, lD, lbias, lz, None, ly,  # noqa
                                           None, lws, lnb)
    total, per, mn, _ = time_calls(f, max(3, steps // 2), warm, torch)
    lel = (1 << 20) * 256 * N
    out["complex_long_b1_l1048576_d256_s4dlin"] = {
        "ms": round(per, 4), "ms_min": round(mn, 4), "elements_per_s": lel / (per * 1e-3),
        "chunks": "workspace %d B" % lnb}
    del lu, ldl, lB, lC, lz, ly, lws, li
    torch.cuda.empty_cache()
    # the decode step on a (B, D, N, 2) state, 100 steps captured in one graph
    h = torch.zeros((Bt, D, N, 2), dtype=f32, device="cuda")
    u1, dl1, z1 = (t[:, 0].contiguous() for t in (u, dl, z))
    B1, C1 = Bm[:, 0].contiguous(), Cm[:, 0].contiguous()
    y1 = torch.empty((Bt, D), dtype=f32, device="cuda")
    sdesc = Bnd.make_desc(Bt, 1, D, N, Bnd.SS_BF16, Bnd.SS_F32, Bnd.SS_ZOH, True)

    def run_steps(k):
        for _ in range(k):
            rc = Bnd.ss_scan_step_complex(sdesc, h, u1, dl1, A, B1, C1, Dk, bias, z1, y1)
            if rc != 0:
                raise RuntimeError(Bnd.ss_scan_strerror(rc))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_steps(3)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_steps(100)
    _, per_g, _, _ = time_calls(g.replay, 10, 2, torch)
    sbytes = Bt * D * N * 2 * 4 * 2
    out["complex_step_b8_d5120_n16"] = {"us_per_step": round(per_g * 10, 3), "state_bytes": sbytes,
                                        "state_gbs": round(sbytes / (per_g * 1e-5) / 1e9, 1),
                                        "how": "100 steps captured in one graph, 10 replays"}
    del g, h, u, dl, Bm, Cm, z, y
    torch.cuda.empty_cache()
    return out


def time_step(torch, Bnd, synth):
    """Decode step (row a10) at the Mamba-2.8B width: a 100-step decode loop
    captured in one graph, so the figure is GPU time per step without the host's
    per-launch cost."""
    Bt, D, N = 8, 5120, 16
    inp = synth.make_inputs(Bt, 1, D, N, seed=77, dtype="bf16", with_h0=True)
    d = upload(inp, torch)
    h = torch.from_numpy(inp.h0).cuda()
    u1, dl1 = (d[k][:, 0].contiguous() for k in ("u", "delta"))
    Bc, Cc, zc = (d[k][:, 0].contiguous() for k in ("B", "C", "z"))
    y1 = torch.empty(Bt, D, dtype=torch.float32, device="cuda")
    sdesc = Bnd.make_desc(Bt, 1, D, N, Bnd.SS_BF16, Bnd.SS_F32, Bnd.SS_ZOH, True)

    def steps(k):
        for _ in range(k):
            rc = Bnd.ss_scan_step(sdesc, h, u1, dl1, d["A"], Bc, Cc, d["D"], d["delta_bias"], zc, y1)
            if rc != 0:
                raise RuntimeError(Bnd.ss_scan_strerror(rc))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps(3)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(100)
    total, per, mn, _ = time_calls(g.replay, 10, 2, torch)
    sbytes = Bt * D * N * 4 * 2
    del g
    return {"step_b8_d5120": {"us_per_step": round(per * 10, 3), "state_bytes": sbytes,
                              "state_gbs": round(sbytes / (per * 1e-5) / 1e9, 1),
                              "how": "100 steps captured in one graph, 10 replays"}}


if __name__ == "__main__":
    main()
