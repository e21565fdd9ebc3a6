#!/usr/bin/env python3
"""Benchmark of the tiled GEMM C = A·Bᵀ on one MI355X.

One step = one GEMM launch over resident device inputs (the whole hot path:
remap, HBM->LDS loads, the in-CU MFMA loop -- the 4-wave interleave unless
--schedule says otherwise -- and the epilogue).  Default workload: bf16
M = N = K = 8192 with seeded N(0,1) inputs.  Prints one JSON line with the
throughput (TFLOPS), the MFMA roofline of the kernel (live HIP-event timing),
and the CPU oracle timed on a bounded sample as a baseline.

Timing: W warm-up steps, a barrier, then exactly K timed steps.  This is done
twice: first right after the inputs are uploaded ("from_idle" in the line),
then after --settle-ms (200) of untimed steps back to back ("value").  An idle
MI355X under its power cap takes ~50-100 ms of load before its clock settles
(it starts near 1.5 GHz, dips, then rises to its steady clock), and a short
timed region right after an idle gap measures that ramp, not the kernel.
Then the launches run back to back for --hbm-window seconds while amdsmi's
accumulator of the HBM controllers' activity gives the HBM bytes per launch
("hbm"; with the committed L2 counters, the last-level cache's hit rate by
bytes), and K more launches run with cold caches, each after a 1 GiB buffer
fill outside its events ("cold_cache", context only).

  python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--workload 2]
                  [--settle-ms 200] [--hbm-window 2] [--cold-mib 1024] [--all]
                  [--remap W,C | --row-major | --tune]
                  [--schedule interleave|pingpong|lockstep|interleave128|interleave192]
                  [--no-cpu-baseline]
  python bench.py --hbm-calibrate
        the HBM activity reading against a copy, a fill and a sum of known bytes
  python bench.py --clock-ramp 800 [--workload N | --all]
        the clock after 2 s of idle, per window of launches (time record)
  python bench.py --sizes "1024 2048 ..." [--dtype bf16|fp8|mxfp8] [--vendor]
        square-size sweep: each schedule (4-wave 256 and 128 tiles, ping-pong) per
        size, one JSON line each
  python bench.py --sweep "default 1,1 8,32 5,25 8,32,i192 ..." [--workload N | --shape M,N,K --dtype bf16|fp8]
        grid-order sweep: one JSON line per (W, C) on the same resident inputs ("default" = the
        library's default launch, split included), with its HBM bytes per launch (--hbm-window)
        ("1,1" is row-major order; a third field picks the kernel: i = 4-wave on
        256x256 tiles (default), i128 / i192 = on 128x128 / 192x192 tiles, p =
        ping-pong, l = lockstep); used to choose the library's default (W, C)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from dense_gemm_fp8_amd import synth  # noqa: E402

METRIC = "GEMM TFLOPS at 8192³ bf16 (fraction of 2.5 PF peak); L2/LLC hit %"
# Eq. 1 of the HipKittens L2 note (section 4), BW = LLC_BW * LLC_hit + L2_BW * L2_hit, with
# the constants that reproduce every "Mem BW" entry of its Table 4 (section 5) by least
# squares (the fit is re-derived in tests/test_oracle_schedule.py), in TB/s
EQ1_L2_BW_TBS = 17.05
EQ1_LLC_BW_TBS = 5.99
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0}   # MI355X dense MFMA peaks
# HipKittens 8-wave 0P/8C bf16 GEMM at 8192^3 on MI355X (HipKittens L2 note, Table 2 / Q3)
PAGES_BF16_8192_TFLOPS = 1610.0
# the sources that decide what a launch runs: the kernels, the grid remap,
# and the launch planning and launch code (not the argument checks of the
# entry points, the cache model or the autotuner, which do not change what a
# valid call runs)
KERNEL_SOURCES = ("dense_gemm_fp8_amd/csrc/gemm_kernels.hip", "dense_gemm_fp8_amd/csrc/remap.h",
                  "dense_gemm_fp8_amd/csrc/kernels.h", "dense_gemm_fp8_amd/csrc/launch.cpp",
                  "dense_gemm_fp8_amd/csrc/api_internal.h")


def _strip_comments(text: str) -> str:
    """C/C++ source without comments and whitespace (a comment edit keeps the hash)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the kernel and launch code, comments ignored: ties counter facts
    committed under profiles/ to the code they were measured on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(w: synth.Workload) -> int:
    """Bytes the GEMM must move at minimum: read A and B once (MXFP8: and their
    one-byte scales per 32 elements), write C (bf16) once."""
    e = 2 if w.dtype == "bf16" else 1
    scales = (w.M + w.N) * w.K // 32 if w.dtype == "mxfp8" else 0
    return e * (w.M * w.K + w.N * w.K) + scales + 2 * w.M * w.N


def kernel_name(dtype: str, schedule: str) -> str:
    if schedule == "interleave":
        return "gemm4_kernel<%s>" % dtype
    if schedule == "interleave128":
        return "gemm4_kernel<%s,128>" % dtype
    if schedule == "interleave192":
        return "gemm4_kernel<%s,192>" % dtype
    return "gemm_kernel<%s,%s>" % (dtype, schedule)


def load_profile_facts(workload: str) -> dict:
    """Counter-derived facts (HBM traffic, L2 hit rate) committed under
    profiles/, valid only for the kernel source they were measured on."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % workload)
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        facts = json.load(f)
    if facts.get("kernel_source_hash") != kernel_source_hash():
        return {}
    return facts


def wait_event(ev, deadline_s: float, what: str) -> None:
    """Poll a recorded event until the GPU passes it.  A GPU that has not passed
    it after deadline_s seconds is reported as a hang (one JSON line with
    "status": "HANG") and the process exits with status 3 at once, without
    waiting for the GPU."""
    t0 = time.perf_counter()
    while not ev.query():
        waited = time.perf_counter() - t0
        if waited > deadline_s:
            print(json.dumps({"status": "HANG", "where": what, "waited_s": round(waited, 1),
                              "deadline_s": deadline_s}), flush=True)
            os._exit(3)
        time.sleep(0.0002)


def gpu_identity() -> dict:
    """Which box and GPU a line was measured on: host name, the device's
    architecture and compute-unit count, the HIP runtime version, and the GPU's
    serial number and power cap as amdsmi reports them (null where
    unavailable)."""
    import socket
    import torch
    prop = torch.cuda.get_device_properties(0)
    out = {"host": socket.gethostname(), "arch": getattr(prop, "gcnArchName", None),
           "compute_units": prop.multi_processor_count, "hip_version": torch.version.hip,
           "gpu_serial": None, "power_cap_w": None}
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        out["gpu_serial"] = amdsmi.amdsmi_get_gpu_asic_info(h).get("asic_serial")
        cap = amdsmi.amdsmi_get_power_cap_info(h).get("power_cap")
        out["power_cap_w"] = round(cap / 1e6) if isinstance(cap, (int, float)) else None
    except Exception as e:  # pragma: no cover - no amdsmi / no device
        out["note"] = "amdsmi unavailable: %s" % e
    return out


def clock_from_trace(rec: np.ndarray, launches: int) -> dict:
    """Clock and per-tile timing from the kernels' own time record (hkg_gemm_opts
    trace: per workgroup the 100 MHz real-time and shader-clock counters at its
    start, K-loop end and last store, and its XCD), over the timed launches.
    rec: uint64 [launches, workgroups, 8]."""
    rec = rec.reshape(launches, -1, 8).astype(np.int64)
    rt0, rt1, rt2 = rec[..., 0], rec[..., 1], rec[..., 2]
    mt0, mt1 = rec[..., 3], rec[..., 4]
    xcd = rec[..., 6] & 0xF
    ok = (rt1 > rt0) & (rt2 >= rt1)
    mhz = np.where(ok, (mt1 - mt0) / np.maximum(rt1 - rt0, 1) * 100.0, np.nan)
    per_xcd = [round(float(np.nanmean(mhz[xcd == x])), 1) if np.any(xcd == x) else None
               for x in range(8)]
    span = (rt2.max(axis=1) - rt0.min(axis=1)) / 100.0          # us per launch
    return {"source": "per-workgroup shader-clock / 100 MHz real-time counters (s_memtime, "
                      "s_memrealtime) written by the kernel on every timed launch",
            "mhz_mean": round(float(np.nanmean(mhz)), 1),
            "mhz_per_xcd": per_xcd,
            "tile_us_mean": round(float(np.mean(rt2 - rt0)) / 100.0, 2),
            "kloop_us_mean": round(float(np.mean(rt1 - rt0)) / 100.0, 2),
            "epilogue_us_mean": round(float(np.mean(rt2 - rt1)) / 100.0, 2),
            "launch_span_us_mean": round(float(span.mean()), 2),
            "workgroups_per_launch": int(rec.shape[1])}


def metrics_reader():
    """A callable returning GPU 0's gpu_metrics accumulators from amdsmi as
    (mem_activity_acc, gfx_activity_acc, accumulation_counter,
    vram_max_bandwidth in GB/s), or None where amdsmi or these fields are
    unavailable.  The accumulators advance by the activity in percent per
    tick of accumulation_counter and are refreshed about once a second."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        keys = ("mem_activity_acc", "gfx_activity_acc", "accumulation_counter", "vram_max_bandwidth")

        def read():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                v = tuple(m[k] for k in keys)
            except Exception:  # pragma: no cover - a failed query mid-run
                return None
            return v if all(isinstance(x, int) for x in v) else None
        return read if read() is not None else None
    except Exception:  # pragma: no cover - no amdsmi / no device
        return None


def hbm_from_accumulators(a, b, launches_per_s: float) -> dict | None:
    """HBM traffic from two gpu_metrics samples a, b (see metrics_reader) taken
    at refreshes while the GPU ran one kind of launch back to back at
    launches_per_s: activity in percent of vram_max_bandwidth, and bytes per
    launch."""
    ticks = b[2] - a[2]
    if ticks <= 0 or launches_per_s <= 0:
        return None
    mem = (b[0] - a[0]) / ticks
    bw = b[3] * 1e9
    return {"mem_activity_pct": round(mem, 3), "gfx_activity_pct": round((b[1] - a[1]) / ticks, 2),
            "bytes_per_s": round(mem / 100.0 * bw), "bytes_per_launch": round(mem / 100.0 * bw / launches_per_s),
            "ticks": ticks, "vram_max_bandwidth_gbs": b[3]}


def hbm_window(step, stream, window_s: float, deadline_s: float, read=None) -> dict | None:
    """Launch `step` back to back (8 to 24 in flight) for about window_s + 2 s
    and read the memory controllers' activity between two accumulator refreshes
    inside that time: the first after 1.1 s of launches, the last at least
    window_s later.  None without amdsmi."""
    import torch
    read = read or metrics_reader()
    if read is None:
        return None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks, n, a, b, first = [], 0, None, None, None
    e0.record(stream)
    t0 = time.perf_counter()
    while b is None:
        for _ in range(8):
            step()
        n += 8
        e = torch.cuda.Event()
        e.record(stream)
        marks.append(e)
        if len(marks) > 2:
            wait_event(marks.pop(0), deadline_s, "HBM window")
        now = time.perf_counter() - t0
        if now < 1.1:
            continue
        cur = read()
        if cur is None:
            break
        if first is None:
            first = cur
        elif a is None:
            if cur[2] != first[2]:
                a, t_a = cur, now
        elif now - t_a >= window_s and cur[2] != a[2] and cur[2] - a[2] >= 1000 * window_s:
            b = cur
        if now > window_s + 6.0:
            break
    e1.record(stream)
    wait_event(e1, deadline_s, "HBM window")
    torch.cuda.synchronize()
    if a is None or b is None:
        return None
    out = hbm_from_accumulators(a, b, n / (e0.elapsed_time(e1) * 1e-3))
    if out is not None:
        out["launches"] = n
        out["ms_per_launch"] = round(e0.elapsed_time(e1) / n, 5)
    return out


def llc_estimate(hbm_bytes_per_launch, past_l2_bytes_per_launch) -> float | None:
    """Share of the bytes moving between the L2s and memory (FETCH_SIZE plus
    WRITE_SIZE, reads and writes together) that never reach HBM, in percent:
    the last-level cache's hit rate by bytes."""
    if not hbm_bytes_per_launch or not past_l2_bytes_per_launch:
        return None
    return round(100.0 * max(0.0, 1.0 - hbm_bytes_per_launch / past_l2_bytes_per_launch), 1)


def cpu_baseline(w: synth.Workload, A, B, sa, sb, target_s: float = 12.0,
                 gpu_rows=None) -> tuple[dict, dict | None]:
    """The oracle as it stands, timed on this host on a sample of whole output
    rows; and, when gpu_rows(rows) gives the GPU's (C_f32, C_bf16 bits) of
    those rows, the acceptance statistics of the GPU output on them."""
    import oracle
    from oracle import parity
    threads = oracle.default_threads()
    flops_per_row = 2.0 * w.N * w.K

    def run(rows):
        idx = np.arange(rows, dtype=np.int64) * max(1, w.M // rows)
        pm = np.repeat(idx, w.N)
        pn = np.tile(np.arange(w.N, dtype=np.int64), rows)
        t0 = time.perf_counter()
        if w.dtype == "bf16":
            ref = oracle.gemm_bf16_pairs(A, B, pm, pn, threads=threads)
        elif w.dtype == "mxfp8":
            ref = oracle.gemm_mxfp8_pairs(A, B, sa, sb, pm, pn, threads=threads)
        else:
            ref = oracle.gemm_fp8_pairs(A, B, sa, sb, pm, pn, threads=threads)
        return time.perf_counter() - t0, idx, ref

    probe_rows = max(1, threads // 2)
    dt, _, _ = run(probe_rows)
    rate = probe_rows * flops_per_row / dt
    rows = int(min(w.M, max(probe_rows, round(target_s * rate / flops_per_row))))
    dt, idx, ref = run(rows)
    sample = "%d full output rows (x %d columns, K=%d) of %s" % (rows, w.N, w.K, w.name)
    info = {"value": rows * flops_per_row / dt / 1e12, "unit": "TFLOPS", "cores": threads,
            "cores_in_affinity_mask": oracle.affinity_cores(),
            "kind": "oracle",
            "sample": "%s, fp64, %.1f s wall" % (sample, dt)}
    check = None
    if gpu_rows is not None:
        c32, cb = gpu_rows(idx)
        check = parity.stats(ref, c32.reshape(-1), cb.reshape(-1), w.K)
        check["sample"] = "the CPU baseline's %s, against its fp64 values" % sample
        check["rule"] = ("(i) |C_f32 - ref| <= tol = 1e-3 sqrt(K); (ii) C_bf16 = RNE(C_f32); "
                         "(iii) C_bf16 within 1 bf16 ulp of RNE(ref) where that ulp exceeds tol, "
                         "else within tol + ulp/2 of ref")
    return info, check


def launch_plan(w: synth.Workload, opts) -> list:
    """The library's own account of what one GEMM of this workload launches."""
    import dense_gemm_fp8_amd as hkg
    rc, launches = hkg.launch_plan(w.M, w.N, w.K, {"bf16": 0, "fp8": 1, "mxfp8": 2}[w.dtype], opts)
    names = {hkg.HKG_SCHED_PINGPONG: "pingpong", hkg.HKG_SCHED_LOCKSTEP: "lockstep",
             hkg.HKG_SCHED_INTERLEAVE: "interleave", hkg.HKG_SCHED_INTERLEAVE_128: "interleave128",
             hkg.HKG_SCHED_INTERLEAVE_192: "interleave192"}
    return [{"schedule": names[d["schedule"]], "tile": d["tile"], "rows": d["rows"],
             "workgroups": d["grid"], "W": d["W"], "C": d["C"]} for d in launches]


def bench_one(w: synth.Workload, steps: int, warmup: int, opts, sched_name: str,
              with_cpu: bool, deadline_s: float = 120.0, settle_ms: float = 200.0,
              tune: bool = False, pad_k: int = 0, cold_bytes: int = 1 << 30,
              hbm_window_s: float = 2.0) -> dict:
    import torch
    import dense_gemm_fp8_amd as hkg

    dev = torch.device("cuda:0")
    A, B, sa, sb = synth.make_inputs(w)
    if w.dtype == "bf16":
        dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(dev)
        dB = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        dA = torch.from_numpy(A).to(dev)
        dB = torch.from_numpy(B).to(dev)
    if pad_k:
        # operand rows pad_k elements longer than K: the GEMM reads views with
        # that row pitch (lda = ldb = K + pad_k)
        def padded(t):
            big = torch.zeros((t.shape[0], t.shape[1] + pad_k), dtype=t.dtype, device=dev)
            big[:, :t.shape[1]] = t
            return big[:, :t.shape[1]]
        dA, dB = padded(dA), padded(dB)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    if w.dtype == "mxfp8":
        # one MXFP8 step packs both operands' scales from their natural
        # [rows][K/32] layout, then runs the GEMM kernel
        dSA = torch.from_numpy(sa).to(dev)
        dSB = torch.from_numpy(sb).to(dev)
        pSA = hkg.mx_pack_scales(dSA, hkg.HKG_MX_OPERAND_A, stream=stream)
        pSB = hkg.mx_pack_scales(dSB, hkg.HKG_MX_OPERAND_B, stream=stream)

    tuned = None
    if tune:
        # the library's autotuner picks the grid order on these buffers first
        if w.dtype == "mxfp8":
            raise ValueError("--tune times bf16 and e4m3 (MXFP8 takes the e4m3 order)")
        opts, tuned_ms, tried = hkg.tune_remap(dA, dB, C, launches=10, stream=stream)
        tuned = {"remap": opts.remap, "W": opts.W, "C": opts.C, "ms_per_launch": round(tuned_ms, 5),
                 "tried": [{"remap": o.remap, "W": o.W, "C": o.C, "ms": round(t, 5)}
                           for o, t in tried]}
    # the kernels' own time record on every timed launch (8 words per workgroup)
    plan = launch_plan(w, opts)
    wgs = sum(d["workgroups"] for d in plan)
    trace = torch.zeros((steps, wgs, 8), dtype=torch.int64, device=dev)
    base = opts if opts is not None else hkg.make_opts()

    def traced(i):
        return hkg.make_opts(remap=base.remap, W=base.W, C=base.C, schedule=base.schedule,
                             trace=trace[i].data_ptr())

    def step(e0=None, e1=None, o=None):
        """One pass of the path; e0/e1 bracket the GEMM kernel launch."""
        if w.dtype == "mxfp8":
            hkg.mx_pack_scales(dSA, hkg.HKG_MX_OPERAND_A, pSA, stream=stream)
            hkg.mx_pack_scales(dSB, hkg.HKG_MX_OPERAND_B, pSB, stream=stream)
        if e0 is not None:
            e0.record(stream)
        o = opts if o is None else o
        if w.dtype == "bf16":
            hkg.gemm_bf16(dA, dB, C, opts=o, stream=stream)
        elif w.dtype == "mxfp8":
            hkg.gemm_mxfp8(dA, dB, pSA, pSB, C, opts=o, stream=stream)
        else:
            hkg.gemm_fp8(dA, dB, sa, sb, C, opts=o, stream=stream)
        if e1 is not None:
            e1.record(stream)

    # events and per-launch options of a timed region, made before any warm-up so
    # that nothing but the barrier separates the warm-up from the timed steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    outer0 = torch.cuda.Event(enable_timing=True)
    outer1 = torch.cuda.Event(enable_timing=True)
    topts = [traced(i) for i in range(steps)]

    def warm_then_time():
        """W untimed warm-up steps, a barrier, then exactly `steps` timed steps,
        every GEMM launch bracketed by HIP events on the launch stream."""
        for _ in range(warmup):
            step()
        mark = torch.cuda.Event()
        mark.record(stream)
        wait_event(mark, deadline_s, "warm-up")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        outer0.record(stream)
        for i, (s, e) in enumerate(ev):
            step(s, e, topts[i])
        outer1.record(stream)
        wait_event(outer1, deadline_s, "timed region")
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return (np.array([s.elapsed_time(e) for s, e in ev]), outer0.elapsed_time(outer1), wall,
                clock_from_trace(trace.cpu().numpy(), steps))

    def settle(ms: float) -> int:
        """Untimed steps back to back for at least `ms` of wall time (8 to 24 in
        flight, so the GPU never idles); returns how many ran."""
        marks, n, t0 = [], 0, time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(8):
                step()
            n += 8
            e = torch.cuda.Event()
            e.record(stream)
            marks.append(e)
            if len(marks) > 2:
                wait_event(marks.pop(0), deadline_s, "settle")
        return n

    # 1. as asked: W warm-up steps right after the inputs arrived (the GPU was
    #    idle while they were drawn), then the K timed steps
    per_launch_ms, region_ms, wall, clock_info = warm_then_time()
    from_idle = {"value": round(w.flops / (region_ms / steps * 1e-3) / 1e12, 2),
                 "ms_per_step": round(region_ms / steps, 5),
                 "kernel_ms_mean": round(float(per_launch_ms.mean()), 5),
                 "mhz_mean": clock_info["mhz_mean"]}
    settle_info = None
    if settle_ms > 0:
        # 2. after any idle gap the power controller takes ~50-100 ms of load to
        #    settle (it starts near 1.5 GHz and dips before it rises to the steady
        #    clock); `value` is measured at that steady clock: untimed steps for
        #    settle_ms, then the same W warm-up and K timed steps again
        t_s = time.perf_counter()
        n_settle = settle(settle_ms)
        settle_info = {"ms": round((time.perf_counter() - t_s) * 1e3, 1), "launches": n_settle,
                       "rule": "untimed steps back to back for at least %g ms before the W warm-up "
                               "steps, so that the K timed steps run at the steady power-capped "
                               "clock, not on the clock ramp that follows an idle GPU; from_idle "
                               "is the same W + K measurement without it" % settle_ms}
        per_launch_ms, region_ms, wall, clock_info = warm_then_time()
    hbm = None
    if hbm_window_s > 0:
        # 3. HBM traffic per launch from the memory controllers' activity, with
        #    the launches back to back at the same steady clock
        hbm = hbm_window(step, stream, hbm_window_s, deadline_s)
    cold = None
    if cold_bytes > 0:
        # 4. context for `value`, which runs with warm caches: the same launches,
        #    each after a fill of a cold_bytes buffer (outside its events) that
        #    evicts the operands from every L2 and the last-level cache
        scratch = torch.empty(cold_bytes // 4, dtype=torch.float32, device=dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i, (s, e) in enumerate(cev):
            scratch.fill_(float(i))
            step(s, e)
        mark = torch.cuda.Event()
        mark.record(stream)
        wait_event(mark, deadline_s, "cold-cache launches")
        torch.cuda.synchronize()
        cold_ms = np.array([s.elapsed_time(e) for s, e in cev])
        cold = {"flush_bytes": cold_bytes,
                "kernel_ms_mean": round(float(cold_ms.mean()), 5),
                "kernel_ms_median": round(float(np.median(cold_ms)), 5),
                "TFLOPS": round(w.flops / (float(cold_ms.mean()) * 1e-3) / 1e12, 2),
                "rule": "each of K launches after writing a %d MiB buffer; HIP events bracket the "
                        "launch only" % (cold_bytes >> 20)}
        del scratch
    ms_per_step = region_ms / steps
    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    kern_ms = float(per_launch_ms.mean())
    achieved = w.flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    # the committed counters were taken on the default launch of this workload
    facts = load_profile_facts(w.name) if opts is None else {}
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(tflops / PAGES_BF16_8192_TFLOPS, 4)
                        if w.name == "bf16_8192" else None),
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "inputs": "seeded N(0,1)%s" % {
                       "bf16": "", "fp8": " quantised to e4m3 with amax/448 scales",
                       "mxfp8": " quantised to MXFP8 (e4m3, one E8M0 scale per 32 along K;"
                                " step includes packing both scale arrays)"}[w.dtype],
                   "schedule": sched_name,
                   "remap": ({"remap": opts.remap, "W": opts.W, "C": opts.C} if opts else "default"),
                   "tuned": tuned,
                   "operand_row_pitch": w.K + pad_k,
                   "launches": plan},
        "fraction_of_peak": round(tflops / peak, 4),
        "roofline": {
            "bound": "mfma",
            "kernel": kernel_name(w.dtype, plan[0]["schedule"] if plan else sched_name),
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": facts.get("hbm_bytes_per_launch"),
            "algorithmic_flops_per_launch": w.flops,
            "algorithmic_bytes_per_launch": algorithmic_bytes(w),
            "kernel_ms_mean": round(kern_ms, 5),
            "kernel_ms_min": round(float(per_launch_ms.min()), 5),
            "kernel_ms_median": round(float(np.median(per_launch_ms)), 5),
        },
        "cache": cache_fields(facts, hbm),
        "hbm": hbm,
        "counters": counter_fields(facts),
        "clock": clock_info,
        "settle": settle_info,
        "from_idle": from_idle,
        "cold_cache": cold,
        "wall_s_timed_region": round(wall, 4),
        "kernel_source_hash": kernel_source_hash(),
        "gpu": torch.cuda.get_device_name(dev),
        "box": gpu_identity(),
    }
    if with_cpu:
        # one more (untimed) launch of the same configuration that also writes
        # the fp32 copy, for the parity of the rows the CPU baseline computes
        Cf = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        o = opts
        if w.dtype == "bf16":
            hkg.gemm_bf16(dA, dB, C, Cf, opts=o, stream=stream)
        elif w.dtype == "mxfp8":
            hkg.gemm_mxfp8(dA, dB, pSA, pSB, C, Cf, opts=o, stream=stream)
        else:
            hkg.gemm_fp8(dA, dB, sa, sb, C, Cf, opts=o, stream=stream)
        done = torch.cuda.Event()
        done.record(stream)
        wait_event(done, deadline_s, "parity launch")
        del dA, dB

        def gpu_rows(idx):
            rows = torch.from_numpy(idx).to(dev)
            c32 = Cf.index_select(0, rows).cpu().numpy()
            cb = C.index_select(0, rows).view(torch.int16).cpu().numpy().view(np.uint16)
            return c32, cb

        res["cpu_baseline"], res["parity"] = cpu_baseline(w, A, B, sa, sb, gpu_rows=gpu_rows)
        res["vs_cpu_baseline"] = round(tflops / res["cpu_baseline"]["value"], 1)
        del C, Cf
    else:
        del dA, dB, C
        res["cpu_baseline"] = None
        res["parity"] = None
    return res


def cache_fields(facts: dict, hbm: dict | None = None) -> dict:
    """L2 / LLC hit rates and the two terms of the pages' Eq. 1 they imply.  The
    L2 hit rate is from the committed counter run of this kernel source.  This
    ROCm has no last-level-cache counter; the LLC hit rate is estimated by bytes
    from this run's HBM traffic (hbm_window) against the bytes past the L2s in
    the same counter run (llc_estimate), when both exist."""
    l2 = facts.get("l2_hit_pct")
    llc = llc_estimate((hbm or {}).get("bytes_per_launch"), facts.get("hbm_bytes_per_launch"))
    out = {"l2_hit_pct": l2, "llc_hit_pct": llc,
           "llc_note": ("estimated: 1 - HBM bytes per launch (memory-controller activity, this run) / "
                        "bytes past the L2s per launch (FETCH_SIZE + WRITE_SIZE, %s)" % facts.get("source")
                        if llc is not None else facts.get("llc_note")),
           "source": facts.get("source")}
    out["eq1"] = {"l2_bw_tbs": EQ1_L2_BW_TBS, "llc_bw_tbs": EQ1_LLC_BW_TBS,
                  "l2_term_tbs": None if l2 is None else round(EQ1_L2_BW_TBS * l2 / 100.0, 2),
                  "llc_term_tbs": None if llc is None else round(EQ1_LLC_BW_TBS * llc / 100.0, 2)}
    return out


def counter_fields(facts: dict) -> dict:
    """MFMA busy and LDS bank conflicts from the committed counter run of this
    kernel source (rocprofv3 --pmc in a separate process; null when the
    kernel source has changed since)."""
    keys = ("mfma_busy_pct", "lds_bank_conflict_cycles", "wait_any_pct", "wait_inst_lds_pct",
            "counter_clock_ghz")
    out = {k: facts.get(k) for k in keys}
    out["source"] = facts.get("source")
    return out


def custom_workload(shape: str, dtype: str) -> synth.Workload:
    M, N, K = (int(v) for v in shape.split(","))
    return synth.Workload("%s_%dx%dx%d" % (dtype, M, N, K), dtype, M, N, K, 7101, 7102)


def sweep(w: synth.Workload, pairs, steps: int, warmup: int, hbm_window_s: float = 0.0,
          deadline_s: float = 120.0) -> None:
    """Time each grid order (W, C) on the same inputs, and with hbm_window_s > 0
    read its HBM bytes per launch (hbm_window); one JSON line each."""
    import torch
    import dense_gemm_fp8_amd as hkg

    dev = torch.device("cuda:0")
    A, B, sa, sb = synth.make_inputs(w)
    if w.dtype == "bf16":
        dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(dev)
        dB = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        dA = torch.from_numpy(A).to(dev)
        dB = torch.from_numpy(B).to(dev)
    del A, B
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    rc, dW, dC = hkg.hkg_default_remap(w.M, w.N, w.K, 0 if w.dtype == "bf16" else 1)

    scheds = {"p": hkg.HKG_SCHED_PINGPONG, "l": hkg.HKG_SCHED_LOCKSTEP,
              "i": hkg.HKG_SCHED_INTERLEAVE, "i128": hkg.HKG_SCHED_INTERLEAVE_128,
              "i192": hkg.HKG_SCHED_INTERLEAVE_192}

    def run(W, Cc, n, sc="i"):
        # "default" (W) = the library's default launch, split included
        opts = None if W == "default" else hkg.make_opts(remap=hkg.HKG_REMAP_XCD, W=W, C=Cc,
                                                         schedule=scheds[sc])
        for _ in range(n):
            if w.dtype == "bf16":
                hkg.gemm_bf16(dA, dB, C, opts=opts, stream=stream)
            else:
                hkg.gemm_fp8(dA, dB, sa, sb, C, opts=opts, stream=stream)

    # bring the part to its steady clock before timing anything (~2 s of GEMMs)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(dW, dC, warmup)
    e1.record(stream)
    torch.cuda.synchronize()
    reps = max(1, int(2000.0 / max(e0.elapsed_time(e1) / max(warmup, 1), 1e-3)))
    run(dW, dC, reps)
    torch.cuda.synchronize()
    times = {p: [] for p in pairs}
    for order in (list(pairs), list(reversed(pairs))):   # forward then reverse
        for key in order:
            run(*key[:2], warmup, *key[2:])
            e0.record(stream)
            run(*key[:2], steps, *key[2:])
            e1.record(stream)
            torch.cuda.synchronize()
            times[key].append(e0.elapsed_time(e1) / steps)
    hbm = {key: (hbm_window(lambda: run(*key[:2], 1, *key[2:]), stream, hbm_window_s, deadline_s)
                 if hbm_window_s > 0 else None) for key in pairs}
    for key in pairs:
        W, Cc = key[:2]
        ms = float(np.mean(times[key]))
        print(json.dumps({"sweep": w.name, "M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype,
                          "W": W, "C": Cc, "schedule": key[2] if len(key) > 2 else "i",
                          "default": W == "default" or [W, Cc] == [dW, dC],
                          "ms": round(ms, 5), "ms_runs": [round(t, 5) for t in times[key]],
                          "TFLOPS": round(w.flops / (ms * 1e-3) / 1e12, 2), "hbm": hbm[key]}), flush=True)


def clock_ramp(w: synth.Workload, launches: int, idle_s: float) -> None:
    """The clock after an idle GPU: `launches` default launches back to back
    after idle_s seconds of idle, each with the kernels' time record; one JSON
    line with the mean clock and throughput over windows of launches."""
    import torch
    import dense_gemm_fp8_amd as hkg

    if w.dtype not in ("bf16", "fp8"):
        raise ValueError("--clock-ramp runs the bf16 and e4m3 workloads")
    dev = torch.device("cuda:0")
    A, B, sa, sb = synth.make_inputs(w)
    if w.dtype == "bf16":
        dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(dev)
        dB = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    del A, B
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    wgs = sum(d["workgroups"] for d in launch_plan(w, None))
    trace = torch.zeros((launches, wgs, 8), dtype=torch.int64, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    opts = [hkg.make_opts(trace=trace[i].data_ptr()) for i in range(launches)]
    torch.cuda.synchronize()
    time.sleep(idle_s)
    for i in range(launches):
        ev[i][0].record(stream)
        if w.dtype == "bf16":
            hkg.gemm_bf16(dA, dB, C, opts=opts[i], stream=stream)
        else:
            hkg.gemm_fp8(dA, dB, sa, sb, C, opts=opts[i], stream=stream)
        ev[i][1].record(stream)
    wait_event(ev[-1][1], 120.0, "clock ramp")
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    rec = trace.cpu().numpy()
    out = {"clock_ramp": w.name, "idle_s": idle_s, "launches": launches, "windows": []}
    lo = 0
    for hi in (5, 10, 25, 50, 100, 200, 400, 800, 1600):
        if hi > launches:
            break
        c = clock_from_trace(rec[lo:hi], hi - lo)
        out["windows"].append({"launches": [lo, hi], "ends_at_ms": round(float(ms[:hi].sum()), 1),
                               "mhz_mean": c["mhz_mean"],
                               "tflops": round(w.flops / (float(ms[lo:hi].mean()) * 1e-3) / 1e12, 1)})
        lo = hi
    print(json.dumps(out), flush=True)


def size_sweep(sizes, dtype: str, warmup: int, vendor: bool = False) -> None:
    """Sizes given as n (n x n x n) or "MxNxK" (any extents: edge tiles are
    masked): every schedule on the same inputs, each timed for ~0.2 s twice
    (forward and reverse order); one JSON line per (size, schedule)."""
    import torch
    import dense_gemm_fp8_amd as hkg

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    scheds = [("interleave", hkg.HKG_SCHED_INTERLEAVE), ("pingpong", hkg.HKG_SCHED_PINGPONG),
              ("interleave128", hkg.HKG_SCHED_INTERLEAVE_128), ("default", hkg.HKG_SCHED_DEFAULT)]
    if dtype != "mxfp8":     # 192 x 192 tiles exist for bf16 and e4m3
        scheds.insert(3, ("interleave192", hkg.HKG_SCHED_INTERLEAVE_192))
    if dtype == "mxfp8":     # the block-scaled path exists in the 4-wave kernel only
        scheds = [sc for sc in scheds if sc[0] != "pingpong"]
    elif vendor:             # context only: the vendor library on the same inputs and timing rule
        scheds.append(("vendor", "vendor"))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for n in sizes:
        M, N, K = (int(v) for v in n.split("x")) if "x" in n else (int(n),) * 3
        w = custom_workload("%d,%d,%d" % (M, N, K), dtype)
        A, B, sa, sb = synth.make_inputs(w)
        if dtype == "bf16":
            dA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(dev)
            dB = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
            if dtype == "mxfp8":   # scales packed once; the sweep times the GEMM kernel
                pSA = hkg.mx_pack_scales(torch.from_numpy(sa).to(dev), hkg.HKG_MX_OPERAND_A)
                pSB = hkg.mx_pack_scales(torch.from_numpy(sb).to(dev), hkg.HKG_MX_OPERAND_B)
        del A, B
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def run(sc, k):
            if sc == "vendor":
                # torch.mm -> hipBLASLt (bf16); torch._scaled_mm on the same
                # e4m3 bytes and per-tensor scales
                if dtype == "bf16":
                    for _ in range(k):
                        torch.mm(dA, dB.t(), out=C)
                else:
                    ta = torch.tensor(sa, dtype=torch.float32, device=dev)
                    tb = torch.tensor(sb, dtype=torch.float32, device=dev)
                    a8, b8 = dA.view(torch.float8_e4m3fn), dB.view(torch.float8_e4m3fn)
                    for _ in range(k):
                        torch._scaled_mm(a8, b8.t(), scale_a=ta, scale_b=tb, out_dtype=torch.bfloat16)
                return
            opts = hkg.make_opts(schedule=sc)
            for _ in range(k):
                if dtype == "bf16":
                    hkg.gemm_bf16(dA, dB, C, opts=opts, stream=stream)
                elif dtype == "mxfp8":
                    hkg.gemm_mxfp8(dA, dB, pSA, pSB, C, opts=opts, stream=stream)
                else:
                    hkg.gemm_fp8(dA, dB, sa, sb, C, opts=opts, stream=stream)

        def timed(sc, k):
            e0.record(stream)
            run(sc, k)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / k

        run(scheds[0][1], warmup)
        est = timed(scheds[0][1], 3)
        steps = int(min(500, max(5, 200.0 / max(est, 1e-3))))
        times = {name: [] for name, _ in scheds}
        for order in (scheds, scheds[::-1]):
            for name, sc in order:
                run(sc, 2)
                times[name].append(timed(sc, steps))
        peak = PEAK_TFLOPS[dtype]
        for name, _ in scheds:
            ms = float(np.mean(times[name]))
            tf = w.flops / (ms * 1e-3) / 1e12
            rec = {"size_sweep": dtype, "n": int(n) if "x" not in n else n, "schedule": name, "steps": steps,
                   "ms": round(ms, 5), "TFLOPS": round(tf, 1), "frac_of_peak": round(tf / peak, 4)}
            if name == "vendor":
                rec["context_only"] = True
            print(json.dumps(rec), flush=True)
        del dA, dB, C
        torch.cuda.empty_cache()


def hbm_calibrate(window_s: float, deadline_s: float) -> None:
    """The memory controllers' activity (hbm_window) under device kernels whose
    HBM traffic is known: a 1 GiB copy (reads and writes), a 4 GiB fill (writes)
    and a 4 GiB sum (reads), each far larger than the last-level cache."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    x = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    big = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    for name, fn, nbytes in (("copy 1 GiB", lambda: y.copy_(x), 2 << 30),
                             ("fill 4 GiB", lambda: big.fill_(2.0), 4 << 30),
                             ("sum 4 GiB", lambda: torch.sum(big), 4 << 30)):
        r = hbm_window(fn, stream, window_s, deadline_s)
        if r is None:
            print(json.dumps({"calibration": name, "hbm": None, "note": "amdsmi unavailable"}), flush=True)
            continue
        known = nbytes / (r["ms_per_launch"] * 1e-3)
        print(json.dumps({"calibration": name, "known_bytes_per_s": round(known),
                          "activity_bytes_per_s": r["bytes_per_s"],
                          "ratio": round(r["bytes_per_s"] / known, 4), "hbm": r}), flush=True)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6],
                    help="1-5: the five configurations; 6: MXFP8 8192^3")
    ap.add_argument("--all", action="store_true", help="one line per workload 1..5")
    ap.add_argument("--remap", type=str, default=None, help="W,C for the XCD remap")
    ap.add_argument("--row-major", action="store_true")
    ap.add_argument("--schedule", choices=["interleave", "pingpong", "lockstep", "interleave128",
                                           "interleave192"],
                    default="interleave", help="in-CU schedule (default: the library's, interleave)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-ramp", type=int, default=0, metavar="N",
                    help="time N default launches after 2 s of idle, each with the time record, "
                         "and print the clock per window of launches")
    ap.add_argument("--pad-k", type=int, default=0,
                    help="lay A and B out with rows this many elements longer than K (row pitch)")
    ap.add_argument("--tune", action="store_true",
                    help="pick the grid order with the library's autotuner (hkg_tune_remap) first")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps (ms of wall time) between a first W + K measurement from "
                         "idle and the W + K measurement reported as value; 0 reports the first")
    ap.add_argument("--deadline", type=float, default=120.0,
                    help="seconds to wait for the GPU to finish the warm-up or the timed "
                         "region before reporting a hang (exit status 3)")
    ap.add_argument("--cold-mib", type=int, default=1024,
                    help="after the timed region, time K more launches, each after writing a "
                         "buffer of this many MiB (cold caches; reported as cold_cache, 0 skips)")
    ap.add_argument("--hbm-window", type=float, default=2.0,
                    help="seconds of launches back to back over which the HBM controllers' activity "
                         "is read (amdsmi), for the line's hbm and LLC estimate (0 skips)")
    ap.add_argument("--hbm-calibrate", action="store_true",
                    help="read the HBM controllers' activity under a copy, a fill and a sum of known "
                         "byte counts and print one JSON line each")
    ap.add_argument("--shape", type=str, default=None, help="M,N,K (custom size)")
    ap.add_argument("--dtype", choices=["bf16", "fp8", "mxfp8"], default="bf16")
    ap.add_argument("--sweep", type=str, default=None, help='"W,C W,C ..." grid orders to time')
    ap.add_argument("--sizes", type=str, default=None,
                    help='"n n ..." square sizes or "MxNxK ...": every schedule per size (with --dtype)')
    ap.add_argument("--vendor", action="store_true",
                    help="with --sizes: also time the vendor library on the same inputs (context)")
    args = ap.parse_args(argv)

    if args.cold_mib < 0 or args.hbm_window < 0:
        print("--cold-mib and --hbm-window must be at least 0", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        return 2
    if args.tune and args.pad_k:
        print("--tune times dense operand rows; it does not combine with --pad-k", file=sys.stderr)
        return 2
    if args.tune and (args.remap or args.row_major or args.schedule != "interleave"):
        print("--tune picks the grid order of the default launch; it does not combine with "
              "--remap, --row-major or --schedule", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print("bench.py measures one GPU only: this GEMM path is single-GPU "
              "(--gpus %d is not supported; run with --gpus 1)" % args.gpus, file=sys.stderr)
        return 2

    import dense_gemm_fp8_amd as hkg
    hkg.load()
    sched = {"pingpong": hkg.HKG_SCHED_PINGPONG, "lockstep": hkg.HKG_SCHED_LOCKSTEP,
             "interleave": hkg.HKG_SCHED_INTERLEAVE,
             "interleave128": hkg.HKG_SCHED_INTERLEAVE_128,
             "interleave192": hkg.HKG_SCHED_INTERLEAVE_192}[args.schedule]
    opts = None
    if args.row_major:
        opts = hkg.make_opts(remap=hkg.HKG_REMAP_ROW_MAJOR, schedule=sched)
    elif args.remap:
        W, C = (int(v) for v in args.remap.split(","))
        opts = hkg.make_opts(remap=hkg.HKG_REMAP_XCD, W=W, C=C, schedule=sched)
    elif sched != hkg.HKG_SCHED_INTERLEAVE:
        opts = hkg.make_opts(schedule=sched)

    if args.sizes:
        size_sweep(args.sizes.split(), args.dtype, args.warmup, args.vendor)
        return 0
    if args.hbm_calibrate:
        hbm_calibrate(args.hbm_window or 2.0, args.deadline)
        return 0
    if args.clock_ramp:
        for i in ([2, 5] if args.all else [args.workload]):
            clock_ramp(synth.workload(i), args.clock_ramp, 2.0)
        return 0
    if args.sweep:
        w = custom_workload(args.shape, args.dtype) if args.shape else synth.workload(args.workload)
        pairs = [("default", 0) if item == "default" else
                 tuple(int(v) if v.isdigit() else v for v in item.split(","))
                 for item in args.sweep.split()]
        sweep(w, pairs, args.steps, args.warmup, args.hbm_window, args.deadline)
        return 0
    ids = [1, 2, 3, 4, 5] if args.all else [args.workload]
    for i in ids:
        w = synth.workload(i) if not args.shape else custom_workload(args.shape, args.dtype)
        steps = args.steps
        res = bench_one(w, steps, args.warmup, opts, args.schedule,
                        with_cpu=(not args.no_cpu_baseline), deadline_s=args.deadline,
                        settle_ms=args.settle_ms, tune=args.tune,
                        pad_k=args.pad_k, cold_bytes=args.cold_mib << 20,
                        hbm_window_s=args.hbm_window)
        print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
