"""Host-side logic of bench.py (no GPU): argument limits, the time-record
decoder, the counter facts, the Eq. 1 field and the CPU-baseline leg's parity
record."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dense_gemm_fp8_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_tune_with_padded_rows_is_refused(capsys):
    assert bench.main(["--tune", "--pad-k", "64"]) == 2
    assert "--pad-k" in capsys.readouterr().err


def test_step_counts_and_tune_combinations_are_refused(capsys):
    for argv in (["--steps", "0"], ["--steps", "-3"], ["--warmup", "-1"]):
        assert bench.main(argv) == 2, argv
        assert "--steps" in capsys.readouterr().err
    for argv in (["--tune", "--remap", "8,32"], ["--tune", "--row-major"],
                 ["--tune", "--schedule", "pingpong"]):
        assert bench.main(argv) == 2, argv
        assert "--tune" in capsys.readouterr().err
    for argv in (["--cold-mib", "-1"], ["--hbm-window", "-0.5"]):
        assert bench.main(argv) == 2, argv
        assert "--cold-mib and --hbm-window" in capsys.readouterr().err


def test_clock_from_trace_decodes_a_known_record():
    # 2 launches x 16 workgroups; workgroup b on XCD b % 8 at (1500 + 20 x) MHz:
    # shader-clock ticks = MHz / 100 per real-time tick
    L, G = 2, 16
    rec = np.zeros((L, G, 8), dtype=np.int64)
    for li in range(L):
        for b in range(G):
            x = b % 8
            rt0 = 1_000_000 + 50_000 * li + 10 * b
            kl, ep = 18_000, 500                     # 180 us K loop, 5 us epilogue
            mhz = 1500 + 20 * x
            rec[li, b, :] = [rt0, rt0 + kl, rt0 + kl + ep, 7, 7 + kl * mhz // 100, 0, x,
                             (b // 4) << 32 | (b % 4)]
    c = bench.clock_from_trace(rec, L)
    assert c["mhz_per_xcd"] == [1500.0 + 20 * x for x in range(8)]
    assert abs(c["mhz_mean"] - 1570.0) < 1e-9
    assert c["kloop_us_mean"] == 180.0 and c["epilogue_us_mean"] == 5.0
    assert c["tile_us_mean"] == 185.0
    assert c["launch_span_us_mean"] == (10 * 15 + kl + ep) / 100.0
    assert c["workgroups_per_launch"] == G


def test_profile_facts_follow_the_kernel_source(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    facts = {"kernel_source_hash": h, "l2_hit_pct": 80.0}
    os.makedirs(tmp_path / "profiles")
    (tmp_path / "profiles" / "counters_x.json").write_text(json.dumps(facts))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    assert bench.load_profile_facts("x")["l2_hit_pct"] == 80.0
    facts["kernel_source_hash"] = "0" * 16
    (tmp_path / "profiles" / "counters_x.json").write_text(json.dumps(facts))
    assert bench.load_profile_facts("x") == {}
    assert bench.load_profile_facts("missing") == {}


def test_committed_facts_match_this_source():
    """Every committed counter file names its kernel source; those of the five
    workloads must match the current one, or bench.py drops them silently."""
    for name in ("bf16_8192", "fp8_e4m3_8192", "mxfp8_8192", "bf16_mlp_16384x14336x4096",
                 "bf16_16384"):
        facts = bench.load_profile_facts(name)
        assert facts, name
        assert 0 < facts["l2_hit_pct"] < 100 and facts["hbm_bytes_per_launch"] > 0


def test_eq1_l2_term():
    c = bench.cache_fields({"l2_hit_pct": 80.0})
    assert abs(c["eq1"]["l2_term_tbs"] - 0.8 * bench.EQ1_L2_BW_TBS) < 0.006
    assert c["eq1"]["llc_term_tbs"] is None
    assert bench.cache_fields({})["eq1"]["l2_term_tbs"] is None


def test_hbm_traffic_from_activity_accumulators():
    # 2 s of ticks (1 ms each) at 25 % memory and 100 % gfx activity of an
    # 8192 GB/s part: 2.048e12 B/s; at 1000 launches per second, 2.048e9 B each
    a = (1_000_000, 5_000_000, 40_000, 8192)
    b = (a[0] + 25 * 2000, a[1] + 100 * 2000, a[2] + 2000, 8192)
    r = bench.hbm_from_accumulators(a, b, 1000.0)
    assert r["mem_activity_pct"] == 25.0 and r["gfx_activity_pct"] == 100.0
    assert r["bytes_per_s"] == 2_048_000_000_000 and r["bytes_per_launch"] == 2_048_000_000
    assert bench.hbm_from_accumulators(a, a, 1000.0) is None      # no refresh in between


def test_llc_estimate_and_eq1_llc_term():
    # 0.25 GB of HBM traffic per launch against 1.75 GB past the L2s: 6/7 served
    # by the last-level cache
    assert bench.llc_estimate(0.25e9, 1.75e9) == 85.7
    assert bench.llc_estimate(None, 1.75e9) is None and bench.llc_estimate(0.25e9, None) is None
    assert bench.llc_estimate(3e9, 1e9) == 0.0
    c = bench.cache_fields({"l2_hit_pct": 80.0, "hbm_bytes_per_launch": 1.75e9, "source": "x"},
                           {"bytes_per_launch": 0.25e9})
    assert c["llc_hit_pct"] == 85.7 and c["llc_note"].startswith("estimated")
    assert abs(c["eq1"]["llc_term_tbs"] - 0.857 * bench.EQ1_LLC_BW_TBS) < 0.006
    assert bench.cache_fields({"l2_hit_pct": 80.0}, None)["llc_hit_pct"] is None


def test_cpu_baseline_reports_parity_of_the_rows_it_computes():
    """bench's CPU-baseline leg compares the GPU output of the rows it computes
    with its fp64 values; fed the oracle's own product (and one flipped code)
    it reports a pass (and the flip)."""
    import oracle
    from oracle import parity
    w = synth.workload(1)                      # bf16 256^3
    A, B, sa, sb = synth.make_inputs(w)
    full = oracle.gemm_bf16(A, B)
    c32 = full.astype(np.float32)
    cb = parity.f32_to_bf16_rne(c32)
    seen = []

    def rows(idx):
        seen.append(idx)
        return c32[idx], cb[idx]

    info, check = bench.cpu_baseline(w, A, B, sa, sb, target_s=0.05, gpu_rows=rows)
    assert info["kind"] == "oracle" and info["value"] > 0
    assert check["pass"] and check["checked"] == len(seen[-1]) * w.N
    # fp64 -> fp32 -> bf16 may differ from one rounding of fp64 by a code
    assert check["ulp_hist"][">=2"] == 0 and check["max_abs_err"] < 1e-4
    bad = cb.copy()
    bad[seen[-1][0], 3] ^= 1

    info, check = bench.cpu_baseline(w, A, B, sa, sb, target_s=0.05,
                                     gpu_rows=lambda idx: (c32[idx], bad[idx]))
    assert not check["pass"] and check["fail_ii"] == 1
    info, check = bench.cpu_baseline(w, A, B, sa, sb, target_s=0.05)
    assert check is None
