"""The benchmark's measurements on the GPU (needs a gfx950 GPU): the bench line
of a small workload carries every field the driver and the roofline read, and
the HBM-traffic reading behind the line's last-level-cache estimate matches a
copy kernel of known traffic."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dense_gemm_fp8_amd import synth  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("no GPU", allow_module_level=True)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_bench_line_fields_small_workload():
    """bf16 256^3 through bench_one, as the bench's default line is made: the
    contract's keys, the roofline from live HIP events, the clock from the time
    record, the cold-cache launches and the CPU baseline with its parity."""
    _say("bench_one bf16_256")
    res = bench.bench_one(synth.workload(1), steps=5, warmup=2, opts=None, sched_name="interleave",
                          with_cpu=True, deadline_s=60.0, settle_ms=20.0, hbm_window_s=0.0)
    line = json.loads(json.dumps(res))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 5 and line["value"] > 0
    assert line["config"]["workload"] == "bf16_256"
    r = line["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and 0 < r["frac"] < 1
    # achieved is printed to 0.01 TFLOP/s and the mean launch time to 10 ns
    assert r["achieved"] == pytest.approx(synth.workload(1).flops / (r["kernel_ms_mean"] * 1e-3) / 1e12,
                                          rel=2e-3, abs=0.006)
    assert 50 < line["clock"]["mhz_mean"] < 3000
    assert line["box"]["arch"].startswith("gfx950") and line["box"]["compute_units"] == 256
    assert line["cold_cache"]["kernel_ms_mean"] > 0
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] >= 1
    assert line["parity"]["pass"] and line["parity"]["checked"] > 0
    assert line["hbm"] is None                      # skipped with hbm_window_s = 0


def test_hbm_activity_reads_a_known_copy():
    """A 1 GiB device-to-device copy moves 2 GiB through HBM per launch, far more
    than the last-level cache holds: the memory controllers' activity read by
    bench.hbm_window must give those bytes within 5 %."""
    if bench.metrics_reader() is None:
        pytest.skip("amdsmi gpu_metrics unavailable")
    _say("hbm window on a 1 GiB copy")
    x = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    r = bench.hbm_window(lambda: y.copy_(x), torch.cuda.current_stream(), 1.0, 60.0)
    assert r is not None, "no accumulator refresh inside the window"
    assert r["gfx_activity_pct"] > 90
    assert r["bytes_per_launch"] == pytest.approx(2 << 30, rel=0.05)
