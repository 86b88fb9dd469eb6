"""Host-side behaviour of bench.py that needs no GPU: the refusal of more
than one GPU, and the rule that HBM traffic from the committed counter
summary is reported only for the kernel source it was measured on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one MI355X" in r.stderr


def test_traffic_only_for_the_measured_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    # no summary at all
    assert bench.traffic_for_current_kernel() is None
    # a summary taken on the current source
    f.write_text(json.dumps({"kernel_digest": bench.kernel_digest(), "hbm_bytes_per_launch": 1234.0}))
    assert bench.traffic_for_current_kernel() == 1234.0
    # one taken on another source
    f.write_text(json.dumps({"kernel_digest": "0" * 16, "hbm_bytes_per_launch": 1234.0}))
    assert bench.traffic_for_current_kernel() is None
    # an unreadable one
    f.write_text("{not json")
    assert bench.traffic_for_current_kernel() is None


def test_committed_traffic_summary_is_well_formed():
    with open(os.path.join(ROOT, "profiles", "seg_attn_fullcache_traffic.json")) as fh:
        t = json.load(fh)
    assert len(t["kernel_digest"]) == 16
    assert t["hbm_bytes_per_launch"] > 0


def test_clock_summary_is_robust_to_dips():
    """The bench's clock figure is the median of the SMU samples: single
    readings dip far below the clock a long kernel runs at, and must not pull
    the reported clock (or the fraction of the peak at that clock) down."""
    import bench
    cs = bench.ClockSampler.__new__(bench.ClockSampler)
    cs._thread, cs._h = None, None
    cs.samples = [1720.0] * 90 + [157.5] * 12 + [1748.0] * 10
    cs.avg_samples = []
    s = cs.stop()
    assert s["median_mhz"] == 1720.0 and s["samples"] == 112
    assert s["p10_mhz"] == 157.5 and s["p90_mhz"] == 1720.0     # sorted indices 11 and 100 of 112
    cs.samples = []
    assert cs.stop() is None


def test_clock_fraction_rejects_impossible_clock():
    """A clock at which the measured rate would exceed the MFMA peak is not
    the clock the kernel ran at; the bench line then gives no fraction."""
    import bench
    ok = bench.clock_fraction({"median_mhz": 1720.0}, 1294.3)
    assert ok["peak_at_clock_tflops"] == 1803.6 and abs(ok["frac_at_clock"] - 1294.3 / 1803.6) < 1e-4
    bad = bench.clock_fraction({"median_mhz": 95.0}, 1291.5)
    assert bad["frac_at_clock"] is None and bad["peak_at_clock_tflops"] is None and "95 MHz" in bad["note"]
