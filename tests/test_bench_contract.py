"""CPU checks of bench.py's own logic: the one-GPU guard, the rule that a committed counter
figure is reported only while the kernel's sources are unchanged, and the roofline's choice of
bound on the layer's real shapes (no GPU is touched)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import inputs as S  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    good = bench.kernel_source_hash("k_dec_gateup")
    assert good is not None and bench.kernel_source_hash("k_unknown") is None
    t = {"fetch_scale": 2.0, "write_scale": 1.0,
         "kernels": {"k_dec_gateup": {"source_hash": good, "fetch_kib": 10.0, "write_kib": 3.0},
                     "k_dec_down": {"source_hash": "0" * 16, "fetch_kib": 10.0, "write_kib": 3.0}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.traffic_for("k_dec_gateup") == 10 * 1024 * 2 + 3 * 1024
    assert bench.traffic_for("k_dec_down") is None      # sources changed since the counters
    assert bench.traffic_for("k_combine@prefill") is None  # no entry
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("k_dec_gateup") is None


@pytest.mark.parametrize("q4,bound", [(False, "hbm"), (True, "mfma")])
def test_gateup_roofline_bound_at_prefill(q4, bound):
    """At M = 4096 with every expert non-empty the bf16 gate/up GEMM needs longer on HBM than on
    MFMA at datasheet peaks (1.09 GB vs 137 GFLOP), the 4-bit one longer on MFMA (0.32 GB)."""
    w = S.PREFILL
    peaks = {"hbm_gbs": 6400.0, "mfma_tflops": 2000.0}
    r = bench.gateup_roofline({"gemm_gateup": [0.25, 0.25]}, w, w.M, w.E, q4, peaks)
    assert r["bound"] == bound and r["avg_us"] == 250.0
    flops = w.M * w.k * 2 * w.I * w.H * 2
    wb = 0.5625 if q4 else 2
    # algorithmic bytes only: gate/up weights of the non-empty routed experts, x once (the shared
    # expert's gate/up tiles run in the down launch)
    nbytes = int(w.E * 2 * w.I * w.H * wb) + w.M * w.H * 2
    assert r["bytes_per_launch"] == nbytes and r["flops_per_launch"] == flops
    if bound == "hbm":
        assert r["frac"] == pytest.approx(nbytes / 250e-6 / 1e9 / bench.HBM_PEAK_GBS, abs=1e-4)
        assert r["frac_measured"] == pytest.approx(nbytes / 250e-6 / 1e9 / 6400.0, abs=1e-4)
    else:
        assert r["frac"] == pytest.approx(flops / 250e-6 / 1e12 / bench.BF16_PEAK_TFLOPS, abs=1e-4)
        assert r["frac_measured"] == pytest.approx(flops / 250e-6 / 1e12 / 2000.0, abs=1e-4)


@pytest.mark.parametrize("total", [1, 4, 5, 20, 23, 200])
def test_rounds_cover_exactly_the_steps(total):
    """The timed steps are split into at most 5 rounds that together run exactly `total` steps."""
    sizes = bench.round_sizes(total)
    assert sum(sizes) == total and len(sizes) == min(5, total) and max(sizes) - min(sizes) <= 1


def test_rounds_rewarm_after_the_cpu_arm_untimed():
    """With a CPU arm between rounds, each arm is followed by untimed re-warm calls (at least
    REWARM_MIN); the timed calls are exactly `total`, numbered 0..total-1, and no re-warm call or
    CPU arm falls inside a timed round."""
    log = []

    class Ev:
        def record(self):
            log.append("rec")

        def elapsed_time(self, other):
            return 1.0

    nr = len(bench.round_sizes(23))
    bench.timed_rounds(lambda i: log.append(("step", i)), 23, between=lambda r: log.append("cpu"),
                       sync=lambda: log.append("sync"), event=Ev, rewarm_ms=0.0)
    steps = [e for e in log if isinstance(e, tuple)]
    assert len(steps) == 23 + bench.REWARM_MIN * nr
    timed, inside, rounds, after_cpu = [], False, 0, None
    for e in log:
        if e == "rec":
            inside = not inside
            rounds += not inside
        elif isinstance(e, tuple):
            if inside:
                timed.append(e[1])
            else:
                assert after_cpu is not None and e[1] == 0, "an untimed call before any CPU arm"
                after_cpu += 1
        elif e == "cpu":
            assert not inside
            assert after_cpu is None or after_cpu == bench.REWARM_MIN
            after_cpu = 0
    assert timed == list(range(23)) and rounds == nr and after_cpu == bench.REWARM_MIN
