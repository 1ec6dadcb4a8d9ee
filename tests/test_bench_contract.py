"""The benchmark's output contract: one JSON line with the fields its readers
rely on (metric, value, steps, roofline of the dominant kernel, the oracle's
host baseline), and a refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
def test_bench_prints_one_complete_json_line():
    cmd = [sys.executable, BENCH, "--workload", "basic_s4096", "--steps", "3", "--warmup", "1",
           "--no-other", "--no-peaks", "--cpu-budget", "2"]
    print("bench:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])

    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d.get(key), typ), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None            # the pages publish no throughput
    assert d["dtype"] == "bf16"
    assert isinstance(d["config"].get("workload"), str)

    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["peak"] > 0 and roof["achieved"] > 0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    assert "traffic" in roof                   # bytes, or null without a matching profile
    assert roof["traffic"] is None or roof["traffic"] > 0

    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle"
    assert cpu["value"] > 0 and isinstance(cpu["unit"], str)
    assert isinstance(cpu["cores"], int) and cpu["cores"] >= 1
    assert isinstance(cpu["sample"], str) and cpu["sample"]


@pytest.mark.gpu
def test_bench_peaks_only_reports_every_measured_peak():
    """bench.py --peaks-only: the MFMA-only rates (nearly constant and
    data-like operands) and the streaming bandwidths, each positive and below
    the spec peak it is compared with, and the fractions consistent."""
    cmd = [sys.executable, BENCH, "--peaks-only"]
    print("bench:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    p = json.loads(lines[0])["measured_peaks"]
    spec = p["spec"]
    for rate, frac in (("mfma_only_bf16_TFLOP/s", "mfma_only_frac_of_spec"),
                       ("mfma_only_bf16_random_operands_TFLOP/s", "mfma_only_random_operands_frac_of_spec")):
        assert 0 < p[rate] < spec["bf16_TFLOP/s"], (rate, p[rate])
        assert p[frac] == pytest.approx(p[rate] / spec["bf16_TFLOP/s"], rel=1e-9)
    for kind in ("copy", "stream_copy", "stream_add", "stream_read"):
        gbs = p[f"{kind}_GB/s"]
        assert 0 < gbs < spec["hbm_GB/s"], (kind, gbs)
        assert p[f"{kind}_frac_of_spec"] == pytest.approx(gbs / spec["hbm_GB/s"], rel=1e-9)
    assert set(p["stream_best_config"]) == {"copy", "add", "read"}
