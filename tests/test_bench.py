"""bench.py's output contract: one JSON line with the metric, the step time, the roofline of
the dominant kernel and the oracle baseline; more than one GPU is refused."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_more_than_one_gpu():
    """The build runs on one GPU: --gpus above 1 exits with status 2 and says so (before any
    device is touched)."""
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    """A short default-workload run: exactly one JSON line on stdout, with the fields the metric
    needs, the requested step and warm-up counts exactly (7 steps over 2 rotated sets: three
    whole cycles and one more), a roofline whose fraction is achieved / peak, and the target
    shape's own record."""
    print("bench.py --steps 7 --warmup 3 (subprocess)", flush=True)
    r = subprocess.run([sys.executable, "-u", BENCH, "--steps", "7", "--warmup", "3", "--rotate", "2",
                        "--targets", "dit_xl2_256", "--cpu-seconds", "1"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    res = json.loads(lines[0])
    sys.path.insert(0, ROOT)
    import bench
    assert res["metric"] == bench.METRIC
    assert res["n_gpus"] == 1 and res["steps"] == 7 and res["warmup"] == 3 and res["higher_is_better"] is True
    assert res["unit"] == "TOPS" and res["value"] > 0 and res["ms_per_step"] > 0
    assert res["vs_baseline"] is None and res["data"] == "synthetic"
    cfg = res["config"]
    assert cfg["workload"] == "highres_16k" and (cfg["B"], cfg["H"], cfg["N"], cfg["d"]) == (2, 16, 16384, 64)
    assert cfg["rotated_input_sets"] == 2
    ops = 4.0 * 2 * 16 * 16384 * 16384 * 64
    assert abs(res["value"] - ops / (res["ms_per_step"] * 1e-3) / 1e12) <= 1e-6 * res["value"]
    roof = res["roofline"]
    assert roof["bound"] in ("hbm", "mfma")
    assert roof["unit"] == ("GB/s" if roof["bound"] == "hbm" else "TOPS")
    assert 0 < roof["achieved"] and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) <= 1e-9
    assert roof["traffic"] is None or roof["traffic"] > 0
    t = res["targets"]["dit_xl2_256"]
    assert (t["B"], t["H"], t["N"], t["d"]) == (64, 16, 256, 72)
    assert t["ms_per_step"] > 0 and t["fwd_ms_per_call"] > 0 and 0 < t["fwd_hbm_frac"] < 1
    bw = t["backward"]
    assert bw["ms_per_call"] > 0 and 0 < bw["frac_of_bf16_mfma_peak"] < 1
    for name in ("highres_16k", "dit_xl2_256"):
        p = res["producer"][name]
        assert p["ms_per_call"] > 0 and 0 < p["frac_of_fp16_mfma_peak"] < 1 and p["unfused_ms"] > 0
    cpu = res["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]


def test_bench_refuses_bad_counts():
    """--steps below 1 or a negative --warmup exit with status 2 before any device is touched."""
    for extra in (["--steps", "0"], ["--warmup", "-1"]):
        r = subprocess.run([sys.executable, BENCH, *extra], capture_output=True, text=True, timeout=120)
        assert r.returncode == 2 and r.stdout == ""
