"""The benchmark's command-line contract: one JSON line with the fields its
consumers read, and a refusal of multi-GPU runs (the path runs on one GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def _json_line(stdout):
    lines = [l for l in stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, stdout[-2000:]
    return json.loads(lines[0])


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"], timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()


def test_flop_count_is_the_oracles_definition():
    """bench.py counts algorithmic flops itself (the timed legs import
    nothing from the oracle); the count must equal the oracle's."""
    import bench
    from oracle.ns import ns_iteration_flops
    for m, n in ((256, 512), (2048, 2048), (3072, 8192), (8192, 3072), (144, 400)):
        assert bench.iteration_flops(m, n) == ns_iteration_flops(m, n)
    assert abs(5 * bench.iteration_flops(3072, 8192) - 1.305e12) < 1e9


def _roofline_ok(roof, bound, unit):
    assert roof["bound"] == bound and roof["unit"] == unit
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert 0 < roof["frac"] < 1
    assert roof["traffic"] is None or roof["traffic"] > 0


@pytest.mark.gpu
def test_short_bench_line_has_the_contract_fields():
    r = _run(["--steps", "2", "--warmup", "1", "--no-cpu", "--no-grouped", "--no-accuracy",
              "--quant-steps", "2", "--quant-warmup", "1"], timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    d = _json_line(r.stdout)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "step_ms", "quant", "ns2048"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    assert "workload" in d["config"] and "model" not in d["config"]
    # value is the algorithmic rate of the timed steps
    assert abs(d["value"] - 1.305e12 / (d["ms_per_step"] * 1e-3) / 1e12) < 0.02 * d["value"]
    _roofline_ok(d["roofline"], "mfma", "TFLOP/s")
    _roofline_ok(d["quant"]["roofline"], "hbm", "GB/s")
    assert d["step_ms"]["min"] <= d["step_ms"]["median"] <= d["step_ms"]["max"]
    print(f"[bench] {d['value']} TFLOP/s, roofline frac {d['roofline']['frac']}", flush=True)
