"""The bench.py output contract: one JSON line with the metric, the timed
throughput, the dominant kernel's roofline object and (default run) the CPU
oracle baseline; more than one GPU is refused."""

import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    sys.path.insert(0, ROOT)
    import bench

    return bench


def _run(monkeypatch, *args):
    """bench.main() in this process (no child process: the tests' process may
    already hold the GPU)."""
    monkeypatch.setattr(sys, "argv", ["bench.py", *args])
    _bench().main()


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    with pytest.raises(SystemExit) as ex:
        _run(monkeypatch, "--gpus", "2")
    assert ex.value.code == 2
    assert "exactly one GPU" in capsys.readouterr().err


def test_cpu_baseline_object():
    from token_routing_grouped_amd import configs

    cb = _bench().cpu_baseline(configs.get("tiny"), "router", 32, min_seconds=0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "32 of 256 tokens" in cb["sample"]


@pytest.mark.gpu
def test_bench_line_fields(monkeypatch, capsys):
    _run(monkeypatch, "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-gates", "--config", "small")
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    # the vendor library's dense GEMM of the dominant kernel's size, for reference
    ref = d["dense_gemm_ref"]
    assert ref["kernel"] == rf["kernel"] and ref["M"] == d["config"]["T"] * d["config"]["k"]
    assert ref["avg_us"] > 0 and 0 < ref["frac"] < 1
    # tokens/s is the timed loop's: T tokens per ms_per_step
    assert abs(d["value"] - d["config"]["T"] / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
