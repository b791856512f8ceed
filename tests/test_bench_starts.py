"""Host logic of the benchmark's multi-start mode: the median-of-starts summary (no GPU)."""
import importlib.util
import os
import statistics

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def line(value, us, dec, cpu=None):
    return {"value": value, "us_per_step": us, "cold_single_shot": {"us_median": us + 6},
            "prefill_fp8": {"us_per_step": us - 6, "cold_single_shot": {"us_median": us}},
            "t128_us": {"decode_bf16": {"us_single_shot_median": dec},
                        "decode_fp8": {"us_single_shot_median": dec + 0.3}},
            "cpu_baseline": cpu, "tag": f"start-{value}"}


def test_median_start_keeps_its_line_and_figures_are_summarised(bench):
    lines = [line(5100.0, 52.6, 12.3, cpu={"value": 1.0}), line(5157.0, 52.0, 12.1),
             line(4990.0, 53.8, 12.6)]
    out = bench.aggregate_starts(lines)
    assert out["tag"] == "start-5100.0" and out["value"] == 5100.0   # the median start
    st = out["starts"]
    assert st["n"] == 3 and st["picked_start"] == 0
    assert st["value_per_start"] == [5100.0, 5157.0, 4990.0]
    f = st["prefill_bf16 us_per_step"]
    xs = [52.6, 52.0, 53.8]
    assert f["median"] == 52.6 and f["min"] == 52.0 and f["max"] == 53.8
    assert f["cv"] == pytest.approx(statistics.stdev(xs) / statistics.fmean(xs), abs=1e-4)
    assert st["decode_fp8 us_single_shot_median"]["median"] == pytest.approx(12.6)
    assert st["prefill_fp8 cold us_median"]["per_start"] == xs
    assert out["cpu_baseline"] == {"value": 1.0}


def test_even_count_takes_the_low_median_and_borrows_the_cpu_baseline(bench):
    lines = [line(5000.0, 53.0, 12.2, cpu={"value": 2.0}), line(5200.0, 51.6, 12.0)]
    out = bench.aggregate_starts(lines)
    assert out["value"] == 5000.0 and out["starts"]["picked_start"] == 0
    lines = [line(5200.0, 51.6, 12.0, cpu={"value": 2.0}), line(5000.0, 53.0, 12.2)]
    out = bench.aggregate_starts(lines)
    assert out["value"] == 5000.0 and out["starts"]["picked_start"] == 1
    assert out["cpu_baseline"] == {"value": 2.0}      # only the first start timed the oracle


def test_missing_figures_are_left_out_and_no_lines_is_an_error(bench):
    out = bench.aggregate_starts([{"value": 1.0}])
    assert out["starts"]["n"] == 1 and "prefill_bf16 us_per_step" not in out["starts"]
    with pytest.raises(ValueError):
        bench.aggregate_starts([])


def test_default_is_three_starts_and_each_child_runs_one(bench, monkeypatch, capsys):
    import json
    import subprocess
    import sys

    monkeypatch.setattr(sys, "argv", ["bench.py"])
    assert bench.parse().starts is None              # main() turns None into 3, or 1 with --only
    calls = []

    class Done:
        returncode = 0

        def __init__(self, value):
            self.stdout = "[noise]\n" + json.dumps(line(value, 52.0, 12.0)) + "\n"

    def fake_run(cmd, **kw):
        calls.append(cmd)
        return Done(5000.0 + len(calls))

    monkeypatch.setattr(subprocess, "run", fake_run)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "7", "--warmup", "2"])
    bench.main()
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert len(calls) == 3 and out["starts"]["n"] == 3
    for k, cmd in enumerate(calls):
        assert cmd[cmd.index("--starts") + 1] == "1"          # a child never forks again
        assert cmd[cmd.index("--rotate") + 1] == str(k)
        assert cmd[cmd.index("--steps") + 1] == "7"
        assert ("--no-cpu-baseline" in cmd) == (k > 0)         # only the first times the oracle
