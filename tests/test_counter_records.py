"""Host logic of the HBM counter records (no GPU): the counter module's scaling of rocprofv3
passes into per-launch bytes, its trace tables, and the benchmark's use of a record only while
the kernel's sources still hash to what the record says."""
import csv
import hashlib
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def H():
    import sys
    sys.path.insert(0, ROOT)
    from combine_ep_layout_06_amd import hbm_counters
    return hbm_counters


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_for_counters", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def write_pass(H, out, counter, wl, rows, pass_name=None):
    d = H.pass_dir(out, pass_name or counter, wl)
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, f"{wl}_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, name, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": name, "Counter_Value": value})


def test_summarize_scales_each_counter_by_the_copy(H, tmp_path):
    out = str(tmp_path / "pmc")
    copy_kib = H.COPY_BYTES / 1024
    # the copy reads half its size on FETCH_SIZE and its size on WRITE_SIZE: scales 2 and 1
    write_pass(H, out, "FETCH_SIZE", "copy_probe", [("copy", "FETCH_SIZE", copy_kib / 2)] * 3)
    write_pass(H, out, "WRITE_SIZE", "copy_probe", [("copy", "WRITE_SIZE", copy_kib)] * 3)
    for wl in H.WORKLOADS:
        write_pass(H, out, "FETCH_SIZE", wl,
                   [("void ep::combine_kernel<2>", "FETCH_SIZE", 1000.0),
                    ("void ep::combine_kernel<2>", "FETCH_SIZE", 1002.0),
                    ("void ep::combine_kernel<2>", "FETCH_SIZE", 998.0),
                    ("void ep::layout_dispatch_bf16_kernel<8>", "FETCH_SIZE", 10.0),
                    ("at::fill", "FETCH_SIZE", 5e6)])
        write_pass(H, out, "WRITE_SIZE", wl,
                   [("void ep::combine_kernel<2>", "WRITE_SIZE", 300.0),
                    ("void ep::layout_dispatch_bf16_kernel<8>", "WRITE_SIZE", 4000.0)])
    js, md = tmp_path / "traffic.json", tmp_path / "md"
    md.mkdir()
    assert H.summarize(out, str(js), str(md)) == 0
    rec = json.loads(js.read_text())
    assert rec["copy_probe"]["fetch_kib"] == copy_kib / 2
    by = {(r["kernel"], r["workload"]): r for r in rec["records"]}
    assert set(by) == {(k, wl) for k in H.KERNELS for wl in H.WORKLOADS}
    cb = by[("combine", H.WORKLOADS[0])]
    assert cb["fetch_kib"] == 1000.0 and cb["write_kib"] == 300.0     # medians
    assert cb["fetch_scale"] == 2.0 and cb["write_scale"] == 1.0
    assert cb["traffic_bytes"] == round((1000.0 * 2 + 300.0) * 1024)
    assert cb["sources_sha256"] == H.sources_sha256(cb["sources"])
    ld = by[("layout_dispatch", H.WORKLOADS[0])]
    assert ld["traffic_bytes"] == round((10.0 * 2 + 4000.0) * 1024)   # torch's fill left out
    for wl in H.WORKLOADS:
        assert (md / f"hbm_counters_{wl}.md").exists()


def test_trace_and_step_tables(H, tmp_path):
    path = tmp_path / "t_kernel_trace.csv"
    rows = []
    t = 1_000_000
    for _ in range(3):          # three steps: fused kernel, gap of 1 us, combine
        rows.append(("void ep::(anonymous namespace)::layout_dispatch_bf16_kernel<8, 2>(int)", t, t + 25_000))
        rows.append(("void ep::(anonymous namespace)::combine_kernel<2, 4>(int)", t + 26_000, t + 52_000))
        t += 100_000
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"])
        for name, s, e in rows:
            w.writerow([name, s, e, 1024, 256])
    table = H.trace_table(str(path))
    assert "| layout_dispatch_bf16_kernel<8, 2> | 1024 | 256 | 3 | 25.00 |" in table
    steps = H.step_table([str(path)])
    assert "| 3 | - | 25.00 (25.00) | 1.00 (1.00) | 26.00 (26.00) | 52.00 (52.00) |" in steps


def test_bench_uses_a_record_only_while_the_sources_match(bench, tmp_path):
    root = tmp_path
    (root / "src").mkdir()
    (root / "profiles").mkdir()
    src = root / "src" / "k.hip"
    src.write_text("kernel v1\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    rec = {"records": [{"kernel": "combine", "workload": "prefill_bf16", "traffic_bytes": 1234,
                        "sources": ["src/k.hip"], "sources_sha256": digest}]}
    (root / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    assert bench.counter_traffic("combine", "prefill_bf16", root=str(root)) == 1234
    assert bench.counter_traffic("combine", "prefill_fp8", root=str(root)) is None
    src.write_text("kernel v2\n")                     # the kernel changed since the counters
    assert bench.counter_traffic("combine", "prefill_bf16", root=str(root)) is None


def test_coverage_table_counts_built_and_launched(H, tmp_path):
    """coverage: the build's kernel list against a trace; a kernel the trace never launched is
    named, foreign kernels (torch's) are ignored."""
    import shutil
    if shutil.which("c++filt") is None or not os.path.exists(
            os.path.join(ROOT, "combine_ep_layout_06_amd", "kernel_resources.json")):
        pytest.skip("needs c++filt and a built kernel_resources.json")
    import subprocess
    with open(os.path.join(ROOT, "combine_ep_layout_06_amd", "kernel_resources.json")) as f:
        mangled = sorted(json.load(f)["kernels"])
    names = subprocess.run(["c++filt"], input="\n".join(mangled), capture_output=True,
                           text=True, check=True).stdout.splitlines()
    trace = tmp_path / "t_kernel_trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name"])
        w.writeheader()
        for n in names[1:]:                       # every kernel but the first, twice
            w.writerow({"Kernel_Name": n})
            w.writerow({"Kernel_Name": n})
        w.writerow({"Kernel_Name": "void at::native::vectorized_elementwise_kernel<4>(int)"})
    text = H.coverage_table([str(trace)])
    n = len(set(names))
    assert text.splitlines()[0] == (f"{n} kernels built, {n - 1} launched at least once, "
                                    f"1 never launched; {2 * (n - 1)} launches of them in all.")
    missing = names[0].replace("(anonymous namespace)::", "").split("(")[0].strip()
    assert text.splitlines()[-1] == f"- {missing}"
