"""HBM traffic of the benchmark's kernels from rocprofv3 counters, and kernel-trace summaries.

``python -m combine_ep_layout_06_amd.hbm_counters collect --out DIR`` runs, for each workload
and for a plain 256 MiB device copy (``bench.py --only copy_probe``), one rocprofv3 pass per
counter (FETCH_SIZE, then WRITE_SIZE; each in a process of its own under a time limit).

``python -m combine_ep_layout_06_amd.hbm_counters summarize --out DIR`` reads those passes and
writes ``profiles/hbm_traffic.json`` (the record bench.py reads for ``roofline.traffic``) and one
markdown table per workload. Per kernel, the median KiB per dispatch of each counter is scaled
by the factor that makes the same counter read the known size of the copy, and set beside the
kernel's algorithmic bytes (accounting.py). A record holds the SHA-256 of the kernel's sources,
so the benchmark stops using it once they change.

``collect-detail`` and ``detail`` do the same for two more passes per workload: the L2's
write requests to memory (all, and those of 64 bytes; the rest are 32 bytes) and the mean
number of wavefronts resident per CU over each dispatch, written to
``profiles/launch_counters_prefill.md``; and three memory-path passes on the bf16 step (wave
and instruction counts, L2 hits, misses and DRAM credit stalls, L2 read latency), written to
``profiles/memory_path_counters_prefill_bf16.md``.

``python -m combine_ep_layout_06_amd.hbm_counters trace --csv FILE`` prints the per-kernel
duration summary of a ``rocprofv3 --kernel-trace`` CSV as a markdown table; ``steps --csv FILE
...`` the durations and gaps of the benchmark step's two kernels in each trace; ``coverage
--csv FILE ...`` how many of the kernels the build holds the traces launched, and which never.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COUNTERS = ("FETCH_SIZE", "WRITE_SIZE")
WORKLOADS = ("prefill_bf16", "prefill_fp8")
COPY_BYTES = 256 << 20

# the kernels of the benchmark step, the name fragment that finds them in a trace, and the
# sources whose hash keys the record
KERNELS = {
    "combine": ("combine_kernel", ["combine_ep_layout_06_amd/csrc/ep_combine.hip",
                                   "combine_ep_layout_06_amd/csrc/ep_device.h",
                                   "combine_ep_layout_06_amd/csrc/ep_internal.h"]),
    "layout_dispatch": ("layout_dispatch_", ["combine_ep_layout_06_amd/csrc/ep_fused.hip",
                                             "combine_ep_layout_06_amd/csrc/ep_layout_tile.h",
                                             "combine_ep_layout_06_amd/csrc/ep_dispatch_item.h",
                                             "combine_ep_layout_06_amd/csrc/ep_device.h",
                                             "combine_ep_layout_06_amd/csrc/ep_internal.h"]),
}


# counter groups of the detail passes, each within one pass's per-block limits (TCC: 2 of 4;
# SQ: 4 of 8 with the accumulation's own counter; GRBM: 1 of 2)
DETAIL_PASSES = {
    "wrreq": ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"),
    "occupancy": ("MeanOccupancyPerCU", "SQ_WAVES", "SQ_BUSY_CU_CYCLES"),
}
# memory-path passes on the bf16 prefill step (SQ: 8 of 8; TCC: 4 of 4; TA 2, TCP 3 of 4)
MEMORY_WORKLOAD = "prefill_bf16"
MEMORY_PASSES = {
    "diag1": ("SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VMEM",
              "SQ_INST_LEVEL_VMEM", "SQ_INSTS_VMEM_RD", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU"),
    "diag2": ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_sum",
              "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"),
    "diag3": ("TA_BUSY_avr", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TCP_PENDING_STALL_CYCLES_sum",
              "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum"),
}


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def pass_dir(out, counter, wl):
    return os.path.join(out, f"pmc_{counter}_{wl}")


def collect_command(out, counter, wl, display=False, counters=None):
    """The rocprofv3 pass (counters: the pass's counters, default the one named counter);
    display: with $R for the repository root and plain python3."""
    py, bench = (("python3", "$R/bench.py") if display
                 else (sys.executable, os.path.join(ROOT, "bench.py")))
    return ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", *(counters or (counter,)),
            "-d", pass_dir(out, counter, wl), "-o", wl, "--output-format", "csv", "--", py,
            bench, "--only", wl, "--steps", "12", "--warmup", "4"]


def run_passes(passes):
    """Runs (pass name, workload, counters) passes one by one; stops at the first failure."""
    for name, wl, counters, out in passes:
        cmd = collect_command(out, name, wl, counters=counters)
        print("[counters] " + " ".join(cmd), flush=True)
        res = subprocess.run(cmd, cwd="/tmp")
        if res.returncode != 0:
            print(f"[counters] pass failed with {res.returncode}", flush=True)
            return res.returncode
    return 0


def collect(out):
    os.makedirs(out, exist_ok=True)
    return run_passes([(c, wl, None, out) for wl in ("copy_probe",) + WORKLOADS
                       for c in COUNTERS])


def collect_detail(out):
    os.makedirs(out, exist_ok=True)
    return run_passes([(name, wl, counters, out) for wl in WORKLOADS
                       for name, counters in DETAIL_PASSES.items()]
                      + [(name, MEMORY_WORKLOAD, counters, out)
                         for name, counters in MEMORY_PASSES.items()])


def read_counter(out, counter, wl, pass_name=None):
    """Kernel name -> list of the counter's value per dispatch (pass_name: the pass that
    collected it, default the counter's own)."""
    files = glob.glob(os.path.join(pass_dir(out, pass_name or counter, wl), "**",
                                   "*counter_collection.csv"), recursive=True)
    per = {}
    for path in files:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def pick(per, fragment):
    """The values of the kernels whose name holds the fragment (one kernel per workload)."""
    vals = [v for k, vs in per.items() if fragment in k for v in vs]
    return vals


def summarize(out, json_path, md_dir):
    sys.path.insert(0, ROOT)
    from combine_ep_layout_06_amd import accounting as A
    from combine_ep_layout_06_amd import workloads as W

    copy = {c: statistics.median(pick(read_counter(out, c, "copy_probe"), "")) for c in COUNTERS}
    scale = {c: (COPY_BYTES / 1024) / copy[c] for c in COUNTERS}
    records, tables = [], {}
    for wl in WORKLOADS:
        cfg = W.get_config(wl)
        assert cfg.C >= cfg.T and cfg.route == "uniform"   # no drops: every pair is kept
        n_kept = cfg.T * cfg.K
        alg = {"combine": A.combine_bytes(cfg.T, cfg.K, cfg.H, n_kept),
               "layout_dispatch": A.layout_bytes(cfg.T, cfg.K)
               + A.dispatch_bytes(cfg.T, cfg.K, cfg.H, n_kept, cfg.fp8)}
        rows = []
        for kernel, (frag, srcs) in KERNELS.items():
            v = {c: pick(read_counter(out, c, wl), frag) for c in COUNTERS}
            if not v["FETCH_SIZE"] or not v["WRITE_SIZE"]:
                continue
            fk, wk = statistics.median(v["FETCH_SIZE"]), statistics.median(v["WRITE_SIZE"])
            traffic = int(round((fk * scale["FETCH_SIZE"] + wk * scale["WRITE_SIZE"]) * 1024))
            records.append({"kernel": kernel, "workload": wl,
                            "launches_sampled": [len(v["FETCH_SIZE"]), len(v["WRITE_SIZE"])],
                            "fetch_kib": fk, "write_kib": wk,
                            "fetch_scale": round(scale["FETCH_SIZE"], 5),
                            "write_scale": round(scale["WRITE_SIZE"], 5),
                            "traffic_bytes": traffic, "algorithmic_bytes": alg[kernel],
                            "sources": srcs, "sources_sha256": sources_sha256(srcs)})
            rows.append((kernel, fk, scale["FETCH_SIZE"], wk, scale["WRITE_SIZE"], traffic,
                         alg[kernel]))
        tables[wl] = (cfg, rows)
    rec = {"what": "HBM bytes per launch: median FETCH_SIZE and WRITE_SIZE (KiB per dispatch) "
                   "over the sampled launches, each scaled by the factor that makes the same "
                   "counter read the known size of a plain 256 MiB device copy (copy_probe). "
                   "The benchmark reports traffic only while the kernel's sources still hash "
                   "to sources_sha256. Written by combine_ep_layout_06_amd/hbm_counters.py.",
           "copy_probe": {"bytes": COPY_BYTES, "fetch_kib": copy["FETCH_SIZE"],
                          "write_kib": copy["WRITE_SIZE"]},
           "commands": [" ".join(collect_command("$OUT", c, "<wl>", display=True))
                        for c in COUNTERS]
                       + ["<wl> in {copy_probe, " + ", ".join(WORKLOADS) + "}; run from /tmp"],
           "records": records}
    with open(json_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    for wl, (cfg, rows) in tables.items():
        lines = [f"# HBM traffic per launch: {wl} (T={cfg.T}, H={cfg.H}, E={cfg.E}, K={cfg.K}, "
                 f"C={cfg.C}, {'FP8' if cfg.fp8 else 'bf16'} dispatch)", "",
                 "rocprofv3 counter passes, one counter per run, median KiB per dispatch over "
                 "the sampled launches, each scaled by the factor that makes the counter read "
                 f"the known size of a plain 256 MiB device copy (FETCH_SIZE reads "
                 f"{copy['FETCH_SIZE']:.1f} KiB, WRITE_SIZE {copy['WRITE_SIZE']:.1f} KiB for "
                 f"{COPY_BYTES // 1024} KiB).", "",
                 "Commands (run from /tmp; the package module prints and runs them):", "", "```",
                 "python3 -m combine_ep_layout_06_amd.hbm_counters collect --out $OUT", *rec["commands"],
                 "python3 -m combine_ep_layout_06_amd.hbm_counters summarize --out $OUT",
                 "```", "",
                 "| kernel | FETCH_SIZE KiB | x scale | WRITE_SIZE KiB | x scale | HBM bytes | "
                 "algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|---|"]
        for kernel, fk, fs, wk, ws, traffic, alg in rows:
            lines.append(f"| {kernel} | {fk:.1f} | {fs:.5f} | {wk:.1f} | {ws:.5f} | "
                         f"{traffic:,} | {alg:,} | {traffic / alg:.3f} |")
        with open(os.path.join(md_dir, f"hbm_counters_{wl}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    return 0


def detail(out, md_dir):
    """Median per dispatch of each detail counter for the step's kernels, as a markdown file."""
    sys.path.insert(0, ROOT)
    from combine_ep_layout_06_amd import workloads as W

    lines = ["# Write requests and occupancy per launch: prefill_bf16 and prefill_fp8", "",
             "rocprofv3 counter passes over the benchmark's step (12 timed + 4 warmup steps, "
             "median per dispatch). TCC_EA0_WRREQ_sum counts the L2's write requests to memory, "
             "TCC_EA0_WRREQ_64B_sum those that carry 64 bytes (the others carry 32); "
             "MeanOccupancyPerCU is the mean number of wavefronts resident per CU over the "
             "dispatch (a 1024-lane workgroup is 16 wavefronts); SQ_BUSY_CU_CYCLES the summed "
             "busy cycles of the CUs.", "",
             "Commands (run from /tmp; the package module prints and runs them):", "", "```",
             "python3 -m combine_ep_layout_06_amd.hbm_counters collect-detail --out $OUT",
             *[" ".join(collect_command("$OUT", name, "<wl>", display=True, counters=c))
               for name, c in DETAIL_PASSES.items()],
             "<wl> in {" + ", ".join(WORKLOADS) + "}; run from /tmp",
             "python3 -m combine_ep_layout_06_amd.hbm_counters detail --out $OUT",
             "```", "",
             "| workload | kernel | dispatches | WRREQ | WRREQ 64 B | bytes they carry | "
             "mean waves per CU | waves | busy CU cycles |", "|---|---|---|---|---|---|---|---|---|"]
    for wl in WORKLOADS:
        cfg = W.get_config(wl)
        for kernel, (frag, _) in KERNELS.items():
            v = {c: pick(read_counter(out, c, wl, name), frag)
                 for name, cs in DETAIL_PASSES.items() for c in cs}
            if not all(v.values()):
                continue
            m = {c: statistics.median(x) for c, x in v.items()}
            wr, w64 = m["TCC_EA0_WRREQ_sum"], m["TCC_EA0_WRREQ_64B_sum"]
            carried = (wr - w64) * 32 + w64 * 64
            lines.append(f"| {wl} ({'FP8' if cfg.fp8 else 'bf16'}) | {kernel} | "
                         f"{len(v['TCC_EA0_WRREQ_sum'])} | {wr:,.0f} | {w64:,.0f} | "
                         f"{carried:,.0f} | {m['MeanOccupancyPerCU']:.1f} | "
                         f"{m['SQ_WAVES']:,.0f} | {m['SQ_BUSY_CU_CYCLES']:,.0f} |")
    with open(os.path.join(md_dir, "launch_counters_prefill.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return memory_detail(out, md_dir)


def memory_detail(out, md_dir):
    """The memory-path passes: every counter per kernel (median per dispatch), and the ratios
    that locate combine's limit, as a markdown file."""
    wl = MEMORY_WORKLOAD
    med = {k: {} for k in KERNELS}
    for name, cs in MEMORY_PASSES.items():
        for c in cs:
            for kernel, (frag, _) in KERNELS.items():
                v = pick(read_counter(out, c, wl, name), frag)
                if v:
                    med[kernel][c] = statistics.median(v)
    if not all(med.values()):
        return 0
    lines = [f"# Memory-path counters: {wl} step kernels (T=4096, H=2048, E=128, K=8)", "",
             "Three rocprofv3 counter passes, each its own run of the benchmark on the one "
             "workload (12 timed steps after 4 warm-up steps); median per dispatch over the "
             "sampled launches of each kernel. Commands (R = repository root, run from /tmp; "
             "`python3 -m combine_ep_layout_06_amd.hbm_counters collect-detail` runs them, "
             "`detail` writes this file):", "", "```",
             *[" ".join(collect_command("$OUT", name, wl, display=True, counters=c))
               for name, c in MEMORY_PASSES.items()], "```", "",
             "| counter | layout_dispatch | combine |", "|---|---|---|"]
    for c in sorted({c for cs in MEMORY_PASSES.values() for c in cs}):
        a, b = med["layout_dispatch"].get(c), med["combine"].get(c)
        lines.append(f"| {c} | {a:,.0f} | {b:,.0f} |")
    cb, ld = med["combine"], med["layout_dispatch"]
    ratio = lambda m, a, b: m[a] / m[b] if m.get(b) else float("nan")
    lines += ["", "Ratios:", "",
              f"* L2 read latency under load (TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum):"
              f" combine {ratio(cb, 'TCP_TCC_READ_REQ_LATENCY_sum', 'TCP_TCC_READ_REQ_sum'):,.0f}"
              f" cycles, layout_dispatch "
              f"{ratio(ld, 'TCP_TCC_READ_REQ_LATENCY_sum', 'TCP_TCC_READ_REQ_sum'):,.0f}.",
              f"* DRAM credit stalls per DRAM read request: combine "
              f"{ratio(cb, 'TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum', 'TCC_EA0_RDREQ_sum'):.2f}, "
              f"layout_dispatch "
              f"{ratio(ld, 'TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum', 'TCC_EA0_RDREQ_sum'):.2f}.",
              f"* L2 miss rate (TCC_MISS_sum / (TCC_HIT_sum + TCC_MISS_sum)): combine "
              f"{cb['TCC_MISS_sum'] / (cb['TCC_HIT_sum'] + cb['TCC_MISS_sum']):.2f}, "
              f"layout_dispatch "
              f"{ld['TCC_MISS_sum'] / (ld['TCC_HIT_sum'] + ld['TCC_MISS_sum']):.2f}."]
    with open(os.path.join(md_dir, f"memory_path_counters_{wl}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return 0


def trace_table(path, top=0):
    """Per-kernel duration summary of a --kernel-trace CSV (us), as markdown rows."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "")
            key = (name.split("(")[0].replace("ep::", ""), int(r["Grid_Size_X"]),
                   int(r["Workgroup_Size_X"]))
            per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                                           / 1e3)
    rows = sorted(per.items(), key=lambda kv: -sum(kv[1]))
    out = ["| kernel | grid (lanes) | workgroup | launches | mean | median | min | max |",
           "|---|---|---|---|---|---|---|---|"]
    for (name, grid, wg), ts in rows[:top or None]:
        out.append(f"| {name[:70]} | {grid} | {wg} | {len(ts)} | {statistics.fmean(ts):.2f} | "
                   f"{statistics.median(ts):.2f} | {min(ts):.2f} | {max(ts):.2f} |")
    return "\n".join(out)


def coverage_table(paths):
    """The kernels the build holds (``kernel_resources.json`` beside the library) against the
    ones the --kernel-trace CSVs launched, as markdown: counts, then every kernel never
    launched (names demangled with c++filt)."""
    with open(os.path.join(PKG, "kernel_resources.json")) as f:
        mangled = sorted(json.load(f)["kernels"])
    names = subprocess.run(["c++filt"], input="\n".join(mangled), capture_output=True,
                           text=True, check=True).stdout.splitlines()
    short = lambda n: n.replace("(anonymous namespace)::", "").split("(")[0].strip()
    built = {short(n) for n in names}
    launched = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                k = short(r["Kernel_Name"])
                if k in built:
                    launched[k] = launched.get(k, 0) + 1
    never = sorted(built - set(launched))
    fams = {}
    for k in built:
        fam = k.split("<")[0].replace("void ", "").replace("ep::", "")
        n_l = fams.setdefault(fam, [0, 0])
        n_l[0] += 1
        n_l[1] += k in launched
    out = [f"{len(built)} kernels built, {len(launched)} launched at least once, "
           f"{len(never)} never launched; {sum(launched.values())} launches of them in all.", "",
           "| kernel template | built | launched |", "|---|---|---|"]
    out += [f"| {fam} | {b} | {l} |" for fam, (b, l) in sorted(fams.items())]
    if never:
        out += ["", "Never launched:", ""] + [f"- {k}" for k in never]
    return "\n".join(out)


def step_table(paths):
    """Per trace: the step's two kernels (a fused layout + dispatch launch followed by a combine
    launch) and the gaps around them, median and min over the steps, as markdown rows. A step
    that follows a fill (the cold protocol) also gives the gap from the fill's end to the
    first kernel's start."""
    out = ["| trace | steps | fill end -> first kernel | layout + dispatch | gap | combine | "
           "first start -> combine end | combine end -> next step |",
           "|---|---|---|---|---|---|---|---|"]
    for path in paths:
        ks = []
        with open(path) as f:
            for r in csv.DictReader(f):
                n = r["Kernel_Name"]
                kind = ("ld" if "layout_dispatch_" in n else "cb" if "combine_kernel" in n
                        else "fill" if "FillFunctor" in n else "other")
                ks.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kind))
        ks.sort()
        cols = {"fill": [], "ld": [], "gap": [], "cb": [], "span": [], "next": []}
        for i in range(len(ks) - 1):
            (s0, e0, k0), (s1, e1, k1) = ks[i], ks[i + 1]
            if k0 != "ld" or k1 != "cb":
                continue
            cols["ld"].append((e0 - s0) / 1e3)
            cols["cb"].append((e1 - s1) / 1e3)
            cols["gap"].append((s1 - e0) / 1e3)
            cols["span"].append((e1 - s0) / 1e3)
            if i > 0 and ks[i - 1][2] == "fill":
                cols["fill"].append((s0 - ks[i - 1][1]) / 1e3)
            if i + 2 < len(ks) and ks[i + 2][2] == "ld":     # back to back: the next step's start
                cols["next"].append((ks[i + 2][0] - e1) / 1e3)
        f = lambda v: f"{statistics.median(v):.2f} ({min(v):.2f})" if v else "-"
        out.append(f"| {os.path.basename(os.path.dirname(path))} | {len(cols['ld'])} | "
                   f"{f(cols['fill'])} | {f(cols['ld'])} | {f(cols['gap'])} | {f(cols['cb'])} | "
                   f"{f(cols['span'])} | {f(cols['next'])} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("action", choices=("collect", "summarize", "collect-detail", "detail",
                                       "trace", "steps", "coverage"))
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "pmc"))
    ap.add_argument("--json", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    ap.add_argument("--md-dir", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--csv", default=None, nargs="+")
    ap.add_argument("--top", type=int, default=0)
    a = ap.parse_args()
    if a.action == "collect":
        return collect(a.out)
    if a.action == "summarize":
        return summarize(a.out, a.json, a.md_dir)
    if a.action == "collect-detail":
        return collect_detail(a.out)
    if a.action == "detail":
        return detail(a.out, a.md_dir)
    if a.action == "steps":
        print(step_table(a.csv))
        return 0
    if a.action == "coverage":
        print(coverage_table(a.csv))
        return 0
    print(trace_table(a.csv[0], a.top))
    return 0


if __name__ == "__main__":
    sys.exit(main())
