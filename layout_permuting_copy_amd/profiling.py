"""rocprofv3 collection and summaries for the tile-copy kernels.

    python -m layout_permuting_copy_amd.profiling --raw <raw output dir> --out profiles [--quick]

runs, as child processes (this process never touches the GPU):

* the kernel trace of the benchmark command
  ``rocprofv3 --kernel-trace --stats --output-format csv ... -- python3 bench.py --no-sweep --no-cpu``
  -> ``kernel_trace_<workload>.md`` (rocprofv3's average kernel duration next to the benchmark's own
  HIP-event figure);
* one counter pass per group and workload
  ``rocprofv3 --pmc <group> --kernel-trace --output-format csv ... -- python3 bench.py --only <w>``:
  FETCH_SIZE; WRITE_SIZE; SQ_LDS_BANK_CONFLICT + SQ_INSTS_LDS; TCC_HIT_sum + TCC_MISS_sum.
  The identity copy of 2^28 float32 (1 GiB read, 1 GiB written) calibrates FETCH_SIZE and
  WRITE_SIZE: each counter is scaled by (known bytes / what it reads for that copy).
  -> ``counters_<workload>.md`` and ``traffic.json`` (HBM bytes per launch, with a hash of the kernel
  sources: a summary taken on other sources is not used).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import tempfile
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layout_permuting_copy_amd", "csrc")
KERNEL_SOURCES = ("device_common.hpp", "transpose.hpp", "kernels.hip", "transpose_eb1.hip", "transpose_eb2.hip",
                  "transpose_eb4.hip", "transpose_eb8.hip", "transpose_eb16.hip", "plan.hpp", "plan.cpp", "bank.cpp")
CALIBRATION = "identity_268435456_float32"
CALIBRATION_BYTES = 1 << 30  # read and written once each
GROUPS = {"fetch": ["FETCH_SIZE"], "write": ["WRITE_SIZE"], "lds": ["SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"],
          "tcc": ["TCC_HIT_sum", "TCC_MISS_sum"]}
WORKLOADS = ["sf_transpose_65536x2x1x4x32_f32", "transpose_16384x16384_float32", "transpose_16384x16384_bfloat16",
             "transpose_8192x8192_int8", "transpose_8192x8192_float16", "transpose_8192x8192_float64",
             "transpose_8192x8192_int4vec", "transpose_8191x8190_float16", "transpose_8191x8190_int8",
             "slice_8192x8192[1:8191:1,0:8190:2]_float16",
             "permute0213_32x32x2048x128_bfloat16", CALIBRATION]


def kernel_source_hash(paths=None) -> str:
    h = hashlib.sha256()
    for path in paths or [os.path.join(CSRC, name) for name in KERNEL_SOURCES]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the device primitives and their example kernels (the wave permute's counters)
DEV_SOURCES = (os.path.join(ROOT, "include", "tile_copy_dev.hpp"), os.path.join(CSRC, "dev_examples.hip"))


def _run(cmd, log, timeout):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(timeout)] + cmd, stdout=f, stderr=subprocess.STDOUT,
                           cwd=ROOT)
    if r.returncode != 0:
        tail = open(log).read()[-2000:]
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{tail}")
    return open(log).read()


def _csv(path_glob):
    files = glob.glob(path_glob, recursive=True)
    if not files:
        raise FileNotFoundError(path_glob)
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def counters_per_kernel(raw_dir, match="tc::"):
    """{kernel name: {counter: mean over dispatches}} for the kernels whose name contains `match`
    (default: the library's tc:: kernels)."""
    rows = _csv(os.path.join(glob.escape(raw_dir), "**", "*counter_collection.csv"))
    per = defaultdict(lambda: defaultdict(float))
    name = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        name[d] = r["Kernel_Name"]
    out = defaultdict(lambda: defaultdict(list))
    for d, cs in per.items():
        if match not in name[d]:
            continue
        for c, v in cs.items():
            out[name[d]][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} | {"dispatches": len(next(iter(cs.values())))}
            for k, cs in out.items()}


def file_stem(workload: str) -> str:
    """A workload name as a portable file name (slice brackets, colons and commas become _)."""
    return re.sub(r"[^A-Za-z0-9.-]+", "_", workload).strip("_")


def short_kernel(name: str) -> str:
    return name.split("(")[0].replace("void ", "").replace("tc::dev::", "").replace("tc::(anonymous namespace)::", "")


def collect(raw: str, out: str, quick: bool = False) -> None:
    os.makedirs(raw, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    py = sys.executable or "python3"
    # 1. kernel trace of the benchmark command
    tdir = os.path.join(raw, "trace")
    bench_cmd = [py, "bench.py", "--no-sweep", "--no-cpu", "--steps", "200", "--warmup", "10"]
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", tdir, "-o", "bench", "--"] + bench_cmd
    log = _run(cmd, os.path.join(raw, "trace.log"), 600)
    line = next(l for l in log.splitlines() if l.startswith('{"metric"'))
    bench = json.loads(line)
    stats = _csv(os.path.join(glob.escape(tdir), "**", "*kernel_stats.csv"))
    wl = bench["config"]["workload"]
    md = [f"# Kernel trace: {wl} (benchmark command)", "",
          "Command (repo root, library built):", "```", " ".join(cmd).replace(tdir, "<raw>/trace"), "```", "",
          f"Benchmark line: value {bench['value']} GB/s; average launch duration (HIP events around the "
          f"timed region / launches) {bench['roofline']['kernel_us_mean']} us -> "
          f"{bench['roofline']['achieved']} GB/s = {100 * bench['roofline']['frac']:.1f}% of 8 TB/s.", "",
          "| kernel | calls | average (us) | total (us) | % |", "|---|---|---|---|---|"]
    for r in stats:
        avg_ns = float(r.get("AverageNs") or float(r["TotalDurationNs"]) / max(1, int(r["Calls"])))
        md.append(f"| `{short_kernel(r['Name'])[:90]}` | {r['Calls']} | {avg_ns / 1e3:.3f} | "
                  f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    tc_rows = [r for r in stats if "tc::" in r["Name"]]
    if tc_rows:
        avg = float(tc_rows[0].get("AverageNs") or float(tc_rows[0]["TotalDurationNs"]) / int(tc_rows[0]["Calls"])) / 1e3
        alg = bench["roofline"]["algorithmic_bytes_per_launch"]
        md += ["", f"rocprofv3 average of the copy kernel: {avg:.3f} us -> {alg / (avg * 1e-6) / 1e9:.1f} GB/s "
                   f"({alg / (avg * 1e-6) / 1e9 / 80:.1f}% of 8 TB/s); the benchmark's HIP-event figure also "
                   f"counts the dispatch gap between back-to-back launches "
                   f"({bench['roofline']['kernel_us_mean'] - avg:.2f} us per launch here)."]
    with open(os.path.join(out, f"kernel_trace_{file_stem(wl)}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    # 2. counter passes
    workloads = [wl, CALIBRATION] if quick else WORKLOADS
    results = defaultdict(dict)
    cmds = {}
    for w in workloads:
        for g, cs in GROUPS.items():
            d = os.path.join(raw, f"{g}_{w}")
            cmd = ["rocprofv3", "--pmc", *cs, "--kernel-trace", "--output-format", "csv", "-d", d, "-o", "run", "--",
                   py, "bench.py", "--only", w, "--steps", "4", "--warmup", "1"]
            _run(cmd, d + ".log", 120)
            cmds[(g, w)] = " ".join(cmd).replace(d, f"<raw>/{g}_{w}")
            for k, vals in counters_per_kernel(d).items():
                results[w].setdefault("kernel", short_kernel(k))
                for c in cs:
                    results[w][c] = vals.get(c)
    cal = results[CALIBRATION]
    f_fetch = CALIBRATION_BYTES / (cal["FETCH_SIZE"] * 1024)
    f_write = CALIBRATION_BYTES / (cal["WRITE_SIZE"] * 1024)
    traffic = {"kernel_source_hash": kernel_source_hash(), "calibration": {
        "kernel": cal["kernel"], "workload": CALIBRATION, "known_bytes_each_way": CALIBRATION_BYTES,
        "FETCH_SIZE_KiB": cal["FETCH_SIZE"], "WRITE_SIZE_KiB": cal["WRITE_SIZE"],
        "fetch_factor": f_fetch, "write_factor": f_write}, "workloads": {}}
    for w, r in results.items():
        fetch = r["FETCH_SIZE"] * 1024 * f_fetch
        write = r["WRITE_SIZE"] * 1024 * f_write
        traffic["workloads"][w] = {"kernel": r["kernel"], "fetch_bytes": fetch, "write_bytes": write,
                                   "hbm_bytes_per_launch": fetch + write,
                                   "SQ_LDS_BANK_CONFLICT": r.get("SQ_LDS_BANK_CONFLICT"),
                                   "SQ_INSTS_LDS": r.get("SQ_INSTS_LDS"),
                                   "TCC_HIT_sum": r.get("TCC_HIT_sum"), "TCC_MISS_sum": r.get("TCC_MISS_sum")}
        md = [f"# Counters: {w}", "", f"Kernel: `{r['kernel']}`", "", "Commands (repo root, one pass each):", "```"]
        md += [cmds[(g, w)] for g in GROUPS]
        md += ["```", "", "| counter | mean per dispatch |", "|---|---|"]
        for c in sum(GROUPS.values(), []):
            md.append(f"| {c} | {r.get(c)} |")
        md += ["", f"FETCH_SIZE x {f_fetch:.3f} and WRITE_SIZE x {f_write:.3f} (calibrated on the identity copy of "
                   f"1 GiB): {fetch / 2**20:.1f} MiB fetched, {write / 2**20:.1f} MiB written per launch."]
        hits, miss = r.get("TCC_HIT_sum"), r.get("TCC_MISS_sum")
        if hits is not None and miss:
            md.append(f"TCC hit rate: {100 * hits / (hits + miss):.1f}%.")
        with open(os.path.join(out, f"counters_{file_stem(w)}.md"), "w") as f:
            f.write("\n".join(md) + "\n")
    with open(os.path.join(out, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    print(json.dumps({w: {k: v for k, v in d.items() if k != "kernel"} for w, d in traffic["workloads"].items()}))


# (which tile, k, shift) of the wave permute example: 0 = the scale-factor tile (2,1,4,32),
# 1 = the 4 x 64 transpose; the library's chooser takes (2, 3) for tile 1 and declines tile 0
WAVE_PERMUTE_CASES = [(1, 0, 0), (1, 2, 3), (1, 1, 3), (0, 0, 0), (0, 1, 3), (0, 2, 3)]
WAVE_PERMUTE_TILES = 65536


def collect_wave_permute(raw: str, out: str) -> None:
    """SQ_LDS_BANK_CONFLICT and SQ_INSTS_LDS per dispatch of the device wave permute example
    (tcd::wave_permute in place on LDS tiles, one wave per tile), one counter pass per
    (tile, k, shift), and its kernel time -> counters_wave_permute.md and wave_permute.json."""
    os.makedirs(raw, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    py = sys.executable or "python3"
    rows, cmds = [], []
    for which, k, shift in WAVE_PERMUTE_CASES:
        d = os.path.join(raw, f"wp_{which}_{k}_{shift}")
        args = ["-m", "layout_permuting_copy_amd.dev", "permute", "--which", str(which), "--k", str(k), "--shift",
                str(shift), "--tiles", str(WAVE_PERMUTE_TILES)]
        cmd = ["rocprofv3", "--pmc", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "--kernel-trace", "--output-format", "csv",
               "-d", d, "-o", "run", "--", py, *args, "--reps", "3"]
        _run(cmd, d + ".log", 120)
        cmds.append(" ".join(cmd).replace(d, f"<raw>/wp_{which}_{k}_{shift}"))
        cnt = next(iter(counters_per_kernel(d, match="permute_tiles").values()))
        timing = _run([py, *args, "--reps", "20"], d + "_time.log", 120)
        t = json.loads(next(l for l in timing.splitlines() if l.startswith("{")))
        rows.append({"which": which, "k": k, "shift": shift, "tiles": WAVE_PERMUTE_TILES,
                     "SQ_LDS_BANK_CONFLICT": cnt["SQ_LDS_BANK_CONFLICT"], "SQ_INSTS_LDS": cnt["SQ_INSTS_LDS"],
                     "kernel_us_mean": t["kernel_us_mean"], "gbs": t["gbs"]})
    with open(os.path.join(out, "wave_permute.json"), "w") as f:
        json.dump({"device_source_hash": kernel_source_hash(DEV_SOURCES), "cases": rows}, f, indent=1)
    md = ["# Counters: device wave permute (tcd::wave_permute, in place in LDS)", "",
          f"{WAVE_PERMUTE_TILES} tiles of 256 fp32 per dispatch, one wave per tile, four waves per workgroup; "
          "each tile is loaded (16-byte vectors), permuted in LDS, stored. Tile 0: the scale-factor tile "
          "(2,1,4,32) strides (128,128,32,1) -> (128,128,1,4); tile 1: (4,64) strides (64,1) -> (1,4).", "",
          "Commands (repo root, one pass each; the timing runs drop the rocprofv3 prefix and use --reps 20):",
          "```", *cmds, "```", "",
          "| tile | k | shift | SQ_LDS_BANK_CONFLICT / dispatch | per tile | SQ_INSTS_LDS / dispatch | kernel (us) | GB/s |",
          "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {r['which']} | {r['k']} | {r['shift']} | {r['SQ_LDS_BANK_CONFLICT']:.0f} | "
                  f"{r['SQ_LDS_BANK_CONFLICT'] / r['tiles']:.2f} | {r['SQ_INSTS_LDS']:.0f} | {r['kernel_us_mean']} | "
                  f"{r['gbs']} |")
    with open(os.path.join(out, "counters_wave_permute.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(rows))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--raw", default=os.path.join(tempfile.gettempdir(), "tile_copy_prof"))
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--quick", action="store_true", help="counters for the benchmark workload and calibration only")
    ap.add_argument("--wave-permute", action="store_true", help="only the device wave permute's counters")
    args = ap.parse_args()
    if args.wave_permute:
        collect_wave_permute(args.raw, args.out)
    else:
        collect(args.raw, args.out, args.quick)
    return 0


if __name__ == "__main__":
    sys.exit(main())
