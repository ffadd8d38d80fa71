"""rocprofv3 collection and summaries for the tile-copy kernels.

    python -m layout_permuting_copy_amd.profiling --raw <raw output dir> --out profiles [--quick]
    python -m layout_permuting_copy_amd.profiling --bank-pin      (the LDS tile's bank counts)
    python -m layout_permuting_copy_amd.profiling --wave-permute  (the device wave permute's)

runs, as child processes (this process never touches the GPU):

* the kernel trace of the benchmark command
  ``rocprofv3 --kernel-trace --stats --output-format csv ... -- python3 bench.py --no-sweep --no-cpu``
  -> ``kernel_trace_<workload>.md`` (rocprofv3's average kernel duration next to the benchmark's own
  HIP-event figure);
* one counter pass per group and workload
  ``rocprofv3 --pmc <group> --kernel-trace --output-format csv ... -- python3 bench.py --only <w>``:
  FETCH_SIZE; WRITE_SIZE; SQ_LDS_BANK_CONFLICT + SQ_INSTS_LDS; TCC_HIT_sum + TCC_MISS_sum.
  A device-to-device hipMemcpy of 1 GiB (read once, written once; the runtime's own copy kernel)
  calibrates FETCH_SIZE and WRITE_SIZE: each counter is scaled by (known bytes / what it reads for
  that copy).  The library's identity copy of the same size is recorded beside it as a check.
  -> ``counters_<workload>.md`` and ``traffic.json`` (HBM bytes per launch, with a hash of the kernel
  sources: a summary taken on other sources is not used);
* with --bank-pin, SQ_LDS_BANK_CONFLICT and SQ_INSTS_LDS per dispatch of the LDS transpose tile on
  exactly tiled copies, with the swizzle switched off, forced to candidates the search passes over
  (the tuning override's xk/xs/xt/xcs/xcm keys), or as chosen -> ``bank_pin_transpose_tiles.json``
  and ``counters_bank_pin_transpose_tiles.md``; a CPU test compares every count with the oracle's
  simulation of the tile.
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
CALIBRATION = "memcpy_dtod_1024MiB"      # hipMemcpy device to device, 1 GiB
IDENTITY = "identity_268435456_float32"  # the library's own 1 GiB copy (a check of the calibration)
CALIBRATION_BYTES = 1 << 30  # read and written once each
GROUPS = {"fetch": ["FETCH_SIZE"], "write": ["WRITE_SIZE"], "lds": ["SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"],
          "tcc": ["TCC_HIT_sum", "TCC_MISS_sum"]}
WORKLOADS = ["sf_transpose_65536x2x1x4x32_f32", "transpose_16384x16384_float32", "transpose_16384x16384_bfloat16",
             "transpose_8192x8192_int8", "transpose_8192x8192_float16", "transpose_8192x8192_float64",
             "transpose_8192x8192_int4vec", "transpose_8191x8190_float16", "transpose_8191x8190_int8",
             "transpose_8191x8190_float64", "transpose_8191x8190_int4vec",
             "slice_8192x8192[1:8191:1,0:8190:2]_int8", "slice_8192x8192[1:8191:1,0:8190:2]_float16",
             "slice_8192x8192[1:8191:1,0:8190:2]_float64", "slice_8192x8192[1:8191:1,0:8190:2]_int4vec",
             "slice_rows_8192x8192[1:8191:1,0:8190:2]_int8", "slice_rows_8192x8192[1:8191:1,0:8190:2]_float16",
             "slice_rows_8192x8192[1:8191:1,0:8190:2]_float64",
             "permute0213_32x32x2048x128_bfloat16", IDENTITY, CALIBRATION]


def kernel_source_hash(paths=None) -> str:
    h = hashlib.sha256()
    for path in paths or [os.path.join(CSRC, name) for name in KERNEL_SOURCES]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the device primitives and their example kernels (the wave permute's counters)
DEV_SOURCES = (os.path.join(ROOT, "include", "tile_copy_dev.hpp"), os.path.join(CSRC, "dev_examples.hip"))


def _run(cmd, log, timeout, env=None):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(timeout)] + cmd, stdout=f, stderr=subprocess.STDOUT,
                           cwd=ROOT, env=env)
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
    (default: the library's tc:: kernels; a tuple matches any of its strings)."""
    rows = _csv(os.path.join(glob.escape(raw_dir), "**", "*counter_collection.csv"))
    per = defaultdict(lambda: defaultdict(float))
    name = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        name[d] = r["Kernel_Name"]
    out = defaultdict(lambda: defaultdict(list))
    for d, cs in per.items():
        if not any(m in name[d] for m in ((match,) if isinstance(match, str) else match)):
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


def _kernel_trace(raw: str, out: str, py: str) -> None:
    """Kernel trace of the benchmark command -> kernel_trace_<workload>.md."""
    tdir = os.path.join(raw, "trace")
    bench_cmd = [py, "bench.py", "--no-sweep", "--no-cpu", "--steps", "100", "--warmup", "10"]
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", tdir, "-o", "bench", "--"] + bench_cmd
    log = _run(cmd, os.path.join(raw, "trace.log"), 600)
    line = next(l for l in log.splitlines() if l.startswith('{"metric"'))
    bench = json.loads(line)
    stats = _csv(os.path.join(glob.escape(tdir), "**", "*kernel_stats.csv"))
    wl = bench["config"]["workload"]
    roof = bench["roofline"]
    md = [f"# Kernel trace: {wl} (benchmark command)", "",
          "Command (repo root, library built):", "```", " ".join(cmd).replace(tdir, "<raw>/trace"), "```", "",
          f"Benchmark line: value {bench['value']} GB/s; average launch duration (HIP events around the "
          f"timed region / launches) {roof['region_us_per_launch']} us -> "
          f"{roof['achieved']} GB/s = {100 * roof['frac']:.1f}% of 8 TB/s.", "",
          "| kernel | calls | average (us) | total (us) | % |", "|---|---|---|---|---|"]
    for r in stats:
        avg_ns = float(r.get("AverageNs") or float(r["TotalDurationNs"]) / max(1, int(r["Calls"])))
        md.append(f"| `{short_kernel(r['Name'])[:90]}` | {r['Calls']} | {avg_ns / 1e3:.3f} | "
                  f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    tc_rows = [r for r in stats if "tc::" in r["Name"]]
    if tc_rows:
        avg = float(tc_rows[0].get("AverageNs") or float(tc_rows[0]["TotalDurationNs"]) / int(tc_rows[0]["Calls"])) / 1e3
        alg = roof["algorithmic_bytes_per_launch"]
        md += ["", f"rocprofv3 average of the copy kernel: {avg:.3f} us -> {alg / (avg * 1e-6) / 1e9:.1f} GB/s "
                   f"({alg / (avg * 1e-6) / 1e9 / 80:.1f}% of 8 TB/s); the benchmark's HIP-event figure also "
                   f"counts the dispatch gap between back-to-back launches "
                   f"({roof['region_us_per_launch'] - avg:.2f} us per launch here)."]
    with open(os.path.join(out, f"kernel_trace_{file_stem(wl)}.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def collect(raw: str, out: str, quick: bool = False, trace: bool = True) -> None:
    os.makedirs(raw, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    py = sys.executable or "python3"
    # 1. kernel trace of the benchmark command
    if trace:
        _kernel_trace(raw, out, py)
    # 2. counter passes
    sys.path.insert(0, ROOT)
    import bench  # the workload list (no GPU work at import)
    headline = bench.headline_workload().name
    workloads = [headline, IDENTITY, CALIBRATION] if quick else WORKLOADS
    results = defaultdict(dict)
    cmds = {}
    for w in workloads:
        for g, cs in GROUPS.items():
            if w == CALIBRATION and g not in ("fetch", "write"):
                continue
            d = os.path.join(raw, f"{g}_{file_stem(w)}")
            cmd = ["rocprofv3", "--pmc", *cs, "--kernel-trace", "--output-format", "csv", "-d", d, "-o", "run", "--",
                   py, "bench.py", "--only", w, "--steps", "4", "--warmup", "1"]
            _run(cmd, d + ".log", 180)
            cmds[(g, w)] = " ".join(cmd).replace(d, f"<raw>/{g}_{file_stem(w)}")
            # the runtime's copy kernel for the hipMemcpy calibration, the library's otherwise
            match = ("copy", "Copy") if w == CALIBRATION else "tc::"
            for k, vals in counters_per_kernel(d, match=match).items():
                if "tc::" in k and w == CALIBRATION:
                    continue
                results[w].setdefault("kernel", short_kernel(k))
                for c in cs:
                    results[w][c] = vals.get(c)
    cal = results.get(CALIBRATION, {})
    if cal.get("FETCH_SIZE") and cal.get("WRITE_SIZE"):
        cal_name = CALIBRATION
    else:  # no dispatch of the runtime's copy was seen: the library's identity copy calibrates
        cal_name, cal = IDENTITY, results[IDENTITY]
    f_fetch = CALIBRATION_BYTES / (cal["FETCH_SIZE"] * 1024)
    f_write = CALIBRATION_BYTES / (cal["WRITE_SIZE"] * 1024)
    ident = results.get(IDENTITY, {})
    traffic = {"kernel_source_hash": kernel_source_hash(), "calibration": {
        "kernel": cal["kernel"], "workload": cal_name, "known_bytes_each_way": CALIBRATION_BYTES,
        "FETCH_SIZE_KiB": cal["FETCH_SIZE"], "WRITE_SIZE_KiB": cal["WRITE_SIZE"],
        "fetch_factor": f_fetch, "write_factor": f_write,
        "identity_copy_factors": ([CALIBRATION_BYTES / (ident["FETCH_SIZE"] * 1024),
                                   CALIBRATION_BYTES / (ident["WRITE_SIZE"] * 1024)]
                                  if ident.get("FETCH_SIZE") and ident.get("WRITE_SIZE") else None)},
        "workloads": {}}
    for w, r in results.items():
        if w == CALIBRATION:
            continue
        fetch = r["FETCH_SIZE"] * 1024 * f_fetch
        write = r["WRITE_SIZE"] * 1024 * f_write
        traffic["workloads"][w] = {"kernel": r["kernel"], "fetch_bytes": fetch, "write_bytes": write,
                                   "hbm_bytes_per_launch": fetch + write,
                                   "SQ_LDS_BANK_CONFLICT": r.get("SQ_LDS_BANK_CONFLICT"),
                                   "SQ_INSTS_LDS": r.get("SQ_INSTS_LDS"),
                                   "TCC_HIT_sum": r.get("TCC_HIT_sum"), "TCC_MISS_sum": r.get("TCC_MISS_sum")}
        md = [f"# Counters: {w}", "", f"Kernel: `{r['kernel']}`", "", "Commands (repo root, one pass each):", "```"]
        md += [cmds[(g, w)] for g in GROUPS if (g, w) in cmds]
        md += ["```", "", "| counter | mean per dispatch |", "|---|---|"]
        for c in sum(GROUPS.values(), []):
            md.append(f"| {c} | {r.get(c)} |")
        md += ["", f"FETCH_SIZE x {f_fetch:.3f} and WRITE_SIZE x {f_write:.3f} (calibrated on {cal_name}, "
                   f"1 GiB each way): {fetch / 2**20:.1f} MiB fetched, {write / 2**20:.1f} MiB written per launch."]
        hits, miss = r.get("TCC_HIT_sum"), r.get("TCC_MISS_sum")
        if hits is not None and miss:
            md.append(f"TCC hit rate: {100 * hits / (hits + miss):.1f}%.")
        with open(os.path.join(out, f"counters_{file_stem(w)}.md"), "w") as f:
            f.write("\n".join(md) + "\n")
    md = ["# Counters: calibration of FETCH_SIZE and WRITE_SIZE", "",
          f"Calibrating copy: {cal_name} (kernel `{cal['kernel']}`), 1 GiB read and 1 GiB written per dispatch.", "",
          "Commands (repo root, one pass each):", "```"]
    md += [cmds[(g, cal_name)] for g in ("fetch", "write") if (g, cal_name) in cmds]
    md += ["```", "", "| counter | KiB per dispatch | factor (known bytes / counter bytes) |", "|---|---|---|",
           f"| FETCH_SIZE | {cal['FETCH_SIZE']} | {f_fetch:.4f} |", f"| WRITE_SIZE | {cal['WRITE_SIZE']} | {f_write:.4f} |"]
    if traffic["calibration"]["identity_copy_factors"] and cal_name != IDENTITY:
        fi, wi = traffic["calibration"]["identity_copy_factors"]
        md += ["", f"The library's identity copy of the same size ({ident.get('kernel')}) reads the same way: "
                   f"factors {fi:.4f} and {wi:.4f}."]
    with open(os.path.join(out, "counters_calibration_memcpy_dtod_1024MiB.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(os.path.join(out, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    print(json.dumps({w: {k: v for k, v in d.items() if k != "kernel"} for w, d in traffic["workloads"].items()}))


# LDS bank-count pins of the transpose tile: (label, workload, TC_FLAG_* bits, tuning override).
# Flags 0x10 = no swizzle (k = 0 on the default plan's tile), 0x20 = the LDS tile instead of the
# register butterfly.  The override fixes the tile (tile bytes, threads, destination run, LDS unit)
# and forces swizzles (xk, xs, xt, xcs, xcm = k, shift, target bit, column shift, column mask).
_U4 = "tile=16384,threads=256,trb=256,unit=4,nt=3,order=0"
_U8 = "tile=16384,threads=256,trb=128,unit=8,nt=3,order=0"
BANK_PIN_CASES = [
    ("fp32 256x64 u16 no swizzle", "transpose_16384x16384_float32", 0x10, ""),
    ("fp32 256x64 u16 chosen", "transpose_16384x16384_float32", 0, ""),
    ("fp32 256x64 u16 k=3", "transpose_16384x16384_float32", 0, "xk=3,xs=0,xt=0,xcs=3,xcm=3"),
    ("fp32 256x64 u16 k=2", "transpose_16384x16384_float32", 0, "xk=2,xs=0,xt=0,xcs=3,xcm=3"),
    ("fp32 256x64 u16 k=1", "transpose_16384x16384_float32", 0, "xk=1,xs=0,xt=0,xcs=3,xcm=3"),
    ("fp32 256x64 u16 k=1 no column term", "transpose_16384x16384_float32", 0, "xk=1,xs=0,xt=0"),
    ("fp32 256x64 u16 k=2 shift 1 tbit 1", "transpose_16384x16384_float32", 0, "xk=2,xs=1,xt=1,xcs=3,xcm=3"),
    ("bf16 1024x64 u16 no swizzle", "transpose_16384x16384_bfloat16", 0x10, ""),
    ("bf16 1024x64 u16 k=3", "transpose_16384x16384_bfloat16", 0, "xk=3,xs=0,xt=0,xcs=3,xcm=7"),
    ("int8 512x256 u16 no swizzle", "transpose_8192x8192_int8", 0x10, ""),
    ("int8 512x256 u16 chosen", "transpose_8192x8192_int8", 0, ""),
    ("int8 512x256 u16 k=3", "transpose_8192x8192_int8", 0, "xk=3,xs=0,xt=0,xcs=4,xcm=7"),
    ("int8 512x256 u16 k=1", "transpose_8192x8192_int8", 0, "xk=1,xs=0,xt=0,xcs=4,xcm=7"),
    ("int8 512x256 u16 k=2 shift 1 tbit 1", "transpose_8192x8192_int8", 0, "xk=2,xs=1,xt=1,xcs=3,xcm=3"),
    ("fp16 256x64 u16 no swizzle", "transpose_8192x8192_float16", 0x10, ""),
    ("fp64 256x64 u16 no swizzle", "transpose_8192x8192_float64", 0x10,
     "tile=131072,threads=512,trb=2048,unit=16,order=1,nt=3"),
    ("fp64 128x128 u16 no swizzle", "transpose_8192x8192_float64", 0x10, ""),
    ("fp64 128x128 u16 chosen", "transpose_8192x8192_float64", 0, ""),
    ("fp64 128x128 u16 k=3", "transpose_8192x8192_float64", 0, "xk=3,xs=0,xt=0,xcs=3,xcm=1"),
    ("fp64 128x128 u16 k=2", "transpose_8192x8192_float64", 0, "xk=2,xs=0,xt=0,xcs=3,xcm=1"),
    ("fp64 128x128 u16 k=1", "transpose_8192x8192_float64", 0, "xk=1,xs=0,xt=0,xcs=3,xcm=1"),
    ("16-byte 64x8 u16 no swizzle", "transpose_8192x8192_int4vec", 0x10, ""),
    ("SF 4x32x16 u4 LDS tile", "sf_transpose_65536x2x1x4x32_f32", 0x20, ""),
    ("fp32 64x64 u4 no swizzle", "transpose_16384x16384_float32", 0x10, _U4),
    ("bf16 128x64 u4 no swizzle", "transpose_16384x16384_bfloat16", 0x10, _U4),
    ("int8 128x128 u4 no swizzle", "transpose_8192x8192_int8", 0x10, _U4),
    ("int8 128x128 u4 k=1", "transpose_8192x8192_int8", 0, _U4 + ",xk=1,xs=2,xt=0,xcs=3,xcm=3"),
    ("int8 128x128 u4 k=2", "transpose_8192x8192_int8", 0, _U4 + ",xk=2,xs=2,xt=0,xcs=3,xcm=3"),
    ("int8 128x128 u4 chosen", "transpose_8192x8192_int8", 0, _U4),
    ("fp32 32x128 u8 no swizzle", "transpose_16384x16384_float32", 0x10, _U8),
    ("fp64 16x128 u8 no swizzle", "transpose_8192x8192_float64", 0x10, _U8),
]


def collect_bank_pin(raw: str, out: str, cases=None) -> None:
    """SQ_LDS_BANK_CONFLICT and SQ_INSTS_LDS per dispatch of the transpose tile kernel, one counter
    pass per case, with the tile and swizzle each dispatch ran -> bank_pin_transpose_tiles.json and
    counters_bank_pin_transpose_tiles.md."""
    os.makedirs(raw, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    py = sys.executable or "python3"
    rows = []
    for i, (label, w, flags, tune) in enumerate(cases or BANK_PIN_CASES):
        d = os.path.join(raw, f"bank_{i:02d}")
        env = dict(os.environ)
        env.pop("TC_TUNE", None)
        if tune:
            env["TC_TUNE"] = tune
        cmd = ["rocprofv3", "--pmc", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "--kernel-trace", "--output-format", "csv",
               "-d", d, "-o", "run", "--", py, "bench.py", "--only", w, "--flags", str(flags), "--steps", "2",
               "--warmup", "1"]
        log = _run(cmd, d + ".log", 180, env=env)
        info = json.loads(next(l for l in log.splitlines() if l.startswith('{"workload"')))
        cnt = counters_per_kernel(d)
        assert len(cnt) == 1, f"{label}: expected one tile-copy kernel, got {list(cnt)}"
        kname, vals = next(iter(cnt.items()))
        tr, tcol, nb = info["tile"]
        rows.append({"label": label, "workload": w, "flags": flags, "tuning": tune, "kernel": short_kernel(kname),
                     "elem_bytes": info["elem_bytes"], "vec_bytes": info["vec_bytes"], "tile": [tr, tcol, nb],
                     "threads": info["threads"], "lds_unit_bytes": info["lds_read_bytes"],
                     "lds_write_bytes": info["lds_write_bytes"], "xor": info["xor"],
                     "tiles": info["elements"] // (tr * tcol * nb), "workgroups": info["workgroups"],
                     "edge_tiles": info["edge_tiles"], "planned_conflicts_per_tile": info["planned_conflicts"],
                     "SQ_LDS_BANK_CONFLICT": vals["SQ_LDS_BANK_CONFLICT"], "SQ_INSTS_LDS": vals["SQ_INSTS_LDS"],
                     "dispatches": vals["dispatches"], "sampled_parity": info["sampled_parity"],
                     "command": ("TC_TUNE=" + tune + " " if tune else "") +
                                " ".join(cmd).replace(d, f"<raw>/bank_{i:02d}")})
        print(json.dumps({k: rows[-1][k] for k in ("label", "xor", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS",
                                                    "planned_conflicts_per_tile", "tiles")}), flush=True)
    with open(os.path.join(out, "bank_pin_transpose_tiles.json"), "w") as f:
        json.dump({"kernel_source_hash": kernel_source_hash(), "cases": rows}, f, indent=1)
    md = ["# Counters: LDS bank conflicts of the transpose tile (hardware vs the bank model)", "",
          "Each row is one rocprofv3 counter pass over `bench.py --only <workload> --flags <f>` (2 timed launches "
          "after 1 warm-up, plus the planning launch), run from the repo root with the library built; "
          "`TC_TUNE` in the command is the environment of that run.  Counts are means per dispatch of the "
          "tile-copy kernel.  The oracle's simulation of each tile (per tile, times the tiles) is compared with "
          "them by a CPU test.", "",
          "| case | kernel | tile (R x C x B) | threads | unit B | xor (k, shift, tbit, cshift, cmask) | tiles | "
          "SQ_LDS_BANK_CONFLICT | per tile | SQ_INSTS_LDS | parity |",
          "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {r['label']} | `{r['kernel']}` | {'x'.join(map(str, r['tile']))} | {r['threads']} | "
                  f"{r['lds_unit_bytes']} | {tuple(r['xor'])} | {r['tiles']} | {r['SQ_LDS_BANK_CONFLICT']:.0f} | "
                  f"{r['SQ_LDS_BANK_CONFLICT'] / r['tiles']:.2f} | {r['SQ_INSTS_LDS']:.0f} | {r['sampled_parity']} |")
    md += ["", "Commands:", "```"] + [r["command"] for r in rows] + ["```"]
    with open(os.path.join(out, "counters_bank_pin_transpose_tiles.md"), "w") as f:
        f.write("\n".join(md) + "\n")


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
    ap.add_argument("--bank-pin", action="store_true", help="only the transpose tile's LDS bank counts")
    ap.add_argument("--no-trace", action="store_true", help="counter passes only (no kernel trace)")
    args = ap.parse_args()
    if args.wave_permute:
        collect_wave_permute(args.raw, args.out)
    elif args.bank_pin:
        collect_bank_pin(args.raw, args.out)
    else:
        collect(args.raw, args.out, args.quick, trace=not args.no_trace)
    return 0


if __name__ == "__main__":
    sys.exit(main())
