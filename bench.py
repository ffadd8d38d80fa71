#!/usr/bin/env python3
"""Benchmark of the layout-permuting tile copy on one MI355X.

A step is one tile_copy of the largest workload that fits one GPU: the dense transpose of a
16384 x 16384 float32 matrix, source strides (16384, 1) -> destination strides (1, 16384), 2 GiB
moved -- every step runs the whole hot path (layout algebra and plan lookup, [outer, threads, vec]
partition, swizzled LDS tile kernel).  The inputs are resident in HBM before timing starts;
successive steps rotate over two source/destination pairs (4 GiB touched between reuses of a pair,
so the 256 MB MALL cannot serve them).

Prints one JSON line: throughput as achieved HBM GB/s (algorithmic bytes read + written per
second of wall clock over the timed steps), the roofline of the kernel (average launch duration:
HIP events on the launch stream around the timed region, divided by the launches; against
8 TB/s), the oracle's CPU throughput on a bounded sample of the same workload, and a compact sweep
of the other workloads (same metric, context only: one short record each).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth_inputs as SI  # noqa: E402

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD specification
METRIC = "achieved HBM GB/s (read+write) and % of peak for layout-permuting tile copy"
MALL_BYTES = 256 << 20


def traffic_from_profiles(workload: str, launches_bytes: int):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    entry = doc.get("workloads", {}).get(workload)
    from layout_permuting_copy_amd.profiling import kernel_source_hash
    if not entry or doc.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def device_tensors(torch, w: SI.Workload, pairs: int, host_src: np.ndarray | None, seed: int):
    n_src = SI.storage_elems(w, "src") * w.eb
    n_dst = SI.storage_elems(w, "dst") * w.eb
    srcs, dsts = [], []
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for i in range(pairs):
        if host_src is not None:
            s = torch.from_numpy(host_src).to("cuda")
        else:  # bench-only inputs for the sweep: random bits made on the device
            s = torch.empty(n_src, dtype=torch.uint8, device="cuda")
            s.random_(0, 256, generator=g)
        srcs.append(s)
        dsts.append(torch.empty(n_dst, dtype=torch.uint8, device="cuda"))
    return srcs, dsts


def time_workload(torch, L, w: SI.Workload, steps: int, warmup: int, host_src=None, seed=0, flags: int = 0):
    """Returns dict with wall ms/step and mean per-launch event ms.  `flags` (TC_FLAG_*) apply to
    every launch of the measurement."""
    prev = L.tc_set_flags(flags)
    try:
        out = _time_workload(torch, L, w, steps, warmup, host_src, seed, flags)
    finally:
        L.tc_set_flags(prev)
    if flags:
        out["flags"] = flags
    return out


def _time_workload(torch, L, w: SI.Workload, steps: int, warmup: int, host_src, seed, flags):
    bytes_step = 2 * int(np.prod(w.src.shape)) * w.eb
    pair_bytes = (SI.storage_elems(w, "src") + SI.storage_elems(w, "dst")) * w.eb
    # rotate so that more than 2x the MALL is touched between reuses of a pair (cap: 8 GiB)
    pairs = max(2, -(-2 * MALL_BYTES // pair_bytes) + 1)
    pairs = max(1, min(pairs, (8 << 30) // pair_bytes, 64))  # (tiny copies: latency, not bandwidth)
    srcs, dsts = device_tensors(torch, w, pairs, host_src, seed)
    # marshalled once, as a caller issuing the same copy repeatedly would
    sl = L.make_layout(w.src.shape, w.src.stride, w.src.offset)
    dl = L.make_layout(w.dst.shape, w.dst.stride, w.dst.offset)
    sp = [int(t.data_ptr()) for t in srcs]
    dp = [int(t.data_ptr()) for t in dsts]
    code = L.DTYPE_BY_NAME[w.dtype]
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)
    plan = L.tile_copy_ex(sp[0], sl, dp[0], dl, code, sh, flags=flags)
    for i in range(warmup):
        L.tile_copy(sp[i % pairs], sl, dp[i % pairs], dl, code, sh)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    # timed region 1: back-to-back launches; wall clock and one event pair around all of them
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(steps):
        L.tile_copy(sp[i % pairs], sl, dp[i % pairs], dl, code, sh)
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = region[0].elapsed_time(region[1])
    # timed region 2: an event pair around every launch (distribution; includes dispatch gaps)
    for i in range(steps):
        ev[i][0].record(stream)
        L.tile_copy(sp[i % pairs], sl, dp[i % pairs], dl, code, sh)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in ev]
    out = {"workload": w.name, "path": plan["path_name"], "elem_bytes": w.eb, "elements": int(np.prod(w.src.shape)),
           "bytes_per_step": bytes_step, "ms_per_step": wall * 1e3 / steps,
           "region_ms_per_launch": region_ms / steps, "event_pair_ms_mean": float(np.mean(kms)),
           "event_pair_ms_median": float(np.median(kms)),
           "event_pair_ms_min": float(np.min(kms)), "rotating_pairs": pairs,
           "tile": [plan["tile_r"], plan["tile_c"], plan["tile_b"]], "threads": plan["threads"],
           "vec_bytes": plan["vec_bytes"], "lds_write_bytes": plan["lds_write_bytes"],
           "lds_read_bytes": plan["lds_read_bytes"],
           "xor": [plan["xor_k"], plan["xor_shift"], plan["xor_tbit"], plan["xor_cshift"], plan["xor_cmask"]],
           "planned_conflicts": [plan["write_conflicts"], plan["read_conflicts"]],
           "edge_tiles": plan["edge_tiles"], "grid_order": plan["grid_order"],
           "workgroups": plan["workgroups"]}
    out["gbs_wall"] = bytes_step / (out["ms_per_step"] * 1e-3) / 1e9
    out["gbs_region"] = bytes_step / (out["region_ms_per_launch"] * 1e-3) / 1e9
    out["gbs_event_pair_median"] = bytes_step / (out["event_pair_ms_median"] * 1e-3) / 1e9
    out["pct_peak_region"] = 100 * out["gbs_region"] / PEAK_HBM_GBS
    out["us_per_launch"] = out["region_ms_per_launch"] * 1e3
    # sampled parity of the last destination written against the oracle's offsets
    out["_last"] = (srcs[(steps - 1) % pairs], dsts[(steps - 1) % pairs])
    del srcs, dsts
    return out


def sampled_parity(torch, w: SI.Workload, src_d, dst_d, n: int = 1 << 16) -> bool:
    from oracle import ref as R
    count = int(np.prod(w.src.shape))
    rng = np.random.default_rng(7)
    flat = np.unique(np.concatenate([rng.integers(0, count, n), [0, count - 1]]))
    so, do = R.sample_offsets((w.src.shape, w.src.stride, w.src.offset), (w.dst.shape, w.dst.stride, w.dst.offset),
                              flat)
    eb = w.eb
    s = src_d.view(-1, eb) if eb > 1 else src_d.view(-1, 1)
    d = dst_d.view(-1, eb) if eb > 1 else dst_d.view(-1, 1)
    a = s[torch.from_numpy(so).to("cuda")].cpu().numpy()
    b = d[torch.from_numpy(do).to("cuda")].cpu().numpy()
    return bool(np.array_equal(a, b))


def cpu_baseline(w: SI.Workload, host_src: np.ndarray, budget_s: float = 12.0):
    """The oracle (C, OpenMP) on a bounded sample of the workload: the first `tiles` tiles of
    the outermost mode, repeated for about budget_s seconds."""
    from oracle import ref as R
    outer = w.src.shape[0]
    tiles = max(1, outer // 8)
    shape = (tiles,) + tuple(w.src.shape[1:])
    sl = (shape, w.src.stride, w.src.offset)
    dl = (shape, w.dst.stride, w.dst.offset)
    n_dst = SI.span(SI.Side(shape, w.dst.stride, w.dst.offset))
    dst = np.empty(n_dst * w.eb, dtype=np.uint8)
    src = host_src[: SI.span(SI.Side(shape, w.src.stride, w.src.offset)) * w.eb].copy()
    bytes_rep = 2 * int(np.prod(shape)) * w.eb

    def rate(nthreads, seconds):
        R.copy(src, sl, dst, dl, w.eb, nthreads=nthreads)  # warm-up
        reps, t0 = 0, time.perf_counter()
        while True:
            R.copy(src, sl, dst, dl, w.eb, nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el > seconds:
                return bytes_rep * reps / el / 1e9, reps, el

    cores = R.max_threads()
    value, reps, el = rate(cores, budget_s)
    one, reps1, el1 = rate(1, budget_s / 3)
    return {"value": value, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "value_1core": round(one, 3),
            "sample": f"{tiles} of {outer} outer tiles ({bytes_rep / 2**20:.1f} MiB moved per copy), "
                      f"{reps} copies in {el:.1f} s on {cores} threads, {reps1} in {el1:.1f} s on 1"}


def time_memcpy(torch, nbytes: int = 1 << 30, steps: int = 30):
    """Context row: device-to-device hipMemcpy (torch copy_ of contiguous bytes), 2 buffer pairs."""
    a = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    b = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for i in range(3):
        b[i % 2].copy_(a[i % 2])
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        b[i % 2].copy_(a[i % 2])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([x.elapsed_time(y) for x, y in ev]))
    del a, b
    return {"workload": f"memcpy_dtod_{nbytes >> 20}MiB", "path": "hipMemcpy (context)", "bytes_per_step": 2 * nbytes,
            "event_pair_ms_mean": ms, "gbs_region": 2 * nbytes / (ms * 1e-3) / 1e9,
            "pct_peak_region": 100 * 2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def time_device_permute(torch, tiles: int = 65536, steps: int = 30, seed: int = 21):
    """Context row: the SF transpose done with the device primitives instead (tcd::g2s,
    tcd::wave_permute in place, tcd::s2g; one wave per 4x32 block pair), rotating buffer pairs;
    a sample of its tiles is checked against the oracle."""
    import layout_permuting_copy_amd as L
    import layout_permuting_copy_amd.dev as D
    from oracle import ref as R
    sl, dl = ((2, 1, 4, 32), (128, 128, 32, 1)), ((2, 1, 4, 32), (128, 128, 1, 4))
    plan = L.tc_wave_permute_plan(sl, dl, L.TC_F32, raise_on_error=False)  # declines: the cheapest (k, shift)
    k, shift = plan["k"], plan["shift"]
    nbytes = tiles * 1024
    pairs = max(2, -(-2 * MALL_BYTES // (2 * nbytes)) + 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    srcs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 256, generator=g) for _ in range(pairs)]
    dsts = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(pairs)]
    stream = torch.cuda.current_stream()
    for i in range(3):
        D.permute_tiles(srcs[i % pairs], dsts[i % pairs], tiles, 0, k, shift, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        D.permute_tiles(srcs[i % pairs], dsts[i % pairs], tiles, 0, k, shift, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    last = (steps - 1) % pairs
    rng = np.random.default_rng(seed)
    ok = True
    for t in sorted(set(int(x) for x in rng.integers(0, tiles, 64)) | {0, tiles - 1}):
        src_t = srcs[last][t * 1024:(t + 1) * 1024].cpu().numpy()
        want = src_t.copy()
        R.copy(src_t, R.layout(*sl), want, R.layout(*dl), 4)
        ok = ok and bool(np.array_equal(dsts[last][t * 1024:(t + 1) * 1024].cpu().numpy(), want))
    del srcs, dsts
    return {"workload": "sf_transpose_65536x2x1x4x32_f32 via device primitives", "path": "tcd::wave_permute (context)",
            "k": k, "shift": shift, "bytes_per_step": 2 * nbytes, "region_ms_per_launch": ms,
            "gbs_region": 2 * nbytes / (ms * 1e-3) / 1e9, "pct_peak_region": 100 * 2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "sampled_parity": ok}


def time_tile_stream(torch, mode: int, steps: int = 30, seed: int = 23):
    """Context row for the device primitives' staging step: 64 x 64 bf16 tiles of a 16384 x 16384
    matrix, g2s into an LDS tile and s2g back in place, one workgroup of 256 lanes per tile (mode 0
    plain LDS tile, 1 XOR-swizzled tile with the recognised rounds lowered to adds, 2 the swizzled
    tile with the swizzle applied every round); rotating buffer pairs; a sample of the result is
    checked against the source (a copy in place is the identity on the tiles)."""
    import layout_permuting_copy_amd.dev as D
    n = 16384
    nbytes = n * n * 2
    pairs = 2
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    srcs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 256, generator=g) for _ in range(pairs)]
    dsts = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(pairs)]
    stream = torch.cuda.current_stream()
    for i in range(3):
        D.tile_stream(srcs[i % pairs], dsts[i % pairs], n // 64, n // 64, mode, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        D.tile_stream(srcs[i % pairs], dsts[i % pairs], n // 64, n // 64, mode, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    last = (steps - 1) % pairs
    idx = torch.from_numpy(np.random.default_rng(seed).integers(0, nbytes, 1 << 16)).to("cuda")
    ok = bool(torch.equal(srcs[last][idx], dsts[last][idx]))
    del srcs, dsts
    names = {0: "plain LDS tile", 1: "swizzled tile, recognised rounds", 2: "swizzled tile, general rounds"}
    return {"workload": f"tcd g2s/s2g 64x64 bf16 tiles of 16384^2: {names[mode]}", "path": "device primitives",
            "bytes_per_step": 2 * nbytes, "region_ms_per_launch": ms, "gbs_region": 2 * nbytes / (ms * 1e-3) / 1e9,
            "pct_peak_region": 100 * 2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "sampled_parity": ok}


def device_props(torch) -> dict:
    """The GPU the line was measured on (name, architecture, compute units, memory)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2 ** 30, 1)}


def identity_workload(n: int = 1 << 28) -> SI.Workload:
    return SI.Workload(f"identity_{n}_float32", SI.Side((n,), (1,)), SI.Side((n,), (1,)), "float32", "bits", 12)


def sweep_workloads():
    ws = [SI.sf_transpose(), SI.transpose2d(dtype="bfloat16"), SI.permute0213()]
    ws += [SI.sweep_dense(dt) for dt in SI.SWEEP_DTYPES]
    ws += [SI.sweep_odd(dt) for dt in SI.SWEEP_DTYPES]
    ws += [SI.sweep_slice(dt) for dt in SI.SWEEP_DTYPES]
    ws += [SI.sweep_slice_rows(dt) for dt in SI.SWEEP_DTYPES]
    ws += [SI.a2a_pack_permute0213(), SI.a2a_unpack_permute0213()]
    return ws


def headline_workload() -> SI.Workload:
    """The largest single-GPU configuration: the 16384 x 16384 float32 transpose (2 GiB moved)."""
    return SI.transpose2d(dtype="float32")


def compact(r: dict) -> dict:
    """One short sweep record: workload, path, flags, GB/s and % of peak over the timed region of
    back-to-back launches, and the sampled parity."""
    out = {"w": r["workload"], "path": r.get("path")}
    if r.get("flags"):
        out["flags"] = r["flags"]
    out["GBs"] = round(r["gbs_region"], 1)
    out["pct"] = round(r["pct_peak_region"], 2)
    if "sampled_parity" in r:
        out["ok"] = r["sampled_parity"]
    for k in ("us_per_launch", "k", "shift"):
        if k in r and (k != "us_per_launch" or r["bytes_per_step"] < (1 << 20)):
            out[k] = round(r[k], 3) if isinstance(r[k], float) else r[k]
    return out


def run_only(torch, L, name: str, flags: int, steps: int, warmup: int) -> dict:
    """One workload alone (profiling runs): its timing, plan and sampled parity."""
    if name.startswith("memcpy_dtod"):
        return time_memcpy(torch, steps=steps)
    w = next(w for w in [headline_workload(), identity_workload()] + sweep_workloads() if w.name == name)
    r = time_workload(torch, L, w, steps, warmup, seed=11, flags=flags)
    s_src, s_dst = r.pop("_last")
    r["sampled_parity"] = sampled_parity(torch, w, s_src, s_dst, 1 << 14)
    return r


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-sweep", action="store_true", help="skip the per-workload context sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", default=None, help="time only the named workload (profiling runs)")
    ap.add_argument("--flags", type=int, default=0, help="TC_FLAG_* bits for --only")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the copy has no multi-GPU path "
                                   "(--gpus must be 1)"}))
        return 2
    for k in ("RANK", "WORLD_SIZE"):
        if int(os.environ.get(k, "0" if k == "RANK" else "1")) != (0 if k == "RANK" else 1):
            print(json.dumps({"error": "run on one GPU without torch.distributed"}))
            return 2
    import torch
    import layout_permuting_copy_amd as L
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        return 2
    L.load_library()
    if args.only:
        r = run_only(torch, L, args.only, args.flags, args.steps, args.warmup)
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}), flush=True)
        return 0 if r.get("sampled_parity", True) else 1

    w = headline_workload()
    host_src = SI.make_source(w)
    r = time_workload(torch, L, w, args.steps, args.warmup, host_src=host_src)
    src_d, dst_d = r.pop("_last")
    parity = sampled_parity(torch, w, src_d, dst_d)
    del src_d, dst_d
    torch.cuda.empty_cache()
    sweep = []
    if not args.no_sweep:
        sweep.append(compact(time_memcpy(torch)))
        torch.cuda.empty_cache()
        sweep.append(compact(time_device_permute(torch)))
        torch.cuda.empty_cache()
        for mode in (0, 1, 2):
            sweep.append(compact(time_tile_stream(torch, mode)))
            torch.cuda.empty_cache()
        # context first (the 32 x 32 round trip by one wave is a latency case: see its
        # us_per_launch; the odd and sliced copies; the alternatives the planner does not pick: the
        # SF tiles on the LDS tile kernel, the (0,2,1,3) permute staged through LDS), then the
        # configurations with the 80% target, last so that they end the line
        target = [SI.sf_transpose(), SI.transpose2d(dtype="bfloat16"), SI.permute0213()]
        target += [SI.sweep_dense(dt) for dt in SI.SWEEP_DTYPES]
        context = [SI.tile32_roundtrip(), identity_workload()]
        context += [SI.sweep_odd(dt) for dt in SI.SWEEP_DTYPES] + [SI.sweep_slice(dt) for dt in SI.SWEEP_DTYPES]
        context += [SI.sweep_slice_rows(dt) for dt in SI.SWEEP_DTYPES]
        context += [SI.a2a_pack_permute0213(), SI.a2a_unpack_permute0213()]  # one GPU's share, 8 GPUs
        runs = [(sw, 0) for sw in context]
        runs += [(SI.sf_transpose(), L.TC_FLAG_NO_SHUFFLE), (SI.permute0213(), L.TC_FLAG_FORCE_LDS)]
        runs += [(sw, 0) for sw in target]
        for sw, fl in runs:
            s = time_workload(torch, L, sw, 30, 3, seed=11, flags=fl)
            s_src, s_dst = s.pop("_last")
            s["sampled_parity"] = sampled_parity(torch, sw, s_src, s_dst, 1 << 14)
            del s_src, s_dst
            torch.cuda.empty_cache()
            sweep.append(compact(s))
    traffic = traffic_from_profiles(w.name, r["bytes_per_step"])
    achieved = r["gbs_region"]
    line = {
        "metric": METRIC,
        "value": round(r["gbs_wall"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": w.name, "shape": list(w.src.shape), "src_stride": list(w.src.stride),
                   "dst_stride": list(w.dst.stride), "element": "float32 moved as raw 32-bit words",
                   "bytes_per_step": r["bytes_per_step"], "path": r["path"], "tile": r["tile"],
                   "threads": r["threads"], "vec_bytes": r["vec_bytes"], "xor": r["xor"],
                   "workgroups": r["workgroups"], "rotating_buffer_pairs": r["rotating_pairs"],
                   "sampled_parity": parity, "pct_of_peak_wall": round(100 * r["gbs_wall"] / PEAK_HBM_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "region_us_per_launch": round(r["region_ms_per_launch"] * 1e3, 3),
                     "event_pair_us_median": round(r["event_pair_ms_median"] * 1e3, 3),
                     "timing": "HIP events on the launch stream around the timed region of back-to-back "
                               "launches, divided by the launches",
                     "algorithmic_bytes_per_launch": r["bytes_per_step"]},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, host_src)
        line["cpu_baseline"]["value"] = round(line["cpu_baseline"]["value"], 3)
    line["device"] = device_props(torch)
    if sweep:
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
