"""Builds the tile-copy library for gfx950, in-tree: libtile_copy.so (C ABI declared in
include/tile_copy.h) and the LDS bank probe (bin/lds_bank_probe)."""
import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtile_copy.so")
PROBE = os.path.join(PKG, "bin", "lds_bank_probe")
# example kernels of the device primitives (include/tile_copy_dev.hpp), with their own C ABI
DEV_LIB = os.path.join(PKG, "libtile_copy_dev.so")
DEV_SOURCES = ["dev_examples.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "--offload-arch=gfx950"
# packed fp32 ops are disabled for all device code
NO_PK = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# per-kernel register, scratch and occupancy figures, from the compiler's resource-usage remarks
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
REMARK = ["-Rpass-analysis=kernel-resource-usage"]
SOURCES = ["layout.cpp", "bank.cpp", "plan.cpp", "permute.cpp", "abi.cpp", "kernels.hip", "transpose_eb1.hip", "transpose_eb2.hip",
           "transpose_eb4.hip", "transpose_eb8.hip", "transpose_eb16.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _resources(remarks: str) -> dict:
    """{kernel: {"vgprs", "scratch_bytes", "occupancy"}} from kernel-resource-usage remarks."""
    out, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            key = {"VGPRs": "vgprs", "ScratchSize [bytes/lane]": "scratch_bytes", "Occupancy [waves/SIMD]": "occupancy"}
            out[name][key[m.group(1)]] = int(m.group(2))
    return out


def _compile(src, build_dir, extra):
    obj = os.path.join(build_dir, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, ARCH, *NO_PK, *COMMON, *REMARK, *extra, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *extra, "-c", path, "-o", obj]
    out = _run(cmd)
    res = _resources(out)
    # drop the remarks and the source excerpts printed under them
    rest = "\n".join(l for l in out.splitlines()
                     if "kernel-resource-usage" not in l and not l.startswith("In file included from")
                     and not re.match(r"\s*(\d+\s*)?\|", l))
    if rest.strip():
        print(rest, file=sys.stderr)
    return obj, res


def build(verbose: bool = False, extra=(), lib_path: str = LIB, with_probe: bool = True) -> str:
    """Compiles every source (in parallel) and links lib_path.  `extra` adds compiler flags,
    e.g. -DTC_ROW_ROUNDS=1 to build a tuning variant (see csrc/plan.hpp; the transpose's tile
    configuration is a plan parameter, overridable at run time with TC_TUNE)."""
    extra = list(extra)
    build_dir = BUILD if lib_path == LIB else os.path.join(os.path.dirname(os.path.abspath(lib_path)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(PROBE), exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        done = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
        objs = [o for o, _ in done]
        resources = {}
        for _, r in done:
            resources.update(r)
        with open(os.path.join(build_dir, "kernel_resources.json"), "w") as f:
            json.dump(resources, f, indent=1, sort_keys=True)
        probe = None
        if with_probe:
            probe = ex.submit(_run, [HIPCC, ARCH, *NO_PK, "-O3", "-std=c++17",
                                     os.path.join(CSRC, "probe", "lds_bank_probe.hip"), "-o", PROBE + ".tmp"])
        dev = [ex.submit(_compile, src, build_dir, extra) for src in DEV_SOURCES] if lib_path == LIB else []
        tmp = lib_path + ".tmp"
        _run([HIPCC, ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, lib_path)
        if dev:
            dev_done = [f.result() for f in dev]
            for _, r in dev_done:
                resources.update(r)
            with open(os.path.join(build_dir, "kernel_resources.json"), "w") as f:
                json.dump(resources, f, indent=1, sort_keys=True)
            _run([HIPCC, ARCH, "-shared", "-fPIC", *[o for o, _ in dev_done], "-o", DEV_LIB + ".tmp"])
            os.replace(DEV_LIB + ".tmp", DEV_LIB)
        if probe is not None:
            probe.result()
            os.replace(PROBE + ".tmp", PROBE)
    if verbose:
        print(lib_path)
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
