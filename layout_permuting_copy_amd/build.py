"""Builds the tile-copy library for gfx950, in-tree: libtile_copy.so (C ABI declared in
include/tile_copy.h) and the LDS bank probe (bin/lds_bank_probe)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtile_copy.so")
PROBE = os.path.join(PKG, "bin", "lds_bank_probe")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "--offload-arch=gfx950"
# packed fp32 ops are disabled for all device code
NO_PK = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
SOURCES = ["layout.cpp", "bank.cpp", "plan.cpp", "abi.cpp", "kernels.hip", "transpose_eb1.hip", "transpose_eb2.hip",
           "transpose_eb4.hip", "transpose_eb8.hip", "transpose_eb16.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _compile(src, build_dir, extra):
    obj = os.path.join(build_dir, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, ARCH, *NO_PK, *COMMON, *extra, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *extra, "-c", path, "-o", obj]
    out = _run(cmd)
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, extra=(), lib_path: str = LIB, with_probe: bool = True) -> str:
    """Compiles every source (in parallel) and links lib_path.  `extra` adds compiler flags,
    e.g. -DTC_ROW_ROUNDS=1 to build a tuning variant (see csrc/plan.hpp; the transpose's tile
    configuration is a plan parameter, overridable at run time with TC_TUNE)."""
    extra = list(extra)
    build_dir = BUILD if lib_path == LIB else os.path.join(os.path.dirname(os.path.abspath(lib_path)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(PROBE), exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
        probe = None
        if with_probe:
            probe = ex.submit(_run, [HIPCC, ARCH, *NO_PK, "-O3", "-std=c++17",
                                     os.path.join(CSRC, "probe", "lds_bank_probe.hip"), "-o", PROBE + ".tmp"])
        tmp = lib_path + ".tmp"
        _run([HIPCC, ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, lib_path)
        if probe is not None:
            probe.result()
            os.replace(PROBE + ".tmp", PROBE)
    if verbose:
        print(lib_path)
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
