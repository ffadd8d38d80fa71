"""ctypes binding of libtile_copy_dev.so: example kernels built on the device primitives of
include/tile_copy_dev.hpp (argument marshalling only; every step runs in the HIP kernels)."""

from __future__ import annotations

import ctypes
import os

from . import _ptr, _stream

DEV_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtile_copy_dev.so")
_dev = None


def load_dev_library(path: str = DEV_LIB_PATH):
    """Loads libtile_copy_dev.so; raises if it has not been built."""
    global _dev
    if _dev is not None:
        return _dev
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python layout_permuting_copy_amd/build.py`")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name, args in [("tcd_ex_roundtrip32", [vp, vp, vp]), ("tcd_ex_permute_tiles", [vp, vp, i, i, i, i, vp]),
                       ("tcd_ex_swizzled_transpose", [vp, vp, vp, i, i, vp]), ("tcd_ex_lane_copy", [vp, vp, vp]),
                       ("tcd_ex_waves2_copy", [vp, vp, vp]), ("tcd_ex_plan", [i, ctypes.POINTER(ctypes.c_int)]),
                       ("tcd_ex_tile_stream", [vp, vp, i, i, i, vp])]:
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = ctypes.c_int
    _dev = lib
    return lib


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: HIP error {rc}")


def roundtrip32(src, dst, stream=None) -> None:
    _ok(load_dev_library().tcd_ex_roundtrip32(_ptr(src), _ptr(dst), _stream(stream)), "tcd_ex_roundtrip32")


def permute_tiles(src, dst, ntiles: int, which: int, k: int, shift: int, stream=None) -> None:
    _ok(load_dev_library().tcd_ex_permute_tiles(_ptr(src), _ptr(dst), int(ntiles), int(which), int(k), int(shift),
                                                _stream(stream)), "tcd_ex_permute_tiles")


def swizzled_transpose(src, dst, lds_dump, tiles_r: int, tiles_c: int, stream=None) -> None:
    _ok(load_dev_library().tcd_ex_swizzled_transpose(_ptr(src), _ptr(dst), _ptr(lds_dump), int(tiles_r), int(tiles_c),
                                                     _stream(stream)), "tcd_ex_swizzled_transpose")


def lane_copy(src, dst, stream=None) -> None:
    _ok(load_dev_library().tcd_ex_lane_copy(_ptr(src), _ptr(dst), _stream(stream)), "tcd_ex_lane_copy")


def waves2_copy(src, dst, stream=None) -> None:
    _ok(load_dev_library().tcd_ex_waves2_copy(_ptr(src), _ptr(dst), _stream(stream)), "tcd_ex_waves2_copy")


def tile_stream(src, dst, tiles_r: int, tiles_c: int, mode: int, stream=None) -> None:
    """64 x 64 bf16 tiles of a pitch-16384 matrix staged through LDS and written back in place
    (mode 0 plain LDS tile, 1 swizzled with recognised rounds, 2 swizzled with the general rounds)."""
    _ok(load_dev_library().tcd_ex_tile_stream(_ptr(src), _ptr(dst), int(tiles_r), int(tiles_c), int(mode),
                                              _stream(stream)), "tcd_ex_tile_stream")


def example_plan(which: int, lowered: bool = False) -> dict:
    """(vec, outer, exact) the example's copy compiled to (see tcd_ex_plan); with lowered=True
    also whether its rounds were recognised (per-round adds)."""
    out = (ctypes.c_int * 4)()
    if load_dev_library().tcd_ex_plan(int(which), out) != 0:
        raise ValueError(f"no example plan {which}")
    d = {"vec": out[0], "outer": out[1], "exact": bool(out[2])}
    if lowered:
        d["lowered"] = bool(out[3])
    return d


def _main(argv=None) -> int:
    """python -m layout_permuting_copy_amd.dev permute --which W --k K --shift S --tiles N --reps R

    Runs the in-place wave permute example R times on N tiles of random bits (rotating buffer
    pairs, so that the MALL does not serve them) and prints one JSON line with the mean kernel time
    (HIP events on the launch stream around the back-to-back launches) and the global bytes moved."""
    import argparse
    import json

    import torch

    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["permute"])
    ap.add_argument("--which", type=int, default=1)
    ap.add_argument("--k", type=int, default=0)
    ap.add_argument("--shift", type=int, default=0)
    ap.add_argument("--tiles", type=int, default=65536)
    ap.add_argument("--reps", type=int, default=20)
    a = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        return 2
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    # rotate buffer pairs so that more than twice the 256 MB MALL is touched between reuses
    pair = 2 * a.tiles * 1024
    pairs = max(2, -(-(2 * (256 << 20)) // pair) + 1)
    srcs, dsts = [], []
    for _ in range(pairs):
        srcs.append(torch.empty(a.tiles * 1024, dtype=torch.uint8, device="cuda"))
        srcs[-1].random_(0, 256, generator=g)
        dsts.append(torch.empty_like(srcs[-1]))
    stream = torch.cuda.current_stream()
    permute_tiles(srcs[0], dsts[0], a.tiles, a.which, a.k, a.shift, stream)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(a.reps):
        permute_tiles(srcs[i % pairs], dsts[i % pairs], a.tiles, a.which, a.k, a.shift, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / a.reps
    moved = 2 * a.tiles * 1024
    print(json.dumps({"what": "wave_permute", "which": a.which, "k": a.k, "shift": a.shift, "tiles": a.tiles,
                      "kernel_us_mean": round(us, 3), "global_bytes": moved, "gbs": round(moved / (us * 1e-6) / 1e9, 1)}))
    return 0


if __name__ == "__main__":
    import sys
    sys.exit(_main())
