"""Helpers of the GPU parity tests: seeded inputs on the device, the copy through the C ABI,
and the oracle's answer on the host for comparison."""

import sys

import numpy as np

import layout_permuting_copy_amd as L
import synth_inputs as SI
from oracle import ref as R


def torch_mod():
    import torch
    return torch


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dtype_code(name: str) -> int:
    return L.DTYPE_BY_NAME[name]


def run_copy(src_host: np.ndarray, src_lay, dst_elems: int, dst_lay, eb: int, dtype: int, flags: int = 0,
             sentinel: int = 0xA5):
    """Upload src bytes, prefill dst with a sentinel, run the library copy, return (dst bytes, plan)."""
    torch = torch_mod()
    src_d = torch.from_numpy(src_host).to("cuda")
    dst_d = torch.full((dst_elems * eb,), sentinel, dtype=torch.uint8, device="cuda")
    plan = L.tile_copy_ex(src_d, src_lay, dst_d, dst_lay, dtype, flags=flags)
    torch.cuda.synchronize()
    out = dst_d.cpu().numpy()
    del src_d, dst_d
    return out, plan


def oracle_copy(src_host: np.ndarray, src_lay, dst_elems: int, dst_lay, eb: int, sentinel: int = 0xA5) -> np.ndarray:
    want = np.full(dst_elems * eb, sentinel, dtype=np.uint8)
    R.copy(src_host, src_lay, want, dst_lay, eb)
    return want


def check_workload(w: SI.Workload, flags: int = 0, expect_path=None):
    eb = w.eb
    src = SI.make_source(w)
    sl = (w.src.shape, w.src.stride, w.src.offset)
    dl = (w.dst.shape, w.dst.stride, w.dst.offset)
    n_dst = SI.storage_elems(w, "dst")
    say(f"[gpu] {w.name} eb={eb} flags={flags}")
    got, plan = run_copy(src, sl, n_dst, dl, eb, dtype_code(w.dtype), flags)
    want = oracle_copy(src, sl, n_dst, dl, eb)
    assert_same(got, want, eb, w.name)
    if expect_path is not None:
        assert plan["path_name"] == expect_path, plan
    return plan


def assert_same(got: np.ndarray, want: np.ndarray, eb: int, name: str) -> None:
    if np.array_equal(got, want):
        return
    bad = np.nonzero(got != want)[0]
    first = bad[0] // eb
    raise AssertionError(f"{name}: {bad.size} bytes differ; first element {first}: got "
                         f"{got[first * eb:(first + 1) * eb].tolist()} want {want[first * eb:(first + 1) * eb].tolist()}")
