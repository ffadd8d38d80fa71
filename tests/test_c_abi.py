"""The C ABI used from plain C (tests/c_abi_demo.c, built with gcc against include/tile_copy.h and
libtile_copy.so, HIP runtime for device memory): its output bytes equal the oracle's."""

import os
import subprocess
import tempfile

import numpy as np
import pytest

import layout_permuting_copy_amd as L
from conftest import ROOT
from oracle import ref as R


def _build(tmp):
    exe = os.path.join(tmp, "c_abi_demo")
    lib_dir = os.path.dirname(L.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_demo.c"),
                           "-L", lib_dir, "-ltile_copy", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath," + lib_dir,
                           "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    return exe


def test_c_program_builds_against_the_header():
    with tempfile.TemporaryDirectory() as tmp:
        assert os.access(_build(tmp), os.X_OK)


@pytest.mark.gpu
def test_c_program_copies_match_oracle():
    n, m, tiles = 256, 192, 3
    total = n * m + tiles * 256
    vals = ((np.arange(total, dtype=np.uint64) * 2654435761) % 100003).astype(np.float32) - np.float32(50000.0)
    src = vals.view(np.uint8)
    with tempfile.TemporaryDirectory() as tmp:
        exe = _build(tmp)
        out = os.path.join(tmp, "out.bin")
        r = subprocess.run([exe, out], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        got = np.fromfile(out, dtype=np.uint8)
    want = np.full(total * 4, 0xA5, dtype=np.uint8)
    R.copy(src, R.layout((n, m), (m, 1)), want, R.layout((n, m), (1, n)), 4)
    R.copy(src, R.layout((tiles, 2, 1, 4, 32), (256, 128, 128, 32, 1), n * m), want,
           R.layout((tiles, 2, 1, 4, 32), (256, 128, 128, 1, 4), n * m), 4)
    assert np.array_equal(got, want)
    assert "scale-factor plan: path 6" in r.stderr  # the register butterfly
