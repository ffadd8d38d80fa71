"""Copies planned under the tuning override (TC_TUNE, read once per process): forced XOR swizzles
-- the ones the LDS bank-count pins run -- and other XCD super-tile extents give the same bytes
as the oracle.  Each setting runs in one child process (sequentially), which checks its copies
against the oracle."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# (shape, src stride, src offset, dst stride, dst offset, element bytes, flags, seed, plan fields)
SWIZZLE_CASES = [
    [[1024, 448], [448, 1], 0, [1, 1024], 0, 4, 0, 1, {"xor_k": 1, "xor_shift": 2}],
    [[1536, 320], [320, 1], 0, [1, 1536], 0, 1, 0, 2, {"xor_k": 1, "xor_shift": 2}],
    [[520, 200], [200, 1], 0, [1, 520], 0, 2, 0, 3, {"xor_k": 1, "xor_shift": 2}],
    [[640, 96], [96, 1], 0, [1, 640], 0, 8, 0, 4, {"xor_k": 1, "xor_shift": 2}],
]
SUPER_CASES = [
    [[8191, 1030], [1030, 1], 0, [1, 8191], 0, 1, 0, 5, {"grid_order": 2}],
    [[1027, 2050], [2050, 1], 3, [1, 1029], 1, 8, 0, 6, {"grid_order": 2}],
    [[3, 700, 650], [700 * 650 + 7, 650, 1], 0, [650 * 701, 1, 701], 0, 1, 0, 7, {"grid_order": 2}],
]
SETTINGS = [
    ("xk=1,xs=2,xt=0,xcs=3,xcm=3", SWIZZLE_CASES),
    ("xk=1,xs=2,xt=1", SWIZZLE_CASES),
    ("ssr=4,ssc=16", SUPER_CASES),
    ("ssr=32,ssc=2", SUPER_CASES),
    ("ssr=1,ssc=1", SUPER_CASES),
]


@pytest.mark.parametrize("tune,cases", SETTINGS, ids=[s for s, _ in SETTINGS])
def test_copies_under_tuning_override(tune, cases):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ)
    env["TC_TUNE"] = tune
    env["PYTHONPATH"] = os.pathsep.join([HERE, ROOT, env.get("PYTHONPATH", "")])
    print(f"[tuning] TC_TUNE={tune}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "tuned_copies.py"), json.dumps(cases)],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=110)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0
    assert r.stdout.count('"ok": true') == len(cases)
