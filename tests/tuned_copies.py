"""Child process of tests/test_gpu_tuning.py: copies planned under the tuning override given in
the environment (TC_TUNE, read once per process), each checked byte for byte against the oracle.
Prints one line per case and exits non-zero on the first mismatch."""

import json
import sys

import numpy as np

import layout_permuting_copy_amd as L
from gpu_util import assert_same, oracle_copy, run_copy, say

DT = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}


def span(shape, stride, off):
    return off + sum((e - 1) * s for e, s in zip(shape, stride) if s > 0) + 1


def main() -> int:
    import torch
    assert torch.cuda.is_available()
    L.load_library()
    cases = json.loads(sys.argv[1])
    for shape, ss, so, ds, do, eb, flags, seed, want in cases:
        shape, ss, ds = tuple(shape), tuple(ss), tuple(ds)
        src = np.frombuffer(np.random.default_rng(seed).bytes(span(shape, ss, so) * eb), dtype=np.uint8).copy()
        n_dst = span(shape, ds, do)
        say(f"[tuned] shape={shape} src={ss}+{so} dst={ds}+{do} eb={eb} flags={flags}")
        got, plan = run_copy(src, (shape, ss, so), n_dst, (shape, ds, do), eb, DT[eb], flags)
        assert_same(got, oracle_copy(src, (shape, ss, so), n_dst, (shape, ds, do), eb), eb, str(shape))
        for k, v in want.items():
            assert plan[k] == v, (k, plan[k], v, plan)
        print(json.dumps({"shape": shape, "eb": eb, "tile": [plan["tile_r"], plan["tile_c"], plan["tile_b"]],
                          "xor": [plan["xor_k"], plan["xor_shift"], plan["xor_tbit"], plan["xor_cshift"],
                                  plan["xor_cmask"]], "order": plan["grid_order"], "ok": True}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
