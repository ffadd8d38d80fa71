"""tc_autotune on the GPU: the copy is bit-exact against the oracle after tuning, the chosen plan
is one of tc_plan_variants' and becomes the cached plan later copies of the same layouts run,
and a capturing stream is refused without a launch."""

import numpy as np
import pytest

import layout_permuting_copy_amd as L
from gpu_util import assert_same, oracle_copy, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    yield
    torch.cuda.synchronize()


def _key(p):
    return tuple(p[k] for k in ("path_name", "tile_r", "tile_c", "tile_b", "threads", "grid_order", "super_rows",
                                "super_cols", "loads_in_flight", "nontemporal", "edge_tiles", "lds_write_bytes",
                                "lds_read_bytes", "load_outer", "workgroups"))


@pytest.mark.parametrize("shape,ss,so,ds,eb", [
    ((1024, 4096), (4096, 1), 0, (1, 1024), 4),        # fp32 transpose
    ((777, 1029), (1030, 1), 3, (1, 777), 1),          # odd int8 transpose at element alignment
    ((300, 257), (257 * 2, 2), 0, (1, 300), 2),        # stride-2 source
    ((1 << 22,), (1,), 0, (1,), 4),                    # contiguous rows
    ((2000, 1999), (2048, 1), 2049, (1999, 1), 1),     # a window at an odd offset (element-aligned rows)
    ((64, 96, 128), (96 * 128, 128, 1), 0, (128, 64 * 128, 1), 2),  # permuted rows
])
def test_autotune_copies_and_caches(shape, ss, so, ds, eb):
    import torch
    dt = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32}[eb]
    n_src = so + sum((e - 1) * s for e, s in zip(shape, ss) if s > 0) + 1
    n_dst = sum((e - 1) * d for e, d in zip(shape, ds) if d > 0) + 1
    src = np.frombuffer(np.random.default_rng(sum(shape)).bytes(n_src * eb), dtype=np.uint8).copy()
    sl, dl = (shape, ss, so), (shape, ds, 0)
    say(f"[gpu] autotune shape={shape} src={ss}+{so} dst={ds} eb={eb}")
    src_d = torch.from_numpy(src).cuda()
    dst_d = torch.full((n_dst * eb,), 0xA5, dtype=torch.uint8, device="cuda")
    variants = L.tc_plan_variants(sl, dl, dt)
    tuned = L.tc_autotune(src_d, sl, dst_d, dl, dt, reps=3)
    torch.cuda.synchronize()
    assert tuned["tuned_ms"] > 0
    assert _key(tuned) in {_key(v) for v in variants}, tuned
    want = oracle_copy(src, sl, n_dst, dl, eb)
    assert_same(dst_d.cpu().numpy(), want, eb, f"autotune {shape}")
    # later copies of the same layouts run the tuned plan, and are bit-exact too
    dst_d.fill_(0x5A)
    again = L.tile_copy_ex(src_d, sl, dst_d, dl, dt)
    torch.cuda.synchronize()
    assert _key(again) == _key(tuned)
    want = oracle_copy(src, sl, n_dst, dl, eb, sentinel=0x5A)
    assert_same(dst_d.cpu().numpy(), want, eb, f"after autotune {shape}")


def test_autotune_refuses_a_capturing_stream():
    import torch
    n = 512
    src_d = torch.zeros(n * n, dtype=torch.float32, device="cuda")
    dst_d = torch.zeros(n * n, dtype=torch.float32, device="cuda")
    sl, dl = ((n, n), (n, 1)), ((n, n), (1, n))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    rc = None
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            try:
                L.tc_autotune(src_d, sl, dst_d, dl, L.TC_F32, stream=s)
            except L.TileCopyError as e:
                rc, why = e.code, e.reason
    torch.cuda.synchronize()
    assert rc == L.TC_E_ARG and "capturing" in why
