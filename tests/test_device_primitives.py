"""The device primitives of include/tile_copy_dev.hpp: the wave permute's host-side bank plan
(tc_wave_permute_plan) against the oracle's re-derivation, the compile-time [outer, threads, vec]
plans of the example kernels against the oracle's partition, and (GPU) every example kernel
bit-exact against the oracle."""

import os
import subprocess

import numpy as np
import pytest

import layout_permuting_copy_amd as L
from conftest import ROOT
from oracle import ref as R

DTS = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}
PERMUTE_CASES = [((2, 1, 4, 32), (128, 128, 32, 1), (128, 128, 1, 4)), ((4, 64), (64, 1), (1, 4)),
                 ((64, 4), (4, 1), (1, 64)), ((32, 32), (32, 1), (1, 32)), ((16, 64), (64, 1), (1, 16)),
                 ((8, 32), (32, 1), (1, 8)), ((64, 64), (64, 1), (1, 64)), ((2, 4, 32), (128, 32, 1), (4, 1, 8)),
                 ((128,), (1,), (1,)), ((8, 8, 4), (32, 4, 1), (1, 8, 64)), ((4, 16, 8), (128, 8, 1), (1, 32, 4))]


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_wave_permute_plan_matches_oracle(eb):
    m = R.gfx950_model()
    for shape, ss, ds in PERMUTE_CASES:
        p = L.tc_wave_permute_plan((shape, ss), (shape, ds), DTS[eb], raise_on_error=False)
        ext, s2, d2, _, _ = R.permute_shard(R.layout(shape, ss), R.layout(shape, ds))
        assert (p["extent"], p["src_stride"], p["dst_stride"]) == (ext, s2, d2)
        o = R.choose_xor_k(ext, s2, d2, eb, m)
        if o is None:
            assert p["status"] == L.TC_E_DECLINED and "conflict-free" in p["error"]
        else:
            assert p["status"] == L.TC_OK and (p["k"], p["shift"], p["mask"]) == o
        # the reported (or, when declined, cheapest) candidate's counts are the oracle's
        assert R.permute_conflicts(ext, s2, d2, eb, p["k"], p["shift"], m) == (p["read_conflicts"], p["write_conflicts"])
    bad = L.tc_wave_permute_plan(((3, 5), (5, 1)), ((3, 5), (1, 3)), DTS[eb], raise_on_error=False)
    assert bad["status"] == L.TC_E_DECLINED and "no integer P" in bad["error"]


def test_library_exports_device_examples():
    import layout_permuting_copy_amd.dev as D
    D.load_dev_library()
    out = subprocess.run(["nm", "-D", "--defined-only", D.DEV_LIB_PATH], capture_output=True, text=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {"tcd_ex_roundtrip32", "tcd_ex_permute_tiles", "tcd_ex_swizzled_transpose", "tcd_ex_lane_copy",
            "tcd_ex_waves2_copy", "tcd_ex_plan", "tcd_ex_tile_stream"} <= names
    assert "tc_wave_permute_plan" in subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                                                     text=True).stdout


def test_example_plans_match_oracle_partition():
    """The examples' compile-time plans are the gmem_smem partition the oracle derives (global
    side driving the order), except that a count not divisible by the lanes runs guarded (the
    page declines there)."""
    import layout_permuting_copy_amd.dev as D
    cases = {
        0: (R.layout((32, 32), (32, 1)), R.layout((32, 32), (32, 1)), 64, 4),
        1: (R.layout((64, 64), (192, 1)), R.layout((64, 64), (64, 1)), 256, 2),
        2: (R.layout((64, 64), (1, 192)), R.layout((64, 64), (64, 1)), 256, 2),
        3: (R.layout((3, 5, 7), (80, 9, 1)), R.layout((3, 5, 7), (1, 3, 15)), 1, 1),
    }
    for which, (g, s, threads, eb) in cases.items():
        o = R.gmem_smem_partition(g, s, threads, eb)
        p = D.example_plan(which)
        assert not o["declined"] and (p["vec"], p["outer"], p["exact"]) == (o["vec"], o["outer"], True), which
    o = R.gmem_smem_partition(R.layout((45, 40), (56, 1)), R.layout((45, 40), (40, 1)), 128, 2)
    assert o["declined"]
    assert D.example_plan(4) == {"vec": 1, "outer": 15, "exact": False}


def test_recognised_rounds_match_oracle():
    """The copy lowers a swizzled copy to per-round adds exactly where the oracle's partition shows
    that every lane's offsets on both sides (swizzle applied) are its round-0 offsets plus a
    per-round constant (TVM TIRx "copy -> gmem_smem", "How inputs change the algorithm", last
    paragraph).  Examples 1, 5, 6: global <-> the XOR-swizzled 64 x 64 bf16 tile (16-byte chunks,
    chunk ^= row % 8), rounds of 32 whole rows -> recognised; example 2: the transposed store from
    it, rounds of 4 columns -> the swizzle changes within a round, not recognised."""
    import layout_permuting_copy_amd.dev as D
    swz = lambda o: R.xor_swizzle(o, 3, 3, 3)
    ident = lambda o: o
    cases = {  # which: (global layout, LDS layout, threads, elem bytes, swizzle of the LDS side)
        0: (R.layout((32, 32), (32, 1)), R.layout((32, 32), (32, 1)), 64, 4, ident),
        1: (R.layout((64, 64), (192, 1)), R.layout((64, 64), (64, 1)), 256, 2, swz),
        2: (R.layout((64, 64), (1, 192)), R.layout((64, 64), (64, 1)), 256, 2, swz),
        5: (R.layout((64, 64), (16384, 1)), R.layout((64, 64), (64, 1)), 256, 2, swz),
        6: (R.layout((64, 64), (16384, 1)), R.layout((64, 64), (64, 1)), 256, 2, swz),
        7: (R.layout((64, 64), (16384, 1)), R.layout((64, 64), (64, 1)), 256, 2, ident),
    }
    for which, (g, s, threads, eb, f_s) in cases.items():
        o = R.gmem_smem_partition(g, s, threads, eb, vec_bits=(128, 64, 32))
        gl = np.array(o["g_lin"])
        sl = np.vectorize(f_s)(np.array(o["s_lin"]))
        affine = all(len(set((gl[f] - gl[0]).tolist())) == 1 and len(set((sl[f] - sl[0]).tolist())) == 1
                     for f in range(o["outer"]))
        p = D.example_plan(which, lowered=True)
        assert (p["vec"], p["outer"]) == (o["vec"], o["outer"]), which
        assert p["lowered"] == affine, which
    assert [D.example_plan(w, lowered=True)["lowered"] for w in (1, 2, 5)] == [True, False, True]


# ---- GPU -------------------------------------------------------------------------------------

def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _bits(n, seed):
    return np.frombuffer(np.random.default_rng(seed).bytes(n), dtype=np.uint8).copy()


@pytest.mark.gpu
def test_roundtrip32_wave_scope():
    torch = _torch()
    import layout_permuting_copy_amd.dev as D
    src = _bits(4096, 1)
    s = torch.from_numpy(src).cuda()
    d = torch.full((4096,), 0xA5, dtype=torch.uint8, device="cuda")
    D.roundtrip32(s, d)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), src)


@pytest.mark.gpu
@pytest.mark.parametrize("which,k,shift", [(0, 0, 0), (0, 1, 3), (0, 2, 5), (1, 2, 3), (1, 0, 0), (1, 1, 6)])
def test_wave_permute_in_place(which, k, shift):
    """Every (k, shift) gives the same permuted tile (the swizzle only reorders the lanes' work),
    equal to the oracle's copy through the two layouts and to its literal register-staged run."""
    torch = _torch()
    import layout_permuting_copy_amd.dev as D
    ntiles = 37
    src = _bits(ntiles * 1024, 7 + which)
    s = torch.from_numpy(src).cuda()
    d = torch.full_like(s, 0xA5)
    D.permute_tiles(s, d, ntiles, which, k, shift)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    if which == 0:
        sl, dl = R.layout((2, 1, 4, 32), (128, 128, 32, 1)), R.layout((2, 1, 4, 32), (128, 128, 1, 4))
    else:
        sl, dl = R.layout((4, 64), (64, 1)), R.layout((4, 64), (1, 4))
    for t in (0, 1, ntiles - 1):
        tile = src[t * 1024:(t + 1) * 1024]
        want = tile.copy()
        R.copy(tile, sl, want, dl, 4)
        lit = tile.copy()
        R.permute_layout_py(tile, sl, lit, dl, 4, 64, k, shift)
        assert np.array_equal(want, lit)
        assert np.array_equal(got[t * 1024:(t + 1) * 1024], want), (t, which, k, shift)
    want_all = np.concatenate([_perm_tile(src[t * 1024:(t + 1) * 1024], sl, dl) for t in range(ntiles)])
    assert np.array_equal(got, want_all)


def _perm_tile(tile, sl, dl):
    out = tile.copy()
    R.copy(tile, sl, out, dl, 4)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("tiles_r,tiles_c", [(1, 1), (2, 3), (3, 2)])
def test_swizzled_lds_transpose(tiles_r, tiles_c):
    """Global -> XOR-swizzled LDS -> global transposed, by a workgroup: the LDS image holds element
    (r, c) at xor_swizzle(64 r + c) and the result is the transpose."""
    torch = _torch()
    import layout_permuting_copy_amd.dev as D
    n, m = 64 * tiles_r, 64 * tiles_c
    src = _bits(n * 192 * 2, 11 + tiles_r).view(np.uint16)
    s = torch.from_numpy(src.view(np.uint8)).cuda()
    d = torch.full((64 * tiles_c * 192 * 2,), 0xA5, dtype=torch.uint8, device="cuda")
    dump = torch.zeros((tiles_r * tiles_c * 4096 * 2,), dtype=torch.uint8, device="cuda")
    D.swizzled_transpose(s, d, dump, tiles_r, tiles_c)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    want = np.full_like(got, 0xA5)
    R.copy(src.view(np.uint8), R.layout((n, m), (192, 1)), want, R.layout((n, m), (1, 192)), 2)
    assert np.array_equal(got, want)
    lds = dump.cpu().numpy().view(np.uint16).reshape(tiles_r * tiles_c, 4096)
    sw = np.array([R.xor_swizzle(o, 3, 3, 3) for o in range(4096)])
    mat = src.reshape(-1, 192)
    for t in range(tiles_r * tiles_c):
        tr, tc = divmod(t, tiles_c)
        tile = mat[tr * 64:(tr + 1) * 64, tc * 64:(tc + 1) * 64].reshape(-1)
        image = np.empty(4096, dtype=np.uint16)
        image[sw] = tile
        assert np.array_equal(lds[t], image), t


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_tile_stream_through_lds(mode):
    """64 x 64 bf16 tiles of a pitch-16384 matrix staged through a plain (0) or XOR-swizzled LDS
    tile with recognised (1) or general (2) rounds and written back in place: bit-exact, and
    nothing outside the tiles is written."""
    torch = _torch()
    import layout_permuting_copy_amd.dev as D
    tiles_r, tiles_c = 3, 5
    n_el = 64 * tiles_r * 16384
    src = _bits(n_el * 2, 21 + mode)
    s = torch.from_numpy(src).cuda()
    d = torch.full((n_el * 2,), 0xA5, dtype=torch.uint8, device="cuda")
    D.tile_stream(s, d, tiles_r, tiles_c, mode)
    torch.cuda.synchronize()
    want = np.full(n_el * 2, 0xA5, dtype=np.uint8)
    lay = R.layout((64 * tiles_r, 64 * tiles_c), (16384, 1))
    R.copy(src, lay, want, lay, 2)
    assert np.array_equal(d.cpu().numpy(), want)


@pytest.mark.gpu
def test_lane_scope_copy():
    torch = _torch()
    import layout_permuting_copy_amd.dev as D
    src = _bits(240, 3)
    s = torch.from_numpy(src).cuda()
    d = torch.full((105,), 0xA5, dtype=torch.uint8, device="cuda")
    D.lane_copy(s, d)
    torch.cuda.synchronize()
    want = np.full(105, 0xA5, dtype=np.uint8)
    R.copy(src, R.layout((3, 5, 7), (80, 9, 1)), want, R.layout((3, 5, 7), (1, 3, 15)), 1)
    assert np.array_equal(d.cpu().numpy(), want)


@pytest.mark.gpu
def test_two_wave_guarded_copy():
    torch = _torch()
    import layout_permuting_copy_amd.dev as D
    src = _bits(45 * 56 * 2, 5)
    s = torch.from_numpy(src).cuda()
    d = torch.full((45 * 40 * 2 + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    D.waves2_copy(s, d)
    torch.cuda.synchronize()
    want = np.full(45 * 40 * 2 + 64, 0xA5, dtype=np.uint8)
    R.copy(src, R.layout((45, 40), (56, 1)), want, R.layout((45, 40), (40, 1)), 2)
    assert np.array_equal(d.cpu().numpy(), want)  # nothing written past the 1800 elements


def test_wave_permute_hardware_counts_match_bank_model():
    """The committed rocprofv3 counts of the device wave permute (SQ_LDS_BANK_CONFLICT per
    dispatch, profiles/wave_permute.json) equal the oracle's simulated extra cycles per tile
    times the tiles, for every (tile, k, shift) measured: the chooser's (2, 3) on the 4 x 64 tile
    is conflict-free on the hardware, the others cost what the model predicts."""
    import json
    path = os.path.join(ROOT, "profiles", "wave_permute.json")
    doc = json.load(open(path))
    m = R.gfx950_model()
    layouts = {0: (R.layout((2, 1, 4, 32), (128, 128, 32, 1)), R.layout((2, 1, 4, 32), (128, 128, 1, 4))),
               1: (R.layout((4, 64), (64, 1)), R.layout((4, 64), (1, 4)))}
    assert len(doc["cases"]) >= 6
    for c in doc["cases"]:
        ext, ss, ds, _, _ = R.permute_shard(*layouts[c["which"]])
        per_tile = sum(R.permute_conflicts(ext, ss, ds, 4, c["k"], c["shift"], m))
        assert c["SQ_LDS_BANK_CONFLICT"] == per_tile * c["tiles"], c
    assert any(c["which"] == 1 and (c["k"], c["shift"]) == (2, 3) and c["SQ_LDS_BANK_CONFLICT"] == 0 for c in doc["cases"])
