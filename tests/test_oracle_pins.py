"""Pins of the oracle to things other than itself: values the pages print, library routines the
copy reduces to in special cases, stated invariants, closed forms, brute force and hardware
measurements.  CPU only."""

import itertools
import math

import numpy as np
import pytest

from conftest import read_golden

import synth_inputs as SI


# ---------------------------------------------------------------------------------------------
# copy: special cases that reduce to NumPy routines
# ---------------------------------------------------------------------------------------------

def _np_type(eb):
    return {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64, 16: np.dtype("V16")}[eb]


def _rand(n_bytes, seed):
    return np.frombuffer(np.random.default_rng(seed).bytes(n_bytes), dtype=np.uint8).copy()


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n,m", [(1, 7), (5, 3), (64, 64), (33, 65), (128, 40)])
def test_copy_2d_transpose_is_numpy_transpose(oracle_lib, eb, n, m):
    R = oracle_lib
    src = _rand(n * m * eb, n * 131 + m + eb)
    dst = np.zeros_like(src)
    R.copy(src, R.layout((n, m), (m, 1)), dst, R.layout((n, m), (1, n)), eb)
    a = src.view(_np_type(eb)).reshape(n, m)
    assert np.array_equal(dst.view(_np_type(eb)).reshape(m, n), np.ascontiguousarray(a.T))


def test_copy_py_matches_numpy_on_tiny(oracle_lib):
    R = oracle_lib
    for eb in (1, 2, 4, 8, 16):
        src = _rand(6 * 5 * eb, eb)
        dst = np.zeros_like(src)
        R.copy_py(src, R.layout((6, 5), (5, 1)), dst, R.layout((6, 5), (1, 6)), eb)
        a = src.view(_np_type(eb)).reshape(6, 5)
        assert np.array_equal(dst.view(_np_type(eb)).reshape(5, 6), np.ascontiguousarray(a.T))


def test_copy_py_with_offsets_matches_numpy_slice(oracle_lib):
    R = oracle_lib
    n = 10
    src = _rand(n * n * 4, 11)
    dst = np.full((n + 3) * n * 4, 0x5A, dtype=np.uint8)
    # source view [1:9, 0:8:2] (offset n), destination transposed with offset 5 and pitch n + 3
    R.copy_py(src, R.layout((8, 4), (n, 2), n), dst, R.layout((8, 4), (1, n + 3), 5), 4)
    a = src.view(np.uint32).reshape(n, n)
    d = dst.view(np.uint32)
    for c in range(4):
        assert np.array_equal(d[5 + c * (n + 3): 5 + c * (n + 3) + 8], a[1:9, 2 * c])


def test_permute0213_is_numpy_transpose(oracle_lib):
    R = oracle_lib
    w = SI.permute0213(b=2, h=3, s=16, d=8)
    src = _rand(SI.storage_elems(w, "src") * 2, 4)
    dst = np.zeros(SI.storage_elems(w, "dst") * 2, dtype=np.uint8)
    R.copy(src, R.layout(w.src.shape, w.src.stride), dst, R.layout(w.dst.shape, w.dst.stride), 2)
    a = src.view(np.uint16).reshape(2, 3, 16, 8)
    assert np.array_equal(dst.view(np.uint16).reshape(2, 16, 3, 8), a.transpose(0, 2, 1, 3))


def test_sf_transpose_is_numpy_transpose(oracle_lib):
    R = oracle_lib
    w = SI.sf_transpose(tiles=9)
    src = _rand(SI.storage_elems(w, "src") * 4, 2)
    dst = np.zeros_like(src)
    R.copy(src, R.layout(w.src.shape, w.src.stride), dst, R.layout(w.dst.shape, w.dst.stride), 4)
    a = src.view(np.uint32).reshape(9, 2, 4, 32)
    # destination (tile, stage, c, r) with stride (256, 128, 4, 1): every 4x32 block transposed
    assert np.array_equal(dst.view(np.uint32).reshape(9, 2, 32, 4), a.transpose(0, 1, 3, 2))


@pytest.mark.parametrize("eb", [1, 2, 8, 16])
def test_slice_is_numpy_slice(oracle_lib, eb):
    R = oracle_lib
    n = 12
    w = SI.sweep_slice(SI.SWEEP_DTYPES[[1, 2, 8, 16].index(eb)], n=n)
    src = _rand(n * n * eb, 54)
    dst = np.zeros(SI.storage_elems(w, "dst") * eb, dtype=np.uint8)
    R.copy(src, R.layout(w.src.shape, w.src.stride, w.src.offset), dst,
           R.layout(w.dst.shape, w.dst.stride, w.dst.offset), eb)
    a = src.view(_np_type(eb)).reshape(n, n)
    want = np.ascontiguousarray(a[1:n - 1:1, 0:n - 2:2].T)
    assert np.array_equal(dst.view(_np_type(eb)).reshape(want.shape), want)


def test_negative_strides_match_numpy_flip(oracle_lib):
    R = oracle_lib
    src = _rand(7 * 9 * 4, 9)
    dst = np.zeros_like(src)
    # logical (i, j) reads src[6 - i][j] (a row-flipped view), writes dst row-major
    R.copy(src, R.layout((7, 9), (-9, 1), 6 * 9), dst, R.layout((7, 9), (9, 1)), 4)
    a = src.view(np.uint32).reshape(7, 9)
    assert np.array_equal(dst.view(np.uint32).reshape(7, 9), a[::-1])


def test_identity_round_trip_and_double_transpose(oracle_lib):
    R = oracle_lib
    w = SI.tile32_roundtrip()
    src = SI.make_source(w)
    dst = np.zeros_like(src)
    R.copy(src, R.layout(w.src.shape, w.src.stride), dst, R.layout(w.dst.shape, w.dst.stride), 4)
    assert np.array_equal(src, dst)
    t = np.zeros_like(src)
    back = np.zeros_like(src)
    R.copy(src, R.layout((32, 32), (32, 1)), t, R.layout((32, 32), (1, 32)), 4)
    R.copy(t, R.layout((32, 32), (32, 1)), back, R.layout((32, 32), (1, 32)), 4)
    assert np.array_equal(back, src) and not np.array_equal(t, src)


def test_sentinel_outside_dst_image_untouched(oracle_lib):
    R = oracle_lib
    src = _rand(4 * 6 * 4, 1)
    dst = np.full(4 * 16 * 4, 0xA5, dtype=np.uint8)
    # dst rows have a pitch of 16 elements, only 6 written per row, offset 3
    R.copy(src, R.layout((4, 6)), dst, R.layout((4, 6), (16, 1), 3), 4)
    d = dst.view(np.uint32).reshape(4, 16)
    assert np.array_equal(d[:, 3:9], src.view(np.uint32).reshape(4, 6))
    untouched = np.ones((4, 16), bool)
    untouched[:, 3:9] = False
    assert np.all(dst.reshape(4, 16, 4)[untouched] == 0xA5)


def test_unit_modes_dropped_and_extent_mismatch_rejected(oracle_lib):
    R = oracle_lib
    src = _rand(4 * 32 * 4, 3)
    dst = np.zeros_like(src)
    R.copy(src, R.layout((1, 4, 32)), dst, R.layout((4, 1, 32), (32, 7, 1)), 4)
    assert np.array_equal(src, dst)
    with pytest.raises(ValueError):
        R.copy(src, R.layout((4, 32)), dst, R.layout((32, 4)), 4)


def test_sample_offsets_agree_with_definition(oracle_lib):
    R = oracle_lib
    s, d = R.layout((3, 4, 5), (20, 1, 4), 7), R.layout((3, 4, 5), (1, 15, 3), 2)
    flat = np.arange(60)
    so, do = R.sample_offsets(s, d, flat)
    for f in range(60):
        idx = np.unravel_index(f, (3, 4, 5))
        assert so[f] == 7 + 20 * idx[0] + idx[1] + 4 * idx[2]
        assert do[f] == 2 + idx[0] + 15 * idx[1] + 3 * idx[2]


# ---------------------------------------------------------------------------------------------
# partition: TVM TIRx "copy -> gmem_smem" worked example and table; TileLang loop_mapping prose
# ---------------------------------------------------------------------------------------------

def test_gmem_smem_demo_values(oracle_lib):
    R = oracle_lib
    g = read_golden("gmem_smem_demo.txt")
    shape = tuple(int(x) for x in g["shape"][0].split(","))
    T = int(g["threads"][0])
    for row in g["row"]:
        name, eb, vec, copy_bytes, outer = row.split()
        p = R.gmem_smem_partition(R.layout(shape), R.layout(shape), T, int(eb))
        assert (p["vec"], p["copy_bytes"], p["outer"]) == (int(vec), int(copy_bytes), int(outer)), name
    p = R.gmem_smem_partition(R.layout(shape), R.layout(shape), T, 4)
    expr = g["lin_expr"][0]
    for f in range(p["outer"]):
        for tid in range(T):
            want = eval(expr, {}, {"f": f, "tid": tid})
            assert p["g_lin"][f][tid] == want and p["s_lin"][f][tid] == want


def test_gmem_smem_declines_when_count_does_not_divide_threads(oracle_lib):
    R = oracle_lib
    p = R.gmem_smem_partition(R.layout((3, 11)), R.layout((3, 11)), 32, 4)
    assert p["declined"] and "not divisible" in p["reason"]


def test_gmem_smem_vector_rule(oracle_lib):
    R = oracle_lib
    # shared side transposed -> no two consecutive global elements are adjacent in shared
    p = R.gmem_smem_partition(R.layout((32, 32)), R.layout((32, 32), (1, 32)), 32, 4)
    assert p["vec"] == 1 and p["outer"] == 32
    # base offset 2 (float32) is 8-byte but not 16-byte aligned -> 64-bit vectors
    p = R.gmem_smem_partition(R.layout((32, 32), None, 2), R.layout((32, 32)), 32, 4)
    assert p["vec"] == 2
    # global rows of 34 elements (pitch not a multiple of 4) with 32 used -> vec 2
    p = R.gmem_smem_partition(R.layout((32, 32), (34, 1)), R.layout((32, 32)), 32, 4)
    assert p["vec"] == 2
    # the global side drives the order: a column-major global tile still vectorizes along it
    p = R.gmem_smem_partition(R.layout((32, 32), (1, 32)), R.layout((32, 32), (1, 32)), 32, 4)
    assert p["vec"] == 4 and p["g_lin"][0][:3] == [0, 4, 8]


def _loop_cases():
    g = read_golden("loop_mapping_cases.txt")
    cases = []
    for c in g["case"]:
        ext, thr, vec = (s.strip() for s in c.split("|"))
        cases.append((tuple(int(x) for x in ext.split(",")), int(thr), int(vec)))
    return cases


@pytest.mark.parametrize("extents,T,vec", _loop_cases())
def test_loop_partition_nesting(oracle_lib, extents, T, vec):
    """Page prose: three nested levels, fastest first -- lane (vector), thread, serial
    replication.  These properties determine the map without restating the formula."""
    R = oracle_lib
    plan = R.loop_partition(extents, T, vec)
    total = math.prod(extents)
    by_flat = {}
    for idx, (t, slot) in plan.items():
        by_flat[R.flat_of_index(idx, extents)] = (t, slot)
    assert len(set(plan.values())) == total  # every (thread, slot) is used once
    for flat in range(total):
        t, slot = by_flat[flat]
        if flat % vec:  # consecutive iterations share a lane-set (vectorize)
            pt, ps = by_flat[flat - 1]
            assert (pt, ps + 1) == (t, slot)
        elif flat % (vec * T):  # the next vector goes to the next thread (coalesce)
            pt, ps = by_flat[flat - vec]
            assert (pt + 1, ps - (vec - 1)) == (t, slot - (vec - 1)) and slot % vec == 0
        else:  # only then a per-thread serial loop grows
            assert t == 0 and slot == (flat // (vec * T)) * vec
    used = {t for t, _ in plan.values()}
    if total < T * vec:  # fewer points than threads*vec: some threads get no work (guarded)
        assert used == set(range(-(-total // vec)))
    else:
        assert used == set(range(T))


def test_compare_shapes_same_count_per_thread(oracle_lib):
    R = oracle_lib
    g = read_golden("loop_mapping_cases.txt")
    T, vec = int(g["compare_threads"][0]), int(g["compare_vector"][0])
    for c in g["compare"]:
        ext = tuple(int(x) for x in c.split(","))
        plan = R.loop_partition(ext, T, vec)
        per = {}
        for t, _ in plan.values():
            per[t] = per.get(t, 0) + 1
        assert set(per.values()) == {math.prod(ext) // T}


def test_loop_partition_agrees_with_gmem_smem_listing(oracle_lib):
    """Two pages, one worked example: the TileLang formula applied to the 32x32 row-major tile
    with 32 threads and vector 4 gives the offsets the TIRx listing prints (f*128 + tid*4)."""
    R = oracle_lib
    plan = R.loop_partition((32, 32), 32, 4)
    for idx, (t, slot) in plan.items():
        f = slot // 4
        if slot % 4 == 0:
            assert R.flat_of_index(idx, (32, 32)) == f * 128 + t * 4


# ---------------------------------------------------------------------------------------------
# XOR swizzle chooser (TVM TIRx "permute_layout")
# ---------------------------------------------------------------------------------------------

def _sf_demo():
    g = read_golden("permute_sf_demo.txt")
    ints = lambda key: tuple(int(x) for x in g[key][0].split(","))
    return g, ints("shape"), ints("src_strides"), ints("dst_strides")


def test_permute_demo_plan(oracle_lib):
    R = oracle_lib
    g, shape, ss, ds = _sf_demo()
    src = R.layout(shape, ss)
    dst = R.layout(shape, ds)
    # region B_buf[s, 0:1, 0:4, 0:32] for one stage
    stage = (1, 1, 4, 32)
    extent, s_str, d_str, _, _ = R.permute_shard(R.layout(stage, ss), R.layout(stage, ds))
    lanes = int(g["lanes"][0])
    assert math.prod(extent) // lanes == int(g["P"][0])
    k, shift, mask = R.choose_xor_k(extent, s_str, d_str, int(g["elem_bytes"][0]))
    assert (k, shift, mask) == (int(g["k"][0]), int(g["shift"][0]), int(g["mask"][0]))
    # every (stage, step, lane) address equals the generated IR's
    for s in range(int(g["pipe"][0])):
        for r in range(int(g["P"][0])):
            for tx in range(lanes):
                so, do = R.permute_access(extent, s_str, d_str, lanes, k, shift, r, tx)
                env = {"s": s, "r": r, "tx": tx}
                assert s * 128 + so == eval(g["read_expr"][0], {}, env)
                assert s * 128 + do == eval(g["write_expr"][0], {}, env)
    assert src and dst


def test_permute_demo_k0_and_k1_conflict(oracle_lib):
    """Brute force: without the swizzle the write phase is 4-way conflicted (lanes 0, 8, 16, 24
    share a bank), one XOR bit halves it; the read phase is always conflict-free."""
    R = oracle_lib
    ext, ss, ds = (4, 32), (32, 1), (1, 4)
    assert R.permute_conflicts(ext, ss, ds, 4, 0, 0) == (0, 4 * 3)
    assert min(R.permute_conflicts(ext, ss, ds, 4, 1, s)[1] for s in range(5)) == 4 * 1
    assert R.permute_conflicts(ext, ss, ds, 4, 2, 3) == (0, 0)


def test_four_byte_dtypes_always_admit_k(oracle_lib):
    """Page: 4-byte dtypes always admit a valid k (one element per bank)."""
    R = oracle_lib
    for a, b in [(4, 32), (8, 32), (2, 64), (32, 32), (16, 16), (16, 32), (64, 16), (8, 8), (4, 64), (128, 8)]:
        assert R.choose_xor_k((a, b), (b, 1), (1, a), 4) is not None, (a, b)


def test_sub_word_reads_can_fail(oracle_lib):
    """Page: stride-1 sub-4-byte reads can pack several lanes into one bank and make the
    dispatch fail -- true when lanes are counted per bank (no same-word broadcast)."""
    R = oracle_lib
    assert R.choose_xor_k((4, 32), (32, 1), (1, 4), 2, R.page_model("lane")) is None
    assert R.choose_xor_k((4, 32), (32, 1), (1, 4), 2, R.page_model("dword")) == (2, 3, 3)


def test_swizzle_does_not_change_result(oracle_lib):
    """The XOR permutes which register holds which iteration, not the data: every k gives
    the plain copy's result."""
    R = oracle_lib
    src = _rand(2 * 128 * 4, 7)
    want = np.zeros_like(src)
    s_lay, d_lay = R.layout((4, 32), (32, 1)), R.layout((4, 32), (1, 4))
    R.copy_py(src, s_lay, want, d_lay, 4)
    for k in range(3):
        for shift in range(6 - k):
            got = np.zeros_like(src)
            R.permute_layout_py(src, s_lay, got, d_lay, 4, 32, k, shift)
            assert np.array_equal(got, want)


def test_k0_is_no_swizzle(oracle_lib):
    R = oracle_lib
    for lane in range(32):
        for r in range(4):
            assert R.permute_access((4, 32), (32, 1), (1, 4), 32, 0, 0, r, lane) == (r * 32 + lane, lane * 4 + r)


# ---------------------------------------------------------------------------------------------
# bank-conflict counting: closed forms and the gfx950 hardware measurements
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("stride", [1, 2, 3, 4, 6, 8, 12, 16, 32, 33, 64])
def test_conflicts_closed_form_strided_words(oracle_lib, stride):
    """32 lanes reading words l*stride from 32 banks: 32/gcd banks are used, each by gcd lanes
    (all different words), so the access costs gcd(stride, 32) - 1 extra cycles."""
    R = oracle_lib
    addrs = [4 * l * stride for l in range(32)]
    assert R.conflict_cycles(addrs, 4, "read", R.page_model("dword")) == math.gcd(stride, 32) - 1


def test_conflicts_broadcast_rule(oracle_lib):
    R = oracle_lib
    same = [0] * 32
    assert R.conflict_cycles(same, 4, "read", R.page_model("dword")) == 0
    assert R.conflict_cycles(same, 4, "read", R.page_model("lane")) == 31


def test_gfx950_model_matches_probe_measurements(oracle_lib):
    R = oracle_lib
    m = R.gfx950_model()
    n = 0
    from conftest import golden_path
    for line in open(golden_path("lds_probe_gfx950.txt")):
        if line.startswith("#"):
            continue
        head, addrs = line.split(":")
        w, op, name, conf = head.split()
        addrs = [int(a) for a in addrs.split(",")]
        assert R.conflict_cycles(addrs, int(w), op, m) == float(conf), (w, op, name)
        n += 1
    assert n == 84


def test_tile_wave_locality_pins():
    """Which waves own which LDS units follows from the two loop partitions by hand:
    * the scale-factor 4x32 fp32 block: 8 loads of 16 bytes per row x 4 rows = 32 loads, and
      32 columns x 1 store vector each = 32 stores, both in block-major order, so lanes 0-31
      and 32-63 of every wave load and store the same two whole blocks -> wave-local;
    * a 32x256 fp32 tile of 256 lanes: a wave loads one row per round (64 x 16 bytes), but its
      first store round reads 8 columns x all 32 rows, rows loaded by all four waves -> not;
    * one wave per workgroup is wave-local whatever the tile."""
    from oracle import ref as R
    assert R.tile_wave_local(4, 16, 4, 32, 16, 256)
    assert not R.tile_wave_local(4, 16, 32, 256, 1, 256)
    assert R.tile_wave_local(4, 16, 32, 256, 1, 64) and R.tile_wave_local(1, 16, 128, 128, 1, 64)
    # 8-byte elements: a 4x32 block is 16 loads per row x 4 rows = 64 loads and 32 columns x 2
    # store vectors = 64 stores, one whole block per wave and round -> wave-local; with 16
    # columns per block it is 32 loads but 16 x 2 = 32 stores -> still whole blocks
    assert R.tile_wave_local(8, 16, 4, 32, 8, 256) and R.tile_wave_local(8, 16, 4, 16, 16, 256)
    # a 16x64 fp32 tile: 16 loads per row -> a wave loads 4 rows; a store vector covers 4 rows
    # of a column, 4 vectors per column -> a wave stores 16 columns x all 16 rows -> not
    assert not R.tile_wave_local(4, 16, 16, 64, 1, 256)


def test_synthetic_inputs_are_seeded_and_shaped():
    w = SI.transpose2d(n=64, dtype="bfloat16")
    a, b = SI.make_source(w), SI.make_source(w)
    assert np.array_equal(a, b) and a.size == 64 * 64 * 2
    w2 = SI.sweep_slice("int4vec", n=16)
    assert SI.storage_elems(w2, "src") == 256 and w2.src.shape == (14, 7) and w2.src.offset == 16
    # bfloat16 values are round-to-nearest-even of float32 normals
    f = np.array([1.0, 1.00390625, 1.01171875, -2.5], dtype=np.float32)
    assert list(SI._bf16_bits_from_f32(f)) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_xor_swizzle_offsets_pins():
    """The swizzled shared layout's offset function, checked by hand and by its properties:
    64 x 64 elements, 8-element chunks (base 3), chunk index XOR row mod 8 (bits 3, shift 3)."""
    from oracle import ref as R
    # row 0 is unchanged; row 1 chunk 0 -> chunk 1; row 5 chunk 2 -> chunk 7; row 9 == row 1
    assert [R.xor_swizzle(o, 3, 3, 3) for o in (0, 7, 64, 64 + 8 * 2 + 5, 5 * 64 + 2 * 8 + 3, 9 * 64)] == \
        [0, 7, 72, 64 + 8 * 3 + 5, 5 * 64 + 7 * 8 + 3, 9 * 64 + 8]
    image = [R.xor_swizzle(o, 3, 3, 3) for o in range(4096)]
    assert sorted(image) == list(range(4096))  # a permutation of the tile
    for o in range(0, 4096, 8):  # chunks stay whole and in their row
        assert image[o] % 8 == 0 and image[o + 7] == image[o] + 7 and image[o] // 64 == o // 64
    assert all(R.xor_swizzle(o, 0, 3, 3) == o for o in range(256))  # no bits: identity


def test_wave64_permute_reproduces_page_result_on_4x64():
    """At 64 lanes the page's printed plan (k, shift, mask) = (2, 3, 3) is the answer for the
    4 x 64 fp32 tile, the wave64 counterpart of its 4 x 32 demo at 32 lanes; the 4 x 32 demo tile
    itself has no conflict-free k on gfx950 (32-lane bank groups see only even rows of it)."""
    from oracle import ref as R
    m = R.gfx950_model()
    ext, ss, ds, _, _ = R.permute_shard(R.layout((4, 64), (64, 1)), R.layout((4, 64), (1, 4)))
    assert R.choose_xor_k(ext, ss, ds, 4, m) == (2, 3, 3)
    ext, ss, ds, _, _ = R.permute_shard(R.layout((2, 1, 4, 32), (128, 128, 32, 1)), R.layout((2, 1, 4, 32), (128, 128, 1, 4)))
    assert R.choose_xor_k(ext, ss, ds, 4, m) is None
    assert R.permute_conflicts(ext, ss, ds, 4, 0, 0, m) == (0, 24)


# ---------------------------------------------------------------------------------------------
# LDS tile of the global -> LDS -> global transpose: the oracle's bank simulation against the
# hardware counter (SQ_LDS_BANK_CONFLICT per dispatch) and a closed form
# ---------------------------------------------------------------------------------------------

def _bank_pin_cases():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                        "bank_pin_transpose_tiles.json")
    with open(path) as f:
        return json.load(f)["cases"]


def test_transpose_tile_hardware_counts_match_oracle(oracle_lib):
    """Every measured tile -- swizzle off, swizzles the search passes over, and the chosen ones, on
    4-, 8- and 16-byte LDS units and 1- to 16-byte elements -- costs exactly the extra cycles the
    oracle simulates (per tile, times the tiles), and issues the LDS instructions its two TileLang
    partitions imply.  Non-zero counts in both phases are among them."""
    R = oracle_lib
    cases = _bank_pin_cases()
    assert len(cases) >= 20
    nonzero_w = nonzero_r = 0
    for c in cases:
        tr, tc, nb = c["tile"]
        k, shift, tbit, cshift, cmask = c["xor"]
        args = (c["elem_bytes"], c["vec_bytes"], tr, tc, nb, c["threads"])
        w, r = R.lds_tile_conflicts(*args, k, shift, tbit, cshift, cmask, U=c["lds_unit_bytes"])
        assert (w + r) * c["tiles"] == c["SQ_LDS_BANK_CONFLICT"], c["label"]
        assert R.lds_tile_wave_instructions(*args, U=c["lds_unit_bytes"]) * c["tiles"] == c["SQ_INSTS_LDS"], c["label"]
        assert c["sampled_parity"] and c["edge_tiles"] in (0, 1)
        nonzero_w += w > 0
        nonzero_r += r > 0
    assert nonzero_w >= 5 and nonzero_r >= 15


def test_transpose_tile_swizzle_is_minimal_on_hardware(oracle_lib):
    """The permute page's rule (Algorithm step 2): the smallest k that leaves both phases
    conflict-free.  For each measured geometry the oracle's search lands on the swizzle the
    hardware counted 0 for, and every measured swizzle with fewer bits conflicts on the hardware."""
    R = oracle_lib
    cases = _bank_pin_cases()
    geom = lambda c: (c["elem_bytes"], c["vec_bytes"], *c["tile"], c["threads"], c["lds_unit_bytes"])
    chosen = [c for c in cases if c["label"].endswith("chosen")]
    assert len(chosen) >= 3
    for c in chosen:
        eb, vb, tr, tc, nb, nt, u = geom(c)
        best = R.lds_tile_swizzle(eb, vb, tr, tc, nb, nt, U=u)
        assert [best[x] for x in ("k", "shift", "tbit", "cshift", "cmask")] == c["xor"], c["label"]
        assert c["SQ_LDS_BANK_CONFLICT"] == 0
        fewer = [o for o in cases if geom(o) == geom(c) and o["xor"][0] < best["k"]]
        assert {o["xor"][0] for o in fewer} == set(range(best["k"])), c["label"]  # every smaller k measured
        for o in fewer:
            assert o["SQ_LDS_BANK_CONFLICT"] > 0, o["label"]


@pytest.mark.parametrize("TR,TC", [(64, 64), (32, 64), (128, 32), (16, 128), (64, 256)])
def test_unswizzled_4byte_unit_tile_closed_form(oracle_lib, TR, TC):
    """Hand-derived count for 4-byte elements in 4-byte LDS units, no swizzle, 256 lanes.  Store
    phase: a read instruction's lanes cover columns of TR/4 row vectors each; with TC a multiple of
    32 a column's units all sit in one bank, so each 32-lane group of a 4-byte read (gfx950: 32
    banks, 32 lanes) has TR/4 dwords in one bank -> TR/4 - 1 extra cycles, two groups per wave
    instruction, TR*TC/64 wave instructions per tile.  Load phase: a 16-byte write of 8 lanes
    covers 32 consecutive dwords of one row -> conflict-free."""
    R = oracle_lib
    w, r = R.lds_tile_conflicts(4, 16, TR, TC, 1, 256, U=4)
    assert w == 0
    assert r == (TR * TC // 64) * 2 * (TR // 4 - 1)
