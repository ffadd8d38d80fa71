"""Bit-exact parity of the HIP path (through the C ABI) with the oracle, on seeded inputs.
Every destination is prefilled with a sentinel, so writes outside the destination image fail
the comparison too."""

import itertools

import numpy as np
import pytest

import layout_permuting_copy_amd as L
import synth_inputs as SI
from gpu_util import assert_same, check_workload, dtype_code, oracle_copy, run_copy, say

pytestmark = pytest.mark.gpu

DT_BY_EB = {1: "int8", 2: "bfloat16", 4: "float32", 8: "float64", 16: "int4vec"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    yield
    torch.cuda.synchronize()


def _bits(n_bytes, seed):
    return np.frombuffer(np.random.default_rng(seed).bytes(n_bytes), dtype=np.uint8).copy()


def _check(shape, s_stride, d_stride, eb, s_off=0, d_off=0, src_elems=None, dst_elems=None, flags=0, seed=0,
           expect=None):
    sl = (shape, s_stride, s_off)
    dl = (shape, d_stride, d_off)

    def span(st, off):
        if any(e == 0 for e in shape):
            return off + 1
        return off + sum((e - 1) * s for e, s in zip(shape, st) if s > 0) + 1

    n_src = src_elems or span(s_stride, s_off)
    n_dst = dst_elems or span(d_stride, d_off)
    src = _bits(n_src * eb, seed)
    say(f"[gpu] shape={shape} src={s_stride}+{s_off} dst={d_stride}+{d_off} eb={eb} flags={flags}")
    got, plan = run_copy(src, sl, n_dst, dl, eb, dtype_code(DT_BY_EB[eb]), flags)
    want = oracle_copy(src, sl, n_dst, dl, eb)
    assert_same(got, want, eb, f"{shape}/{eb}")
    if expect is not None:
        assert plan["path_name"] == expect, plan
    return plan


# --- the five workloads -----------------------------------------------------------------------

def test_tile32_roundtrip_one_wave():
    plan = check_workload(SI.tile32_roundtrip(), expect_path="roundtrip")
    assert (plan["threads"], plan["load_outer"], plan["vec_bytes"], plan["workgroups"]) == (64, 4, 16, 1)


def test_sf_transpose_full():
    plan = check_workload(SI.sf_transpose(), expect_path="shuffle")
    assert (plan["tile_r"], plan["tile_c"]) == (4, 32)


def test_sf_transpose_full_lds_tile():
    plan = check_workload(SI.sf_transpose(), flags=L.TC_FLAG_NO_SHUFFLE, expect_path="transpose")
    assert plan["write_conflicts"] == 0 and plan["read_conflicts"] == 0 and plan["wave_local"] == 1


@pytest.mark.parametrize("C", [8, 16, 32])
@pytest.mark.parametrize("nb,pad_s,pad_d,soff,doff", [(1000, 0, 0, 0, 0), (16, 0, 0, 4, 8), (37, 8, 4, 0, 0),
                                                      (515, 4, 12, 8, 4), (3, 0, 0, 0, 0)])
def test_shuffle_blocks(C, nb, pad_s, pad_d, soff, doff):
    """Batches of 4 x C fp32 blocks through the register butterfly (padded pitches, offsets,
    a ragged last workgroup)."""
    shape, ss, ds = (nb, 4, C), (4 * C + pad_s, C, 1), (4 * C + pad_d, 1, 4)
    p = _check(shape, ss, ds, 4, s_off=soff, d_off=doff, seed=nb + C)
    # (an element count that does not divide the wavefront declines the page's split, but the
    # vectors are whole and aligned: the butterfly still runs, its last workgroup guarded)
    assert p["path_name"] == "shuffle" and p["declined"] == int((nb * 4 * C) % 64 != 0), p


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_transpose_16384(dtype):
    plan = check_workload(SI.transpose2d(dtype=dtype), expect_path="transpose")
    assert plan["write_conflicts"] == 0 and plan["read_conflicts"] == 0


def test_permute0213_full():
    check_workload(SI.permute0213(), expect_path="rows")


@pytest.mark.parametrize("which", ["pack", "unpack"])
def test_all_to_all_pack_unpack_full_size(which):
    """One GPU's share of the (0,2,1,3) permute sharded over 8 GPUs (heads in, sequence out): the
    pack into per-destination blocks before the all-to-all and the unpack after it, at their
    per-GPU shape (32 x 4 x 2048 x 128 bf16, 64 MiB a side)."""
    w = SI.a2a_pack_permute0213() if which == "pack" else SI.a2a_unpack_permute0213()
    check_workload(w, expect_path="rows")


@pytest.mark.parametrize("dtype", SI.SWEEP_DTYPES)
def test_dense_transposes_8192(dtype):
    check_workload(SI.sweep_dense(dtype), expect_path="transpose")


@pytest.mark.parametrize("dtype", SI.SWEEP_DTYPES)
def test_slice_8192(dtype):
    plan = check_workload(SI.sweep_slice(dtype))
    assert plan["declined"] == 1 and plan["path_name"] == "transpose" and plan["src_step"] == 2


@pytest.mark.parametrize("dtype", SI.SWEEP_DTYPES)
def test_slice_rows_8192(dtype):
    """The same slice written out densely in its own row order: gathered rows (16-byte elements:
    the element-wise rows, one element per access)."""
    plan = check_workload(SI.sweep_slice_rows(dtype))
    wide = SI.elem_bytes(dtype) == 16
    assert plan["path_name"] == ("guarded_rows" if wide else "rows") and plan["src_step"] == (0 if wide else 2)


@pytest.mark.parametrize("dtype", SI.SWEEP_DTYPES)
def test_odd_8191x8190(dtype):
    plan = check_workload(SI.sweep_odd(dtype))
    # (16-byte elements are whole aligned vectors: the aligned kernels, the page's reason kept)
    wide = SI.elem_bytes(dtype) == 16
    assert plan["declined"] == 1 and plan["path_name"] == "transpose" and plan["unaligned"] == int(not wide)


def test_odd_strict_declines():
    import torch
    w = SI.sweep_odd("float32", 191, 190)
    src = torch.zeros(191 * 190, dtype=torch.float32, device="cuda")
    dst = torch.zeros_like(src)
    with pytest.raises(L.TileCopyError) as e:
        L.tile_copy_ex(src, (w.src.shape, w.src.stride), dst, (w.dst.shape, w.dst.stride), L.TC_F32,
                       flags=L.TC_FLAG_STRICT)
    assert e.value.code == L.TC_E_DECLINED and "not divisible" in e.value.reason


# --- several tiles, ragged tails, every element width ----------------------------------------

@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n,m,soff,doff,batch", [(67, 45, 0, 0, 1), (65, 64, 0, 0, 1), (64, 65, 0, 0, 1),
                                                 (131, 257, 0, 0, 1), (7, 3, 0, 0, 1), (300, 129, 0, 0, 1),
                                                 (67, 45, 3, 5, 1), (67, 45, 0, 0, 3)])
def test_transpose_unaligned(eb, n, m, soff, doff, batch):
    """Extents with no aligned vector (or counts not divisible by 64): the transpose runs with
    vectors at element alignment, element accesses where a vector would leave the copy."""
    if batch == 1:
        shape, ss, ds = (n, m), (m, 1), (1, n)
    else:
        shape, ss, ds = (batch, n, m), (n * m, m, 1), (n * m, 1, n)
    p = L.tc_plan((shape, ss, soff), (shape, ds, doff), {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64,
                                                          16: L.TC_B128}[eb])
    assert p["path_name"] == "transpose"
    # 65 x 64 and 64 x 65 have an aligned vector of one element from 4-byte elements up: the
    # page's plan (strict mode) takes it; by default narrower vectors give way to 16-byte ones at
    # element alignment, and 16-byte elements, always whole aligned vectors, take the aligned
    # kernels (also where only the count rule declines)
    page_vec = eb >= 4 and (n, m) in ((65, 64), (64, 65)) and batch == 1 and soff == doff == 0
    assert p["unaligned"] == (eb < 16)
    _check(shape, ss, ds, eb, s_off=soff, d_off=doff, seed=n + m + eb, expect="transpose")
    if page_vec and eb < 16:
        sp = _check(shape, ss, ds, eb, seed=n + m + eb, flags=L.TC_FLAG_STRICT, expect="transpose")
        assert sp["vec_bytes"] == max(eb, 4) and not sp["unaligned"], sp


@pytest.mark.parametrize("eb,shape", [(1, (1000, 700)), (1, (3, 1001, 1300)), (1, (2047, 1023)), (8, (301, 299)),
                                      (8, (2, 515, 1031)), (8, (1101, 93)), (2, (1000, 700)), (2, (2, 515, 1031)),
                                      (2, (4097, 65))])
def test_transpose_xcd_super_tiles(eb, shape):
    """The XCD super-tile grid order of the element-aligned int8, fp16 and fp64 plans: 8 x 8 tiles
    per super-tile, padding workgroups where the tile grid is not a multiple of it."""
    n, m = shape[-2], shape[-1]
    ss, ds = (m, 1), (1, n)
    if len(shape) == 3:
        ss, ds = (n * m,) + ss, (n * m,) + ds
    p = _check(shape, ss, ds, eb, seed=n * 3 + m + eb, expect="transpose")
    assert p["unaligned"] and p["grid_order"] == 2, p
    assert (p["super_rows"], p["super_cols"]) == (8, 8), p


@pytest.mark.parametrize("to_planes,c", [(True, 64), (False, 64), (True, 32), (False, 128)])
def test_int8_channel_permutes_on_narrow_tall_tiles(to_planes, c):
    """int8 NHWC <-> NCHW with 32-128 channels (rows of channels packed shorter than a line): the
    128 KiB tiles of 16-byte LDS units with row tiles first and every load in flight."""
    h, w = 112, 112
    hw = h * w
    n = -(-(16 << 20) // (hw * c))  # at least 16 Mi elements
    if to_planes:   # logical (n, c, hw): source NHWC, destination NCHW
        shape, ss, ds = (n, c, hw), (hw * c, 1, c), (c * hw, hw, 1)
    else:           # logical (n, hw, c): source NCHW, destination NHWC
        shape, ss, ds = (n, hw, c), (c * hw, 1, hw), (hw * c, c, 1)
    p = _check(shape, ss, ds, 1, seed=c + int(to_planes), expect="transpose")
    assert (p["lds_bytes"], p["lds_read_bytes"], p["threads"], p["grid_order"], p["loads_in_flight"]) == \
        (131072, 16, 512, 1, 0), p


@pytest.mark.parametrize("n,m", [(8176, 8192), (16368, 4224)])
def test_int8_tall_tiles_destination_off_the_lines(n, m):
    """int8 transposes whose destination columns alone start off the 128-byte lines: 512 x 256
    tiles with 2 loads in flight, plain stores and XCD super-tiles (ragged tiles along both modes in
    the second shape)."""
    p = _check((n, m), (m, 1), (1, n), 1, seed=n + m, expect="transpose")
    assert (p["tile_r"], p["tile_c"], p["loads_in_flight"], p["nontemporal"], p["grid_order"]) == (512, 256, 2, 0, 2), p
    assert (p["super_rows"], p["super_cols"]) == (16, 2), p


@pytest.mark.parametrize("eb,n,m", [(1, 8191, 8192), (1, 8193, 8320), (2, 8191, 8192), (2, 1025, 256), (2, 2047, 4160)])
def test_tall_tiles_destination_at_element_alignment(eb, n, m):
    """Source rows on the 128-byte lines, destination columns at element alignment only (odd
    destination pitch): int8 on the 512 x 256 tiles and fp16 on 512 x 64 tiles, both with
    nontemporal accesses, 2 loads in flight and XCD super-tiles, ragged tiles along both modes."""
    p = _check((n, m), (m, 1), (1, n), eb, seed=n + 7 * m + eb, expect="transpose")
    want_tile = (512, 256) if eb == 1 else (512, 64)
    assert p["unaligned"] and (p["tile_r"], p["tile_c"]) == want_tile, p
    assert (p["loads_in_flight"], p["nontemporal"], p["grid_order"]) == (2, 3, 2), p
    if eb == 1:
        assert (p["super_rows"], p["super_cols"]) == (16, 2), p


@pytest.mark.parametrize("shape,strides,soff", [
    ((600, 100), (256, 2), 0),            # one column tile, ragged rows
    ((1001, 333), (1000, 2), 1000),       # ragged both ways, the last pair's high byte past the span
    ((512, 64), (128, 2), 0),             # exactly one tile wide: every tile holds a row's end
    ((2049, 4095), (8192, 2), 8192),      # the slice [1:2050, 0:8190:2] of an 8192-wide matrix
    ((3, 700, 130), (700 * 262, 262, 2), 4),  # a batch mode
    ((800, 90), (-184, 2), 799 * 184),    # rows in reverse order
    ((600, 100), (256, 2), 1),            # odd offsets: the high bytes of the pairs kept
    ((1001, 333), (1000, 2), 999),
    ((512, 64), (128, 2), 3),
    ((3, 700, 130), (700 * 262, 262, 2), 5),
    ((800, 90), (-184, 2), 799 * 184 + 1),
])
def test_int8_stride2_source_read_in_pairs(shape, strides, soff):
    """1-byte copies whose column mode has source stride 2 (even strides): the source is read as
    2-byte pairs on the tall 2-byte tiles and the low (even offset) or high (odd offset) bytes
    stored; the pair holding a row's last (low) or first (high) element is read as that byte
    only."""
    n, m = shape[-2], shape[-1]
    ds = (1, n) if len(shape) == 2 else (n * m, 1, n)
    p = _check(shape, strides, ds, 1, s_off=soff, seed=n + m + len(shape), expect="transpose")
    assert p["src_view_bytes"] == 2 and p["src_step"] == 2 and (p["tile_r"], p["tile_c"]) == (512, 64), p


@pytest.mark.parametrize("shape,strides,soff", [
    ((600, 100), (256, 2), 0),            # one column tile, ragged rows
    ((1001, 333), (1000, 2), 1000),       # ragged both ways, the last pair's high half past the span
    ((512, 64), (128, 2), 0),             # whole tiles
    ((3, 700, 130), (700 * 262, 262, 2), 4),  # a batch mode
    ((800, 90), (-184, 2), 799 * 184),    # rows in reverse order
])
@pytest.mark.parametrize("eb", [2, 4, 8])
def test_wide_stride2_source_read_in_pairs(shape, strides, soff, eb):
    """2-, 4- and 8-byte copies whose column mode has source stride 2 (even strides and offset): the
    source is read as 4-, 8- or 16-byte pairs on the tiles of that width and the low half of each pair
    stored; the pair holding a row's last element is read as that element only.  An odd offset
    keeps the stride-2 tile of the element width."""
    n, m = shape[-2], shape[-1]
    ds = (1, n) if len(shape) == 2 else (n * m, 1, n)
    p = _check(shape, strides, ds, eb, s_off=soff, seed=n + m + len(shape) + eb, expect="transpose")
    assert p["src_view_bytes"] == 2 * eb and p["src_step"] == 2, p
    p = _check(shape, strides, ds, eb, s_off=soff + 1, seed=n + m + eb + 1, expect="transpose")
    assert p["src_view_bytes"] == eb and p["src_step"] == 2, p


def test_int8_stride2_pairs_not_taken_at_odd_strides():
    """An odd row stride (rows alternate between low and high bytes of the pairs) keeps the stride-2
    tile of 1-byte elements; same bytes."""
    p = _check((700, 130), (261, 2), (1, 700), 1, s_off=4, seed=77, expect="transpose")
    assert p["src_view_bytes"] == 1 and p["src_step"] == 2, p


@pytest.mark.parametrize("shape,strides,soff", [
    ((600, 100), (512, 4), 0),            # one column tile, ragged rows
    ((1001, 333), (1336, 4), 1336),       # ragged both ways, the last word's upper bytes past the span
    ((512, 64), (256, 4), 0),             # exactly one tile wide: every tile holds a row's end
    ((2049, 2047), (8192, 4), 8192),      # the slice [1:2050, 0:8188:4] of an 8192-wide matrix
    ((3, 700, 130), (700 * 524, 524, 4), 8),  # a batch mode
    ((800, 90), (-368, 4), 799 * 368),    # rows in reverse order
])
@pytest.mark.parametrize("eb", [1, 2, 4])
def test_stride4_source_read_in_groups(shape, strides, soff, eb):
    """1-, 2- and 4-byte copies whose column mode has source stride 4 (every source stride and the
    offset multiples of 4): the source is read in groups of 4 elements (4-, 8- or 16-byte groups)
    on the tiles of that width and the first element of each stored; the group holding a row's
    last element is read as that element only."""
    n, m = shape[-2], shape[-1]
    ds = (1, n) if len(shape) == 2 else (n * m, 1, n)
    p = _check(shape, strides, ds, eb, s_off=soff, seed=n + m + len(shape) + 4 + eb, expect="transpose")
    assert p["src_view_bytes"] == 4 * eb and p["src_step"] == 4, p


@pytest.mark.parametrize("eb,n", [(1, 8192), (2, 8192), (4, 4096)])
def test_stride4_source_read_in_groups_full_size(eb, n):
    """Every 4th element of an n x 4n matrix, transposed (int8 and fp16 8192 x 8192 from 8192 x
    32768, fp32 4096 x 4096 from 4096 x 16384)."""
    p = _check((n, n), (4 * n, 4), (1, n), eb, seed=eb + 4000, expect="transpose")
    assert p["src_view_bytes"] == 4 * eb, p


@pytest.mark.parametrize("k,eb", [(2, 1), (4, 1), (4, 2), (4, 4)])
def test_pairs_and_groups_random(k, eb):
    """Random transposes from stride-2 (int8) and stride-4 (int8, fp16, fp32) sources on the pair
    and group paths: random extents (ragged against the tiles), row pitches and offsets (multiples
    of k; for k = 2 odd offsets too), rows in either order, with or without a batch mode."""
    rng = np.random.default_rng(900 + k + 10 * eb)
    for case in range(12):
        n = int(rng.integers(512, 2200))
        m = int(rng.integers(64, 600))
        pitch = k * m + k * int(rng.integers(0, 40))
        soff = k * int(rng.integers(0, 50)) + (int(rng.integers(0, 2)) if k == 2 else 0)
        batch = int(rng.integers(1, 4)) if case % 3 == 2 else 0
        if case % 4 == 3:  # rows in reverse order
            shape, ss, ds = (n, m), (-pitch, k), (1, n)
            soff += (n - 1) * pitch
        elif batch:
            shape, ss, ds = (batch, n, m), (n * pitch + k * 8, pitch, k), (n * m, 1, n)
        else:
            shape, ss, ds = (n, m), (pitch, k), (1, n)
        p = _check(shape, ss, ds, eb, s_off=soff, seed=case * 7 + k + eb, expect="transpose")
        assert p["src_view_bytes"] == k * eb and p["src_step"] == k, (shape, ss, soff, p)


def test_int8_stride4_words_not_taken_off_word_boundaries():
    """A source offset or a row stride that is not a multiple of 4 keeps the stride-4 tile of
    1-byte elements; same bytes."""
    p = _check((700, 130), (524, 4), (1, 700), 1, s_off=2, seed=78, expect="transpose")
    assert p["src_view_bytes"] == 1 and p["src_step"] == 4, p
    p = _check((700, 130), (522, 4), (1, 700), 1, s_off=0, seed=79, expect="transpose")
    assert p["src_view_bytes"] == 1 and p["src_step"] == 4, p


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
@pytest.mark.parametrize("k", [2, 3, 4, -1, -2, -3, -4])
@pytest.mark.parametrize("n,m,pitch,soff", [(40, 48, 200, 0), (37, 69, 300, 3), (5, 16, 64, 1), (300, 515, 2100, 7),
                                            (2, 3, 13, 0), (129, 1, 9, 2)])
def test_rows_gathered_from_strided_source(eb, k, n, m, pitch, soff):
    """A destination contiguous along rows whose source elements lie k apart (a strided slice
    written out densely; k < 0: a flipped row): whole 16-byte destination vectors gathered from
    the source bytes between their first and last element, a row's short last vector moved back
    over its neighbour; ragged rows, odd offsets and rows shorter than one vector."""
    pitch = max(pitch, (m - 1) * abs(k) + 1)
    if k < 0:
        soff += (m - 1) * -k  # each row's first element is its highest-addressed one
    p = _check((n, m), (pitch, k), (m, 1), eb, s_off=soff, seed=n * m + k + eb)
    if m > 1:
        assert p["path_name"] == "rows" and p["src_step"] == k and p["vec_bytes"] == 16, p


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_rows_gathered_batched_and_padded(eb):
    """Gathered rows under two outer modes, a padded destination pitch and a destination offset;
    then every other column of a matrix at full width (the 8192 x 8192 slice [1:8191, 0:8190:2]
    written out densely, 1-byte elements only: the others at 1024 x 1024)."""
    p = _check((3, 21, 77), (21 * 400, 400, 3), (21 * 90, 90, 1), eb, s_off=5, d_off=2, seed=eb + 100)
    assert p["path_name"] == "rows" and p["src_step"] == 3, p
    n = 8192 if eb == 1 else 1024
    p = _check((n - 2, (n - 1) // 2), (n, 2), ((n - 1) // 2, 1), eb, s_off=n, src_elems=n * n, seed=eb + 200)
    assert p["path_name"] == "rows" and p["src_step"] == 2, p


def test_rows_gather_limits():
    """Source strides beyond 4 either way, and 16-byte elements, stay on the element-wise path."""
    p = _check((50, 40), (300, 5), (40, 1), 1, seed=5, expect="guarded_rows")
    assert p["src_step"] == 0
    _check((50, 40), (300, -5), (40, 1), 1, s_off=200, seed=7, expect="guarded_rows")
    _check((50, 40), (200, 2), (40, 1), 16, seed=6, expect="guarded_rows")
    _check((50, 40), (200, -1), (40, 1), 16, s_off=39, seed=8, expect="guarded_rows")


def test_rows_flipped_at_full_width():
    """torch.flip along the last dimension of an 8192 x 8192 matrix (bytes and floats), and along
    both dimensions."""
    n = 8192
    for eb in (1, 4):
        p = _check((n, n), (n, -1), (n, 1), eb, s_off=n - 1, src_elems=n * n, seed=eb + 300)
        assert p["path_name"] == "rows" and p["src_step"] == -1, p
    p = _check((n, n), (-n, -1), (n, 1), 2, s_off=n * n - 1, src_elems=n * n, seed=303)
    assert p["path_name"] == "rows" and p["src_step"] == -1, p


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n,m,pitch,soff", [(40, 30, 60, 0), (129, 67, 140, 3), (64, 64, 128, 0), (33, 300, 601, 1),
                                            (7, 5, 11, 0), (300, 257, 515, 2)])
def test_transpose_stride2_source(eb, n, m, pitch, soff):
    """Source columns two elements apart (a [.., ::2] slice): each vector is read as two
    contiguous ones and compacted; a row's last vector element by element."""
    p = _check((n, m), (pitch, 2), (1, n), eb, s_off=soff, seed=n * m + eb, expect="transpose")
    assert p["src_step"] == 2


@pytest.mark.parametrize("eb,k", [(1, 3), (1, 4), (2, 3), (2, 4), (4, 3)])
@pytest.mark.parametrize("n,m,pitch,soff", [(40, 30, 130, 0), (129, 67, 300, 3), (64, 64, 260, 0), (33, 300, 1201, 1),
                                            (7, 5, 23, 0), (300, 257, 1030, 2)])
def test_transpose_stride34_source(eb, k, n, m, pitch, soff):
    """Source columns three or four elements apart (at most 12 bytes): each whole vector is read
    as the 16-byte loads of the bytes between its first and last element and compacted; a row's
    last vector element by element."""
    p = _check((n, m), (pitch, k), (1, n), eb, s_off=soff, seed=n * m + eb + k, expect="transpose")
    assert p["src_step"] == k


@pytest.mark.parametrize("eb,k", [(1, -1), (2, -1), (4, -1), (8, -1), (16, -1), (1, -2), (4, -2), (16, -2), (1, -3),
                                  (2, -4), (4, -3)])
@pytest.mark.parametrize("n,m,pitch", [(40, 30, 130), (129, 67, 300), (64, 64, 260), (300, 257, 1030), (7, 5, 23)])
def test_transpose_reversed_source_columns(eb, k, n, m, pitch):
    """Source columns in reverse order (k = -1: the column index is reversed by the planner, the
    destination rows then run backwards; k = -2 to -4, reversed and strided: each whole vector is
    read as the 16-byte loads of the bytes between its lowest- and highest-addressed element and
    reordered; a row's last vector element by element)."""
    soff = (m - 1) * -k + 2
    p = _check((n, m), (pitch, k), (1, n), eb, s_off=soff, seed=n * m + eb - k, expect="transpose")
    assert p["src_step"] == (1 if k == -1 else k)


def test_rotate90_full_size():
    """torch.rot90 of an 8192 x 8192 matrix (the transpose of the column-flipped matrix), at
    every width: the reversed source columns become an aligned transpose into destination rows
    that run backwards."""
    n = 8192
    for eb in (1, 2, 4, 8, 16):
        m = n if eb <= 4 else n // 4
        p = _check((m, m), (-1, m), (m, 1), eb, s_off=m - 1, src_elems=m * m, seed=eb + 400, expect="transpose")
        assert p["src_step"] == 1 and p["unaligned"] == 0 and p["dst_stride"][0] == -m, p


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_reversed_modes(eb):
    """Modes walked backwards: into a row-flipped destination (the source contiguous: gathered
    rows reversed), a destination rotated by 90 degrees (an ordinary transpose after the planner
    reverses the mode), both sides flipped the same way (one contiguous copy), and the rows
    reversed on both sides."""
    n, m = 300, 257
    p = _check((n, m), (m, 1), (m, -1), eb, d_off=m - 1, seed=eb + 500)
    assert p["path_name"] == ("guarded_rows" if eb == 16 else "rows"), p
    p = _check((n, m), (m, 1), (-1, n), eb, d_off=n - 1, seed=eb + 501, expect="transpose")
    assert p["src_step"] == 1, p
    p = _check((n, m), (m, -1), (m, -1), eb, s_off=m - 1, d_off=m - 1, seed=eb + 502, expect="rows")
    assert p["rank"] == 1, p
    p = _check((n, m), (-m, 1), (-m, 1), eb, s_off=(n - 1) * m, d_off=(n - 1) * m, seed=eb + 503, expect="rows")
    assert p["rank"] == 1 and p["src_stride"][0] == 1 and p["dst_stride"][0] == 1, p


def test_transpose_stride34_batched_and_limits():
    for eb, k in ((1, 3), (1, 4), (2, 3), (2, 4), (4, 3)):
        p = _check((3, 37, 45), (37 * 200, 200, k), (37 * 45, 1, 37), eb, seed=eb + k, expect="transpose")
        assert p["src_step"] == k
    # elements more than 12 bytes apart, or stride 5: the guarded tile
    for eb, k in ((4, 4), (8, 3), (16, 3)):
        _check((37, 45), (200, k), (1, 37), eb, seed=eb * k, expect="guarded_tile")
    # stride 5: the guarded tile
    _check((40, 30), (200, 5), (1, 40), 1, seed=9, expect="guarded_tile")


def test_transpose_stride2_batched():
    for eb in (1, 2, 4, 8, 16):
        p = _check((3, 37, 45), (37 * 100, 100, 2), (37 * 45, 1, 37), eb, seed=eb, expect="transpose")
        assert p["src_step"] == 2


@pytest.mark.parametrize("eb", [2, 4, 8, 16])
@pytest.mark.parametrize("n,m", [(512, 128), (256, 64), (1024, 320), (768, 136), (64, 8)])
def test_transpose_tall_tiles(eb, n, m):
    """Tall tiles with 16-byte LDS units and row-tile-first order (2- to 16-byte elements)."""
    min_rows, min_cols = {2: (256, 64), 4: (256, 32), 8: (128, 16), 16: (64, 8)}[eb]
    p = _check((n, m), (m, 1), (1, n), eb, seed=n + 3 * m + eb)
    if n < min_rows or m < min_cols:
        # below the extents where tall tiles are planned: the default tile, or for 8 columns of
        # 8-byte elements the channel interleave
        if (eb, m) == (8, 8):
            assert p["path_name"] == "interleave", p
        else:
            assert p["path_name"] == "transpose" and p["grid_order"] == 0 and p["lds_read_bytes"] == 4, p
    else:
        assert p["path_name"] == "transpose" and p["lds_read_bytes"] == 16 and p["grid_order"] == 1


@pytest.mark.parametrize("eb,n,m,tile", [(1, 8320, 8320, (512, 256)), (2, 16448, 16392, (1024, 64)),
                                          (8, 8208, 8208, (128, 128))])
def test_transpose_128k_tiles_ragged(eb, n, m, tile):
    """128 KiB tiles (one workgroup per CU), with partial tiles along both tile modes (destination
    columns on 128-byte lines: other pitches take the element-aligned plans' configuration)."""
    p = _check((n, m), (m, 1), (1, n), eb, seed=n + m + eb, expect="transpose")
    assert p["lds_bytes"] == 131072 and (p["tile_r"], p["tile_c"]) == tile, p


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n,m", [(64, 64), (96, 272), (272, 48), (16, 1040), (1024, 16), (528, 400)])
def test_transpose_small_ragged(eb, n, m):
    _check((n, m), (m, 1), (1, n), eb, seed=n * 7 + m + eb, expect="transpose")


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n", [72, 68, 66, 65])
def test_transpose_vector_widths(eb, n):
    """n x 64 tiles: the row extent admits 16-, 8- or 4-byte vectors only, or none."""
    plan = _check((n, 64), (64, 1), (1, n), eb, seed=n + eb)
    assert plan["path_name"] == "transpose"
    # the page's plan (strict mode): the widest aligned vector, 16, 8 or 4 bytes
    dt = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}[eb]
    sp = L.tc_plan(((n, 64), (64, 1)), ((n, 64), (1, n)), dt, flags=L.TC_FLAG_STRICT, raise_on_error=False)
    if sp["status"] == L.TC_OK:
        sp = _check((n, 64), (64, 1), (1, n), eb, seed=n + eb, flags=L.TC_FLAG_STRICT, expect="transpose")
        ve = sp["vec_bytes"] // eb
        assert not sp["unaligned"]
        assert n % ve == 0 and all(n % (v // eb) for v in (16, 8) if v > sp["vec_bytes"] and v >= eb)


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
@pytest.mark.parametrize("ch", [2, 3, 4, 8])
@pytest.mark.parametrize("to_planes", [True, False])
def test_interleave_channels(eb, ch, to_planes):
    """A few interleaved channels to planes (NHWC -> NCHW): each lane transposes 16/eb pixels of
    every channel in its registers (where that path is chosen; the way back and the wider pixels
    take the transpose kernel).  With element offsets of 16, and a pixel count that is not a
    multiple of the group."""
    n, h, w = 3, 17, 48
    hw = h * w
    if to_planes:  # (n, h, w, c) interleaved -> (n, c, h, w) planes
        shape, ss, ds = (n, h, w, ch), (hw * ch, w * ch, ch, 1), (ch * hw, w, 1, hw)
    else:          # (n, c, h, w) planes -> (n, h, w, c) interleaved
        shape, ss, ds = (n, ch, h, w), (ch * hw, hw, w, 1), (hw * ch, 1, w * ch, ch)
    interleave = to_planes and (ch * eb <= 12 or eb == 8)
    p = _check(shape, ss, ds, eb, s_off=16, d_off=32, seed=ch * 10 + eb,
               expect="interleave" if interleave else None)
    if interleave:
        assert p["tile_c"] == ch and p["tile_r"] == 16 // eb
    w2 = w - 1  # 17 * 47 pixels: not a multiple of 16 / eb for eb < 8
    hw2 = h * w2
    if to_planes:
        shape, ss, ds = (n, h, w2, ch), (hw2 * ch, w2 * ch, ch, 1), (ch * hw2, w2, 1, hw2)
    else:
        shape, ss, ds = (n, ch, h, w2), (ch * hw2, hw2, w2, 1), (hw2 * ch, 1, w2 * ch, ch)
    _check(shape, ss, ds, eb, seed=ch * 10 + eb + 1)


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
@pytest.mark.parametrize("shape,pitch,soff,doff", [((37, 45), 50, 3, 0), ((64, 64), 65, 65 + 1, 7), ((5, 3), 9, 1, 2),
                                                    ((300, 129), 130, 131, 0), ((2, 33, 70), 71, 5, 3),
                                                    ((1000,), 1, 1, 0), ((4096,), 1, 3, 5), ((7, 1), 2, 1, 0),
                                                    ((300, 128), 130, 131, 0), ((100003,), 1, 1, 0)])
def test_rows_at_element_alignment(eb, shape, pitch, soff, doff):
    """Co-contiguous copies the aligned rule declines (windows of a matrix, odd offsets, row
    lengths that are not multiples of a vector): rows of 16-byte vectors at element alignment, a
    row's short last vector moved back over its neighbour (or, in rows shorter than a vector and
    with buffer accesses, copied in narrower accesses); with the destination vectors on the
    16-byte grid and no short last vector (the (300, 128) shape) as buffer accesses."""
    if len(shape) == 1:
        ss, ds = (1,), (1,)
    elif len(shape) == 2:
        ss, ds = (pitch, 1), (shape[1], 1)
    else:
        ss, ds = (shape[1] * pitch, pitch, 1), (shape[1] * shape[2], shape[2], 1)
    p = _check(shape, ss, ds, eb, s_off=soff, d_off=doff, seed=sum(shape) + eb)
    assert p["path_name"] in ("rows", "roundtrip", "guarded_rows"), p
    if p["path_name"] == "rows" and p["vec_bytes"] == 16:
        assert p["unaligned"] or (soff % (16 // eb) == 0 and doff % (16 // eb) == 0)


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_transpose_with_offsets_and_pitches(eb):
    # source rows of pitch 80 starting at element 16, destination columns of pitch 40 at 8
    _check((32, 64), (80, 1), (1, 40), eb, s_off=16, d_off=8, src_elems=80 * 33, dst_elems=40 * 65,
           seed=eb)


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_sf_tiles_small(eb):
    w = SI.sf_transpose(tiles=37)
    _check(w.src.shape, w.src.stride, w.dst.stride, eb, seed=37 + eb)


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_permute0213_small(eb):
    w = SI.permute0213(b=3, h=5, s=24, d=16)
    _check(w.src.shape, w.src.stride, w.dst.stride, eb, seed=5 + eb)


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_identity_rows_and_roundtrip(eb):
    _check((8, 256), (256, 1), (256, 1), eb, seed=eb, expect="roundtrip" if 8 * 256 * eb <= 16384 else "rows")
    _check((300, 512), (512, 1), (512, 1), eb, seed=eb + 1, expect="rows")
    _check((300, 512), (512, 1), (512, 1), eb, seed=eb + 2, flags=L.TC_FLAG_FORCE_LDS, expect="roundtrip")


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_guarded_paths(eb):
    _check((67, 45), (45, 1), (1, 67), eb, seed=eb, expect="transpose")  # odd: unaligned vectors
    _check((67, 45), (45, 1), (1, 67), eb, seed=eb, flags=L.TC_FLAG_FORCE_GUARDED, expect="guarded_tile")
    _check((40, 30), (60, 2), (1, 40), eb, src_elems=60 * 40, seed=eb)   # strided source
    _check((7, 9), (9, 1), (9, 1), eb, seed=eb)                           # 63 elements: guarded rows
    _check((64, 64), (64, 1), (1, 64), eb, flags=L.TC_FLAG_FORCE_GUARDED, seed=eb, expect="guarded_tile")


@pytest.mark.parametrize("n", [3 * 65536 + 36, (1 << 26) + 4100])
def test_rows_with_negative_layout_offsets(n):
    """Pointers into the middle of the buffers with negative layout offsets (an offset is any
    element displacement from the pointer): every element below the pointers is copied, on the
    rows path with all loads at once (up to 256 MiB) and with paced loads beyond, both with
    buffer bases at the lowest byte of the copy.  The bytes around the destination keep the
    sentinel."""
    import torch
    eb, k, m, pad = 4, 1000, 2048, 4096
    say(f"[gpu] rows n={n} with offsets -{k} / -{m}")
    src = SI.device_bits(torch, n * eb, 17)
    dst = torch.full((n * eb + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    plan = L.tile_copy_ex(src.data_ptr() + k * eb, ((n,), (1,), -k), dst.data_ptr() + pad + m * eb,
                          ((n,), (1,), -m), L.TC_F32)
    torch.cuda.synchronize()
    assert plan["path_name"] == "rows" and plan["vec_bytes"] == 16, plan
    assert torch.equal(dst[pad:pad + n * eb], src)
    assert bool((dst[:pad] == 0xA5).all()) and bool((dst[pad + n * eb:] == 0xA5).all())
    del src, dst
    torch.cuda.empty_cache()


@pytest.mark.parametrize("b,h,sq,d,eb", [(3, 5, 37, 64, 2), (4, 7, 33, 32, 4), (2, 9, 65, 256, 1), (4, 3, 41, 16, 8),
                                         (4, 4, 29, 8, 16), (2, 16, 300, 64, 2)])
def test_permuted_rows_in_source_order(b, h, sq, d, eb):
    """(0,2,1,3) permutes with rows shorter than 1 KiB: the rows grid walks the source order with 2
    vectors per lane (ragged last workgroups); the same copies with a head-reversed destination and
    an offset source."""
    shape = (b, h, sq, d)
    ss = (h * sq * d, sq * d, d, 1)
    ds = (sq * h * d, d, h * d, 1)
    p = _check(shape, ss, ds, eb, seed=b * 100 + d + eb, expect="rows")
    assert p["grid_order"] == 1 and p["load_outer"] == 2, p
    ds_rev = (sq * h * d, -d, h * d, 1)
    n = b * h * sq * d
    p = _check(shape, ss, ds_rev, eb, s_off=16 // eb, d_off=(h - 1) * d, src_elems=n + 16 // eb, dst_elems=n,
               seed=b * 100 + d + eb + 1, expect="rows")
    assert p["grid_order"] == 1, p


def test_rows_and_blocks_with_negative_strides():
    """A row-flipped destination on the rows path (its buffer base is the last row) and a
    negative batch stride on the scale-factor butterfly (global accesses there)."""
    _check((300, 256), (256, 1), (-256, 1), 4, d_off=299 * 256, seed=21, expect="rows")
    _check((1000, 4, 32), (-128, 32, 1), (128, 1, 4), 4, s_off=999 * 128, src_elems=1000 * 128, seed=22,
           expect="shuffle")
    _check((1000, 4, 32), (128, 32, 1), (-128, 1, 4), 4, d_off=999 * 128, dst_elems=1000 * 128, seed=23,
           expect="shuffle")


def test_no_swizzle_flag_same_result():
    plan = _check((256, 256), (256, 1), (1, 256), 4, flags=L.TC_FLAG_NO_SWIZZLE, seed=3)
    assert plan["xor_k"] == 0 and plan["xor_cmask"] == 0


def test_edge_cases():
    import torch
    # empty copies launch nothing and touch nothing
    _check((0, 5), (5, 1), (1, 0), 4, src_elems=1, dst_elems=4, expect="empty")
    # one element (rank 0 and a 1x1 tile)
    _check((), (), (), 4, src_elems=1, dst_elems=1)
    _check((1, 1), (1, 1), (1, 1), 8, src_elems=1, dst_elems=1)
    # negative source stride (row-flipped view) and a broadcast source (stride 0)
    _check((64, 32), (-32, 1), (1, 64), 4, s_off=63 * 32, src_elems=64 * 32, seed=9)
    _check((64, 32), (0, 1), (32, 1), 2, src_elems=32, seed=10)
    # maximum rank, permuted
    shape = (2, 3, 2, 4, 2, 3, 2, 4)
    st = np.cumprod((1,) + shape[:0:-1])[::-1]
    perm = (7, 0, 3, 1, 6, 2, 5, 4)
    dst_st = [0] * 8
    acc = 1
    for k in reversed(perm):
        dst_st[k] = acc
        acc *= shape[k]
    _check(shape, tuple(int(x) for x in st), tuple(dst_st), 4, seed=11)
    # errors: non-injective destination and overlapping buffers
    t = torch.zeros(1024, dtype=torch.float32, device="cuda")
    u = torch.zeros(1024, dtype=torch.float32, device="cuda")
    with pytest.raises(L.TileCopyError) as e:
        L.tile_copy(t, ((32, 32), (32, 1)), u, ((32, 32), (1, 1)), L.TC_F32)
    assert e.value.code == L.TC_E_NONINJECTIVE
    with pytest.raises(L.TileCopyError) as e:
        L.tile_copy(t, ((32, 32), (32, 1)), t.data_ptr() + 64, ((32, 32), (1, 32)), L.TC_F32)
    assert e.value.code == L.TC_E_ALIAS


def test_random_layouts():
    for case, (shape, s_stride, d_stride, eb, src_elems) in enumerate(SI.random_layouts(1234, 60)):
        _check(shape, s_stride, d_stride, eb, src_elems=src_elems, seed=case)


def test_random_layouts_wide():
    """Negative and zero source strides, unit modes with arbitrary strides, offsets, all widths."""
    paths = set()
    for case, (sshape, ss, so, dshape, ds, do, eb, ns, nd) in enumerate(SI.random_layouts_wide(4321, 120)):
        src = _bits(ns * eb, 1000 + case)
        sl, dl = (sshape, ss, so), (dshape, ds, do)
        say(f"[gpu] wide case {case}: src={sl} dst={dl} eb={eb}")
        got, plan = run_copy(src, sl, nd, dl, eb, dtype_code(DT_BY_EB[eb]))
        assert_same(got, oracle_copy(src, sl, nd, dl, eb), eb, f"wide {case}")
        paths.add(plan["path_name"])
    assert len(paths) >= 3, paths


def test_random_layouts_large():
    """Multi-tile copies with ragged edges: padded pitches off the 16- and 128-byte grids, stride-2
    sources, offsets, a small batch mode, every element width (element-aligned and stride-2
    transposes in both grid orders, rows, guarded paths)."""
    paths = set()
    for case, (shape, ss, so, ds, do, eb, ns, nd) in enumerate(SI.random_layouts_large(777, 150)):
        src = _bits(ns * eb, 5000 + case)
        sl, dl = (shape, ss, so), (shape, ds, do)
        say(f"[gpu] large case {case}: src={sl} dst={dl} eb={eb}")
        got, plan = run_copy(src, sl, nd, dl, eb, dtype_code(DT_BY_EB[eb]))
        assert_same(got, oracle_copy(src, sl, nd, dl, eb), eb, f"large {case}")
        paths.add((plan["path_name"], plan["src_step"], plan["grid_order"]))
    assert len(paths) >= 5, paths


def test_random_layouts_steps():
    """Multi-tile copies from sources stepping -4 to -1 or 2 to 4 elements along their innermost
    mode, outer modes and destination modes walked backwards, padded pitches and offsets, every
    element width (gathered rows, stride-2 to -4 and reversed transposes, reversed modes, guarded
    paths)."""
    paths = set()
    for case, (shape, ss, so, ds, do, eb, ns, nd) in enumerate(SI.random_layouts_steps(2468, 120)):
        src = _bits(ns * eb, 7000 + case)
        sl, dl = (shape, ss, so), (shape, ds, do)
        say(f"[gpu] steps case {case}: src={sl} dst={dl} eb={eb}")
        got, plan = run_copy(src, sl, nd, dl, eb, dtype_code(DT_BY_EB[eb]))
        assert_same(got, oracle_copy(src, sl, nd, dl, eb), eb, f"steps {case}")
        paths.add((plan["path_name"], plan["src_step"]))
    assert len(paths) >= 8, paths


def test_adjacent_buffers_are_not_aliases():
    """A destination that starts right after the source's last byte (or ends right before its
    first) shares no byte: the copy runs."""
    import torch
    buf = torch.from_numpy(_bits(3 * 4096, 31)).cuda()
    want = buf[4096:8192].cpu().numpy()
    base = buf.data_ptr()
    lay = ((1024,), (1,))
    L.tile_copy(base + 4096, lay, base + 8192, lay, L.TC_F32)   # dst right after src
    L.tile_copy(base + 4096, lay, base, lay, L.TC_F32)          # dst right before src
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert np.array_equal(out[8192:], want) and np.array_equal(out[:4096], want)


def test_stream_ordering_on_side_stream():
    import torch
    s = torch.cuda.Stream()
    src_h = _bits(512 * 512 * 4, 77)
    src = torch.from_numpy(src_h).cuda()
    dst = torch.full_like(src, 0xA5)
    with torch.cuda.stream(s):
        L.tile_copy(src, ((512, 512), (512, 1)), dst, ((512, 512), (1, 512)), L.TC_F32, stream=s)
    s.synchronize()
    want = oracle_copy(src_h, ((512, 512), (512, 1), 0), 512 * 512, ((512, 512), (1, 512), 0), 4)
    assert_same(dst.cpu().numpy(), want, 4, "side stream")


def test_hip_graph_capture_and_replays():
    """tile_copy can be captured in a graph (it allocates nothing and records no memset): the
    captured transpose, permute and guarded copies replay correctly several times, with eager
    work in between and new source values each time."""
    import torch
    w1 = SI.transpose2d(512, 768, dtype="float32")
    w2 = SI.permute0213(b=2, h=4, s=64, d=32)
    w3 = SI.sweep_odd("float16", 67, 45)
    ws = [w1, w2, w3]
    srcs = [torch.from_numpy(SI.make_source(w)).cuda() for w in ws]
    dsts = [torch.full((SI.storage_elems(w, "dst") * w.eb,), 0xA5, dtype=torch.uint8, device="cuda") for w in ws]
    lays = [(L.make_layout(w.src.shape, w.src.stride, w.src.offset), L.make_layout(w.dst.shape, w.dst.stride, w.dst.offset))
            for w in ws]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # plans are made (and cached) before capture
        for w, a, b, (sl, dl) in zip(ws, srcs, dsts, lays):
            L.tile_copy(a, sl, b, dl, L.DTYPE_BY_NAME[w.dtype], stream=s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for w, a, b, (sl, dl) in zip(ws, srcs, dsts, lays):
            L.tile_copy(a, sl, b, dl, L.DTYPE_BY_NAME[w.dtype], stream=s)
    for rep in range(4):
        for i, w in enumerate(ws):  # new inputs and a fresh sentinel through eager work
            srcs[i].copy_(torch.from_numpy(SI.make_values(w.dtype, "bits", srcs[i].numel() // w.eb, 100 + rep)).cuda())
            dsts[i].fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, a, b in zip(ws, srcs, dsts):
            want = oracle_copy(a.cpu().numpy(), (w.src.shape, w.src.stride, w.src.offset), SI.storage_elems(w, "dst"),
                               (w.dst.shape, w.dst.stride, w.dst.offset), w.eb)
            assert_same(b.cpu().numpy(), want, w.eb, f"graph replay {rep} {w.name}")
