"""Host-side tests of the library (no GPU): the C ABI loads and exports what the header declares,
the layout algebra and planner decide as the pages prescribe, and the planner's partition and
LDS swizzle agree with the oracle's independent re-derivation."""

import os
import re
import subprocess

import numpy as np
import pytest

import layout_permuting_copy_amd as L
import synth_inputs as SI
from conftest import ROOT


def _plan(w, flags=0, align=16):
    return L.tc_plan((w.src.shape, w.src.stride, w.src.offset), (w.dst.shape, w.dst.stride, w.dst.offset),
                     L.DTYPE_BY_NAME[w.dtype], flags=flags, ptr_align=align, raise_on_error=False)


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "tile_copy.h")).read()
    declared = set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", header, re.M))
    assert {"tile_copy", "tile_copy_ex", "tc_plan", "tc_last_error", "tc_set_flags", "tc_get_flags",
            "tc_layout_slice", "tc_version"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert declared <= exported, declared - exported
    lib = L.load_library()
    for name in declared:
        assert hasattr(lib, name)
    assert L.tc_version() >= 100


def test_abi_struct_layout_matches_header():
    """Compile a C program against the header: every field offset of tc_layout and tc_plan_info
    and both sizes must equal the ctypes structures of the binding."""
    import ctypes
    import tempfile
    fields = [("tc_plan_info", n) for n, _ in L.TcPlanInfo._fields_] + [("tc_layout", n) for n, _ in L.TcLayout._fields_]
    body = "".join(f'printf("%zu\\n", offsetof({st}, {f}));' for st, f in fields)
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "tile_copy.h"\n'
           'int main(){printf("%zu\\n%zu\\n", sizeof(tc_layout), sizeof(tc_plan_info));' + body + 'return 0;}\n')
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "s.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "s")
        subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        got = [int(x) for x in subprocess.check_output([exe]).split()]
    want = [ctypes.sizeof(L.TcLayout), ctypes.sizeof(L.TcPlanInfo)]
    want += [getattr(L.TcPlanInfo if st == "tc_plan_info" else L.TcLayout, f).offset for st, f in fields]
    assert got == want


def test_workload_paths_and_declines():
    expect = {"tile32x32_f32_roundtrip": "roundtrip", "sf_transpose": "shuffle", "transpose_16384": "transpose",
              "permute0213": "rows", "transpose_8192x8192": "transpose", "slice_rows_": "rows",
              "slice_": "transpose", "transpose_8191x8190": "transpose"}
    for w in SI.all_workloads():
        p = _plan(w)
        assert p["status"] == 0, (w.name, p["error"])
        key = next(k for k in expect if w.name.startswith(k))
        # 16-byte elements of the slice written out densely: one element per access already
        wide_rows = key == "slice_rows_" and w.eb == 16
        assert p["path_name"] == ("guarded_rows" if wide_rows else expect[key]), (w.name, p["path_name"])
        if p["path_name"] == "transpose":
            assert p["write_conflicts"] == 0 and p["read_conflicts"] == 0, w.name
        declined = w.name.startswith(("slice_", "transpose_8191x8190"))
        assert p["declined"] == int(declined), w.name
        # (16-byte elements of the odd transpose are whole aligned vectors: the aligned kernels
        # run it, with the page's reason kept)
        whole = w.name.startswith("transpose_8191x8190") and w.eb == 16
        assert p["unaligned"] == int(declined and not wide_rows and not whole), w.name
        # the stride-2 slice reads every vector as two contiguous ones (transposed), or gathers
        # each destination vector from its source span (rows)
        step = 0 if wide_rows else 2 if w.name.startswith("slice_") else 1 if p["path_name"] == "transpose" else 0
        assert p["src_step"] == step, (w.name, p["src_step"])
        if declined:
            assert "not divisible by the thread count 64" in p["reason"]
            s = _plan(w, flags=L.TC_FLAG_STRICT)
            assert s["status"] == L.TC_E_DECLINED and "no integer solution" in s["error"]


def test_canonical_modes_of_the_workloads():
    p = _plan(SI.sf_transpose())
    # (65536, 2) merge into one batch mode of stride 128 on both sides; the 4x32 block stays
    assert p["extent"] == (131072, 32, 4)
    assert p["src_stride"] == (128, 1, 32) and p["dst_stride"] == (128, 4, 1)
    p = _plan(SI.permute0213())
    assert p["extent"] == (32, 2048, 32, 128) and p["dst_stride"] == (8388608, 4096, 128, 1)
    p = _plan(SI.tile32_roundtrip())
    assert p["extent"] == (1024,) and p["src_stride"] == (1,)


def test_roundtrip_partition_matches_oracle_gmem_smem():
    """The 32x32 fp32 round trip on one wave64: the oracle's [outer, threads, vec] split of the
    same copy (global side = source, shared side = an identical LDS tile) gives the plan."""
    from oracle import ref as R
    w = SI.tile32_roundtrip()
    p = _plan(w)
    o = R.gmem_smem_partition(R.layout(w.src.shape, w.src.stride), R.layout((32, 32)), 64, 4)
    assert (p["threads"], p["load_outer"], p["vec_bytes"]) == (o["threads"], o["outer"], o["copy_bytes"])
    assert o["g_lin"][1][:3] == [256, 260, 264]  # f*256 + tid*4 on a wave64


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
def test_vector_width_rule(eb):
    dt = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}[eb]
    for n in (72, 68, 66, 65, 64):
        p = L.tc_plan(((n, 64), (64, 1)), ((n, 64), (1, n)), dt, raise_on_error=False)
        widths = [v for v in (16, 8, 4) if v >= eb and n % (v // eb) == 0 and 64 % (v // eb) == 0]
        if widths:
            # strict mode: the page's plan, the widest vector that divides
            s = L.tc_plan(((n, 64), (64, 1)), ((n, 64), (1, n)), dt, flags=L.TC_FLAG_STRICT, raise_on_error=False)
            assert s["path_name"] == "transpose" and s["vec_bytes"] == widths[0], (eb, n, s["vec_bytes"])
            assert not s["unaligned"]
            # 64-byte int8 source rows leave the XOR search a few cycles short of conflict-free:
            # strict mode declines with the reason
            assert s["status"] == L.TC_OK or "XOR swizzle" in s["reason"], s["reason"]
            if widths[0] == 16:
                assert p["path_name"] == "transpose" and p["vec_bytes"] == 16 and not p["unaligned"]
                # (the cheapest swizzle runs, and the plan says why it is not the page's plan)
                assert not p["declined"] or ("XOR swizzle" in p["reason"] and p["write_conflicts"] + p["read_conflicts"] > 0)
            else:  # by default, 16-byte vectors at element alignment instead of narrower ones
                assert p["path_name"] == "transpose" and p["vec_bytes"] == 16 and p["unaligned"], (eb, n, p)
                assert not p["declined"] and "allows only %d-byte" % widths[0] in p["reason"], p["reason"]
        else:  # the page's rule declines; the transpose runs with vectors at element alignment
            assert p["path_name"] == "transpose" and p["unaligned"] and "no vector" in p["reason"]
            s = L.tc_plan(((n, 64), (64, 1)), ((n, 64), (1, n)), dt, flags=L.TC_FLAG_STRICT, raise_on_error=False)
            assert s["status"] == L.TC_E_DECLINED
    # pointer alignment limits the vector of the page's plan
    p = L.tc_plan(((64, 64), (64, 1)), ((64, 64), (1, 64)), dt, flags=L.TC_FLAG_STRICT, ptr_align=max(eb, 4),
                  raise_on_error=False)
    assert p["vec_bytes"] == max(eb, 4) or p["path_name"] != "transpose"


def test_errors():
    f32 = L.TC_F32
    p = L.tc_plan(((4, 32), (32, 1)), ((32, 4), (4, 1)), f32, raise_on_error=False)
    assert p["status"] == L.TC_E_EXTENT and "extent mismatch" in p["error"]
    p = L.tc_plan(((4, 32), (32, 1)), ((4, 32), (1, 1)), f32, raise_on_error=False)
    assert p["status"] == L.TC_E_NONINJECTIVE
    p = L.tc_plan(((4, 32), (32, 1)), ((4, 32), (32, 1)), 99, raise_on_error=False)
    assert p["status"] == L.TC_E_DTYPE
    p = L.tc_plan(((4, 32), (32, 1)), ((4, 32), (32, 1)), f32, flags=0x100, raise_on_error=False)
    assert p["status"] == L.TC_E_ARG
    bad = L.make_layout((4, 32), (32, 1))
    bad.rank = 9
    p = L.tc_plan(bad, ((4, 32), (32, 1)), f32, raise_on_error=False)
    assert p["status"] == L.TC_E_RANK
    p = L.tc_plan(((-1, 32), (32, 1)), ((4, 32), (32, 1)), f32, raise_on_error=False)
    assert p["status"] == L.TC_E_EXTENT
    # unit modes are ignored on both sides (TIRx: equal non-unit extents)
    p = L.tc_plan(((1, 4, 1, 32), (7, 32, 9, 1)), ((4, 32), (1, 4)), f32)
    assert p["extent"] == (32, 4)
    with pytest.raises(L.TileCopyError):
        L.tc_set_flags(0x400)
    old = L.tc_set_flags(L.TC_FLAG_STRICT)
    assert L.tc_get_flags() == L.TC_FLAG_STRICT
    L.tc_set_flags(old)


def test_null_pointers_rejected_without_gpu():
    import ctypes
    lib = L.load_library()
    lay = L.make_layout((4, 32))
    assert lib.tile_copy(None, ctypes.byref(lay), None, ctypes.byref(lay), L.TC_F32, None) == L.TC_E_NULL
    assert "null" in L.tc_last_error()
    # misaligned base pointer (a fake address; nothing is launched when the check fails)
    assert lib.tile_copy(ctypes.c_void_p(0x1002), ctypes.byref(lay), ctypes.c_void_p(0x10000),
                         ctypes.byref(lay), L.TC_F32, None) == L.TC_E_ALIGN


@pytest.mark.parametrize("n", [5, 8, 13])
def test_layout_slice_matches_python_slicing(n):
    rng = np.random.default_rng(n)
    base = np.arange(n * (n + 3)).reshape(n, n + 3)
    for _ in range(200):
        sl = []
        for ext in base.shape:
            step = int(rng.choice([-3, -2, -1, 1, 2, 3]))
            a, b = (int(x) for x in rng.integers(-ext - 2, ext + 3, size=2))
            sl.append((a, b, step))
        view = base[tuple(slice(*s) for s in sl)]
        out = L.tc_layout_slice(((n, n + 3), (n + 3, 1), 0), [s[0] for s in sl], [s[1] for s in sl],
                                [s[2] for s in sl])
        shape, stride, off = out.as_tuple()
        assert shape == view.shape
        if view.size:
            idx = np.indices(shape).reshape(2, -1)
            flat = off + (np.array(stride)[:, None] * idx).sum(0)
            assert np.array_equal(base.reshape(-1)[flat], view.reshape(-1))
    with pytest.raises(L.TileCopyError):
        L.tc_layout_slice(((4,), (1,), 0), [0], [4], [0])


def test_config5_slice_through_tc_layout_slice():
    w = SI.sweep_slice("int8")
    full = L.make_layout((8192, 8192), (8192, 1))
    out = L.tc_layout_slice(full, [1, 0], [8191, 8190], [1, 2])
    assert out.as_tuple() == (w.src.shape, w.src.stride, w.src.offset)


def _transposing(dtypes=("int8", "float16", "bfloat16", "float32", "float64", "int4vec")):
    ws = [SI.sf_transpose()]
    for dt in dtypes:
        ws.append(SI.transpose2d(4096, 8192, dtype=dt, seed=1, values="bits"))
    return ws


@pytest.mark.parametrize("w", _transposing(), ids=lambda w: w.name)
def test_swizzle_matches_oracle_rederivation(w):
    """The oracle re-derives the LDS swizzle for the planner's tile geometry by brute force
    (TileLang partition of each phase, gfx950 bank model, same search order): the planner's
    choice must be the oracle's, and conflict-free under the oracle's own counting."""
    from oracle import ref as R
    p = _plan(w, flags=L.TC_FLAG_NO_SHUFFLE)  # the SF tiles' LDS plan, not their register butterfly
    assert p["path_name"] == "transpose"
    geo = dict(eb=p["elem_bytes"], vb=p["vec_bytes"], TR=p["tile_r"], TC=p["tile_c"], NB=p["tile_b"],
               U=p["lds_read_bytes"], NT=p["threads"])
    o = R.lds_tile_swizzle(**geo)
    assert o is not None
    assert (o["k"], o["shift"], o["tbit"], o["cshift"], o["cmask"]) == (
        p["xor_k"], p["xor_shift"], p["xor_tbit"], p["xor_cshift"], p["xor_cmask"])
    assert R.lds_tile_conflicts(**geo, k=p["xor_k"], shift=p["xor_shift"], tbit=p["xor_tbit"],
                                cshift=p["xor_cshift"], cmask=p["xor_cmask"]) == (0, 0)


def test_wave_locality_matches_oracle():
    """The planner drops the workgroup barrier only where the oracle's enumeration of both
    partitions shows every wave reading back its own LDS units."""
    from oracle import ref as R
    ws = _transposing() + [SI.sf_transpose(tiles=37)]
    cases = [(w.src.shape, w.src.stride, w.src.offset, w.dst.stride, w.dst.offset, L.DTYPE_BY_NAME[w.dtype]) for w in ws]
    dts = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}
    w = SI.sf_transpose(tiles=37)
    cases += [(w.src.shape, w.src.stride, 0, w.dst.stride, 0, dt) for dt in dts.values()]
    cases += [(sh, ss, 0, ds, 0, dts[eb]) for sh, ss, ds, eb, _ in SI.random_layouts(5, 120)]
    seen = {True: 0, False: 0}
    for shape, ss, so, ds, do, dt in cases:
        p = L.tc_plan((shape, ss, so), (shape, ds, do), dt, flags=L.TC_FLAG_NO_SHUFFLE, raise_on_error=False)
        if p["path_name"] != "transpose":
            continue
        o = R.tile_wave_local(p["elem_bytes"], p["vec_bytes"], p["tile_r"], p["tile_c"], p["tile_b"], p["threads"],
                              U=p["lds_read_bytes"])
        # the planner may keep the barrier where it holds no wave-local kernel, never the reverse
        assert p["wave_local"] <= int(o), (shape, ss, ds, dt)
        seen[bool(p["wave_local"])] += 1
    assert seen[True] >= 2 and seen[False] >= 5
    sf = _plan(SI.sf_transpose(), flags=L.TC_FLAG_NO_SHUFFLE)
    assert sf["wave_local"] == 1


def test_no_swizzle_has_conflicts_for_transposes():
    """Without the swizzle the 2-D transposes pay bank conflicts (which the swizzle removes):
    the planner's simulation and the oracle's agree on the count."""
    from oracle import ref as R
    w = SI.transpose2d(4096, 4096, dtype="float32", seed=1)
    p = _plan(w, flags=L.TC_FLAG_NO_SWIZZLE)
    assert p["xor_k"] == 0 and p["read_conflicts"] > 0
    geo = dict(eb=4, vb=16, TR=p["tile_r"], TC=p["tile_c"], NB=p["tile_b"], U=p["lds_read_bytes"], NT=p["threads"])
    assert R.lds_tile_conflicts(**geo) == (p["write_conflicts"], p["read_conflicts"])


# (vector bytes, tile bytes, threads) of the transpose kernel instances the library is built with
TRANSPOSE_INSTANCES = {(16, t, n) for t, n in [(8192, 256), (16384, 256), (16384, 512), (32768, 256), (32768, 512),
                                                (65536, 256), (65536, 512), (65536, 1024), (131072, 512),
                                                (131072, 1024)]} | {(8, 16384, 256), (4, 16384, 256)}


def test_every_plan_has_a_kernel_instance():
    """Random layouts and small 2-D transposes of every width plan without error, and every
    transpose plan names a configuration the library holds a kernel for."""
    dts = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}
    cases = [(shape, ss, ds, eb) for seed in (1234, 7, 99) for shape, ss, ds, eb, _ in SI.random_layouts(seed, 200)]
    for eb in dts:
        for n in (1, 3, 4, 16, 31, 64, 65, 100, 128, 129, 256, 1000, 4096):
            for m in (1, 2, 5, 16, 64, 67, 256, 300, 2048):
                cases.append(((n, m), (m, 1), (1, n), eb))
    cases += [((16384, 16384), (16384, 1), (1, 16384), 2), ((8192, 8192), (8192, 1), (1, 8192), 1),
              ((8192, 8192), (8192, 1), (1, 8192), 8)]
    seen = set()
    for shape, ss, ds, eb in cases:
        p = L.tc_plan((shape, ss), (shape, ds), dts[eb], raise_on_error=False)
        assert p["status"] == L.TC_OK, (shape, ss, ds, eb, p["error"])
        if p["path_name"] == "transpose":
            cfg = (p["vec_bytes"], p["lds_bytes"], p["threads"])
            assert cfg in TRANSPOSE_INSTANCES, (shape, ss, ds, eb, cfg)
            seen.add(cfg)
    assert len(seen) >= 5


def test_interior_kernel_only_for_exact_tilings():
    """The kernel without guarded code runs only where every tile lies inside the copy (and not
    for 16-byte elements, which measured faster with the guarded kernel)."""
    def edge(shape, ss, ds, dt, soff=0):
        p = L.tc_plan((shape, ss, soff), (shape, ds), dt)
        assert p["path_name"] == "transpose", p
        return p["edge_tiles"]
    assert edge((16384, 16384), (16384, 1), (1, 16384), L.TC_BF16) == 0
    assert edge((16384, 16384), (16384, 1), (1, 16384), L.TC_F32) == 0
    assert edge((8192, 8192), (8192, 1), (1, 8192), L.TC_I8) == 0
    assert edge((4096, 1024), (1024, 1), (1, 4096), L.TC_F64) == 0
    assert edge((16392, 16392), (16392, 1), (1, 16392), L.TC_BF16) == 1   # partial tiles
    assert edge((1000, 600), (600, 1), (1, 1000), L.TC_F32) == 1
    assert edge((8192, 8192), (8192, 1), (1, 8192), L.TC_B128) == 1        # 16-byte elements
    assert edge((8191, 8190), (8190, 1), (1, 8191), L.TC_F16) == 1         # element-aligned vectors
    assert edge((8190, 4095), (8192, 2), (1, 8190), L.TC_F16, 8192) == 1   # stride-2 source


def test_load_caps_of_the_tall_tiles():
    """The tall tiles of 1- and 2-byte elements keep at most 2 loads in flight per lane (also where
    only the destination is off the cache lines or at element alignment, the source rows on them);
    fp32, fp64, 16-byte elements and the plans with the source at element alignment keep all of
    them in flight (0)."""
    def cap(shape, ss, ds, dt):
        p = L.tc_plan((shape, ss), (shape, ds), dt)
        assert p["path_name"] == "transpose", p
        return p["loads_in_flight"]
    assert cap((16384, 16384), (16384, 1), (1, 16384), L.TC_BF16) == 2
    assert cap((8192, 8192), (8192, 1), (1, 8192), L.TC_F16) == 2
    assert cap((8192, 8192), (8192, 1), (1, 8192), L.TC_I8) == 2
    assert cap((8192, 8192), (8192, 1), (1, 8192), L.TC_F64) == 0
    assert cap((16384, 16384), (16384, 1), (1, 16384), L.TC_F32) == 0
    assert cap((8192, 8192), (8192, 1), (1, 8192), L.TC_B128) == 0
    assert cap((8191, 8190), (8190, 1), (1, 8191), L.TC_F16) == 0        # element-aligned vectors
    assert cap((8176, 8192), (8192, 1), (1, 8176), L.TC_U8) == 2         # int8, destination off the lines
    assert cap((8191, 8192), (8192, 1), (1, 8191), L.TC_U8) == 2         # int8, destination at element alignment
    assert cap((8191, 8190), (8190, 1), (1, 8191), L.TC_U8) == 0         # int8, both sides at element alignment
    assert cap((8192, 4096), (4096, 1), (1, 8192), L.TC_F64) == 0


def test_super_tile_extents():
    """The XCD super-tile extents the plans report: 16 x 2 tiles for the int8 tall tiles (aligned,
    destination off the lines, destination at element alignment), 8 x 8 for the element-aligned
    int8 and fp64 plans; 0 x 0 where the grid is not in super-tile order."""
    def sup(shape, ss, ds, dt):
        p = L.tc_plan((shape, ss), (shape, ds), dt)
        return p["grid_order"], p["super_rows"], p["super_cols"]
    assert sup((8192, 8192), (8192, 1), (1, 8192), L.TC_I8) == (2, 16, 2)
    assert sup((16384, 16384), (16384, 1), (1, 16384), L.TC_I8) == (2, 16, 2)
    assert sup((8176, 8192), (8192, 1), (1, 8176), L.TC_U8) == (2, 16, 2)
    assert sup((8191, 8192), (8192, 1), (1, 8191), L.TC_U8) == (2, 16, 2)
    assert sup((8191, 8190), (8190, 1), (1, 8191), L.TC_U8) == (2, 8, 8)
    assert sup((8191, 8190), (8190, 1), (1, 8191), L.TC_F64) == (2, 8, 8)
    assert sup((16384, 16384), (16384, 1), (1, 16384), L.TC_F32) == (1, 0, 0)
    assert sup((8192, 8192), (8192, 1), (1, 8192), L.TC_F16) == (1, 0, 0)


def test_permuted_rows_walk_the_source_order():
    """Rows shorter than 1 KiB whose outer modes are ordered differently on the two sides run in
    source order with 2 vectors per lane (grid_order 1); longer rows, and copies whose sides agree,
    keep the destination order with 4 paced vectors (grid_order 0)."""
    def rows(w):
        p = L.tc_plan((w.src.shape, w.src.stride), (w.dst.shape, w.dst.stride), L.DTYPE_BY_NAME[w.dtype])
        assert p["path_name"] == "rows", p
        return p["grid_order"], p["load_outer"]
    assert rows(SI.permute0213()) == (1, 2)
    assert rows(SI.permute0213(d=32, dtype="float32")) == (1, 2)
    assert rows(SI.permute0213(b=8, h=16, s=1024, d=512)) == (0, 4)          # 1 KiB rows
    box = SI.Workload("box", SI.Side((64, 128, 256), (65536, 512, 1)), SI.Side((64, 128, 256), (32768, 256, 1)),
                      "float32", "bits", 1)
    assert rows(box) == (0, 4)                                                 # both sides in one order
    # the split into launches follows the source-ordered outermost mode
    p = L.tc_plan(((2, 64, 1 << 20, 128), (64 << 27, 128 << 20, 128, 1)),
                  ((2, 64, 1 << 20, 128), (64 << 27, 128, 128 * 64, 1)), L.TC_BF16)
    assert p["path_name"] == "rows" and p["grid_order"] == 1 and p["status"] == 0, p


def test_copies_beyond_2_31_vectors_plan():
    """Contiguous and shuffle copies of 2^31 vectors or more (32 GiB and up, sized for a 288 GB
    GPU) plan as several launches; only a single outermost index of more than 2^30 vectors is
    out of range."""
    n = 1 << 33  # fp32 elements: 2^31 16-byte vectors
    p = L.tc_plan(((n,), (1,)), ((n,), (1,)), L.TC_F32)
    assert p["path_name"] == "rows" and p["workgroups"] == (1 << 31) // (p["threads"] * p["load_outer"])
    # two non-mergeable rows of 2^32 elements (2^30 vectors each): fits one launch per row
    p = L.tc_plan(((2, 1 << 32), ((1 << 32) + 64, 1)), ((2, 1 << 32), (1 << 32, 1)), L.TC_F32)
    assert p["status"] == L.TC_OK and p["path_name"] == "rows", p["error"]
    # a row of 2^33 elements (2^31 vectors) under an outer mode: out of range
    p = L.tc_plan(((2, 1 << 33), ((1 << 33) + 64, 1)), ((2, 1 << 33), (1 << 33, 1)), L.TC_F32, raise_on_error=False)
    assert p["status"] == L.TC_E_RANGE and "outermost" in p["error"]
    # 2^26 scale-factor blocks of 4 x 32 fp32: 2^31 vectors on the register butterfly
    b = 1 << 26
    p = L.tc_plan(((b, 4, 32), (128, 32, 1)), ((b, 4, 32), (128, 1, 4)), L.TC_F32)
    assert p["path_name"] == "shuffle" and p["workgroups"] == (b * 32) // (256 * 8)
    # element-wise guarded rows of 2^31 elements
    p = L.tc_plan(((1 << 31,), (3,)), ((1 << 31,), (2,)), L.TC_I8)
    assert p["status"] == L.TC_OK and p["path_name"] == "guarded_rows", p


def test_window_copies_take_element_aligned_rows():
    """A [1:8191, 1:8191] window of an 8192^2 matrix into a dense buffer: the page's rule declines
    (no integer split), strict mode reports it, the default runs rows of 16-byte vectors at element
    alignment; an odd element offset on a 1-D copy likewise."""
    for dt in (L.TC_I8, L.TC_F16, L.TC_F32, L.TC_F64):
        src, dst = ((8190, 8190), (8192, 1), 8193), ((8190, 8190), (8190, 1))
        p = L.tc_plan(src, dst, dt)
        assert p["path_name"] == "rows" and p["unaligned"] and p["vec_bytes"] == 16, p
        eb = p["elem_bytes"]
        assert p["workgroups"] == -(-8190 * -(-8190 // (16 // eb)) // (p["threads"] * 4))
        assert L.tc_plan(src, dst, dt, flags=L.TC_FLAG_STRICT, raise_on_error=False)["status"] == L.TC_E_DECLINED
        p = L.tc_plan(((1 << 20,), (1,), 1), ((1 << 20,), (1,)), dt)
        assert p["path_name"] == "rows" and p["unaligned"] and p["vec_bytes"] == 16, p
        # the page's plan in strict mode: the widest aligned vector (4 bytes at most here)
        sp = L.tc_plan(((1 << 20,), (1,), 1), ((1 << 20,), (1,)), dt, flags=L.TC_FLAG_STRICT, raise_on_error=False)
        assert sp["status"] == L.TC_E_DECLINED or (sp["vec_bytes"] == eb and not sp["unaligned"]), sp


def test_interleave_path_selection():
    """NHWC -> NCHW with 3 channels takes the interleave path at every width; the way back, 5
    channels, misaligned planes, strict mode and TC_FLAG_NO_SHUFFLE do not; the scale-factor
    blocks keep the butterfly."""
    n, h, w, ch = 2, 224, 224, 3
    hw = h * w
    to = (((n, h, w, ch), (hw * ch, w * ch, ch, 1)), ((n, h, w, ch), (ch * hw, w, 1, hw)))
    back = (((n, ch, h, w), (ch * hw, hw, w, 1)), ((n, ch, h, w), (hw * ch, 1, w * ch, ch)))
    for dt in (L.TC_U8, L.TC_BF16, L.TC_F32, L.TC_F64):
        p = L.tc_plan(*to, dt)
        assert p["path_name"] == "interleave" and p["tile_c"] == ch, p
        assert L.tc_plan(*to, dt, flags=L.TC_FLAG_NO_SHUFFLE)["path_name"] == "transpose"
        assert L.tc_plan(*to, dt, flags=L.TC_FLAG_STRICT, raise_on_error=False)["path_name"] != "interleave"
        # planes to interleaved channels: the transpose kernel (measured faster)
        assert L.tc_plan(*back, dt)["path_name"] == "transpose"
    # 5 channels, or a plane stride that breaks 16-byte alignment: the transpose kernel
    five = (((n, h, w, 5), (hw * 5, w * 5, 5, 1)), ((n, h, w, 5), (5 * hw, w, 1, hw)))
    assert L.tc_plan(*five, L.TC_F32)["path_name"] == "transpose"
    odd = (((n, h, w, ch), (hw * ch, w * ch, ch, 1)), ((n, h, w, ch), (ch * (hw + 1), w, 1, hw + 1)))
    assert L.tc_plan(*odd, L.TC_F32)["path_name"] == "transpose"
    sf = ((65536, 2, 1, 4, 32), (256, 128, 128, 32, 1)), ((65536, 2, 1, 4, 32), (256, 128, 128, 1, 4))
    assert L.tc_plan(*sf, L.TC_F32)["path_name"] == "shuffle"


def test_no_kernel_uses_scratch_memory():
    """Every kernel keeps its per-lane data in registers: the compiler reports no scratch (a
    private array it cannot promote would turn into extra memory instructions per tile)."""
    import json
    path = os.path.join(ROOT, "layout_permuting_copy_amd", "_build", "kernel_resources.json")
    if not os.path.exists(path):
        pytest.skip("library not built by layout_permuting_copy_amd/build.py")
    res = json.load(open(path))
    kernels = {k: v for k, v in res.items() if "tc3dev" in k}
    assert sum("transpose_kernel" in k for k in kernels) >= 50
    assert not {k: v for k, v in kernels.items() if v.get("scratch_bytes", 0) != 0}


def test_shuffle_path_selection():
    """4 x C blocks of 4-byte elements, contiguous on both sides, take the register butterfly;
    anything else (other widths, C = 64, blocks not contiguous, the flag) does not."""
    f32 = L.TC_F32
    for C in (8, 16, 32):
        p = L.tc_plan(((64, 4, C), (4 * C, C, 1)), ((64, 4, C), (4 * C, 1, 4)), f32)
        assert p["path_name"] == "shuffle" and (p["tile_r"], p["tile_c"]) == (4, C)
        # padded block pitch on either side is fine
        p = L.tc_plan(((64, 4, C), (4 * C + 8, C, 1)), ((64, 4, C), (4 * C + 16, 1, 4)), f32)
        assert p["path_name"] == "shuffle"
    for shape, ss, ds, dt in [((64, 4, 64), (256, 64, 1), (256, 1, 4), f32),      # C = 64
                              ((64, 4, 32), (128, 32, 1), (128, 1, 4), L.TC_BF16),  # 2-byte elements
                              ((64, 4, 32), (256, 64, 1), (128, 1, 4), f32),      # source rows apart
                              ((64, 8, 32), (256, 32, 1), (256, 1, 8), f32)]:     # 8 rows
        assert L.tc_plan((shape, ss), (shape, ds), dt)["path_name"] != "shuffle", (shape, ss, ds)
    sf = SI.sf_transpose()
    assert _plan(sf)["path_name"] == "shuffle"
    assert _plan(sf, flags=L.TC_FLAG_NO_SHUFFLE)["path_name"] == "transpose"


def test_alias_check_covers_the_last_element():
    """Overlap is judged on whole elements: a destination that starts inside the source's last
    element, or ends inside its first, shares bytes and is rejected before anything is launched
    (host-only: the addresses are never dereferenced).  Adjacent buffers are accepted (GPU test)."""
    lay = ((4,), (1,))
    src = 0x10000
    for dst in (src + 12, src + 8, src - 12):
        with pytest.raises(L.TileCopyError) as e:
            L.tile_copy_ex(src, lay, dst, lay, L.TC_F32)
        assert e.value.code == L.TC_E_ALIAS, hex(dst)


def test_planning_is_thread_safe():
    """Plans made concurrently from many threads (shared plan cache and swizzle memo) equal the
    plans made one at a time."""
    from concurrent.futures import ThreadPoolExecutor
    dts = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}
    cases = [((sh, ss), (sh, ds), dts[eb]) for sh, ss, ds, eb, _ in SI.random_layouts(2024, 150)]
    cases += [(((n, m), (m, 1)), ((n, m), (1, n)), dts[eb]) for eb in dts for n, m in [(512, 256), (300, 129), (1024, 64)]]
    keys = ("status", "path_name", "vec_bytes", "tile_r", "tile_c", "tile_b", "threads", "xor_k", "xor_shift",
            "xor_tbit", "xor_cshift", "xor_cmask", "workgroups", "wave_local", "unaligned")

    def plan(c):
        p = L.tc_plan(*c, raise_on_error=False)
        return tuple(p[k] for k in keys)

    serial = [plan(c) for c in cases]
    with ThreadPoolExecutor(max_workers=8) as ex:
        for _ in range(3):
            assert list(ex.map(plan, cases)) == serial

    # the launch entry point's plan cache: overlapping (fake, never dereferenced) addresses make
    # tile_copy_ex plan through the cache, fill the plan info and stop at the alias check
    import ctypes
    lib = L.load_library()

    def cached(c):
        info = L.TcPlanInfo()
        s, d = L._as_layout(c[0]), L._as_layout(c[1])
        rc = lib.tile_copy_ex(0x100000, ctypes.byref(s), 0x100000, ctypes.byref(d), int(c[2]), None, 0,
                              ctypes.byref(info))
        p = info.to_dict()
        p["status"] = 0 if rc == L.TC_E_ALIAS else rc
        return tuple(p[k] for k in keys)

    ok = [i for i, c in enumerate(cases) if serial[i][0] == 0 and serial[i][1] != "empty"]
    with ThreadPoolExecutor(max_workers=8) as ex:
        for _ in range(3):
            got = list(ex.map(cached, [cases[i] for i in ok]))
            assert got == [serial[i] for i in ok]


# layouts planned cold from several threads at once (shapes no other test plans, so that the swizzle
# search and its memo are exercised concurrently), with strict-mode declines and argument errors
_THREAD_CASES = [
    (((1000 + 64 * k, 960 + 32 * k), (960 + 32 * k, 1)), ((1000 + 64 * k, 960 + 32 * k), (1, 1000 + 64 * k)), dt, fl)
    for k in range(6) for dt, fl in ((L.TC_I8, 0), (L.TC_F16, 0), (L.TC_F32, 0), (L.TC_F64, 0), (L.TC_B128, 0))
] + [
    (((1001, 37), (37, 1)), ((1001, 37), (1, 1001)), L.TC_F32, L.TC_FLAG_STRICT),   # declined: count % 64
    (((64, 32), (32, 1)), ((64, 33), (1, 64)), L.TC_F32, 0),                       # extents differ
    (((8, 4, 2), (8, 2, 1)), ((8, 4, 2), (1, 8, 32)), L.TC_BF16, L.TC_FLAG_STRICT),
]


def _plan_cases_json(cases):
    out = []
    for s, d, dt, fl in cases:
        p = L.tc_plan(s, d, dt, flags=fl, raise_on_error=False)
        out.append({k: (list(v) if isinstance(v, (list, tuple)) else v) for k, v in p.items()})
    return out


def test_planner_is_thread_safe():
    """tc_plan from 8 threads at once (ctypes releases the GIL during the call), on a cold plan
    cache: every result, including the reason of each decline or error (thread-local, read back by
    the same thread), equals the one a separate process computes sequentially."""
    import json
    import sys
    import threading
    code = ("import json, sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
            "import test_host_planner as T\nprint(json.dumps(T._plan_cases_json(T._THREAD_CASES)))\n"
            % (ROOT, os.path.join(ROOT, "tests")))
    want = json.loads(subprocess.check_output([sys.executable, "-c", code], cwd=ROOT, text=True))
    got, errors = {}, []

    def worker(t):
        try:
            order = list(range(len(_THREAD_CASES)))
            order = order[t:] + order[:t]  # each thread starts at a different case
            for _ in range(3):
                for i in order:
                    r = _plan_cases_json([_THREAD_CASES[i]])[0]
                    if r != want[i]:
                        errors.append((t, i, r, want[i]))
                    got[(t, i)] = r
        except Exception as e:  # surfaced below
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:3]
    assert len(got) == 8 * len(_THREAD_CASES)
    assert any(w["status"] == L.TC_E_DECLINED for w in want) and any(w["status"] == L.TC_E_EXTENT for w in want)


def test_sizes_beyond_64_bit_addresses_are_rejected():
    """Element counts or element offsets beyond 2^58 (byte offsets of 16-byte elements would pass
    2^62) are TC_E_RANGE before any planning, rather than wrapping around: a 2^80-element copy
    must not read as empty, nor a stride of 2^62 as a small one."""
    big = [
        (((1 << 40, 1 << 40), (1 << 40, 1)), ((1 << 40, 1 << 40), (1, 1 << 40))),  # count 2^80
        (((1 << 62,), (1,)), ((1 << 62,), (1,))),                                 # count 2^62
        (((3, 1 << 61), (1 << 61, 1)), ((3, 1 << 61), (1, 3))),                    # offsets 2^62
        (((4, 4), (1 << 62, 1)), ((4, 4), (4, 1))),                                 # source stride
        (((4, 4), (4, 1), 1 << 59), ((4, 4), (4, 1))),                              # source offset
        (((4, 4), (4, 1)), ((4, 4), (-(1 << 60), 1), 1 << 62)),                     # negative side
    ]
    for s, d in big:
        p = L.tc_plan(s, d, L.TC_B128, raise_on_error=False)
        assert p["status"] == L.TC_E_RANGE and "2^58" in p["error"], (s, d, p["status"], p["error"])
    # the limit itself, and an empty copy with huge strides, are fine
    ok = [(((1 << 29, 4), (4, 1)), ((1 << 29, 4), (4, 1))),
          (((0, 1 << 62), (1 << 62, 1)), ((0, 1 << 62), (1, 0)))]
    for s, d in ok:
        assert L.tc_plan(s, d, L.TC_I8, raise_on_error=False)["status"] == L.TC_OK, (s, d)


def test_slices_beyond_64_bits_are_rejected():
    """tc_layout_slice computes offsets and strides without wrapping: results beyond 64 bits, and
    the one step whose negation does not exist, are TC_E_RANGE; ordinary extreme steps still give
    the Python slice lengths."""
    lay = ((1 << 40,), (1 << 30,), 0)
    with pytest.raises(L.TileCopyError) as e:
        L.tc_layout_slice(lay, [0], [1 << 40], [1 << 40])      # stride 2^70
    assert e.value.code == L.TC_E_RANGE
    with pytest.raises(L.TileCopyError) as e:
        L.tc_layout_slice(((10,), (1,), 0), [0], [10], [-(1 << 63)])
    assert e.value.code == L.TC_E_RANGE
    big = (1 << 63) - 1
    out = L.tc_layout_slice(((10,), (1,), 0), [0], [10], [big])
    assert (out.shape[0], out.stride[0], out.offset) == (len(range(0, 10, big)), big, 0)
    out = L.tc_layout_slice(((10,), (1,), 0), [9], [-11], [-big])
    assert (out.shape[0], out.offset) == (len(range(10)[9::-big]), 9)


def test_int8_stride2_sources_read_in_pairs():
    """1-byte copies whose column mode has source stride 2 read the source as 2-byte pairs
    (src_view_bytes 2) where every source stride is even (the offset's parity picks the low or
    high byte), the source pointer is 2-byte aligned and the tile is at least 512 x 64; otherwise
    the stride-2 tile of 1-byte elements (src_view_bytes 1).  2-, 4- and 8-byte elements at even
    offsets are read as 4-, 8- and 16-byte pairs."""
    n = 8192
    R, C = n - 2, (n - 1) // 2

    def plan(ss, so, dt=L.TC_I8, align=16, shape=(R, C)):
        p = L.tc_plan((shape, ss, so), (shape, (1, shape[0])), dt, ptr_align=align)
        assert p["path_name"] == "transpose" and p["src_step"] == 2, p
        return p["src_view_bytes"], p["tile_r"], p["tile_c"], p["grid_order"], p["super_rows"], p["super_cols"]

    assert plan((n, 2), n) == (2, 512, 64, 2, 16, 4)
    assert plan((n, 2), n, dt=L.TC_U8) == (2, 512, 64, 2, 16, 4)
    assert plan((n, 2), n + 1)[0] == 2            # odd source offset: high bytes kept
    assert plan((-n, 2), n * (R - 1) - 1)[0] == 2  # negative row stride, odd offset
    assert plan((n + 1, 2), n)[0] == 1            # odd row stride
    assert plan((n, 2), n, align=1)[0] == 1       # source pointer not 2-byte aligned
    assert plan((n, 2), n, shape=(511, C))[0] == 1  # rows too few for the 512-row tile
    assert plan((n, 2), n, shape=(R, 63))[0] == 1   # columns too few for the 64-column tile
    # 2-byte elements: read as 4-byte pairs on 256 x 32 tiles in 16 x 16 super-tiles; at an odd
    # offset their own width
    assert plan((n, 2), n, dt=L.TC_F16) == (4, 256, 32, 2, 16, 16)
    assert plan((n, 2), n + 1, dt=L.TC_F16)[0] == 2
    # 4- and 8-byte elements: 8- and 16-byte pairs on 128 x 32 and 64 x 8 tiles
    assert plan((n, 2), n, dt=L.TC_F64) == (16, 64, 8, 2, 16, 16)
    assert plan((n, 2), n, dt=L.TC_F32) == (8, 128, 32, 2, 16, 16)
    assert plan((n, 2), n + 1, dt=L.TC_F32)[0] == 4


def test_rows_gathered_from_strided_sources():
    """A destination contiguous along the innermost mode whose source steps 2, 3 or 4 elements
    along it, or -1 to -4 (reversed), and has no unit-stride mode runs on the element-aligned rows
    path with gathered vectors (src_step = the source stride); other strides, 16-byte elements, a
    transposing copy and strict mode do not."""
    def plan(shape, ss, ds, dt=L.TC_I8, flags=0, so=0):
        return L.tc_plan((shape, ss, so), (shape, ds), dt, flags=flags)

    for dt in (L.TC_I8, L.TC_F16, L.TC_F32, L.TC_F64):
        for k in (2, 3, 4):
            p = plan((100, 77), (1000, k), (77, 1), dt=dt, so=3)
            assert (p["path_name"], p["src_step"], p["vec_bytes"], p["unaligned"], p["declined"]) == ("rows", k, 16, 1, 1), p
            assert p["workgroups"] == -(-100 * -(-77 // (16 // p["elem_bytes"])) // (p["threads"] * p["load_outer"]))
    # batched: the source strides of the outer modes may be anything
    p = plan((3, 21, 77), (21 * 400, 400, 3), (21 * 90, 90, 1))
    assert (p["path_name"], p["src_step"]) == ("rows", 3)
    # reversed rows (a flip) and reversed strided slices: negative steps down to -4
    for k in (-1, -2, -3, -4):
        p = plan((100, 77), (1000, k), (77, 1), so=400)
        assert (p["path_name"], p["src_step"], p["vec_bytes"]) == ("rows", k, 16), p
    assert plan((100, 77), (1000, 5), (77, 1))["path_name"] == "guarded_rows"
    assert plan((100, 77), (1000, -5), (77, 1), so=400)["path_name"] == "guarded_rows"
    assert plan((100, 77), (1000, 2), (77, 1), dt=L.TC_B128)["path_name"] == "guarded_rows"
    assert plan((100, 77), (1000, 2), (77, 1), flags=L.TC_FLAG_FORCE_GUARDED)["path_name"] == "guarded_rows"
    # the source has a unit-stride mode elsewhere: a transpose
    assert plan((100, 77), (1, 200), (77, 1))["path_name"] == "transpose"
    with pytest.raises(L.TileCopyError):
        plan((100, 77), (1000, 2), (77, 1), flags=L.TC_FLAG_STRICT)


def test_transposes_from_sources_of_stride_3_and_4():
    """A transpose whose source has no unit-stride mode but a mode of stride 3 or 4 (and no
    stride-2 mode), its elements at most 12 bytes apart, reads 16-byte vectors along it (src_step
    3 or 4) on the element-aligned tile; wider strides take the guarded tile."""
    def plan(shape, ss, ds, dt=L.TC_I8):
        return L.tc_plan((shape, ss, 0), (shape, ds), dt)

    for dt in (L.TC_I8, L.TC_F16, L.TC_F32, L.TC_F64, L.TC_B128):
        for k in (3, 4):
            p = plan((500, 300), (2000, k), (1, 500), dt=dt)
            if k * L.ELEM_BYTES[dt] > 12:  # elements more than 12 bytes apart: the guarded tile
                assert p["path_name"] == "guarded_tile", p
                continue
            assert (p["path_name"], p["src_step"], p["vec_bytes"], p["unaligned"]) == ("transpose", k, 16, 1), p
            assert p["write_conflicts"] == 0 and p["read_conflicts"] == 0, p
    # the same strides without a transposition: gathered rows
    p = plan((20, 30, 40), (3, 60 * 40, 60), (1, 20 * 40, 20))
    assert p["path_name"] == "rows" and p["src_step"] == 3 and p["rank"] == 1, p
    assert plan((500, 300), (2000, 5), (1, 500))["path_name"] == "guarded_tile"


def test_transposes_from_reversed_source_columns():
    """A transpose whose source has no unit-stride mode but a mode of stride -1 has that mode's
    index reversed (an ordinary transpose then); one of stride -2 (or -3, -4 with elements at most
    12 bytes apart) reads 16-byte vectors along it in reverse (src_step negative); a stride of
    smaller magnitude wins, the positive one on a tie."""
    def plan(shape, ss, ds, dt=L.TC_I8, so=0):
        return L.tc_plan((shape, ss, so), (shape, ds), dt)

    for dt in (L.TC_I8, L.TC_F16, L.TC_F32, L.TC_F64, L.TC_B128):
        for k in (-1, -2, -3, -4):
            p = plan((500, 300), (-k * 300 + 7, k), (1, 500), dt=dt, so=-k * 299)
            if -k >= 3 and -k * L.ELEM_BYTES[dt] > 12:
                assert p["path_name"] == "guarded_tile", p
                continue
            # stride -1: the column index reversed, read forwards (16-byte elements: then whole
            # aligned vectors, the aligned kernels)
            unaligned = 0 if (k == -1 and L.ELEM_BYTES[dt] == 16) else 1
            assert (p["path_name"], p["src_step"], p["unaligned"]) == ("transpose", 1 if k == -1 else k, unaligned), p
            assert p["write_conflicts"] == 0 and p["read_conflicts"] == 0, p
    # rot90, the transpose of the column-flipped matrix: the column index reversed (both strides
    # negated, the offsets moved to its other end), then the aligned transpose
    p = plan((256, 256), (-1, 256), (256, 1), so=255)
    assert (p["path_name"], p["src_step"], p["declined"], p["unaligned"]) == ("transpose", 1, 0, 0), p
    assert (p["src_stride"][:2], p["dst_stride"][:2], p["src_offset"], p["dst_offset"]) == ((1, 256), (-256, 1), 0, 255 * 256)
    # two candidate modes: stride 2 beats stride -2 and -3
    p = plan((30, 40, 50), (2, -3 * 30, 3 * 30 * 40 + 1), (40 * 50, 50, 1), so=3 * 30 * 39)
    assert p["path_name"] == "transpose" and p["src_step"] == 2, p
    p = plan((30, 40, 50), (-2, 2, 2 * 30 * 40 + 1), (40 * 50, 50, 1), so=2 * 29)
    assert p["path_name"] == "transpose" and p["src_step"] == 2 and p["mode_c"] == 1, p


def test_modes_walked_backwards_are_reversed():
    """The planner reverses modes (both strides negated, the offsets moved to the other end; the
    same pairs of elements): those both sides walk backwards, then a destination mode of stride -1
    where none has stride 1, then a source mode of stride -1 other than the destination's
    contiguous one where none has stride 1.  A source row walked backwards into a contiguous
    destination row is not reversed (gathered rows)."""
    def plan(shape, ss, so, ds, do, dt=L.TC_F32):
        return L.tc_plan((shape, ss, so), (shape, ds, do), dt)

    n = 512
    p = plan((n, n), (n, -1), n - 1, (n, -1), n - 1)
    assert (p["path_name"], p["rank"], p["src_offset"], p["dst_offset"]) == ("rows", 1, 0, 0), p
    p = plan((n, n), (-n, 1), n * (n - 1), (-n, 1), n * (n - 1))
    assert (p["path_name"], p["rank"], p["src_stride"][0], p["dst_stride"][0]) == ("rows", 1, 1, 1), p
    p = plan((n, n), (n, 1), 0, (n, -1), n - 1)   # into a flipped view: the source read backwards
    assert (p["path_name"], p["src_step"], p["src_stride"][:2], p["dst_stride"][:2]) == ("rows", -1, (n, -1), (n, 1)), p
    p = plan((n, n), (n, 1), 0, (-1, n), n - 1)   # into a rotated view: an aligned transpose
    assert (p["path_name"], p["declined"], p["src_step"]) == ("transpose", 0, 1), p
    p = plan((n, n), (-1, n), n - 1, (n, 1), 0)   # rot90 of the source
    assert (p["path_name"], p["declined"], p["dst_stride"][:2]) == ("transpose", 0, (-n, 1)), p
    p = plan((n, n), (n, -1), n - 1, (n, 1), 0)   # a flipped source row: gathered rows, not reversed
    assert (p["path_name"], p["src_step"], p["src_offset"]) == ("rows", -1, n - 1), p


def test_plan_variants_for_autotune():
    """The configurations tc_autotune times: the planner's plan first, then the same copy on other
    tiles (transposes: conflict-free, distinct, the same path and modes) or other vector counts
    (rows); one plan under TC_FLAG_NO_SWIZZLE; the planner's error for a copy it rejects."""
    n = 4096
    s, d = ((n, n), (n, 1), 0), ((n, n), (1, n), 0)
    for dt in (L.TC_I8, L.TC_BF16, L.TC_F32, L.TC_F64, L.TC_B128):
        v = L.tc_plan_variants(s, d, dt)
        base = L.tc_plan(s, d, dt)
        assert v[0] == {k: base[k] for k in v[0]}, dt
        assert len(v) >= 3, (dt, len(v))
        seen = set()
        for p in v:
            assert p["path_name"] == "transpose" and p["count"] == n * n
            assert p["write_conflicts"] == 0 and p["read_conflicts"] == 0
            key = (p["tile_r"], p["tile_c"], p["tile_b"], p["threads"], p["grid_order"], p["super_rows"],
                   p["super_cols"], p["loads_in_flight"], p["nontemporal"], p["edge_tiles"], p["lds_write_bytes"],
                   p["lds_read_bytes"])
            assert key not in seen, key
            seen.add(key)
    # odd extents: the element-aligned tiles in three grid orders
    v = L.tc_plan_variants(((8191, 8190), (8190, 1), 0), ((8191, 8190), (1, 8191), 0), L.TC_I8)
    assert len(v) >= 3 and all(p["unaligned"] == 1 for p in v)
    # rows: vectors per lane (aligned rows, and element-aligned rows such as a window at an odd
    # offset)
    v = L.tc_plan_variants(((1 << 24,), (1,), 0), ((1 << 24,), (1,), 0), L.TC_F32)
    assert {p["load_outer"] for p in v} == {1, 2, 4} and all(p["path_name"] == "rows" for p in v)
    v = L.tc_plan_variants(((1000, 1000), (1024, 1), 1025), ((1000, 1000), (1000, 1), 0), L.TC_I8)
    assert [p["load_outer"] for p in v] == [4, 1, 2] and all(p["unaligned"] == 1 for p in v), v
    assert len(L.tc_plan_variants(s, d, L.TC_F32, flags=L.TC_FLAG_NO_SWIZZLE)) == 1
    with pytest.raises(L.TileCopyError):
        L.tc_plan_variants(((8191, 8190), (8190, 1), 0), ((8191, 8190), (1, 8191), 0), L.TC_I8, flags=L.TC_FLAG_STRICT)


def test_all_to_all_pack_and_unpack_compose_the_sharded_permute():
    """The (0,2,1,3) permute of X[B, H, S, D] sharded on H over G GPUs, with its output sharded on
    S: each GPU packs its heads into per-destination blocks (a2a_pack_permute0213), an
    all-to-all swaps the blocks, and each GPU unpacks what it received (a2a_unpack_permute0213).
    Run with the oracle copy and a host all-to-all on a small case, every output shard equals the
    permuted tensor's slice; both copies plan as rows (the head dimension contiguous on both
    sides)."""
    from oracle import ref as R
    g, b, h, s, d = 4, 2, 8, 16, 3
    hl, sl = h // g, s // g
    x = np.random.default_rng(5).standard_normal((b, h, s, d)).astype(np.float32)
    wp, wu = SI.a2a_pack_permute0213(g, b, h, s, d, "float32"), SI.a2a_unpack_permute0213(g, b, h, s, d, "float32")
    sent = []
    for r in range(g):
        xr = np.ascontiguousarray(x[:, r * hl:(r + 1) * hl])
        out = np.zeros(g * b * sl * hl * d, dtype=np.float32)
        R.copy(xr.view(np.uint8).ravel(), (wp.src.shape, wp.src.stride, 0), out.view(np.uint8),
               (wp.dst.shape, wp.dst.stride, 0), 4)
        sent.append(out.reshape(g, b * sl * hl * d))
    want = x.transpose(0, 2, 1, 3)  # [B, S, H, D]
    for q in range(g):
        recv = np.stack([sent[r][q] for r in range(g)]).ravel()  # from every sender, in rank order
        y = np.zeros(b * sl * h * d, dtype=np.float32)
        R.copy(recv.view(np.uint8), (wu.src.shape, wu.src.stride, 0), y.view(np.uint8),
               (wu.dst.shape, wu.dst.stride, 0), 4)
        assert np.array_equal(y.reshape(b, sl, h, d), want[:, q * sl:(q + 1) * sl]), q
    for w in (SI.a2a_pack_permute0213(), SI.a2a_unpack_permute0213()):
        assert _plan(w)["path_name"] == "rows", w.name


def test_count_declines_with_whole_aligned_vectors_take_the_aligned_kernels():
    """A copy the page's count rule declines (count not a multiple of 64) but whose 16-byte
    vectors are whole and aligned on both sides runs the aligned kernels outside strict mode
    (unaligned 0, the page's reason kept); with odd rows it stays on the element-aligned ones."""
    def plan(shape, ss, ds, dt, so=0, flags=0):
        return L.tc_plan((shape, ss, so), (shape, ds, 0), dt, flags=flags, raise_on_error=False)

    p = plan((8190 * 8176,), (1,), (1,), L.TC_I8)
    assert (p["path_name"], p["declined"], p["unaligned"], p["vec_bytes"]) == ("rows", 1, 0, 16), p
    assert "no integer solution" in p["reason"]
    p = plan((8191, 8184), (8184, 1), (8184, 1), L.TC_F32)   # rows of whole vectors
    assert (p["path_name"], p["declined"], p["unaligned"]) == ("rows", 1, 0), p
    p = plan((8184, 8191), (8191, 1), (1, 8184), L.TC_F32)   # source rows odd: element-aligned
    assert (p["path_name"], p["declined"], p["unaligned"]) == ("transpose", 1, 1), p
    p = plan((1000,), (1,), (1,), L.TC_F32, so=1)            # misaligned: element-aligned rows
    assert (p["path_name"], p["unaligned"]) == ("rows", 1), p
    assert plan((8190 * 8176,), (1,), (1,), L.TC_I8, flags=L.TC_FLAG_STRICT)["status"] == L.TC_E_DECLINED
