"""Seeded synthetic inputs for the layout-permuting tile copy.

This module is shared by the tests, ``bench.py`` and the oracle checks.  It holds
workload *data* only -- shapes, element strides, offsets, element types, value
distributions and seeds -- and the random generators that fill source buffers.
It contains no part of the copy, the layout algebra, the partition or the bank
planning: both the product path and the oracle derive everything else on their
own from these plain tuples.

Layouts are given in elements as ``(shape, stride, offset)`` tuples over one
storage buffer, the shape:stride form used by the TileLayout pages.  Values are
generated on the host with NumPy's PCG64 (``numpy.random.default_rng(seed)``)
and handled as raw bytes: floating point values are produced in their own type
and then only ever moved as bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# element type name -> (bytes per element, numpy type used to make values)
ELEMENT_TYPES = {
    "int8": (1, np.int8),
    "uint8": (1, np.uint8),
    "float16": (2, np.float16),
    "bfloat16": (2, None),  # made from float32 by round-to-nearest-even
    "float32": (4, np.float32),
    "int32": (4, np.int32),
    "float64": (8, np.float64),
    "int64": (8, np.int64),
    "int4vec": (16, None),  # 16-byte struct of four int32 (a vector type, not 4-bit ints)
}


def elem_bytes(dtype: str) -> int:
    return ELEMENT_TYPES[dtype][0]


@dataclass(frozen=True)
class Side:
    shape: tuple
    stride: tuple
    offset: int = 0


@dataclass(frozen=True)
class Workload:
    name: str
    src: Side
    dst: Side
    dtype: str
    values: str  # "uniform_pm1" | "uniform01" | "normal" | "bits"
    seed: int
    src_storage: Optional[int] = None  # storage elements; default = span of the layout
    dst_storage: Optional[int] = None
    notes: str = field(default="", compare=False)

    @property
    def eb(self) -> int:
        return elem_bytes(self.dtype)


def span(side: Side) -> int:
    """Number of storage elements needed to hold every element the layout names: one past its
    highest offset (negative strides count from the offset down, which must stay >= 0)."""
    if any(e == 0 for e in side.shape):
        return side.offset
    low = side.offset + sum((e - 1) * s for e, s in zip(side.shape, side.stride) if s < 0)
    if low < 0:
        raise ValueError(f"layout reaches below offset 0 (lowest offset {low})")
    return side.offset + sum((e - 1) * s for e, s in zip(side.shape, side.stride) if s > 0) + 1


def storage_elems(w: Workload, which: str) -> int:
    side = w.src if which == "src" else w.dst
    given = w.src_storage if which == "src" else w.dst_storage
    return given if given is not None else span(side)


def _row_major(shape):
    st, acc = [], 1
    for e in reversed(shape):
        st.append(acc)
        acc *= e
    return tuple(reversed(st))


# --- the five workloads, at their full sizes ------------------------------------------------

def tile32_roundtrip() -> Workload:
    return Workload("tile32x32_f32_roundtrip",
                    Side((32, 32), (32, 1)), Side((32, 32), (32, 1)),
                    "float32", "uniform_pm1", seed=1,
                    notes="one 32x32 fp32 tile, identity row-major layouts, one wave64")


def sf_transpose(tiles: int = 65536) -> Workload:
    shape = (tiles, 2, 1, 4, 32)
    return Workload(f"sf_transpose_{tiles}x2x1x4x32_f32",
                    Side(shape, (256, 128, 128, 32, 1)), Side(shape, (256, 128, 128, 1, 4)),
                    "float32", "uniform_pm1", seed=2,
                    notes="scale-factor tile transpose, tiles contiguous in HBM (tile t at 256*t)")


def transpose2d(n: int = 16384, m: Optional[int] = None, dtype: str = "float32", seed: Optional[int] = None,
                values: Optional[str] = None) -> Workload:
    m = n if m is None else m
    if seed is None:
        seed = {"float32": 3, "bfloat16": 31}.get(dtype, 50)
    if values is None:
        values = "normal" if dtype in ("float32", "bfloat16") else "bits"
    return Workload(f"transpose_{n}x{m}_{dtype}",
                    Side((n, m), (m, 1)), Side((n, m), (1, n)), dtype, values, seed)


def permute0213(b: int = 32, h: int = 32, s: int = 2048, d: int = 128, dtype: str = "bfloat16") -> Workload:
    # logical index (b, h, s, d); source [B,H,S,D] row-major, destination [B,S,H,D] row-major
    return Workload(f"permute0213_{b}x{h}x{s}x{d}_{dtype}",
                    Side((b, h, s, d), (h * s * d, s * d, d, 1)),
                    Side((b, h, s, d), (s * h * d, d, h * d, 1)),
                    dtype, "normal", seed=4)


def a2a_pack_permute0213(g: int = 8, b: int = 32, h: int = 32, s: int = 2048, d: int = 128,
                         dtype: str = "bfloat16") -> Workload:
    """One GPU's pack before the all-to-all that turns the (0,2,1,3) permute sharded on H into
    its output sharded on S, over g GPUs: the local shard X[b, h/g, s, d] (row-major) goes to a
    send buffer P[g, b, s/g, h/g, d] (row-major) with P[q, i, j, k, l] = X[i, k, q*s/g + j, l]."""
    hl, sl = h // g, s // g
    return Workload(f"a2a_pack_permute0213_g{g}_{b}x{h}x{s}x{d}_{dtype}",
                    Side((g, b, sl, hl, d), (sl * d, hl * s * d, d, s * d, 1)),
                    Side((g, b, sl, hl, d), (b * sl * hl * d, sl * hl * d, hl * d, d, 1)),
                    dtype, "bits", seed=57)


def a2a_unpack_permute0213(g: int = 8, b: int = 32, h: int = 32, s: int = 2048, d: int = 128,
                           dtype: str = "bfloat16") -> Workload:
    """The receiving GPU's unpack after that all-to-all: the buffer R[g, b, s/g, h/g, d] received
    from the g senders (row-major) into its output shard Y[b, s/g, h, d] (row-major), with
    Y[i, j, q*h/g + k, l] = R[q, i, j, k, l]."""
    hl, sl = h // g, s // g
    return Workload(f"a2a_unpack_permute0213_g{g}_{b}x{h}x{s}x{d}_{dtype}",
                    Side((g, b, sl, hl, d), (b * sl * hl * d, sl * hl * d, hl * d, d, 1)),
                    Side((g, b, sl, hl, d), (hl * d, sl * h * d, h * d, d, 1)),
                    dtype, "bits", seed=58)


SWEEP_DTYPES = ("int8", "float16", "float64", "int4vec")
SWEEP_SEEDS = {"int8": 50, "float16": 51, "float64": 52, "int4vec": 53}


def sweep_dense(dtype: str, n: int = 8192) -> Workload:
    return Workload(f"transpose_{n}x{n}_{dtype}",
                    Side((n, n), (n, 1)), Side((n, n), (1, n)), dtype, "bits", SWEEP_SEEDS[dtype])


def sweep_slice(dtype: str, n: int = 8192) -> Workload:
    # source view [1:n-1:1, 0:n-2:2] of an n x n row-major buffer; dense transposed destination
    rows = n - 2          # range(1, n-1)
    cols = (n - 2 + 1) // 2  # range(0, n-2, 2)
    return Workload(f"slice_{n}x{n}[1:{n-1}:1,0:{n-2}:2]_{dtype}",
                    Side((rows, cols), (n, 2), offset=n), Side((rows, cols), (1, rows)),
                    dtype, "bits", seed=54, src_storage=n * n)


def sweep_slice_rows(dtype: str, n: int = 8192) -> Workload:
    # the same source view [1:n-1:1, 0:n-2:2], written out densely in its own row order
    rows, cols = n - 2, (n - 2 + 1) // 2
    return Workload(f"slice_rows_{n}x{n}[1:{n-1}:1,0:{n-2}:2]_{dtype}",
                    Side((rows, cols), (n, 2), offset=n), Side((rows, cols), (cols, 1)),
                    dtype, "bits", seed=56, src_storage=n * n)


def sweep_odd(dtype: str, rows: int = 8191, cols: int = 8190) -> Workload:
    return Workload(f"transpose_{rows}x{cols}_{dtype}",
                    Side((rows, cols), (cols, 1)), Side((rows, cols), (1, rows)),
                    dtype, "bits", seed=55)


def all_workloads():
    ws = [tile32_roundtrip(), sf_transpose(), transpose2d(dtype="float32"), transpose2d(dtype="bfloat16"),
          permute0213()]
    for dt in SWEEP_DTYPES:
        ws += [sweep_dense(dt), sweep_slice(dt), sweep_odd(dt), sweep_slice_rows(dt)]
    return ws


# --- generators -----------------------------------------------------------------------------

def _bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, rounded to nearest even (finite inputs)."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def make_values(dtype: str, values: str, count: int, seed: int) -> np.ndarray:
    """``count`` elements of ``dtype`` as a flat uint8 array of count*eb bytes."""
    rng = np.random.default_rng(seed)
    eb = elem_bytes(dtype)
    if values == "bits" or dtype == "int4vec":
        return np.frombuffer(rng.bytes(count * eb), dtype=np.uint8).copy()
    if dtype == "bfloat16":
        f = (rng.standard_normal(count, dtype=np.float32) if values == "normal"
             else _uniform(rng, values, count, np.float32))
        return _bf16_bits_from_f32(f).view(np.uint8)
    npt = ELEMENT_TYPES[dtype][1]
    if values == "normal":
        if npt in (np.float32, np.float64):
            arr = rng.standard_normal(count, dtype=npt)
        else:
            arr = rng.standard_normal(count).astype(npt)
    elif values in ("uniform_pm1", "uniform01"):
        arr = _uniform(rng, values, count, npt)
    else:
        raise ValueError(values)
    return np.ascontiguousarray(arr).view(np.uint8)


def _uniform(rng, values, count, npt):
    if npt in (np.float32, np.float64):
        u = rng.random(count, dtype=npt)
    else:
        u = rng.random(count).astype(npt)
    return (u * 2 - 1).astype(npt) if values == "uniform_pm1" else u


def make_source(w: Workload) -> np.ndarray:
    """The whole source storage buffer (uint8, storage_elems*eb bytes), seeded."""
    return make_values(w.dtype, w.values, storage_elems(w, "src"), w.seed)


def device_bits(torch, nbytes: int, seed: int):
    """`nbytes` uniformly random bytes generated on the GPU from a seeded torch generator, for
    copies too large to stage through the host (tens of GiB)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)


def sentinel_dst(w: Workload, byte: int = 0xA5) -> np.ndarray:
    """Destination storage prefilled with a sentinel byte, so writes outside the
    destination image are visible."""
    return np.full(storage_elems(w, "dst") * w.eb, byte, dtype=np.uint8)


def scaled_2d(w: Workload, n: int, m: int) -> Workload:
    """The same 2-D transpose family at another size (row-major source, transposed destination)."""
    return Workload(f"{w.name}@{n}x{m}", Side((n, m), (m, 1)), Side((n, m), (1, n)), w.dtype, w.values, w.seed)


__all__ = [n for n in dir() if not n.startswith("_")]
_row_major = _row_major


def random_layouts(seed: int = 1234, count: int = 60):
    """Random layout pairs: a permuted row-major source buffer, optionally sliced with steps of
    2, into a destination that is row-major in another mode order.  Yields
    (shape, src_stride, dst_stride, elem_bytes, src_elems)."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        rank = int(rng.integers(1, 6))
        shape = tuple(int(x) for x in rng.integers(1, 9, size=rank) * rng.choice([1, 2, 4], size=rank))
        eb = int(rng.choice([1, 2, 4, 8, 16]))
        perm_s = rng.permutation(rank)
        perm_d = rng.permutation(rank)
        steps = rng.choice([1, 1, 1, 2], size=rank)
        full = [shape[k] * steps[k] for k in range(rank)]
        st_full = [0] * rank
        acc = 1
        for k in reversed(perm_s):
            st_full[k] = acc
            acc *= full[k]
        s_stride = tuple(int(st_full[k] * steps[k]) for k in range(rank))
        d_stride = [0] * rank
        acc = 1
        for k in reversed(perm_d):
            d_stride[k] = acc
            acc *= shape[k]
        yield shape, s_stride, tuple(d_stride), eb, acc * int(np.prod(steps)) + 1


def random_layouts_large(seed: int = 777, count: int = 60, max_elems: int = 3 << 20):
    """Multi-tile layout pairs for the tiled paths: two large modes (extents up to a few
    thousand, so that copies span many tiles and end in ragged ones), an optional small batch
    mode, padded pitches on both sides (so rows start off the 16-byte and 128-byte grids), a
    source step of 1 or 2 along its innermost mode, element offsets, and a destination that is
    dense in a random mode order with its own padding.  Yields (shape, src_stride, src_offset,
    dst_stride, dst_offset, elem_bytes, src_elems, dst_elems); every offset a layout reaches lies
    in [0, *_elems), and the destination is injective."""
    rng = np.random.default_rng(seed)
    made = 0
    while made < count:
        eb = int(rng.choice([1, 2, 4, 8, 16]))
        big = [int(rng.integers(1, 3000)), int(rng.integers(1, 3000))]
        rank = int(rng.integers(2, 4))
        shape = big + [int(rng.integers(1, 6)) for _ in range(rank - 2)]
        order = list(rng.permutation(rank))
        if int(np.prod(shape)) > max_elems // max(1, eb // 4) or int(np.prod(shape)) == 0:
            continue
        # source: row-major in `order` (last = innermost), innermost step 1 or 2, padded pitches
        step = int(rng.choice([1, 1, 1, 2]))
        ss = [0] * rank
        acc = step
        ss[order[-1]] = step
        acc = shape[order[-1]] * step
        for k in reversed(order[:-1]):
            acc += int(rng.integers(0, 40))
            ss[k] = acc
            acc *= shape[k]
        so = int(rng.integers(0, 9))
        # destination: dense in another order, padded pitches
        dorder = list(rng.permutation(rank))
        ds = [0] * rank
        ds[dorder[-1]] = 1
        dacc = shape[dorder[-1]]
        for k in reversed(dorder[:-1]):
            dacc += int(rng.integers(0, 40))
            ds[k] = dacc
            dacc *= shape[k]
        do = int(rng.integers(0, 9))
        span_s = so + sum((e - 1) * st for e, st in zip(shape, ss)) + step
        span_d = do + sum((e - 1) * d for e, d in zip(shape, ds)) + 1
        made += 1
        yield tuple(shape), tuple(ss), so, tuple(ds), do, eb, span_s, span_d


def random_layouts_steps(seed: int = 2468, count: int = 120, max_elems: int = 1 << 20):
    """Multi-tile layout pairs whose source steps along its innermost mode by -4 to -1 or 2 to 4
    elements (strided slices, flips), some outer source modes walked backwards, and destinations
    dense in a random mode order with padded pitches and modes maybe walked backwards (flipped or
    rotated views); extents up to ~1500 so that copies end in ragged tiles and rows, element
    offsets on both sides.  Yields (shape, src_stride, src_offset, dst_stride, dst_offset,
    elem_bytes, src_elems, dst_elems); every offset a layout reaches lies in [0, *_elems), and the
    destination is injective."""
    rng = np.random.default_rng(seed)
    made = 0
    while made < count:
        eb = int(rng.choice([1, 2, 4, 8, 16]))
        rank = int(rng.integers(1, 4))
        shape = [int(rng.integers(1, 1500)) for _ in range(min(rank, 2))] + [int(rng.integers(1, 5)) for _ in range(rank - 2)]
        if int(np.prod(shape)) > max_elems // max(1, eb // 4):
            continue
        order = list(rng.permutation(rank))
        step = int(rng.choice([-4, -3, -2, -1, -1, 2, 2, 3, 4]))
        ss = [0] * rank
        ss[order[-1]] = step
        acc = shape[order[-1]] * abs(step)
        for k in reversed(order[:-1]):
            acc += int(rng.integers(0, 20))
            ss[k] = acc * (-1 if rng.integers(0, 4) == 0 else 1)
            acc *= shape[k]
        dorder = list(rng.permutation(rank))
        ds = [0] * rank
        ds[dorder[-1]] = 1
        dacc = shape[dorder[-1]]
        for k in reversed(dorder[:-1]):
            dacc += int(rng.integers(0, 20))
            ds[k] = dacc
            dacc *= shape[k]
        ds = [-d if rng.integers(0, 4) == 0 else d for d in ds]
        so = -sum((e - 1) * st for e, st in zip(shape, ss) if st < 0) + int(rng.integers(0, 9))
        do = -sum((e - 1) * d for e, d in zip(shape, ds) if d < 0) + int(rng.integers(0, 9))
        span_s = so + sum((e - 1) * st for e, st in zip(shape, ss) if st > 0) + 1
        span_d = do + sum((e - 1) * d for e, d in zip(shape, ds) if d > 0) + 1
        made += 1
        yield tuple(shape), tuple(ss), so, tuple(ds), do, eb, span_s, span_d


def random_layouts_wide(seed: int = 4321, count: int = 120):
    """Like random_layouts, plus negative source strides, broadcast (stride-0) source modes,
    inserted extent-1 modes with arbitrary strides, and element offsets on both sides.  Yields
    (src_shape, src_stride, src_offset, dst_shape, dst_stride, dst_offset, elem_bytes,
    src_elems, dst_elems); every offset a layout reaches lies in [0, *_elems)."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        rank = int(rng.integers(1, 5))
        shape = [int(x) for x in rng.integers(1, 9, size=rank) * rng.choice([1, 2, 4, 8], size=rank)]
        eb = int(rng.choice([1, 2, 4, 8, 16]))
        perm_s, perm_d = rng.permutation(rank), rng.permutation(rank)
        steps = rng.choice([1, 1, 1, 2, -1], size=rank)
        ss, acc = [0] * rank, 1
        for k in reversed(perm_s):
            ss[k] = int(acc * steps[k])
            acc *= shape[k] * abs(int(steps[k]))
        if rank > 1 and rng.integers(0, 6) == 0:
            ss[int(rng.integers(0, rank))] = 0
        ds, dacc = [0] * rank, 1
        for k in reversed(perm_d):
            ds[k] = dacc
            dacc *= shape[k]
        neg = -sum((e - 1) * s for e, s in zip(shape, ss) if s < 0)
        so = neg + int(rng.integers(0, 5))
        do = int(rng.integers(0, 5))
        src_shape, src_stride = list(shape), list(ss)
        if rng.integers(0, 3) == 0:
            pos = int(rng.integers(0, rank + 1))
            src_shape.insert(pos, 1)
            src_stride.insert(pos, int(rng.integers(-100, 100)))
        span_s = so + sum((e - 1) * s for e, s in zip(shape, ss) if s > 0) + 1
        span_d = do + sum((e - 1) * d for e, d in zip(shape, ds)) + 1
        yield (tuple(src_shape), tuple(src_stride), so, tuple(shape), tuple(ds), do, eb, span_s, span_d)
