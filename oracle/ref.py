"""Oracle for the layout-permuting tile copy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library neither imports it
nor shares any code, header, table or helper with it.

Everything here is a plain, slow, obviously-correct restatement of what the
pages define, with each function naming the passage it follows:

* the copy itself: for every logical index i of the common shape,
  ``dst[dst_layout(i)] = src[src_layout(i)]`` (TVM TIRx docs "copy -> gmem_smem",
  intro / "What it accepts"; "permute_layout", intro);
* the TileLang default loop partition (TileLang tutorial "loop_mapping.py",
  module docstring: the nest's points in row-major order, grouped into vectors dealt to threads);
* the ``[outer, threads, vec]`` global<->shared partition and its vector-width
  rule (TVM TIRx docs "copy -> gmem_smem", Algorithm steps 1-2, the
  "Generated TIRx IR" listing and the dtype table of "How inputs change");
* the XOR bank-swizzle search of the register-staged permute (TVM TIRx docs
  "permute_layout", Algorithm steps 1-3 and "What it accepts");
* shared-memory / LDS bank-conflict counting by brute force.

Layouts are plain tuples ``(shape, stride, offset)`` in elements.
"""

from __future__ import annotations

import ctypes
import itertools
import math
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

Layout = Tuple[Tuple[int, ...], Tuple[int, ...], int]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_copy.so")


# ----------------------------------------------------------------------------------------------
# Layout map (TVM TIRx "copy -> gmem_smem": TileLayout(S[shape : strides]); the default strides
# of S[shape] are row-major).
# ----------------------------------------------------------------------------------------------

def layout(shape, stride=None, offset=0) -> Layout:
    shape = tuple(int(e) for e in shape)
    if stride is None:  # S[shape] without strides is row-major
        st, acc = [], 1
        for e in reversed(shape):
            st.append(acc)
            acc *= e
        stride = tuple(reversed(st))
    return shape, tuple(int(s) for s in stride), int(offset)


def offset_of(lay: Layout, idx: Sequence[int]) -> int:
    shape, stride, off = lay
    return off + sum(i * s for i, s in zip(idx, stride))


def non_unit_modes(lay: Layout) -> List[Tuple[int, int]]:
    """(extent, stride) of the modes whose extent is not 1, in order."""
    shape, stride, _ = lay
    return [(e, s) for e, s in zip(shape, stride) if e != 1]


def common_modes(src: Layout, dst: Layout) -> List[Tuple[int, int, int]]:
    """Joint modes (extent, src_stride, dst_stride) after dropping unit modes.

    The copy is valid only for equal non-unit extents (TVM TIRx "copy -> gmem_smem",
    "What it accepts": ``_is_valid_copy`` -> equal dtype / equal non-unit extents)."""
    a, b = non_unit_modes(src), non_unit_modes(dst)
    if [e for e, _ in a] != [e for e, _ in b]:
        raise ValueError(f"extent mismatch: {[e for e, _ in a]} vs {[e for e, _ in b]}")
    return [(e, s, d) for (e, s), (_, d) in zip(a, b)]


def index_of_flat(flat: int, extents: Sequence[int]) -> Tuple[int, ...]:
    """The multi-index at row-major position ``flat`` of a nest with these extents (the last mode
    varies fastest; TileLang loop_mapping.py: the nest is linearised row-major).  NumPy's
    ``unravel_index`` does the decomposition."""
    if len(extents) == 0:
        return ()
    return tuple(int(i) for i in np.unravel_index(int(flat), tuple(int(e) for e in extents)))


def flat_of_index(index: Sequence[int], extents: Sequence[int]) -> int:
    """Row-major position of a multi-index (the inverse of ``index_of_flat``; NumPy's
    ``ravel_multi_index``)."""
    if len(extents) == 0:
        return 0
    return int(np.ravel_multi_index(tuple(int(i) for i in index), tuple(int(e) for e in extents)))


# ----------------------------------------------------------------------------------------------
# The copy
# ----------------------------------------------------------------------------------------------

def copy_py(src: np.ndarray, src_lay: Layout, dst: np.ndarray, dst_lay: Layout, elem_bytes: int) -> None:
    """dst[dst(i)] = src[src(i)] for every logical index i, one element at a time.

    ``src``/``dst`` are flat uint8 storage buffers.  Pure Python: tiny cases only."""
    modes = common_modes(src_lay, dst_lay)
    extents = [e for e, _, _ in modes]
    so0, do0 = src_lay[2], dst_lay[2]
    for idx in itertools.product(*(range(e) for e in extents)):
        so = so0 + sum(i * s for i, (_, s, _) in zip(idx, modes))
        do = do0 + sum(i * d for i, (_, _, d) in zip(idx, modes))
        dst[do * elem_bytes:(do + 1) * elem_bytes] = src[so * elem_bytes:(so + 1) * elem_bytes]


_lib = None


def _load_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_copy.argtypes = [ctypes.c_void_p, ctypes.c_int, i64p, i64p, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_int, i64p, i64p, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int]
        lib.oracle_copy.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _i64(seq):
    arr = (ctypes.c_int64 * max(1, len(seq)))(*seq)
    return arr


def copy(src: np.ndarray, src_lay: Layout, dst: np.ndarray, dst_lay: Layout, elem_bytes: int,
         nthreads: int = 0) -> None:
    """The same definition, run by the C odometer in ``copy_ref.c`` (OpenMP over the
    outermost mode).  Buffers are flat, C-contiguous uint8 arrays."""
    assert src.dtype == np.uint8 and dst.dtype == np.uint8
    assert src.flags["C_CONTIGUOUS"] and dst.flags["C_CONTIGUOUS"] and dst.flags["WRITEABLE"]
    _check_bounds(src_lay, src.size // elem_bytes)
    _check_bounds(dst_lay, dst.size // elem_bytes)
    lib = _load_lib()
    (ss, sst, so), (ds, dstt, do) = src_lay, dst_lay
    rc = lib.oracle_copy(src.ctypes.data, len(ss), _i64(ss), _i64(sst), so,
                         dst.ctypes.data, len(ds), _i64(ds), _i64(dstt), do, elem_bytes, nthreads)
    if rc == -1:
        raise ValueError("extent mismatch")
    if rc != 0:
        raise ValueError(f"oracle_copy failed rc={rc}")


def max_threads() -> int:
    return _load_lib().oracle_max_threads()


def _check_bounds(lay: Layout, n_elems: int) -> None:
    shape, stride, off = lay
    if any(e == 0 for e in shape):
        return
    lo = off + sum((e - 1) * s for e, s in zip(shape, stride) if s < 0)
    hi = off + sum((e - 1) * s for e, s in zip(shape, stride) if s > 0)
    if lo < 0 or hi >= n_elems:
        raise ValueError(f"layout {lay} addresses [{lo}, {hi}] outside a buffer of {n_elems} elements")


def sample_offsets(src_lay: Layout, dst_lay: Layout, flat: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(src_offsets, dst_offsets) of the logical indices whose row-major flat number is
    ``flat`` -- for checking sampled outputs of copies too large to redo whole."""
    modes = common_modes(src_lay, dst_lay)
    extents = [e for e, _, _ in modes]
    flat = np.asarray(flat, dtype=np.int64)
    so = np.full(flat.shape, src_lay[2], dtype=np.int64)
    do = np.full(flat.shape, dst_lay[2], dtype=np.int64)
    rem = flat.copy()
    for k in range(len(extents) - 1, -1, -1):
        i = rem % extents[k]
        rem //= extents[k]
        so += i * modes[k][1]
        do += i * modes[k][2]
    return so, do


# ----------------------------------------------------------------------------------------------
# TileLang default loop partition (TileLang tutorial "loop_mapping.py", module docstring).  The
# points of the loop nest, taken in row-major order, are grouped into vectors of `vector_size`
# consecutive points; vector number a goes to thread a mod T, and a thread's vectors follow one
# another in its local slots, each vector's points in order.  Computed here for every point of the
# nest at once, as NumPy arrays shaped like the nest.
# ----------------------------------------------------------------------------------------------

def loop_partition_arrays(extents: Sequence[int], num_thread: int, vector_size: int):
    """(thread, slot): two integer arrays of shape ``extents``; entry [idx] is the thread that
    runs point idx and the local slot it uses."""
    shape = tuple(int(e) for e in extents)
    pos = np.arange(math.prod(shape), dtype=np.int64).reshape(shape)  # row-major position
    vector_no = pos // vector_size
    thread = vector_no % num_thread
    slot = (vector_no // num_thread) * vector_size + pos % vector_size
    return thread, slot


def loop_partition(extents: Sequence[int], num_thread: int,
                   vector_size: int) -> Dict[Tuple[int, ...], Tuple[int, int]]:
    """{point: (thread, slot)} for every point of the nest (see loop_partition_arrays)."""
    thread, slot = loop_partition_arrays(extents, num_thread, vector_size)
    return {idx: (int(thread[idx]), int(slot[idx])) for idx in np.ndindex(*thread.shape)}


# ----------------------------------------------------------------------------------------------
# [outer, threads, vec] partition of a global<->shared copy (TVM TIRx "copy -> gmem_smem",
# Algorithm 1-3): slice both sides to the region, let the global side drive the canonical
# (stride-descending) order, choose the widest vector of {128, 64, 32, 16, 8} bits whose
# elements are contiguous and naturally aligned on both sides, outer = count / (threads*vec).
# Declines when the element count does not divide the thread count ("What it accepts",
# divisibility row).
# ----------------------------------------------------------------------------------------------

VEC_BITS = (128, 64, 32, 16, 8)


def gmem_smem_partition(g_lay: Layout, s_lay: Layout, num_thread: int, elem_bytes: int,
                        vec_bits: Sequence[int] = VEC_BITS) -> dict:
    modes = common_modes(g_lay, s_lay)
    # global side drives the canonical order: modes sorted by |global stride|, descending (stable)
    order = sorted(range(len(modes)), key=lambda k: -abs(modes[k][1]))
    modes = [modes[k] for k in order]
    extents = [e for e, _, _ in modes]
    count = math.prod(extents) if extents else 1
    if count % num_thread != 0:
        return {"declined": True,
                "reason": f"element count {count} is not divisible by thread count {num_thread}"}

    def offsets(flat):
        idx = index_of_flat(flat, extents)
        g = g_lay[2] + sum(i * gs for i, (_, gs, _) in zip(idx, modes))
        s = s_lay[2] + sum(i * ss for i, (_, _, ss) in zip(idx, modes))
        return g, s

    chosen = None
    for bits in vec_bits:
        if bits % (8 * elem_bytes) != 0:
            continue
        vec = bits // (8 * elem_bytes)
        if count % (num_thread * vec) != 0:
            continue
        ok = True
        for start in range(0, count, vec):
            g0, s0 = offsets(start)
            if g0 % vec or s0 % vec:
                ok = False
                break
            for v in range(1, vec):
                g, s = offsets(start + v)
                if g != g0 + v or s != s0 + v:
                    ok = False
                    break
            if not ok:
                break
        if ok:
            chosen = vec
            break
    if chosen is None:  # an element-wide access always exists when count % threads == 0
        chosen = 1
    vec = chosen
    outer = count // (num_thread * vec)
    g_lin = [[0] * num_thread for _ in range(outer)]
    s_lin = [[0] * num_thread for _ in range(outer)]
    for f in range(outer):
        for t in range(num_thread):
            g_lin[f][t], s_lin[f][t] = offsets((f * num_thread + t) * vec)
    return {"declined": False, "outer": outer, "threads": num_thread, "vec": vec,
            "copy_bytes": vec * elem_bytes, "g_lin": g_lin, "s_lin": s_lin}


# ----------------------------------------------------------------------------------------------
# Bank models and conflict counting.
#
# A model gives, per (operation, access width in bytes), the number of 4-byte banks and how
# many consecutive lanes the hardware serves together.  Within one such lane group, a bank that
# must deliver n different 4-byte words costs n-1 extra cycles ("dword" rule: lanes asking for
# the same word share it); the "lane" rule instead counts every lane that touches the bank.
# An access is conflict-free when every group costs 0.
# ----------------------------------------------------------------------------------------------

class BankModel:
    def __init__(self, name: str, lanes: int, table: Dict[Tuple[str, int], Tuple[int, int]], rule: str):
        self.name, self.lanes, self.table, self.rule = name, lanes, table, rule

    def geometry(self, op: str, width: int) -> Tuple[int, int]:
        return self.table[(op, width)]


def _uniform_table(banks, lanes_by_width):
    return {(op, w): (banks, g) for op in ("read", "write") for w, g in lanes_by_width.items()}


def page_model(rule: str = "lane") -> BankModel:
    """NVIDIA-style shared memory the permute page simulates: 32 banks of 4 bytes, one
    32-lane warp (TVM TIRx "permute_layout": "one element per bank" for 4-byte dtypes).
    The page does not say how 8/16-byte accesses are split; the plainest reading is that a
    warp's request is served in as many 128-byte phases as it needs (16 / 8 lanes each)."""
    return BankModel(f"page32-{rule}", 32, _uniform_table(32, {1: 32, 2: 32, 4: 32, 8: 16, 16: 8}), rule)


def gfx950_model() -> BankModel:
    """gfx950 LDS as measured by the bank probe (cycles per access and SQ_LDS_BANK_CONFLICT per
    dispatch, every probe pattern matched): 1/2/4-byte reads and writes use 32 banks with 32
    lanes per group; 8-byte reads 64 banks x 32 lanes, 8-byte writes 32 banks x 16 lanes;
    16-byte reads 64 banks x 16 lanes, 16-byte writes 32 banks x 8 lanes; lanes that ask for
    the same dword share it."""
    table = {}
    for op in ("read", "write"):
        for w in (1, 2, 4):
            table[(op, w)] = (32, 32)
    table[("read", 8)] = (64, 32)
    table[("write", 8)] = (32, 16)
    table[("read", 16)] = (64, 16)
    table[("write", 16)] = (32, 8)
    return BankModel("gfx950", 64, table, "dword")


def conflict_cycles(byte_addrs: Sequence[int], width: int, op: str, model: BankModel,
                    active: Optional[Sequence[bool]] = None) -> int:
    """Extra cycles one access instruction costs under ``model``; byte_addrs[l] is lane l's
    address (lanes beyond len(byte_addrs) or with active[l] False do not access)."""
    banks, group = model.geometry(op, width)
    total = 0
    n = len(byte_addrs)
    for g0 in range(0, n, group):
        per_bank: Dict[int, set] = {}
        for lane in range(g0, min(n, g0 + group)):
            if active is not None and not active[lane]:
                continue
            a = byte_addrs[lane]
            first, last = a // 4, (a + width - 1) // 4
            for word in range(first, last + 1):
                key = word if model.rule == "dword" else (lane, word)
                per_bank.setdefault(word % banks, set()).add(key)
        worst = max((len(v) for v in per_bank.values()), default=1)
        total += max(0, worst - 1)
    return total


# ----------------------------------------------------------------------------------------------
# Register-staged permute with an XOR swizzle (TVM TIRx "permute_layout").
# ----------------------------------------------------------------------------------------------

def _canon_joint(modes):
    """Merge adjacent joint modes (outer o, inner n) when both sides allow it:
    stride_o == extent_n * stride_n on the source and on the destination."""
    out = []
    for e, s, d in modes:
        if out:
            pe, ps, pd = out[-1]
            if ps == e * s and pd == e * d:
                out[-1] = (pe * e, s, d)
                continue
        out.append((e, s, d))
    return out


def permute_shard(src_lay: Layout, dst_lay: Layout):
    """Algorithm step 1: slice/canonicalize both sides; the source is regrouped to the
    destination's shard.  Returns (extent, src_str, dst_str, src_base, dst_base).  A merge
    is taken only where both sides allow it, which is what regrouping one side onto the
    other's shard amounts to; the modes keep their logical order."""
    modes = _canon_joint(common_modes(src_lay, dst_lay))
    extent = tuple(e for e, _, _ in modes)
    return extent, tuple(s for _, s, _ in modes), tuple(d for _, _, d in modes), src_lay[2], dst_lay[2]


def xor_swizzle(off: int, bits: int, base: int, shift: int) -> int:
    """Element offset inside an XOR-swizzled shared layout (TVM TIRx "copy -> gmem_smem", closing
    remarks: a swizzle wraps the shared side's layout and a vector never spans more than one
    swizzle chunk).  The page does not print the function; the reading taken is the usual bit-field
    XOR: a chunk is 2**base consecutive elements, and the chunk-index bits [base, base + bits) are
    XORed with bits [base + shift, base + shift + bits) of the same offset (for a row of 2**shift
    chunks, the chunk index within a row XOR the row index modulo 2**bits)."""
    field = (off >> (base + shift)) & ((1 << bits) - 1)
    return off ^ (field << base)


def project(idx, st):
    return sum(i * s for i, s in zip(idx, st))


def permute_access(extent, src_str, dst_str, lanes, k, shift, r, lane):
    """(src offset, dst offset) lane ``lane`` touches at unrolled step ``r``:
    j = r ^ ((lane >> shift) & mask), idx = decompose(lane + j*lanes, extent)."""
    mask = (1 << k) - 1
    j = r ^ ((lane >> shift) & mask)
    idx = index_of_flat(lane + j * lanes, extent)
    return project(idx, src_str), project(idx, dst_str)


def _phase_conflicts(extent, strides, elem_bytes, model, k, shift, op):
    lanes = model.lanes
    P = math.prod(extent) // lanes
    worst = 0
    for r in range(P):
        addrs = []
        for lane in range(lanes):
            mask = (1 << k) - 1
            j = r ^ ((lane >> shift) & mask)
            idx = index_of_flat(lane + j * lanes, extent)
            addrs.append(project(idx, strides) * elem_bytes)
        worst += conflict_cycles(addrs, elem_bytes, op, model)
    return worst


def choose_xor_k(extent, src_str, dst_str, elem_bytes, model: Optional[BankModel] = None):
    """Algorithm step 2 (``_choose_xor_k``): P = prod(extent) / lanes; for k = 0..log2(P) take
    the first k (and, for it, the first shift) whose swizzle leaves both the read phase
    (source layout) and the write phase (destination layout) conflict-free.  mask = 2^k - 1.
    Returns (k, shift, mask) or None (the dispatch declines).

    The page prints only the result for its demo; the shift search range [0, log2(lanes) - k]
    (ascending, smallest k first) is the plainest reading that reproduces it."""
    model = model or page_model()
    lanes = model.lanes
    total = math.prod(extent)
    if total % lanes:
        return None
    P = total // lanes
    log2p = P.bit_length() - 1
    kmax = log2p if (1 << log2p) == P else 0  # an XOR of k>0 bits permutes [0, P) only for P = 2^m
    log2l = lanes.bit_length() - 1
    for k in range(0, kmax + 1):
        shifts = [0] if k == 0 else range(0, log2l - k + 1)
        for shift in shifts:
            if (_phase_conflicts(extent, src_str, elem_bytes, model, k, shift, "read") == 0 and
                    _phase_conflicts(extent, dst_str, elem_bytes, model, k, shift, "write") == 0):
                return k, shift, (1 << k) - 1
    return None


def permute_conflicts(extent, src_str, dst_str, elem_bytes, k, shift, model=None):
    """(read-phase, write-phase) extra cycles summed over the P unrolled steps."""
    model = model or page_model()
    return (_phase_conflicts(extent, src_str, elem_bytes, model, k, shift, "read"),
            _phase_conflicts(extent, dst_str, elem_bytes, model, k, shift, "write"))


def permute_layout_py(src: np.ndarray, src_lay: Layout, dst: np.ndarray, dst_lay: Layout,
                      elem_bytes: int, lanes: int, k: int, shift: int) -> None:
    """Algorithm step 3 executed literally on flat byte buffers: every lane reads its P elements
    (swizzled order) through the source layout into registers, then writes them through the
    destination layout.  Used to show the swizzle does not change the result."""
    extent, ss, ds, sb, db = permute_shard(src_lay, dst_lay)
    P = math.prod(extent) // lanes
    regs = {}
    for lane in range(lanes):
        for r in range(P):
            so, _ = permute_access(extent, ss, ds, lanes, k, shift, r, lane)
            so += sb
            regs[(lane, r)] = src[so * elem_bytes:(so + 1) * elem_bytes].copy()
    for lane in range(lanes):
        for r in range(P):
            _, do = permute_access(extent, ss, ds, lanes, k, shift, r, lane)
            do += db
            dst[do * elem_bytes:(do + 1) * elem_bytes] = regs[(lane, r)]


# ----------------------------------------------------------------------------------------------
# LDS tile of the global -> LDS -> global transpose on gfx950 (the library's kernel design; the
# pages fix the method -- the [outer, threads, vec] partition of each phase and the smallest-k XOR
# search over both phases -- but not this tile, so it is pinned by the hardware instead of printed
# values: SQ_LDS_BANK_CONFLICT and SQ_INSTS_LDS per dispatch of the kernel, on tiles with the
# swizzle off, with swizzles the search passes over and with the chosen ones, equal what the
# functions below simulate, non-zero counts included; and by a hand-derived closed form).
#
# The tile holds NB x TR x TC elements (TR along the destination-contiguous mode, TC along the
# source-contiguous mode).  In LDS it is a grid of units of U bytes (U in {4, 8, 16}, U >= eb,
# default max(eb, 4)): a unit is one column of B = U/eb consecutive rows.  Unit (nb, ru, c) is
# stored at byte ((nb*TRu + ru)*TC + chunk'*CW + c % CW) * U, where CW units form one LDS write
# (WW = min(16, VE*U) bytes), chunk = c // CW and
#     chunk' = chunk ^ (((ru >> shift) & (2^k - 1)) << tbit) ^ ((chunk >> cshift) & cmask).
# Load phase: the TileLang partition of the unit grid (NB, TRu, TC) in source order, vector VE
# units, NT threads; each write instruction stores CW consecutive units of a thread's vector.
# Store phase: the TileLang partition of the unit grid (NB, TC, TRu) in destination order, vector
# RPV = vb / U units; each read instruction loads one unit.
# ----------------------------------------------------------------------------------------------

def _tile_units(eb, vb, TR, TC, NB, U=None):
    U = U or max(eb, 4)
    B = U // eb
    VE = vb // eb
    WW = min(16, VE * U)
    return U, B, VE, WW // U, vb // U, TR // B, WW


def _tile_instructions(eb, vb, TR, TC, NB, NT, U=None):
    """[(op, width, {thread: (nb, ru, c)})] for every LDS instruction of the tile, from the
    TileLang partitions of both phases."""
    U, B, VE, CW, RPV, TRu, WW = _tile_units(eb, vb, TR, TC, NB, U)
    insts = {}
    for (nb, ru, c), (t, slot) in loop_partition((NB, TRu, TC), NT, VE).items():
        if slot % CW == 0:  # first unit of a write instruction
            insts.setdefault(("write", slot // CW), {})[t] = (nb, ru, c)
    for (nb, c, ru), (t, slot) in loop_partition((NB, TC, TRu), NT, RPV).items():
        insts.setdefault(("read", slot), {})[t] = (nb, ru, c)
    out = []
    for (op, _), lanes in sorted(insts.items()):
        out.append((op, WW if op == "write" else U, lanes))
    return out


def tile_wave_local(eb, vb, TR, TC, NB, NT, U=None, wave=64):
    """Whether every LDS unit a wave reads in the store phase was written by that same wave in the
    load phase, under the two TileLang partitions of the tile (then the phases need no
    workgroup-wide barrier, only ordering within each wave).  Positions are logical (nb, row
    unit, column): an XOR swizzle permutes addresses one to one and does not change the answer."""
    U, B, VE, CW, RPV, TRu, WW = _tile_units(eb, vb, TR, TC, NB, U)
    owner = {}
    for op, width, lanes in _tile_instructions(eb, vb, TR, TC, NB, NT, U):
        if op == "write":
            for t, (nb, ru, c) in lanes.items():
                for u in range(CW):
                    owner[(nb, ru, c + u)] = t // wave
    for op, width, lanes in _tile_instructions(eb, vb, TR, TC, NB, NT, U):
        if op == "read":
            for t, pos in lanes.items():
                if owner.get(pos) != t // wave:
                    return False
    return True


def lds_tile_wave_instructions(eb, vb, TR, TC, NB, NT=256, U=None, wave=64):
    """LDS instructions one tile issues, counted per wave (an instruction of a wave with at least
    one lane that accesses LDS), over both phases."""
    total = 0
    for op, width, lanes in _tile_instructions(eb, vb, TR, TC, NB, NT, U):
        total += len({t // wave for t in lanes})
    return total


_TILE_CACHE = {}


def lds_tile_conflicts(eb, vb, TR, TC, NB, NT=256, k=0, shift=0, tbit=0, cshift=0, cmask=0,
                       model=None, stop_at_first=False, U=None):
    """(write-phase, read-phase) extra LDS cycles of one tile under the gfx950 model."""
    model = model or gfx950_model()
    key = (eb, vb, TR, TC, NB, NT, U)
    if key not in _TILE_CACHE:
        _TILE_CACHE[key] = _tile_instructions(eb, vb, TR, TC, NB, NT, U)
    U, B, VE, CW, RPV, TRu, WW = _tile_units(eb, vb, TR, TC, NB, U)
    mask = (1 << k) - 1

    def addr(nb, ru, c):
        ch = c // CW
        chs = ch ^ (((ru >> shift) & mask) << tbit) ^ ((ch >> cshift) & cmask)
        return ((nb * TRu + ru) * TC + chs * CW + c % CW) * U

    wc = rc = 0
    for op, width, lanes in _TILE_CACHE[key]:
        for w0 in range(0, NT, model.lanes):
            wave = [lanes.get(t) for t in range(w0, w0 + model.lanes)]
            if all(x is None for x in wave):
                continue
            addrs = [addr(*x) if x is not None else 0 for x in wave]
            cyc = conflict_cycles(addrs, width, op, model, active=[x is not None for x in wave])
            if op == "write":
                wc += cyc
            else:
                rc += cyc
            if stop_at_first and cyc:
                return wc, rc
    return wc, rc


def lds_tile_candidates(eb, vb, TR, TC, NB, U=None):
    """The swizzles of the tile in the search order (the permute page's Algorithm step 2: k
    ascending; for each k the row shift, then the target bit, then the column term -- none, then
    (cshift, cmask) by increasing cshift and cmask in (1, 3, 7)).  Yields dicts."""
    U, B, VE, CW, RPV, TRu, WW = _tile_units(eb, vb, TR, TC, NB, U)
    chunks = TC // CW
    chunk_bits = chunks.bit_length() - 1
    row_bits = TRu.bit_length() - 1
    cols = [(0, 0)] + [(cs, cm) for cs in range(1, chunk_bits) for cm in (1, 3, 7) if cm < (1 << cs)]
    for k in range(0, chunk_bits + 1):
        for shift in (range(0, max(0, row_bits - 1) + 1) if k else [0]):
            for tbit in (range(0, chunk_bits - k + 1) if k else [0]):
                if k and (1 << (k + tbit)) > chunks:
                    continue
                for cs, cm in cols:
                    if cm and (1 << cs) >= chunks:
                        continue
                    yield {"k": k, "shift": shift, "tbit": tbit, "cshift": cs, "cmask": cm, "mask": (1 << k) - 1}


def lds_tile_swizzle(eb, vb, TR, TC, NB, NT=256, model=None, U=None):
    """Smallest-k XOR swizzle of the tile that leaves both phases conflict-free (the first such
    candidate of lds_tile_candidates).  Returns a dict, or None when no candidate is
    conflict-free."""
    for c in lds_tile_candidates(eb, vb, TR, TC, NB, U):
        w, r = lds_tile_conflicts(eb, vb, TR, TC, NB, NT, c["k"], c["shift"], c["tbit"], c["cshift"], c["cmask"],
                                  model, stop_at_first=True, U=U)
        if w == 0 and r == 0:
            return c
    return None


def lds_tile_cheapest_per_k(eb, vb, TR, TC, NB, NT=256, model=None, U=None):
    """{k: (candidate, write cycles, read cycles)}: for every k, the first candidate in search order
    with the fewest extra cycles per tile."""
    best = {}
    for c in lds_tile_candidates(eb, vb, TR, TC, NB, U):
        w, r = lds_tile_conflicts(eb, vb, TR, TC, NB, NT, c["k"], c["shift"], c["tbit"], c["cshift"], c["cmask"],
                                  model, U=U)
        if c["k"] not in best or w + r < sum(best[c["k"]][1:]):
            best[c["k"]] = (c, w, r)
    return best
