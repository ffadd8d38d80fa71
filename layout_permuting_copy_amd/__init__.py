"""Layout-permuting tile copy for AMD MI355X (gfx950): Python binding of libtile_copy.so.

Thin ctypes marshalling over the C ABI declared in ``include/tile_copy.h``; every step of
the copy (planning, kernels) runs in the native library.  Names match the C entry points:
``tile_copy``, ``tile_copy_ex``, ``tc_plan``, ``tc_last_error``, ``tc_set_flags``,
``tc_get_flags``, ``tc_layout_slice``, ``tc_version``.

Layouts are ``(shape, stride, offset)`` tuples in elements (TileLayout S[shape : stride]),
or ``TcLayout`` structs.  Source and destination are device pointers (ints) or torch
tensors (their ``data_ptr()`` is the base the layout offsets count from).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtile_copy.so")

TC_MAX_RANK = 8

# dtypes (enum tc_dtype)
TC_U8, TC_I8, TC_F16, TC_BF16, TC_F32, TC_I32, TC_F64, TC_I64, TC_B128 = range(9)
ELEM_BYTES = {TC_U8: 1, TC_I8: 1, TC_F16: 2, TC_BF16: 2, TC_F32: 4, TC_I32: 4, TC_F64: 8, TC_I64: 8, TC_B128: 16}
DTYPE_BY_NAME = {"uint8": TC_U8, "int8": TC_I8, "float16": TC_F16, "bfloat16": TC_BF16, "float32": TC_F32,
                 "int32": TC_I32, "float64": TC_F64, "int64": TC_I64, "int4vec": TC_B128}

# status codes (enum tc_status)
TC_OK = 0
TC_E_NULL, TC_E_RANK, TC_E_EXTENT, TC_E_DTYPE, TC_E_ALIGN, TC_E_NONINJECTIVE, TC_E_ALIAS, \
    TC_E_DECLINED, TC_E_HIP, TC_E_RANGE, TC_E_ARG = range(-1, -12, -1)
STATUS_NAMES = {0: "TC_OK", -1: "TC_E_NULL", -2: "TC_E_RANK", -3: "TC_E_EXTENT", -4: "TC_E_DTYPE",
                -5: "TC_E_ALIGN", -6: "TC_E_NONINJECTIVE", -7: "TC_E_ALIAS", -8: "TC_E_DECLINED",
                -9: "TC_E_HIP", -10: "TC_E_RANGE", -11: "TC_E_ARG"}

# flags
TC_FLAG_STRICT = 0x01
TC_FLAG_FORCE_GUARDED = 0x02
TC_FLAG_FORCE_REGS = 0x04
TC_FLAG_FORCE_LDS = 0x08
TC_FLAG_NO_SWIZZLE = 0x10
TC_FLAG_NO_SHUFFLE = 0x20

# paths (enum tc_path)
TC_PATH_EMPTY, TC_PATH_TRANSPOSE, TC_PATH_ROWS, TC_PATH_ROUNDTRIP, TC_PATH_GUARDED_TILE, \
    TC_PATH_GUARDED_ROWS, TC_PATH_SHUFFLE, TC_PATH_INTERLEAVE = range(8)
PATH_NAMES = {0: "empty", 1: "transpose", 2: "rows", 3: "roundtrip", 4: "guarded_tile", 5: "guarded_rows",
              6: "shuffle", 7: "interleave"}


class TcLayout(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("reserved", ctypes.c_int32), ("offset", ctypes.c_int64),
                ("shape", ctypes.c_int64 * TC_MAX_RANK), ("stride", ctypes.c_int64 * TC_MAX_RANK)]

    def as_tuple(self):
        r = self.rank
        return tuple(self.shape[:r]), tuple(self.stride[:r]), int(self.offset)


class TcPlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("elem_bytes", ctypes.c_int32), ("count", ctypes.c_int64),
                ("rank", ctypes.c_int32), ("declined", ctypes.c_int32),
                ("extent", ctypes.c_int64 * TC_MAX_RANK), ("src_stride", ctypes.c_int64 * TC_MAX_RANK),
                ("dst_stride", ctypes.c_int64 * TC_MAX_RANK), ("src_offset", ctypes.c_int64),
                ("dst_offset", ctypes.c_int64), ("threads", ctypes.c_int32), ("vec_bytes", ctypes.c_int32),
                ("load_outer", ctypes.c_int32), ("store_outer", ctypes.c_int32), ("mode_r", ctypes.c_int32),
                ("mode_c", ctypes.c_int32), ("mode_b", ctypes.c_int32), ("tile_r", ctypes.c_int32),
                ("tile_c", ctypes.c_int32), ("tile_b", ctypes.c_int32), ("workgroups", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int32), ("xor_k", ctypes.c_int32), ("xor_shift", ctypes.c_int32),
                ("xor_mask", ctypes.c_int32), ("xor_tbit", ctypes.c_int32), ("xor_cshift", ctypes.c_int32),
                ("xor_cmask", ctypes.c_int32), ("grid_order", ctypes.c_int32), ("nontemporal", ctypes.c_int32),
                ("unaligned", ctypes.c_int32), ("src_step", ctypes.c_int32), ("wave_local", ctypes.c_int32),
                ("lds_write_bytes", ctypes.c_int32), ("lds_read_bytes", ctypes.c_int32), ("edge_tiles", ctypes.c_int32),
                ("loads_in_flight", ctypes.c_int32), ("super_rows", ctypes.c_int32), ("super_cols", ctypes.c_int32),
                ("src_view_bytes", ctypes.c_int32),
                ("write_conflicts", ctypes.c_int64),
                ("read_conflicts", ctypes.c_int64), ("reason", ctypes.c_char * 192)]

    def to_dict(self) -> dict:
        d = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            if name == "reason":
                v = v.decode()
            elif name in ("extent", "src_stride", "dst_stride"):
                v = tuple(v[: self.rank])
            d[name] = v
        d["path_name"] = PATH_NAMES.get(self.path, "?")
        return d


class TcPermuteInfo(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("elements_per_lane", ctypes.c_int32),
                ("extent", ctypes.c_int64 * TC_MAX_RANK), ("src_stride", ctypes.c_int64 * TC_MAX_RANK),
                ("dst_stride", ctypes.c_int64 * TC_MAX_RANK), ("k", ctypes.c_int32), ("shift", ctypes.c_int32),
                ("mask", ctypes.c_int32), ("reserved", ctypes.c_int32), ("read_conflicts", ctypes.c_int64),
                ("write_conflicts", ctypes.c_int64), ("reason", ctypes.c_char * 192)]

    def to_dict(self) -> dict:
        d = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            if name == "reason":
                v = v.decode()
            elif name in ("extent", "src_stride", "dst_stride"):
                v = tuple(v[: self.rank])
            d[name] = v
        return d


class TileCopyError(RuntimeError):
    def __init__(self, code: int, reason: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {reason}")
        self.code = code
        self.reason = reason


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libtile_copy.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python layout_permuting_copy_amd/build.py` "
                          "(or __graft_entry__.build()); the copy has no non-native fallback")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.tile_copy.argtypes = [ctypes.c_void_p, P(TcLayout), ctypes.c_void_p, P(TcLayout), ctypes.c_int, ctypes.c_void_p]
    lib.tile_copy.restype = ctypes.c_int
    lib.tile_copy_ex.argtypes = [ctypes.c_void_p, P(TcLayout), ctypes.c_void_p, P(TcLayout), ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_int, P(TcPlanInfo)]
    lib.tile_copy_ex.restype = ctypes.c_int
    lib.tc_autotune.argtypes = [ctypes.c_void_p, P(TcLayout), ctypes.c_void_p, P(TcLayout), ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_int, ctypes.c_int, P(TcPlanInfo), P(ctypes.c_float)]
    lib.tc_autotune.restype = ctypes.c_int
    lib.tc_plan_variants.argtypes = [P(TcLayout), P(TcLayout), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     P(TcPlanInfo), ctypes.c_int]
    lib.tc_plan_variants.restype = ctypes.c_int
    lib.tc_plan.argtypes = [P(TcLayout), P(TcLayout), ctypes.c_int, ctypes.c_int, ctypes.c_int, P(TcPlanInfo)]
    lib.tc_plan.restype = ctypes.c_int
    lib.tc_last_error.argtypes = []
    lib.tc_last_error.restype = ctypes.c_char_p
    lib.tc_set_flags.argtypes = [ctypes.c_int]
    lib.tc_set_flags.restype = ctypes.c_int
    lib.tc_get_flags.argtypes = []
    lib.tc_get_flags.restype = ctypes.c_int
    i64p = P(ctypes.c_int64)
    lib.tc_layout_slice.argtypes = [P(TcLayout), i64p, i64p, i64p, P(TcLayout)]
    lib.tc_layout_slice.restype = ctypes.c_int
    lib.tc_version.argtypes = []
    lib.tc_version.restype = ctypes.c_int
    lib.tc_wave_permute_plan.argtypes = [P(TcLayout), P(TcLayout), ctypes.c_int, P(TcPermuteInfo)]
    lib.tc_wave_permute_plan.restype = ctypes.c_int
    _lib = lib
    return lib


LayoutLike = Union[TcLayout, Tuple[Sequence[int], Sequence[int], int], Tuple[Sequence[int], Sequence[int]]]


def make_layout(shape: Sequence[int], stride: Optional[Sequence[int]] = None, offset: int = 0) -> TcLayout:
    """TileLayout S[shape : stride] with an element offset (row-major strides by default)."""
    shape = [int(e) for e in shape]
    if stride is None:
        stride, acc = [], 1
        for e in reversed(shape):
            stride.append(acc)
            acc *= e
        stride.reverse()
    if len(shape) != len(stride) or len(shape) > TC_MAX_RANK:
        raise ValueError("shape and stride must have the same length, at most 8")
    lay = TcLayout()
    lay.rank = len(shape)
    lay.offset = int(offset)
    for k, (e, s) in enumerate(zip(shape, stride)):
        lay.shape[k] = e
        lay.stride[k] = int(s)
    return lay


def _as_layout(x: LayoutLike) -> TcLayout:
    if isinstance(x, TcLayout):
        return x
    if len(x) == 2:
        return make_layout(x[0], x[1], 0)
    return make_layout(x[0], x[1], x[2])


def _ptr(x) -> int:
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError("expected a device pointer (int) or a tensor")


def _stream(stream) -> int:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except ImportError:
            pass
        return 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def tc_last_error() -> str:
    return load_library().tc_last_error().decode()


def _check(rc: int) -> int:
    if rc != TC_OK:
        raise TileCopyError(rc, tc_last_error())
    return rc


def tile_copy(src, src_layout: LayoutLike, dst, dst_layout: LayoutLike, dtype: int, stream=None) -> None:
    """dst[dst_layout(i)] = src[src_layout(i)] for every logical index i, on `stream`
    (default: torch's current stream).  Raises TileCopyError on a non-zero status."""
    lib = load_library()
    s, d = _as_layout(src_layout), _as_layout(dst_layout)
    _check(lib.tile_copy(_ptr(src), ctypes.byref(s), _ptr(dst), ctypes.byref(d), int(dtype), _stream(stream)))


def tile_copy_ex(src, src_layout: LayoutLike, dst, dst_layout: LayoutLike, dtype: int, stream=None,
                 flags: int = 0) -> dict:
    """tile_copy with explicit flags; returns the plan that ran (as a dict)."""
    lib = load_library()
    s, d = _as_layout(src_layout), _as_layout(dst_layout)
    info = TcPlanInfo()
    _check(lib.tile_copy_ex(_ptr(src), ctypes.byref(s), _ptr(dst), ctypes.byref(d), int(dtype), _stream(stream),
                            int(flags), ctypes.byref(info)))
    return info.to_dict()


def tc_autotune(src, src_layout: LayoutLike, dst, dst_layout: LayoutLike, dtype: int, stream=None, flags: int = 0,
                reps: int = 5) -> dict:
    """tile_copy_ex that times the copy on the library's candidate configurations and keeps the
    fastest as the cached plan of these layouts; returns that plan, with its mean time per launch
    in 'tuned_ms'.  Blocks until the timed launches end."""
    lib = load_library()
    s, d = _as_layout(src_layout), _as_layout(dst_layout)
    info = TcPlanInfo()
    ms = ctypes.c_float(0.0)
    _check(lib.tc_autotune(_ptr(src), ctypes.byref(s), _ptr(dst), ctypes.byref(d), int(dtype), _stream(stream),
                           int(flags), int(reps), ctypes.byref(info), ctypes.byref(ms)))
    out = info.to_dict()
    out["tuned_ms"] = float(ms.value)
    return out


def tc_plan(src_layout: LayoutLike, dst_layout: LayoutLike, dtype: int, flags: int = 0, ptr_align: int = 16,
            raise_on_error: bool = True) -> dict:
    """Host-only plan of a copy (no GPU).  With raise_on_error=False the dict carries
    'status' and 'error' instead of raising."""
    lib = load_library()
    s, d = _as_layout(src_layout), _as_layout(dst_layout)
    info = TcPlanInfo()
    rc = lib.tc_plan(ctypes.byref(s), ctypes.byref(d), int(dtype), int(flags), int(ptr_align), ctypes.byref(info))
    out = info.to_dict()
    out["status"] = rc
    out["error"] = tc_last_error() if rc != TC_OK else ""
    if rc != TC_OK and raise_on_error:
        raise TileCopyError(rc, out["error"])
    return out


def tc_plan_variants(src_layout: LayoutLike, dst_layout: LayoutLike, dtype: int, flags: int = 0,
                     ptr_align: int = 16, max_out: int = 64) -> list:
    """Host-only list of the plans tc_autotune would time (the planner's own first)."""
    lib = load_library()
    s, d = _as_layout(src_layout), _as_layout(dst_layout)
    arr = (TcPlanInfo * max_out)()
    n = lib.tc_plan_variants(ctypes.byref(s), ctypes.byref(d), int(dtype), int(flags), int(ptr_align), arr,
                             int(max_out))
    if n < 0:
        raise TileCopyError(n, tc_last_error())
    return [arr[i].to_dict() for i in range(min(n, max_out))]


def tc_set_flags(flags: int) -> int:
    rc = load_library().tc_set_flags(int(flags))
    if rc < 0:
        raise TileCopyError(rc, tc_last_error())
    return rc


def tc_get_flags() -> int:
    return load_library().tc_get_flags()


def tc_layout_slice(layout: LayoutLike, start: Sequence[int], stop: Sequence[int], step: Sequence[int]) -> TcLayout:
    lib = load_library()
    lay = _as_layout(layout)
    n = max(1, lay.rank)
    arr = lambda xs: (ctypes.c_int64 * n)(*[int(x) for x in xs])
    out = TcLayout()
    _check(lib.tc_layout_slice(ctypes.byref(lay), arr(start), arr(stop), arr(step), ctypes.byref(out)))
    return out


def tc_version() -> int:
    return load_library().tc_version()


def tc_wave_permute_plan(src_layout: LayoutLike, dst_layout: LayoutLike, dtype: int,
                         raise_on_error: bool = True) -> dict:
    """Host-only bank plan (k, shift, mask) of the wave-scope permute tcd::wave_permute."""
    lib = load_library()
    s, d = _as_layout(src_layout), _as_layout(dst_layout)
    info = TcPermuteInfo()
    rc = lib.tc_wave_permute_plan(ctypes.byref(s), ctypes.byref(d), int(dtype), ctypes.byref(info))
    out = info.to_dict()
    out["status"] = rc
    out["error"] = tc_last_error() if rc != TC_OK else ""
    if rc != TC_OK and raise_on_error:
        raise TileCopyError(rc, out["error"])
    return out


def torch_dtype_code(torch_dtype) -> int:
    """enum tc_dtype of a torch dtype (by width; the copy moves raw bytes)."""
    import torch
    table = {torch.uint8: TC_U8, torch.int8: TC_I8, torch.float16: TC_F16, torch.bfloat16: TC_BF16,
             torch.float32: TC_F32, torch.int32: TC_I32, torch.float64: TC_F64, torch.int64: TC_I64,
             torch.int16: TC_F16, torch.uint16: TC_F16 if hasattr(torch, "uint16") else TC_F16}
    return table[torch_dtype]


def copy_tensor(dst, src, stream=None) -> dict:
    """dst[...] = src[...] for two device tensors of the same shape and element width, through
    their own strides (views: transposes, permutes, slices, expanded sources): the layouts are the
    tensors' shape and strides from their data pointers.  Returns the plan that ran."""
    if tuple(dst.shape) != tuple(src.shape):
        raise ValueError(f"shapes differ: {tuple(dst.shape)} and {tuple(src.shape)}")
    if dst.element_size() != src.element_size():
        raise ValueError("element widths differ")
    code = torch_dtype_code(src.dtype)
    shape = tuple(int(e) for e in src.shape)
    return tile_copy_ex(src, (shape, tuple(int(s) for s in src.stride()), 0), dst,
                        (shape, tuple(int(s) for s in dst.stride()), 0), code, stream)
