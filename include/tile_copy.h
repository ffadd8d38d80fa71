/*
 * tile_copy.h -- layout-permuting tile copy for AMD MI355X (gfx950), C ABI.
 *
 * The operation (TVM TIRx docs, "copy -> gmem_smem" intro and "What it accepts";
 * "permute_layout" intro): a region described by a source shape:stride
 * TileLayout is copied to a destination TileLayout.  A layout maps a logical
 * index i = (i_0 .. i_{r-1}) to the element offset
 *
 *     offset + sum_k i_k * stride_k
 *
 * and the copy writes, for every logical index i of the common shape,
 *
 *     dst[dst_layout(i)] = src[src_layout(i)]
 *
 * as raw element bytes (no conversion; floating point payloads, NaNs and
 * denormals are moved as bit patterns).  Extent-1 modes are ignored on both
 * sides; the remaining extents must be equal and in the same order.  Bytes of
 * the destination buffer that no logical index names are not written.
 *
 * The work runs on the GPU: global -> LDS -> global through a synthesized
 * [outer, threads, vec] thread partition (TVM TIRx "copy -> gmem_smem",
 * Algorithm; TileLang tutorial "loop_mapping.py", the partition formula) and an
 * XOR-swizzled LDS stage chosen by simulating gfx950's LDS banks (TVM TIRx
 * "permute_layout", Algorithm step 2).  The host part (layout algebra,
 * partition planner, swizzle chooser) is exposed through tc_plan for
 * inspection; it needs no GPU.
 *
 * Thread safety: all entry points may be called from several host threads;
 * plans are cached in a library-owned, locked cache.  The error string is
 * per host thread.
 */
#ifndef TILE_COPY_H
#define TILE_COPY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TC_MAX_RANK 8

/*
 * A TileLayout, S[shape : stride] (TVM TIRx "copy -> gmem_smem", demonstration
 * program).  All quantities are in elements of the copy's dtype.
 *   rank    number of modes, 0..TC_MAX_RANK (rank 0 = one element)
 *   offset  element offset of logical index (0, .., 0) from the base pointer;
 *           region slices fold into it (see tc_layout_slice)
 *   shape   extents, >= 0 (an extent of 0 makes the copy empty)
 *   stride  element strides; a source stride may be 0 (broadcast read) or
 *           negative; destination strides must make the layout injective
 * Only the first `rank` entries of shape/stride are read.
 */
typedef struct tc_layout {
  int32_t rank;
  int32_t reserved;
  int64_t offset;
  int64_t shape[TC_MAX_RANK];
  int64_t stride[TC_MAX_RANK];
} tc_layout;

/* Element types.  Only the width matters: 1, 2, 4, 8 or 16 bytes
 * (TVM TIRx "permute_layout", "What it accepts": dtype byte width in
 * {1, 2, 4, 8, 16}).  TC_B128 is a 16-byte struct such as four int32. */
enum tc_dtype {
  TC_U8 = 0, TC_I8 = 1, TC_F16 = 2, TC_BF16 = 3, TC_F32 = 4, TC_I32 = 5,
  TC_F64 = 6, TC_I64 = 7, TC_B128 = 8
};

/* Return codes: 0 = success, negative = error (tc_last_error() has the reason). */
enum tc_status {
  TC_OK = 0,
  TC_E_NULL = -1,          /* a required pointer is null */
  TC_E_RANK = -2,          /* rank outside 0..TC_MAX_RANK */
  TC_E_EXTENT = -3,        /* negative extent, or non-unit extents differ */
  TC_E_DTYPE = -4,         /* unknown dtype */
  TC_E_ALIGN = -5,         /* a base pointer is not aligned to the element size */
  TC_E_NONINJECTIVE = -6,  /* two logical indices map to one destination element */
  TC_E_ALIAS = -7,         /* the source and destination byte ranges overlap */
  TC_E_DECLINED = -8,      /* strict mode: no integer [outer, threads, vec] partition,
                              no vector of >= 4 bytes, or no conflict-free swizzle */
  TC_E_HIP = -9,           /* a HIP runtime call failed (launch or device query) */
  TC_E_RANGE = -10,        /* sizes beyond what the kernels index: a transpose of 2^31 tiles or
                              more, a row-wise copy one of whose outermost indices holds more
                              than 2^30 vectors (copies of 2^31 vectors and more otherwise run
                              as several launches on the stream), or an element count or element
                              offset beyond 2^58 (checked before anything else is computed) */
  TC_E_ARG = -11           /* other invalid argument (bad slice, unknown flag) */
};

/* Flags for tc_set_flags / tc_plan.  Unknown bits are rejected (TC_E_ARG). */
#define TC_FLAG_STRICT        0x01 /* the pages' acceptance rules as written: decline
                                      (TC_E_DECLINED) where TVM TIRx "copy -> gmem_smem", "What it
                                      accepts", rejects the copy (element count not divisible by
                                      the thread count; no aligned vector of 16, 8 or 4 bytes) or
                                      where no XOR swizzle is conflict-free ("permute_layout",
                                      "What it accepts": the dispatch fails if no k is found),
                                      instead of falling back (to the transpose with unaligned
                                      vectors, or the guarded paths) */
#define TC_FLAG_FORCE_GUARDED 0x02 /* always take the guarded element-wise path */
#define TC_FLAG_FORCE_REGS    0x04 /* co-contiguous copies: stage through registers only */
#define TC_FLAG_FORCE_LDS     0x08 /* co-contiguous copies: stage through LDS */
#define TC_FLAG_NO_SWIZZLE    0x10 /* transposes: no XOR swizzle (k = 0), to measure its effect */
#define TC_FLAG_NO_SHUFFLE    0x20 /* the LDS tile kernel instead of the register paths (the 4-row
                                      butterfly, the channel interleave), to measure their effect */
#define TC_FLAG_ALL           0x3f

/* Which kernel a plan runs. */
enum tc_path {
  TC_PATH_EMPTY = 0,       /* nothing to copy */
  TC_PATH_TRANSPOSE = 1,   /* the source- and destination-contiguous modes differ:
                              LDS tile, 16/8/4-byte vectors, XOR swizzle */
  TC_PATH_ROWS = 2,        /* both sides contiguous along the same mode: vectors staged in
                              registers (no LDS needed); also a destination contiguous along the
                              innermost mode with a source stepping 2, 3 or 4 elements along it
                              (src_step): each vector gathered from 16-byte loads of the source
                              bytes between its first and last element */
  TC_PATH_ROUNDTRIP = 3,   /* co-contiguous and small: one workgroup, global -> LDS ->
                              global with the [outer, threads, vec] partition */
  TC_PATH_GUARDED_TILE = 4,/* fallback: LDS tile with element-wide accesses and guards */
  TC_PATH_GUARDED_ROWS = 5,/* fallback: element-wise, destination order, guarded */
  TC_PATH_SHUFFLE = 6,     /* batches of 4 x C blocks of 4-byte elements (C = 8, 16, 32), each
                              block contiguous on both sides (e.g. the scale-factor tiles):
                              16-byte vectors exchanged between lanes by a two-stage butterfly,
                              no LDS (a v_permlane16_swap row swap at lane distance 16, bank-masked
                              DPP row rotations at distances 8 and 4, ds_swizzle only at
                              distance 2) */
  TC_PATH_INTERLEAVE = 7   /* a few (2, 3, 4 or 8) interleaved channels to planes or back (e.g.
                              NHWC <-> NCHW with 3 channels): each lane moves 16/elem_bytes
                              pixels of every channel, transposed within its registers */
};

/*
 * What the planner decided, for inspection and tests (filled by tc_plan, and by
 * tile_copy_ex).  Modes are the joint canonical modes (extent, src stride, dst
 * stride), outermost first in destination-stride order.
 */
typedef struct tc_plan_info {
  int32_t path;             /* enum tc_path */
  int32_t elem_bytes;
  int64_t count;            /* elements copied */
  int32_t rank;             /* joint canonical rank */
  int32_t declined;         /* 1 if the aligned [outer, threads, vec] split was declined (reason below) */
  int64_t extent[TC_MAX_RANK];
  int64_t src_stride[TC_MAX_RANK];
  int64_t dst_stride[TC_MAX_RANK];
  int64_t src_offset, dst_offset;
  /* partition: per workgroup, [outer, threads, vec] in each phase */
  int32_t threads;          /* threads per workgroup (multiple of 64) */
  int32_t vec_bytes;        /* bytes per global access (16, 8, 4, or the element size) */
  int32_t load_outer;       /* accesses per thread in the load phase (global -> LDS/regs) */
  int32_t store_outer;      /* accesses per thread in the store phase (LDS/regs -> global) */
  /* tile (transpose paths): index of the modes and tile extents in elements */
  int32_t mode_r, mode_c, mode_b; /* dst-contiguous mode, src-contiguous (or stride-2) mode, batch
                                     mode (-1 none) */
  int32_t tile_r, tile_c, tile_b;
  int64_t workgroups;       /* workgroups launched */
  int32_t lds_bytes;        /* LDS per workgroup */
  /* XOR swizzle of the LDS tile's 16-byte (write-width) column chunks:
   chunk' = chunk ^ (((row >> shift) & mask) << tbit) ^ ((chunk >> cshift) & cmask), k = log2(mask+1) */
  int32_t xor_k, xor_shift, xor_mask, xor_tbit;
  int32_t xor_cshift, xor_cmask;
  int32_t grid_order;       /* transpose grid: 0 column tiles fastest, 1 row tiles fastest, 2 super-tiles
                               of super_rows x super_cols tiles, each on one XCD (workgroup i runs on
                               XCD i mod 8); rows path: 0 destination order, 1 the outer modes in
                               source order */
  int32_t nontemporal;      /* nontemporal global accesses: bit 0 loads, bit 1 stores */
  int32_t unaligned;        /* 1: declined split run with 16-byte vectors at element alignment
                               (transpose kernel: element accesses at the edges of the copy; rows:
                               a row's short last vector copied in a few narrower accesses) */
  int32_t src_step;         /* transpose: source stride of mode_c, 1 to 4 (2: each vector read as two
                               contiguous ones and compacted; 3, 4: read as the 16-byte loads of
                               the bytes between its first and last element and compacted); rows: source stride of the innermost
                               mode where it is 2, 3 or 4 (gathered vectors), else 0; 0 on the
                               other paths */
  int32_t wave_local;       /* transpose: 1 if every wave reads back only LDS data it wrote itself,
                               so the phases are ordered per wave instead of by a workgroup barrier */
  int32_t lds_write_bytes, lds_read_bytes;       /* LDS instruction widths */
  int32_t edge_tiles;       /* transpose: 1 if the kernel carries its guarded code for tiles that
                               reach past an extent; 0 if every tile lies inside the copy and the
                               interior-only kernel runs */
  int32_t loads_in_flight;  /* transpose: most global loads a lane keeps outstanding in the load
                               phase (a wait after each load beyond them); 0 = all at once */
  int32_t super_rows, super_cols; /* grid_order 2: super-tile extents in row and column tiles;
                                     0 otherwise */
  int32_t src_view_bytes;   /* transpose: bytes the source elements are read as -- elem_bytes;
                               2 x elem_bytes for a stride-2 source read in pairs (src_step 2): 1-byte
                               elements (the low byte of each pair stored where the source offset
                               is even, the high byte where it is odd) and 2-, 4- and 8-byte elements
                               at even offsets (the low half stored); or 4 x elem_bytes for 1-, 2- and
                               4-byte elements of a stride-4 source (every source stride and the
                               offset multiples of 4) read in groups of 4 elements, of which the
                               first is stored (src_step 4) */
  int64_t write_conflicts, read_conflicts;       /* simulated extra LDS cycles per tile */
  char reason[192];         /* why the fast path was declined ("" if it was not) */
} tc_plan_info;

/*
 * Copy `src` (device pointer, read through src_layout) into `dst` (device
 * pointer, written through dst_layout), on `stream` (a hipStream_t; NULL = the
 * null stream).  Asynchronous: returns after the launch; kernel faults surface
 * at the caller's next synchronisation.  Layout structs are read during the
 * call only.  The library allocates no device memory (LDS only).
 * Errors: TC_E_NULL, TC_E_RANK, TC_E_EXTENT, TC_E_DTYPE, TC_E_ALIGN,
 * TC_E_NONINJECTIVE, TC_E_ALIAS, TC_E_DECLINED (strict mode), TC_E_RANGE,
 * TC_E_HIP; nothing is launched when an error is returned.
 */
int tile_copy(const void* src, const tc_layout* src_layout, void* dst, const tc_layout* dst_layout,
              int dtype, void* stream);

/* tile_copy with explicit flags (instead of the process-wide ones) and, when
 * info is not NULL, the plan that ran. */
int tile_copy_ex(const void* src, const tc_layout* src_layout, void* dst, const tc_layout* dst_layout,
                 int dtype, void* stream, int flags, tc_plan_info* info);

/*
 * tile_copy_ex that also picks the plan by measurement: the same copy (the pages' operation,
 * dst[dst_layout(i)] = src[src_layout(i)]; TVM TIRx docs, "copy -> gmem_smem") is run on the
 * planner's choice and on the other kernel configurations the library holds for it (transposes:
 * conflict-free tiles of a fixed list of shapes and grid orders; the rows paths: vectors per
 * lane, and buffer accesses on the aligned one), in three rounds over the candidates, each time once to warm up
 * and then `reps` times (0 or less: 5) between two HIP events on `stream`; the candidate with the
 * lowest median round becomes the cached plan of these layouts, dtype, flags and pointer
 * alignment, which later tile_copy / tile_copy_ex calls reuse -- the planner's own plan unless
 * another is at least 3% faster (10% where source and destination span less than 512 MiB: the
 * launches run back to back on the caller's buffers, and copies that fit the 256 MB MALL then
 * find much of their data cached, which can rank configurations differently than copies of fresh
 * data do).  The tuning itself is
 * the library's own addition (the pages plan by rule only).  Every configuration writes the same
 * bytes, so `dst` holds the copy on return.  Blocks the calling thread until the timed launches
 * end; `stream` must not be capturing (TC_E_ARG).  `info` (may be NULL) receives the chosen plan,
 * `best_ms` (may be NULL) its mean time per launch in milliseconds.  Errors: those of
 * tile_copy_ex, TC_E_ARG (capturing stream), TC_E_HIP (an event or launch failed; the cache is
 * then unchanged).
 */
int tc_autotune(const void* src, const tc_layout* src_layout, void* dst, const tc_layout* dst_layout,
                int dtype, void* stream, int flags, int reps, tc_plan_info* info, float* best_ms);

/*
 * Host only: the configurations tc_autotune would time for the copy, the planner's own first;
 * fills out[0 .. min(count, max_out) - 1] (caller-owned) and returns the count (>= 1), or the
 * planner's error status (out[0] then holds the failed plan when max_out > 0).
 */
int tc_plan_variants(const tc_layout* src_layout, const tc_layout* dst_layout, int dtype, int flags,
                     int ptr_align, tc_plan_info* out, int max_out);

/*
 * Host only: plan the copy without running it (no GPU needed).
 * `ptr_align` is the byte alignment both base pointers will have (a power of
 * two; 0 means 16).  Fills *out.  Returns the status tile_copy would return
 * for the layouts (alias and pointer checks aside).
 */
int tc_plan(const tc_layout* src_layout, const tc_layout* dst_layout, int dtype, int flags,
            int ptr_align, tc_plan_info* out);

/* The reason for the last error on this host thread ("" after success): the
 * counterpart of the pages' acceptance predicates, which return a reason with
 * their verdict (TVM TIRx docs, "copy -> gmem_smem", "What it accepts"; the
 * rejection reasons of "permute_layout", "What it accepts").  A declined copy's
 * text is the page's reason, e.g. "... the [outer, threads, vec] split has no
 * integer solution".  The string is owned by the library and stays valid until
 * the next call of an entry point on the same thread. */
const char* tc_last_error(void);

/* Process-wide default flags for tile_copy (tile_copy_ex takes its own).
 * TC_FLAG_STRICT selects the pages' acceptance rules as written (see above);
 * the other bits pick among paths that give the same bytes, for measurement.
 * Returns the previous flags, or TC_E_ARG for unknown bits (the flags are then
 * unchanged).  Thread safe; affects copies planned after the call. */
int tc_set_flags(int flags);
int tc_get_flags(void);

/*
 * Tuning override (environment variable TC_TUNE, read once, at the first plan
 * of the process), for measurement sweeps only: a comma-separated list of
 * key=value integers that pins the planner's measured choices --
 *   tile, threads, trb, unit   transpose tile bytes, threads per workgroup,
 *                              destination run in bytes, LDS unit bytes
 *   nt, order, wl, cap         nontemporal bits, grid order, wave-local phases
 *                              (0 = keep the barrier), loads in flight per lane
 *   rr, so, buf                rows path: vectors per lane, source-order grid,
 *                              buffer accesses (0 = global accesses)
 *   xk, xs, xt, xcs, xcm       the transpose's XOR swizzle (k, shift, target
 *                              bit, column shift, column mask) forced onto the
 *                              chosen tile, conflict-free or not
 *   ssr, ssc                   grid order 2: super-tile extents in tiles
 *                              (powers of two; the plan's own by default:
 *                              16 x 2 on the int8 tall tiles, else 8 x 8)
 * Every setting gives the same bytes.  A setting no compiled kernel instance
 * matches makes the copy fail with TC_E_ARG ("internal: no tile geometry");
 * unknown keys are ignored.  Unset, the planner's own choices apply.
 */

/*
 * Region slice of a layout (TVM TIRx "copy -> gmem_smem", demonstration
 * program: A[fs] with fs a tuple of slices).  For every mode k, Python slice
 * semantics with start/stop/step (step != 0; negative start/stop count from
 * the end; out-of-range values are clipped): the new extent is the number of
 * indices in range(start, stop, step), offset += start * stride,
 * stride *= step.  `start`, `stop`, `step` have in->rank entries.
 * Returns TC_OK or TC_E_NULL / TC_E_RANK / TC_E_ARG.
 */
int tc_layout_slice(const tc_layout* in, const int64_t* start, const int64_t* stop, const int64_t* step,
                    tc_layout* out);

/*
 * The bank plan of a wave-scope register-staged permute of an LDS tile (the device primitive
 * tcd::wave_permute in tile_copy_dev.hpp), TVM TIRx docs, "permute_layout":
 *   step 1 -- both layouts keep their logical mode order with unit modes dropped; neighbouring
 *             modes merge where they are contiguous on both sides (the source is regrouped onto
 *             the destination's shard); P = element count / 64 elements per lane;
 *   step 2 -- for k = 0 .. log2 P (k = 0 only when P is not a power of two) and, for k > 0,
 *             shift = 0 .. 6 - k ascending: lane l's element at step r is flat index
 *             l + 64 * (r ^ ((l >> shift) & (2^k - 1))); the LDS accesses of all P steps are
 *             simulated under gfx950's bank model (read phase through the source layout, write
 *             phase through the destination layout, element-wide accesses) and the first
 *             (k, shift) with no extra cycle in either phase is taken.
 * Host only: no GPU is touched.  `out` (caller-owned) receives the canonical shard and the
 * result.  On TC_E_DECLINED (the page's "fails if none") it still holds the first candidate with
 * the fewest extra cycles, its counts and the reason, for callers that accept conflicts.
 * Errors: TC_E_NULL, TC_E_RANK, TC_E_EXTENT, TC_E_DTYPE; TC_E_DECLINED when the count is not a
 * multiple of 64 (no integer P) or no k is conflict-free in both phases; TC_E_RANGE when an
 * offset needs more than 31 bits.
 */
typedef struct tc_permute_info {
  int32_t rank;             /* canonical shard modes */
  int32_t elements_per_lane;/* P */
  int64_t extent[TC_MAX_RANK], src_stride[TC_MAX_RANK], dst_stride[TC_MAX_RANK];
  int32_t k, shift, mask;   /* chosen swizzle (when declined: the cheapest candidate) */
  int32_t reserved;
  int64_t read_conflicts, write_conflicts; /* simulated extra cycles over the P steps */
  char reason[192];         /* why it declined ("" otherwise) */
} tc_permute_info;

int tc_wave_permute_plan(const tc_layout* src_layout, const tc_layout* dst_layout, int dtype,
                         tc_permute_info* out);

/* Library version, major * 10000 + minor * 100 + patch. */
int tc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TILE_COPY_H */
