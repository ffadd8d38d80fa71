// Internal host-side types of the tile-copy library: layout algebra, partition
// planner, LDS swizzle chooser, and the argument blocks the kernels take.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "tile_copy.h"

namespace tc {

// Build-time constants of the rows path (measured choices on MI355X).
#ifndef TC_ROW_THREADS
#define TC_ROW_THREADS 256   // threads per workgroup of the register-staged rows path
#endif
#ifndef TC_ROW_ROUNDS
#define TC_ROW_ROUNDS 4      // vectors per thread of the rows path
#endif

constexpr int kMaxRank = TC_MAX_RANK;
constexpr int kWave = 64;                      // gfx950 wavefront
constexpr int kSmallCopyBytes = 16384;         // co-contiguous copies up to this size: one LDS round trip
constexpr int kRowThreads = TC_ROW_THREADS;    // threads per workgroup on the rows path
constexpr int kRowRounds = TC_ROW_ROUNDS;      // vectors per thread on the rows path
constexpr int64_t kRowSmallBytes = int64_t(256) << 20;  // rows path: "small" contiguous copies
constexpr int kGuardThreads = 256;             // threads per workgroup on the guarded paths
// Rows-type and shuffle copies of 2^31 vectors or more run as several launches of at most this
// many vectors each (the kernels index vectors and workgroups with 32-bit integers).
constexpr int64_t kLaunchVectors = int64_t(1) << 30;
constexpr int kInterleaveRounds = 2;  // pixel groups per lane on the interleave path
constexpr int kSuperLog = 3;          // transpose grid order 2: super-tiles of 8 x 8 tiles by default

// One joint mode: extent, source stride, destination stride (elements).
struct Mode {
  int64_t e, s, d;
};

// Both layouts over the common logical shape, after extent-1 modes are dropped.
struct Joint {
  int rank = 0;
  Mode m[kMaxRank];
  int64_t so = 0, dof = 0;  // element offsets
  int64_t count = 1;
};

struct Plan;
// The joint modes in the rows path's grid order, innermost last: the destination's (canonical)
// order, or with row_src_order the outer modes by descending source stride.
Joint rows_grid(const Plan& p);

// ---- layout algebra (layout.cpp) -------------------------------------------------------------
int make_joint(const tc_layout& src, const tc_layout& dst, Joint* out, std::string* err);
// Sort by destination stride (descending |d|, stable) and merge adjacent modes that are
// contiguous on both sides.
void canonicalize(Joint* j);
// 1 injective, 0 not, -1 undecided (too large to check by enumeration)
int dst_injective(const Joint& j);
// [lo, hi) element range a layout side touches (for the alias check)
// Element offsets a side touches: [lo, hi), hi one past the last element.
void side_range(const Joint& j, bool src_side, int64_t* lo, int64_t* hi);
int slice_layout(const tc_layout& in, const int64_t* start, const int64_t* stop, const int64_t* step,
                 tc_layout* out, std::string* err);

// ---- LDS bank model (bank.cpp) ----------------------------------------------------------------
// gfx950 LDS geometry per access: number of 4-byte banks and lanes served together.
struct BankGeom {
  int banks, group;
};
BankGeom gfx950_bank_geom(bool write, int width_bytes);
// Extra cycles one LDS instruction costs: byte_addr[l] for lanes with active[l].
int64_t lds_conflict_cycles(const int64_t* byte_addr, const bool* active, int lanes, int width_bytes,
                            bool write);

// ---- transpose tile geometry -------------------------------------------------------------------
// The LDS tile is NB x TRu x TC units of U bytes (U in {4, 8, 16}, U >= eb).  A unit is one
// column of B = U/eb consecutive rows, assembled in registers from B loaded row vectors (a
// register regrouping for 4-byte and wider elements, a BxB byte/halfword micro-transpose with
// v_perm_b32 for narrower ones).  One store vector (VE consecutive rows of one column) is then
// RPV = vb/U whole units, so the store phase reads it with RPV LDS reads of U bytes.  The tile's
// column chunks of CW units (one 16-byte LDS write, or less) are XOR-swizzled by row and by
// their own higher bits:  chunk' = chunk ^ (((ru >> shift) & mask) << tbit) ^ ((chunk >> cshift) & cmask).
// The row term spreads the lanes of one read instruction (same column, different rows) over the
// banks; the column term spreads the chunks one write instruction stores when a lane writes
// several adjacent chunks.  Both are bijections of a row's chunks.
struct TileGeom {
  int eb = 4, vb = 16;  // element bytes, global vector bytes
  int U = 0, B = 1;     // LDS unit bytes (0: the smallest allowed), rows per unit
  int VE = 4;           // elements per global vector
  int TR = 32, TC = 128, NB = 1;  // tile extents: rows (dst-contiguous mode), cols (src-contiguous mode), batch
  int NT = 256;                   // threads per workgroup
  int tile_bytes = 16384;         // LDS tile per workgroup
  int ntm = 0;                    // nontemporal global accesses: bit 0 loads, bit 1 stores
  int order = 0;                  // grid order: 0 column tiles fastest, 1 row tiles fastest,
                                  // 2 XCD super-tiles (see tile_at)
  int step = 1;                   // source element stride along the column mode (1; 2: every
                                  // vector read as two contiguous ones and compacted in registers;
                                  // 3, 4: read as the loads of its span and compacted)
  bool wave_local = false;        // every wave reads back only LDS units it wrote itself: the
                                  // phases are ordered per wave, without a workgroup barrier
  bool edges = true;              // some tile reaches past an extent (the kernel needs its guards)
  bool pad_rows = false;          // order 1 with source rows off the 128-byte lines: the row-tile
                                  // count of the grid is padded to a multiple of kXcds (tile_at)
  int cap = 0;                    // loads a lane keeps in flight in the interior load phase (0: all)
  int nar = 0;                    // 1-byte elements of a stride-2 source read in 2-byte pairs (eb is
                                  // then the pair's 2 bytes), the low (1) or high (2) byte stored;
                                  // of a stride-4 source read in 4-byte words, the low byte (3)
  int lsr = kSuperLog, lsc = kSuperLog;  // order 2: log2 of the super-tile extents in tiles
  int loads = 4, stores = 4;  // accesses per thread per phase
  int ww = 16, rw = 4;        // LDS write / read instruction bytes
  int k = 0, shift = 0, tbit = 0;
  int cshift = 0, cmask = 0;
  int CW() const { return ww / U; }  // units per write chunk
  int TRu() const { return TR / B; }
  int RPV() const { return vb / U; }  // LDS unit reads per store vector
  int64_t unit_addr(int nb, int ru, int c) const {
    const int cw = CW();
    const int ch = c / cw;
    const int chs = ch ^ (((ru >> shift) & ((1 << k) - 1)) << tbit) ^ ((ch >> cshift) & cmask);
    return (int64_t(nb) * TRu() + ru) * TC + int64_t(chs) * cw + (c % cw);
  }
};
// Fill loads/stores/ww/rw/U/B/VE from eb, vb, TR, TC, NB.  False if the geometry is invalid.
bool finish_geom(TileGeom* g);
// Whether every LDS unit a wave reads in the store phase was written by the same wave in the
// load phase (then no workgroup barrier is needed between the phases).
bool tile_wave_local(const TileGeom& g);
// Simulated extra LDS cycles of one interior tile: write phase and read phase.  With limit >= 0
// the simulation stops once write + read cycles reach the limit (the counts are then partial).
void simulate_tile(const TileGeom& g, int64_t* write_cycles, int64_t* read_cycles, int64_t limit = -1);

// ---- plan -------------------------------------------------------------------------------------
struct Plan {
  int status = TC_OK;
  int path = TC_PATH_EMPTY;
  int eb = 4;
  Joint j;
  int vb = 0;                       // global vector bytes
  int ntm = 0;                      // rows path: nontemporal global accesses (bit 0 loads, bit 1 stores)
  bool unaligned = false;           // transpose or rows with vectors at element alignment (extents or strides
                                    // not multiples of the vector; edges element by element)
  int step = 1;                     // source stride of the transpose's column mode (1 to 4), or
                                    // of the gathered rows' mode (2 to 4)
  int nar = 0;                      // transpose of 1-byte elements whose column mode has source
                                    // stride 2, read as 2-byte pairs (the tile planned for eb = 2,
                                    // source strides and offset halved at launch), of which the
                                    // low (1: even offset) or high (2: odd offset) byte is kept;
                                    // 3: stride 4, read as 4-byte words (eb = 4), the low byte kept
  int shuffle_c = 0;                // shuffle path: block columns C (8, 16 or 32; 4 rows); interleave
                                    // path: the channels (2, 3, 4 or 8)
  bool to_planes = false;           // interleave path: interleaved source, planar destination
  bool row_burst = false;           // rows path: every load of a thread issued at once (else one at
                                    // a time, each after its offsets are decoded)
  int row_rounds = kRowRounds;      // rows path: vectors per thread (1, 2 or 4)
  bool row_src_order = false;       // rows path: the outer grid modes in source order (see rows_grid)
  bool buffers = false;             // rows (16-byte vectors) and shuffle paths: buffer accesses with
                                    // streaming cache policies, in every launch whose offsets fit
  int mode_r = -1, mode_c = -1, mode_b = -1;
  TileGeom g;
  int threads = 0, load_outer = 0, store_outer = 0;
  int64_t workgroups = 0;
  int lds_bytes = 0;
  int64_t wconf = 0, rconf = 0;
  bool declined = false;
  std::string reason;
};

int elem_bytes_of(int dtype);
// Plans a copy.  ptr_align: byte alignment of both base pointers (power of two, <= 16).
Plan make_plan(const tc_layout& src, const tc_layout& dst, int dtype, int flags, int ptr_align);
// The plan first, then the same copy on other kernel configurations (tc_autotune).
std::vector<Plan> plan_variants(const Plan& p, int flags);
void plan_to_info(const Plan& p, tc_plan_info* info);

// ---- kernel argument blocks (passed by value) ------------------------------------------------
// 32-bit division by a runtime constant d: q = (umulhi(n, mul) + n) >> shr, exact for n < 2^32.
struct Div32 {
  uint32_t d, mul, shr;
};
Div32 make_div32(uint32_t d);

struct TransposeArgs {
  const unsigned char* src;
  unsigned char* dst;
  int64_t src_off, dst_off;  // elements
  int64_t eR, eC, eB;        // extents of the tile modes (eB = 1 without a batch mode)
  int64_t sR, sC, sB;        // source strides of R, C, B
  int64_t dR, dC, dB;        // destination strides of R, C, B
  Div32 tilesR, tilesC, tilesB;
  Div32 tilesRg;             // order 1: row tiles per column of the grid (tilesR, or padded)
  int32_t nbatch;            // further modes walked by the grid, innermost last
  Div32 bdiv[kMaxRank];      // their extents
  int64_t bs[kMaxRank], bd[kMaxRank];
  int32_t lTR, lTC, lNB;     // log2 of the tile extents
  int32_t xshift, xmask, xtbit;
  int32_t xcshift, xcmask;
  int32_t order;             // 0: column tiles fastest, 1: row tiles fastest, 2: XCD super-tiles
  Div32 stC;                 // order 2: super-tiles along the column mode, per 2-D slice
  uint32_t nst;              // order 2: super-tiles per 2-D slice
  uint32_t nslices;          // order 2: 2-D slices (batch tiles times the other grid modes)
  int32_t lsr, lsc;          // order 2: log2 of the super-tile's extents in tiles (rows, columns)
};

// The shuffle path: nvec 16-byte vectors, C/4 per block row; block b starts at element
// so + b * sB (source, row-major 4 x C) and dof + b * dB (destination, column-major).
constexpr int kShuffleThreads = 256;  // lanes per workgroup
constexpr int kShuffleRounds = 8;     // vectors per lane
struct ShuffleArgs {
  const unsigned char* src;
  unsigned char* dst;
  int64_t so, dof, sB, dB;
  int64_t nvec;
};

struct RowArgs {
  const unsigned char* src;
  unsigned char* dst;
  int64_t src_off, dst_off;  // bytes
  int32_t rank;              // modes of the vector grid, innermost last
  int32_t pad0;
  uint32_t ext[kMaxRank];    // extents; the innermost counts vectors
  uint32_t mul[kMaxRank];    // fast division: q = (umulhi(n, mul) + n) >> shr
  uint32_t shr[kMaxRank];
  int64_t s[kMaxRank], d[kMaxRank];  // byte strides per step of each grid mode
  int64_t nvec;              // vectors in the whole copy (of this launch)
  int64_t row_elems;         // element-aligned rows: elements per row (its last vector may be short)
  int64_t sbuf, dbuf;        // buffer accesses: byte offsets of the buffer bases (the lowest bytes
                             // the launch reads / writes) from src / dst
};

// Order 2: super-tiles of 2^lsr x 2^lsc tiles (rows x columns; kSuperLog each by default), each run
// on one XCD (the dispatcher sends workgroup i to XCD i % kXcds), so that neighbouring tiles, which
// share cache lines when the layouts are not line-aligned, meet in one L2.
constexpr int kXcds = 8;

// ---- launch (kernels.hip) ------------------------------------------------------------------------
int launch_plan(const Plan& p, const void* src, void* dst, void* stream, std::string* err);

// Sets the calling thread's tc_last_error() text; returns `code`.
int set_last_error(int code, const std::string& why);
// The wave-scope permute's bank plan (tc_wave_permute_plan).
int wave_permute_plan(const tc_layout& src, const tc_layout& dst, int dtype, tc_permute_info* out, std::string* err);

// A transpose kernel configuration: vector bytes, LDS unit bytes, tile bytes, threads,
// nontemporal mode, source step, wave-local phase ordering, edge code and load cap.  One launcher
// per element width holds the instances it was built with: it launches `ta` on `stream`, or with
// ta == nullptr only reports whether the instance exists.
struct TransposeCfg {
  int vb, unit, tile, threads, ntm, step;
  bool wave_local;
  bool edges = true;  // false: every tile lies wholly inside the copy (the interior-only kernel)
  int cap = 0;        // loads in flight per lane in the load phase (0: all of them)
  int nar = 0;        // source read in 2-byte pairs, low (1) or high (2) bytes stored, or words (3)
};
// The kernel configuration a planned tile geometry runs with (every field of it).
inline TransposeCfg transpose_cfg(const TileGeom& g) {
  return TransposeCfg{g.vb, g.U, g.tile_bytes, g.NT, g.ntm, g.step, g.wave_local, g.edges, g.cap, g.nar};
}
bool launch_transpose_eb1(const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream);
bool launch_transpose_eb2(const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream);
bool launch_transpose_eb4(const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream);
bool launch_transpose_eb8(const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream);
bool launch_transpose_eb16(const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream);
bool launch_transpose(int eb, const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream);

}  // namespace tc
