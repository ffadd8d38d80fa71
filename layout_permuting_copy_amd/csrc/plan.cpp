// Partition planner and LDS swizzle chooser.
//
// Synthesizing the thread partition follows TVM TIRx docs, "copy -> gmem_smem", Algorithm:
//  1. slice and canonicalize both layouts (the destination side drives the canonical order of
//     the joint modes; each phase is then coalesced on its own global side);
//  2. choose the vector width widest first -- here 16, 8 then 4 bytes -- accepting it when the
//     contiguous tail divides it and every other stride and both base offsets are multiples of it;
//  3. split into [outer, threads, vec] with the TileLang default mapping (tutorial
//     "loop_mapping.py": access_idx = flat // vec, thread = access_idx % threads,
//     local_idx = (access_idx // threads) * vec + flat % vec).
// The copy declines ("What it accepts", divisibility) when the element count is not a multiple
// of the thread count of a wavefront (64 on gfx950): there is no integer [outer, threads, vec]
// split.  Strict mode reports that (TC_E_DECLINED); otherwise the transpose kernel runs with
// 16-byte vectors at element alignment where the layouts have unit-stride (or stride-2 source)
// modes, else a guarded path.  Outside strict mode the same element-aligned vectors also replace
// the page's 8- and 4-byte ones, which measured slower.
//
// Tile shapes, thread counts, nontemporal hints and grid orders are chosen per element width
// and layout class from measurements on MI355X (each rule below names what it measured);
// TC_TUNE (environment) overrides them for sweeps.
//
// When the source- and destination-contiguous modes differ, a workgroup stages a tile through
// LDS.  The swizzle of that tile is chosen as in TVM TIRx docs, "permute_layout", Algorithm
// step 2: simulate the banks for the write phase and the read phase and keep the smallest XOR
// bit count k (then the smallest shift and target bit) that leaves both conflict-free.
#include <algorithm>
#include <array>
#include <map>
#include <mutex>
#include <cstdlib>
#include <string>

#include "plan.hpp"

namespace tc {

int elem_bytes_of(int dtype) {
  switch (dtype) {
    case TC_U8: case TC_I8: return 1;
    case TC_F16: case TC_BF16: return 2;
    case TC_F32: case TC_I32: return 4;
    case TC_F64: case TC_I64: return 8;
    case TC_B128: return 16;
    default: return -1;
  }
}

static int ilog2i(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

static int64_t pow2ceil(int64_t x) { return int64_t(1) << ilog2i(std::max<int64_t>(1, x)); }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Step 2 of the page: widest vector whose tail divides it and whose other strides/offsets are
// multiples of it.  `inner_src`/`inner_dst` are the modes vectorized on each side.
static int choose_vec(const Joint& j, int eb, int inner_src, int inner_dst, int ptr_align, int max_vb = 16) {
  for (int vb : {16, 8, 4}) {
    if (vb > max_vb) continue;
    if (vb < eb || vb % eb || vb > ptr_align) continue;
    const int64_t ve = vb / eb;
    bool ok = j.so % ve == 0 && j.dof % ve == 0;
    ok = ok && j.m[inner_src].e % ve == 0 && j.m[inner_dst].e % ve == 0;
    for (int k = 0; ok && k < j.rank; ++k) {
      if (k != inner_src && j.m[k].s % ve) ok = false;
      if (k != inner_dst && j.m[k].d % ve) ok = false;
    }
    if (ok) return vb;
  }
  return 0;
}

static void decline(Plan* p, int flags, const std::string& why) {
  p->declined = true;
  if (p->reason.empty()) p->reason = why;
  if (flags & TC_FLAG_STRICT) p->status = TC_E_DECLINED;
}

// Tile geometry and swizzle of the transpose path.  Tile extents are powers of two filling the
// tile.  Candidates are tried in a fixed order of destination run length (bytes of one column
// segment, TR * eb) and LDS unit size; the first one with a conflict-free swizzle wins.
//
// Tile bytes, threads per workgroup and the nontemporal hint are chosen per element width from
// measurements on MI355X (16384x16384 / 8192x8192 transposes and the batched 4x32 scale-factor
// tiles, HIP-event timed, HBM-resident inputs).  TC_TUNE (environment, read once) overrides
// them for tuning sweeps: "tile=32768,threads=512,nt=3,order=0,trb=128,unit=4,wl=0,rr=2,buf=0,cap=0"
// (order: 0 column tiles first, 1 row tiles first, 2 XCD super-tiles; wl=0: keep the workgroup
// barrier even where the phases are wave-local; rr: vectors per thread of the 16-byte rows path;
// buf=0: global instead of buffer accesses on the rows and shuffle paths; cap: loads in flight
// per lane in the transpose's load phase, 0 = all, where the library holds such an instance;
// so: 1 / 0 the rows path's outer grid modes in source / destination order; xk, xs, xt, xcs, xcm:
// the transpose's XOR swizzle (k, shift, target bit, column shift, column mask) forced onto the
// tile the planner picks, conflict-free or not, so that the bank model can be checked against the
// hardware counter on swizzles the search passes over).  A setting no kernel instance matches
// makes the copy fail with TC_E_ARG ("no tile geometry").
struct TuneCfg {
  int tile = 0, threads = 0, nt = -1, order = -1, trb = 0, unit = 0, wl = -1, rr = 0, buf = -1, cap = -1, so = -1;
  int xk = -1, xs = 0, xt = 0, xcs = 0, xcm = 0;
  int ssr = 0, ssc = 0;  // order 2: super-tile extents in tiles (powers of two)
  int nar = 0;           // 1, 2: pairs, 3: words read (set by the planner, not by TC_TUNE)
};

static TuneCfg tune_override() {
  static const TuneCfg cfg = [] {
    TuneCfg c;
    const char* env = std::getenv("TC_TUNE");
    if (!env) return c;
    std::string s(env);
    size_t pos = 0;
    while (pos < s.size()) {
      size_t end = s.find(',', pos);
      if (end == std::string::npos) end = s.size();
      const std::string kv = s.substr(pos, end - pos);
      const size_t eq = kv.find('=');
      if (eq != std::string::npos) {
        const std::string k = kv.substr(0, eq);
        const int v = std::atoi(kv.c_str() + eq + 1);
        if (k == "tile") c.tile = v;
        else if (k == "threads") c.threads = v;
        else if (k == "nt") c.nt = v;
        else if (k == "order") c.order = v;
        else if (k == "trb") c.trb = v;
        else if (k == "unit") c.unit = v;
        else if (k == "wl") c.wl = v;
        else if (k == "rr") c.rr = v;
        else if (k == "buf") c.buf = v;
        else if (k == "cap") c.cap = v;
        else if (k == "so") c.so = v;
        else if (k == "xk") c.xk = v;
        else if (k == "xs") c.xs = v;
        else if (k == "xt") c.xt = v;
        else if (k == "xcs") c.xcs = v;
        else if (k == "xcm") c.xcm = v;
        else if (k == "ssr") c.ssr = v;
        else if (k == "ssc") c.ssc = v;
      }
      pos = end + 1;
    }
    return c;
  }();
  return cfg;
}

Joint rows_grid(const Plan& p) {
  Joint g = p.j;
  if (p.row_src_order && g.rank > 2)
    std::stable_sort(g.m, g.m + g.rank - 1,
                     [](const Mode& x, const Mode& y) { return std::llabs(x.s) > std::llabs(y.s); });
  return g;
}

// Permuted rows shorter than 1 KiB walk the source order (reads contiguous, each row written to
// its place), where it differs from the destination's: the (0,2,1,3) bf16 permute with 256-byte
// rows 6.11 -> 6.44 TB/s, with 128-byte rows 6.21 -> 6.47-6.50, fp32 with 128-byte rows 6.16 ->
// 6.44; 8 heads of 256-byte rows equal (6.17); 1 KiB rows 6.25 against 6.23 in source order.
static bool row_src_order(const Joint& j, int eb) {
  if (j.rank < 3 || j.m[j.rank - 1].e * eb >= 1024) return false;
  for (int k = 0; k + 2 < j.rank; ++k)
    if (std::llabs(j.m[k].s) < std::llabs(j.m[k + 1].s)) return true;
  return false;
}

// Vectors per thread on the 16-byte rows path (buffer accesses), measured on MI355X: one
// contiguous mode: 2 up to 256 MiB each way, 1 beyond (a 64 MiB copy 6.15 TB/s with 2, 5.93-6.06
// with 1, 5.93-6.00 with 4; 1 GiB 6.52 with 1, 6.43-6.46 with 2, 6.37-6.39 with 4); permuted rows
// in source order 2 (the (0,2,1,3) permute 6.44 TB/s, 5.89-5.93 with 1, 6.32-6.33 with 4), in
// destination order 4 (6.23-6.25 TB/s with 4, 5.71-5.73 with 1 or 2).
static int row_rounds(const Joint& j, int eb, bool src_order) {
  if (j.rank != 1) return src_order ? 2 : 4;
  return j.count * eb <= kRowSmallBytes ? 2 : 1;
}

// Defaults per element width: {tile bytes, threads, nontemporal mode, grid order}.  `batched` =
// the destination-contiguous extent is shorter than one 128-byte run, so the tile is filled from
// a batch mode (the scale-factor case).  `lines_shared` = vectors at element alignment, or
// destination columns off the 128-byte lines: neighbouring tiles then share cache lines, and
// nontemporal stores of partial lines were measured 1.5-2x slower than plain ones.
static TuneCfg default_cfg(int eb, bool batched, bool lines_shared) {
  TuneCfg c;
  if (lines_shared) {
    c.tile = eb == 2 ? 8192 : 16384;
    c.threads = eb == 2 ? 256 : 512;
    c.nt = 0;
    c.order = 0;
    return c;
  }
  if (batched) { c.tile = 8192; c.threads = 256; c.nt = 3; c.order = 0; return c; }
  switch (eb) {
    case 1: c.tile = 65536; c.threads = 512; c.nt = 3; c.order = 1; break;
    case 2: c.tile = 65536; c.threads = 512; c.nt = 3; c.order = 0; break;
    case 4: c.tile = 32768; c.threads = 256; c.nt = 3; c.order = 0; break;
    case 8: c.tile = 65536; c.threads = 256; c.nt = 3; c.order = 0; break;
    default: c.tile = 16384; c.threads = 512; c.nt = 3; c.order = 0; break;
  }
  return c;
}

// The XOR swizzle of one tile geometry: the first candidate, in search order, with the fewest
// simulated extra LDS cycles (search order: k ascending, then the row shift, the target bit and
// the column term).  A candidate's simulation stops once it can no longer beat the best so far.
// The result depends on the geometry alone, so it is kept for the life of the process.
static bool search_swizzle_pass(const TileGeom& g, bool no_swizzle, bool zero_only, TileGeom* out, int64_t* out_w,
                                int64_t* out_r) {
  const int chunk_bits = ilog2i(g.TC / g.CW());
  const int row_bits = ilog2i(g.TRu());
  const int kmax = no_swizzle ? 0 : chunk_bits;
  // column terms: none first, then (cshift, cmask) by increasing cshift and mask
  int col_terms[32][2];
  int ncol = 0;
  col_terms[ncol][0] = 0; col_terms[ncol][1] = 0; ++ncol;
  if (!no_swizzle)
    for (int cs = 1; cs < chunk_bits && ncol < 32; ++cs)
      for (int cm = 1; cm < (1 << cs) && cm <= 7 && ncol < 32; cm = 2 * cm + 1) {
        col_terms[ncol][0] = cs; col_terms[ncol][1] = cm; ++ncol;
      }
  int64_t best_cost = -1;
  for (int k = 0; k <= kmax; ++k)
    for (int shift = 0; shift <= (k ? std::max(0, row_bits - 1) : 0); ++shift)
      for (int tbit = 0; tbit <= (k ? chunk_bits - k : 0); ++tbit)
        for (int ct = 0; ct < ncol; ++ct) {
          TileGeom c = g;
          c.k = k;
          c.shift = shift;
          c.tbit = tbit;
          c.cshift = col_terms[ct][0];
          c.cmask = col_terms[ct][1];
          if (!finish_geom(&c)) continue;
          int64_t wc, rc;
          simulate_tile(c, &wc, &rc, zero_only ? 1 : best_cost);
          if (zero_only && wc + rc > 0) continue;
          if (best_cost < 0 || wc + rc < best_cost) {
            best_cost = wc + rc;
            *out = c;
            *out_w = wc;
            *out_r = rc;
            if (best_cost == 0) return true;
          }
        }
  return best_cost >= 0;
}

// First a pass that only looks for a conflict-free candidate (each simulation stops at the first
// extra cycle), then, if there is none, the full search for the fewest extra cycles.
static bool search_swizzle_uncached(const TileGeom& g, bool no_swizzle, TileGeom* out, int64_t* out_w,
                                    int64_t* out_r) {
  if (search_swizzle_pass(g, no_swizzle, true, out, out_w, out_r)) return true;
  return search_swizzle_pass(g, no_swizzle, false, out, out_w, out_r);
}

static bool search_swizzle(const TileGeom& g, bool no_swizzle, TileGeom* out, int64_t* out_w, int64_t* out_r) {
  struct Found {
    bool any;
    TileGeom g;
    int64_t w, r;
  };
  static std::mutex mu;
  static std::map<std::array<int, 10>, Found> memo;
  const std::array<int, 10> key{g.eb, g.vb, g.U, g.TR, g.TC, g.NB, g.NT, g.tile_bytes, g.ntm * 8 + g.order,
                                no_swizzle ? 1 : 0};
  // the swizzle fields only: the rest of the geometry is the caller's
  auto apply = [&](const Found& f) {
    *out = g;
    out->k = f.g.k;
    out->shift = f.g.shift;
    out->tbit = f.g.tbit;
    out->cshift = f.g.cshift;
    out->cmask = f.g.cmask;
    *out_w = f.w;
    *out_r = f.r;
    return f.any;
  };
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = memo.find(key);
    if (it != memo.end()) return apply(it->second);
  }
  Found f{false, g, 0, 0};
  f.any = search_swizzle_uncached(g, no_swizzle, &f.g, &f.w, &f.r);
  std::lock_guard<std::mutex> lock(mu);
  memo.emplace(key, f);
  return apply(f);
}

// Tall tiles in row-tile-first grid order, where measured faster than the default shape: runs of
// 1-2 KiB along the destination-contiguous mode and 128-256 bytes along the source-contiguous
// mode, 16-byte LDS units (a store vector is one ds_read_b128), so that the workgroups running
// together write whole destination columns.  On MI355X, against the default tiles: fp32 16384^2
// 5700 -> 6250 GB/s, bf16 16384^2 5370 -> 5720, fp16 8192^2 4780 -> 5310, fp64 8192^2 5370 ->
// 5780, 16-byte elements 8192^2 5520 -> 5950.  64 KiB tiles where they still give 8192
// workgroups, else smaller.  128 KiB tiles (one workgroup per CU) where the copy is large enough
// to give every CU many of them: bf16 16384^2 as 1024 x 64 on 1024 lanes 5730 -> 5830, fp64 8192^2
// as 256 x 64 5750 -> 5980 and then as 128 x 128 on 1024 lanes (1 KiB runs on both sides) 6.00 ->
// 6.10 TB/s, int8 8192^2 as 512 x 256 5000 -> 5190 (the default tile for 1-byte elements
// otherwise); fp32 and smaller fp16 copies are faster on 64 KiB tiles.
// Loads in flight per lane (`cap`): all of a lane's loads at once had been the rule, but for the
// tall tiles of 1- and 2-byte elements two measured faster (a wait in the load phase keeps at most
// `cap` outstanding), on every buffer placement tried: bf16 16384^2 5.85-5.89 -> 6.09-6.19 TB/s,
// int8 8192^2 5.20-5.39 -> 5.51-5.62, fp16 8192^2 5.30-5.41 -> 5.54-5.60.  fp64 with 8 of its 16
// loads ran at 6.4-6.6 TB/s on some placements of the same buffers and 5.6-5.9 on others (mean no
// better than 6.0 with all in flight), fp32 at 6.04-6.19 against 6.24; they keep all in flight, as
// do the element-aligned plans.
static bool tall_cfg(int eb, int64_t eR, int64_t eC, int64_t others, TuneCfg* c) {
  c->nt = 3;
  c->order = 1;
  c->unit = 16;
  c->cap = 0;
  auto tiles = [&](int64_t tr, int64_t tc) { return ceil_div(eR, tr) * ceil_div(eC, tc) * others; };
  switch (eb) {
    case 1:
      if (eR < 512 || eC < 256 || tiles(512, 256) < 512) {
        // narrower copies of at least 16 MiB (e.g. NCHW <-> NHWC with 32-128 channels): the same
        // 128 KiB tiles with row tiles first and every load in flight (measured on MI355X against
        // the default 16 KiB tiles: NHWC -> NCHW with 64 channels 2.42 -> 4.61 TB/s, with 32
        // 1.82 -> 3.46, NCHW -> NHWC with 64 4.27 -> 5.14, 128 channels either way +2-6%; with 2
        // loads in flight and 16 x 2 super-tiles 2.0-3.2)
        if (eR < 64 || eC < 32 || eR * eC * others < (int64_t(16) << 20)) return false;
        c->tile = 131072; c->threads = 512; c->trb = 512;
        return true;
      }
      c->tile = 131072; c->threads = 512; c->trb = 512; c->cap = 2;  // 512 x 256
      // XCD super-tiles of 16 row tiles by 2 column tiles: an XCD's 32 workgroups (one per CU)
      // are one super-tile, and the chip runs 16 x 16 tiles at a time, whatever the extents.
      // Against row tiles first: int8 16384^2 4.79 -> 5.37-5.43 TB/s, 16384 x 8192 4.70 -> 5.12,
      // 32768 x 4096 4.41 -> 5.30, 4096 x 32768 5.28 -> 5.63-5.73, 12288^2 4.96 -> 5.27, 8192^2
      // 5.32-5.34 -> 5.42-5.43 (8192 x 16384 level); 8 x 8, 8 x 4, 16 x 4 or 32 x 1 super-tiles
      // were slower than 16 x 2 on 16384^2 and 8192^2
      c->order = 2; c->ssr = 16; c->ssc = 2;
      return true;
    case 16:
      if (eR < 64 || eC < 8) return false;
      c->tile = 8192; c->threads = 256; c->trb = 1024;  // 64 x 8 elements
      return true;
    case 8:
      if (eR < 128 || eC < 16) return false;
      // 128 KiB: square 128 x 128 tiles on 1024 lanes, 1 KiB runs on both sides (fp64 8192^2 6.00
      // -> 6.10 TB/s against 256 x 64 on 512 lanes, interleaved over 7 placements; on 512 lanes
      // the square tile ran at 5.96)
      if (tiles(128, 128) >= 4096) { c->tile = 131072; c->threads = 1024; c->trb = 1024; }
      else if (tiles(256, 32) >= 8192) { c->tile = 65536; c->threads = 512; c->trb = 2048; }  // 256 x 32
      else { c->tile = 16384; c->threads = 256; c->trb = 1024; }                          // 128 x 16
      return true;
    case 4:
      if (eR < 256 || eC < 32) return false;
      // 256 x 64 tiles for the large copies (16384^2), 256 x 32 below 8192 such tiles, except for
      // destination rows of at most 2048 elements: 128 x 64 tiles there (measured on MI355X against
      // 256 x 32, 0.25-1 GiB moved: 1024 x 4096 3.76 -> 4.63 TB/s, 2048^2 3.91 -> 4.54, 512 x 8192
      // 4.25 -> 4.79, 1024 x 16384 4.59 -> 5.14, 1024 x 65536 5.04 -> 5.73, 512 x 131072 4.85 ->
      // 5.71, 2048 x 32768 5.50 -> 5.78, 768 x 32768 5.38 -> 5.62, 2048 x 8192 level; with 4096
      // elements they were 3-7% slower: 4096^2 5.11 -> 4.75).  Other shapes showed no rule: 256 x 64
      // tiles in XCD super-tiles of 4 x 4 ran 13-19% faster on 65536 x 1024, 32768 x 2048,
      // 16384 x 4096 and 262144 x 256, but 2-7% slower on 6144^2, 8192 x 4096, 24576 x 1536 and
      // 131072 x 512.
      if (tiles(256, 64) >= 8192) { c->tile = 65536; c->threads = 512; c->trb = 1024; }  // 256 x 64
      else if (eR <= 2048) { c->tile = 32768; c->threads = 512; c->trb = 512; }          // 128 x 64
      else { c->tile = 32768; c->threads = 512; c->trb = 1024; }                         // 256 x 32
      return true;
    case 2:
      if (eR < 256 || eC < 64) return false;
      if (tiles(1024, 64) >= 4096) { c->tile = 131072; c->threads = 1024; c->trb = 2048; }  // 1024 x 64
      else if (tiles(512, 64) >= 8192) { c->tile = 65536; c->threads = 512; c->trb = 1024; }  // 512 x 64
      else { c->tile = 32768; c->threads = 256; c->trb = 512; }                          // 256 x 64
      c->cap = 2;
      return true;
    default:
      return false;
  }
}

// log2 of a power of two (the next one up otherwise)
static int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// The tile geometries of one configuration, in the candidate order of destination run length
// (the configuration's own, then 128, 256, 64 bytes): the first with a conflict-free swizzle, else
// the one with the fewest extra LDS cycles.  False if no geometry fits a kernel instance.
static bool plan_with_cfg(const Plan& p, int flags, TuneCfg cfg, bool tile_pinned, TileGeom* out, int64_t* out_w,
                          int64_t* out_r) {
  const Joint& j = p.j;
  const Mode& R = j.m[p.mode_r];
  const Mode& C = j.m[p.mode_c];
  const int unit_min = p.eb < 4 ? 4 : p.eb;
  // no bigger than the copy needs: shrink small copies' tiles (instances exist for 8, 16, 32 and
  // 64 KiB), rather than filling them with positions outside the copy
  const int64_t eB = p.mode_b >= 0 ? j.m[p.mode_b].e : 1;
  const int64_t useful = pow2ceil(R.e) * pow2ceil(C.e) * pow2ceil(eB) * p.eb;
  while (!tile_pinned && cfg.tile > 8192 && cfg.tile / 2 >= useful) cfg.tile /= 2;
  // only configurations the library holds a kernel for (each gives every thread whole loads):
  // the same tile with 256 threads, else 16 KiB tiles of 256 threads (every vector width)
  const int unit0 = cfg.unit ? cfg.unit : unit_min;
  auto instance = [&](int tile, int threads) {
    return launch_transpose(p.eb, TransposeCfg{p.vb, unit0, tile, threads, cfg.nt, p.step, false, true, std::max(cfg.cap, 0),
                                               cfg.nar},
                            nullptr, 0, nullptr);
  };
  if (!instance(cfg.tile, cfg.threads)) {
    if (instance(cfg.tile, 256)) {
      cfg.threads = 256;
    } else {
      cfg.tile = 16384;
      cfg.threads = 256;
    }
  }
  const int trb_list[] = {cfg.trb ? cfg.trb : 128, 128, 256, 64};
  bool have = false;
  int64_t best_cost = -1;
  int seen[64][4];
  int nseen = 0;
  // Without the swizzle only the first geometry is planned, so that TC_FLAG_NO_SWIZZLE measures
  // the swizzle on the tile the default plan uses.
  const bool first_only = flags & TC_FLAG_NO_SWIZZLE;
  for (int trb : trb_list) {
    if (first_only && have) break;
    const int unit = unit0;
    TileGeom g;
    g.eb = p.eb;
    g.vb = p.vb;
    g.U = unit;
    g.NT = cfg.threads;
    g.tile_bytes = cfg.tile;
    g.ntm = cfg.nt;
    g.order = cfg.order;
    g.step = p.step;
    g.cap = std::max(cfg.cap, 0);
    g.nar = cfg.nar;
    if (cfg.ssr > 0) g.lsr = ilog2(cfg.ssr);
    if (cfg.ssc > 0) g.lsc = ilog2(cfg.ssc);
    if (unit < p.eb || unit < 4 || unit > p.vb) continue;
    const int ve = p.vb / p.eb;
    const int bmin = unit / p.eb;
    int64_t TR = std::max<int64_t>(trb / p.eb, 1);
    TR = std::max<int64_t>(std::min<int64_t>(TR, pow2ceil(R.e)), std::max(ve, bmin));
    int64_t TC = std::max<int64_t>(cfg.tile / (TR * p.eb), 1);
    TC = std::max<int64_t>(std::min<int64_t>(TC, pow2ceil(C.e)), ve);
    // source runs of at least one 128-byte cache line where the extent has them
    if (TC * p.eb < 128 && TC < pow2ceil(C.e)) continue;
    int64_t NB = cfg.tile / (TR * TC * p.eb);
    if (NB < 1) continue;
    g.TR = int(TR);
    g.TC = int(TC);
    g.NB = int(NB);
    bool dup = false;
    for (int i = 0; i < nseen; ++i)
      if (seen[i][0] == g.TR && seen[i][1] == g.TC && seen[i][2] == g.NB && seen[i][3] == g.U) dup = true;
    if (dup || nseen >= 64) continue;
    seen[nseen][0] = g.TR; seen[nseen][1] = g.TC; seen[nseen][2] = g.NB; seen[nseen][3] = g.U; ++nseen;
    if (!finish_geom(&g)) continue;
    if (!launch_transpose(g.eb, TransposeCfg{g.vb, g.U, g.tile_bytes, g.NT, g.ntm, g.step, false, true, g.cap, g.nar},
                          nullptr, 0, nullptr))
      continue;
    TileGeom c;
    int64_t wc, rc;
    if (!search_swizzle(g, flags & TC_FLAG_NO_SWIZZLE, &c, &wc, &rc)) continue;
    if (best_cost < 0 || wc + rc < best_cost) {
      best_cost = wc + rc;
      *out = c;
      *out_w = wc;
      *out_r = rc;
      have = true;
    }
    if (wc + rc == 0) return true;
  }
  return have;
}

// The tile configuration of a transpose.  Three classes of layout, each configuration measured on
// MI355X (TC_TUNE pins one for sweeps):
//  - both sides on 128-byte lines: the tall tiles where tall_cfg has them (row tiles first,
//    nontemporal accesses), else default_cfg;
//  - neighbouring tiles sharing cache lines (`line_cfg`): vectors at element alignment, or, for
//    1-, 2- and 8-byte elements, destination columns off the lines, or, for 1-byte elements,
//    source rows off the lines: plain stores and the element-aligned configuration of the width
//    (int8 small tiles and fp16 tall tiles in the XCD super-tile order, fp64 16 KiB tiles);
//  - row tiles first with source rows off the lines: the row-tile count padded to a multiple of
//    kXcds (with_phase_order below).
static bool plan_transpose_tile(Plan* p, int flags) {
  const Joint& j = p->j;
  const Mode& R = j.m[p->mode_r];
  const Mode& C = j.m[p->mode_c];
  const bool batched = pow2ceil(R.e) * p->eb < 128;
  const TuneCfg ov = tune_override();
  if (p->nar) {
    // int8 with a stride-2 source read as 2-byte pairs (make_plan): the tall 512 x 64 tiles of
    // 2-byte elements with nontemporal accesses, 2 loads in flight and super-tiles of 16 x 4
    // tiles; the low byte of each pair is stored.  Measured on the 8192^2 slice [1:8191, 0:8190:2]
    // against the stride-2 tile of 1-byte elements: 2.25-2.28 -> 2.75-2.76 TB/s (16 x 2, 32 x 2,
    // 32 x 4, 16 x 8 and 8 x 8 super-tiles 2.53-2.63, row tiles first 2.44, 1024 x 64 tiles on
    // 1024 lanes 2.47-2.66).  The same reading of a 2-byte source as 4-byte pairs measured slower
    // than its own stride-2 tile (fp16 slice 2.80 against 2.19-2.50), so only 1-byte copies take it.
    TuneCfg t;
    t.tile = 65536; t.threads = 512; t.trb = 1024; t.unit = 16; t.nt = 3; t.order = 2; t.cap = 2;
    t.ssr = 16; t.ssc = 4; t.nar = p->nar;
    if (p->eb == 16) {
      // fp64 with a stride-2 source read as 16-byte pairs: 64 x 8 tiles of pairs on 256 lanes in XCD
      // super-tiles of 16 x 16 tiles, every load in flight.  Measured against the stride-2 tile of
      // 8-byte elements (16 x 128 on 512 lanes, column tiles first): the slice [1:8191, 0:8190:2]
      // of 8192^2 3.20-3.23 -> 3.70-3.74 TB/s, every other column of 16384 x 8192 3.40 -> 3.74-3.75,
      // of 8192 x 16384 3.20-3.21 -> 3.95-3.96, of 4096^2 3.28 -> 4.00-4.02 (8 x 16 super-tiles
      // 3.70 / 3.75 / 3.84-3.85 / 3.98-4.00, 16 x 8 3.34-3.97, 8 x 8 3.25-3.49, row tiles first
      // 2.64, column tiles first 2.93-2.96; 64 x 16 tiles 2.73-3.55, 64 x 32 on 512 lanes 2.68-3.28)
      t.tile = 8192; t.threads = 256; t.trb = 1024; t.order = 2; t.cap = 0; t.ssr = 16; t.ssc = 16;
    }
    if (p->eb == 8 && p->nar == 1) {
      // fp32 with a stride-2 source read as 8-byte pairs: 128 x 32 tiles of pairs on 512 lanes in
      // 16 x 16 super-tiles, 2 loads in flight.  Against the stride-2 tile of 4-byte elements: the
      // slice [1:8191, 0:8190:2] of 8192^2 3.35 -> 3.75-3.78 TB/s, every other column of 8192^2
      // 3.49 -> 3.87-3.91, of 4096 x 8192 3.32-3.34 -> 3.61-3.63, of 16384 x 4096 3.40 -> 3.43-3.46
      // (8 x 8 super-tiles 3.95 on the slice but 3.23 on 16384 x 4096; row tiles first 2.85)
      t.tile = 32768; t.threads = 512; t.trb = 1024; t.order = 2; t.cap = 2; t.ssr = 16; t.ssc = 16;
    }
    if (p->eb == 4 && p->nar == 1) {
      // fp16 with a stride-2 source read as 4-byte pairs: 256 x 32 tiles of pairs on 512 lanes in
      // XCD super-tiles of 16 x 16 tiles, 2 loads in flight.  Measured on the slice
      // [1:8191, 0:8190:2] of 8192^2 against the stride-2 tile of 2-byte elements (2.82 TB/s):
      // 3.43 (8 x 8 super-tiles 3.41; 256 x 64 tiles 2.29-2.72 in four orders, 32 x 128 on 256
      // lanes 1.59)
      t.tile = 32768; t.threads = 512; t.trb = 1024; t.order = 2; t.cap = 2; t.ssr = 16; t.ssc = 16;
    }
    if (p->nar == 3) {
      // a stride-4 source read in groups of 4 elements: tiles of 32 groups by 1 KiB (4- and 8-byte
      // groups: 256 x 32 and 128 x 32) or 512 bytes on 256 lanes (16-byte groups: 32 x 32) in
      // row-tile-first order with 2 loads in flight.  Measured against the stride-4 tile of the
      // element width: every 4th byte of 8192 x 32768 transposed 1.33 -> 2.35-2.36 TB/s (256 x 64
      // tiles 1.83-1.85, with all loads in flight 1.63-1.70; 128 x 64 2.18; 128 x 32 on 256 lanes
      // 2.32; 16 x 2 or 8 x 8 super-tiles 2.18-2.23, column tiles first 1.53); every 4th fp16 of
      // 8192 x 16384 1.75-1.76 -> 2.00-2.03 (128 x 64 1.76, 64 x 32 and 128 x 16 on 256 lanes
      // 1.97-2.01, 16 x 2 super-tiles 2.04-2.06); every 4th fp32 of 8192 x 8192 (the guarded tile
      // before) 1.60-1.61 -> 2.13-2.16 (64 x 32 on 512 lanes 1.98, 64 x 64 1.97-1.98, 32 x 64 2.08-2.11)
      t.tile = p->eb == 16 ? 16384 : 32768;
      t.threads = p->eb == 16 ? 256 : 512;
      t.trb = p->eb == 16 ? 512 : 1024;
      t.order = 1; t.cap = 2; t.ssr = 0; t.ssc = 0;
    }
    // (the tuning override's tile, threads, trb, nt, order, cap and super-tile keys apply here too)
    if (ov.tile) t.tile = ov.tile;
    if (ov.nt >= 0) t.nt = ov.nt;
    if (ov.threads) t.threads = ov.threads;
    if (ov.trb) t.trb = ov.trb;
    if (ov.order >= 0) t.order = ov.order;
    if (ov.cap >= 0) t.cap = ov.cap;
    if (ov.ssr > 0) t.ssr = ov.ssr;
    if (ov.ssc > 0) t.ssc = ov.ssc;
    TileGeom g;
    int64_t wc, rc;
    if (!plan_with_cfg(*p, flags, t, true, &g, &wc, &rc)) return false;
    p->g = g;
    p->wconf = wc;
    p->rconf = rc;
    return true;
  }
  const bool pinned = ov.tile || ov.threads || ov.nt >= 0 || ov.order >= 0 || ov.trb || ov.unit;
  // 1-, 2- and 8-byte elements whose destination columns do not start on 128-byte lines (a
  // line-aligned base pointer assumed): the configurations of the element-aligned plans (plain
  // stores; below) measured faster than the tall tiles with nontemporal stores: fp64 8190 x 8192
  // 3.63 -> 5.24 TB/s and 8184 x 8184 3.71 -> 4.97, fp16 8184 x 8184 3.59 -> 4.22, int8 8176 x 8192
  // 3.34 -> 3.51.  (fp32 such copies were 4-7% slower with it, 16-byte elements equal.)
  // 1-byte rows shorter than a line but packed one after another on a side (the channels of an
  // NCHW <-> NHWC permute: 32 or 64 bytes per pixel) count as on the lines there: a tile spans
  // whole rows, so its block is contiguous and shares no line with its neighbours.
  const Mode& mR = j.m[p->mode_r];
  const Mode& mC = j.m[p->mode_c];
  const bool packed_dst = p->eb == 1 && !p->unaligned && mC.d == mR.e && mR.e * p->eb < 128;
  const bool packed_src = p->eb == 1 && !p->unaligned && mR.s == mC.e && mC.e * p->eb < 128;
  bool dst_lines = (j.dof * p->eb) % 128 == 0;
  for (int k = 0; k < j.rank; ++k)
    if (k != p->mode_r && (std::llabs(j.m[k].d) * p->eb) % 128 != 0 && !(k == p->mode_c && packed_dst))
      dst_lines = false;
  // (and whether the source rows start on 128-byte lines: for 1-byte elements either side off
  // the lines takes the element-aligned configuration, int8 8192 x 8208 3.9 -> 4.5 TB/s and
  // 8320 x 8224 3.84 -> 4.77)
  bool src_lines = (j.so * p->eb) % 128 == 0;
  for (int k = 0; k < j.rank; ++k)
    if (k != p->mode_c && (std::llabs(j.m[k].s) * p->eb) % 128 != 0 && !(k == p->mode_r && packed_src))
      src_lines = false;
  const bool line_cfg = p->unaligned || ((p->eb == 1 || p->eb == 2 || p->eb == 8) && !dst_lines) ||
                        (p->eb == 1 && !src_lines);
  TuneCfg base = default_cfg(p->eb, batched, line_cfg);
  // 1-byte elements there, and element-aligned 8-byte elements read with unit stride: the XCD
  // super-tile order, so that the neighbouring tiles that share cache lines at element alignment
  // run in one L2 (measured: int8 8191 x 8190 3.02 -> 3.20 TB/s, the int8 slice 1.75 -> 2.06,
  // fp64 8191 x 8190 4.81 -> 5.17; the 8- and 16-byte slices 8-10% slower with it)
  if (line_cfg && (p->eb == 1 || (p->eb == 8 && p->unaligned && p->step == 1))) base.order = 2;
  if (ov.tile) base.tile = ov.tile;
  if (ov.threads) base.threads = ov.threads;
  if (ov.nt >= 0) base.nt = ov.nt;
  if (ov.order >= 0) base.order = ov.order;
  base.trb = ov.trb;
  base.unit = ov.unit;
  // candidate configurations: the tall tile where it pays (not under TC_TUNE), then the default
  // (at most one of the rules below applies to a copy; room for all of them)
  TuneCfg cands[5];
  int ncand = 0;
  TuneCfg tall;
  const int64_t others = j.count / (R.e * C.e);
  // (element-aligned plans: only 16-byte elements gained, 4870 -> 5140 GB/s on 8191 x 8190)
  // (1-byte rows of 64 bytes or more count as long enough for the narrow int8 tiles)
  const bool short_rows = batched && !(p->eb == 1 && R.e >= 64);
  if (!pinned && !short_rows && (!line_cfg || (p->unaligned && p->eb == 16)) && p->vb == 16 && p->step == 1 &&
      tall_cfg(p->eb, R.e, C.e, others, &tall))
    cands[ncand++] = tall;
  // 2-byte elements there, read with unit stride: tall 512 x 64 tiles with plain stores in the XCD
  // super-tile order (fp16 8191 x 8190 3.86 -> 4.15 TB/s; with column tiles first such tiles had
  // been slower than 64 x 64 ones)
  // Where the source rows are on the lines and only the destination is off them, with nontemporal
  // accesses and 2 loads in flight (fp16 8191 x 8192 4.28-4.36 -> 4.55-4.57 TB/s, 16383 x 8192 4.66
  // -> 5.05-5.06, 8190 x 8192 4.41 -> 4.80-4.81, 8191 x 16384 4.41 -> 4.60-4.61; with the source off
  // the lines too they measured slower: 8191 x 8190 4.33 -> 3.84-3.86)
  if (!pinned && !batched && line_cfg && p->eb == 2 && p->step == 1 && R.e >= 512 && C.e >= 64) {
    TuneCfg t;
    t.tile = 65536; t.threads = 512; t.trb = 1024; t.unit = 16; t.nt = 0; t.order = 2;
    if (src_lines) { t.nt = 3; t.cap = 2; }
    cands[ncand++] = t;
  }
  // 1-byte elements whose vectors are at element alignment only on the destination side (source
  // rows on the lines): the tall 512 x 256 tiles of tall_cfg, nontemporal accesses, 2 loads in
  // flight, 16 x 2 super-tiles (int8 8191 x 8192 3.64-3.66 -> 4.01-4.05 TB/s, 8191 x 16384 3.63 ->
  // 3.97-3.98, 12287^2 3.37-3.39 -> 3.85, 8190 x 8192 3.53-3.59 -> 4.09-4.11, 16383 x 8192 level;
  // a source off the lines makes these tiles slower than the small ones: 8191 x 8190 3.67 -> 2.70,
  // 8192 x 8190 4.07 -> 3.30)
  if (!pinned && !batched && p->unaligned && p->eb == 1 && src_lines && p->step == 1 && R.e >= 512 &&
      C.e >= 256 && ceil_div(R.e, 512) * ceil_div(C.e, 256) * others >= 512) {
    TuneCfg t;
    t.tile = 131072; t.threads = 512; t.trb = 512; t.unit = 16; t.nt = 3; t.order = 2; t.cap = 2;
    t.ssr = 16; t.ssc = 2;
    cands[ncand++] = t;
  }
  // 1-byte elements at vector alignment whose destination columns alone are off the lines: the
  // tall 512 x 256 tiles with 2 loads in flight, plain stores and XCD super-tiles of 16 x 2 tiles
  // as in tall_cfg (int8 8176 x 8192 3.56-3.57 -> 4.02-4.08 TB/s with 8 x 8 super-tiles, 4.08-4.17
  // with 16 x 2; 8160 x 8192 3.63-3.64 -> 4.10-4.16; the odd and source-misaligned int8 copies ran
  // slower on these tiles)
  if (!pinned && !batched && line_cfg && p->eb == 1 && !p->unaligned && src_lines && p->step == 1 && R.e >= 512 &&
      C.e >= 256 && ceil_div(R.e, 512) * ceil_div(C.e, 256) * others >= 512) {
    TuneCfg t;
    t.tile = 131072; t.threads = 512; t.trb = 512; t.unit = 16; t.nt = 0; t.order = 2; t.cap = 2;
    t.ssr = 16; t.ssc = 2;
    cands[ncand++] = t;
  }
  cands[ncand++] = base;
  if (flags & TC_FLAG_NO_SWIZZLE) ncand = 1;  // the swizzle is measured on the default plan's tile
  if (ov.cap >= 0)
    for (int i = 0; i < ncand; ++i) cands[i].cap = ov.cap;
  // Row tiles first with source rows off the lines: neighbouring column tiles read the same lines.
  // They are tilesR workgroups apart, so the grid pads tilesR to a multiple of kXcds and puts them
  // on one XCD (bf16 16448 x 16392 3.48 -> 4.3 TB/s, fp32 16416 x 16400 5.07 -> 5.4).  Wave-local
  // phases drop the workgroup barrier where the library holds such an instance.
  auto with_phase_order = [&](TileGeom g) {
    g.pad_rows = g.order == 1 && !src_lines;
    if (ov.ssr > 0) g.lsr = ilog2(ov.ssr);
    if (ov.ssc > 0) g.lsc = ilog2(ov.ssc);
    g.wave_local = ov.wl != 0 && tile_wave_local(g) &&
                   launch_transpose(g.eb, TransposeCfg{g.vb, g.U, g.tile_bytes, g.NT, g.ntm, g.step, true, true, g.cap},
                                    nullptr, 0, nullptr);
    return g;
  };
  // a swizzle forced by the tuning override replaces the chosen one on the chosen tile
  auto forced_swizzle = [&](TileGeom* g, int64_t* wc, int64_t* rc) {
    if (ov.xk < 0) return true;
    g->k = ov.xk;
    g->shift = ov.xs;
    g->tbit = ov.xt;
    g->cshift = ov.xcs;
    g->cmask = ov.xcm;
    if (!finish_geom(g)) return false;
    simulate_tile(*g, wc, rc);
    return true;
  };
  bool have = false;
  TileGeom best;
  int64_t best_w = 0, best_r = 0;
  for (int i = 0; i < ncand; ++i) {
    TileGeom g;
    int64_t wc, rc;
    if (!plan_with_cfg(*p, flags, cands[i], ov.tile != 0, &g, &wc, &rc)) continue;
    if (wc + rc == 0) {
      if (!forced_swizzle(&g, &wc, &rc)) return false;
      p->g = with_phase_order(g);
      p->wconf = wc;
      p->rconf = rc;
      return true;
    }
    if (!have || wc + rc < best_w + best_r) {
      best = g;
      best_w = wc;
      best_r = rc;
      have = true;
    }
  }
  if (!have) return false;
  if (ov.xk >= 0) {
    if (!forced_swizzle(&best, &best_w, &best_r)) return false;
    p->g = with_phase_order(best);
    p->wconf = best_w;
    p->rconf = best_r;
    return true;
  }
  p->g = with_phase_order(best);
  p->wconf = best_w;
  p->rconf = best_r;
  decline(p, flags, "no XOR swizzle leaves both LDS phases conflict-free (best: " + std::to_string(best_w) +
                        " write + " + std::to_string(best_r) + " read extra cycles per tile)");
  return true;
}

// Workgroups of a transpose plan over modes r, c and batch mode b (the XCD super-tile order pads
// the grid to whole groups of kXcds super-tiles; its padding workgroups return at once).
static int64_t transpose_workgroups(const Plan& p, int r, int c, int b) {
  const Joint& j = p.j;
  int64_t tR = ceil_div(j.m[r].e, p.g.TR);
  const int64_t tC = ceil_div(j.m[c].e, p.g.TC);
  if (p.g.pad_rows) tR = ceil_div(tR, kXcds) * kXcds;
  int64_t slices = ceil_div(b >= 0 ? j.m[b].e : 1, p.g.NB);
  for (int k = 0; k < j.rank; ++k)
    if (k != r && k != c && k != b) slices *= j.m[k].e;
  if (p.g.order != 2) return tR * tC * slices;
  const int64_t nst = ceil_div(tR, int64_t(1) << p.g.lsr) * ceil_div(tC, int64_t(1) << p.g.lsc);
  return ceil_div(nst * slices, kXcds) * kXcds * (int64_t(1) << (p.g.lsr + p.g.lsc));
}

// Rows-type copies of 2^31 vectors or more launch ranges of the outermost grid mode, at most
// kLaunchVectors vectors each: one index of that mode must fit one launch.
static bool rows_fit(const Joint& j, int64_t nvec) {
  if (nvec < (int64_t(1) << 31) || j.rank <= 1) return true;
  return nvec / j.m[0].e <= kLaunchVectors;
}

Plan make_plan(const tc_layout& src, const tc_layout& dst, int dtype, int flags, int ptr_align) {
  Plan p;
  std::string err;
  if (ptr_align <= 0) ptr_align = 16;
  p.eb = elem_bytes_of(dtype);
  if (p.eb < 0) {
    p.status = TC_E_DTYPE;
    p.reason = "unknown dtype " + std::to_string(dtype);
    return p;
  }
  if (flags & ~TC_FLAG_ALL) {
    p.status = TC_E_ARG;
    p.reason = "unknown flag bits";
    return p;
  }
  int st = make_joint(src, dst, &p.j, &err);
  if (st != TC_OK) {
    p.status = st;
    p.reason = err;
    return p;
  }
  if (p.j.count == 0) {
    p.path = TC_PATH_EMPTY;
    return p;
  }
  canonicalize(&p.j);
  const int inj = dst_injective(p.j);
  if (inj != 1) {
    p.status = TC_E_NONINJECTIVE;
    p.reason = inj == 0 ? "destination layout maps two logical indices to one element"
                        : "destination layout could not be shown injective";
    return p;
  }
  Joint& j = p.j;
  // modes contiguous on each side
  int r = -1, c = -1;
  for (int k = 0; k < j.rank; ++k) {
    if (j.m[k].d == 1 && r < 0) r = k;
    if (j.m[k].s == 1 && c < 0) c = k;
  }
  // Modes walked backwards.  Reversing a mode's logical index (i -> e - 1 - i: both strides
  // negated, both offsets moved to the mode's other end) names the same pairs of elements, so the
  // planner reverses: every mode both sides walk backwards; then a mode the destination walks
  // backwards with unit stride when none is contiguous there (a copy into a flipped view); then a
  // mode the source walks backwards with unit stride, other than the destination's contiguous
  // one, when none is contiguous there (a matrix rotated by 90 degrees, or flipped along its
  // columns and transposed).  Each side then reads or writes it forwards and the ordinary paths
  // take it.  (A row the source walks backwards, with the destination contiguous along it, stays
  // as it is: gathered rows.)
  auto reverse_mode = [&](int k) {
    j.so += (j.m[k].e - 1) * j.m[k].s;
    j.dof += (j.m[k].e - 1) * j.m[k].d;
    j.m[k].s = -j.m[k].s;
    j.m[k].d = -j.m[k].d;
  };
  bool reversed = false;
  for (int k = 0; k < j.rank; ++k)  // walked backwards on both sides: forwards on both
    if (j.m[k].s < 0 && j.m[k].d < 0) {
      reverse_mode(k);
      reversed = true;
    }
  if (reversed) {
    r = c = -1;
    for (int k = 0; k < j.rank; ++k) {
      if (j.m[k].d == 1 && r < 0) r = k;
      if (j.m[k].s == 1 && c < 0) c = k;
    }
  }
  if (r < 0)
    for (int k = 0; k < j.rank; ++k)
      if (j.m[k].d == -1) {
        reverse_mode(k);
        r = k;
        c = -1;
        for (int q = 0; q < j.rank && c < 0; ++q)
          if (j.m[q].s == 1) c = q;
        reversed = true;
        break;
      }
  if (c < 0)
    for (int k = 0; k < j.rank; ++k)
      if (k != r && j.m[k].s == -1) {
        reverse_mode(k);
        reversed = true;
        break;
      }
  if (reversed) {  // modes that now line up merge (a copy flipped on both sides: one contiguous run)
    canonicalize(&j);
    r = c = -1;
    for (int k = 0; k < j.rank; ++k) {
      if (j.m[k].d == 1 && r < 0) r = k;
      if (j.m[k].s == 1 && c < 0) c = k;
    }
  }
  const int c_unit = c;
  const bool forced_guarded = flags & TC_FLAG_FORCE_GUARDED;
  if (j.count % kWave != 0)
    decline(&p, flags, "element count " + std::to_string(j.count) + " is not divisible by the thread count " +
                           std::to_string(kWave) + ": the [outer, threads, vec] split has no integer solution");
  if (p.status != TC_OK) return p;

  bool fast = !p.declined && !forced_guarded && j.rank >= 1;
  // Outside strict mode, a copy declined by the count rule alone whose 16-byte vectors are whole
  // and aligned on both sides still takes the aligned kernels, whose guards cover a partial last
  // workgroup (rows) or partial tiles (transposes); the plan keeps the page's reason.  (Such a
  // contiguous int8 copy of 64 MiB: 5.46 TB/s on the element-aligned rows, against about 6.1 for
  // the aligned rows kernel at that size.)
  if (p.declined && !forced_guarded && j.rank >= 1 && r >= 0 && c >= 0 && choose_vec(j, p.eb, c, r, ptr_align) == 16)
    fast = true;
  if (fast && (r < 0 || c < 0)) {
    decline(&p, flags, std::string("no unit-stride mode on the ") + (r < 0 ? "destination" : "source") +
                           " side: no vector of 4 bytes or more is contiguous there");
    fast = false;
  }
  if (fast) {
    p.vb = choose_vec(j, p.eb, c, r, ptr_align);
    if (p.vb == 0) {
      decline(&p, flags, "no vector of 16, 8 or 4 bytes is contiguous and aligned on both sides");
      fast = false;
    }
  }
  if (p.status != TC_OK) return p;
  // The page's rule can leave a transpose 8- or 4-byte vectors (pitches that are multiples of
  // them but not of 16 bytes).  Outside strict mode such a transpose takes 16-byte vectors at
  // element alignment instead, which measured 1.1-2.8x faster on MI355X (8192 x 8192 copies with
  // pitch 8188 or 8190: int8 1960 -> ~3600 GB/s, fp16 1440-1720 -> ~4000).  Strict mode keeps the
  // page's plan.
  if (fast && p.vb < 16 && !(flags & TC_FLAG_STRICT)) {
    p.reason = "the aligned split allows only " + std::to_string(p.vb) +
               "-byte vectors: 16-byte vectors at element alignment instead";
    fast = false;
  }

  if (fast && r == c) {
    // Both sides contiguous along one mode: no cross-lane exchange needed.
    const bool small = j.count * p.eb <= kSmallCopyBytes;
    const bool lds = (flags & TC_FLAG_FORCE_LDS) || (small && !(flags & TC_FLAG_FORCE_REGS));
    p.path = lds ? TC_PATH_ROUNDTRIP : TC_PATH_ROWS;
    p.ntm = lds ? 0 : 3;  // streaming copies: nontemporal loads and stores (measured faster)
    p.threads = lds ? kWave : kRowThreads;
    const int64_t nvec = j.count / (p.vb / p.eb);
    // Loads of a thread all at once for contiguous copies of <= 256 MiB each way (measured 4-5%
    // faster there); one at a time elsewhere: permuted rows (the (0,2,1,3) permute: 6.2 vs 5.8
    // TB/s) and large contiguous copies (6.33 vs 6.26 TB/s) ran faster with the paced loads.
    p.row_burst = !lds && j.rank == 1 && j.count * p.eb <= kRowSmallBytes;
    if (!lds && p.vb == 16) {
      const TuneCfg tc = tune_override();
      p.buffers = tc.buf != 0;
      p.row_src_order = tc.so >= 0 ? tc.so == 1 : row_src_order(j, p.eb);
      p.row_rounds = row_rounds(j, p.eb, p.row_src_order);
      if (tc.rr == 1 || tc.rr == 2 || tc.rr == 4) p.row_rounds = tc.rr;
    }
    const int64_t per_wg = int64_t(p.threads) * p.row_rounds;
    p.workgroups = ceil_div(nvec, per_wg);
    p.load_outer = p.store_outer = int(std::min<int64_t>(p.row_rounds, ceil_div(nvec, p.threads)));
    p.lds_bytes = lds ? int(per_wg * p.vb) : 0;
    if (!rows_fit(rows_grid(p), nvec)) {
      p.status = TC_E_RANGE;
      p.reason = "more than 2^30 vectors per index of the outermost mode";
    }
    return p;
  }
  if (fast && !(flags & TC_FLAG_NO_SHUFFLE) && p.eb == 4 && p.vb == 16 && j.rank <= 3) {
    // 4 x C blocks, row-major in the source and column-major in the destination, one batch mode:
    // the lanes' 16-byte vectors are exchanged in registers (a two-stage butterfly), no LDS
    const Mode& R = j.m[r];
    const Mode& C = j.m[c];
    int b = -1;
    for (int k = 0; k < j.rank; ++k)
      if (k != r && k != c) b = k;
    const bool block = R.e == 4 && (C.e == 8 || C.e == 16 || C.e == 32) && r != c && R.s == C.e && C.s == 1 &&
                       R.d == 1 && C.d == 4;
    if (block) {
      p.path = TC_PATH_SHUFFLE;
      p.mode_r = r;
      p.mode_c = c;
      p.mode_b = b;
      p.shuffle_c = int(C.e);
      p.threads = kShuffleThreads;
      p.load_outer = p.store_outer = kShuffleRounds;
      p.ntm = 3;
      p.buffers = tune_override().buf != 0;
      const int64_t nvec = j.count / 4;
      p.workgroups = ceil_div(nvec, int64_t(kShuffleThreads) * kShuffleRounds);  // over all launches
      return p;
    }
  }
  // A few interleaved channels to planes (NHWC -> NCHW with 3 channels): the channel mode is too
  // short for a vector, so each lane takes 16/eb pixels of every channel (C 16-byte loads),
  // transposes them in its registers and stores C vectors, one per plane.  Needs 16-byte alignment
  // of every pixel group on both sides and a pixel count that is a multiple of 16/eb.
  if (!forced_guarded && !(flags & (TC_FLAG_STRICT | TC_FLAG_NO_SHUFFLE)) && r >= 0 && c >= 0 && r != c &&
      p.eb <= 8 && ptr_align >= 16) {
    const Mode& R = j.m[r];  // destination-contiguous
    const Mode& C = j.m[c];  // source-contiguous
    const int64_t ve = 16 / p.eb;
    auto channels_ok = [](int64_t e) { return e == 2 || e == 3 || e == 4 || e == 8; };
    // to planes: channels are the source-contiguous mode; from planes: the destination's
    // (measured on 32 x 224 x 224 images against the transpose kernel: faster up to 12 bytes of
    // channels per pixel and for 8-byte elements, e.g. fp32 with 3 channels 2.8 -> 3.7 TB/s, fp64
    // with 4 channels 1.7 -> 4.0; slower for bf16 with 8 channels and fp32 with 8)
    const bool to = channels_ok(C.e) && (C.e * p.eb <= 12 || p.eb == 8) && R.s == C.e && R.e % ve == 0;
    // (planes to interleaved channels ran slower than the transpose kernel: a lane's C vectors
    // are adjacent in the destination, so each store instruction writes 16 of every 16*C bytes)
    const bool from = false;
    bool ok = to || from;
    const Mode& S = to ? C : R;  // channels
    const int64_t plane = to ? S.d : S.s;  // planar side's channel stride
    ok = ok && (plane * p.eb) % 16 == 0 && (j.so * p.eb) % 16 == 0 && (j.dof * p.eb) % 16 == 0;
    for (int k = 0; ok && k < j.rank; ++k)
      if (k != r && k != c && ((j.m[k].s * p.eb) % 16 != 0 || (j.m[k].d * p.eb) % 16 != 0)) ok = false;
    if (ok) {
      p.path = TC_PATH_INTERLEAVE;
      p.to_planes = to;
      p.mode_r = r;
      p.mode_c = c;
      p.shuffle_c = int(S.e);
      p.vb = 16;
      p.ntm = 3;
      p.threads = kRowThreads;
      p.load_outer = p.store_outer = int(S.e) * kInterleaveRounds;
      const int64_t groups = j.count / (S.e * ve);
      p.workgroups = ceil_div(groups, int64_t(kRowThreads) * kInterleaveRounds);
      if (groups >= (int64_t(1) << 31)) {
        p.status = TC_E_RANGE;
        p.reason = "more than 2^31 pixel groups";
      }
      return p;
    }
  }
  if (fast) {
    p.path = TC_PATH_TRANSPOSE;
    p.mode_r = r;
    p.mode_c = c;
    // batch mode folded into the tile: the remaining mode with the smallest strides
    int b = -1;
    for (int k = 0; k < j.rank; ++k) {
      if (k == r || k == c) continue;
      if (b < 0 || std::llabs(j.m[k].s) + std::llabs(j.m[k].d) < std::llabs(j.m[b].s) + std::llabs(j.m[b].d)) b = k;
    }
    p.mode_b = b;
    // the widest vector whose tile gives every thread whole loads and stores
    while (!plan_transpose_tile(&p, flags)) {
      p.vb = p.vb > 4 ? choose_vec(j, p.eb, c, r, ptr_align, p.vb / 2) : 0;
      if (p.vb == 0) {
        p.path = TC_PATH_EMPTY;
        p.status = TC_E_ARG;
        p.reason = "internal: no tile geometry";
        return p;
      }
    }
    if (p.status != TC_OK) return p;
    p.threads = p.g.NT;
    p.load_outer = p.g.loads;
    p.store_outer = p.g.stores;
    p.lds_bytes = p.g.tile_bytes;
    const int64_t eB = b >= 0 ? j.m[b].e : 1;
    // Copies tiled exactly run the interior-only kernel (fewer registers: two bf16 workgroups per
    // CU instead of one).  Measured against the kernel with its guards, interleaved on MI355X:
    // int8 8192^2 +6%, fp64 8192^2 +1-4%, fp16 8192^2 +1%, bf16 and fp32 16384^2 equal, but
    // 16-byte elements 8192^2 -5% (5.70 against 6.00 TB/s), so those keep the guarded kernel.
    p.g.edges = j.m[r].e % p.g.TR != 0 || j.m[c].e % p.g.TC != 0 || eB % p.g.NB != 0 ||
                p.g.step != 1 || p.eb == 16;
    p.workgroups = transpose_workgroups(p, r, c, b);
    if (p.workgroups >= (int64_t(1) << 31)) {
      p.status = TC_E_RANGE;
      p.reason = "more than 2^31 workgroups";
    }
    return p;
  }

  // Declined by the aligned-vector rule, but the destination has a unit-stride mode and the
  // source a distinct mode of stride 1 to 4: the transpose kernel with 16-byte vectors at element
  // alignment (gfx950 global memory takes unaligned vector accesses), whole vectors where the
  // extents allow and element accesses at the edges of the copy.  Along a stride-2 mode every
  // vector is read as two contiguous ones (the elements in between are fetched and dropped), along
  // a stride-3 or -4 mode as the 16-byte loads of its span.
  // Other strides only where the source has no unit-stride mode at all: -1 and -2 (reversed
  // columns, e.g. a rotation by 90 degrees), and strides of magnitude 3 and 4 where the elements
  // lie at most 12 bytes apart: measured against the guarded tile on 8192-row copies on MI355X,
  // int8 stride 3 1.10 -> 1.97 TB/s, stride 4 1.11 -> 1.28, fp16 stride 3 1.90 -> 2.48, fp32
  // stride 3 2.14 -> 2.26; fp16 stride 4 level (1.65 / 1.67), and fp32 stride 4, fp64 and 16-byte
  // elements 1-8% slower than the guarded tile, which they keep.  (Each lane's loads then touch a
  // 64-byte segment apiece, so a wave's load requests, not the bytes, set the pace.)  The stride
  // of smallest magnitude is taken, the positive one on a tie.
  int c2 = c;
  if (c2 < 0 || c2 == r)
    for (int k = 0; k < j.rank; ++k) {
      const int64_t s = j.m[k].s, as = std::llabs(s);
      const bool strided =
          s == 2 || (c < 0 && s != 1 && (s == -1 || s == -2 || ((as == 3 || as == 4) && as * p.eb <= 12)));
      const auto better = [&](int q) {
        const int64_t aq = std::llabs(j.m[q].s);
        return as < aq || (as == aq && s > 0 && j.m[q].s < 0);
      };
      if (k != r && strided && (c2 < 0 || c2 == r || better(c2))) c2 = k;
    }
  // 1-byte elements whose column mode has source stride 2, every other source stride even, the
  // source pointer 2-byte aligned: the source is read as 2-byte pairs (a dense 2-byte transpose
  // of the pairs, on its tall tiles) and one byte of each pair is stored: the low byte where the
  // source offset is even, the high byte where it is odd.  Only bytes between the copy's first
  // and last source byte are read: with low bytes kept a pair ends before its row's next element
  // and the pair holding a row's last element is read as that one byte; with high bytes kept a
  // pair starts after the row's previous element and the pair holding a row's first element is
  // read as that one byte (the tiles holding them take the guarded code).
  // The same for a column-mode source stride of 4 with every source stride and the source offset
  // multiples of 4, for 1-, 2- and 4-byte elements: the source is read in groups of 4 elements (a
  // dense transpose of 4-, 8- or 16-byte groups) and each group's first element is stored; the
  // group holding a row's last element is read as that one element.  (A stride-4 mode of 4-byte
  // elements is no candidate above, its elements lying 16 bytes apart: it is looked for here.)
  int cg = c2;
  if ((cg < 0 || cg == r) && c < 0 && p.eb == 4)
    for (int k = 0; k < j.rank; ++k)
      if (k != r && j.m[k].s == 4) cg = k;
  const int64_t gs = cg >= 0 && cg != r ? j.m[cg].s : 0;
  // 2-, 4- and 8-byte elements of a stride-2 source at an even offset are read as 4-, 8- and
  // 16-byte pairs the same way.
  if (!forced_guarded && r >= 0 && ((gs == 2 && (p.eb == 1 || (p.eb >= 2 && p.eb <= 8 && j.so % 2 == 0))) || (gs == 4 && p.eb <= 4)) &&
      ptr_align >= std::min<int64_t>(16, gs * p.eb) && j.m[r].e >= 512 && j.m[cg].e >= 64) {
    bool even = true;
    for (int k = 0; k < j.rank; ++k) even = even && j.m[k].s % gs == 0;
    if (gs == 4) even = even && j.so % 4 == 0;
    if (even) {
      const int sel = gs == 4 ? 3 : j.so % 2 == 0 ? 1 : 2;  // (offsets may be negative: so % 2 is then -1)
      Plan q = p;
      q.eb = int(gs) * p.eb;
      q.nar = sel;
      q.vb = 16;
      q.unaligned = true;
      q.step = 1;
      q.j.so = (sel == 2 ? j.so - 1 : j.so) / gs;  // the pair or group holding the first element (exact)
      for (int k = 0; k < j.rank; ++k) q.j.m[k].s = j.m[k].s / gs;
      q.path = TC_PATH_TRANSPOSE;
      q.mode_r = r;
      q.mode_c = cg;
      int b = -1;
      for (int k = 0; k < j.rank; ++k) {
        if (k == r || k == cg) continue;
        if (b < 0 || std::llabs(j.m[k].s) + std::llabs(j.m[k].d) < std::llabs(j.m[b].s) + std::llabs(j.m[b].d)) b = k;
      }
      q.mode_b = b;
      if (plan_transpose_tile(&q, flags & ~TC_FLAG_STRICT)) {
        p.path = TC_PATH_TRANSPOSE;
        p.nar = sel;
        p.g = q.g;
        p.wconf = q.wconf;
        p.rconf = q.rconf;
        p.vb = 16;
        p.unaligned = true;
        p.step = int(gs);
        p.mode_r = r;
        p.mode_c = cg;
        p.mode_b = b;
        p.threads = p.g.NT;
        p.load_outer = p.g.loads;
        p.store_outer = p.g.stores;
        p.lds_bytes = p.g.tile_bytes;
        p.workgroups = transpose_workgroups(p, r, cg, b);
        if (p.workgroups >= (int64_t(1) << 31)) {
          p.status = TC_E_RANGE;
          p.reason = "more than 2^31 workgroups";
        }
        return p;
      }
    }
  }
  if (!forced_guarded && r >= 0 && c2 >= 0 && r != c2) {
    c = c2;
    p.vb = 16;
    p.unaligned = true;
    p.step = int(j.m[c].s);
    p.path = TC_PATH_TRANSPOSE;
    p.mode_r = r;
    p.mode_c = c;
    int b = -1;
    for (int k = 0; k < j.rank; ++k) {
      if (k == r || k == c) continue;
      if (b < 0 || std::llabs(j.m[k].s) + std::llabs(j.m[k].d) < std::llabs(j.m[b].s) + std::llabs(j.m[b].d)) b = k;
    }
    p.mode_b = b;
    const std::string reason = p.reason;
    const bool declined = p.declined;
    if (plan_transpose_tile(&p, flags & ~TC_FLAG_STRICT)) {
      p.reason = reason;
      p.declined = declined;
      p.threads = p.g.NT;
      p.load_outer = p.g.loads;
      p.store_outer = p.g.stores;
      p.lds_bytes = p.g.tile_bytes;
      p.workgroups = transpose_workgroups(p, r, c, b);
      if (p.workgroups >= (int64_t(1) << 31)) {
        p.status = TC_E_RANGE;
        p.reason = "more than 2^31 workgroups";
      }
      return p;
    }
    p.unaligned = false;
    p.step = 1;
    p.reason = reason;
    p.declined = declined;
  }

  // Declined (or left narrower vectors) by the aligned rule, with both sides contiguous along the
  // same mode: rows of 16-byte vectors at element alignment (gfx950 global memory takes unaligned
  // vector accesses), a row's short last vector in at most four accesses.  Window copies of a
  // matrix at any offset, and copies at odd element offsets, run here instead of element-wise:
  // the 8190^2 window of an 8192^2 matrix, int8 1.01 -> 4.5 TB/s, fp16 2.04 -> 5.4, fp32 4.5 ->
  // 6.0, fp64 5.6 -> 6.3; an int8 copy at an odd offset 1.10 -> 5.8.
  // The same rows where the source steps 2, 3 or 4 elements along them, or -1 to -4 (in reverse
  // order), and has no unit-stride mode (a strided slice written out densely, e.g. every other
  // column of a matrix; a flipped row): each destination vector is gathered from the source bytes
  // between its first and last element (16-byte loads) and compacted in registers; 1- to 8-byte
  // elements.
  const int64_t gstep = r >= 0 ? j.m[r].s : 0;
  const bool gather = c_unit < 0 && p.eb <= 8 && gstep != 0 && gstep != 1 && gstep >= -4 && gstep <= 4;
  if (!forced_guarded && r >= 0 && (r == c || gather) && r == j.rank - 1 && p.eb < 16) {
    const int64_t ve = 16 / p.eb;
    const int64_t rows = j.count / j.m[r].e;
    const int64_t nvec = rows * ceil_div(j.m[r].e, ve);
    p.path = TC_PATH_ROWS;
    p.vb = 16;
    p.unaligned = true;
    p.step = gather ? int(gstep) : 1;
    p.ntm = 3;
    p.threads = kRowThreads;
    {
      const TuneCfg tc = tune_override();
      p.buffers = !gather && tc.buf != 0;
      // one vector per lane for gathered rows (measured against 4 on 8192-row copies: int8 every
      // 2nd / 3rd / 4th column 3.36 -> 3.59, 2.36 -> 2.58, 1.93 -> 2.09 TB/s, fp32 every 4th
      // 2.16 -> 2.41, fp16 / fp32 / fp64 every 2nd +3%, the 8190 x 4095 int8 slice 3.21 -> 3.52,
      // rows flipped: int8 5.28 -> 5.59, fp16 5.69 -> 5.9), except rows flipped with 4- and 8-byte
      // elements (one load per vector), which keep 4 (fp32 6.26 against 5.91-5.99, fp64 6.35
      // against 5.79-5.83)
      p.row_rounds = gather && !(gstep == -1 && p.eb >= 4) ? 1 : kRowRounds;
      if (!gather && (tc.rr == 1 || tc.rr == 2 || tc.rr == 4)) p.row_rounds = tc.rr;
    }
    p.workgroups = ceil_div(nvec, int64_t(kRowThreads) * p.row_rounds);
    p.load_outer = p.store_outer = int(std::min<int64_t>(p.row_rounds, ceil_div(nvec, p.threads)));
    if (!rows_fit(j, nvec)) {
      p.status = TC_E_RANGE;
      p.reason = "more than 2^30 vectors per index of the outermost mode";
    }
    return p;
  }

  // Guarded fallback: an LDS tile over the two modes with the smallest strides on each side
  // (element-wide accesses), or an element-wise copy in destination order.
  p.vb = p.eb;
  int gr = -1, gc = -1;
  for (int k = 0; k < j.rank; ++k)
    if (j.m[k].d != 0 && (gr < 0 || std::llabs(j.m[k].d) < std::llabs(j.m[gr].d))) gr = k;
  for (int k = 0; k < j.rank; ++k)
    if (k != gr && (gc < 0 || std::llabs(j.m[k].s) < std::llabs(j.m[gc].s))) gc = k;
  const bool tile = gr >= 0 && gc >= 0 && std::llabs(j.m[gc].s) < std::llabs(j.m[gr].s);
  if (tile) {
    p.path = TC_PATH_GUARDED_TILE;
    p.mode_r = gr;
    p.mode_c = gc;
    p.g = TileGeom();
    p.g.eb = p.eb;
    p.g.vb = p.eb;
    p.g.TR = p.eb <= 4 ? 64 : 32;
    p.g.TC = p.eb <= 4 ? 64 : (p.eb == 8 ? 64 : 32);
    p.g.NB = 1;
    p.threads = kGuardThreads;
    p.load_outer = p.store_outer = p.g.TR * p.g.TC / kGuardThreads;
    const int pad = std::max(1, 4 / p.eb);
    p.lds_bytes = p.g.TR * (p.g.TC + pad) * p.eb;
    p.workgroups = ceil_div(j.m[gr].e, p.g.TR) * ceil_div(j.m[gc].e, p.g.TC);
    for (int k = 0; k < j.rank; ++k)
      if (k != gr && k != gc) p.workgroups *= j.m[k].e;
    if (p.workgroups >= (int64_t(1) << 31)) { p.status = TC_E_RANGE; p.reason = "more than 2^31 workgroups"; }
  } else {
    p.path = TC_PATH_GUARDED_ROWS;
    p.threads = kGuardThreads;
    p.load_outer = p.store_outer = kRowRounds;
    p.workgroups = ceil_div(j.count, int64_t(kGuardThreads) * kRowRounds);
    if (!rows_fit(j, j.count)) {
      p.status = TC_E_RANGE;
      p.reason = "more than 2^30 elements per index of the outermost mode on the guarded path";
    }
  }
  return p;
}

// The same copy on other kernel configurations, for tc_autotune: the plan itself first, then, for
// a transpose (not the pair-reading one), the conflict-free tiles of a fixed list of
// configurations the library holds kernels for (tall 16-byte-unit tiles of 32-128 KiB in both
// row-tile-first and XCD super-tile orders, the width's default tile in both plain orders, loads
// capped at 2 for 1- and 2-byte elements; for element-aligned plans, their small tiles in three
// orders), and for the aligned 16-byte rows path its vectors per lane (1, 2, 4) with and without
// buffer accesses.  Duplicates are dropped.  No configuration is better everywhere: measured on
// MI355X, the best fp32 tile of 0.25-1 GiB transposes changed with the extents in no pattern the
// planner's rules capture.
std::vector<Plan> plan_variants(const Plan& p, int flags) {
  std::vector<Plan> out{p};
  if (p.status != TC_OK || (flags & TC_FLAG_NO_SWIZZLE)) return out;  // (a measurement of the plan's tile)
  const Joint& j = p.j;
  if (p.path == TC_PATH_TRANSPOSE && !p.nar) {
    const int unit0 = p.eb < 4 ? 4 : p.eb;
    std::vector<TuneCfg> cands;
    auto add = [&](int tile, int threads, int trb, int unit, int nt, int order, int cap, int ssr, int ssc) {
      TuneCfg t;
      t.tile = tile; t.threads = threads; t.trb = trb; t.unit = unit; t.nt = nt; t.order = order; t.cap = cap;
      t.ssr = ssr; t.ssc = ssc;
      cands.push_back(t);
    };
    if (!p.unaligned && p.step == 1) {
      const int tall[][3] = {{65536, 512, 1024}, {32768, 512, 512}, {32768, 512, 1024}, {32768, 256, 512},
                             {65536, 512, 2048}, {131072, 1024, 1024}, {131072, 1024, 2048}, {131072, 512, 512}};
      for (const auto& t : tall) {
        add(t[0], t[1], t[2], 16, 3, 1, 0, 0, 0);
        add(t[0], t[1], t[2], 16, 3, 2, 0, 4, 4);
        if (p.eb <= 2) add(t[0], t[1], t[2], 16, 3, 1, 2, 0, 0);
      }
      add(65536, 512, 1024, 16, 3, 2, 0, 2, 8);
      add(65536, 512, 1024, 16, 3, 2, 0, 8, 2);
      if (p.eb == 1) add(131072, 512, 512, 16, 3, 2, 2, 16, 2);
      const TuneCfg d = default_cfg(p.eb, pow2ceil(j.m[p.mode_r].e) * p.eb < 128, false);
      add(d.tile, d.threads, 0, unit0, 3, 0, 0, 0, 0);
      add(d.tile, d.threads, 0, unit0, 3, 1, 0, 0, 0);
    } else {
      const int small[][2] = {{8192, 256}, {16384, 256}, {16384, 512}};
      for (const auto& t : small)
        for (int order = 0; order <= 2; ++order) add(t[0], t[1], 0, unit0, 0, order, 0, 0, 0);
      if (p.step == 1) {  // the tall tiles of the destination-misaligned 1- and 2-byte plans
        add(65536, 512, 1024, 16, 0, 2, 0, 0, 0);
        add(65536, 512, 1024, 16, 3, 2, 2, 0, 0);
        add(131072, 512, 512, 16, 3, 2, 2, 16, 2);
        add(131072, 512, 512, 16, 0, 2, 2, 16, 2);
      }
    }
    bool src_lines = (j.so * p.eb) % 128 == 0;
    for (int k = 0; k < j.rank; ++k)
      if (k != p.mode_c && (std::llabs(j.m[k].s) * p.eb) % 128 != 0) src_lines = false;
    const int64_t eB = p.mode_b >= 0 ? j.m[p.mode_b].e : 1;
    for (const TuneCfg& t : cands) {
      TileGeom g;
      int64_t wc, rc;
      if (!plan_with_cfg(p, flags & ~TC_FLAG_NO_SWIZZLE, t, true, &g, &wc, &rc) || wc + rc != 0) continue;
      g.pad_rows = g.order == 1 && !src_lines;
      g.wave_local = false;
      g.edges = j.m[p.mode_r].e % g.TR != 0 || j.m[p.mode_c].e % g.TC != 0 || eB % g.NB != 0 || g.step != 1 ||
                p.eb == 16 || p.unaligned;
      // (the interior-only kernels exist for the nontemporal configurations only)
      if (!g.edges && !launch_transpose(g.eb, transpose_cfg(g), nullptr, 0, nullptr)) g.edges = true;
      if (!launch_transpose(g.eb, transpose_cfg(g), nullptr, 0, nullptr)) continue;
      Plan q = p;
      q.g = g;
      q.wconf = wc;
      q.rconf = rc;
      q.threads = g.NT;
      q.load_outer = g.loads;
      q.store_outer = g.stores;
      q.lds_bytes = g.tile_bytes;
      q.workgroups = transpose_workgroups(q, q.mode_r, q.mode_c, q.mode_b);
      if (q.workgroups >= (int64_t(1) << 31)) continue;
      bool dup = false;
      for (const Plan& o : out) {
        const TileGeom& h = o.g;
        dup = dup || (h.TR == g.TR && h.TC == g.TC && h.NB == g.NB && h.NT == g.NT && h.U == g.U &&
                      h.tile_bytes == g.tile_bytes && h.ntm == g.ntm && h.order == g.order && h.cap == g.cap &&
                      h.edges == g.edges && h.wave_local == g.wave_local &&
                      (g.order != 2 || (h.lsr == g.lsr && h.lsc == g.lsc)));
      }
      if (!dup) out.push_back(q);
    }
  } else if (p.path == TC_PATH_ROWS && p.unaligned && p.step == 1) {
    // element-aligned rows: 1, 2 or 4 vectors per lane (measured 2-4% apart either way on 64 MiB
    // int8 copies at odd offsets, in no pattern)
    const int64_t rows = j.count / j.m[j.rank - 1].e;
    const int64_t nvec = rows * ceil_div(j.m[j.rank - 1].e, int64_t(16 / p.eb));
    for (int rr : {1, 2, 4}) {
      if (rr == p.row_rounds) continue;
      Plan q = p;
      q.row_rounds = rr;
      q.workgroups = ceil_div(nvec, int64_t(q.threads) * rr);
      q.load_outer = q.store_outer = int(std::min<int64_t>(rr, ceil_div(nvec, q.threads)));
      out.push_back(q);
    }
  } else if (p.path == TC_PATH_ROWS && p.vb == 16 && !p.unaligned) {
    for (int rr : {1, 2, 4})
      for (int buf = 0; buf <= 1; ++buf) {
        Plan q = p;
        q.row_rounds = rr;
        q.buffers = buf != 0;
        q.row_burst = p.row_burst;
        const int64_t nvec = j.count / (p.vb / p.eb);
        q.workgroups = ceil_div(nvec, int64_t(q.threads) * rr);
        q.load_outer = q.store_outer = int(std::min<int64_t>(rr, ceil_div(nvec, q.threads)));
        if (rr == p.row_rounds && q.buffers == p.buffers) continue;
        if (!rows_fit(rows_grid(q), nvec)) continue;
        out.push_back(q);
      }
  }
  return out;
}

void plan_to_info(const Plan& p, tc_plan_info* info) {
  *info = tc_plan_info{};
  info->path = p.path;
  info->elem_bytes = p.eb;
  info->count = p.j.count;
  info->rank = p.j.rank;
  info->declined = p.declined ? 1 : 0;
  info->unaligned = p.unaligned ? 1 : 0;
  info->src_step = p.path == TC_PATH_TRANSPOSE ? p.step : p.path == TC_PATH_ROWS && p.step != 1 ? p.step : 0;
  info->wave_local = p.path == TC_PATH_TRANSPOSE && p.g.wave_local ? 1 : 0;
  for (int k = 0; k < p.j.rank; ++k) {
    info->extent[k] = p.j.m[k].e;
    info->src_stride[k] = p.j.m[k].s;
    info->dst_stride[k] = p.j.m[k].d;
  }
  info->src_offset = p.j.so;
  info->dst_offset = p.j.dof;
  info->threads = p.threads;
  info->vec_bytes = p.vb;
  info->load_outer = p.load_outer;
  info->store_outer = p.store_outer;
  info->mode_r = p.mode_r;
  info->mode_c = p.mode_c;
  info->mode_b = p.mode_b;
  const bool tiled = p.path == TC_PATH_TRANSPOSE || p.path == TC_PATH_GUARDED_TILE;
  info->tile_r = tiled ? p.g.TR : 0;
  info->tile_c = tiled ? p.g.TC : 0;
  info->tile_b = tiled ? p.g.NB : 0;
  info->workgroups = p.workgroups;
  info->lds_bytes = p.lds_bytes;
  if (p.path == TC_PATH_ROWS || p.path == TC_PATH_SHUFFLE) info->nontemporal = p.ntm;
  if (p.path == TC_PATH_ROWS) info->grid_order = p.row_src_order ? 1 : 0;
  if (p.path == TC_PATH_SHUFFLE) {
    info->tile_r = 4;
    info->tile_c = p.shuffle_c;
    info->tile_b = 1;
  }
  if (p.path == TC_PATH_INTERLEAVE) {
    info->nontemporal = p.ntm;
    info->tile_r = 16 / p.eb;  // pixels per lane and group
    info->tile_c = p.shuffle_c;  // channels
    info->tile_b = 1;
  }
  if (p.path == TC_PATH_TRANSPOSE) {
    info->xor_k = p.g.k;
    info->xor_shift = p.g.shift;
    info->xor_mask = (1 << p.g.k) - 1;
    info->xor_tbit = p.g.tbit;
    info->xor_cshift = p.g.cshift;
    info->xor_cmask = p.g.cmask;
    info->grid_order = p.g.order;
    info->nontemporal = p.g.ntm;
    info->lds_write_bytes = p.g.ww;
    info->lds_read_bytes = p.g.rw;
    info->edge_tiles = p.g.edges ? 1 : 0;
    info->loads_in_flight = p.g.cap;
    info->src_view_bytes = p.nar == 3 ? 4 * p.eb : p.nar ? 2 * p.eb : p.eb;
    info->super_rows = p.g.order == 2 ? 1 << p.g.lsr : 0;
    info->super_cols = p.g.order == 2 ? 1 << p.g.lsc : 0;
    info->write_conflicts = p.wconf;
    info->read_conflicts = p.rconf;
  }
  const size_t n = std::min(p.reason.size(), sizeof(info->reason) - 1);
  p.reason.copy(info->reason, n);
  info->reason[n] = 0;
}

}  // namespace tc
