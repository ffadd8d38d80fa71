// The LDS-tiled transpose kernel (gfx950, wave64): one tile of TILE bytes per workgroup of NT
// lanes, global -> registers -> LDS -> registers -> global.
//
// Load phase: the tile in source order, split [outer, threads, vec] with the TileLang default
// mapping (tutorial "loop_mapping.py": access_idx = flat // vec, thread = access_idx % threads,
// local_idx = (access_idx // threads) * vec + flat % vec), vectors of VB bytes along the
// source-contiguous mode, every load of a thread issued back to back.  Store phase: the same
// split of the tile in destination order, vectors of VB bytes along the destination-contiguous
// mode.  Between them the LDS exchange, whose XOR swizzle is chosen on the host by simulating
// gfx950's banks for both phases (TVM TIRx docs, "permute_layout", Algorithm step 2) and an
// s_barrier (TVM TIRx docs, "copy -> gmem_smem", demonstration program: cta_sync between the
// two copies).  Elements narrower than 4 bytes are grouped into 4-byte units in registers first
// (v_perm_b32 micro-transposes), so the LDS stage moves whole dwords.
#pragma once

#include "device_common.hpp"

namespace tc {
namespace dev {

// Geometry of the tile for element width EB, vector width VB, LDS unit U, tile bytes TILE and
// NT threads.  A unit is one column of B = U/EB consecutive rows.
template <int EB, int VB, int U, int TILE, int NT>
struct Geo {
  static constexpr int B = U / EB;               // rows per unit
  static constexpr int VE = VB / EB;             // elements per global vector
  static constexpr int LOADS = TILE / (NT * VB * B);
  static constexpr int STORES = TILE / (NT * VB);
  static constexpr int RPV = VB / U;             // units per store vector
  static constexpr int UB = VE * U;              // LDS bytes written per load access
  static constexpr int WW = UB < 16 ? UB : 16;   // LDS write instruction bytes
  static constexpr int CW = WW / U;              // units per write chunk
  static constexpr int LB = clog2(B), LVE = clog2(VE), LRPV = clog2(RPV), LCW = clog2(CW);
  static constexpr int VW = VB / 4;              // dwords per global vector
  static constexpr bool valid = U >= 4 && U >= EB && U <= VB && TILE % (NT * VB * B) == 0 &&
                                TILE / (NT * VB * B) >= 1 && TILE % (NT * VB) == 0;
};

template <typename G>
struct TileRegs {
  uint32_t w[G::LOADS][G::B][G::VW];
};

// Load phase of one tile: global -> registers.  GUARD (tile reaches past an extent): only
// positions inside the copy are loaded; the registers of the others are never stored.  S: source
// stride of the column mode (1, or 2: each vector is read as two contiguous ones, which stay
// inside the allocation as long as the row's next element exists; the vector holding a row's
// last element is loaded element by element).
//
// NAR (EB = 2): the elements are 2-byte pairs of a 1-byte stride-2 source, of which the store
// phase keeps the low (NAR = 1) or high (NAR = 2) bytes (EB = 4 or 16, NAR = 1: 4- or 16-byte
// pairs of a 2- or 8-byte stride-2 source, the low halves kept); NAR = 3 (EB = 4, 8, 16): groups of 4
// elements of a stride-4 source of 1-, 2- or 4-byte elements, the low EB/4 bytes of each kept.  A pair must not be read whole where its
// other byte lies past the row's last element (1) or before its first (2): guarded tiles read the
// vector holding it with gload_pairs_last / gload_pairs_first, and tiles holding a row's last (1)
// or first (2) element always take the guarded code (see transpose_kernel).
template <int EB, int VB, typename G, int NT, int NTM, int S, bool GUARD, int CAP = 0, int NAR = 0>
__device__ __forceinline__ void load_tile(const TransposeArgs& a, const TileAt& t, TileRegs<G>& r) {
  const int lTRu = a.lTR - G::LB;
  const int lnCV = a.lTC - G::LVE;  // load vectors per unit-row
  const int TRu = 1 << lTRu, NB = 1 << a.lNB;
  const int64_t sR = a.sR;
#pragma unroll
  for (int f = 0; f < G::LOADS; ++f) {
    const int acc = f * NT + threadIdx.x;
    const int cv = acc & ((1 << lnCV) - 1);
    const int ru = (acc >> lnCV) & (TRu - 1);
    const int nb = acc >> (lnCV + lTRu);
    const int64_t off = t.sbase + nb * a.sB + (int64_t(ru) << G::LB) * sR + (cv << G::LVE) * S;
    const unsigned char* p = a.src + off * EB;
    if constexpr (GUARD) {
      // whole vectors inside the copy load as one access (alignment is only the element's:
      // gfx950 global memory takes unaligned 16-byte accesses); vectors reaching past the
      // column extent load their valid elements one by one; the rest are not loaded (their
      // LDS contents are never stored)
      const bool in_b = nb < NB && nb < t.remB;
      const int64_t cols = t.remC - (int64_t(cv) << G::LVE);
      const bool first = NAR == 2 && cv == 0 && t.remC == a.eC;
#pragma unroll
      for (int i = 0; i < G::B; ++i) {
        const bool in_row = in_b && (int64_t(ru) << G::LB) + i < t.remR && cols > 0;
        const bool whole = S == 1 && NAR != 1 && NAR != 3 ? cols >= G::VE : cols > G::VE;
        const int n = int(cols < G::VE ? cols : G::VE);
        // NAR = 2: the row's first vector (the first one of the first column tile) is read from
        // its first kept byte on, and moved up one byte below (pairs_up_one_byte)
        const unsigned char* q = p + i * sR * EB + (first ? 1 : 0);
        if (in_row && whole) {
          gload_step<EB, VB, S, NTM>(q, r.w[f][i]);
        } else if (in_row) {
          if constexpr (NAR == 1) gload_pairs_last<EB, EB / 2>(q, n, r.w[f][i]);
          else if constexpr (NAR == 3) gload_pairs_last<EB, EB / 4>(q, n, r.w[f][i]);
          else gload_partial<EB, VB, S>(q, n, r.w[f][i]);
        }
      }
      if constexpr (NAR == 2)
        if (first)
#pragma unroll
          for (int i = 0; i < G::B; ++i) pairs_up_one_byte(r.w[f][i]);
    } else {
#pragma unroll
      for (int i = 0; i < G::B; ++i) {
        gload_step<EB, VB, S, NTM>(p + i * sR * EB, r.w[f][i]);
        if constexpr (CAP > 0)
          if (f * G::B + i >= CAP) wait_vmem_at_most<CAP>();
      }
    }
  }
}

// Registers -> LDS: the VE units (columns) of each access, U/4 dwords each, into swizzled chunks.
// Unit j, dword m holds rows m*4/EB .. of column j (EB < 4: packed with v_perm_b32) or part
// m % (EB/4) of row m / (EB/4) (EB >= 4: a plain register regrouping).
template <int EB, int VB, int U, typename G, int NT>
__device__ __forceinline__ void write_lds(const TransposeArgs& a, unsigned char* __restrict__ lds,
                                          const TileRegs<G>& r) {
  constexpr int UW = U / 4;  // dwords per unit
  const int lTRu = a.lTR - G::LB;
  const int lnCV = a.lTC - G::LVE;
  const int TRu = 1 << lTRu;
  const int xmask = a.xmask, xshift = a.xshift, xtbit = a.xtbit, xcshift = a.xcshift, xcmask = a.xcmask;
#pragma unroll
  for (int f = 0; f < G::LOADS; ++f) {
    const int acc = f * NT + threadIdx.x;
    const int cv = acc & ((1 << lnCV) - 1);
    const int ru = (acc >> lnCV) & (TRu - 1);
    const int nb = acc >> (lnCV + lTRu);
    const int xr = ((ru >> xshift) & xmask) << xtbit;
    const int row = (nb << lTRu) + ru;
    if constexpr (EB >= 4) {
      // each write chunk straight from the loaded rows (a staging array here was kept in scratch)
      constexpr int DPE = EB / 4;  // dwords per element
#pragma unroll
      for (int q = 0; q < G::UB / G::WW; ++q) {
        uint32_t chunk[G::WW / 4];
#pragma unroll
        for (int uu = 0; uu < G::CW; ++uu)
#pragma unroll
          for (int m = 0; m < UW; ++m) chunk[uu * UW + m] = r.w[f][m / DPE][(q * G::CW + uu) * DPE + m % DPE];
        const int ch = ((cv << G::LVE) >> G::LCW) + q;
        const int chs = ch ^ xr ^ ((ch >> xcshift) & xcmask);
        store_words<G::WW>(lds + ((row << a.lTC) + (chs << G::LCW)) * U, chunk);
      }
      continue;
    }
    uint32_t unit[G::UB / 4];
    if constexpr (EB == 2) {
#pragma unroll
      for (int m = 0; m < UW; ++m)
#pragma unroll
        for (int d = 0; d < VB / 4; ++d) {
          unit[(2 * d) * UW + m] = perm(r.w[f][2 * m + 1][d], r.w[f][2 * m][d], 0x05040100u);
          unit[(2 * d + 1) * UW + m] = perm(r.w[f][2 * m + 1][d], r.w[f][2 * m][d], 0x07060302u);
        }
    } else {
#pragma unroll
      for (int m = 0; m < UW; ++m)
#pragma unroll
        for (int d = 0; d < VB / 4; ++d) {
          const uint32_t p01 = perm(r.w[f][4 * m + 1][d], r.w[f][4 * m][d], 0x05010400u);
          const uint32_t q01 = perm(r.w[f][4 * m + 1][d], r.w[f][4 * m][d], 0x07030602u);
          const uint32_t p23 = perm(r.w[f][4 * m + 3][d], r.w[f][4 * m + 2][d], 0x05010400u);
          const uint32_t q23 = perm(r.w[f][4 * m + 3][d], r.w[f][4 * m + 2][d], 0x07030602u);
          unit[(4 * d) * UW + m] = perm(p23, p01, 0x05040100u);
          unit[(4 * d + 1) * UW + m] = perm(p23, p01, 0x07060302u);
          unit[(4 * d + 2) * UW + m] = perm(q23, q01, 0x05040100u);
          unit[(4 * d + 3) * UW + m] = perm(q23, q01, 0x07060302u);
        }
    }
#pragma unroll
    for (int q = 0; q < G::UB / G::WW; ++q) {
      const int ch = ((cv << G::LVE) >> G::LCW) + q;
      const int chs = ch ^ xr ^ ((ch >> xcshift) & xcmask);
      store_words<G::WW>(lds + ((row << a.lTC) + (chs << G::LCW)) * U, unit + q * (G::WW / 4));
    }
  }
}

// LDS -> registers (all reads first), then registers -> global.  GUARD skips stores of
// positions outside the copy.  NAR: each 16-byte vector of 2-byte pairs is stored as its 8 low
// (1) or high (2) bytes, or of groups of 4 elements (3) as the 4 bytes of the groups' first
// elements, the destination addressed in its own elements (1 byte for pairs, EB/4 for groups).
template <int EB, int VB, int U, typename G, int NT, int NTM, bool GUARD, int NAR = 0>
__device__ __forceinline__ void read_store(const TransposeArgs& a, const TileAt& t,
                                           const unsigned char* __restrict__ lds) {
  const int lTRu = a.lTR - G::LB;
  const int lnRV = lTRu - G::LRPV;  // store vectors per column
  const int TC = 1 << a.lTC, NB = 1 << a.lNB;
  const int xmask = a.xmask, xshift = a.xshift, xtbit = a.xtbit, xcshift = a.xcshift, xcmask = a.xcmask;
  uint32_t out[G::STORES][VB / 4];
#pragma unroll
  for (int f = 0; f < G::STORES; ++f) {
    const int acc = f * NT + threadIdx.x;
    const int rv = acc & ((1 << lnRV) - 1);
    const int c = (acc >> lnRV) & (TC - 1);
    const int nb = acc >> (lnRV + a.lTC);
    const int ch = c >> G::LCW, cin = c & (G::CW - 1);
#pragma unroll
    for (int v = 0; v < G::RPV; ++v) {
      const int ru = (rv << G::LRPV) + v;
      const int xr = ((ru >> xshift) & xmask) << xtbit;
      const int chs = ch ^ xr ^ ((ch >> xcshift) & xcmask);
      load_words<U>(lds + ((((nb << lTRu) + ru) << a.lTC) + (chs << G::LCW) + cin) * U, out[f] + v * (U / 4));
    }
  }
#pragma unroll
  for (int f = 0; f < G::STORES; ++f) {
    const int acc = f * NT + threadIdx.x;
    const int rv = acc & ((1 << lnRV) - 1);
    const int c = (acc >> lnRV) & (TC - 1);
    const int nb = acc >> (lnRV + a.lTC);
    if constexpr (NAR && EB >= 8) {
      // only part of each 16-byte unit is stored: the compiler would narrow the LDS read to those
      // bytes (8 or 4 at a 16-byte stride, which conflict in the banks); the empty statement keeps
      // every word read, so the read stays the conflict-free 16-byte access the swizzle is chosen for
      asm volatile("" : : "v"(out[f][0]), "v"(out[f][1]), "v"(out[f][2]), "v"(out[f][3]));
    }
    if constexpr (NAR == 3) {
      static_assert((EB == 4 || EB == 8 || EB == 16) && VB == 16, "groups of 4 elements in 16-byte vectors");
      constexpr int KB = EB / 4;  // bytes kept per group
      unsigned char* p =
          a.dst + (t.dbase + nb * a.dB + int64_t(c) * a.dC + (int64_t(rv) << (G::LRPV + G::LB))) * KB;
      // the groups' first elements, packed: byte 0 of words 0-3, bytes 0-1 of words 0 and 2, or
      // word 0 (0x0c: a zero byte)
      uint32_t lo;
      if constexpr (EB == 4) lo = perm(out[f][1], out[f][0], 0x0c0c0400u) | perm(out[f][3], out[f][2], 0x04000c0cu);
      else if constexpr (EB == 8) lo = perm(out[f][2], out[f][0], 0x05040100u);
      else lo = out[f][0];
      if constexpr (GUARD) {
        const int64_t rows = t.remR - (int64_t(rv) << (G::LRPV + G::LB));
        const bool ok = nb < NB && nb < t.remB && c < t.remC && rows > 0;
        if (ok && rows >= G::VE) gstore<4, NTM>(p, &lo);
        else if (ok) gstore_partial<KB, 4>(p, int(rows), &lo);
      } else {
        gstore<4, NTM>(p, &lo);
      }
      continue;
    } else if constexpr (NAR) {
      static_assert((EB == 2 || (EB >= 4 && NAR == 1)) && VB == 16,
                    "pairs of 1-, 2-, 4- or 8-byte elements in 16-byte vectors");
      constexpr int KB = EB / 2;  // bytes kept per pair
      unsigned char* p =
          a.dst + (t.dbase + nb * a.dB + int64_t(c) * a.dC + (int64_t(rv) << (G::LRPV + G::LB))) * KB;
      constexpr uint32_t kSel = NAR == 1 ? 0x06040200u : 0x07050301u;  // bytes 0, 2 or 1, 3 of each word
      uint32_t lo[2];
      if constexpr (EB == 2) {
        lo[0] = perm(out[f][1], out[f][0], kSel);
        lo[1] = perm(out[f][3], out[f][2], kSel);
      } else if constexpr (EB == 4) {  // the low 2 bytes of each word
        lo[0] = perm(out[f][1], out[f][0], 0x05040100u);
        lo[1] = perm(out[f][3], out[f][2], 0x05040100u);
      } else if constexpr (EB == 8) {  // the low word of each pair
        lo[0] = out[f][0];
        lo[1] = out[f][2];
      } else {  // one pair of 8-byte elements: its low half
        lo[0] = out[f][0];
        lo[1] = out[f][1];
      }
      if constexpr (GUARD) {
        const int64_t rows = t.remR - (int64_t(rv) << (G::LRPV + G::LB));
        const bool ok = nb < NB && nb < t.remB && c < t.remC && rows > 0;
        if (ok && rows >= G::VE) gstore<8, NTM>(p, lo);
        else if (ok) gstore_partial<KB, 8>(p, int(rows), lo);
      } else {
        gstore<8, NTM>(p, lo);
      }
      continue;
    }
    unsigned char* p = a.dst + (t.dbase + nb * a.dB + int64_t(c) * a.dC + (int64_t(rv) << (G::LRPV + G::LB))) * EB;
    if constexpr (GUARD) {
      // whole vectors as one store, vectors reaching past the row extent element by element
      const int64_t rows = t.remR - (int64_t(rv) << (G::LRPV + G::LB));
      const bool ok = nb < NB && nb < t.remB && c < t.remC && rows > 0;
      if (ok && rows >= G::VE) gstore<VB, NTM>(p, out[f]);
      else if (ok) gstore_partial<EB, VB>(p, int(rows), out[f]);
    } else {
      gstore<VB, NTM>(p, out[f]);
    }
  }
}

// One tile per workgroup.  Interior tiles (the common case) take the unguarded path, which has
// no per-lane conditions at all; tiles at the edges of the copy take the guarded one (with S = 2
// also the tiles holding a row's last element).  WL: the planner has shown that every wave reads
// back only LDS units it wrote itself, so the phases are ordered per wave and the waves of the
// workgroup never wait for each other.
//
// EDGE = false: the host has shown that every tile lies wholly inside the copy, and the guarded
// code is not compiled in (it needs more registers than the interior code, which can then
// lower the number of workgroups per CU).
//
// CAP > 0: the interior load phase keeps at most CAP loads of a lane outstanding (measured faster
// than all at once for the tall tiles of 1- and 2-byte elements).
//
// NAR: 2-byte pairs of a 1-byte stride-2 source, the low (1) or high (2) bytes stored
// (load_tile, read_store).
template <int EB, int VB, int U, int TILE, int NT, int NTM, int S, bool WL, bool EDGE = true, int CAP = 0,
          int NAR = 0>
__global__ void __launch_bounds__(NT) transpose_kernel(TransposeArgs a) {
  typedef Geo<EB, VB, U, TILE, NT> G;
  __shared__ __attribute__((aligned(16))) unsigned char lds[TILE];
  const TileAt t = tile_at(a, blockIdx.x);
  if (!t.valid) return;  // padding of the XCD super-tile order (whole workgroup, before any barrier)
  TileRegs<G> r;
  // (tiles holding a row's last element: guarded for S = 2 and NAR = 1, 3; its first: for NAR = 2)
  const bool full = !EDGE || (tile_full(a, t) && ((S == 1 && NAR != 1 && NAR != 3) || t.remC > (int64_t(1) << a.lTC)) &&
                              (NAR != 2 || t.remC < a.eC));
  if constexpr (!EDGE) load_tile<EB, VB, G, NT, NTM, S, false, CAP, NAR>(a, t, r);
  else if (full) load_tile<EB, VB, G, NT, NTM, S, false, CAP, NAR>(a, t, r);
  else load_tile<EB, VB, G, NT, NTM, S, true, 0, NAR>(a, t, r);
  write_lds<EB, VB, U, G, NT>(a, lds, r);
  if constexpr (WL) wave_lds_sync();
  else __syncthreads();
  if constexpr (!EDGE) read_store<EB, VB, U, G, NT, NTM, false, NAR>(a, t, lds);
  else if (full) read_store<EB, VB, U, G, NT, NTM, false, NAR>(a, t, lds);
  else read_store<EB, VB, U, G, NT, NTM, true, NAR>(a, t, lds);
}

// Launches the instance (ta != nullptr) or only reports whether it exists (ta == nullptr).
template <int EB, int VB, int U, int TILE, int NT, int NTM, int S, bool WL = false, bool EDGE = true, int CAP = 0,
          int NAR = 0>
bool launch_transpose_cfg(const TransposeArgs* ta, int64_t wgs, hipStream_t s) {
  // (source steps of magnitude 3 and 4 only where the elements lie at most 12 bytes apart, as
  // planned)
  constexpr int AS = S < 0 ? -S : S;
  if constexpr (Geo<EB, VB, U, TILE, NT>::valid && (AS <= 2 || EB * AS <= 12)) {
    if (ta)
      hipLaunchKernelGGL((transpose_kernel<EB, VB, U, TILE, NT, NTM, S, WL, EDGE, CAP, NAR>), dim3(uint32_t(wgs)), dim3(NT),
                         0, s, *ta);
    return true;
  }
  return false;
}

}  // namespace dev
}  // namespace tc

// Instantiation list of one element width: every (vector bytes, LDS unit, tile bytes, threads,
// nontemporal mode, source step, phase ordering, edge code) the planner can choose.  16- and
// 8-byte LDS units for the tall tiles; steps 2 to 4 and -1 to -4 (strided and reversed sources)
// only in the configurations of the element-aligned plans; wave-local ordering in the small batched tiles, where it occurs; the
// interior-only variants (EDGE = false) of the nontemporal configurations.
#define TC_TRANSPOSE_DISPATCH(EB)                                                                           \
  bool launch_transpose_eb##EB(const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream) {   \
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);                                             \
    const int vb = c.vb, tile = c.tile, nt = c.threads, ntm = c.ntm;                                         \
    constexpr int U = EB < 4 ? 4 : EB;                                                                       \
    if (c.nar) {                                                                                             \
      TC_NAR_EB##EB                                                                                          \
      return false;                                                                                          \
    }                                                                                                        \
    if (c.cap != 0) {                                                                                        \
      TC_CAPS_EB##EB                                                                                         \
      return false;                                                                                          \
    }                                                                                                        \
    if (c.unit == 16 && U != 16) {                                                                           \
      TC_CFG_UNIT(EB, 16, 16384, 256) TC_CFG_UNIT(EB, 16, 32768, 256) TC_CFG_UNIT(EB, 16, 65536, 256)         \
      TC_CFG_UNIT(EB, 16, 32768, 512) TC_CFG_UNIT(EB, 16, 65536, 512) TC_CFG_UNIT(EB, 16, 65536, 1024)       \
      TC_CFG_UNIT(EB, 16, 131072, 512) TC_CFG_UNIT(EB, 16, 131072, 1024)                                      \
      return false;                                                                                          \
    }                                                                                                        \
    if (c.unit == 8 && U < 8) {                                                                              \
      TC_CFG_UNIT(EB, 8, 16384, 256) TC_CFG_UNIT(EB, 8, 32768, 256) TC_CFG_UNIT(EB, 8, 65536, 256)            \
      TC_CFG_UNIT(EB, 8, 32768, 512) TC_CFG_UNIT(EB, 8, 65536, 512)                                          \
      return false;                                                                                          \
    }                                                                                                        \
    if (c.unit != U) return false;                                                                           \
    TC_CFG(EB, 16, U, 8192, 256) TC_CFG(EB, 16, U, 16384, 256) TC_CFG(EB, 16, U, 16384, 512)                  \
    TC_CFG(EB, 16, U, 32768, 256) TC_CFG(EB, 16, U, 32768, 512) TC_CFG(EB, 16, U, 65536, 256)                 \
    TC_CFG(EB, 16, U, 65536, 512)                                                                            \
    TC_CFG(EB, 8, U, 16384, 256) TC_CFG(EB, 4, U, 16384, 256)                                                \
    TC_CFG_STEP2(EB, U, 8192, 256) TC_CFG_STEP2(EB, U, 16384, 256) TC_CFG_STEP2(EB, U, 16384, 512)             \
    TC_CFG_WL(EB, U, 8192, 256) TC_CFG_WL(EB, U, 16384, 256)                                                 \
    return false;                                                                                            \
  }

#define TC_CFG(EB, VB, U, TILE, NT)                                                                          \
  if (vb == VB && tile == TILE && nt == NT && c.step == 1 && !c.wave_local) {                                \
    if (ntm == 3 && !c.edges) return dev::launch_transpose_cfg<EB, VB, U, TILE, NT, 3, 1, false, false>(ta, wgs, s);    \
    if (ntm == 3) return dev::launch_transpose_cfg<EB, VB, U, TILE, NT, 3, 1>(ta, wgs, s);                   \
    if (ntm == 0) return dev::launch_transpose_cfg<EB, VB, U, TILE, NT, 0, 1>(ta, wgs, s);                   \
  }

#define TC_CFG_STEP2(EB, U, TILE, NT)                                                                        \
  if (vb == 16 && tile == TILE && nt == NT && c.step != 1 && ntm == 0 && !c.wave_local) {                    \
    if (c.step == 2) return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 0, 2>(ta, wgs, s);                \
    if (c.step == 3) return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 0, 3>(ta, wgs, s);                \
    if (c.step == 4) return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 0, 4>(ta, wgs, s);                \
    if (c.step == -1) return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 0, -1>(ta, wgs, s);              \
    if (c.step == -2) return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 0, -2>(ta, wgs, s);              \
    if (c.step == -3) return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 0, -3>(ta, wgs, s);              \
    if (c.step == -4) return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 0, -4>(ta, wgs, s);              \
  }

// Wider LDS units (UNIT/EB rows of one column): tall tiles whose store lanes run down a column
#define TC_CFG_UNIT(EB, UNIT, TILE, NT)                                                                      \
  if (vb == 16 && tile == TILE && nt == NT && c.step == 1 && !c.wave_local) {                                \
    if (ntm == 3 && !c.edges) return dev::launch_transpose_cfg<EB, 16, UNIT, TILE, NT, 3, 1, false, false>(ta, wgs, s);    \
    if (ntm == 3) return dev::launch_transpose_cfg<EB, 16, UNIT, TILE, NT, 3, 1>(ta, wgs, s);                \
    if (ntm == 0) return dev::launch_transpose_cfg<EB, 16, UNIT, TILE, NT, 0, 1>(ta, wgs, s);                \
  }

// The tall configurations that run with a load cap (plan.cpp, tall_cfg): 16-byte LDS units,
// nontemporal accesses, with and without the edge code; and (TC_CFG_CAP_PLAIN) plain stores with
// the edge code, for destinations off the cache lines.
#define TC_CFG_CAP(EB, TILE, NT, CAP)                                                                        \
  if (c.cap == CAP && c.unit == 16 && vb == 16 && tile == TILE && nt == NT && c.step == 1 && !c.wave_local &&  \
      ntm == 3) {                                                                                            \
    if (!c.edges) return dev::launch_transpose_cfg<EB, 16, 16, TILE, NT, 3, 1, false, false, CAP>(ta, wgs, s);  \
    return dev::launch_transpose_cfg<EB, 16, 16, TILE, NT, 3, 1, false, true, CAP>(ta, wgs, s);               \
  }
#define TC_CFG_CAP_PLAIN(EB, TILE, NT, CAP)                                                                  \
  if (c.cap == CAP && c.unit == 16 && vb == 16 && tile == TILE && nt == NT && c.step == 1 && !c.wave_local &&  \
      ntm == 0)                                                                                              \
    return dev::launch_transpose_cfg<EB, 16, 16, TILE, NT, 0, 1, false, true, CAP>(ta, wgs, s);
#define TC_CAPS_EB1 TC_CFG_CAP(1, 131072, 512, 2) TC_CFG_CAP_PLAIN(1, 131072, 512, 2)
#define TC_CAPS_EB2 TC_CFG_CAP(2, 131072, 1024, 2) TC_CFG_CAP(2, 65536, 512, 2) TC_CFG_CAP(2, 32768, 256, 2)
#define TC_CAPS_EB4
#define TC_CAPS_EB8
#define TC_CAPS_EB16

// 2-byte pairs of a 1-byte stride-2 source, low or high bytes stored (plan.cpp, make_plan): the
// tall 512 x 64 tiles of 2-byte elements with nontemporal accesses and 2 loads in flight; 4-byte
// groups of 4 elements of a stride-4 source, the first element of each stored: 4-, 8- and
// 16-byte tiles of 1 KiB or 512 bytes by 32 groups; 16-byte pairs of an 8-byte stride-2 source:
// 64 x 8 tiles with every load in flight; 4- and 8-byte pairs of a 2- and 4-byte stride-2 source:
// the group tiles of that width.  Always with the edge
// code (the tiles holding a row's last element need it).
#define TC_CFG_NAR(EB, TILE, NT, CAP)                                                                        \
  if (c.cap == CAP && c.unit == 16 && vb == 16 && tile == TILE && nt == NT && c.step == 1 && !c.wave_local &&  \
      ntm == 3 && c.edges) {                                                                                 \
    if constexpr (EB != 1) {                                                                                 \
      if (c.nar == 1) return dev::launch_transpose_cfg<EB, 16, 16, TILE, NT, 3, 1, false, true, CAP, 1>(ta, wgs, s); \
    }                                                                                                        \
    if constexpr (EB == 2) {                                                                                 \
      if (c.nar == 2) return dev::launch_transpose_cfg<EB, 16, 16, TILE, NT, 3, 1, false, true, CAP, 2>(ta, wgs, s); \
    }                                                                                                        \
    if constexpr (EB >= 4) {                                                                                 \
      if (c.nar == 3) return dev::launch_transpose_cfg<EB, 16, 16, TILE, NT, 3, 1, false, true, CAP, 3>(ta, wgs, s); \
    }                                                                                                        \
  }
#define TC_NAR_EB1
#define TC_NAR_EB2 TC_CFG_NAR(2, 65536, 512, 2)
#define TC_NAR_EB4 TC_CFG_NAR(4, 32768, 512, 2)
#define TC_NAR_EB8 TC_CFG_NAR(8, 32768, 512, 2)
#define TC_NAR_EB16 TC_CFG_NAR(16, 16384, 256, 2) TC_CFG_NAR(16, 8192, 256, 0)

#define TC_CFG_WL(EB, U, TILE, NT)                                                                           \
  if (vb == 16 && tile == TILE && nt == NT && c.step == 1 && ntm == 3 && c.wave_local)                       \
    return dev::launch_transpose_cfg<EB, 16, U, TILE, NT, 3, 1, true>(ta, wgs, s);
