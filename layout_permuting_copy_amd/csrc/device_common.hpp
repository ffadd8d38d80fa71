// Device helpers shared by the tile-copy kernels (gfx950): raw word moves, global accesses with
// an optional nontemporal hint, buffer accesses with explicit cache-policy bits, byte permutes
// and 32-bit division by a runtime constant.
// All data moves as unsigned integers: floating point payloads are never touched.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.hpp"

namespace tc {
namespace dev {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int N>
struct Bytes;
template <>
struct Bytes<1> { typedef uint8_t T; };
template <>
struct Bytes<2> { typedef uint16_t T; };
template <>
struct Bytes<4> { typedef uint32_t T; };
template <>
struct Bytes<8> { typedef u32x2 T; };
template <>
struct Bytes<16> { typedef u32x4 T; };

constexpr int clog2(int x) { return x <= 1 ? 0 : 1 + clog2(x / 2); }

// N bytes (N = 4, 8, 16) between memory (LDS or global) and N/4 dwords.
template <int N>
__device__ __forceinline__ void load_words(const unsigned char* p, uint32_t* w) {
  if constexpr (N == 16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 8) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

template <int N>
__device__ __forceinline__ void store_words(unsigned char* p, const uint32_t* w) {
  if constexpr (N == 16) {
    *reinterpret_cast<u32x4*>(p) = u32x4{w[0], w[1], w[2], w[3]};
  } else if constexpr (N == 8) {
    *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
  } else {
    *reinterpret_cast<uint32_t*>(p) = w[0];
  }
}

// v_perm_b32: byte i of the result is byte sel.i of {hi:lo} (0-3 from lo, 4-7 from hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Global accesses of N bytes (N = 4, 8, 16).  NTM bit 0: nontemporal loads, bit 1: nontemporal
// stores (streaming data that is read or written once).
template <int N, int NTM>
__device__ __forceinline__ void gload(const unsigned char* p, uint32_t* w) {
  if constexpr (!(NTM & 1)) {
    load_words<N>(p, w);
  } else if constexpr (N == 16) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 8) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
}

template <int N, int NTM>
__device__ __forceinline__ void gstore(unsigned char* p, const uint32_t* w) {
  if constexpr (!(NTM & 2)) {
    store_words<N>(p, w);
  } else if constexpr (N == 16) {
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(p));
  } else if constexpr (N == 8) {
    __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(p));
  } else {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
  }
}

// Bytes at offset o of a VB-byte register vector w: `v` (b <= 4 bytes, o % b == 0) is or-ed in, or
// a word is read out from there, by masks rather than by indexing w with a run-time value (which
// would move w to scratch memory).
template <int VB>
__device__ __forceinline__ void put_bytes(uint32_t* w, int o, uint32_t v) {
  const uint32_t x = v << (8 * (o & 3));
  const int q = o >> 2;
#pragma unroll
  for (int k = 0; k < VB / 4; ++k) w[k] |= x & (0u - uint32_t(q == k));
}
template <int VB>
__device__ __forceinline__ uint32_t get_word(const uint32_t* w, int o) {
  const int q = o >> 2;
  uint32_t r = 0;
#pragma unroll
  for (int k = 0; k < VB / 4; ++k) r |= w[k] & (0u - uint32_t(q == k));
  return r >> (8 * (o & 3));
}

// The first n (0 < n < VB/EB) elements of a VB-byte vector whose elements lie S elements apart
// in memory (the vector reaches past an extent of the copy, or is the last of a strided row);
// the other bytes of w are zero.  S = 1: the n*EB bytes in at most four accesses of 8, 4, 2 and 1
// bytes, largest first (gfx950 global memory takes unaligned accesses); S = 2: one access per
// element.
template <int EB, int VB, int S = 1>
__device__ __forceinline__ void gload_partial(const unsigned char* p, int n, uint32_t* w) {
#pragma unroll
  for (int k = 0; k < VB / 4; ++k) w[k] = 0;
  if constexpr (S == 1 && EB < VB) {
    const int nb = n * EB;
    if constexpr (VB == 16) {
      if (nb & 8) {
        const uint64_t v = *reinterpret_cast<const uint64_t*>(p);
        w[0] = uint32_t(v);
        w[1] = uint32_t(v >> 32);
      }
    }
    if constexpr (VB >= 8 && EB <= 4)
      if (nb & 4) put_bytes<VB>(w, nb & 8, *reinterpret_cast<const uint32_t*>(p + (nb & 8)));
    if constexpr (EB <= 2)
      if (nb & 2) put_bytes<VB>(w, nb & 12, *reinterpret_cast<const uint16_t*>(p + (nb & 12)));
    if constexpr (EB == 1)
      if (nb & 1) put_bytes<VB>(w, nb & 14, p[nb & 14]);
    return;
  }
#pragma unroll
  for (int e = 0; e < VB / EB; ++e) {
    if (e < n) {
      const unsigned char* q = p + e * S * EB;
      if constexpr (EB >= 4) {
#pragma unroll
        for (int m = 0; m < EB / 4; ++m) w[e * (EB / 4) + m] = reinterpret_cast<const uint32_t*>(q)[m];
      } else if constexpr (EB == 2) {
        w[e / 2] |= uint32_t(*reinterpret_cast<const uint16_t*>(q)) << (16 * (e & 1));
      } else {
        w[e / 4] |= uint32_t(*q) << (8 * (e & 3));
      }
    }
  }
}

// The first n (0 < n <= 16/EB) EB-byte groups of a 16-byte vector read as groups of KB-byte
// elements (a stride-2 source of 1- or 8-byte elements read in 2- or 16-byte pairs, or a stride-4 source of 1-,
// 2- or 4-byte elements in 4-, 8- or 16-byte groups), when the vector holds its row's last
// element: the first n - 1 groups whole (in at most four accesses), then only the low KB bytes of
// the last group (that element), so that no byte past the row's last element is read; the other
// bytes of w are zero.
template <int EB, int KB = 1>
__device__ __forceinline__ void gload_pairs_last(const unsigned char* p, int n, uint32_t* w) {
  static_assert(KB == 1 || KB == 2 || KB == 4 || (KB == 8 && EB == 16), "1-, 2-, 4- or 8-byte elements");
  if constexpr (KB == 8) {  // one pair of 8-byte elements per vector (n == 1): its low element
    const uint64_t v = *reinterpret_cast<const uint64_t*>(p);
    w[0] = uint32_t(v);
    w[1] = uint32_t(v >> 32);
    w[2] = w[3] = 0;
    return;
  }
  gload_partial<EB, 16>(p, n - 1, w);  // (n - 1 == 0: nothing loaded, w zeroed)
  const unsigned char* q = p + EB * (n - 1);
  const uint32_t v = KB == 1 ? uint32_t(*q)
                     : KB == 2 ? uint32_t(*reinterpret_cast<const uint16_t*>(q))
                               : *reinterpret_cast<const uint32_t*>(q);
  put_bytes<16>(w, EB * (n - 1), v);
}

// A vector holding its row's first element when the high bytes of the pairs are kept is read
// from that element on (16 bytes, ending before the row's ninth element, so inside the copy
// for rows of more than 8 elements; nothing before the row's first element is read) and then
// moved up one byte here, so that the kept bytes sit in the high bytes of the pairs.
__device__ __forceinline__ void pairs_up_one_byte(uint32_t* w) {
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
  w[0] = w0 << 8;
  w[1] = __builtin_amdgcn_alignbyte(w1, w0, 3);
  w[2] = __builtin_amdgcn_alignbyte(w2, w1, 3);
  w[3] = __builtin_amdgcn_alignbyte(w3, w2, 3);
}

// A 16-byte vector of 16/EB elements gathered from a source that steps K elements between them
// (a strided slice along the vector's mode; K < 0: in reverse order, e.g. a flipped row): its
// elements lie in the L = ((VE - 1) * |K| + 1) * EB bytes from its lowest-addressed element to its
// highest, which start `base` bytes from its first element (0, or (VE - 1) * K * EB for K < 0).
// They are read as NL 16-byte loads at byte offsets 0, 16, ..., 16 * (NL - 2) and L - 16 of the
// span (the last overlapping its neighbour), so that no byte outside it is read.  K = 1 is the
// plain vector (L = 16, one load), K = -1 one load reversed.  (On the rows path, loads at 16 * m
// up to the next vector's first element, for all but a row's last vector, measured no faster.)
template <int EB, int K>
struct Span {
  static_assert(K != 0 && K >= -4 && K <= 4, "source steps -4 to -1 and 1 to 4");
  static constexpr int VE = 16 / EB;
  static constexpr int AK = K < 0 ? -K : K;
  static constexpr int L = ((VE - 1) * AK + 1) * EB;
  static constexpr int NL = (L + 15) / 16;
  static constexpr int last = L - 16;
  static constexpr int base = K < 0 ? (VE - 1) * K * EB : 0;
  // the loaded word (of the NL * 4) and the byte in it that hold byte P of the span
  static constexpr int word(int P) { return P < 16 * (NL - 1) ? P / 4 : 4 * (NL - 1) + (P - last) / 4; }
  static constexpr int byte(int P) { return P < 16 * (NL - 1) ? P % 4 : (P - last) % 4; }
  // the span byte that byte b of the gathered vector comes from
  static constexpr int from(int b) { return (K < 0 ? VE - 1 - b / EB : b / EB) * AK * EB + b % EB; }
  // rows path: nontemporal loads for |K| = 1, and for |K| = 2 with 4- or 8-byte elements only
  // (measured on 8192-row copies on MI355X: fp32 with K = 2 3.94 against 3.77 TB/s, fp64 4.00
  // against 3.74; 1- and 2-byte elements 2-3% slower, and K = 3 or 4 25-35% slower: int8 K = 4
  // 1.42 against 1.96 TB/s, fp32 K = 4 1.63 against 2.15, as each line is read by K load
  // instructions one after another)
  static constexpr int NTM = AK == 1 || (AK == 2 && EB >= 4) ? 3 : 2;
};

// Word O of a gathered vector from the loaded words w: one byte permute where its four bytes come
// from at most two words, else two (each half from at most two words, the other half zero: v_perm
// selector 0x0c) or-ed together.  Every index and selector is a compile-time constant.
template <int EB, int K, int O>
__device__ __forceinline__ uint32_t gather_word(const uint32_t* w) {
  using S = Span<EB, K>;
  constexpr int w0 = S::word(S::from(4 * O)), w1 = S::word(S::from(4 * O + 1));
  constexpr int w2 = S::word(S::from(4 * O + 2)), w3 = S::word(S::from(4 * O + 3));
  constexpr int b0 = S::byte(S::from(4 * O)), b1 = S::byte(S::from(4 * O + 1));
  constexpr int b2 = S::byte(S::from(4 * O + 2)), b3 = S::byte(S::from(4 * O + 3));
  // a second word besides w0 among the four, if any
  constexpr int wb = w1 != w0 ? w1 : w2 != w0 ? w2 : w3;
  constexpr bool two = (w1 == w0 || w1 == wb) && (w2 == w0 || w2 == wb) && (w3 == w0 || w3 == wb);
  if constexpr (two) {
    constexpr uint32_t sel = uint32_t(b0) | uint32_t(w1 == w0 ? b1 : 4 + b1) << 8 |
                             uint32_t(w2 == w0 ? b2 : 4 + b2) << 16 | uint32_t(w3 == w0 ? b3 : 4 + b3) << 24;
    if constexpr (sel == 0x03020100u) return w[w0];
    else return perm(w[wb], w[w0], sel);
  } else {
    constexpr uint32_t lo = uint32_t(b0) | uint32_t(w1 == w0 ? b1 : 4 + b1) << 8 | 0x0c0c0000u;
    constexpr uint32_t hi = 0x00000c0cu | uint32_t(b2) << 16 | uint32_t(w3 == w2 ? b3 : 4 + b3) << 24;
    return perm(w[w1], w[w0], lo) | perm(w[w3], w[w2], hi);
  }
}

// A VB-byte vector of elements S apart in memory (S = 1 to 4, or -1 to -4: elements in reverse
// address order).  S = 2: the 2*VB contiguous bytes from p are loaded as two vectors and every
// other element kept (v_perm_b32 for 1- and 2-byte elements, dword selection for wider ones); the
// caller guarantees that those bytes lie inside the source allocation (they end before the row's
// next element).  Other steps (16-byte vectors): the loads of the vector's span only (Span), from
// p + Span::base, compacted by gather_word.  A one-element vector is a single load at any S.
template <int EB, int VB, int S, int NTM>
__device__ __forceinline__ void gload_step(const unsigned char* p, uint32_t* w) {
  if constexpr (S == 1 || VB == EB) {
    gload<VB, NTM>(p, w);
  } else if constexpr (S != 2) {
    static_assert(VB == 16, "source steps other than 1 and 2: 16-byte vectors");
    using Sp = Span<EB, S>;
    uint32_t a[4 * Sp::NL];
#pragma unroll
    for (int m = 0; m + 1 < Sp::NL; ++m) gload<16, NTM>(p + Sp::base + 16 * m, a + 4 * m);
    gload<16, NTM>(p + Sp::base + Sp::last, a + 4 * (Sp::NL - 1));
    w[0] = gather_word<EB, S, 0>(a);
    w[1] = gather_word<EB, S, 1>(a);
    w[2] = gather_word<EB, S, 2>(a);
    w[3] = gather_word<EB, S, 3>(a);
  } else {
    uint32_t a[2 * (VB / 4)];
    gload<VB, NTM>(p, a);
    gload<VB, NTM>(p + VB, a + VB / 4);
#pragma unroll
    for (int k = 0; k < VB / 4; ++k) {
      if constexpr (EB == 1) w[k] = perm(a[2 * k + 1], a[2 * k], 0x06040200u);
      else if constexpr (EB == 2) w[k] = perm(a[2 * k + 1], a[2 * k], 0x05040100u);
      else if constexpr (EB == 4) w[k] = a[2 * k];
      else w[k] = a[4 * (k / 2) + (k & 1)];  // EB == 8: dwords 0, 1 of every 16 bytes
    }
  }
}

// The first n (0 < n < VB/EB) elements of w to consecutive elements at p, in at most four accesses
// of 8, 4, 2 and 1 bytes, largest first.
template <int EB, int VB>
__device__ __forceinline__ void gstore_partial(unsigned char* p, int n, const uint32_t* w) {
  if constexpr (EB < VB) {
    const int nb = n * EB;
    if constexpr (VB == 16) {
      if (nb & 8) *reinterpret_cast<uint64_t*>(p) = uint64_t(w[0]) | (uint64_t(w[1]) << 32);
    }
    if constexpr (VB >= 8 && EB <= 4)
      if (nb & 4) *reinterpret_cast<uint32_t*>(p + (nb & 8)) = get_word<VB>(w, nb & 8);
    if constexpr (EB <= 2)
      if (nb & 2) *reinterpret_cast<uint16_t*>(p + (nb & 12)) = uint16_t(get_word<VB>(w, nb & 12));
    if constexpr (EB == 1)
      if (nb & 1) p[nb & 14] = uint8_t(get_word<VB>(w, nb & 14));
    return;
  }
#pragma unroll
  for (int e = 0; e < VB / EB; ++e) {
    if (e < n) {
      if constexpr (EB >= 4) {
#pragma unroll
        for (int m = 0; m < EB / 4; ++m) reinterpret_cast<uint32_t*>(p + e * EB)[m] = w[e * (EB / 4) + m];
      } else if constexpr (EB == 2) {
        *reinterpret_cast<uint16_t*>(p + 2 * e) = uint16_t(w[e / 2] >> (16 * (e & 1)));
      } else {
        p[e] = uint8_t(w[e / 4] >> (8 * (e & 3)));
      }
    }
  }
}

template <typename V, int NTM>
__device__ __forceinline__ V gload_v(const V* p) {
  if constexpr (NTM & 1) return __builtin_nontemporal_load(p);
  else return *p;
}

template <typename V, int NTM>
__device__ __forceinline__ void gstore_v(V* p, V v) {
  if constexpr (NTM & 2) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Buffer accesses of 16 bytes.  A raw buffer resource (no swizzle, no index stride, 32-bit data
// format, no range limit below 4 GiB) over the memory above a base address that is the same for
// the whole workgroup; lanes address it with 32-bit byte offsets, so the host only takes this
// form where every offset of a launch (or a workgroup) stays below 2^31 (kBufSpan).  Unlike the global instructions
// these carry the CDNA cache-policy bits directly: loads nontemporal (nt), stores written through
// at device scope (sc1).  Measured on MI355X against global accesses with nontemporal loads and
// stores: contiguous copies of 1 GiB 6.21-6.29 -> 6.52 TB/s (one vector per lane), the batched
// 4 x 32 scale-factor tiles 5.92-5.96 -> 6.05-6.20 TB/s.  (The transposes' tiled stores measured
// the same or 1-5% slower with sc1, and keep the global form.)
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // buffer data format: 32 bits
constexpr int kPolNT = 2;               // cache policy: nontemporal
constexpr int kPolSC1 = 16;             // cache policy: device scope (write-through)
// Largest byte span (highest offset + access bytes) a launch may address this way: every offset
// then stays below 2^31, where the offset register reads the same as a signed or unsigned value.
constexpr int64_t kBufSpan = int64_t(1) << 31;

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): waits for the lane's outstanding
// vector memory accesses.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): waits until at most N of the lane's vector memory accesses are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N >= 0 && N < 16, "vmcnt immediates below 16");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

__device__ __forceinline__ Rsrc make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, kRsrcWord3);
}

__device__ __forceinline__ u32x4 bload16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kPolNT));
}

__device__ __forceinline__ void bstore16(Rsrc r, uint32_t off, u32x4 v) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, int(off), 0, kPolSC1);
}

// Orders one wave's LDS writes before its later LDS reads (other lanes' data included): a wave's
// LDS operations execute in issue order, so a wave-scope release/acquire pair around a wave
// barrier (which keeps the compiler from moving accesses across it) is enough; no s_barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t udiv(uint32_t n, const Div32& d) {
  return uint32_t((uint64_t(__umulhi(n, d.mul)) + n) >> d.shr);
}

// Tile `tile` of the grid: column tiles fastest, then row tiles (or the other way round when
// a.order is 1; XCD super-tiles of 2^lsr x 2^lsc tiles when it is 2), then batch tiles, then the
// remaining grid modes (innermost last).  Returns the tile's first element on both sides and how
// much of each tile extent lies inside the copy.
struct TileAt {
  int64_t sbase, dbase;
  int64_t remR, remC, remB;
  bool valid;  // false: a padding workgroup of order 2 (no tile; it returns at once)
};

__device__ __forceinline__ TileAt tile_at(const TransposeArgs& a, uint32_t tile) {
  uint32_t idx = tile, q, tcI, trI;
  bool valid = true;
  if (a.order == 2) {
    // XCD x = idx % kXcds takes super-tiles x, x + kXcds, ..; the 2^(lsr + lsc) tiles of a super-tile
    // are consecutive in that XCD's share of the grid, column tiles fastest inside it
    const uint32_t x = idx % kXcds, k = idx / kXcds;
    const uint32_t per = 1u << (a.lsr + a.lsc);  // tiles per super-tile
    const uint32_t w = k & (per - 1);
    const uint32_t gst = (k >> (a.lsr + a.lsc)) * kXcds + x;  // super-tile over all slices
    const uint32_t slice = gst / a.nst, st = gst - slice * a.nst;
    q = udiv(st, a.stC);
    trI = (q << a.lsr) + (w >> a.lsc);
    tcI = ((st - q * a.stC.d) << a.lsc) + (w & ((1u << a.lsc) - 1));
    valid = slice < a.nslices && trI < a.tilesR.d && tcI < a.tilesC.d;
    idx = valid ? slice : 0;
  } else {
    const Div32& first = a.order ? a.tilesRg : a.tilesC;
    const Div32& second = a.order ? a.tilesC : a.tilesR;
    q = udiv(idx, first);
    const uint32_t i0 = idx - q * first.d;
    idx = q;
    q = udiv(idx, second);
    const uint32_t i1 = idx - q * second.d;
    tcI = a.order ? i1 : i0;
    trI = a.order ? i0 : i1;
    idx = q;
    // order 1 with a padded row-tile count: the neighbours along a source row are a multiple of
    // kXcds workgroups apart, so on one XCD, where they share the cache lines they both read
    valid = trI < a.tilesR.d;
  }
  q = udiv(idx, a.tilesB);
  const uint32_t tbI = idx - q * a.tilesB.d;
  idx = q;
  int64_t s = a.src_off, d = a.dst_off;
  for (int k = a.nbatch - 1; k >= 0; --k) {
    q = udiv(idx, a.bdiv[k]);
    const uint32_t i = idx - q * a.bdiv[k].d;
    idx = q;
    s += int64_t(i) * a.bs[k];
    d += int64_t(i) * a.bd[k];
  }
  const int64_t r0 = int64_t(trI) << a.lTR, c0 = int64_t(tcI) << a.lTC, b0 = int64_t(tbI) << a.lNB;
  TileAt t;
  t.sbase = s + r0 * a.sR + c0 * a.sC + b0 * a.sB;
  t.dbase = d + r0 * a.dR + c0 * a.dC + b0 * a.dB;
  t.remR = a.eR - r0;
  t.remC = a.eC - c0;
  t.remB = a.eB - b0;
  t.valid = valid;
  return t;
}

__device__ __forceinline__ bool tile_full(const TransposeArgs& a, const TileAt& t) {
  return t.remR >= (int64_t(1) << a.lTR) && t.remC >= (int64_t(1) << a.lTC) && t.remB >= (int64_t(1) << a.lNB);
}

}  // namespace dev
}  // namespace tc
