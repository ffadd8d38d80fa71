// Device kernels of the layout-permuting tile copy for gfx950 (CDNA4, wave64), other than the
// LDS-tiled transpose (transpose.hpp), and the launcher of every plan.
//
// rows_kernel: both sides contiguous along one mode; vectors are staged in registers (or, for
//   the round-trip variant, through LDS as in the gmem_smem demonstration program).  With one
//   element per "vector" it is also the guarded element-wise fallback.
// shuffle_kernel: batches of 4 x C blocks of 4-byte elements, transposed by exchanging 16-byte
//   vectors between lanes, no LDS: a v_permlane16_swap row swap at lane distance 16, bank-masked
//   DPP row rotations at distances 8 and 4, ds_swizzle only at distance 2.
// guarded_tile_kernel: fallback LDS tile with element-wide accesses and per-element guards,
//   for layouts the vector paths do not take (FORCE_GUARDED, or no unit-stride mode to vectorize).
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "transpose.hpp"

namespace tc {
namespace dev {

// Vector index -> source / destination byte offsets over the grid modes (innermost last).
__device__ __forceinline__ void row_offsets(const RowArgs& a, uint32_t n, int64_t* so, int64_t* dof) {
  int64_t s = a.src_off, d = a.dst_off;
#pragma unroll
  for (int k = kMaxRank - 1; k >= 0; --k) {
    if (k < a.rank) {
      const uint32_t q = uint32_t((uint64_t(__umulhi(n, a.mul[k])) + n) >> a.shr[k]);
      const uint32_t i = n - q * a.ext[k];
      s += int64_t(i) * a.s[k];
      d += int64_t(i) * a.d[k];
      n = q;
    }
  }
  *so = s;
  *dof = d;
}

// [outer, threads, vec] copy: access v = blockIdx * NT*ROUNDS + f*NT + t.  With USE_LDS the
// vectors make the round trip global -> LDS -> global of the gmem_smem demonstration.  BUF:
// 16-byte buffer accesses from the bases a.sbuf / a.dbuf (the host has checked that every offset
// of the launch stays below 2^31) with the streaming cache policies.
template <int VB, int NT, int ROUNDS, bool USE_LDS, int NTM, bool GUARD, bool BURST, bool BUF>
__device__ __forceinline__ void rows_body(const RowArgs& a, typename Bytes<VB>::T* lds) {
  typedef typename Bytes<VB>::T V;
  static_assert(!BUF || (VB == 16 && !USE_LDS), "buffer accesses: 16-byte vectors in registers");
  const int t = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * NT * ROUNDS;
  // (the buffer bases exist only in the BUF instances: a.sbuf / a.dbuf are not offsets otherwise)
  const Rsrc rs = make_rsrc(BUF ? a.src + a.sbuf : a.src), rd = make_rsrc(BUF ? a.dst + a.dbuf : a.dst);
  V reg[ROUNDS];
  int64_t soff[ROUNDS], doff[ROUNDS];
  bool live[ROUNDS];
  auto load = [&](int f) {
    if constexpr (BUF) reg[f] = bload16(rs, uint32_t(soff[f] - a.sbuf));
    else reg[f] = gload_v<V, NTM>(reinterpret_cast<const V*>(a.src + soff[f]));
  };
  if constexpr (BURST) {
    // all offsets first (the decode loop has a run-time trip count), then every load back to back
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f) {
      const int64_t v = base + f * NT + t;
      live[f] = !GUARD || v < a.nvec;
      if (live[f]) row_offsets(a, uint32_t(v), &soff[f], &doff[f]);
    }
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f)
      if (live[f]) load(f);
  } else {
    // paced: each load after its offsets, and one load in flight per lane (an explicit wait before
    // the next decode); measured faster than all loads at once for permuted rows and large copies
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f) {
      const int64_t v = base + f * NT + t;
      live[f] = !GUARD || v < a.nvec;
      if (live[f]) {
        row_offsets(a, uint32_t(v), &soff[f], &doff[f]);
        load(f);
      }
      if (f + 1 < ROUNDS) wait_vmem();
    }
  }
  if constexpr (USE_LDS) {
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f) lds[f * NT + t] = reg[f];
    __syncthreads();
#pragma unroll
    for (int f = 0; f < ROUNDS; ++f) reg[f] = lds[f * NT + t];
  }
#pragma unroll
  for (int f = 0; f < ROUNDS; ++f) {
    if (!live[f]) continue;
    if constexpr (BUF) bstore16(rd, uint32_t(doff[f] - a.dbuf), reg[f]);
    else gstore_v<V, NTM>(reinterpret_cast<V*>(a.dst + doff[f]), reg[f]);
  }
}

// BURST: workgroups wholly inside the copy take the unguarded body, all loads in flight.  Else
// every workgroup takes the guarded body, whose per-vector branch paces the loads one at a time.
template <int VB, int NT, int ROUNDS, bool USE_LDS, int NTM, bool BURST = false, bool BUF = false>
__global__ void __launch_bounds__(NT) rows_kernel(RowArgs a) {
  typedef typename Bytes<VB>::T V;
  __shared__ __attribute__((aligned(16))) V lds[USE_LDS ? NT * ROUNDS : 1];
  if (BURST && (int64_t(blockIdx.x) + 1) * NT * ROUNDS <= a.nvec)
    rows_body<VB, NT, ROUNDS, USE_LDS, NTM, false, BURST, BUF>(a, lds);
  else
    rows_body<VB, NT, ROUNDS, USE_LDS, NTM, true, BURST, BUF>(a, lds);
}

// Copies n < 16 bytes in at most four accesses of 8, 4, 2 and 1 bytes (at any alignment: gfx950
// global memory takes unaligned accesses), rather than one access per element.
__device__ __forceinline__ void copy_short(const unsigned char* __restrict__ p, unsigned char* __restrict__ q, int n) {
  int o = 0;
  if (n & 8) {
    *reinterpret_cast<uint64_t*>(q) = *reinterpret_cast<const uint64_t*>(p);
    o = 8;
  }
  if (n & 4) {
    *reinterpret_cast<uint32_t*>(q + o) = *reinterpret_cast<const uint32_t*>(p + o);
    o += 4;
  }
  if (n & 2) {
    *reinterpret_cast<uint16_t*>(q + o) = *reinterpret_cast<const uint16_t*>(p + o);
    o += 2;
  }
  if (n & 1) q[o] = p[o];
}

// Element-aligned rows: 16-byte vectors at element alignment along rows of `row_elems` elements
// (the destination contiguous along them).  K = 1: the source is contiguous along the rows too,
// one 16-byte load per vector.  K = 2, 3, 4, or -1 to -4: the source steps K elements along the
// rows (a strided slice written out densely; a negative K reverses the order, e.g. a flipped row),
// each vector read as 16-byte loads of its span (Span) and compacted in registers (gather_word).
// A row's short last vector moves back to end at the row's end, a whole vector overlapping its
// neighbour (measured against copying it in a few narrower accesses: the 8190 x 4095 int8 slice
// 2.13 -> 3.1 TB/s, the 8190^2 int8 window of an 8192^2 matrix 4.54 -> 4.96, fp32 5.94 -> 6.04);
// rows shorter than one vector, and the BUF instances (whose stores stay on the 16-byte grid), go
// in at most four accesses (K = 1, copy_short) or element by element.  All offsets first, then
// every load of a thread, then the stores; whole vectors nontemporal (measured 5-12% faster than
// plain accesses here; gathered loads: Span::NTM).  BUF (K = 1): the whole vectors as buffer
// accesses from the bases a.sbuf / a.dbuf (destination vectors on the 16-byte grid: an fp32 copy
// at an odd element offset 6.21 -> 6.39 TB/s).
template <int EB, int NT, int ROUNDS, bool BUF = false, int K = 1>
__global__ void __launch_bounds__(NT) rows_unaligned_kernel(RowArgs a) {
  static_assert(K == 1 || !BUF, "gathered rows: global accesses");
  using S = Span<EB, K>;
  constexpr int VE = 16 / EB;
  const int t = threadIdx.x;
  const Rsrc rs = make_rsrc(BUF ? a.src + a.sbuf : a.src), rd = make_rsrc(BUF ? a.dst + a.dbuf : a.dst);
  const int64_t base = int64_t(blockIdx.x) * NT * ROUNDS;
  int64_t soff[ROUNDS], doff[ROUNDS];
  int cnt[ROUNDS];
  uint32_t reg[ROUNDS][4 * S::NL];
#pragma unroll
  for (int f = 0; f < ROUNDS; ++f) {
    const int64_t v = base + f * NT + t;
    cnt[f] = 0;
    if (v < a.nvec) {
      const uint32_t inner = a.ext[a.rank - 1];
      const uint32_t k = uint32_t(v) - uint32_t((uint64_t(__umulhi(uint32_t(v), a.mul[a.rank - 1])) + uint32_t(v)) >>
                                                a.shr[a.rank - 1]) * inner;  // vector index within its row
      row_offsets(a, uint32_t(v), &soff[f], &doff[f]);
      const int64_t left = a.row_elems - int64_t(k) * VE;
      cnt[f] = left < VE ? int(left) : VE;
      if (!BUF && cnt[f] < VE && a.row_elems >= VE) {
        // a row's short last vector moves back to end at the row's end, a whole vector that
        // overlaps its neighbour (whose bytes it writes again with the same values)
        soff[f] -= int64_t(VE - cnt[f]) * K * EB;
        doff[f] -= int64_t(VE - cnt[f]) * EB;
        cnt[f] = VE;
      }
    }
  }
#pragma unroll
  for (int f = 0; f < ROUNDS; ++f) {
    if (cnt[f] != VE) continue;
    if constexpr (BUF) {
      const u32x4 v = bload16(rs, uint32_t(soff[f] - a.sbuf));
      reg[f][0] = v.x; reg[f][1] = v.y; reg[f][2] = v.z; reg[f][3] = v.w;
    } else {
#pragma unroll
      for (int m = 0; m + 1 < S::NL; ++m) gload<16, S::NTM>(a.src + soff[f] + S::base + 16 * m, &reg[f][4 * m]);
      gload<16, S::NTM>(a.src + soff[f] + S::base + S::last, &reg[f][4 * (S::NL - 1)]);
    }
  }
#pragma unroll
  for (int f = 0; f < ROUNDS; ++f) {
    if (cnt[f] == VE) {
      if constexpr (BUF) {
        bstore16(rd, uint32_t(doff[f] - a.dbuf), u32x4{reg[f][0], reg[f][1], reg[f][2], reg[f][3]});
      } else if constexpr (K == 1) {
        gstore<16, 3>(a.dst + doff[f], reg[f]);
      } else {
        const uint32_t o[4] = {gather_word<EB, K, 0>(reg[f]), gather_word<EB, K, 1>(reg[f]),
                               gather_word<EB, K, 2>(reg[f]), gather_word<EB, K, 3>(reg[f])};
        gstore<16, 3>(a.dst + doff[f], o);
      }
    } else if (cnt[f] > 0) {
      if constexpr (K == 1) {
        copy_short(a.src + soff[f], a.dst + doff[f], cnt[f] * EB);
      } else {
        // rows shorter than one vector: element by element, every load issued before the stores
        typedef typename Bytes<EB>::T E;
        E x[VE - 1];
#pragma unroll
        for (int e = 0; e < VE - 1; ++e)
          if (e < cnt[f]) x[e] = reinterpret_cast<const E*>(a.src + soff[f])[e * K];
#pragma unroll
        for (int e = 0; e < VE - 1; ++e)
          if (e < cnt[f]) reinterpret_cast<E*>(a.dst + doff[f])[e] = x[e];
      }
    }
  }
}

// Interleave path: CH channels between interleaved and planar layouts (e.g. NHWC <-> NCHW).  A
// lane holds one group of VE = 16/EB pixels of every channel: element (pixel p, channel c) of the
// interleaved side is element p*CH + c of its CH registers vectors, of the planar side element
// c*VE + p.  The move between the two is a fixed permutation of register bytes (its indices are
// compile-time constants).  TO: interleaved source, planar destination.
template <int EB, int CH, bool TO>
__device__ __forceinline__ void interleave_regs(const uint32_t* in, uint32_t* out) {
  constexpr int VE = 16 / EB, N = CH * VE;
  if constexpr (EB >= 4) {
    constexpr int W = EB / 4;
#pragma unroll
    for (int o = 0; o < N; ++o) {
      const int i = TO ? (o % VE) * CH + o / VE : (o % CH) * VE + o / CH;
#pragma unroll
      for (int m = 0; m < W; ++m) out[o * W + m] = in[i * W + m];
    }
  } else {
    constexpr int PER = 4 / EB;  // elements per dword
    constexpr uint32_t MASK = EB == 1 ? 0xFFu : 0xFFFFu;
#pragma unroll
    for (int k = 0; k < CH * 4; ++k) out[k] = 0;
#pragma unroll
    for (int o = 0; o < N; ++o) {
      const int i = TO ? (o % VE) * CH + o / VE : (o % CH) * VE + o / CH;
      out[o / PER] |= ((in[i / PER] >> (8 * EB * (i % PER))) & MASK) << (8 * EB * (o % PER));
    }
  }
}

template <int EB, int CH, bool TO, bool GUARD>
__device__ __forceinline__ void interleave_body(const RowArgs& a, int64_t plane) {
  constexpr int R = kInterleaveRounds, NT = kRowThreads;
  const int t = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * NT * R;
  int64_t so[R], dof[R];
  bool ok[R];
  uint32_t in[R][CH * 4];
#pragma unroll
  for (int f = 0; f < R; ++f) {
    const int64_t v = base + f * NT + t;
    ok[f] = !GUARD || v < a.nvec;
    if (ok[f]) row_offsets(a, uint32_t(v), &so[f], &dof[f]);
  }
#pragma unroll
  for (int f = 0; f < R; ++f)
    if (ok[f])
#pragma unroll
      for (int k = 0; k < CH; ++k) gload<16, 3>(a.src + so[f] + (TO ? int64_t(k) * 16 : k * plane), in[f] + 4 * k);
#pragma unroll
  for (int f = 0; f < R; ++f) {
    if (!ok[f]) continue;
    uint32_t out[CH * 4];
    interleave_regs<EB, CH, TO>(in[f], out);
#pragma unroll
    for (int k = 0; k < CH; ++k) gstore<16, 3>(a.dst + dof[f] + (TO ? k * plane : int64_t(k) * 16), out + 4 * k);
  }
}

// Workgroups wholly inside the copy run unguarded (all loads in flight); the last one guarded.
template <int EB, int CH, bool TO>
__global__ void __launch_bounds__(kRowThreads) interleave_kernel(RowArgs a, int64_t plane) {
  if ((int64_t(blockIdx.x) + 1) * kRowThreads * kInterleaveRounds <= a.nvec) interleave_body<EB, CH, TO, false>(a, plane);
  else interleave_body<EB, CH, TO, true>(a, plane);
}

// Fallback tile: element-wide accesses, padded LDS rows, guards on every element.
template <int EB>
__global__ void __launch_bounds__(kGuardThreads) guarded_tile_kernel(TransposeArgs a) {
  typedef typename Bytes<EB>::T V;
  constexpr int NT = kGuardThreads;
  constexpr int PAD = EB < 4 ? 4 / EB : 1;
  constexpr int TRC = EB <= 4 ? 64 * 64 : (EB == 8 ? 32 * 64 : 32 * 32);
  constexpr int ROWS = EB <= 8 ? (EB <= 4 ? 64 : 32) : 32;
  constexpr int COLS = TRC / ROWS;
  constexpr int PITCH = COLS + PAD;
  __shared__ V lds[ROWS * PITCH];
  const TileAt tl = tile_at(a, blockIdx.x);
  if (!tl.valid) return;
  const int64_t sbase = tl.sbase, dbase = tl.dbase, remR = tl.remR, remC = tl.remC;
  const V* __restrict__ src = reinterpret_cast<const V*>(a.src);
  V* __restrict__ dst = reinterpret_cast<V*>(a.dst);
  const int t = threadIdx.x;
#pragma unroll 4
  for (int i = 0; i < TRC / NT; ++i) {
    const int e = i * NT + t;
    const int c = e % COLS, r = e / COLS;
    if (r < remR && c < remC) lds[r * PITCH + c] = src[sbase + r * a.sR + c * a.sC];
  }
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < TRC / NT; ++i) {
    const int e = i * NT + t;
    const int r = e % ROWS, c = e / ROWS;
    if (r < remR && c < remC) dst[dbase + r * a.dR + c * a.dC] = lds[r * PITCH + c];
  }
}


// Batches of 4 x C blocks of 4-byte elements: each lane loads 16-byte vectors (row i = l / (C/4),
// columns 4q.. of block row i, l the lane's index within the block), then two exchanges with the
// partner lane move register bit 1 against lane bit log2(C/2) and register bit 0 against lane bit
// log2(C/4) -- afterwards lane l = a (C/4) + q holds column 4q + a, rows 0..3: one 16-byte vector
// of the column-major destination.  The exchanges are row swaps and bank-masked DPP moves
// (ds_swizzle only for the 2-lane distance of C = 8; `exchange`); every lane takes part (lanes past
// the end load and store nothing, and whole blocks are past the end together).  The permute page's
// register-staged exchange, with the staging done by cross-lane moves instead of shared memory
// (TVM TIRx docs, "permute_layout", Algorithm step 3).
template <int DIST>
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v) {
  static_assert(DIST >= 1 && DIST <= 16, "ds_swizzle bit mode exchanges within 32 lanes");
  return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), 0x1F | (DIST << 10)));
}

// DPP move within 16-lane rows (CTRL: row_ror:N = 0x120 + N, lane i takes lane i - N mod 16) into
// the banks of BANKS (4 lanes each, 4 per row); the other banks keep `keep`.
template <int CTRL, int BANKS>
__device__ __forceinline__ uint32_t dpp_into(uint32_t keep, uint32_t src) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(keep), int(src), CTRL, 0xF, BANKS, false));
}

// One butterfly exchange between lanes D apart (D = 2, 4, 8, 16): a lane whose lane bit log2(D) is
// set takes its partner's b into a, the others take the partner's a into b.  D = 16: the gfx950 row
// swap (odd 16-lane rows of the first register with even rows of the second); D = 8 and 4: DPP row
// rotations whose bank masks pick the receiving lanes (8: banks 2-3 from 0-1 and back; 4: odd banks
// from even with ror 4, even from odd with ror 12); D = 2 (partners in one bank): ds_swizzle and
// selects.
template <int D>
__device__ __forceinline__ void exchange(uint32_t& a, uint32_t& b, bool hi) {
  if constexpr (D == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  } else if constexpr (D == 8) {
    const uint32_t na = dpp_into<0x128, 0xC>(a, b), nb = dpp_into<0x128, 0x3>(b, a);
    a = na;
    b = nb;
  } else if constexpr (D == 4) {
    const uint32_t na = dpp_into<0x124, 0xA>(a, b), nb = dpp_into<0x12C, 0x5>(b, a);
    a = na;
    b = nb;
  } else {
    const uint32_t t = xor_lanes<D>(hi ? a : b);
    if (hi) a = t;
    else b = t;
  }
}

template <int LC, int NTM, bool GUARD, bool BUF>
__device__ __forceinline__ void shuffle_rounds(const ShuffleArgs& a) {
  constexpr int LQ = LC - 2;  // log2 of the vectors per block row
  constexpr int R = kShuffleRounds, NT = kShuffleThreads;
  const int lane = int(threadIdx.x) & 63;
  const bool hi1 = (lane >> (LQ + 1)) & 1, hi0 = (lane >> LQ) & 1;
  const int row = (lane >> LQ) & 3, q = lane & ((1 << LQ) - 1);
  const int col = 4 * q + row;  // destination column after the exchanges
  const int64_t g0 = int64_t(blockIdx.x) * R * NT + threadIdx.x;
  // BUF: buffer bases at the workgroup's first block (the host has checked that the workgroup's
  // blocks lie within 2 GiB above it on both sides)
  const int64_t blk0 = (int64_t(blockIdx.x) * R * NT) >> LC;
  const Rsrc rs = make_rsrc(a.src + (a.so + blk0 * a.sB) * 4), rd = make_rsrc(a.dst + (a.dof + blk0 * a.dB) * 4);
  u32x4 v[R];
#pragma unroll
  for (int f = 0; f < R; ++f) {
    const int64_t g = g0 + int64_t(f) * NT;  // g % 64 == lane
    const int64_t blk = g >> LC;
    const u32x4* p = reinterpret_cast<const u32x4*>(a.src) + ((a.so + blk * a.sB) >> 2) + row * (1 << LQ) + q;
    if constexpr (GUARD) {
      v[f] = u32x4{0, 0, 0, 0};
      if (g < a.nvec) v[f] = gload_v<u32x4, NTM>(p);
    } else if constexpr (BUF) {
      v[f] = bload16(rs, uint32_t(((blk - blk0) * a.sB + (row * (1 << LQ) + q) * 4) * 4));
    } else {
      v[f] = gload_v<u32x4, NTM>(p);
    }
  }
#pragma unroll
  for (int f = 0; f < R; ++f) {
    uint32_t w0 = v[f].x, w1 = v[f].y, w2 = v[f].z, w3 = v[f].w;
    exchange<(2 << LQ)>(w0, w2, hi1);
    exchange<(2 << LQ)>(w1, w3, hi1);
    exchange<(1 << LQ)>(w0, w1, hi0);
    exchange<(1 << LQ)>(w2, w3, hi0);
    const int64_t g = g0 + int64_t(f) * NT;
    const int64_t blk = g >> LC;
    u32x4* p = reinterpret_cast<u32x4*>(a.dst) + ((a.dof + blk * a.dB) >> 2) + col;
    if constexpr (!GUARD && BUF) bstore16(rd, uint32_t(((blk - blk0) * a.dB + col * 4) * 4), u32x4{w0, w1, w2, w3});
    else if (!GUARD || g < a.nvec) gstore_v<u32x4, NTM>(p, u32x4{w0, w1, w2, w3});
  }
}

// Workgroups wholly inside the copy run with no per-lane condition (all loads in flight); the
// last one, if ragged, is guarded.
template <int LC, int NTM, bool BUF>
__global__ void __launch_bounds__(kShuffleThreads) shuffle_kernel(ShuffleArgs a) {
  if ((int64_t(blockIdx.x) + 1) * kShuffleRounds * kShuffleThreads <= a.nvec) shuffle_rounds<LC, NTM, false, BUF>(a);
  else shuffle_rounds<LC, NTM, true, BUF>(a);
}

}  // namespace dev

namespace {

void fill_batch(const Plan& p, TransposeArgs* ta, int skip0, int skip1, int skip2) {
  ta->nbatch = 0;
  for (int k = 0; k < p.j.rank; ++k) {
    if (k == skip0 || k == skip1 || k == skip2) continue;
    ta->bdiv[ta->nbatch] = make_div32(uint32_t(p.j.m[k].e));
    ta->bs[ta->nbatch] = p.j.m[k].s;
    ta->bd[ta->nbatch] = p.j.m[k].d;
    ++ta->nbatch;
  }
}

int lg(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

template <int VB, int NT, bool LDS, int NTM, bool BURST = false, bool BUF = false, int ROUNDS = kRowRounds>
void launch_rows_t(const RowArgs& ra, int64_t wgs, hipStream_t s) {
  hipLaunchKernelGGL((dev::rows_kernel<VB, NT, ROUNDS, LDS, NTM, BURST, BUF>), dim3(uint32_t(wgs)), dim3(NT), 0, s, ra);
}

// The 16-byte rows kernel for `rounds` vectors per thread, paced or burst loads, global or
// buffer accesses.
template <bool BURST, bool BUF>
void launch_rows16(int rounds, const RowArgs& ra, int64_t wgs, hipStream_t s) {
  if (rounds == 1) launch_rows_t<16, kRowThreads, false, 3, BURST, BUF, 1>(ra, wgs, s);
  if (rounds == 2) launch_rows_t<16, kRowThreads, false, 3, BURST, BUF, 2>(ra, wgs, s);
  if (rounds == 4) launch_rows_t<16, kRowThreads, false, 3, BURST, BUF, 4>(ra, wgs, s);
}

// Lowest byte offset of a launch's accesses on one side (offset `off`, grid extents `ext`, byte
// strides `st`, accesses of `vb` bytes) and whether all of them lie within kBufSpan bytes of it.
bool buffer_window(int64_t off, const uint32_t* ext, const int64_t* st, int rank, int vb, int64_t* lo) {
  int64_t mn = off, mx = off;
  for (int k = 0; k < rank; ++k) {
    if (ext[k] == 0) return false;
    const int64_t step = int64_t(ext[k] - 1) * st[k];
    if (step < 0) mn += step;
    else mx += step;
  }
  *lo = mn;
  return mx + vb - mn <= dev::kBufSpan;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kNoBuffer = INT64_MIN;  // RowArgs::sbuf of a launch that uses global accesses

// The rows-type kernel of a plan over the vectors of `ra`, in `wgs` workgroups.
void launch_rows(const Plan& p, const RowArgs& ra, int64_t wgs, hipStream_t s) {
  if (p.path == TC_PATH_ROWS && p.unaligned) {
    const dim3 grid = dim3(uint32_t(wgs)), block = dim3(kRowThreads);
    const bool buf = p.buffers && ra.sbuf != kNoBuffer;
#define TC_RU(E, R)                                                                                          \
  if (p.eb == E && p.row_rounds == R && p.step == 1) {                                                       \
    if (buf) hipLaunchKernelGGL((dev::rows_unaligned_kernel<E, kRowThreads, R, true>), grid, block, 0, s, ra); \
    else hipLaunchKernelGGL((dev::rows_unaligned_kernel<E, kRowThreads, R, false>), grid, block, 0, s, ra);    \
  }
#define TC_RG(E, K)                                                                                              \
  if (p.eb == E && p.step == K && p.row_rounds == 1)                                                             \
    hipLaunchKernelGGL((dev::rows_unaligned_kernel<E, kRowThreads, 1, false, K>), grid, block, 0, s, ra);          \
  if (p.eb == E && p.step == K && p.row_rounds == kRowRounds && kRowRounds != 1)                                 \
    hipLaunchKernelGGL((dev::rows_unaligned_kernel<E, kRowThreads, kRowRounds, false, K>), grid, block, 0, s, ra);
#define TC_RU3(E) TC_RU(E, 1) TC_RU(E, 2) TC_RU(E, 4)                                      \
  TC_RG(E, 2) TC_RG(E, 3) TC_RG(E, 4) TC_RG(E, -1) TC_RG(E, -2) TC_RG(E, -3) TC_RG(E, -4)
    TC_RU3(1) TC_RU3(2) TC_RU3(4) TC_RU3(8)
#undef TC_RU3
#undef TC_RG
#undef TC_RU
  } else if (p.path == TC_PATH_ROUNDTRIP) {
    if (p.vb == 16) launch_rows_t<16, kWave, true, 0>(ra, wgs, s);
    if (p.vb == 8) launch_rows_t<8, kWave, true, 0>(ra, wgs, s);
    if (p.vb == 4) launch_rows_t<4, kWave, true, 0>(ra, wgs, s);
  } else if (p.path == TC_PATH_ROWS && p.vb == 16) {
    // buffer accesses where every offset of this launch fits (the caller has set sbuf / dbuf)
    const bool buf = p.buffers && ra.sbuf != kNoBuffer;
    if (p.row_burst && buf) launch_rows16<true, true>(p.row_rounds, ra, wgs, s);
    if (p.row_burst && !buf) launch_rows16<true, false>(p.row_rounds, ra, wgs, s);
    if (!p.row_burst && buf) launch_rows16<false, true>(p.row_rounds, ra, wgs, s);
    if (!p.row_burst && !buf) launch_rows16<false, false>(p.row_rounds, ra, wgs, s);
  } else if (p.path == TC_PATH_ROWS && p.row_burst) {
    if (p.vb == 8) launch_rows_t<8, kRowThreads, false, 3, true>(ra, wgs, s);
    if (p.vb == 4) launch_rows_t<4, kRowThreads, false, 3, true>(ra, wgs, s);
  } else if (p.path == TC_PATH_ROWS) {
    if (p.vb == 4) launch_rows_t<4, kRowThreads, false, 3>(ra, wgs, s);
  } else {
    if (p.eb == 1) launch_rows_t<1, kGuardThreads, false, 0>(ra, wgs, s);
    if (p.eb == 2) launch_rows_t<2, kGuardThreads, false, 0>(ra, wgs, s);
    if (p.eb == 4) launch_rows_t<4, kGuardThreads, false, 0>(ra, wgs, s);
    if (p.eb == 8) launch_rows_t<8, kGuardThreads, false, 0>(ra, wgs, s);
    if (p.eb == 16) launch_rows_t<16, kGuardThreads, false, 0>(ra, wgs, s);
  }
}

}  // namespace

Div32 make_div32(uint32_t d) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  Div32 v;
  v.d = d;
  v.shr = s;
  v.mul = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return v;
}

bool launch_transpose(int eb, const TransposeCfg& c, const TransposeArgs* ta, int64_t wgs, void* stream) {
  switch (eb) {
    case 1: return launch_transpose_eb1(c, ta, wgs, stream);
    case 2: return launch_transpose_eb2(c, ta, wgs, stream);
    case 4: return launch_transpose_eb4(c, ta, wgs, stream);
    case 8: return launch_transpose_eb8(c, ta, wgs, stream);
    case 16: return launch_transpose_eb16(c, ta, wgs, stream);
    default: return false;
  }
}

int launch_plan(const Plan& p, const void* src, void* dst, void* stream, std::string* err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.path == TC_PATH_EMPTY) return TC_OK;
  const Joint& j = p.j;
  if (p.path == TC_PATH_SHUFFLE) {
    ShuffleArgs sa{};
    sa.src = static_cast<const unsigned char*>(src);
    sa.dst = static_cast<unsigned char*>(dst);
    sa.so = j.so;
    sa.dof = j.dof;
    sa.sB = p.mode_b >= 0 ? j.m[p.mode_b].s : 0;
    sa.dB = p.mode_b >= 0 ? j.m[p.mode_b].d : 0;
    // one launch, or (2^31 vectors and more) launches of kLaunchVectors vectors, a whole number
    // of blocks each (a block is C vectors)
    const int64_t total = j.count / 4;
    const int64_t per = total < (int64_t(1) << 31) ? total : kLaunchVectors;
    for (int64_t v0 = 0; v0 < total; v0 += per) {
      ShuffleArgs sc = sa;
      const int64_t b0 = v0 / p.shuffle_c;
      sc.so = sa.so + b0 * sa.sB;
      sc.dof = sa.dof + b0 * sa.dB;
      sc.nvec = std::min(per, total - v0);
      const dim3 grid(uint32_t(ceil_div(sc.nvec, int64_t(kShuffleThreads) * kShuffleRounds))), block(kShuffleThreads);
      // buffer accesses: a workgroup's blocks (4 x C elements each) within 2 GiB above its first
      const int64_t bpw = int64_t(kShuffleRounds) * kShuffleThreads / p.shuffle_c;
      const bool buf = p.buffers && sa.sB >= 0 && sa.dB >= 0 &&
                       ((bpw - 1) * sa.sB + 4 * p.shuffle_c) * 4 <= dev::kBufSpan &&
                       ((bpw - 1) * sa.dB + 4 * p.shuffle_c) * 4 <= dev::kBufSpan;
#define TC_SH(LC)                                                                  \
  if (buf) hipLaunchKernelGGL((dev::shuffle_kernel<LC, 3, true>), grid, block, 0, s, sc); \
  else hipLaunchKernelGGL((dev::shuffle_kernel<LC, 3, false>), grid, block, 0, s, sc)
      switch (p.shuffle_c) {
        case 8: TC_SH(3); break;
        case 16: TC_SH(4); break;
        case 32: TC_SH(5); break;
        default:
          *err = "no shuffle kernel for this block width";
          return TC_E_ARG;
      }
#undef TC_SH
      if (hipPeekAtLastError() != hipSuccess) break;
    }
  } else if (p.path == TC_PATH_INTERLEAVE) {
    // grid of pixel groups: the modes other than the two of the exchange, then the pixel mode
    const int ve = 16 / p.eb;
    const int px = p.to_planes ? p.mode_r : p.mode_c, ch = p.to_planes ? p.mode_c : p.mode_r;
    RowArgs ra{};
    ra.src = static_cast<const unsigned char*>(src);
    ra.dst = static_cast<unsigned char*>(dst);
    ra.src_off = j.so * p.eb;
    ra.dst_off = j.dof * p.eb;
    int n = 0;
    for (int k = 0; k <= j.rank; ++k) {
      if (k == px || k == ch) continue;
      const bool pix = k == j.rank;  // the pixel mode goes last (innermost)
      const Mode& m = pix ? j.m[px] : j.m[k];
      const int64_t e = pix ? m.e / ve : m.e;
      ra.ext[n] = uint32_t(e);
      const Div32 dv = make_div32(uint32_t(e));
      ra.mul[n] = dv.mul;
      ra.shr[n] = dv.shr;
      ra.s[n] = m.s * p.eb * (pix ? ve : 1);
      ra.d[n] = m.d * p.eb * (pix ? ve : 1);
      ++n;
    }
    ra.rank = n;
    ra.nvec = j.count / (int64_t(ve) * p.shuffle_c);
    const int64_t plane = (p.to_planes ? j.m[ch].d : j.m[ch].s) * p.eb;
    const dim3 grid = dim3(uint32_t(p.workgroups)), block = dim3(kRowThreads);
#define TC_IL(E, CHN)                                                                                      \
  if (p.eb == E && p.shuffle_c == CHN) {                                                                   \
    if (p.to_planes) hipLaunchKernelGGL((dev::interleave_kernel<E, CHN, true>), grid, block, 0, s, ra, plane); \
    else hipLaunchKernelGGL((dev::interleave_kernel<E, CHN, false>), grid, block, 0, s, ra, plane);        \
  }
#define TC_IL4(E) TC_IL(E, 2) TC_IL(E, 3) TC_IL(E, 4) TC_IL(E, 8)
    TC_IL4(1) TC_IL4(2) TC_IL4(4) TC_IL4(8)
#undef TC_IL4
#undef TC_IL
  } else if (p.path == TC_PATH_TRANSPOSE || p.path == TC_PATH_GUARDED_TILE) {
    TransposeArgs ta{};
    ta.src = static_cast<const unsigned char*>(src);
    ta.dst = static_cast<unsigned char*>(dst);
    ta.src_off = j.so;
    ta.dst_off = j.dof;
    const Mode& R = j.m[p.mode_r];
    const Mode& C = j.m[p.mode_c];
    ta.eR = R.e;
    ta.eC = C.e;
    ta.sR = R.s;
    ta.sC = C.s;
    ta.dR = R.d;
    ta.dC = C.d;
    ta.lTR = lg(p.g.TR);
    ta.lTC = lg(p.g.TC);
    ta.tilesR = make_div32(uint32_t((R.e + p.g.TR - 1) / p.g.TR));
    ta.tilesC = make_div32(uint32_t((C.e + p.g.TC - 1) / p.g.TC));
    {
      const uint32_t tR = uint32_t((R.e + p.g.TR - 1) / p.g.TR);
      ta.tilesRg = make_div32(p.g.pad_rows ? (tR + kXcds - 1) / kXcds * kXcds : tR);
    }
    if (p.path == TC_PATH_TRANSPOSE) {
      const bool hasB = p.mode_b >= 0;
      ta.eB = hasB ? j.m[p.mode_b].e : 1;
      ta.sB = hasB ? j.m[p.mode_b].s : 0;
      ta.dB = hasB ? j.m[p.mode_b].d : 0;
      ta.lNB = lg(p.g.NB);
      ta.tilesB = make_div32(uint32_t((ta.eB + p.g.NB - 1) / p.g.NB));
      ta.xshift = p.g.shift;
      ta.xmask = (1 << p.g.k) - 1;
      ta.xtbit = p.g.tbit;
      ta.xcshift = p.g.cshift;
      ta.xcmask = p.g.cmask;
      ta.order = p.g.order;
      fill_batch(p, &ta, p.mode_r, p.mode_c, p.mode_b);
      if (p.g.order == 2) {  // (after fill_batch: the slices count the batch modes)
        const uint32_t sr = 1u << p.g.lsr, sc = 1u << p.g.lsc;
        ta.lsr = p.g.lsr;
        ta.lsc = p.g.lsc;
        const uint32_t stC = (ta.tilesC.d + sc - 1) / sc, stR = (ta.tilesR.d + sr - 1) / sr;
        ta.stC = make_div32(stC);
        ta.nst = stR * stC;
        ta.nslices = ta.tilesB.d;
        for (int k = 0; k < ta.nbatch; ++k) ta.nslices *= ta.bdiv[k].d;
      }
      const int gw = p.nar == 3 ? 4 : 2;  // elements per group of a source read in pairs or groups
      if (p.nar) {
        // the source read in pairs or groups of 4 elements: its offset (of the group holding the
        // first element) and strides (multiples of the group, checked by the planner) in groups;
        // the destination stays in its elements
        ta.src_off = (p.nar == 2 ? ta.src_off - 1 : ta.src_off) / gw;
        ta.sR /= gw;
        ta.sC /= gw;
        ta.sB /= gw;
        for (int k = 0; k < ta.nbatch; ++k) ta.bs[k] /= gw;
      }
      const TransposeCfg cfg = transpose_cfg(p.g);
      if (!launch_transpose(p.nar ? gw * p.eb : p.eb, cfg, &ta, p.workgroups, stream)) {
        *err = "no transpose kernel instance for this element width, vector width, tile size and thread count";
        return TC_E_ARG;
      }
    } else {
      ta.eB = 1;
      ta.lNB = 0;
      ta.tilesB = make_div32(1);
      fill_batch(p, &ta, p.mode_r, p.mode_c, -1);
      const uint32_t g = uint32_t(p.workgroups);
#define TC_G(E) if (p.eb == E) hipLaunchKernelGGL((dev::guarded_tile_kernel<E>), dim3(g), dim3(kGuardThreads), 0, s, ta)
      TC_G(1); TC_G(2); TC_G(4); TC_G(8); TC_G(16);
#undef TC_G
    }
  } else {
    // rows: grid modes in the plan's grid order (rows_grid); the contiguous mode counts vectors
    const Joint jg = rows_grid(p);
    RowArgs ra{};
    ra.src = static_cast<const unsigned char*>(src);
    ra.dst = static_cast<unsigned char*>(dst);
    ra.src_off = jg.so * p.eb;
    ra.dst_off = jg.dof * p.eb;
    const int ve = p.vb / p.eb;
    ra.rank = jg.rank;
    int64_t ext[kMaxRank] = {};
    int64_t total = 1;
    for (int k = 0; k < jg.rank; ++k) {
      const bool inner = (p.path != TC_PATH_GUARDED_ROWS) && k == jg.rank - 1;
      // (element-aligned rows: the last vector of a row may be short)
      ext[k] = inner ? (jg.m[k].e + ve - 1) / ve : jg.m[k].e;
      ra.s[k] = jg.m[k].s * p.eb * (inner ? ve : 1);
      ra.d[k] = jg.m[k].d * p.eb * (inner ? ve : 1);
      total *= ext[k];
    }
    ra.row_elems = jg.rank >= 1 ? jg.m[jg.rank - 1].e : 1;
    // one launch, or (2^31 vectors and more) launches over ranges of the outermost grid mode of
    // at most kLaunchVectors vectors each (the planner has checked that one index fits)
    const int64_t per0 = jg.rank >= 1 ? total / ext[0] : 1;  // vectors per index of mode 0
    const int64_t step0 = total < (int64_t(1) << 31) || jg.rank < 1 ? std::max<int64_t>(ext[0], 1)
                                                                    : std::max<int64_t>(kLaunchVectors / per0, 1);
    for (int64_t i0 = 0; i0 < std::max<int64_t>(ext[0], 1); i0 += step0) {
      RowArgs rc = ra;
      if (jg.rank >= 1) {
        const int64_t n0 = std::min(step0, ext[0] - i0);
        rc.src_off = ra.src_off + i0 * ra.s[0];
        rc.dst_off = ra.dst_off + i0 * ra.d[0];
        for (int k = 0; k < jg.rank; ++k) {
          const int64_t e = k == 0 ? n0 : ext[k];
          rc.ext[k] = uint32_t(e);
          const Div32 dv = make_div32(uint32_t(e));
          rc.mul[k] = dv.mul;
          rc.shr[k] = dv.shr;
        }
        rc.nvec = n0 * per0;
      } else {
        rc.nvec = total;
      }
      rc.sbuf = rc.dbuf = kNoBuffer;
      int64_t slo = 0, dlo = 0;
      bool buf = p.buffers && buffer_window(rc.src_off, rc.ext, rc.s, rc.rank, p.vb, &slo) &&
                 buffer_window(rc.dst_off, rc.ext, rc.d, rc.rank, p.vb, &dlo);
      // element-aligned rows: buffer stores off the 16-byte grid measured 1.3-1.7x slower than
      // global ones (loads were not), so only copies whose destination vectors all sit on it; and
      // only rows without a short last vector (the global instances move it back over its
      // neighbour; with buffer accesses and the tails copied in narrower accesses, rows of 8190
      // int8 elements at pitch 8192 ran at 3.15 against 5.00 TB/s, fp32 3.83 against 6.21)
      if (buf && p.unaligned) {
        buf = (rc.dst_off & 15) == 0 && rc.row_elems % (16 / p.eb) == 0;
        for (int k = 0; k < rc.rank; ++k) buf = buf && (rc.d[k] & 15) == 0;
      }
      if (buf) {
        rc.sbuf = slo;
        rc.dbuf = dlo;
      }
      launch_rows(p, rc, ceil_div(rc.nvec, int64_t(p.threads) * p.row_rounds), s);
      if (hipPeekAtLastError() != hipSuccess) break;
    }
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("kernel launch failed: ") + hipGetErrorString(e);
    return TC_E_HIP;
  }
  return TC_OK;
}

}  // namespace tc
