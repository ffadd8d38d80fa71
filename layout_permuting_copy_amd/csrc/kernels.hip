// Device kernels of the layout-permuting tile copy, for gfx950 (CDNA4, wave64).
//
// transpose_kernel: the source- and destination-contiguous modes differ.  A workgroup of 256
//   lanes moves one 16 KiB tile: global -> registers -> LDS (load phase, 16/8/4-byte vectors
//   along the source-contiguous mode, [outer, threads, vec] split of the tile in source order),
//   s_barrier, LDS -> registers -> global (store phase, the same split of the tile in
//   destination order).  TVM TIRx docs, "copy -> gmem_smem", Algorithm steps 1-3, for the two
//   global<->shared halves; "permute_layout" for the register-staged exchange and its
//   XOR swizzle, which here permutes 16-byte column chunks of the LDS tile by row so that
//   both phases are free of bank conflicts (swizzle chosen on the host by simulating gfx950's
//   LDS banks).  Elements narrower than 4 bytes are grouped in registers first: a BxB
//   micro-transpose (v_perm_b32) turns B rows of a loaded vector into 4-byte column units, so
//   the LDS stage always moves whole dwords.
// rows_kernel: both sides contiguous along one mode; vectors are staged in registers (or, for
//   the round-trip variant, through LDS as in the gmem_smem demonstration program).  Also the
//   guarded element-wise fallback (one element per "vector").
// guarded_tile_kernel: fallback LDS tile with element-wide accesses and per-element guards,
//   for extents or strides that admit no vector (e.g. odd extents, strided slices).
//
// All data moves as unsigned integers: floating point payloads are never touched.
#include <hip/hip_runtime.h>

#include "plan.hpp"

namespace tc {
namespace {

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

// N bytes (N = 4, 8, 16) between memory and N/4 dwords.
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

template <int EB, int VB>
__global__ void __launch_bounds__(kTileThreads) transpose_kernel(TransposeArgs a) {
  constexpr int NT = kTileThreads;
  constexpr int U = EB < 4 ? 4 : EB;         // LDS unit bytes
  constexpr int B = EB < 4 ? 4 / EB : 1;     // rows per unit
  constexpr int VE = VB / EB;                // elements per global vector
  constexpr int LOADS = kTileBytes / (NT * VB * B);
  constexpr int STORES = kTileBytes / (NT * VB);
  constexpr int RPV = VB / U;                // units per store vector
  constexpr int UB = VE * U;                 // LDS bytes written per load access
  constexpr int WW = UB < 16 ? UB : 16;      // LDS write instruction bytes
  constexpr int CW = WW / U;                 // units per write chunk
  constexpr int LB = clog2(B), LVE = clog2(VE), LRPV = clog2(RPV), LCW = clog2(CW);
  static_assert(LOADS >= 1 && STORES >= 1 && RPV >= 1, "tile geometry");

  __shared__ __attribute__((aligned(16))) unsigned char lds[kTileBytes];

  // tile coordinates: column tiles fastest, then row tiles, then batch tiles, then the grid modes
  int64_t idx = blockIdx.x;
  const int64_t tcI = idx % a.tilesC;
  idx /= a.tilesC;
  const int64_t trI = idx % a.tilesR;
  idx /= a.tilesR;
  const int64_t tbI = idx % a.tilesB;
  idx /= a.tilesB;
  int64_t sbase = a.src_off, dbase = a.dst_off;
  for (int k = a.nbatch - 1; k >= 0; --k) {
    const int64_t i = idx % a.bext[k];
    idx /= a.bext[k];
    sbase += i * a.bs[k];
    dbase += i * a.bd[k];
  }
  const int64_t r0 = trI << a.lTR, c0 = tcI << a.lTC, b0 = tbI << a.lNB;
  sbase += r0 * a.sR + c0 + b0 * a.sB;
  dbase += r0 + c0 * a.dC + b0 * a.dB;
  const int64_t remR = a.eR - r0, remC = a.eC - c0, remB = a.eB - b0;
  const int lTRu = a.lTR - LB;
  const int TRu = 1 << lTRu, TC = 1 << a.lTC, NB = 1 << a.lNB;
  const int lnCV = a.lTC - LVE;  // load vectors per unit-row
  const int lnRV = lTRu - LRPV;  // store vectors per column
  const int xmask = a.xmask, xshift = a.xshift, xtbit = a.xtbit, xcshift = a.xcshift, xcmask = a.xcmask;
  const int t = threadIdx.x;
  const unsigned char* __restrict__ src = a.src;
  unsigned char* __restrict__ dst = a.dst;

  // ---- load phase: global -> registers -> LDS ------------------------------------------
  uint32_t reg[LOADS][B][VB / 4] = {};
#pragma unroll
  for (int f = 0; f < LOADS; ++f) {
    const int acc = f * NT + t;
    const int cv = acc & ((1 << lnCV) - 1);
    const int ru = (acc >> lnCV) & (TRu - 1);
    const int nb = acc >> (lnCV + lTRu);
    const bool ok = nb < NB && nb < remB && (int64_t(ru) << LB) < remR && (int64_t(cv) << LVE) < remC;
    if (ok) {
      const unsigned char* p = src + (sbase + nb * a.sB + (int64_t(ru) << LB) * a.sR + (cv << LVE)) * EB;
#pragma unroll
      for (int i = 0; i < B; ++i) load_words<VB>(p + i * a.sR * EB, reg[f][i]);
    }
  }
#pragma unroll
  for (int f = 0; f < LOADS; ++f) {
    const int acc = f * NT + t;
    const int cv = acc & ((1 << lnCV) - 1);
    const int ru = (acc >> lnCV) & (TRu - 1);
    const int nb = acc >> (lnCV + lTRu);
    // the VE units of this access, as dwords (U/4 per unit)
    uint32_t unit[UB / 4];
    if constexpr (EB >= 4) {
#pragma unroll
      for (int w = 0; w < VB / 4; ++w) unit[w] = reg[f][0][w];
    } else if constexpr (EB == 2) {
#pragma unroll
      for (int w = 0; w < VB / 4; ++w) {
        unit[2 * w] = perm(reg[f][1][w], reg[f][0][w], 0x05040100u);
        unit[2 * w + 1] = perm(reg[f][1][w], reg[f][0][w], 0x07060302u);
      }
    } else {
#pragma unroll
      for (int w = 0; w < VB / 4; ++w) {
        const uint32_t p01 = perm(reg[f][1][w], reg[f][0][w], 0x05010400u);
        const uint32_t q01 = perm(reg[f][1][w], reg[f][0][w], 0x07030602u);
        const uint32_t p23 = perm(reg[f][3][w], reg[f][2][w], 0x05010400u);
        const uint32_t q23 = perm(reg[f][3][w], reg[f][2][w], 0x07030602u);
        unit[4 * w] = perm(p23, p01, 0x05040100u);
        unit[4 * w + 1] = perm(p23, p01, 0x07060302u);
        unit[4 * w + 2] = perm(q23, q01, 0x05040100u);
        unit[4 * w + 3] = perm(q23, q01, 0x07060302u);
      }
    }
    const int xr = ((ru >> xshift) & xmask) << xtbit;
    const int row = (nb << lTRu) + ru;
#pragma unroll
    for (int q = 0; q < UB / WW; ++q) {
      const int ch = ((cv << LVE) >> LCW) + q;
      const int chs = ch ^ xr ^ ((ch >> xcshift) & xcmask);
      const int off = ((row << a.lTC) + (chs << LCW)) * U;
      store_words<WW>(lds + off, unit + q * (WW / 4));
    }
  }
  __syncthreads();

  // ---- store phase: LDS -> registers -> global -------------------------------------------
#pragma unroll
  for (int f = 0; f < STORES; ++f) {
    const int acc = f * NT + t;
    const int rv = acc & ((1 << lnRV) - 1);
    const int c = (acc >> lnRV) & (TC - 1);
    const int nb = acc >> (lnRV + a.lTC);
    const bool ok = nb < NB && nb < remB && (int64_t(rv) << (LRPV + LB)) < remR && c < remC;
    uint32_t out[VB / 4];
    const int ch = c >> LCW, cin = c & (CW - 1);
#pragma unroll
    for (int v = 0; v < RPV; ++v) {
      const int ru = (rv << LRPV) + v;
      const int xr = ((ru >> xshift) & xmask) << xtbit;
      const int chs = ch ^ xr ^ ((ch >> xcshift) & xcmask);
      const int off = ((((nb << lTRu) + ru) << a.lTC) + (chs << LCW) + cin) * U;
      load_words<U>(lds + off, out + v * (U / 4));
    }
    if (ok) {
      unsigned char* p = dst + (dbase + nb * a.dB + int64_t(c) * a.dC + (int64_t(rv) << (LRPV + LB))) * EB;
      store_words<VB>(p, out);
    }
  }
}

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
// vectors make the round trip global -> LDS -> global of the gmem_smem demonstration.
template <int VB, int NT, int ROUNDS, bool USE_LDS>
__global__ void __launch_bounds__(NT) rows_kernel(RowArgs a) {
  typedef typename Bytes<VB>::T V;
  __shared__ __attribute__((aligned(16))) V lds[USE_LDS ? NT * ROUNDS : 1];
  const int t = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * NT * ROUNDS;
  V reg[ROUNDS];
  int64_t doff[ROUNDS];
#pragma unroll
  for (int f = 0; f < ROUNDS; ++f) {
    const int64_t v = base + f * NT + t;
    doff[f] = -1;
    if (v < a.nvec) {
      int64_t so, dof;
      row_offsets(a, uint32_t(v), &so, &dof);
      reg[f] = *reinterpret_cast<const V*>(a.src + so);
      doff[f] = dof;
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
  for (int f = 0; f < ROUNDS; ++f)
    if (doff[f] >= 0) *reinterpret_cast<V*>(a.dst + doff[f]) = reg[f];
}

// Fallback tile: element-wide accesses, padded LDS rows, guards on every element.
template <int EB>
__global__ void __launch_bounds__(kTileThreads) guarded_tile_kernel(TransposeArgs a) {
  typedef typename Bytes<EB>::T V;
  constexpr int NT = kTileThreads;
  constexpr int PAD = EB < 4 ? 4 / EB : 1;
  constexpr int TRC = EB <= 4 ? 64 * 64 : (EB == 8 ? 32 * 64 : 32 * 32);
  constexpr int ROWS = EB <= 8 ? (EB <= 4 ? 64 : 32) : 32;
  constexpr int COLS = TRC / ROWS;
  constexpr int PITCH = COLS + PAD;
  __shared__ V lds[ROWS * PITCH];
  int64_t idx = blockIdx.x;
  const int64_t tcI = idx % a.tilesC;
  idx /= a.tilesC;
  const int64_t trI = idx % a.tilesR;
  idx /= a.tilesR;
  int64_t sbase = a.src_off, dbase = a.dst_off;
  for (int k = a.nbatch - 1; k >= 0; --k) {
    const int64_t i = idx % a.bext[k];
    idx /= a.bext[k];
    sbase += i * a.bs[k];
    dbase += i * a.bd[k];
  }
  const int64_t r0 = trI * ROWS, c0 = tcI * COLS;
  sbase += r0 * a.sR + c0 * a.sC;
  dbase += r0 * a.dR + c0 * a.dC;
  const int64_t remR = a.eR - r0, remC = a.eC - c0;
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

// ---- host side ---------------------------------------------------------------------------------

void make_divider(uint32_t d, uint32_t* mul, uint32_t* shr) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  *shr = s;
  *mul = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
}

void fill_batch(const Plan& p, TransposeArgs* ta, int skip0, int skip1, int skip2) {
  ta->nbatch = 0;
  for (int k = 0; k < p.j.rank; ++k) {
    if (k == skip0 || k == skip1 || k == skip2) continue;
    ta->bext[ta->nbatch] = p.j.m[k].e;
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

template <int EB, int VB>
void launch_transpose_t(const TransposeArgs& ta, int64_t wgs, hipStream_t s) {
  hipLaunchKernelGGL((transpose_kernel<EB, VB>), dim3(uint32_t(wgs)), dim3(kTileThreads), 0, s, ta);
}

void launch_transpose(const Plan& p, const TransposeArgs& ta, hipStream_t s) {
  const int eb = p.eb, vb = p.vb;
#define TC_T(E, V) if (eb == E && vb == V) return launch_transpose_t<E, V>(ta, p.workgroups, s)
  TC_T(1, 16); TC_T(1, 8); TC_T(1, 4);
  TC_T(2, 16); TC_T(2, 8); TC_T(2, 4);
  TC_T(4, 16); TC_T(4, 8); TC_T(4, 4);
  TC_T(8, 16); TC_T(8, 8);
  TC_T(16, 16);
#undef TC_T
}

template <int VB, int NT, bool LDS>
void launch_rows_t(const RowArgs& ra, int64_t wgs, hipStream_t s) {
  hipLaunchKernelGGL((rows_kernel<VB, NT, kRowRounds, LDS>), dim3(uint32_t(wgs)), dim3(NT), 0, s, ra);
}

}  // namespace

int launch_plan(const Plan& p, const void* src, void* dst, void* stream, std::string* err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.path == TC_PATH_EMPTY) return TC_OK;
  const Joint& j = p.j;
  if (p.path == TC_PATH_TRANSPOSE || p.path == TC_PATH_GUARDED_TILE) {
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
    if (p.path == TC_PATH_TRANSPOSE) {
      const bool hasB = p.mode_b >= 0;
      ta.eB = hasB ? j.m[p.mode_b].e : 1;
      ta.sB = hasB ? j.m[p.mode_b].s : 0;
      ta.dB = hasB ? j.m[p.mode_b].d : 0;
      ta.lTR = lg(p.g.TR);
      ta.lTC = lg(p.g.TC);
      ta.lNB = lg(p.g.NB);
      ta.tilesR = (R.e + p.g.TR - 1) / p.g.TR;
      ta.tilesC = (C.e + p.g.TC - 1) / p.g.TC;
      ta.tilesB = (ta.eB + p.g.NB - 1) / p.g.NB;
      ta.xshift = p.g.shift;
      ta.xmask = (1 << p.g.k) - 1;
      ta.xtbit = p.g.tbit;
      ta.xcshift = p.g.cshift;
      ta.xcmask = p.g.cmask;
      fill_batch(p, &ta, p.mode_r, p.mode_c, p.mode_b);
      launch_transpose(p, ta, s);
    } else {
      ta.eB = 1;
      ta.tilesR = (R.e + p.g.TR - 1) / p.g.TR;
      ta.tilesC = (C.e + p.g.TC - 1) / p.g.TC;
      ta.tilesB = 1;
      fill_batch(p, &ta, p.mode_r, p.mode_c, -1);
      const uint32_t g = uint32_t(p.workgroups);
#define TC_G(E) if (p.eb == E) hipLaunchKernelGGL((guarded_tile_kernel<E>), dim3(g), dim3(kTileThreads), 0, s, ta)
      TC_G(1); TC_G(2); TC_G(4); TC_G(8); TC_G(16);
#undef TC_G
    }
  } else {
    // rows: grid modes in canonical (destination) order; the contiguous mode counts vectors
    RowArgs ra{};
    ra.src = static_cast<const unsigned char*>(src);
    ra.dst = static_cast<unsigned char*>(dst);
    ra.src_off = j.so * p.eb;
    ra.dst_off = j.dof * p.eb;
    const int ve = p.vb / p.eb;
    ra.rank = j.rank;
    for (int k = 0; k < j.rank; ++k) {
      const bool inner = (p.path != TC_PATH_GUARDED_ROWS) && k == j.rank - 1;
      const int64_t e = inner ? j.m[k].e / ve : j.m[k].e;
      ra.ext[k] = uint32_t(e);
      make_divider(uint32_t(e), &ra.mul[k], &ra.shr[k]);
      ra.s[k] = j.m[k].s * p.eb * (inner ? ve : 1);
      ra.d[k] = j.m[k].d * p.eb * (inner ? ve : 1);
    }
    ra.nvec = j.count / (p.path == TC_PATH_GUARDED_ROWS ? 1 : ve);
    const int64_t wgs = p.workgroups;
    if (p.path == TC_PATH_ROUNDTRIP) {
      if (p.vb == 16) launch_rows_t<16, kWave, true>(ra, wgs, s);
      if (p.vb == 8) launch_rows_t<8, kWave, true>(ra, wgs, s);
      if (p.vb == 4) launch_rows_t<4, kWave, true>(ra, wgs, s);
    } else if (p.path == TC_PATH_ROWS) {
      if (p.vb == 16) launch_rows_t<16, kTileThreads, false>(ra, wgs, s);
      if (p.vb == 8) launch_rows_t<8, kTileThreads, false>(ra, wgs, s);
      if (p.vb == 4) launch_rows_t<4, kTileThreads, false>(ra, wgs, s);
    } else {
      if (p.eb == 1) launch_rows_t<1, kTileThreads, false>(ra, wgs, s);
      if (p.eb == 2) launch_rows_t<2, kTileThreads, false>(ra, wgs, s);
      if (p.eb == 4) launch_rows_t<4, kTileThreads, false>(ra, wgs, s);
      if (p.eb == 8) launch_rows_t<8, kTileThreads, false>(ra, wgs, s);
      if (p.eb == 16) launch_rows_t<16, kTileThreads, false>(ra, wgs, s);
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
