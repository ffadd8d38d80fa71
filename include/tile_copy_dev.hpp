/*
 * tile_copy_dev.hpp -- device-side tile primitives for gfx950 (wave64), header-only HIP.
 *
 * The same operations the host library runs as whole kernels, as functions a kernel calls on
 * its own tiles:
 *
 *   tcd::copy<Scope, Drive, DstLayout, SrcLayout>(dst, src)
 *       Copy between two memories (global <-> LDS, or LDS <-> LDS) executed by every lane of a
 *       scope: one lane, one wave64, W waves, or a workgroup.  TVM TIRx docs, "copy ->
 *       gmem_smem", Algorithms 1-3: both layouts are sliced (the caller passes the region's
 *       layout), the driving (global) side orders the modes by descending stride, modes that are
 *       contiguous on both sides merge, a vector of 16, 8 or 4 bytes (else one element) is carved
 *       from the innermost mode, and the flat index is split [outer, threads, vec] with the
 *       TileLang mapping (tutorial "loop_mapping.py": access = flat / vec, thread = access %
 *       threads, round = access / threads).  An LDS-side layout may carry an XOR swizzle; the
 *       vector then never exceeds one swizzle chunk (gmem_smem, "What it accepts" and the
 *       closing remarks on swizzled shared layouts).  When the element count is not a multiple
 *       of threads x vec the last round is guarded (the TileLang guard on idle threads);
 *       tcd::copy_plan<...>::exact says whether it is.
 *
 *   tcd::wave_permute<DstLayout, SrcLayout>(dst, src, k, shift)
 *       The register-staged permute of an LDS tile by one wave64 (TVM TIRx docs,
 *       "permute_layout", Algorithm steps 1 and 3): both layouts keep their logical mode order
 *       (the source is regrouped onto the destination's shard), P = count / 64 elements per
 *       lane; at step r lane l handles flat index l + 64 * (r ^ ((l >> shift) & (2^k - 1))),
 *       reads all P through the source layout into registers, orders the wave's LDS accesses,
 *       then writes them through the destination layout.  dst and src may be the same buffer
 *       (alias-safe).  k and shift come from tc_wave_permute_plan (tile_copy.h), which
 *       simulates gfx950's LDS banks for both phases and picks the smallest conflict-free k.
 *       Any other k and shift stay in bounds: the XOR mask is cut to P - 1 (to 0 when P is not a
 *       power of two) and the shift to 0..6, so every step still touches only the tile.
 *
 * Layouts are compile-time types: tcd::layout<tcd::ints<extents...>, tcd::ints<strides...>,
 * offset, swizzle>, in elements.  Pointers are typed by the element (1, 2, 4, 8 or 16 bytes;
 * tcd::b128 for 16).  Both base pointers must be 16-byte aligned (the vector chooser assumes it);
 * LDS pointers are __shared__ arrays or pointers derived from them.
 *
 * Ownership and ordering: the primitives own no memory.  A copy or permute leaves the caller's
 * data ordered for the lanes that wrote it; before other lanes read it the caller orders the
 * scope (Scope::sync(), or wave_permute's own ordering, which it performs before it returns).
 */
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tcd {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

/* A 16-byte element (e.g. a struct of four 32-bit ints). */
struct alignas(16) b128 {
  uint32_t w[4];
};

/* ---- compile-time integer lists and layouts ------------------------------------------------ */

template <int... V>
struct ints {
  static constexpr int size = sizeof...(V);
  static constexpr int v[sizeof...(V) > 0 ? sizeof...(V) : 1] = {V...};
};

/* No swizzle. */
struct no_swizzle {
  static constexpr int chunk = 1 << 30;  // elements: no cap on the vector
  static constexpr bool active = false;
  __host__ __device__ static constexpr int apply(int off) { return off; }
};

/* XOR swizzle on element offsets: bits [BASE, BASE + BITS) are XORed with bits
 * [BASE + SHIFT, BASE + SHIFT + BITS).  A chunk is 2^BASE consecutive elements, which the
 * swizzle keeps together (e.g. BASE = 3 with 2-byte elements: 16-byte chunks, and the chunk
 * index within a row XORed with the row index when SHIFT = log2(row length / 8)). */
template <int BITS, int BASE, int SHIFT>
struct xor_swizzle {
  static_assert(BITS >= 0 && BASE >= 0 && SHIFT >= BITS, "xor_swizzle: SHIFT must be >= BITS");
  static constexpr int chunk = 1 << BASE;
  static constexpr bool active = BITS > 0;
  __host__ __device__ static constexpr int apply(int off) {
    return off ^ (((off >> (BASE + SHIFT)) & ((1 << BITS) - 1)) << BASE);
  }
};

template <class Shape, class Stride, int Offset = 0, class Swizzle = no_swizzle>
struct layout {
  static_assert(Shape::size == Stride::size, "layout: shape and stride ranks differ");
  static_assert(Shape::size <= 8, "layout: rank above 8");
  using shape = Shape;
  using stride = Stride;
  using swizzle = Swizzle;
  static constexpr int rank = Shape::size;
  static constexpr int offset = Offset;
};

/* ---- scopes ------------------------------------------------------------------------------- */

/* One lane does the whole copy. */
struct lane_scope {
  static constexpr int threads = 1;
  __device__ static int rank() { return 0; }
  __device__ static void sync() {}
};

/* Orders one wave's LDS writes before its later LDS reads (other lanes' data included): a wave's
 * LDS operations execute in issue order; the fences keep the compiler from moving accesses
 * across this point. */
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

/* W consecutive waves of a 1-D workgroup (W = 1: one wave64).  Lane rank = threadIdx.x modulo
 * 64 W, so several groups in one workgroup each work on their own tile.  sync() with W > 1 is the
 * workgroup barrier: every wave of the workgroup must reach it. */
template <int W>
struct waves_scope {
  static_assert(W >= 1, "waves_scope: at least one wave");
  static constexpr int threads = 64 * W;
  __device__ static int rank() { return int(threadIdx.x) % threads; }
  __device__ static void sync() {
    if constexpr (W == 1) wave_sync();
    else __syncthreads();
  }
};
using wave_scope = waves_scope<1>;

/* The whole 1-D workgroup of NT lanes. */
template <int NT>
struct workgroup_scope {
  static constexpr int threads = NT;
  __device__ static int rank() { return int(threadIdx.x); }
  __device__ static void sync() { __syncthreads(); }
};

/* Which side orders the modes (the global side of a global <-> LDS copy). */
enum class drive { src, dst };

/* ---- plans (compile time) ----------------------------------------------------------------- */

namespace detail {

struct modes {
  int n = 0;
  int e[8] = {};  // extents
  int s[8] = {};  // source strides
  int d[8] = {};  // destination strides
  int count = 1;
  bool ok = true;  // equal non-unit extents on both sides
};

/* Joint modes of two layouts: their non-unit modes, which must have equal extents in order. */
template <class Dst, class Src>
constexpr modes joint() {
  modes m;
  int ds[8] = {}, de[8] = {}, nd = 0;
  for (int k = 0; k < Dst::rank; ++k)
    if (Dst::shape::v[k] != 1) { de[nd] = Dst::shape::v[k]; ds[nd] = Dst::stride::v[k]; ++nd; }
  for (int k = 0; k < Src::rank; ++k)
    if (Src::shape::v[k] != 1) {
      if (m.n >= nd || de[m.n] != Src::shape::v[k]) m.ok = false;
      if (m.n < 8) {
        m.e[m.n] = Src::shape::v[k];
        m.s[m.n] = Src::stride::v[k];
        m.d[m.n] = m.n < nd ? ds[m.n] : 0;
      }
      ++m.n;
    }
  if (m.n != nd) m.ok = false;
  for (int k = 0; k < m.n; ++k) m.count *= m.e[k];
  return m;
}

constexpr int iabs(int x) { return x < 0 ? -x : x; }

/* Merge neighbours (outer o, inner i) that are contiguous on both sides:
 * s_o == e_i * s_i and d_o == e_i * d_i. */
constexpr modes merge(modes m) {
  modes out = m;
  out.n = 0;
  for (int k = 0; k < m.n; ++k) {
    if (out.n > 0) {
      const int p = out.n - 1;
      if (out.s[p] == m.e[k] * m.s[k] && out.d[p] == m.e[k] * m.d[k]) {
        out.e[p] *= m.e[k];
        out.s[p] = m.s[k];
        out.d[p] = m.d[k];
        continue;
      }
    }
    out.e[out.n] = m.e[k];
    out.s[out.n] = m.s[k];
    out.d[out.n] = m.d[k];
    ++out.n;
  }
  return out;
}

/* Stable order by the driving side's stride, largest first (innermost mode last). */
constexpr modes sort_by(modes m, bool by_src) {
  for (int i = 1; i < m.n; ++i)
    for (int j = i; j > 0; --j) {
      const int a = iabs(by_src ? m.s[j - 1] : m.d[j - 1]), b = iabs(by_src ? m.s[j] : m.d[j]);
      if (a >= b) break;
      const int te = m.e[j], ts = m.s[j], td = m.d[j];
      m.e[j] = m.e[j - 1]; m.s[j] = m.s[j - 1]; m.d[j] = m.d[j - 1];
      m.e[j - 1] = te; m.s[j - 1] = ts; m.d[j - 1] = td;
    }
  return m;
}

struct copy_plan_t {
  modes m;
  int vec = 1;    // elements per access
  int outer = 0;  // rounds per lane
  bool exact = true;
};

/* The [outer, threads, vec] split: the widest of 16, 8, 4 bytes (>= the element, <= one swizzle
 * chunk on either side) whose vector lies inside the innermost mode on both sides (stride 1 there,
 * extent a multiple) with every other stride and both offsets multiples of it, and which divides
 * the element count by threads x vec (gmem_smem, Algorithm 2 and "What it accepts"); else one
 * element per access. */
constexpr copy_plan_t make_copy_plan(modes m, int eb, int threads, int soff, int doff, int chunk) {
  copy_plan_t p;
  p.m = m;
  for (int bytes = 16; bytes >= 4; bytes /= 2) {
    if (bytes < eb || bytes % eb) continue;
    const int v = bytes / eb;
    if (v > chunk || m.n == 0) continue;
    const int in = m.n - 1;
    bool ok = m.s[in] == 1 && m.d[in] == 1 && m.e[in] % v == 0 && soff % v == 0 && doff % v == 0;
    for (int k = 0; k < in; ++k) ok = ok && m.s[k] % v == 0 && m.d[k] % v == 0;
    ok = ok && m.count % (threads * v) == 0;
    if (ok) { p.vec = v; break; }
  }
  const int per_round = threads * p.vec;
  p.outer = (m.count + per_round - 1) / per_round;
  p.exact = m.count % per_round == 0;
  return p;
}

/* Element offset of row-major position `flat` of the joint modes on one side (innermost last). */
constexpr int side_offset(const modes& m, int flat, bool src, int base) {
  int off = base;
  for (int k = m.n - 1; k >= 0; --k) {
    const int i = flat % m.e[k];
    flat /= m.e[k];
    off += i * (src ? m.s[k] : m.d[k]);
  }
  return off;
}

/* Recognised rounds: for every lane t and round f of the split, the (swizzled) offsets on both
 * sides are those of round 0 plus a per-round constant, i.e.
 *     swz(off(f * NT * V + t * V)) == swz(off(t * V)) + delta[f].
 * Then a lane decomposes and swizzles its first access once and every later round is an add of
 * a compile-time constant (TVM TIRx docs, "copy -> gmem_smem", "How inputs change the
 * algorithm": a recognised swizzle becomes a few register adds per round, otherwise the swizzle
 * is applied every round).  This holds, for example, when a round covers whole periods of an XOR
 * swizzle (2^(BASE + SHIFT + BITS) elements) and whole rows of both layouts.  Checked
 * exhaustively at compile time for splits of at most kAffineChecks accesses (else: not
 * recognised, the general path runs). */
constexpr int kMaxAffineRounds = 64;
constexpr int kAffineChecks = 16384;
struct round_deltas {
  bool ok = false;
  int s[kMaxAffineRounds] = {};
  int d[kMaxAffineRounds] = {};
};

template <class SrcSwz, class DstSwz>
constexpr round_deltas affine_rounds(const copy_plan_t& p, int threads, int soff, int doff) {
  round_deltas r;
  if (p.outer > kMaxAffineRounds || p.outer * threads > kAffineChecks) return r;
  const int step = threads * p.vec;
  for (int f = 0; f < p.outer; ++f) {
    r.s[f] = SrcSwz::apply(side_offset(p.m, f * step, true, soff)) - SrcSwz::apply(side_offset(p.m, 0, true, soff));
    r.d[f] = DstSwz::apply(side_offset(p.m, f * step, false, doff)) - DstSwz::apply(side_offset(p.m, 0, false, doff));
  }
  for (int t = 0; t < threads; ++t) {
    if (t * p.vec >= p.m.count) break;
    const int s0 = SrcSwz::apply(side_offset(p.m, t * p.vec, true, soff));
    const int d0 = DstSwz::apply(side_offset(p.m, t * p.vec, false, doff));
    for (int f = 1; f < p.outer; ++f) {
      const int flat = f * step + t * p.vec;
      if (flat >= p.m.count) break;
      if (SrcSwz::apply(side_offset(p.m, flat, true, soff)) != s0 + r.s[f] ||
          DstSwz::apply(side_offset(p.m, flat, false, doff)) != d0 + r.d[f])
        return round_deltas{};
    }
  }
  r.ok = true;
  return r;
}

template <int N>
struct bytes_t;
template <> struct bytes_t<1> { typedef uint8_t t; };
template <> struct bytes_t<2> { typedef uint16_t t; };
template <> struct bytes_t<4> { typedef uint32_t t; };
template <> struct bytes_t<8> { typedef u32x2 t; };
template <> struct bytes_t<16> { typedef u32x4 t; };

}  // namespace detail

/* The copy plan of a scope and two layouts, at compile time. */
template <class Scope, drive Drive, class Dst, class Src, typename T>
struct copy_plan {
  static constexpr detail::modes joint = detail::joint<Dst, Src>();
  static_assert(joint.ok, "tcd::copy: the layouts' non-unit extents differ");
  static constexpr int chunk = Dst::swizzle::chunk < Src::swizzle::chunk ? Dst::swizzle::chunk : Src::swizzle::chunk;
  static constexpr detail::copy_plan_t plan = detail::make_copy_plan(
      detail::merge(detail::sort_by(joint, Drive == drive::src)), int(sizeof(T)), Scope::threads, Src::offset,
      Dst::offset, chunk);
  static constexpr int vec = plan.vec;
  static constexpr int outer = plan.outer;
  static constexpr bool exact = plan.exact;
  static constexpr int count = joint.count;
  /* Recognised rounds (see detail::affine_rounds): per-round offsets are compile-time adds. */
  static constexpr detail::round_deltas rounds =
      detail::affine_rounds<typename Src::swizzle, typename Dst::swizzle>(plan, Scope::threads, Src::offset,
                                                                          Dst::offset);
  static constexpr bool lowered = rounds.ok;
};

/* ---- copy ----------------------------------------------------------------------------------- */

namespace detail {
/* The general rounds: every round decomposes its access index and applies both swizzles. */
template <class Scope, drive Drive, class Dst, class Src, typename T>
__device__ __forceinline__ void copy_general(T* __restrict__ dst, const T* __restrict__ src) {
  using P = copy_plan<Scope, Drive, Dst, Src, T>;
  constexpr copy_plan_t plan = P::plan;
  constexpr int V = plan.vec, NT = Scope::threads;
  typedef typename bytes_t<V * sizeof(T) <= 16 ? V * sizeof(T) : 16>::t vec_t;
  const int t = Scope::rank();
#pragma unroll
  for (int f = 0; f < plan.outer; ++f) {
    const int flat = (f * NT + t) * V;  // access index f * NT + t, then the vector's first element
    if (!plan.exact && flat >= plan.m.count) break;
    int rem = flat, so = Src::offset, d_o = Dst::offset;
#pragma unroll
    for (int k = plan.m.n - 1; k >= 0; --k) {
      const int i = rem % plan.m.e[k];
      rem /= plan.m.e[k];
      so += i * plan.m.s[k];
      d_o += i * plan.m.d[k];
    }
    so = Src::swizzle::apply(so);
    d_o = Dst::swizzle::apply(d_o);
    *reinterpret_cast<vec_t*>(dst + d_o) = *reinterpret_cast<const vec_t*>(src + so);
  }
}
}  // namespace detail

template <class Scope, drive Drive, class Dst, class Src, typename T>
__device__ __forceinline__ void copy(T* __restrict__ dst, const T* __restrict__ src) {
  using P = copy_plan<Scope, Drive, Dst, Src, T>;
  constexpr detail::copy_plan_t plan = P::plan;
  constexpr int V = plan.vec, NT = Scope::threads;
  static_assert(sizeof(T) == 1 || sizeof(T) == 2 || sizeof(T) == 4 || sizeof(T) == 8 || sizeof(T) == 16,
                "tcd::copy: element of 1, 2, 4, 8 or 16 bytes");
  if constexpr (P::lowered) {
    typedef typename detail::bytes_t<V * sizeof(T) <= 16 ? V * sizeof(T) : 16>::t vec_t;
    const int t = Scope::rank();
    // round 0 decomposed and swizzled once; later rounds add compile-time constants
    const int s0 = Src::swizzle::apply(detail::side_offset(plan.m, t * V, true, Src::offset));
    const int d0 = Dst::swizzle::apply(detail::side_offset(plan.m, t * V, false, Dst::offset));
#pragma unroll
    for (int f = 0; f < plan.outer; ++f) {
      if (!plan.exact && (f * NT + t) * V >= plan.m.count) break;
      *reinterpret_cast<vec_t*>(dst + d0 + P::rounds.d[f]) = *reinterpret_cast<const vec_t*>(src + s0 + P::rounds.s[f]);
    }
  } else {
    detail::copy_general<Scope, Drive, Dst, Src, T>(dst, src);
  }
}

/* Global -> LDS (the global side orders the modes) and LDS -> global. */
template <class Scope, class LdsL, class GL, typename T>
__device__ __forceinline__ void g2s(T* lds, const T* g) {
  copy<Scope, drive::src, LdsL, GL, T>(lds, g);
}
template <class Scope, class GL, class LdsL, typename T>
__device__ __forceinline__ void s2g(T* g, const T* lds) {
  copy<Scope, drive::dst, GL, LdsL, T>(g, lds);
}

/* ---- wave permute ------------------------------------------------------------------------- */

template <class Dst, class Src, typename T>
struct permute_plan {
  static constexpr detail::modes m = detail::merge(detail::joint<Dst, Src>());
  static_assert(detail::joint<Dst, Src>().ok, "tcd::wave_permute: the layouts' non-unit extents differ");
  static_assert(m.count % 64 == 0, "tcd::wave_permute: the element count must be a multiple of 64");
  static constexpr int P = m.count / 64;  // elements per lane
};

template <class Dst, class Src, typename T>
__device__ __forceinline__ void wave_permute(T* dst, const T* src, int k, int shift) {
  using PP = permute_plan<Dst, Src, T>;
  constexpr detail::modes m = PP::m;
  constexpr int P = PP::P;
  const int lane = int(threadIdx.x) & 63;
  // An XOR of k bits permutes the steps [0, P) only when P is a power of two and 2^k <= P: the
  // mask is cut to P - 1 there and to 0 otherwise (k = 0), and the shift to the lane bits, so
  // that j stays in [0, P) for any k and shift a caller passes.
  constexpr bool kPow2 = (P & (P - 1)) == 0;
  const int kk = k < 0 ? 0 : (k > 30 ? 30 : k);
  const int mask = kPow2 ? (((1 << kk) - 1) & (P - 1)) : 0;
  shift = shift < 0 ? 0 : (shift > 6 ? 6 : shift);
  T regs[P];
  int doff[P];
#pragma unroll
  for (int r = 0; r < P; ++r) {
    const int j = r ^ ((lane >> shift) & mask);
    int rem = lane + j * 64, so = Src::offset, d_o = Dst::offset;
#pragma unroll
    for (int q = m.n - 1; q >= 0; --q) {
      const int i = rem % m.e[q];
      rem /= m.e[q];
      so += i * m.s[q];
      d_o += i * m.d[q];
    }
    regs[r] = src[Src::swizzle::apply(so)];
    doff[r] = Dst::swizzle::apply(d_o);
  }
  wave_sync();
#pragma unroll
  for (int r = 0; r < P; ++r) dst[doff[r]] = regs[r];
  wave_sync();
}

}  // namespace tcd
