// Example kernels built on the device primitives of tile_copy_dev.hpp, exported through a small
// C ABI (libtile_copy_dev.so) so that host code and tests can run them.  Each is a complete use
// of one scope: the kernels below are the primitives' reference users, not a second copy path.
#include <hip/hip_runtime.h>

#include "tile_copy_dev.hpp"

namespace {

using tcd::ints;
using tcd::layout;

// 32 x 32 fp32, identity layouts, one wave64: global -> LDS -> global (TVM TIRx docs, "copy ->
// gmem_smem", demonstration program: the two copies with a barrier between them).
using L32 = layout<ints<32, 32>, ints<32, 1>>;

__global__ void __launch_bounds__(64) roundtrip32(const float* __restrict__ src, float* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) float s[32 * 32];
  tcd::g2s<tcd::wave_scope, L32, L32>(s, src);
  tcd::wave_scope::sync();
  tcd::s2g<tcd::wave_scope, L32, L32>(dst, s);
}

// In-place LDS permute by one wave (TVM TIRx docs, "permute_layout"), one tile per wave, four
// waves per workgroup: load the tile (identity), permute it in LDS, store it (identity).
//   which = 0: the scale-factor tile (2,1,4,32): strides (128,128,32,1) -> (128,128,1,4)
//   which = 1: a 4 x 64 transpose: (4,64):(64,1) -> (4,64):(1,4)
using SFLin = layout<ints<256>, ints<1>>;
using SFSrc = layout<ints<2, 1, 4, 32>, ints<128, 128, 32, 1>>;
using SFDst = layout<ints<2, 1, 4, 32>, ints<128, 128, 1, 4>>;
using T4Src = layout<ints<4, 64>, ints<64, 1>>;
using T4Dst = layout<ints<4, 64>, ints<1, 4>>;

template <int WHICH>
__global__ void __launch_bounds__(256) permute_tiles(const float* __restrict__ src, float* __restrict__ dst, int ntiles,
                                                     int k, int shift) {
  __shared__ __attribute__((aligned(16))) float s[4 * 256];
  const int w = int(threadIdx.x) / 64;
  const int tile = int(blockIdx.x) * 4 + w;
  if (tile >= ntiles) return;  // whole waves leave: the permute's ordering is per wave
  float* t = s + w * 256;
  tcd::g2s<tcd::wave_scope, SFLin, SFLin>(t, src + int64_t(tile) * 256);
  tcd::wave_sync();
  if constexpr (WHICH == 0) tcd::wave_permute<SFDst, SFSrc>(t, t, k, shift);
  else tcd::wave_permute<T4Dst, T4Src>(t, t, k, shift);
  tcd::s2g<tcd::wave_scope, SFLin, SFLin>(dst + int64_t(tile) * 256, t);
}

// 64 x 64 bf16 tiles of an n x m row-major matrix (pitch ld_src), one workgroup of 256 lanes per
// tile: global -> LDS into an XOR-swizzled layout (16-byte chunks, chunk index ^= row % 8), a raw
// dump of the LDS tile, then LDS -> global transposed (destination column-major, pitch ld_dst).
using SwzT = layout<ints<64, 64>, ints<64, 1>, 0, tcd::xor_swizzle<3, 3, 3>>;
using Lin4096 = layout<ints<4096>, ints<1>>;

template <int LD_SRC, int LD_DST>
struct SwzGlobal {
  using src = layout<ints<64, 64>, ints<LD_SRC, 1>>;
  using dst = layout<ints<64, 64>, ints<1, LD_DST>>;  // element (r, c) at c * LD_DST + r
};

template <int LD_SRC, int LD_DST>
__global__ void __launch_bounds__(256) swizzled_transpose(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                          uint16_t* __restrict__ lds_dump, int tiles_c) {
  __shared__ __attribute__((aligned(16))) uint16_t s[64 * 64];
  const int tr = int(blockIdx.x) / tiles_c, tc = int(blockIdx.x) % tiles_c;
  using G = SwzGlobal<LD_SRC, LD_DST>;
  tcd::g2s<tcd::workgroup_scope<256>, SwzT, typename G::src>(s, src + tr * 64 * LD_SRC + tc * 64);
  __syncthreads();
  tcd::s2g<tcd::workgroup_scope<256>, Lin4096, Lin4096>(lds_dump + int64_t(blockIdx.x) * 4096, s);
  tcd::s2g<tcd::workgroup_scope<256>, typename G::dst, SwzT>(dst + tc * 64 * LD_DST + tr * 64, s);
}

// 64 x 64 bf16 tiles of a row-major matrix of pitch 16384 staged through LDS by a workgroup of
// 256 lanes and written back to the same place of the destination (a tile copy through LDS, as
// a consumer kernel would stage its operand): mode 0 a plain LDS tile, mode 1 the XOR-swizzled
// tile with the recognised rounds lowered to adds, mode 2 the same swizzled tile with the swizzle
// applied every round (the general path), for timing the lowering against both.
constexpr int kStreamLd = 16384;
using StreamG = layout<ints<64, 64>, ints<kStreamLd, 1>>;
using StreamPlain = layout<ints<64, 64>, ints<64, 1>>;

template <int MODE>
__global__ void __launch_bounds__(256) tile_stream(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                    int tiles_c) {
  __shared__ __attribute__((aligned(16))) uint16_t s[64 * 64];
  const int tr = int(blockIdx.x) / tiles_c, tc = int(blockIdx.x) % tiles_c;
  const int64_t base = int64_t(tr) * 64 * kStreamLd + tc * 64;
  using WG = tcd::workgroup_scope<256>;
  if constexpr (MODE == 0) {
    tcd::g2s<WG, StreamPlain, StreamG>(s, src + base);
    __syncthreads();
    tcd::s2g<WG, StreamG, StreamPlain>(dst + base, s);
  } else if constexpr (MODE == 1) {
    tcd::g2s<WG, SwzT, StreamG>(s, src + base);
    __syncthreads();
    tcd::s2g<WG, StreamG, SwzT>(dst + base, s);
  } else {
    tcd::detail::copy_general<WG, tcd::drive::src, SwzT, StreamG>(s, src + base);
    __syncthreads();
    tcd::detail::copy_general<WG, tcd::drive::dst, StreamG, SwzT>(dst + base, s);
  }
}

// One lane copies a (3, 5, 7) int8 tile: source strides (80, 9, 1) (row pitch 9, plane pitch 80)
// -> destination strides (1, 3, 15) (fully transposed order).
using LaneSrc = layout<ints<3, 5, 7>, ints<80, 9, 1>>;
using LaneDst = layout<ints<3, 5, 7>, ints<1, 3, 15>>;

__global__ void lane_copy(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst) {
  if (threadIdx.x == 0) tcd::copy<tcd::lane_scope, tcd::drive::src, LaneDst, LaneSrc>(dst, src);
}

// Two waves (128 lanes) move a 45 x 40 fp16 tile, source pitch 56, through LDS (pitch 40) to a
// destination of pitch 40: 1800 elements, not a multiple of 128, so the last round is guarded.
using W2Src = layout<ints<45, 40>, ints<56, 1>>;
using W2Lds = layout<ints<45, 40>, ints<40, 1>>;

__global__ void __launch_bounds__(128) waves2_copy(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint16_t s[45 * 40];
  tcd::g2s<tcd::waves_scope<2>, W2Lds, W2Src>(s, src);
  tcd::waves_scope<2>::sync();
  tcd::s2g<tcd::waves_scope<2>, W2Lds, W2Lds>(dst, s);
}

int status() { return int(hipGetLastError()); }

template <class P>
void plan_out(int* out) {
  out[0] = P::vec;
  out[1] = P::outer;
  out[2] = P::exact;
  out[3] = P::lowered;
}

}  // namespace

extern "C" {

/* 32 x 32 fp32 round trip by one wave.  src/dst: device, 1024 floats each. */
int tcd_ex_roundtrip32(const float* src, float* dst, void* stream) {
  hipLaunchKernelGGL(roundtrip32, dim3(1), dim3(64), 0, hipStream_t(stream), src, dst);
  return status();
}

/* ntiles tiles of 256 floats each, permuted in LDS by one wave per tile (which: 0 the
 * scale-factor tile, 1 the 4 x 64 transpose) with the XOR swizzle (k, shift). */
int tcd_ex_permute_tiles(const float* src, float* dst, int ntiles, int which, int k, int shift, void* stream) {
  if (ntiles <= 0) return 0;
  if (k < 0 || k > 2 || shift < 0 || shift > 6) return int(hipErrorInvalidValue);
  const dim3 grid((ntiles + 3) / 4);
  if (which == 0) hipLaunchKernelGGL(permute_tiles<0>, grid, dim3(256), 0, hipStream_t(stream), src, dst, ntiles, k, shift);
  else hipLaunchKernelGGL(permute_tiles<1>, grid, dim3(256), 0, hipStream_t(stream), src, dst, ntiles, k, shift);
  return status();
}

/* (64 tiles_r) x (64 tiles_c) bf16 matrix of pitch 192 (tiles_c <= 3) transposed into a
 * destination of pitch 192 (tiles_r <= 3) through swizzled LDS tiles; lds_dump receives
 * tiles_r * tiles_c raw LDS images of 4096 elements (tile order: row-major over tiles). */
int tcd_ex_swizzled_transpose(const uint16_t* src, uint16_t* dst, uint16_t* lds_dump, int tiles_r, int tiles_c,
                              void* stream) {
  if (tiles_r < 1 || tiles_c < 1 || tiles_r > 3 || tiles_c > 3) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL((swizzled_transpose<192, 192>), dim3(tiles_r * tiles_c), dim3(256), 0, hipStream_t(stream), src,
                     dst, lds_dump, tiles_c);
  return status();
}

/* (64 tiles_r) x (64 tiles_c) bf16 tiles of a row-major matrix of pitch 16384 (tiles_r, tiles_c in
 * 1..256; src and dst hold 64 tiles_r x 16384 elements) copied tile by tile through LDS by one
 * workgroup per tile: mode 0 plain LDS tile, 1 XOR-swizzled tile (recognised rounds, adds), 2 the
 * swizzled tile with the swizzle applied every round. */
int tcd_ex_tile_stream(const uint16_t* src, uint16_t* dst, int tiles_r, int tiles_c, int mode, void* stream) {
  if (tiles_r < 1 || tiles_c < 1 || tiles_r > kStreamLd / 64 || tiles_c > kStreamLd / 64 || mode < 0 || mode > 2)
    return int(hipErrorInvalidValue);
  const dim3 grid(tiles_r * tiles_c);
  if (mode == 0) hipLaunchKernelGGL(tile_stream<0>, grid, dim3(256), 0, hipStream_t(stream), src, dst, tiles_c);
  else if (mode == 1) hipLaunchKernelGGL(tile_stream<1>, grid, dim3(256), 0, hipStream_t(stream), src, dst, tiles_c);
  else hipLaunchKernelGGL(tile_stream<2>, grid, dim3(256), 0, hipStream_t(stream), src, dst, tiles_c);
  return status();
}

/* (3, 5, 7) int8 tile by one lane: src holds 240 bytes, dst 105. */
int tcd_ex_lane_copy(const uint8_t* src, uint8_t* dst, void* stream) {
  hipLaunchKernelGGL(lane_copy, dim3(1), dim3(64), 0, hipStream_t(stream), src, dst);
  return status();
}

/* 45 x 40 fp16 tile by two waves: src holds 45 * 56 elements, dst 45 * 40. */
int tcd_ex_waves2_copy(const uint16_t* src, uint16_t* dst, void* stream) {
  hipLaunchKernelGGL(waves2_copy, dim3(1), dim3(128), 0, hipStream_t(stream), src, dst);
  return status();
}

/* The [outer, threads, vec] plans the examples compile to, for inspection:
 * out[0..3] = (vec, outer, exact, lowered) of: 0 roundtrip32 load, 1 swizzled load, 2 swizzled
 * transposed store, 3 lane copy, 4 two-wave load, 5 the stream example's swizzled load, 6 its
 * swizzled store, 7 its plain load.  lowered = 1: the rounds were recognised (per-round adds of
 * compile-time constants).  Returns 0, or -1 for an unknown index. */
int tcd_ex_plan(int which, int* out) {
  using WG = tcd::workgroup_scope<256>;
  switch (which) {
    case 0: plan_out<tcd::copy_plan<tcd::wave_scope, tcd::drive::src, L32, L32, float>>(out); break;
    case 1: plan_out<tcd::copy_plan<WG, tcd::drive::src, SwzT, SwzGlobal<192, 192>::src, uint16_t>>(out); break;
    case 2: plan_out<tcd::copy_plan<WG, tcd::drive::dst, SwzGlobal<192, 192>::dst, SwzT, uint16_t>>(out); break;
    case 3: plan_out<tcd::copy_plan<tcd::lane_scope, tcd::drive::src, LaneDst, LaneSrc, uint8_t>>(out); break;
    case 4: plan_out<tcd::copy_plan<tcd::waves_scope<2>, tcd::drive::src, W2Lds, W2Src, uint16_t>>(out); break;
    case 5: plan_out<tcd::copy_plan<WG, tcd::drive::src, SwzT, StreamG, uint16_t>>(out); break;
    case 6: plan_out<tcd::copy_plan<WG, tcd::drive::dst, StreamG, SwzT, uint16_t>>(out); break;
    case 7: plan_out<tcd::copy_plan<WG, tcd::drive::src, StreamPlain, StreamG, uint16_t>>(out); break;
    default: return -1;
  }
  return 0;
}

}  // extern "C"
