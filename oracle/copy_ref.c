/*
 * Oracle for the layout-permuting copy.  TEST INFRASTRUCTURE ONLY: the tests,
 * the smoke check and the benchmark's CPU-baseline leg call it; the product
 * library never links or calls it, and it shares no code with it.
 *
 * What it computes is the plain definition of a layout-driven copy
 * (TVM TIRx docs, "copy -> gmem_smem", intro and "What it accepts": both
 * operands carry a shape:stride layout, equal dtype and equal non-unit
 * extents; TVM TIRx docs, "permute_layout", intro: data moves from a source
 * TileLayout to a destination TileLayout).  A layout maps a logical index
 * i = (i_0, ..., i_{r-1}) to the element offset  offset + sum_k i_k * stride_k.
 * For every logical index of the common shape:
 *
 *     dst[dst_layout(i)] = src[src_layout(i)]      (elem_bytes raw bytes)
 *
 * Extent-1 modes are dropped from both sides first; the remaining extents must
 * be equal, in order.  Bytes of dst that no index names are left untouched.
 * The loop is an odometer over the common shape in row-major order (the
 * flatten order of the TileLang loop_mapping.py tutorial); the result does not
 * depend on the order when dst is injective.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC copy_ref.c -o liboracle_copy.so
 */
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_RANK 16

/* Keep the modes whose extent is not 1, in order. Returns the new rank. */
static int drop_unit_modes(int rank, const int64_t* shape, const int64_t* stride,
                           int64_t* out_shape, int64_t* out_stride) {
  int n = 0;
  for (int k = 0; k < rank; ++k) {
    if (shape[k] == 1) continue;
    out_shape[n] = shape[k];
    out_stride[n] = stride[k];
    ++n;
  }
  return n;
}

/*
 * Returns 0 on success, -1 if the non-unit extents differ, -2 on bad
 * arguments (rank out of range, negative extent, bad element size).
 * nthreads <= 0 means "use the OpenMP default".
 */
int oracle_copy(const unsigned char* src, int src_rank, const int64_t* src_shape,
                const int64_t* src_stride, int64_t src_offset, unsigned char* dst,
                int dst_rank, const int64_t* dst_shape, const int64_t* dst_stride,
                int64_t dst_offset, int64_t elem_bytes, int nthreads) {
  int64_t ss[ORACLE_MAX_RANK], sst[ORACLE_MAX_RANK], ds[ORACLE_MAX_RANK], dst_st[ORACLE_MAX_RANK];
  if (src_rank < 0 || dst_rank < 0 || src_rank > ORACLE_MAX_RANK || dst_rank > ORACLE_MAX_RANK) return -2;
  if (elem_bytes <= 0) return -2;
  for (int k = 0; k < src_rank; ++k) if (src_shape[k] < 0) return -2;
  for (int k = 0; k < dst_rank; ++k) if (dst_shape[k] < 0) return -2;
  int rs = drop_unit_modes(src_rank, src_shape, src_stride, ss, sst);
  int rd = drop_unit_modes(dst_rank, dst_shape, dst_stride, ds, dst_st);
  if (rs != rd) return -1;
  for (int k = 0; k < rs; ++k) if (ss[k] != ds[k]) return -1;
  const int r = rs;
  int64_t count = 1;
  for (int k = 0; k < r; ++k) count *= ss[k];
  if (count == 0) return 0;
  if (r == 0) { /* a single element */
    memcpy(dst + dst_offset * elem_bytes, src + src_offset * elem_bytes, (size_t)elem_bytes);
    return 0;
  }
#ifdef _OPENMP
  /* a per-call thread count: it does not change the default of later calls */
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  (void)nthreads;
#endif
  const int64_t outer = ss[0];
  /* One outermost index per iteration; an odometer walks the inner modes. */
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t i0 = 0; i0 < outer; ++i0) {
    int64_t idx[ORACLE_MAX_RANK];
    for (int k = 0; k < r; ++k) idx[k] = 0;
    idx[0] = i0;
    int64_t inner = 1;
    for (int k = 1; k < r; ++k) inner *= ss[k];
    for (int64_t n = 0; n < inner; ++n) {
      int64_t so = src_offset, dof = dst_offset;
      for (int k = 0; k < r; ++k) {
        so += idx[k] * sst[k];
        dof += idx[k] * dst_st[k];
      }
      memcpy(dst + dof * elem_bytes, src + so * elem_bytes, (size_t)elem_bytes);
      /* advance the odometer over modes 1..r-1 (row-major: last mode fastest) */
      for (int k = r - 1; k >= 1; --k) {
        if (++idx[k] < ss[k]) break;
        idx[k] = 0;
      }
    }
  }
  return 0;
}

/* Number of threads the OpenMP runtime would use for a parallel region. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
