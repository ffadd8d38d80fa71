/* A plain C user of the tile-copy C ABI (no Python, no torch): allocates device memory with the
 * HIP runtime, plans and runs a 256 x 192 float transpose and a (2,1,4,32) scale-factor tile
 * batch, and writes the raw destination bytes to the given file for comparison with the oracle.
 * Exit status: 0 on success, 1 on any library or HIP error (message on stderr). */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tile_copy.h"

static int fail(const char* what, int rc) {
  fprintf(stderr, "%s failed (%d): %s\n", what, rc, tc_last_error());
  return 1;
}

static tc_layout make(int rank, const int64_t* shape, const int64_t* stride) {
  tc_layout l;
  memset(&l, 0, sizeof(l));
  l.rank = rank;
  for (int k = 0; k < rank; ++k) {
    l.shape[k] = shape[k];
    l.stride[k] = stride[k];
  }
  return l;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTPUT\n", argv[0]);
    return 2;
  }
  const int n = 256, m = 192, tiles = 3;
  const size_t bytes_t = (size_t)n * m * 4, bytes_sf = (size_t)tiles * 256 * 4;
  float* h = (float*)malloc(bytes_t + bytes_sf);
  for (size_t i = 0; i < (bytes_t + bytes_sf) / 4; ++i) h[i] = (float)((i * 2654435761u) % 100003) - 50000.0f;
  void *src = NULL, *dst = NULL;
  if (hipMalloc(&src, bytes_t + bytes_sf) != hipSuccess || hipMalloc(&dst, bytes_t + bytes_sf) != hipSuccess) {
    fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  hipMemcpy(src, h, bytes_t + bytes_sf, hipMemcpyHostToDevice);
  hipMemset(dst, 0xA5, bytes_t + bytes_sf);

  /* 1. transpose: (n, m):(m, 1) -> (n, m):(1, n) */
  const int64_t sh[2] = {n, m}, ss[2] = {m, 1}, ds[2] = {1, n};
  tc_layout sl = make(2, sh, ss), dl = make(2, sh, ds);
  tc_plan_info info;
  int rc = tc_plan(&sl, &dl, TC_F32, 0, 16, &info);
  if (rc != TC_OK) return fail("tc_plan", rc);
  fprintf(stderr, "transpose plan: path %d, tile %d x %d, vec %d bytes\n", info.path, info.tile_r, info.tile_c,
          info.vec_bytes);
  rc = tile_copy(src, &sl, dst, &dl, TC_F32, NULL);
  if (rc != TC_OK) return fail("tile_copy", rc);

  /* 2. three scale-factor tiles (2,1,4,32):(128,128,32,1) -> (128,128,1,4), after the transpose */
  const int64_t fsh[5] = {tiles, 2, 1, 4, 32}, fss[5] = {256, 128, 128, 32, 1}, fds[5] = {256, 128, 128, 1, 4};
  tc_layout fsl = make(5, fsh, fss), fdl = make(5, fsh, fds);
  fsl.offset = fdl.offset = (int64_t)n * m;
  rc = tile_copy_ex(src, &fsl, dst, &fdl, TC_F32, NULL, 0, &info);
  if (rc != TC_OK) return fail("tile_copy_ex", rc);
  fprintf(stderr, "scale-factor plan: path %d\n", info.path);

  /* 3. errors come back as codes with a reason */
  tc_layout bad = make(2, sh, ss);
  bad.shape[0] = n + 1;
  rc = tile_copy(src, &bad, dst, &dl, TC_F32, NULL);
  if (rc != TC_E_EXTENT) return fail("extent mismatch not reported", rc);

  if (hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "hipDeviceSynchronize failed\n");
    return 1;
  }
  hipMemcpy(h, dst, bytes_t + bytes_sf, hipMemcpyDeviceToHost);
  FILE* f = fopen(argv[1], "wb");
  if (!f || fwrite(h, 1, bytes_t + bytes_sf, f) != bytes_t + bytes_sf) return fail("write output", 0);
  fclose(f);
  hipFree(src);
  hipFree(dst);
  free(h);
  return 0;
}
