// LDS bank-structure probe for gfx950.
//
// The swizzle chooser simulates the LDS bank pattern of the target.  The pages
// model NVIDIA shared memory (32 banks x 4 B, 32-lane warps); CDNA4's bank
// count and the lane grouping it uses for 4/8/16-byte accesses are not stated
// on them, so this program measures them.  One workgroup of one wave64 runs
// each pattern: every lane issues the same LDS access (fixed per-lane byte
// address) ITERS times; the cycle count per access, and the rocprofv3 counters
// SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS of each dispatch, give the conflict
// degree of the pattern.  Every address stays inside the 64 KiB LDS array.
//
// Output: one line per pattern, "idx width op name cycles_per_access", in
// dispatch order (dispatch k of the kernel trace is pattern k).

#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_),       \
              __FILE__, __LINE__);                                            \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

constexpr int LDS_WORDS = 16384;  // 64 KiB
constexpr int ITERS = 512;

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// W = access bytes (1, 2, 4, 8, 16); WRITE selects ds_write over ds_read.
template <int W, bool WRITE>
__global__ void __launch_bounds__(64) probe_kernel(const int* __restrict__ addr,
                                                   unsigned* __restrict__ out,
                                                   long long* __restrict__ cyc) {
  __shared__ __attribute__((aligned(16))) unsigned lds[LDS_WORDS];
  const int lane = threadIdx.x;
  for (int i = lane; i < LDS_WORDS; i += 64) lds[i] = (unsigned)i * 2654435761u;
  __syncthreads();
  const int a = addr[lane];  // byte offset, host-checked: a + W <= 65536, a % W == 0
  // Explicit LDS (address space 3) pointers, so the accesses are ds_* and not flat.
  typedef __attribute__((address_space(3))) volatile unsigned char lu8;
  typedef __attribute__((address_space(3))) volatile unsigned short lu16;
  typedef __attribute__((address_space(3))) volatile unsigned lu32;
  typedef __attribute__((address_space(3))) volatile u32x2 lu64;
  typedef __attribute__((address_space(3))) volatile u32x4 lu128;
  lu8* base = (lu8*)((__attribute__((address_space(3))) unsigned char*)lds) + a;
  unsigned acc = 0;
  long long t0 = clock64();
  if constexpr (WRITE) {
    for (int it = 0; it < ITERS; ++it) {
      if constexpr (W == 1) *reinterpret_cast<lu8*>(base) = (unsigned char)(it + lane);
      if constexpr (W == 2) *reinterpret_cast<lu16*>(base) = (unsigned short)(it + lane);
      if constexpr (W == 4) *reinterpret_cast<lu32*>(base) = (unsigned)(it + lane);
      if constexpr (W == 8) *reinterpret_cast<lu64*>(base) = u32x2{(unsigned)it, (unsigned)lane};
      if constexpr (W == 16)
        *reinterpret_cast<lu128*>(base) = u32x4{(unsigned)it, (unsigned)lane, 1u, 2u};
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    for (int it = 0; it < ITERS; ++it) {
      if constexpr (W == 1) acc += *reinterpret_cast<lu8*>(base);
      if constexpr (W == 2) acc += *reinterpret_cast<lu16*>(base);
      if constexpr (W == 4) acc += *reinterpret_cast<lu32*>(base);
      if constexpr (W == 8) {
        u32x2 v = *reinterpret_cast<lu64*>(base);
        acc += v.x ^ v.y;
      }
      if constexpr (W == 16) {
        u32x4 v = *reinterpret_cast<lu128*>(base);
        acc += v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  long long t1 = clock64();
  __syncthreads();
  out[lane] = acc + lds[lane];
  if (lane == 0) cyc[0] = t1 - t0;
}

struct Pattern {
  int width;
  bool write;
  std::string name;
  std::vector<int> addr;  // 64 byte offsets
};

static void add(std::vector<Pattern>& ps, int w, const std::string& name, int (*f)(int, int)) {
  for (int wr = 0; wr < 2; ++wr) {
    Pattern p{w, wr == 1, name, std::vector<int>(64)};
    for (int l = 0; l < 64; ++l) p.addr[l] = f(l, w);
    ps.push_back(p);
  }
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device %s arch %s CUs %d warpSize %d lds_per_block %zu lds_per_cu %zu l2 %d clock_khz %d memclk_khz %d busbits %d\n",
         prop.name, prop.gcnArchName, prop.multiProcessorCount, prop.warpSize,
         prop.sharedMemPerBlock, prop.maxSharedMemoryPerMultiProcessor, prop.l2CacheSize,
         prop.clockRate, prop.memoryClockRate, prop.memoryBusWidth);

  std::vector<Pattern> ps;
  for (int w : {4, 8, 16}) {
    add(ps, w, "linear", [](int l, int w) { return l * w; });
    add(ps, w, "bcast", [](int, int) { return 0; });
    add(ps, w, "stride2w", [](int l, int w) { return l * 2 * w; });
    add(ps, w, "stride4w", [](int l, int w) { return l * 4 * w; });
    add(ps, w, "stride128B", [](int l, int) { return l * 128 % 65536; });
    add(ps, w, "stride256B", [](int l, int) { return l * 256 % 65536; });
    // lanes 32..63 shifted by 128 B / 256 B / 512 B relative to lanes 0..31
    add(ps, w, "half+128B", [](int l, int w) { return (l % 32) * w % 128 + (l / 32) * 128 + ((l % 32) * w / 128) * 1024; });
    add(ps, w, "half+256B", [](int l, int w) { return (l % 32) * w % 256 + (l / 32) * 256 + ((l % 32) * w / 256) * 1024; });
    // group-of-g lanes covering one 128 B / 256 B row, groups 1 KiB apart
    add(ps, w, "grp8", [](int l, int w) { return (l % 8) * w + (l / 8) * 1024; });
    add(ps, w, "grp16", [](int l, int w) { return (l % 16) * w + (l / 16) * 1024; });
    add(ps, w, "grp32", [](int l, int w) { return (l % 32) * w + (l / 32) * 4096; });
    // two lanes per address (same dword/qword/quad)
    add(ps, w, "pairs", [](int l, int w) { return (l / 2) * w; });
  }
  for (int w : {1, 2}) {
    add(ps, w, "linear", [](int l, int w) { return l * w; });
    add(ps, w, "stride4B", [](int l, int) { return l * 4; });
    add(ps, w, "stride256B", [](int l, int) { return l * 256 % 65536; });
  }
  for (const auto& p : ps)
    for (int a : p.addr)
      if (a < 0 || a % p.width != 0 || a + p.width > LDS_WORDS * 4) {
        fprintf(stderr, "bad pattern %s\n", p.name.c_str());
        return 2;
      }

  int* d_addr;
  unsigned* d_out;
  long long* d_cyc;
  CHECK(hipMalloc(&d_addr, 64 * sizeof(int)));
  CHECK(hipMalloc(&d_out, 64 * sizeof(unsigned)));
  CHECK(hipMalloc(&d_cyc, sizeof(long long)));
  for (size_t i = 0; i < ps.size(); ++i) {
    const Pattern& p = ps[i];
    CHECK(hipMemcpy(d_addr, p.addr.data(), 64 * sizeof(int), hipMemcpyHostToDevice));
#define L(W, WR) hipLaunchKernelGGL((probe_kernel<W, WR>), dim3(1), dim3(64), 0, 0, d_addr, d_out, d_cyc)
    if (p.width == 1) { if (p.write) L(1, true); else L(1, false); }
    if (p.width == 2) { if (p.write) L(2, true); else L(2, false); }
    if (p.width == 4) { if (p.write) L(4, true); else L(4, false); }
    if (p.width == 8) { if (p.write) L(8, true); else L(8, false); }
    if (p.width == 16) { if (p.write) L(16, true); else L(16, false); }
#undef L
    CHECK(hipGetLastError());
    long long cyc = 0;
    CHECK(hipMemcpy(&cyc, d_cyc, sizeof(long long), hipMemcpyDeviceToHost));
    printf("%3zu w%-2d %-5s %-12s %8.2f\n", i, p.width, p.write ? "write" : "read", p.name.c_str(),
           (double)cyc / ITERS);
    fflush(stdout);
  }
  CHECK(hipFree(d_addr));
  CHECK(hipFree(d_out));
  CHECK(hipFree(d_cyc));
  return 0;
}
