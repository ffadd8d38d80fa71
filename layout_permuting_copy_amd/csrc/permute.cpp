// Bank plan of the wave-scope register-staged permute (TVM TIRx docs, "permute_layout",
// Algorithm steps 1 and 2), for tcd::wave_permute: the smallest XOR bit count k, and for it the
// smallest shift, whose lane -> element assignment leaves both the read phase (source layout) and
// the write phase (destination layout) free of LDS bank conflicts under gfx950's model.
#include <cstdio>
#include <cstring>
#include <string>

#include "plan.hpp"

namespace tc {
namespace {

constexpr int kLanes = 64;

struct Shard {
  int rank = 0;
  int64_t e[kMaxRank], s[kMaxRank], d[kMaxRank];
  int64_t count = 1;
};

// Logical order kept (no sorting): neighbours merge where contiguous on both sides.
Shard shard_of(const Joint& j) {
  Shard sh;
  for (int k = 0; k < j.rank; ++k) {
    const Mode& m = j.m[k];
    if (sh.rank > 0) {
      const int p = sh.rank - 1;
      if (sh.s[p] == m.e * m.s && sh.d[p] == m.e * m.d) {
        sh.e[p] *= m.e;
        sh.s[p] = m.s;
        sh.d[p] = m.d;
        continue;
      }
    }
    sh.e[sh.rank] = m.e;
    sh.s[sh.rank] = m.s;
    sh.d[sh.rank] = m.d;
    ++sh.rank;
  }
  sh.count = j.count;
  return sh;
}

// Extra cycles of one phase over the P steps: element-wide accesses through `strides`.
int64_t phase_cycles(const Shard& sh, const int64_t* strides, int eb, bool write, int k, int shift, int P) {
  const int mask = (1 << k) - 1;
  int64_t addr[kLanes];
  int64_t total = 0;
  for (int r = 0; r < P; ++r) {
    for (int l = 0; l < kLanes; ++l) {
      int64_t rem = l + int64_t(r ^ ((l >> shift) & mask)) * kLanes, off = 0;
      for (int q = sh.rank - 1; q >= 0; --q) {
        off += (rem % sh.e[q]) * strides[q];
        rem /= sh.e[q];
      }
      addr[l] = off * eb;
    }
    total += lds_conflict_cycles(addr, nullptr, kLanes, eb, write);
  }
  return total;
}

}  // namespace

int wave_permute_plan(const tc_layout& src, const tc_layout& dst, int dtype, tc_permute_info* out,
                      std::string* err) {
  std::memset(out, 0, sizeof(*out));
  const int eb = elem_bytes_of(dtype);
  if (eb < 0) {
    *err = "unknown dtype " + std::to_string(dtype);
    return TC_E_DTYPE;
  }
  Joint j;
  const int st = make_joint(src, dst, &j, err);
  if (st != TC_OK) return st;
  const Shard sh = shard_of(j);
  out->rank = sh.rank;
  for (int k = 0; k < sh.rank; ++k) {
    out->extent[k] = sh.e[k];
    out->src_stride[k] = sh.s[k];
    out->dst_stride[k] = sh.d[k];
  }
  int64_t lo_s, hi_s, lo_d, hi_d;
  side_range(j, true, &lo_s, &hi_s);
  side_range(j, false, &lo_d, &hi_d);
  const int64_t lim = int64_t(1) << 31;
  if (hi_s >= lim || hi_d >= lim || lo_s < -lim || lo_d < -lim) {
    *err = "tile offsets need more than 31 bits";
    return TC_E_RANGE;
  }
  auto declined = [&](const std::string& why) {
    std::snprintf(out->reason, sizeof(out->reason), "%s", why.c_str());
    *err = why;
    return TC_E_DECLINED;
  };
  if (sh.count == 0 || sh.count % kLanes != 0)
    return declined("element count " + std::to_string(sh.count) + " is not a multiple of the " +
                    std::to_string(kLanes) + " lanes: no integer P");
  if (sh.count / kLanes > 256) return declined("more than 256 elements per lane");
  const int P = int(sh.count / kLanes);
  out->elements_per_lane = P;
  int log2p = 0;
  while ((1 << (log2p + 1)) <= P) ++log2p;
  const int kmax = (1 << log2p) == P ? log2p : 0;  // an XOR of k > 0 bits permutes [0, P) only for P = 2^m
  int64_t best = -1;
  for (int k = 0; k <= kmax; ++k)
    for (int shift = 0; shift <= (k ? 6 - k : 0); ++shift) {
      const int64_t rc = phase_cycles(sh, sh.s, eb, false, k, shift, P);
      const int64_t wc = phase_cycles(sh, sh.d, eb, true, k, shift, P);
      if (best < 0 || rc + wc < best) {  // first candidate with the fewest extra cycles
        best = rc + wc;
        out->k = k;
        out->shift = shift;
        out->mask = (1 << k) - 1;
        out->read_conflicts = rc;
        out->write_conflicts = wc;
      }
      if (rc + wc == 0) return TC_OK;
    }
  return declined("no XOR bit count k in 0.." + std::to_string(kmax) +
                  " leaves both the read and the write phase conflict-free");
}

}  // namespace tc

extern "C" int tc_wave_permute_plan(const tc_layout* src_layout, const tc_layout* dst_layout, int dtype,
                                    tc_permute_info* out) {
  std::string err;
  if (!src_layout || !dst_layout || !out) return tc::set_last_error(TC_E_NULL, "null pointer argument");
  const int rc = tc::wave_permute_plan(*src_layout, *dst_layout, dtype, out, &err);
  tc::set_last_error(rc, rc == TC_OK ? std::string() : err);
  return rc;
}
