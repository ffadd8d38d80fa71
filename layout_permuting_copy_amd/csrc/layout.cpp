// Layout algebra: joint modes of a copy, canonical order and merging, injectivity,
// address ranges and region slices.
//
// A TileLayout S[shape : stride] maps a logical index to offset + sum_k i_k * stride_k
// (TVM TIRx docs, "copy -> gmem_smem", demonstration program).  A copy is valid when both
// operands have equal non-unit extents ("What it accepts", _is_valid_copy), so both layouts
// are handled together as joint modes (extent, src stride, dst stride).  Canonicalization
// (Algorithm step 1 of the same page, and "permute_layout" Algorithm step 1) drops unit
// modes, orders modes by stride, and merges neighbours that are contiguous on both sides;
// the merged form is what the partition planner splits into [outer, threads, vec].
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <unordered_set>
#include <vector>

#include "plan.hpp"

namespace tc {

int make_joint(const tc_layout& src, const tc_layout& dst, Joint* out, std::string* err) {
  if (src.rank < 0 || src.rank > kMaxRank || dst.rank < 0 || dst.rank > kMaxRank) {
    *err = "rank outside 0.." + std::to_string(kMaxRank);
    return TC_E_RANK;
  }
  for (int k = 0; k < src.rank; ++k)
    if (src.shape[k] < 0) { *err = "negative source extent"; return TC_E_EXTENT; }
  for (int k = 0; k < dst.rank; ++k)
    if (dst.shape[k] < 0) { *err = "negative destination extent"; return TC_E_EXTENT; }
  Mode a[kMaxRank], b[kMaxRank];
  int na = 0, nb = 0;
  for (int k = 0; k < src.rank; ++k)
    if (src.shape[k] != 1) a[na++] = Mode{src.shape[k], src.stride[k], 0};
  for (int k = 0; k < dst.rank; ++k)
    if (dst.shape[k] != 1) b[nb++] = Mode{dst.shape[k], 0, dst.stride[k]};
  bool equal = (na == nb);
  for (int k = 0; equal && k < na; ++k) equal = (a[k].e == b[k].e);
  if (!equal) {
    std::string sa, sb;
    for (int k = 0; k < na; ++k) sa += (k ? "," : "") + std::to_string(a[k].e);
    for (int k = 0; k < nb; ++k) sb += (k ? "," : "") + std::to_string(b[k].e);
    *err = "extent mismatch: non-unit extents (" + sa + ") vs (" + sb + ")";
    return TC_E_EXTENT;
  }
  // Sizes a 64-bit address computation holds: the element count and every element offset of
  // both sides (offset plus the extreme index sums) within 2^58, so that byte offsets of 16-byte
  // elements stay below 2^62.  Products and sums in 128 bits, so nothing wraps before the check.
  bool empty = false;
  for (int k = 0; k < na; ++k) empty = empty || a[k].e == 0;
  if (!empty) {
    constexpr __int128 kLim = __int128(1) << 58;
    __int128 cnt = 1, slo = src.offset, shi = src.offset, dlo = dst.offset, dhi = dst.offset;
    bool fits = true;
    for (int k = 0; k < na && fits; ++k) {
      cnt *= a[k].e;
      const __int128 ss = __int128(a[k].e - 1) * a[k].s, ds = __int128(a[k].e - 1) * b[k].d;
      if (ss < 0) slo += ss; else shi += ss;
      if (ds < 0) dlo += ds; else dhi += ds;
      fits = cnt <= kLim && slo >= -kLim && shi <= kLim && dlo >= -kLim && dhi <= kLim;
    }
    if (!fits) {
      *err = "element count or element offsets beyond 2^58 (64-bit byte addresses would overflow)";
      return TC_E_RANGE;
    }
  }
  Joint j;
  j.rank = na;
  j.so = src.offset;
  j.dof = dst.offset;
  j.count = 1;
  for (int k = 0; k < na; ++k) {
    j.m[k] = Mode{a[k].e, a[k].s, b[k].d};
    j.count *= a[k].e;
  }
  *out = j;
  return TC_OK;
}

void canonicalize(Joint* j) {
  if (j->count == 0) return;
  std::stable_sort(j->m, j->m + j->rank, [](const Mode& x, const Mode& y) {
    return std::llabs(x.d) > std::llabs(y.d);
  });
  int n = 0;
  for (int k = 0; k < j->rank; ++k) {
    const Mode cur = j->m[k];
    if (n > 0) {
      Mode& prev = j->m[n - 1];
      if (prev.s == cur.e * cur.s && prev.d == cur.e * cur.d) {
        prev = Mode{prev.e * cur.e, cur.s, cur.d};
        continue;
      }
    }
    j->m[n++] = cur;
  }
  j->rank = n;
}

int dst_injective(const Joint& j) {
  if (j.count <= 1) return 1;
  std::vector<Mode> ms(j.m, j.m + j.rank);
  for (const Mode& m : ms)
    if (m.d == 0) return 0;
  std::sort(ms.begin(), ms.end(), [](const Mode& x, const Mode& y) { return std::llabs(x.d) < std::llabs(y.d); });
  // Sufficient: each stride exceeds the span of all smaller modes.
  int64_t span = 1;
  bool nested = true;
  for (const Mode& m : ms) {
    if (std::llabs(m.d) < span) { nested = false; break; }
    span += (m.e - 1) * std::llabs(m.d);
  }
  if (nested) return 1;
  if (j.count > (int64_t(1) << 24)) return -1;
  std::unordered_set<int64_t> seen;
  seen.reserve(size_t(j.count) * 2);
  std::vector<int64_t> idx(j.rank, 0);
  for (int64_t n = 0; n < j.count; ++n) {
    int64_t off = 0;
    for (int k = 0; k < j.rank; ++k) off += idx[k] * j.m[k].d;
    if (!seen.insert(off).second) return 0;
    for (int k = j.rank - 1; k >= 0; --k) {
      if (++idx[k] < j.m[k].e) break;
      idx[k] = 0;
    }
  }
  return 1;
}

void side_range(const Joint& j, bool src_side, int64_t* lo, int64_t* hi) {
  int64_t base = src_side ? j.so : j.dof;
  int64_t a = base, b = base;
  for (int k = 0; k < j.rank; ++k) {
    const int64_t st = src_side ? j.m[k].s : j.m[k].d;
    const int64_t span = (j.m[k].e - 1) * st;
    if (span < 0) a += span; else b += span;
  }
  *lo = a;
  *hi = b + 1;
}

int slice_layout(const tc_layout& in, const int64_t* start, const int64_t* stop, const int64_t* step,
                 tc_layout* out, std::string* err) {
  if (in.rank < 0 || in.rank > kMaxRank) { *err = "rank outside 0..8"; return TC_E_RANK; }
  tc_layout o = in;
  for (int k = 0; k < in.rank; ++k) {
    const int64_t len = in.shape[k];
    const int64_t st = step[k];
    if (st == 0) { *err = "slice step must not be zero"; return TC_E_ARG; }
    if (st == INT64_MIN) { *err = "slice step out of range"; return TC_E_RANGE; }
    if (len < 0) { *err = "negative extent"; return TC_E_EXTENT; }
    int64_t b = start[k], e = stop[k], n;
    if (st > 0) {
      if (b < 0) b += len;
      if (e < 0) e += len;
      b = std::min(std::max<int64_t>(b, 0), len);
      e = std::min(std::max<int64_t>(e, 0), len);
      n = e > b ? (e - b - 1) / st + 1 : 0;
    } else {
      if (b < 0) b += len;
      if (e < 0) e += len;
      b = std::min(std::max<int64_t>(b, -1), len - 1);
      e = std::min(std::max<int64_t>(e, -1), len - 1);
      n = b > e ? (b - e - 1) / (-st) + 1 : 0;
    }
    // offset and stride in 128 bits; a result that does not fit 64 bits is an error
    const __int128 off = __int128(o.offset) + (n > 0 ? __int128(b) * in.stride[k] : 0);
    const __int128 str = __int128(in.stride[k]) * st;
    if (off > INT64_MAX || off < INT64_MIN || str > INT64_MAX || str < INT64_MIN) {
      *err = "sliced offset or stride beyond 64 bits";
      return TC_E_RANGE;
    }
    o.offset = int64_t(off);
    o.shape[k] = n;
    o.stride[k] = int64_t(str);
  }
  *out = o;
  return TC_OK;
}

}  // namespace tc
