// C ABI of the tile-copy library: argument checks, plan cache, launch.
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>

#include "plan.hpp"

namespace {

thread_local std::string g_err;
std::mutex g_mu;
int g_flags = 0;
std::unordered_map<std::string, std::shared_ptr<const tc::Plan>>* g_cache = nullptr;
constexpr size_t kCacheMax = 4096;

int fail(int code, const std::string& why) {
  g_err = why;
  return code;
}

std::string layout_key(const tc_layout& l) {
  std::string k;
  const int r = (l.rank >= 0 && l.rank <= TC_MAX_RANK) ? l.rank : 0;
  k.append(reinterpret_cast<const char*>(&l.rank), sizeof(l.rank));
  k.append(reinterpret_cast<const char*>(&l.offset), sizeof(l.offset));
  k.append(reinterpret_cast<const char*>(l.shape), sizeof(int64_t) * r);
  k.append(reinterpret_cast<const char*>(l.stride), sizeof(int64_t) * r);
  return k;
}

std::shared_ptr<const tc::Plan> get_plan(const tc_layout& s, const tc_layout& d, int dtype, int flags, int align) {
  std::string key = layout_key(s) + layout_key(d);
  key.append(reinterpret_cast<const char*>(&dtype), sizeof(dtype));
  key.append(reinterpret_cast<const char*>(&flags), sizeof(flags));
  key.append(reinterpret_cast<const char*>(&align), sizeof(align));
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_cache) g_cache = new std::unordered_map<std::string, std::shared_ptr<const tc::Plan>>();
    auto it = g_cache->find(key);
    if (it != g_cache->end()) return it->second;
  }
  auto p = std::make_shared<const tc::Plan>(tc::make_plan(s, d, dtype, flags, align));
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_cache->size() >= kCacheMax) g_cache->clear();
  g_cache->emplace(key, p);
  return p;
}

int ptr_alignment(uintptr_t a, uintptr_t b) {
  const uintptr_t x = a | b | 16;
  return int(x & (~x + 1));
}

}  // namespace

namespace tc {
int set_last_error(int code, const std::string& why) {
  g_err = why;
  return code;
}
}  // namespace tc

extern "C" {

int tile_copy_ex(const void* src, const tc_layout* src_layout, void* dst, const tc_layout* dst_layout, int dtype,
                 void* stream, int flags, tc_plan_info* info) {
  g_err.clear();
  if (!src || !dst || !src_layout || !dst_layout) return fail(TC_E_NULL, "null pointer argument");
  const int eb = tc::elem_bytes_of(dtype);
  if (eb < 0) return fail(TC_E_DTYPE, "unknown dtype " + std::to_string(dtype));
  if (flags & ~TC_FLAG_ALL) return fail(TC_E_ARG, "unknown flag bits");
  const uintptr_t ps = reinterpret_cast<uintptr_t>(src), pd = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t ealign = uintptr_t(eb < 16 ? eb : 16);
  if (ps % ealign || pd % ealign)
    return fail(TC_E_ALIGN, "base pointer not aligned to the element size (" + std::to_string(eb) + " bytes)");
  const int align = ptr_alignment(ps, pd);
  auto plan = get_plan(*src_layout, *dst_layout, dtype, flags, align);
  if (info) tc::plan_to_info(*plan, info);
  if (plan->status != TC_OK) return fail(plan->status, plan->reason);
  if (plan->path == TC_PATH_EMPTY) return TC_OK;
  // the byte images of source and destination must not overlap (side_range gives [lo, hi) in
  // elements: hi is one past the last element)
  int64_t slo, shi, dlo, dhi;
  tc::side_range(plan->j, true, &slo, &shi);
  tc::side_range(plan->j, false, &dlo, &dhi);
  const __int128 s0 = __int128(ps) + __int128(slo) * eb, s1 = __int128(ps) + __int128(shi) * eb;
  const __int128 d0 = __int128(pd) + __int128(dlo) * eb, d1 = __int128(pd) + __int128(dhi) * eb;
  if (s0 < d1 && d0 < s1) return fail(TC_E_ALIAS, "source and destination byte ranges overlap");
  std::string err;
  const int rc = tc::launch_plan(*plan, src, dst, stream, &err);
  if (rc != TC_OK) return fail(rc, err);
  return TC_OK;
}

int tile_copy(const void* src, const tc_layout* src_layout, void* dst, const tc_layout* dst_layout, int dtype,
              void* stream) {
  int flags;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    flags = g_flags;
  }
  return tile_copy_ex(src, src_layout, dst, dst_layout, dtype, stream, flags, nullptr);
}

int tc_plan(const tc_layout* src_layout, const tc_layout* dst_layout, int dtype, int flags, int ptr_align,
            tc_plan_info* out) {
  g_err.clear();
  if (!src_layout || !dst_layout || !out) return fail(TC_E_NULL, "null pointer argument");
  if (ptr_align < 0 || (ptr_align & (ptr_align - 1))) return fail(TC_E_ARG, "ptr_align must be a power of two");
  if (ptr_align == 0 || ptr_align > 16) ptr_align = 16;
  tc::Plan p = tc::make_plan(*src_layout, *dst_layout, dtype, flags, ptr_align);
  tc::plan_to_info(p, out);
  if (p.status != TC_OK) return fail(p.status, p.reason);
  return TC_OK;
}

const char* tc_last_error(void) { return g_err.c_str(); }

int tc_set_flags(int flags) {
  if (flags & ~TC_FLAG_ALL) return fail(TC_E_ARG, "unknown flag bits");
  std::lock_guard<std::mutex> lk(g_mu);
  const int prev = g_flags;
  g_flags = flags;
  return prev;
}

int tc_get_flags(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_flags;
}

int tc_layout_slice(const tc_layout* in, const int64_t* start, const int64_t* stop, const int64_t* step,
                    tc_layout* out) {
  g_err.clear();
  if (!in || !out || (in->rank > 0 && (!start || !stop || !step))) return fail(TC_E_NULL, "null pointer argument");
  std::string err;
  const int rc = tc::slice_layout(*in, start, stop, step, out, &err);
  if (rc != TC_OK) return fail(rc, err);
  return TC_OK;
}

int tc_version(void) { return 200; }

}  // extern "C"
