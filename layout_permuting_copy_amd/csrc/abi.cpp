// C ABI of the tile-copy library: argument checks, plan cache, launch.
#include <hip/hip_runtime_api.h>

#include <algorithm>
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

std::string plan_key(const tc_layout& s, const tc_layout& d, int dtype, int flags, int align) {
  std::string key = layout_key(s) + layout_key(d);
  key.append(reinterpret_cast<const char*>(&dtype), sizeof(dtype));
  key.append(reinterpret_cast<const char*>(&flags), sizeof(flags));
  key.append(reinterpret_cast<const char*>(&align), sizeof(align));
  return key;
}

// Replaces the cached plan of `key` (tc_autotune's choice).
void put_plan(const std::string& key, std::shared_ptr<const tc::Plan> p) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_cache) g_cache = new std::unordered_map<std::string, std::shared_ptr<const tc::Plan>>();
  if (g_cache->size() >= kCacheMax) g_cache->clear();
  (*g_cache)[key] = std::move(p);
}

std::shared_ptr<const tc::Plan> get_plan(const tc_layout& s, const tc_layout& d, int dtype, int flags, int align) {
  const std::string key = plan_key(s, d, dtype, flags, align);
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

namespace {

// The argument checks of a copy and its (cached) plan: TC_OK with *plan set, or an error status
// (with *plan set where the planner ran, for the caller's info).
int checked_plan(const void* src, const tc_layout* src_layout, const void* dst, const tc_layout* dst_layout,
                 int dtype, int flags, std::shared_ptr<const tc::Plan>* plan, std::string* key) {
  if (!src || !dst || !src_layout || !dst_layout) return fail(TC_E_NULL, "null pointer argument");
  const int eb = tc::elem_bytes_of(dtype);
  if (eb < 0) return fail(TC_E_DTYPE, "unknown dtype " + std::to_string(dtype));
  if (flags & ~TC_FLAG_ALL) return fail(TC_E_ARG, "unknown flag bits");
  const uintptr_t ps = reinterpret_cast<uintptr_t>(src), pd = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t ealign = uintptr_t(eb < 16 ? eb : 16);
  if (ps % ealign || pd % ealign)
    return fail(TC_E_ALIGN, "base pointer not aligned to the element size (" + std::to_string(eb) + " bytes)");
  const int align = ptr_alignment(ps, pd);
  if (key) *key = plan_key(*src_layout, *dst_layout, dtype, flags, align);
  *plan = get_plan(*src_layout, *dst_layout, dtype, flags, align);
  const tc::Plan& p = **plan;
  if (p.status != TC_OK) return fail(p.status, p.reason);
  if (p.path == TC_PATH_EMPTY) return TC_OK;
  // the byte images of source and destination must not overlap (side_range gives [lo, hi) in
  // elements: hi is one past the last element)
  int64_t slo, shi, dlo, dhi;
  tc::side_range(p.j, true, &slo, &shi);
  tc::side_range(p.j, false, &dlo, &dhi);
  const __int128 s0 = __int128(ps) + __int128(slo) * eb, s1 = __int128(ps) + __int128(shi) * eb;
  const __int128 d0 = __int128(pd) + __int128(dlo) * eb, d1 = __int128(pd) + __int128(dhi) * eb;
  if (s0 < d1 && d0 < s1) return fail(TC_E_ALIAS, "source and destination byte ranges overlap");
  return TC_OK;
}

}  // namespace

extern "C" {

int tile_copy_ex(const void* src, const tc_layout* src_layout, void* dst, const tc_layout* dst_layout, int dtype,
                 void* stream, int flags, tc_plan_info* info) {
  g_err.clear();
  std::shared_ptr<const tc::Plan> plan;
  const int st = checked_plan(src, src_layout, dst, dst_layout, dtype, flags, &plan, nullptr);
  if (info && plan) tc::plan_to_info(*plan, info);
  if (st != TC_OK) return st;
  if (plan->path == TC_PATH_EMPTY) return TC_OK;
  std::string err;
  const int rc = tc::launch_plan(*plan, src, dst, stream, &err);
  if (rc != TC_OK) return fail(rc, err);
  return TC_OK;
}

int tc_autotune(const void* src, const tc_layout* src_layout, void* dst, const tc_layout* dst_layout, int dtype,
                void* stream, int flags, int reps, tc_plan_info* info, float* best_ms) {
  g_err.clear();
  std::shared_ptr<const tc::Plan> plan;
  std::string key;
  const int st = checked_plan(src, src_layout, dst, dst_layout, dtype, flags, &plan, &key);
  if (info && plan) tc::plan_to_info(*plan, info);
  if (st != TC_OK) return st;
  if (best_ms) *best_ms = 0.0f;
  if (plan->path == TC_PATH_EMPTY) return TC_OK;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return fail(TC_E_ARG, "tc_autotune times launches and cannot run on a capturing stream");
  if (reps <= 0) reps = 5;
  const std::vector<tc::Plan> cands = tc::plan_variants(*plan, flags);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(TC_E_HIP, "hipEventCreate failed");
  }
  // Three rounds over the candidates (each: a warm-up launch, then `reps` launches between the
  // events), so that drift over the measurement hits every candidate alike; a candidate's time is
  // its median round.  The planner's own plan (candidate 0) is kept unless another one is at least
  // 3% faster, or 10% where source and destination span less than twice the 256 MB MALL (the
  // repeated launches then find much of them cached: on the odd fp16 8191 x 8190 transpose a tile
  // 3% slower on fresh data had measured faster that way).
  constexpr int kRounds = 3;
  int64_t slo, shi, dlo, dhi;
  tc::side_range(plan->j, true, &slo, &shi);
  tc::side_range(plan->j, false, &dlo, &dhi);
  const double span = double(shi - slo + dhi - dlo) * plan->eb;
  const float margin = span < 512.0 * 1048576.0 ? 0.90f : 0.97f;
  std::vector<std::vector<float>> times(cands.size());
  std::string err;
  int rc = TC_OK;
  for (int round = 0; round < kRounds && rc == TC_OK; ++round)
    for (size_t i = 0; i < cands.size() && rc == TC_OK; ++i) {
      rc = tc::launch_plan(cands[i], src, dst, stream, &err);  // warm-up (and the copy itself)
      if (rc != TC_OK) break;
      (void)hipEventRecord(e0, s);
      for (int r = 0; r < reps && rc == TC_OK; ++r) rc = tc::launch_plan(cands[i], src, dst, stream, &err);
      (void)hipEventRecord(e1, s);
      if (rc != TC_OK) break;
      if (hipEventSynchronize(e1) != hipSuccess) {
        rc = TC_E_HIP;
        err = "hipEventSynchronize failed";
        break;
      }
      float ms = 0.0f;
      (void)hipEventElapsedTime(&ms, e0, e1);
      times[i].push_back(ms / float(reps));
    }
  int best = 0;
  float best_t = 0.0f;
  if (rc == TC_OK) {
    std::vector<float> med(cands.size());
    for (size_t i = 0; i < cands.size(); ++i) {
      std::vector<float> t = times[i];
      std::sort(t.begin(), t.end());
      med[i] = t[t.size() / 2];
    }
    best_t = med[0];
    for (size_t i = 1; i < cands.size(); ++i)
      if (med[i] < margin * med[0] && med[i] < best_t) {
        best = int(i);
        best_t = med[i];
      }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc != TC_OK) return fail(rc, err);
  auto chosen = std::make_shared<const tc::Plan>(cands[size_t(best)]);
  put_plan(key, chosen);
  if (info) tc::plan_to_info(*chosen, info);
  if (best_ms) *best_ms = best_t;
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

int tc_plan_variants(const tc_layout* src_layout, const tc_layout* dst_layout, int dtype, int flags, int ptr_align,
                     tc_plan_info* out, int max_out) {
  g_err.clear();
  if (!src_layout || !dst_layout || (!out && max_out > 0)) return fail(TC_E_NULL, "null pointer argument");
  if (ptr_align < 0 || (ptr_align & (ptr_align - 1))) return fail(TC_E_ARG, "ptr_align must be a power of two");
  if (ptr_align == 0 || ptr_align > 16) ptr_align = 16;
  const tc::Plan p = tc::make_plan(*src_layout, *dst_layout, dtype, flags, ptr_align);
  if (p.status != TC_OK) {
    if (max_out > 0) tc::plan_to_info(p, out);
    return fail(p.status, p.reason);
  }
  const std::vector<tc::Plan> v = tc::plan_variants(p, flags);
  for (int i = 0; i < max_out && i < int(v.size()); ++i) tc::plan_to_info(v[size_t(i)], out + i);
  return int(v.size());
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
