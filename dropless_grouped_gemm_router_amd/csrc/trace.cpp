// Optional per-kernel timing: when enabled, every libmoe launch is bracketed
// by two hipEvents on its stream, and moe_trace_summary() reports the
// summed duration and count per kernel name. Disabled by default; the only
// cost when disabled is one relaxed atomic load per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {

namespace {

struct Mark {
  const char* name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Mark> g_marks;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void release_marks() {
  for (auto& m : g_marks) {
    if (m.start) g_pool.push_back(m.start);
    if (m.stop) g_pool.push_back(m.stop);
  }
  g_marks.clear();
}

}  // namespace

bool trace_on() { return g_on.load(std::memory_order_relaxed); }

void trace_push(hipStream_t s, const char* name) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Mark m{name, get_event(), nullptr};
  if (m.start) hipEventRecord(m.start, s);
  g_marks.push_back(m);
}

void trace_pop(hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto it = g_marks.rbegin(); it != g_marks.rend(); ++it) {
    if (!it->stop) {
      it->stop = get_event();
      if (it->stop) hipEventRecord(it->stop, s);
      return;
    }
  }
}

}  // namespace moe

MOE_EXPORT int moe_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(moe::g_mu);
  moe::release_marks();
  moe::g_on.store(on != 0);
  return MOE_OK;
}

MOE_EXPORT int moe_trace_summary(char* buf, size_t buf_bytes) {
  if (!buf || buf_bytes == 0) return MOE_ERR_INVALID;
  std::lock_guard<std::mutex> lk(moe::g_mu);
  std::map<std::string, std::pair<double, long>> agg;
  for (auto& m : moe::g_marks) {
    if (!m.start || !m.stop) continue;
    if (hipEventSynchronize(m.stop) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, m.start, m.stop) != hipSuccess) return MOE_ERR_HIP;
    auto& a = agg[m.name];
    a.first += ms;
    a.second += 1;
  }
  std::string out = "{";
  bool first = true;
  for (auto& kv : agg) {
    char tmp[256];
    std::snprintf(tmp, sizeof(tmp), "%s\"%s\": {\"ms\": %.6f, \"count\": %ld}", first ? "" : ", ",
                  kv.first.c_str(), kv.second.first, kv.second.second);
    out += tmp;
    first = false;
  }
  out += "}";
  if (out.size() + 1 > buf_bytes) return MOE_ERR_INVALID;
  std::memcpy(buf, out.c_str(), out.size() + 1);
  return MOE_OK;
}
