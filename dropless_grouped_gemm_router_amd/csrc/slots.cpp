// Resident-workgroup counts for persistent kernels, and the side stream that
// runs the shared expert beside the routed path.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "common.h"

namespace moe {

int persistent_slots(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_pair(dev, kernel);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int slots = cus * per_cu;
  cache[key] = slots;
  return slots;
}

int cu_count() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  cache[dev] = cus;
  return cus;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
hipStream_t g_side[kMaxDevices];
hipEvent_t g_fork[kMaxDevices], g_join[kMaxDevices], g_mark[kMaxDevices];
}  // namespace

SideFork::SideFork() : lock_(g_side_mu) {}

hipError_t SideFork::fork(hipStream_t s) {
  caller_ = s;
  if (trace_on()) {
    side_ = s;
    return hipSuccess;
  }
  hipError_t e = hipGetDevice(&dev_);
  if (e == hipSuccess && (dev_ < 0 || dev_ >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) return e;
  if (!g_side[dev_]) {
    e = hipStreamCreateWithFlags(&g_side[dev_], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&g_fork[dev_], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&g_join[dev_], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&g_mark[dev_], hipEventDisableTiming);
    if (e != hipSuccess) {
      g_side[dev_] = nullptr;
      return e;
    }
  }
  e = hipEventRecord(g_fork[dev_], s);
  if (e == hipSuccess) e = hipStreamWaitEvent(g_side[dev_], g_fork[dev_], 0);
  if (e == hipSuccess) side_ = g_side[dev_];
  return e;
}

hipError_t SideFork::mark() {
  // Nothing to order when the side stream is the caller's own (timer on).
  if (side_ == nullptr || side_ == caller_) return hipSuccess;
  return hipEventRecord(g_mark[dev_], side_);
}

hipError_t SideFork::wait_mark(hipStream_t s) {
  if (side_ == nullptr || side_ == caller_ || side_ == s) return hipSuccess;
  return hipStreamWaitEvent(s, g_mark[dev_], 0);
}

hipError_t SideFork::join(hipStream_t s) {
  if (side_ == s) return hipSuccess;
  hipError_t e = hipEventRecord(g_join[dev_], side_);
  if (e == hipSuccess) e = hipStreamWaitEvent(s, g_join[dev_], 0);
  return e;
}

}  // namespace moe
