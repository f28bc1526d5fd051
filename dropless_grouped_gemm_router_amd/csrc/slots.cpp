// Resident-workgroup counts for persistent kernels, and the fork/join of a
// call's shared-expert work onto the caller's second stream.
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

StreamFork::StreamFork(hipStream_t s, hipStream_t side) : caller_(s), side_(side) {}

hipError_t StreamFork::fork() {
  if (side_ == nullptr || side_ == caller_ || trace_on()) return hipSuccess;
  hipError_t e = hipEventCreateWithFlags(&ev_fork_, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_mark_, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_join_, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(ev_fork_, caller_);
  if (e == hipSuccess) e = hipStreamWaitEvent(side_, ev_fork_, 0);
  if (e == hipSuccess) forked_ = true;
  return e;
}

hipError_t StreamFork::mark() {
  if (!forked_) return hipSuccess;
  return hipEventRecord(ev_mark_, side_);
}

hipError_t StreamFork::wait_mark() {
  if (!forked_) return hipSuccess;
  return hipStreamWaitEvent(caller_, ev_mark_, 0);
}

hipError_t StreamFork::join() {
  if (!forked_ || joined_) return hipSuccess;
  hipError_t e = hipEventRecord(ev_join_, side_);
  if (e == hipSuccess) e = hipStreamWaitEvent(caller_, ev_join_, 0);
  if (e == hipSuccess) joined_ = true;
  return e;
}

StreamFork::~StreamFork() {
  (void)join();
  // An event may be released while work that records or waits for it is
  // still queued; the runtime frees it once that work has run.
  if (ev_fork_) (void)hipEventDestroy(ev_fork_);
  if (ev_mark_) (void)hipEventDestroy(ev_mark_);
  if (ev_join_) (void)hipEventDestroy(ev_join_);
}

}  // namespace moe
