// Host-side helpers shared by the library's entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace {

// How many workgroups of `kern` the current device keeps resident at once,
// and its CUs per XCD (0 when the CU count is not a multiple of the 8 XCDs).
// Queried once per kernel and device and cached: the values never change.
constexpr int kMaxDevices = 64;
struct Residency {
  int resident;
  int cus_per_xcd;
};
Residency residency(const void* kern, int threads, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return {0, 0};
  }
  int packed = cache[dev].load(std::memory_order_relaxed);
  if (packed == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess) {
      (void)hipGetLastError();
      return {0, 0};
    }
    packed = (cus * per_cu) * 1024 + (cus % 8 == 0 ? cus / 8 : 0) + 1;   // + 1: never 0 once known
    cache[dev].store(packed, std::memory_order_relaxed);
  }
  return {(packed - 1) / 1024, (packed - 1) % 1024};
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace
