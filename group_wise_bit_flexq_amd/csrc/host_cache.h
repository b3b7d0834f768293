// Host-side, per-device caches of launch-configuration facts (flexq HIP library).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace flexq {

// Launch-configuration facts the host code looks up once per device (occupancy, CU
// count, kernel attributes set): one slot per device index, published atomically, so
// first calls racing on several threads compute the same value and any one is kept.
// A lookup that fails (no device, runtime error) is not cached.
constexpr int kMaxDevices = 64;

inline int device_slot() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  return dev;
}

struct PerDeviceInt {
  std::atomic<int> v[kMaxDevices];  // zero-initialised as a static: "not known yet"
  // compute() returns a positive value, or <= 0 on failure (then `fallback` is
  // returned and the lookup is repeated on the next call)
  template <class F>
  int get(F compute, int fallback) {
    const int d = device_slot();
    int x = v[d].load(std::memory_order_acquire);
    if (x > 0) return x;
    x = compute();
    if (x <= 0) return fallback;
    v[d].store(x, std::memory_order_release);
    return x;
  }
};

}  // namespace flexq
