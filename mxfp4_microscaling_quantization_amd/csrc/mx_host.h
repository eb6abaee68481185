// Host-side helpers shared by the entry points: status codes and checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mx.h"

namespace mx {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MX_OK : MX_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K plan of a GEMM: n chunks of kchunk K-values (the last may be shorter).
struct SplitPlan {
  int n;
  int64_t kchunk;
};
inline int64_t hmin(int64_t a, int64_t b) { return a < b ? a : b; }

// Compute units of the current device (queried once per device; 256 if the
// runtime cannot tell).
inline int device_cu_count() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static int cus[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace mx

#define MX_REQUIRE(cond, status) \
  do {                           \
    if (!(cond)) return (status); \
  } while (0)
