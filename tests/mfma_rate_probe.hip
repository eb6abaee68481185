// Sustained rate of gfx950's block-scaled FP4 matrix instruction
// (V_MFMA_SCALE_F32_32X32X64_F8F6F4, both operands E2M1) with its operands in
// registers and no memory traffic, under the data the MXFP4 GEMM feeds it:
// the ceiling a GEMM built on this instruction can reach on this chip.
//
// Like the GEMM, one 512-thread workgroup per CU (two waves per SIMD), each wave
// holding eight 32x32 float32 accumulators and issuing independent MFMAs.  The
// operand data is one of:
//   zero     all codes 0 (no multiplier input toggles),
//   fixed    random codes, the same registers for every MFMA of a wave,
//   rotating random codes, a different register set for consecutive MFMAs
//            (what the GEMM does: every MFMA gets new fragments),
//   rotating_scales  as rotating, with random E8M0 scales as well.
// Each mode runs ~0.4 s of back-to-back launches so that the clock settles under
// its power draw; s_memtime (shader clock) and s_memrealtime (100 MHz) bracket
// each wave's loop, so the clock follows without knowing it in advance.
//
// Output: one JSON object per mode on stdout.  The kernel reads nothing and
// writes one word per lane and two per wave, into buffers sized from the grid.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                               \
    }                                                                         \
  } while (0)

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;   // eight waves: two per SIMD
constexpr int kAcc = 8;         // accumulator tiles per wave
constexpr int kIter = 4096;     // rounds of kAcc MFMAs per launch
constexpr int kFp4 = 4;         // operand format E2M1

enum Mode { ZERO, FIXED, ROTATING, ROTATING_SCALES, NMODES };
const char* kModeNames[NMODES] = {"zero", "fixed", "rotating", "rotating_scales"};

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_mfma(float* out, uint64_t* times, uint32_t seed) {
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  // four A and two B operand sets per lane (16 code bytes each)
  v8i a[4], b[2];
  for (int s = 0; s < 4; ++s)
    for (int d = 0; d < 8; ++d)
      a[s][d] = (MODE == ZERO || d >= 4) ? 0 : (int)mix(seed ^ (gid * 64 + s * 8 + d));
  for (int s = 0; s < 2; ++s)
    for (int d = 0; d < 8; ++d)
      b[s][d] = (MODE == ZERO || d >= 4) ? 0 : (int)mix(~seed ^ (gid * 64 + s * 8 + d));
  // scale bytes 127 (x1) or random in [120, 135] (products stay finite)
  int sa[2], sb[2];
  for (int s = 0; s < 2; ++s) {
    const uint32_t r = mix(seed + 77 * gid + s);
    sa[s] = MODE == ROTATING_SCALES ? (int)(120 + (r & 15)) : 127;
    sb[s] = MODE == ROTATING_SCALES ? (int)(120 + ((r >> 8) & 15)) : 127;
  }
  v16f acc[kAcc];
  for (int t = 0; t < kAcc; ++t)
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;

  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < kIter; it += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int t = 0; t < kAcc; ++t) {
        // rotating modes: consecutive MFMAs take different operand registers
        const int ia = (MODE >= ROTATING) ? ((t + 2 * h) & 3) : 0;
        const int ib = (MODE >= ROTATING) ? ((t >> 2) ^ h) & 1 : 0;
        const int is = (MODE == ROTATING_SCALES) ? (t & 1) : 0;
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            b[ib], a[ia], acc[t], kFp4, kFp4, 0, sb[is], 0, sa[is]);
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int t = 0; t < kAcc; ++t)
    for (int e = 0; e < 16; ++e) s += acc[t][e];
  out[gid] = s;
  if ((threadIdx.x & 63) == 0) {
    times[2 * (gid >> 6)] = t1 - t0;
    times[2 * (gid >> 6) + 1] = r1 - r0;
  }
}

template <int MODE>
int measure(int cus, float* out, uint64_t* times) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  // one launch to learn its length, then ~0.4 s of launches, timed in two halves
  CHECK(hipEventRecord(e0));
  k_mfma<MODE><<<cus, kThreads>>>(out, times, 1234u);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms1 = 0.f;
  CHECK(hipEventElapsedTime(&ms1, e0, e1));
  const int reps = std::max(4, (int)(200.0 / std::max(ms1, 0.01f)));
  float ms[2] = {0.f, 0.f};
  for (int half = 0; half < 2; ++half) {
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) k_mfma<MODE><<<cus, kThreads>>>(out, times, 1234u + r);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms[half], e0, e1));
  }
  CHECK(hipGetLastError());
  const int waves = cus * kThreads / 64;
  std::vector<uint64_t> h(2 * (size_t)waves);
  CHECK(hipMemcpy(h.data(), times, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
  std::vector<double> ghz(waves);
  for (int w = 0; w < waves; ++w)
    ghz[w] = h[2 * w + 1] ? (double)h[2 * w] / ((double)h[2 * w + 1] * 10.0) : 0.0;
  std::sort(ghz.begin(), ghz.end());
  const double flop = 2.0 * 32 * 32 * 64 * kAcc * (double)kIter * waves * reps;
  const double tf_first = flop / (ms[0] * 1e-3) / 1e12, tf = flop / (ms[1] * 1e-3) / 1e12;
  // MFMA-busy fraction implied at the measured clock (32 cycles per instruction
  // per SIMD at the 10.1 PFLOP/s nominal rate, 4 SIMDs per CU)
  const double clk = ghz[waves / 2];
  const double busy = tf * 1e12 / (cus * 4.0 * clk * 1e9 * (2.0 * 32 * 32 * 64 / 32.0));
  std::printf("{\"mode\": \"%s\", \"tflops\": %.1f, \"tflops_first_half\": %.1f, "
              "\"frac_of_10100\": %.4f, \"clock_ghz\": %.3f, \"busy_at_clock\": %.3f, "
              "\"seconds\": %.3f}\n",
              kModeNames[MODE], tf, tf_first, tf / 10100.0, clk, busy, (ms[0] + ms[1]) * 1e-3);
  std::fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return 0;
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  float* out = nullptr;
  uint64_t* times = nullptr;
  CHECK(hipMalloc(&out, (size_t)cus * kThreads * sizeof(float)));
  CHECK(hipMalloc(&times, (size_t)cus * (kThreads / 64) * 2 * sizeof(uint64_t)));
  std::printf("{\"cus\": %d, \"arch\": \"%s\"}\n", cus, prop.gcnArchName);
  std::fflush(stdout);
  int rc = measure<ZERO>(cus, out, times) || measure<FIXED>(cus, out, times) ||
           measure<ROTATING>(cus, out, times) || measure<ROTATING_SCALES>(cus, out, times);
  CHECK(hipFree(out));
  CHECK(hipFree(times));
  return rc;
}
