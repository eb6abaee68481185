// Issue rate of the VALU instructions the quantizer kernels are made of, on
// gfx950: each lane runs 16 independent chains of one instruction (inline asm, so
// the compiler can neither fold nor reorder them) for ITER rounds.  Per wave,
// s_memtime (shader clock) and s_memrealtime (100 MHz) bracket the loop, so the
// cycles a SIMD spends per wave-level instruction and the clock follow without
// knowing the clock in advance; hip events give the chip-wide lane-op rate.
//
// A second kernel runs the stochastic quantizers' per-pair sequence from the
// library's own device helpers (one SplitMix64 output and two stochastic FP4
// conversions per element pair), 8 independent pairs per lane: the rate at which
// the chip can produce stochastic-rounding decisions with no memory traffic.
//
// Output: one JSON object per measurement on stdout.  The kernels read no memory
// and write one word per lane and two per wave, into buffers sized from the same
// grid constants.
#include <hip/hip_runtime.h>

#include "../mxfp4_microscaling_quantization_amd/csrc/mx_device.h"

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

constexpr int kIter = 1024;
constexpr int kChains = 16;
constexpr int kThreads = 256;  // four waves per workgroup

enum Op { ADD, XOR, FMAC, MUL_LO, MUL_HI, MAD_U64, LSHR_B64, CVT_PK_FP4, CVT_SR_PK_FP4, NOPS };
const char* kNames[NOPS] = {"v_add_u32",    "v_xor_b32",     "v_fmac_f32",
                            "v_mul_lo_u32", "v_mul_hi_u32",  "v_mad_u64_u32",
                            "v_lshrrev_b64", "v_cvt_scalef32_pk_fp4_f32",
                            "v_cvt_scalef32_sr_pk_fp4_f32"};

template <int OP>
__global__ __launch_bounds__(kThreads) void k_rate(uint32_t* out, uint64_t* times, uint32_t c) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  uint32_t x[kChains];
  uint64_t y[kChains];
  float f[kChains];
  for (int i = 0; i < kChains; ++i) {
    x[i] = threadIdx.x * 7u + i;
    y[i] = ((uint64_t)x[i] << 32) | (x[i] * 3u);
    f[i] = (float)x[i];
  }
  const v2f pair = {1.5f + (float)threadIdx.x, -2.25f};
  const float scale = 1.0f, a = 1.0001f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < kIter; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
      if constexpr (OP == ADD) asm volatile("v_add_u32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
      if constexpr (OP == XOR) asm volatile("v_xor_b32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
      if constexpr (OP == FMAC) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(f[i]) : "v"(a), "v"(scale));
      if constexpr (OP == MUL_LO) asm volatile("v_mul_lo_u32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
      if constexpr (OP == MUL_HI) asm volatile("v_mul_hi_u32 %0, %0, %1" : "+v"(x[i]) : "v"(c));
      if constexpr (OP == MAD_U64) {
        uint64_t carry;
        asm volatile("v_mad_u64_u32 %0, %1, %2, %3, %0" : "+v"(y[i]), "=s"(carry) : "v"(x[i]), "v"(c));
      }
      if constexpr (OP == LSHR_B64) asm volatile("v_lshrrev_b64 %0, 1, %0" : "+v"(y[i]));
      if constexpr (OP == CVT_PK_FP4)
        asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, %3" : "+v"(x[i]) : "v"(f[i]), "v"(a), "v"(scale));
      if constexpr (OP == CVT_SR_PK_FP4)
        asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %0, %2" : "+v"(x[i]) : "v"(pair), "v"(scale));
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  uint32_t acc = 0;
  for (int i = 0; i < kChains; ++i)
    acc ^= x[i] ^ (uint32_t)y[i] ^ (uint32_t)(y[i] >> 32) ^ __float_as_uint(f[i]);
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  out[gid] = acc;
  if ((threadIdx.x & 63) == 0) {
    times[2 * (gid >> 6)] = t1 - t0;
    times[2 * (gid >> 6) + 1] = r1 - r0;
  }
}

template <int OP>
int measure(int cus, int waves_per_simd, uint32_t* out, uint64_t* times) {
  const int blocks = cus * waves_per_simd;  // 4 waves per block, one per SIMD
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int r = 0; r < 2; ++r) k_rate<OP><<<blocks, kThreads>>>(out, times, 3u);
  CHECK(hipGetLastError());
  constexpr int kReps = 5;
  CHECK(hipEventRecord(e0));
  for (int r = 0; r < kReps; ++r) k_rate<OP><<<blocks, kThreads>>>(out, times, 3u);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const int waves = blocks * 4;
  std::vector<uint64_t> h(2 * (size_t)waves);
  CHECK(hipMemcpy(h.data(), times, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
  std::vector<double> cyc(waves), ghz(waves);
  for (int w = 0; w < waves; ++w) {
    cyc[w] = (double)h[2 * w];
    ghz[w] = h[2 * w + 1] ? (double)h[2 * w] / ((double)h[2 * w + 1] * 10.0) : 0.0;
  }
  std::sort(cyc.begin(), cyc.end());
  std::sort(ghz.begin(), ghz.end());
  const double lane_ops = (double)blocks * kThreads * kIter * kChains * kReps;
  std::printf("{\"instr\": \"%s\", \"waves_per_simd\": %d, \"us_per_launch\": %.2f, "
              "\"lane_ops_per_s\": %.4e, \"cycles_per_instr\": %.3f, \"clock_ghz\": %.3f}\n",
              kNames[OP], waves_per_simd, ms * 1e3 / kReps, lane_ops / (ms * 1e-3),
              cyc[waves / 2] / ((double)waves_per_simd * kIter * kChains), ghz[waves / 2]);
  std::fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return 0;
}

template <int OP>
int measure_all(int cus, uint32_t* out, uint64_t* times) {
  for (int w : {1, 4})
    if (measure<OP>(cus, w, out, times)) return 1;
  if constexpr (OP + 1 < NOPS) return measure_all<OP + 1>(cus, out, times);
  return 0;
}

// MODE 0: SplitMix64 words + two conversions + merge (the quantizers' pair);
// MODE 1: the SplitMix64 words alone; MODE 2: one stochastic conversion alone.
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_sr_pairs(uint32_t* out, uint64_t seed, float a) {
  constexpr int kPairs = 8;
  constexpr int kRounds = 256;
  float v0[kPairs], v1[kPairs];
  uint64_t z[kPairs];
  uint32_t acc[kPairs];
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  for (int i = 0; i < kPairs; ++i) {
    v0[i] = a * (float)(threadIdx.x + i);
    v1[i] = -a * (float)(i + 3);
    z[i] = mx::sm64_state(seed, (uint64_t)gid * kPairs + i);
    acc[i] = 0;
  }
  for (int it = 0; it < kRounds; ++it) {
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      if constexpr (MODE == 0) {
        uint32_t hi, lo;
        mx::sm64_words(z[i], hi, lo);
        const uint32_t b0 = mx::cvt_sr_pair(v0[i], v1[i], hi, 0.5f);
        const uint32_t b1 = mx::cvt_sr_pair(v0[i], v1[i], lo, 0.5f);
        acc[i] ^= (b0 & 0x0Fu) | (b1 & ~0x0Fu);
      }
      if constexpr (MODE == 1) {
        uint32_t hi, lo;
        mx::sm64_words(z[i], hi, lo);
        acc[i] ^= hi ^ lo;
      }
      if constexpr (MODE == 2) acc[i] ^= mx::cvt_sr_pair(v0[i], v1[i], acc[i] + (uint32_t)z[i], 0.5f);
      z[i] += 2 * mx::kGamma;
    }
  }
  uint32_t r = 0;
  for (int i = 0; i < kPairs; ++i) r ^= acc[i];
  out[gid] = r;
}

template <int MODE>
int measure_sr(int cus, uint32_t* out) {
  const int blocks = cus * 8;  // eight waves per SIMD
  const char* names[3] = {"sr_pair", "splitmix64_words", "cvt_sr_pair"};
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  k_sr_pairs<MODE><<<blocks, kThreads>>>(out, 1, 1.1f);
  CHECK(hipGetLastError());
  constexpr int kReps = 5;
  CHECK(hipEventRecord(e0));
  for (int r = 0; r < kReps; ++r) k_sr_pairs<MODE><<<blocks, kThreads>>>(out, 1, 1.1f);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double pairs = (double)blocks * kThreads * 256 * 8 * kReps;
  const double per_s = pairs / (ms * 1e-3);
  std::printf("{\"sequence\": \"%s\", \"pairs_per_s\": %.4e, \"us_per_8192sq_elements\": %.2f}\n",
              names[MODE], per_s, 8192.0 * 8192.0 / 2.0 / per_s * 1e6);
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
  const int max_blocks = cus * 8;
  uint32_t* out = nullptr;
  uint64_t* times = nullptr;
  CHECK(hipMalloc(&out, (size_t)max_blocks * kThreads * sizeof(uint32_t)));
  CHECK(hipMalloc(&times, (size_t)max_blocks * 4 * 2 * sizeof(uint64_t)));
  std::printf("{\"cus\": %d, \"arch\": \"%s\"}\n", cus, prop.gcnArchName);
  int rc = measure_all<0>(cus, out, times);
  if (rc == 0) rc = measure_sr<0>(cus, out) || measure_sr<1>(cus, out) || measure_sr<2>(cus, out);
  CHECK(hipFree(out));
  CHECK(hipFree(times));
  return rc;
}
