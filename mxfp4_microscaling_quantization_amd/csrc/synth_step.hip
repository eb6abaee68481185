// The synthetic optimizer step that drives the de-oscillation workload
// (include/mx_synth.h).  A workload generator, not part of the method: it is
// built into its own library, libmx355_synth.so, beside the product library.
//
// It stands in for the AdamW updates after which "ALTO MXFP4 training -- Weight
// de-oscillation" runs its hook: every weight moves by an Irwin-Hall(4) step of
// standard deviation 1e-4 made from four 24-bit SplitMix64 draws (Steele, Lea &
// Flood, OOPSLA 2014), so a CPU replay is bit-exact without a transcendental
// function.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"
#include "mx_host.h"
#include "../../include/mx_synth.h"

namespace mx {

constexpr uint32_t kSynthScaleBits = 0x2D359E63u;  // f32(sqrt(3) * 1e-4 * 2^-24)

__global__ __launch_bounds__(256) void k_synth_step(float* __restrict__ w, int64_t n,
                                                    uint64_t seed, uint64_t step) {
  const float c = __uint_as_float(kSynthScaleBits);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int32_t acc = 0;
#pragma unroll
    for (uint64_t k = 0; k < 4; ++k) {
      const uint64_t ctr = (step << 42) | (k << 40) | (uint64_t)i;
      acc += (int32_t)sm64_top24(sm64_state(seed, ctr));
    }
    const float dw = (float)(acc - (1 << 25)) * c;
    w[i] = w[i] + dw;
  }
}

}  // namespace mx

using namespace mx;

extern "C" int mx_synth_step(float* w, int64_t n, uint64_t seed, int64_t step, void* stream) {
  MX_REQUIRE(n >= 0 && n < ((int64_t)1 << 40) && step >= 0 && step < ((int64_t)1 << 22),
             MX_ERR_SHAPE);
  if (n == 0) return MX_OK;
  MX_REQUIRE(w, MX_ERR_NULL);
  MX_REQUIRE(aligned16(w), MX_ERR_ALIGN);
  const dim3 grid((unsigned)hmin(cdiv(n, 256), 256 * 64));
  k_synth_step<<<grid, 256, 0, as_stream(stream)>>>(w, n, seed, (uint64_t)step);
  return launch_status();
}
