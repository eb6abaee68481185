/*
 * mx_synth.h -- device-side generator of the synthetic optimizer steps that
 * drive the de-oscillation workload, exported by libmx355_synth.so (not by the
 * product library libmx355.so).  It is a workload generator, not part of
 * the method: it stands in for the AdamW updates of a real training run
 * ("ALTO MXFP4 training -- Weight de-oscillation": the hook runs after each
 * AdamW step, which moves every weight by a small step).
 *
 * mx_synth_step: for i in [0, n): w[i] = f32(w[i] + dw_i) with
 *   u_k = SplitMix64(seed, (step << 42) | (k << 40) | i) >> 40, k = 0..3
 *   dw_i = f32(f32(u_0 + u_1 + u_2 + u_3 - 2^25) * c), c = f32(sqrt(3) 1e-4 2^-24)
 * an Irwin-Hall(4) step of standard deviation 1e-4 that needs no
 * transcendental function, so a CPU replay is bit-exact.  SplitMix64 output
 * number ctr+1 from state `seed` (Steele, Lea & Flood, OOPSLA 2014).
 * w: device, 16-byte aligned, n < 2^40, 0 <= step < 2^22.  Returns an mx_status.
 */
#ifndef MX355_MX_SYNTH_H
#define MX355_MX_SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mx_synth_step(float* w, int64_t n, uint64_t seed, int64_t step, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MX355_MX_SYNTH_H */
