// Device-side building blocks of the MXFP4 kernels (gfx950, wave64).
//
// E2M1 code: bit 3 = sign, bits 0-2 = index of the magnitude in
// {0, 0.5, 1, 1.5, 2, 3, 4, 6} (OCP MX v1.0; "ALTO MXFP4 training -- Weight
// de-oscillation", Jargon "E2M1": 2 exponent bits, 1 mantissa bit, about +-6).
// Shared scale: E8M0 byte = clamp(floor(log2 amax) - 2, -127, 127) + 127.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kBlock = 32;

// ---------------------------------------------------------------- shared scale
// Scale byte from the bit pattern of the block's largest magnitude (sign bit
// cleared).  For a normal amax with exponent field f, floor(log2 amax) = f - 127,
// so the byte is max(f - 2, 0); zero and subnormal amax (f = 0) give 0, the
// clamp at e = -127.  NaN/Inf (f = 255) gives the E8M0 NaN byte 0xFF.
__device__ __forceinline__ uint32_t scale_byte_of(uint32_t amax_bits) {
  const uint32_t f = amax_bits >> 23;
  if (f == 255u) return 255u;
  return f > 2u ? f - 2u : 0u;
}

// 2^-e for scale byte b = e + 127 (b <= 252 for any finite block), as a normal float.
__device__ __forceinline__ float inv_scale_of(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// 2^e for scale byte b = e + 127 (b = 0 gives the float32 subnormal 2^-127,
// b = 0xFF gives +Inf, which makes every scaled decode below NaN).
__device__ __forceinline__ float scale_of(uint32_t byte) {
  return __uint_as_float(byte ? byte << 23 : 0x00400000u);
}

// Decode of packed codes with gfx950's scaled FP4 -> float32 conversion, which
// is exact: code * 2^(byte - 127) (subnormal results kept, values beyond the
// float32 range +-Inf), NaN for every code under scale byte 0xFF.  `sel` picks
// the byte of w; the low nibble gives .x.
typedef float mx_v2f __attribute__((ext_vector_type(2)));
template <int SEL>
__device__ __forceinline__ mx_v2f decode_byte(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}

// The 8 codes of w (element i in nibble i) under scale byte `byte`.
__device__ __forceinline__ void decode8(uint32_t w, uint32_t byte, float v[8]) {
  const float s = scale_of(byte);
  const mx_v2f r0 = decode_byte<0>(w, s), r1 = decode_byte<1>(w, s);
  const mx_v2f r2 = decode_byte<2>(w, s), r3 = decode_byte<3>(w, s);
  v[0] = r0.x; v[1] = r0.y; v[2] = r1.x; v[3] = r1.y;
  v[4] = r2.x; v[5] = r2.y; v[6] = r3.x; v[7] = r3.y;
}

// ---------------------------------------------------------------- rounding
// Nearest E2M1 magnitude index for a in [0, 8), ties to the even index.
//  a < 1: the grid is the multiples of 0.5; adding 2^22 (ulp 0.5) rounds to
//         nearest even in hardware, and the bit pattern offset is the index.
//  a >= 1: round the float32 mantissa to one bit, nearest even (carry into the
//         exponent is the next binade); index = (exponent<<1 | mantissa) - 252.
//  Values in (6, 8) saturate to index 7 (= 6).
__device__ __forceinline__ uint32_t e2m1_rne(float a) {
  const uint32_t b = __float_as_uint(a);
  const uint32_t sub = __float_as_uint(a + 4194304.0f) - 0x4A800000u;
  uint32_t nrm = (b + 0x1FFFFFu + ((b >> 22) & 1u) - 0x3F000000u) >> 22;
  nrm = nrm < 7u ? nrm : 7u;
  return a < 1.0f ? sub : nrm;
}

// gfx950 conversions of a pair of float32 values to E2M1 codes after division by
// a power-of-two scale (exact).  Only the low byte of the result is defined: the
// code of v0 in bits 0..3, of v1 in bits 4..7; the sign bit always copies the
// input's, magnitudes at or above 6 give 6 (as do NaN and Inf, which the callers
// never pass: such blocks take the NaN scale byte and zero codes).
//  cvt_rne_pair: nearest magnitude, ties to the even code.
//  cvt_sr_pair:  with a = |v| / scale between neighbours lo <= a < hi and
//                t = floor((a - lo) / (hi - lo) * 2^22), v0 takes hi iff
//                t + (seed >> 10) >= 2^22 and v1 iff t + ((seed >> 9) & (2^22 - 1))
//                >= 2^22 -- 22 random bits added below the kept precision.
__device__ __forceinline__ uint32_t cvt_rne_pair(float v0, float v1, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0, v1, scale, 0);
}

__device__ __forceinline__ uint32_t cvt_sr_pair(float v0, float v1, uint32_t seed, float scale) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f v = {v0, v1};
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v, seed, scale, 0);
}

// ---------------------------------------------------------------- SplitMix64
// Steele, Lea & Flood, "Fast splittable pseudorandom number generators"
// (OOPSLA 2014): output number idx+1 from state `seed` is the variant-13
// finalizer applied to seed + (idx+1) * 0x9E3779B97F4A7C15.
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t sm64_state(uint64_t seed, uint64_t idx) {
  return seed + (idx + 1ull) * kGamma;
}

// Top 24 bits of the output for state z (the synthetic update generator's
// uniforms): the last xor-shift (by 31) leaves bits 33..63 unchanged, so only
// the high word of the last product is needed.
__device__ __forceinline__ uint32_t sm64_top24(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  const uint32_t lo = (uint32_t)z, hi = (uint32_t)(z >> 32);
  const uint32_t h = __umulhi(lo, 0x133111EBu) + lo * 0x94D049BBu + hi * 0x133111EBu;
  return h >> 8;
}

// Stochastic rounding draws one output per adjacent pair (2i, 2i+1) of a block,
// keyed by element 2i's index: element 2i reads bits 42..63 of the output,
// element 2i+1 bits 9..30.  Returns words whose bits 10..31 (hi) and 9..30 (lo)
// are those output bits: the final z ^ (z >> 31) leaves bits 33..63 unchanged,
// and in its low word bits 9..30 of z are xored with z's bits 40..61, which are
// bits 8..29 of the high word: (hi << 1) at bits 9..30.
__device__ __forceinline__ void sm64_words(uint64_t z, uint32_t& hi, uint32_t& lo) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  hi = (uint32_t)(z >> 32);
  lo = (uint32_t)z ^ (hi << 1);
}

// ---------------------------------------------------------------- cross-lane
// DPP quad permutations: lane i of each group of 4 reads lane perm[i].
constexpr int kQuadSwap1 = 0xB1;  // [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;  // [2, 3, 0, 1]

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Largest magnitude of v[0..n) as a float32 bit pattern, with gfx950's
// NaN-propagating maximum and |.| operand modifiers (v_maximum3_f32: half an
// instruction per value).  Non-negative floats order as their bit patterns, so
// this is the integer maximum of the sign-cleared patterns, except that a NaN
// input may come out as another NaN pattern; every NaN pattern (exponent field
// 255) gives the same scale byte 0xFF.
template <int N>
__device__ __forceinline__ uint32_t amax_bits(const float* v) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = __builtin_elementwise_maximum(m, __builtin_fabsf(v[i]));
  return __float_as_uint(m);
}

// Largest sign-cleared bit pattern over the 4 lanes of a quad (integer max of
// |x| patterns: exact, and NaN/Inf patterns win).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadSwap1>(v));
  v = max(v, dpp_u32<kQuadSwap2>(v));
  return v;
}

// ---------------------------------------------------------------- Hadamard
// Unnormalised 32-point Walsh-Hadamard transform (Sylvester order) in float32,
// butterflies (a, b) -> (a + b, a - b) at distance h = 1, 2, 4, 8, 16.
// Quad form: lane q (0..3) of a quad holds elements 8q .. 8q+7.
__device__ __forceinline__ void fwht32_quad(float v[8], int q) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = dpp_f32<kQuadSwap1>(v[i]);  // partner at distance 8
    v[i] = (q & 1) ? (p - v[i]) : (v[i] + p);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = dpp_f32<kQuadSwap2>(v[i]);  // partner at distance 16
    v[i] = (q & 2) ? (p - v[i]) : (v[i] + p);
  }
}

// In-register form: one lane holds all 32 elements.
__device__ __forceinline__ void fwht32_lane(float v[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

__device__ __forceinline__ float apply_sign(float v, uint32_t mask, int j) {
  return ((mask >> j) & 1u) ? -v : v;
}

// ---------------------------------------------------------------- decode
// Signed E2M1 value of a code: twice the magnitudes {0,1,2,3,4,6,8,12} are
// packed as nibbles of one constant and halved.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t twice = (0xC8643210u >> ((code & 7u) * 4u)) & 0xFu;
  const float m = (float)twice * 0.5f;
  return (code & 8u) ? -m : m;
}

// Exact value of code * 2^(byte - 127) (may be subnormal); byte 0xFF -> NaN.
__device__ __forceinline__ float e2m1_decode(uint32_t code, uint32_t byte) {
  if (byte == 255u) return __uint_as_float(0x7FC00000u);
  return __builtin_amdgcn_ldexpf(e2m1_value(code), (int)byte - 127);
}

// bf16 <-> float32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;  // quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace mx
