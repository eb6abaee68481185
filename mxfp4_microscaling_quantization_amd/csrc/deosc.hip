// Weight de-oscillation as a post-optimizer-step pass.
//
// "ALTO MXFP4 training -- Weight de-oscillation": over a window of P = 200
// optimizer steps, sum per element how far the master weight travelled (d_w)
// and how far its quantized value jumped (d_Q); at the end of the window flag
// elements with d_Q / d_w > 4.0 and snap them to the centre of their current
// bin; it runs after each AdamW step and needs no extra matrix multiply.
//
// The bin value q(w) is the forward weight quantizer's output: 1x32 RNE blocks
// along the columns.  One quad (4 lanes) handles one block: each lane holds 8
// consecutive elements of w, w_prev, d_w and d_q (two 16-byte loads each), the
// two block maxima are DPP quad reductions, and all arithmetic is float32 in
// the order the pass is defined (no fused multiply-add).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"
#include "mx_host.h"

namespace mx {

__device__ __forceinline__ void ld8(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void st8(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Q_D of a lane's 8 elements (the quad holds one 1x32 block): returns the 8
// packed codes (element i in nibble i) and the block's scale byte; a NaN/Inf
// block gets scale 0xFF and zero codes.
__device__ __forceinline__ uint32_t quant8_rne(const float v[8], uint32_t& byte_out) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  m = quad_max_u32(m);
  const uint32_t byte = scale_byte_of(m);
  byte_out = byte;
  if (byte == 255u) return 0u;
  const float inv = inv_scale_of(byte);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = e2m1_rne(fabsf(v[i]) * inv) | ((__float_as_uint(v[i]) >> 28) & 8u);
    packed |= code << (4 * i);
  }
  return packed;
}

// Bin values q(v) = deq(Q_D(v)) of a lane's 8 elements; returns the packed codes.
__device__ __forceinline__ uint32_t bin8(const float v[8], float out[8], uint32_t& byte_out) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  m = quad_max_u32(m);
  const uint32_t byte = scale_byte_of(m);
  byte_out = byte;
  const float inv = inv_scale_of(byte);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = e2m1_rne(fabsf(v[i]) * inv) | ((__float_as_uint(v[i]) >> 28) & 8u);
    out[i] = e2m1_decode(code, byte);
    packed |= code << (4 * i);
  }
  return byte == 255u ? 0u : packed;
}

// QOUT: also write Q_D of the updated weight (codes [rows][cols/2], scales
// [rows][cols/32]).  Snapping a flagged element to its bin value leaves the
// block scale and the element's code unchanged, so the codes of w computed for
// d_Q are those of the updated weight.
template <bool END, bool QOUT>
__global__ __launch_bounds__(256) void k_deosc_step(float* __restrict__ w,
                                                    float* __restrict__ w_prev,
                                                    float* __restrict__ d_w,
                                                    float* __restrict__ d_q, int64_t nblk,
                                                    float threshold, uint8_t* __restrict__ flags,
                                                    uint32_t* __restrict__ wq_codes,
                                                    uint8_t* __restrict__ wq_scales) {
  const int q = threadIdx.x & 3;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 2);
  for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 2) + (threadIdx.x >> 2); b < nblk;
       b += stride) {
    const int64_t off = b * 32 + q * 8;
    float cw[8], pw[8], dw[8], dq[8], qn[8], qp[8];
    ld8(w + off, cw);
    ld8(w_prev + off, pw);
    ld8(d_w + off, dw);
    ld8(d_q + off, dq);
    uint32_t byte_n, byte_p;
    const uint32_t codes_n = bin8(cw, qn, byte_n);
    bin8(pw, qp, byte_p);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dw[i] = dw[i] + fabsf(cw[i] - pw[i]);
      dq[i] = dq[i] + fabsf(qn[i] - qp[i]);
    }
    if (END) {
      uint32_t f_lo = 0, f_hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lim = threshold * dw[i];
        const bool flag = dq[i] > lim;
        cw[i] = flag ? qn[i] : cw[i];
        if (i < 4) f_lo |= (flag ? 1u : 0u) << (8 * i);
        else f_hi |= (flag ? 1u : 0u) << (8 * (i - 4));
        dw[i] = 0.0f;
        dq[i] = 0.0f;
      }
      st8(w + off, cw);
      *reinterpret_cast<uint2*>(flags + off) = make_uint2(f_lo, f_hi);
    }
    st8(w_prev + off, cw);
    st8(d_w + off, dw);
    st8(d_q + off, dq);
    if (QOUT) {
      wq_codes[b * 4 + q] = codes_n;
      if (q == 0) wq_scales[b] = (uint8_t)byte_n;
    }
  }
}

// Q-EMA ("Oscillation-Reduced MXFP4 Training for Vision Transformers",
// rebuttal: Question 4 and the overhead / hyperparameter answers): after each
// optimizer step the EMA copy of the weight is updated and the forward pass
// quantizes the EMA.  float32 in this order: ema = (beta ema) + ((1 - beta) w).
// One quad per 1x32 block; the new EMA's Q_D goes straight to the caller.
__global__ __launch_bounds__(256) void k_qema_step(const float* __restrict__ w,
                                                   float* __restrict__ ema, int64_t nblk,
                                                   float beta, uint32_t* __restrict__ wq_codes,
                                                   uint8_t* __restrict__ wq_scales) {
  const int q = threadIdx.x & 3;
  const float omb = 1.0f - beta;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 2);
  for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 2) + (threadIdx.x >> 2); b < nblk;
       b += stride) {
    const int64_t off = b * 32 + q * 8;
    float cw[8], e[8];
    ld8(w + off, cw);
    ld8(ema + off, e);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = beta * e[i] + omb * cw[i];
    st8(ema + off, e);
    uint32_t byte;
    wq_codes[b * 4 + q] = quant8_rne(e, byte);
    if (q == 0) wq_scales[b] = (uint8_t)byte;
  }
}

__global__ __launch_bounds__(256) void k_deosc_init(const float4* __restrict__ w,
                                                    float4* __restrict__ w_prev,
                                                    float4* __restrict__ d_w,
                                                    float4* __restrict__ d_q, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    w_prev[i] = w[i];
    d_w[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    d_q[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

static int deosc_launch(float* w, int64_t rows, int64_t cols, float* w_prev, float* d_w, float* d_q,
                        int end, float threshold, uint8_t* flags, uint32_t* wq_codes,
                        uint8_t* wq_scales, hipStream_t st) {
  const int64_t nblk = rows * cols / 32;
  const dim3 grid((unsigned)hmin(cdiv(nblk, 64), 256 * 32));
#define MX_DEOSC_ARGS w, w_prev, d_w, d_q, nblk, threshold, flags, wq_codes, wq_scales
  if (wq_codes) {
    if (end) k_deosc_step<true, true><<<grid, 256, 0, st>>>(MX_DEOSC_ARGS);
    else k_deosc_step<false, true><<<grid, 256, 0, st>>>(MX_DEOSC_ARGS);
  } else {
    if (end) k_deosc_step<true, false><<<grid, 256, 0, st>>>(MX_DEOSC_ARGS);
    else k_deosc_step<false, false><<<grid, 256, 0, st>>>(MX_DEOSC_ARGS);
  }
#undef MX_DEOSC_ARGS
  return launch_status();
}

}  // namespace mx

using namespace mx;

extern "C" int mx_deosc_init(const float* w, int64_t rows, int64_t cols, float* w_prev,
                             float* d_w, float* d_q, void* stream) {
  MX_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(w && w_prev && d_w && d_q, MX_ERR_NULL);
  MX_REQUIRE(aligned16(w) && aligned16(w_prev) && aligned16(d_w) && aligned16(d_q), MX_ERR_ALIGN);
  const int64_t n4 = rows * cols / 4;
  const dim3 grid((unsigned)hmin(cdiv(n4, 256), 256 * 64));
  k_deosc_init<<<grid, 256, 0, as_stream(stream)>>>(
      reinterpret_cast<const float4*>(w), reinterpret_cast<float4*>(w_prev),
      reinterpret_cast<float4*>(d_w), reinterpret_cast<float4*>(d_q), n4);
  return launch_status();
}

extern "C" int mx_deosc_step(float* w, int64_t rows, int64_t cols, float* w_prev, float* d_w,
                             float* d_q, int end_of_window, float threshold, uint8_t* flags,
                             void* stream) {
  MX_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(end_of_window == 0 || end_of_window == 1, MX_ERR_ENUM);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(w && w_prev && d_w && d_q, MX_ERR_NULL);
  if (end_of_window) MX_REQUIRE(flags, MX_ERR_NULL);
  MX_REQUIRE(aligned16(w) && aligned16(w_prev) && aligned16(d_w) && aligned16(d_q), MX_ERR_ALIGN);
  if (end_of_window) MX_REQUIRE(aligned16(flags), MX_ERR_ALIGN);
  return deosc_launch(w, rows, cols, w_prev, d_w, d_q, end_of_window, threshold, flags, nullptr,
                      nullptr, as_stream(stream));
}

extern "C" int mx_deosc_step_quantize(float* w, int64_t rows, int64_t cols, float* w_prev,
                                      float* d_w, float* d_q, int end_of_window, float threshold,
                                      uint8_t* flags, uint8_t* wq_codes, uint8_t* wq_scales,
                                      void* stream) {
  MX_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(end_of_window == 0 || end_of_window == 1, MX_ERR_ENUM);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(w && w_prev && d_w && d_q && wq_codes && wq_scales, MX_ERR_NULL);
  if (end_of_window) MX_REQUIRE(flags, MX_ERR_NULL);
  MX_REQUIRE(aligned16(w) && aligned16(w_prev) && aligned16(d_w) && aligned16(d_q) &&
                 aligned16(wq_codes), MX_ERR_ALIGN);
  if (end_of_window) MX_REQUIRE(aligned16(flags), MX_ERR_ALIGN);
  return deosc_launch(w, rows, cols, w_prev, d_w, d_q, end_of_window, threshold, flags,
                      reinterpret_cast<uint32_t*>(wq_codes), wq_scales, as_stream(stream));
}

extern "C" int mx_qema_step(const float* w, float* ema, int64_t rows, int64_t cols, float beta,
                            uint8_t* wq_codes, uint8_t* wq_scales, void* stream) {
  MX_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(w && ema && wq_codes && wq_scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(w) && aligned16(ema) && aligned16(wq_codes), MX_ERR_ALIGN);
  const int64_t nblk = rows * cols / 32;
  const dim3 grid((unsigned)hmin(cdiv(nblk, 64), 256 * 32));
  k_qema_step<<<grid, 256, 0, as_stream(stream)>>>(w, ema, nblk, beta,
                                                   reinterpret_cast<uint32_t*>(wq_codes), wq_scales);
  return launch_status();
}
