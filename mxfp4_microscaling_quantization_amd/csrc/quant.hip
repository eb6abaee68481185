// MXFP4 block quantizer kernels for gfx950: 1x32 row blocks, 32x1 column
// blocks (LDS-staged transpose), double quantization and dequantization.
//
// Method: "ALTO MXFP4 training -- Weight de-oscillation" (Jargon: MXFP4, E2M1,
// Bin, RHT, Stochastic rounding) and "Oscillation-Reduced MXFP4 Training for
// Vision Transformers" (rebuttal, Question 2: group shapes 1x32 / 32x1 and
// Q_S(Q_D(X))).  Scale and element conventions: OCP MX v1.0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"
#include "mx_host.h"

namespace mx {

// ============================================================== row blocks
// One quad (4 lanes) per 32-element block; lane q holds elements 8q..8q+7, so
// the loads are 16 B (bf16) or 2 x 16 B (f32) per lane, fully coalesced, and
// the block amax is two DPP quad swaps.  Row blocks are contiguous in memory:
// block b covers logical elements [32 b, 32 b + 32).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float v[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Quantize the 8 values a lane holds, given the block's scale byte; returns the
// 8 packed codes (element i in nibble i).  idx0 = logical index of v[0].
template <int ROUND>
__device__ __forceinline__ uint32_t quant8(const float v[8], uint32_t byte, uint64_t seed,
                                           uint64_t idx0) {
  if (byte == 255u) return 0u;
  const float inv = inv_scale_of(byte);
  uint32_t packed = 0;
  uint64_t z = 0;
  if (ROUND == MX_SR) z = sm64_state(seed, idx0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(v[i]) * inv;
    uint32_t c;
    if (ROUND == MX_SR) {
      c = e2m1_sr(a, sm64_top24(z));
      z += kGamma;
    } else {
      c = e2m1_rne(a);
    }
    c |= (__float_as_uint(v[i]) >> 28) & 8u;
    packed |= c << (4 * i);
  }
  return packed;
}

template <typename T, int ROUND, bool HAD>
__global__ __launch_bounds__(256) void k_quant_row(const T* __restrict__ x, int64_t nblk,
                                                   uint64_t seed, uint32_t sign_mask,
                                                   uint32_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  const int q = threadIdx.x & 3;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 2);
  for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 2) + (threadIdx.x >> 2); b < nblk;
       b += stride) {
    float v[8];
    load8<T>(x + b * 32 + q * 8, v);
    if (HAD) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = apply_sign(v[i], sign_mask, q * 8 + i);
      fwht32_quad(v, q);
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    m = quad_max_u32(m);
    const uint32_t byte = scale_byte_of(m);
    codes[b * 4 + q] = quant8<ROUND>(v, byte, seed, (uint64_t)b * 32 + q * 8);
    if (q == 0) scales[b] = (uint8_t)byte;
  }
}

// ============================================================== column blocks
// A workgroup owns a tile of 256 rows (8 row blocks) x 64 columns, staged in
// LDS in the input type.  Thread (c, g) quantizes column c for row blocks
// 2g, 2g+1 from LDS (consecutive lanes read consecutive columns of one row),
// and the codes go through a second LDS buffer so that each output row
// (= input column) is written as 128 contiguous bytes.
constexpr int kColTileR = 256;
constexpr int kColTileC = 64;

// Quantize 32 values of one column block; returns the 16 code bytes as uint4.
template <int ROUND>
__device__ __forceinline__ uint4 quant_col32(float v[32], uint32_t& byte_out, uint64_t seed,
                                             uint64_t idx0, uint64_t idx_step) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  const uint32_t byte = scale_byte_of(m);
  byte_out = byte;
  uint32_t w[4] = {0, 0, 0, 0};
  if (byte != 255u) {
    const float inv = inv_scale_of(byte);
    uint64_t z = 0, dz = 0;
    if (ROUND == MX_SR) {
      z = sm64_state(seed, idx0);
      dz = idx_step * kGamma;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float a = fabsf(v[i]) * inv;
      uint32_t c;
      if (ROUND == MX_SR) {
        c = e2m1_sr(a, sm64_top24(z));
        z += dz;
      } else {
        c = e2m1_rne(a);
      }
      c |= (__float_as_uint(v[i]) >> 28) & 8u;
      w[i >> 3] |= c << (4 * (i & 7));
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Writes the staged codes/scales of a column tile: out row (col0 + c) gets
// bytes [row0/2, row0/2 + nrb*16) of codes and [row0/32, row0/32 + nrb) of scales.
__device__ __forceinline__ void store_col_tile(const uint4* s_codes, const uint8_t* s_scales,
                                               int64_t rows, int64_t col0, int ncols, int64_t row0,
                                               int nrb, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
  const int64_t ld_c = rows / 2, ld_s = rows / 32;
  for (int i = threadIdx.x; i < kColTileC * 8; i += blockDim.x) {
    const int c = i >> 3, rb = i & 7;
    if (c < ncols && rb < nrb) {
      *reinterpret_cast<uint4*>(codes + (col0 + c) * ld_c + row0 / 2 + rb * 16) = s_codes[c * 8 + rb];
      scales[(col0 + c) * ld_s + row0 / 32 + rb] = s_scales[c * 8 + rb];
    }
  }
}

template <typename T, int ROUND, bool HAD>
__global__ __launch_bounds__(256) void k_quant_col(const T* __restrict__ x, int64_t rows,
                                                   int64_t cols, uint64_t seed, uint32_t sign_mask,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  __shared__ T s_in[kColTileR * kColTileC];
  __shared__ uint4 s_codes[kColTileC * 8];
  __shared__ uint8_t s_scales[kColTileC * 8];

  const int64_t col0 = (int64_t)blockIdx.x * kColTileC;
  const int64_t row0 = (int64_t)blockIdx.y * kColTileR;
  const int ncols = (int)min<int64_t>(kColTileC, cols - col0);
  const int nrows = (int)min<int64_t>(kColTileR, rows - row0);
  const int nrb = nrows / 32;

  // global -> LDS, 16-byte chunks (cols % 8 == 0, so chunks never straddle the edge)
  constexpr int kPerChunk = 16 / sizeof(T);
  constexpr int kChunksPerRow = kColTileC / kPerChunk;
  for (int i = threadIdx.x; i < kColTileR * kChunksPerRow; i += blockDim.x) {
    const int r = i / kChunksPerRow, ch = i % kChunksPerRow;
    if (r < nrows && ch * kPerChunk < ncols) {
      *reinterpret_cast<uint4*>(&s_in[r * kColTileC + ch * kPerChunk]) =
          *reinterpret_cast<const uint4*>(x + (row0 + r) * cols + col0 + ch * kPerChunk);
    }
  }
  __syncthreads();

  const int c = threadIdx.x & 63;
  const int g = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int rb = g * 2 + k;
    if (rb < nrb && c < ncols) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const T e = s_in[(rb * 32 + i) * kColTileC + c];
        if constexpr (sizeof(T) == 2) {
          v[i] = __uint_as_float((uint32_t)e << 16);
        } else {
          v[i] = e;
        }
      }
      if (HAD) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = apply_sign(v[i], sign_mask, i);
        fwht32_lane(v);
      }
      uint32_t byte;
      const uint64_t idx0 = (uint64_t)(row0 + rb * 32) * (uint64_t)cols + (uint64_t)(col0 + c);
      s_codes[c * 8 + rb] = quant_col32<ROUND>(v, byte, seed, idx0, (uint64_t)cols);
      s_scales[c * 8 + rb] = (uint8_t)byte;
    }
  }
  __syncthreads();
  store_col_tile(s_codes, s_scales, rows, col0, ncols, row0, nrb, codes, scales);
}

// ============================================================== double quantization
// Input: packed row-blocked [rows, cols] (codes [rows][cols/2], scales
// [rows][cols/32]).  A workgroup stages 256 rows x 64 columns of codes (32 B
// per row) and their 2 scale bytes per row, decodes each column's 32 values
// exactly and quantizes them as a 32x1 block (output transposed).
template <int ROUND>
__global__ __launch_bounds__(256) void k_requant(const uint8_t* __restrict__ codes_in,
                                                 const uint8_t* __restrict__ scales_in,
                                                 int64_t rows, int64_t cols, uint64_t seed,
                                                 uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales) {
  __shared__ uint4 s_in[kColTileR * 2];          // 256 rows x 32 bytes
  __shared__ uint8_t s_sc[kColTileR * 2];        // 256 rows x 2 scale bytes
  __shared__ uint4 s_codes[kColTileC * 8];
  __shared__ uint8_t s_scales[kColTileC * 8];

  const int64_t col0 = (int64_t)blockIdx.x * kColTileC;
  const int64_t row0 = (int64_t)blockIdx.y * kColTileR;
  const int ncols = (int)min<int64_t>(kColTileC, cols - col0);   // multiple of 32
  const int nrows = (int)min<int64_t>(kColTileR, rows - row0);
  const int nrb = nrows / 32;
  const int64_t ld_in = cols / 2, ld_sin = cols / 32;

  for (int i = threadIdx.x; i < kColTileR * 2; i += blockDim.x) {
    const int r = i >> 1, ch = i & 1;
    if (r < nrows && ch * 32 < ncols) {
      s_in[i] = *reinterpret_cast<const uint4*>(codes_in + (row0 + r) * ld_in + col0 / 2 + ch * 16);
      s_sc[i] = scales_in[(row0 + r) * ld_sin + col0 / 32 + ch];
    }
  }
  __syncthreads();

  const int c = threadIdx.x & 63;
  const int g = threadIdx.x >> 6;
  const uint8_t* s_bytes = reinterpret_cast<const uint8_t*>(s_in);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int rb = g * 2 + k;
    if (rb < nrb && c < ncols) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int r = rb * 32 + i;
        const uint32_t byte = s_bytes[r * 32 + (c >> 1)];
        const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 15u);
        v[i] = e2m1_decode(code, s_sc[r * 2 + (c >> 5)]);
      }
      uint32_t sb;
      const uint64_t idx0 = (uint64_t)(row0 + rb * 32) * (uint64_t)cols + (uint64_t)(col0 + c);
      s_codes[c * 8 + rb] = quant_col32<ROUND>(v, sb, seed, idx0, (uint64_t)cols);
      s_scales[c * 8 + rb] = (uint8_t)sb;
    }
  }
  __syncthreads();
  store_col_tile(s_codes, s_scales, rows, col0, ncols, row0, nrb, codes, scales);
}

// ============================================================== dequantization
template <typename TOut>
__device__ __forceinline__ void store8(TOut* p, const float v[8]);

template <>
__device__ __forceinline__ void store8<float>(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float v[8]) {
  uint4 w;
  w.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
  w.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
  w.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
  w.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = w;
}

template <typename TOut>
__device__ __forceinline__ void store1(TOut* p, float v);
template <>
__device__ __forceinline__ void store1<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t* p, float v) {
  *p = (uint16_t)f32_to_bf16_rne(v);
}

template <typename TOut, bool HAD>
__global__ __launch_bounds__(256) void k_dequant_row(const uint32_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     int64_t nblk, uint32_t sign_mask,
                                                     TOut* __restrict__ out) {
  const int q = threadIdx.x & 3;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 2);
  for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 2) + (threadIdx.x >> 2); b < nblk;
       b += stride) {
    const uint32_t w = codes[b * 4 + q];
    const uint32_t byte = scales[b];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = e2m1_decode((w >> (4 * i)) & 15u, byte);
    if (HAD) {
      fwht32_quad(v, q);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = apply_sign(v[i] * 0.03125f, sign_mask, q * 8 + i);
    }
    store8<TOut>(out + b * 32 + q * 8, v);
  }
}

// Column-blocked input (codes [cols][rows/2]): one thread per 32x1 block,
// writing its 32 outputs down a column.  Used off the hot path.
template <typename TOut, bool HAD>
__global__ __launch_bounds__(256) void k_dequant_col(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     int64_t rows, int64_t cols,
                                                     uint32_t sign_mask, TOut* __restrict__ out) {
  const int64_t nrb = rows / 32;
  const int64_t total = nrb * cols;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % cols, rb = t / cols;
    const uint4 w = *reinterpret_cast<const uint4*>(codes + c * (rows / 2) + rb * 16);
    const uint32_t byte = scales[c * nrb + rb];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = e2m1_decode((ws[i >> 3] >> (4 * (i & 7))) & 15u, byte);
    if (HAD) {
      fwht32_lane(v);
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = apply_sign(v[i] * 0.03125f, sign_mask, i);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) store1<TOut>(out + (rb * 32 + i) * cols + c, v[i]);
  }
}

// ============================================================== launchers
static int grid_for_blocks(int64_t nblk) {
  // 64 blocks per 256-thread workgroup; cap so that each thread loops a few times
  const int64_t g = cdiv(nblk, 64);
  return (int)hmin(g, 256 * 32);
}

template <typename T>
static int launch_quant_row(const T* x, int64_t rows, int64_t cols, int round, uint64_t seed,
                            int had, uint32_t mask, uint8_t* codes, uint8_t* scales,
                            hipStream_t st) {
  const int64_t nblk = rows * cols / 32;
  const dim3 grid(grid_for_blocks(nblk)), block(256);
  uint32_t* c32 = reinterpret_cast<uint32_t*>(codes);
  if (round == MX_RNE) {
    if (had) k_quant_row<T, MX_RNE, true><<<grid, block, 0, st>>>(x, nblk, seed, mask, c32, scales);
    else k_quant_row<T, MX_RNE, false><<<grid, block, 0, st>>>(x, nblk, seed, mask, c32, scales);
  } else {
    if (had) k_quant_row<T, MX_SR, true><<<grid, block, 0, st>>>(x, nblk, seed, mask, c32, scales);
    else k_quant_row<T, MX_SR, false><<<grid, block, 0, st>>>(x, nblk, seed, mask, c32, scales);
  }
  return launch_status();
}

template <typename T>
static int launch_quant_col(const T* x, int64_t rows, int64_t cols, int round, uint64_t seed,
                            int had, uint32_t mask, uint8_t* codes, uint8_t* scales,
                            hipStream_t st) {
  const dim3 grid((unsigned)cdiv(cols, kColTileC), (unsigned)cdiv(rows, kColTileR)), block(256);
  if (round == MX_RNE) {
    if (had) k_quant_col<T, MX_RNE, true><<<grid, block, 0, st>>>(x, rows, cols, seed, mask, codes, scales);
    else k_quant_col<T, MX_RNE, false><<<grid, block, 0, st>>>(x, rows, cols, seed, mask, codes, scales);
  } else {
    if (had) k_quant_col<T, MX_SR, true><<<grid, block, 0, st>>>(x, rows, cols, seed, mask, codes, scales);
    else k_quant_col<T, MX_SR, false><<<grid, block, 0, st>>>(x, rows, cols, seed, mask, codes, scales);
  }
  return launch_status();
}

int quantize_impl(const void* x, int dtype, int64_t rows, int64_t cols, int axis, int round,
                  uint64_t seed, int had, uint32_t mask, uint8_t* codes, uint8_t* scales,
                  hipStream_t st) {
  if (rows == 0 || cols == 0) return MX_OK;
  if (axis == MX_ROW) {
    return dtype == MX_BF16
               ? launch_quant_row(static_cast<const uint16_t*>(x), rows, cols, round, seed, had,
                                  mask, codes, scales, st)
               : launch_quant_row(static_cast<const float*>(x), rows, cols, round, seed, had, mask,
                                  codes, scales, st);
  }
  return dtype == MX_BF16
             ? launch_quant_col(static_cast<const uint16_t*>(x), rows, cols, round, seed, had, mask,
                                codes, scales, st)
             : launch_quant_col(static_cast<const float*>(x), rows, cols, round, seed, had, mask,
                                codes, scales, st);
}

int requantize_impl(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows, int64_t cols,
                    int round, uint64_t seed, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return MX_OK;
  const dim3 grid((unsigned)cdiv(cols, kColTileC), (unsigned)cdiv(rows, kColTileR)), block(256);
  if (round == MX_RNE)
    k_requant<MX_RNE><<<grid, block, 0, st>>>(codes_in, scales_in, rows, cols, seed, codes, scales);
  else
    k_requant<MX_SR><<<grid, block, 0, st>>>(codes_in, scales_in, rows, cols, seed, codes, scales);
  return launch_status();
}

int quantize_dual_impl(const void* x, int dtype, int64_t rows, int64_t cols, int round,
                       uint64_t seed_row, uint64_t seed_col, uint8_t* codes_row,
                       uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                       hipStream_t st) {
  const int s = quantize_impl(x, dtype, rows, cols, MX_ROW, round, seed_row, 0, 0, codes_row,
                              scales_row, st);
  if (s != MX_OK) return s;
  return quantize_impl(x, dtype, rows, cols, MX_COL, round, seed_col, 0, 0, codes_col, scales_col,
                       st);
}

}  // namespace mx

using namespace mx;

extern "C" int mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int axis,
                           int round, uint64_t seed, int hadamard, uint32_t sign_mask,
                           uint8_t* codes, uint8_t* scales, void* stream) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(axis == MX_ROW || axis == MX_COL, MX_ERR_ENUM);
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(hadamard == 0 || hadamard == 1, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0, MX_ERR_SHAPE);
  if (axis == MX_ROW) MX_REQUIRE(cols % 32 == 0, MX_ERR_SHAPE);
  else MX_REQUIRE(rows % 32 == 0 && cols % 8 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && codes && scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(x) && aligned16(codes), MX_ERR_ALIGN);
  return quantize_impl(x, dtype, rows, cols, axis, round, seed, hadamard, sign_mask, codes, scales,
                       as_stream(stream));
}

extern "C" int mx_quantize_dual(const void* x, int dtype, int64_t rows, int64_t cols, int round,
                                uint64_t seed_row, uint64_t seed_col, uint8_t* codes_row,
                                uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                                void* stream) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0 && rows % 32 == 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && codes_row && scales_row && codes_col && scales_col, MX_ERR_NULL);
  MX_REQUIRE(aligned16(x) && aligned16(codes_row) && aligned16(codes_col), MX_ERR_ALIGN);
  return quantize_dual_impl(x, dtype, rows, cols, round, seed_row, seed_col, codes_row, scales_row,
                            codes_col, scales_col, as_stream(stream));
}

extern "C" int mx_requantize(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                             int64_t cols, int round, uint64_t seed, uint8_t* codes_out,
                             uint8_t* scales_out, void* stream) {
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0 && rows % 32 == 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(codes_in && scales_in && codes_out && scales_out, MX_ERR_NULL);
  MX_REQUIRE(aligned16(codes_in) && aligned16(codes_out), MX_ERR_ALIGN);
  return requantize_impl(codes_in, scales_in, rows, cols, round, seed, codes_out, scales_out,
                         as_stream(stream));
}

extern "C" int mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, int axis, int hadamard, uint32_t sign_mask, void* out,
                             int out_dtype, void* stream) {
  MX_REQUIRE(out_dtype == MX_F32 || out_dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(axis == MX_ROW || axis == MX_COL, MX_ERR_ENUM);
  MX_REQUIRE(hadamard == 0 || hadamard == 1, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0, MX_ERR_SHAPE);
  if (axis == MX_ROW) MX_REQUIRE(cols % 32 == 0, MX_ERR_SHAPE);
  else MX_REQUIRE(rows % 32 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(codes && scales && out, MX_ERR_NULL);
  MX_REQUIRE(aligned16(codes) && aligned16(out), MX_ERR_ALIGN);
  const hipStream_t st = as_stream(stream);
  const dim3 block(256);
  if (axis == MX_ROW) {
    const int64_t nblk = rows * cols / 32;
    const dim3 grid(grid_for_blocks(nblk));
    const uint32_t* c32 = reinterpret_cast<const uint32_t*>(codes);
    if (out_dtype == MX_F32) {
      float* o = static_cast<float*>(out);
      if (hadamard) k_dequant_row<float, true><<<grid, block, 0, st>>>(c32, scales, nblk, sign_mask, o);
      else k_dequant_row<float, false><<<grid, block, 0, st>>>(c32, scales, nblk, sign_mask, o);
    } else {
      uint16_t* o = static_cast<uint16_t*>(out);
      if (hadamard) k_dequant_row<uint16_t, true><<<grid, block, 0, st>>>(c32, scales, nblk, sign_mask, o);
      else k_dequant_row<uint16_t, false><<<grid, block, 0, st>>>(c32, scales, nblk, sign_mask, o);
    }
  } else {
    const int64_t total = rows / 32 * cols;
    const dim3 grid((unsigned)hmin(cdiv(total, 256), 4096));
    if (out_dtype == MX_F32) {
      float* o = static_cast<float*>(out);
      if (hadamard) k_dequant_col<float, true><<<grid, block, 0, st>>>(codes, scales, rows, cols, sign_mask, o);
      else k_dequant_col<float, false><<<grid, block, 0, st>>>(codes, scales, rows, cols, sign_mask, o);
    } else {
      uint16_t* o = static_cast<uint16_t*>(out);
      if (hadamard) k_dequant_col<uint16_t, true><<<grid, block, 0, st>>>(codes, scales, rows, cols, sign_mask, o);
      else k_dequant_col<uint16_t, false><<<grid, block, 0, st>>>(codes, scales, rows, cols, sign_mask, o);
    }
  }
  return launch_status();
}
