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

// Codes of the adjacent block elements 2i (bits 0..3) and 2i+1 (bits 4..7) at
// block scale `scale`, in the low byte of the result (the bits above are
// undefined); z is the generator state of the pair's key (element 2i's index),
// whose one output gives both stochastic rounding decisions.  Each element gets
// a conversion of its own, so the two decisions read disjoint bits.
template <int ROUND>
__device__ __forceinline__ uint32_t code_pair(float v0, float v1, float scale, uint64_t z) {
  if (ROUND == MX_SR) {
    uint32_t hi, lo;
    sm64_words(z, hi, lo);
    const uint32_t b0 = cvt_sr_pair(v0, v1, hi, scale);  // v0 reads hi bits 10..31
    const uint32_t b1 = cvt_sr_pair(v0, v1, lo, scale);  // v1 reads lo bits 9..30
    return (b0 & 0x0Fu) | (b1 & ~0x0Fu);
  }
  return cvt_rne_pair(v0, v1, scale);
}

// The low bytes of b0..b3 as one word, b0 in bits 0..7 (byte permutes; the
// bytes above each low byte are ignored).
__device__ __forceinline__ uint32_t low_bytes4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t l = __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);  // [b0, b1, 0, 0]
  const uint32_t h = __builtin_amdgcn_perm(b3, b2, 0x0C0C0400u);  // [b2, b3, 0, 0]
  return __builtin_amdgcn_perm(h, l, 0x05040100u);
}

// Quantize N = 4 or 8 consecutive values of a row block a lane holds (v[0] at an
// even position in its block), given the block's scale byte; returns the packed
// codes (element i in nibble i).  z = generator state keyed by v[0]'s logical
// index (sm64_state(seed, index)); callers step it along with the index, since
// the state is linear in the index.
template <int ROUND, int N>
__device__ __forceinline__ uint32_t quant_run(const float v[N], uint32_t byte, uint64_t z) {
  static_assert(N == 4 || N == 8, "runs of 4 or 8 values");
  if (byte == 255u) return 0u;
  const float sc = scale_of(byte);
  uint32_t b[N / 2];
#pragma unroll
  for (int p = 0; p < N / 2; ++p) {
    b[p] = code_pair<ROUND>(v[2 * p], v[2 * p + 1], sc, z);
    z += 2 * kGamma;
  }
  if constexpr (N == 8) return low_bytes4(b[0], b[1], b[2], b[3]);
  else return __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
}

template <int ROUND>
__device__ __forceinline__ uint32_t quant8(const float v[8], uint32_t byte, uint64_t z) {
  return quant_run<ROUND, 8>(v, byte, z);
}

// A workgroup takes 64 x kRowU consecutive blocks per iteration; its quad j
// handles blocks base + 64 u + j, u < kRowU, whose loads are all issued before
// any of them is quantized (more bytes in flight per lane).
constexpr int kRowU = 4;

// Up to two tensors quantized by one launch (the forward layer's X and W).  The
// grid strides over windows of 64 kRowU consecutive blocks; windows [0, w0)
// cover tensor 0 (n0 blocks), the rest tensor 1 (n1 blocks), so the tensor is
// uniform over a workgroup's window and each is indexed from its own block 0.
template <typename T>
struct RowJobs {  // named fields: selected with ternaries, never indexed at run time
  const T* x0;
  const T* x1;
  uint32_t* codes0;
  uint32_t* codes1;
  uint8_t* scales0;
  uint8_t* scales1;
  uint64_t seed0, seed1;
  int64_t n0, n1;
  int64_t w0;  // windows of tensor 0
  int64_t nwin;
  int64_t nbr, sld;  // one tensor with LD: blocks per row and bytes between scale rows
};

template <typename T, int ROUND, bool HAD, bool PAIR, bool LD = false>
__global__ __launch_bounds__(256) void k_quant_row(const RowJobs<T> jobs, uint32_t sign_mask) {
  const int q = threadIdx.x & 3;
  const int j = threadIdx.x >> 2;
  for (int64_t win = blockIdx.x; win < jobs.nwin; win += gridDim.x) {
    const bool t = PAIR && win >= jobs.w0;  // uniform over the workgroup
    const T* __restrict__ x = t ? jobs.x1 : jobs.x0;
    uint32_t* __restrict__ codes = t ? jobs.codes1 : jobs.codes0;
    uint8_t* __restrict__ scales = t ? jobs.scales1 : jobs.scales0;
    const uint64_t seed = t ? jobs.seed1 : jobs.seed0;
    const int64_t nblk = t ? jobs.n1 : jobs.n0;
    const int64_t base = (win - (t ? jobs.w0 : 0)) * 64 * kRowU;
    float v[kRowU][8];
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      // unconditional (clamped) loads, so that all of them are in flight at once
      const int64_t b = min(base + u * 64 + j, nblk - 1);
      load8<T>(x + b * 32 + q * 8, v[u]);
    }
    // generator state of this lane's first element; block b + 64 is 2048 elements on
    uint64_t z = ROUND == MX_SR ? sm64_state(seed, (uint64_t)(base + j) * 32 + q * 8) : 0;
#pragma unroll
    for (int u = 0; u < kRowU; ++u, z += 2048 * kGamma) {
      const int64_t b = base + u * 64 + j;
      if (b >= nblk) break;  // quads past the end: whole quads, so the DPP partners agree
      if (HAD) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = apply_sign(v[u][i], sign_mask, q * 8 + i);
        fwht32_quad(v[u], q);
      }
      const uint32_t m = quad_max_u32(amax_bits<8>(v[u]));
      const uint32_t byte = scale_byte_of(m);
      codes[b * 4 + q] = quant8<ROUND>(v[u], byte, z);
      if (q == 0) scales[LD ? (b / jobs.nbr) * jobs.sld + b % jobs.nbr : b] = (uint8_t)byte;
    }
  }
}

// ============================================================== row segments
// The 32x1 quantizers can run per token segment of a grouped (mixture-of-
// experts) layer: segment g is rows [row_off[g], row_off[g+1]); its blocks
// start at the segment's first row and its tail is zero-padded to a multiple
// of kSegPad rows, so the transposed output has a padded row axis of out_len
// positions, segment g's starting at out_off[g].  n == 0: one plain segment.
// A caller may space the segments further apart (a multiple of kSegPad rows and
// of the tile heights): the kernels then write each segment's first
// round-up(rows, tile height) positions and leave the rest of its space alone.
constexpr int kSegPad = 128;

struct Segs {
  int n;
  int tile_start[MX_MAX_GROUPS + 1];   // first blockIdx.y of each segment
  int64_t row_off[MX_MAX_GROUPS + 1];
  int64_t out_off[MX_MAX_GROUPS + 1];
  int64_t out_len;
};

// Rows of this workgroup's tile of height TR: input rows [row0, row0 + nreal),
// output positions [out0, out0 + 32 nrb) of an axis of out_len.
struct TileRows {
  int64_t row0, out0, out_len;
  int nreal, nrb;
};

__device__ __forceinline__ TileRows tile_rows(const Segs& s, int TR, int64_t rows, int y) {
  TileRows t;
  if (s.n == 0) {
    t.row0 = (int64_t)y * TR;
    t.nreal = (int)min<int64_t>(TR, rows - t.row0);
    t.out0 = t.row0;
    t.nrb = t.nreal / 32;
    t.out_len = rows;
    return t;
  }
  int g = 0;
  while (g + 1 < s.n && s.tile_start[g + 1] <= y) ++g;
  const int64_t k = (int64_t)y - s.tile_start[g];
  t.row0 = s.row_off[g] + k * TR;
  t.nreal = (int)min<int64_t>(TR, s.row_off[g + 1] - t.row0);
  t.out0 = s.out_off[g] + k * TR;
  t.nrb = (int)(min<int64_t>(TR, s.out_off[g + 1] - t.out0) / 32);
  t.out_len = s.out_len;
  return t;
}

// ============================================================== column blocks
// A workgroup owns a tile of kTileR = 128 rows x 256 bytes of input (128 bf16
// or 64 f32 columns).  Each thread loads 8 chunks of 16 bytes (coalesced) and
// writes them to LDS.  Column pass: thread (p, rb) reads one dword per row of
// row block rb (the column pair 2p, 2p+1 of bf16, or column p of f32; the 64
// lanes of a wave read 64 consecutive dwords) and quantizes those 32x1
// blocks; their codes are staged so that each output row (= input column) gets
// 64 contiguous bytes per tile.  With ROW set (dual quantization) the chunks
// are also quantized as 1x32 blocks straight from registers: the 32 / E lanes
// holding one row block are adjacent, E = elements per chunk.  HAD rotates both
// block shapes (with ROW only for bf16, where a row block is one DPP quad).
constexpr int kTileR = 128;
constexpr int kTileRowBytes = 256;

// Largest sign-cleared bf16 pattern in each half of the words w[0..n), the two
// halves at once (packed 16-bit max: exact, NaN and Inf patterns win).
template <int N>
__device__ __forceinline__ uint32_t bf16_pair_max(const uint32_t* w) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < N; ++i)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  return __builtin_bit_cast(uint32_t, m);
}

// Quantize 32 values of one column block whose largest sign-cleared float32
// pattern is m; returns the 16 code bytes as uint4.  z = generator state keyed
// by the block's first element (sm64_state(seed, index)); the block's elements
// are idx_step apart in the logical tensor.
template <int ROUND>
__device__ __forceinline__ uint4 quant_col32_m(const float v[32], uint32_t m, uint32_t& byte_out,
                                               uint64_t z0, uint64_t idx_step) {
  const uint32_t byte = scale_byte_of(m);
  byte_out = byte;
  uint32_t w[4] = {0, 0, 0, 0};
  if (byte != 255u) {
    const float sc = scale_of(byte);
    uint64_t z = 0, dz = 0;
    if (ROUND == MX_SR) {
      z = z0;
      dz = 2 * idx_step * kGamma;   // next pair's key: two elements further down
    }
    uint32_t b[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      b[p] = code_pair<ROUND>(v[2 * p], v[2 * p + 1], sc, z);
      z += dz;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = low_bytes4(b[4 * q], b[4 * q + 1], b[4 * q + 2], b[4 * q + 3]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int ROUND>
__device__ __forceinline__ uint4 quant_col32(const float v[32], uint32_t& byte_out, uint64_t z0,
                                             uint64_t idx_step) {
  return quant_col32_m<ROUND>(v, amax_bits<32>(v), byte_out, z0, idx_step);
}

// Writes staged column-block codes/scales: output row (col0 + c) gets bytes
// [row0/2, row0/2 + 16 nrb) of codes and [row0/32, row0/32 + nrb) of scales
// (scale rows ld_s bytes apart, at least rows / 32), for c < ncols; staging
// layout [c][rb], NRB row blocks per column.  A column's scale bytes are
// contiguous in its output row, so whole tiles write them as 32-bit words
// (one store per four row blocks instead of four byte stores) when the scale
// rows allow it.
template <int NC, int NRB>
__device__ __forceinline__ void store_col_tile(const uint4* s_codes, const uint8_t* s_scales,
                                               int64_t rows, int64_t ld_s, int64_t col0,
                                               int ncols, int64_t row0, int nrb,
                                               uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
  const int64_t ld_c = rows / 2;
  for (int i = threadIdx.x; i < NC * NRB; i += blockDim.x) {
    const int c = i / NRB, rb = i % NRB;
    if (c < ncols && rb < nrb)
      *reinterpret_cast<uint4*>(codes + (col0 + c) * ld_c + row0 / 2 + rb * 16) = s_codes[i];
  }
  uint8_t* const s0 = scales + col0 * ld_s + row0 / 32;
  const bool words = NRB % 4 == 0 && nrb == NRB && ld_s % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(s0) & 3) == 0;  // uniform over the workgroup
  if (words) {
    constexpr int W = NRB / 4;  // scale words per column
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(s_scales);
    for (int i = threadIdx.x; i < NC * W; i += blockDim.x) {
      const int c = i / W, w = i % W;
      if (c < ncols) *reinterpret_cast<uint32_t*>(s0 + c * ld_s + 4 * w) = sw[i];
    }
  } else {
    for (int i = threadIdx.x; i < NC * NRB; i += blockDim.x) {
      const int c = i / NRB, rb = i % NRB;
      if (c < ncols && rb < nrb) s0[c * ld_s + rb] = s_scales[i];
    }
  }
}

// max over the 32 / E adjacent lanes that hold one row block
template <int E>
__device__ __forceinline__ uint32_t rowblock_max_u32(uint32_t m) {
  m = quad_max_u32(m);
  if constexpr (E == 4) m = max(m, (uint32_t)__shfl_xor((int)m, 4));
  return m;
}

template <typename T, int ROUND, bool ROW, bool HAD>
__global__ __launch_bounds__(256) void k_quant_tile(
    const T* __restrict__ x, int64_t rows, int64_t cols, uint64_t seed_row, uint64_t seed_col,
    uint32_t sign_mask, uint8_t* __restrict__ codes_row, uint8_t* __restrict__ scales_row,
    uint8_t* __restrict__ codes_col, uint8_t* __restrict__ scales_col, const Segs segs,
    int64_t sp_row, int64_t sp_col) {
  constexpr int E = 16 / sizeof(T);               // elements per 16-byte chunk
  constexpr int TC = kTileRowBytes / sizeof(T);   // tile columns
  constexpr int CPR = kTileRowBytes / 16;         // chunks per tile row (16)
  constexpr int CPT = 4 / sizeof(T);              // columns per thread in the column pass
  constexpr int NRB = kTileR / 32;                // row blocks per tile (4)
  constexpr int NLOAD = kTileR * CPR / 256;       // chunks per thread (8)
  __shared__ uint32_t s_in[kTileR * kTileRowBytes / 4];
  // Once the column pass holds its values in registers the tile is no longer
  // read; its first TC * NRB * 16 bytes then stage the column-block codes and
  // the next TC * NRB bytes their scales (32 KB of LDS in all).
  static_assert(TC * NRB * 17 <= kTileR * kTileRowBytes, "code staging fits the tile");
  uint4* const s_codes = reinterpret_cast<uint4*>(s_in);
  uint8_t* const s_scales = reinterpret_cast<uint8_t*>(s_in) + TC * NRB * 16;

  const int64_t col0 = (int64_t)blockIdx.x * TC;
  const TileRows tr = tile_rows(segs, kTileR, rows, (int)blockIdx.y);
  const int64_t row0 = tr.row0;
  const int ncols = (int)min<int64_t>(TC, cols - col0);
  const int nrows = tr.nreal;  // rows past it (segment padding) stay zero in LDS
  const int nrb = tr.nrb;
  const int tid = threadIdx.x;

  // ---- load: chunk (r, c) = (j * 16 + tid / 16, tid % 16)
  const int lc = tid % CPR;
  // Every lane issues all of its loads before the first wait.  Chunk j lies
  // 256 / CPR rows below chunk j - 1 (a uniform step).  In a partial tile a chunk
  // outside it reads the tensor's first chunk instead and is zeroed by a mask;
  // the mask is opaque to the compiler, which would otherwise turn the zeroing
  // back into a branch around each load, and the register copies at those
  // branches' joins wait for the loads one by one.
  uint4 ch[NLOAD];
  const T* const p_a = x + (row0 + tid / CPR) * cols + col0 + lc * E;
  const int64_t d_p = (int64_t)(256 / CPR) * cols;
  if (nrows >= kTileR && ncols >= TC) {  // whole tile (uniform)
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) ch[j] = *reinterpret_cast<const uint4*>(p_a + j * d_p);
  } else {
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) {
      const int r = j * (256 / CPR) + tid / CPR;
      const bool ok = r < nrows && lc * E < ncols;
      const uint4 w = *reinterpret_cast<const uint4*>(ok ? p_a + j * d_p : x);
      uint32_t m = ok ? 0xFFFFFFFFu : 0u;
      asm("" : "+v"(m));
      ch[j] = make_uint4(w.x & m, w.y & m, w.z & m, w.w & m);
    }
  }
#pragma unroll
  for (int j = 0; j < NLOAD; ++j) {
    const int r = j * (256 / CPR) + tid / CPR;
    *reinterpret_cast<uint4*>(&s_in[r * (kTileRowBytes / 4) + lc * 4]) = ch[j];
  }

  // ---- row pass (1x32 blocks) from registers
  static_assert(!(ROW && HAD) || E == 8, "rotated row pass needs one quad per block");
  if constexpr (ROW) {
    // Chunk j lies 256 / CPR rows below chunk j - 1: its logical index, generator
    // state and output addresses step by amounts uniform over the workgroup (the
    // state is linear in the index), so no 64-bit products are formed per chunk.
    const int64_t r_a = row0 + tid / CPR;
    const uint64_t idx_a = (uint64_t)r_a * (uint64_t)cols + (uint64_t)(col0 + lc * E);
    const uint64_t d_idx = (uint64_t)(256 / CPR) * (uint64_t)cols;
    const uint64_t z_a = ROUND == MX_SR ? sm64_state(seed_row, idx_a) : 0;
    uint8_t* const s_a = scales_row + r_a * sp_row + (col0 + lc * E) / 32;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) {
      const int r = j * (256 / CPR) + tid / CPR;
      if (r >= nrows || lc * E >= ncols) continue;  // whole row blocks drop out together
      float v[E];
      const uint32_t w[4] = {ch[j].x, ch[j].y, ch[j].z, ch[j].w};
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if constexpr (sizeof(T) == 2) v[i] = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
        else v[i] = __uint_as_float(w[i]);
      }
      if constexpr (HAD && E == 8) {
        const int qq = lc & 3;  // lane's position in its block's quad
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = apply_sign(v[i], sign_mask, qq * 8 + i);
        fwht32_quad(v, qq);
      }
      uint32_t m = 0;
      if constexpr (sizeof(T) == 2 && !HAD) {  // on the packed words: both halves at once
        const uint32_t pm = bf16_pair_max<4>(w);
        m = max(pm << 16, pm & 0xFFFF0000u);
      } else {
        m = amax_bits<E>(v);
      }
      m = rowblock_max_u32<E>(m);
      const uint32_t byte = scale_byte_of(m);
      const uint64_t idx0 = idx_a + (uint64_t)j * d_idx;
      const uint32_t packed = quant_run<ROUND, E>(v, byte, z_a + (uint64_t)j * (d_idx * kGamma));
      if constexpr (E == 8) reinterpret_cast<uint32_t*>(codes_row)[idx0 / 8] = packed;
      else reinterpret_cast<uint16_t*>(codes_row)[idx0 / 4] = (uint16_t)packed;
      if (lc % (32 / E) == 0) s_a[(int64_t)j * (256 / CPR) * sp_row] = (uint8_t)byte;
    }
  }
  __syncthreads();

  // ---- column pass (32x1 blocks) from LDS
  {
    const int p = tid % 64, rb = tid / 64;
    const bool active = rb < nrb && p * CPT < ncols;
    // every thread reads (rb < NRB, p < 64: inside the tile) so that the values
    // need no copies where the inactive threads' path joins
    uint32_t raw[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) raw[i] = s_in[(rb * 32 + i) * (kTileRowBytes / 4) + p];
    __syncthreads();  // every thread has read the tile: s_codes may overwrite it
    if (active) {
      // generator state of column p * CPT's block; column p * CPT + cc is cc elements on
      const uint64_t zc =
          ROUND == MX_SR ? sm64_state(seed_col, (uint64_t)(row0 + rb * 32) * (uint64_t)cols +
                                                    (uint64_t)(col0 + p * CPT))
                         : 0;
      // bf16 without rotation: both columns' block maxima from the packed words
      const uint32_t pm = sizeof(T) == 2 && !HAD ? bf16_pair_max<32>(raw) : 0u;
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if constexpr (sizeof(T) == 2) v[i] = cc ? bf16_hi(raw[i]) : bf16_lo(raw[i]);
          else v[i] = __uint_as_float(raw[i]);
        }
        if (HAD) {
#pragma unroll
          for (int i = 0; i < 32; ++i) v[i] = apply_sign(v[i], sign_mask, i);
          fwht32_lane(v);
        }
        const int c = p * CPT + cc;
        uint32_t byte;
        if constexpr (sizeof(T) == 2 && !HAD) {
          const uint32_t m = cc ? (pm & 0xFFFF0000u) : (pm << 16);
          s_codes[c * NRB + rb] =
              quant_col32_m<ROUND>(v, m, byte, zc + (uint64_t)cc * kGamma, (uint64_t)cols);
        } else {
          s_codes[c * NRB + rb] =
              quant_col32<ROUND>(v, byte, zc + (uint64_t)cc * kGamma, (uint64_t)cols);
        }
        s_scales[c * NRB + rb] = (uint8_t)byte;
      }
    }
  }
  __syncthreads();
  store_col_tile<TC, NRB>(s_codes, s_scales, tr.out_len, sp_col, col0, ncols, tr.out0, nrb,
                          codes_col, scales_col);
}

// ============================================================== double quantization
// Input: packed row-blocked [rows, cols] (codes [rows][cols/2], scales
// [rows][cols/32]).  A workgroup owns 256 rows x 128 columns; thread (o, rb)
// takes the 4 columns 4o .. 4o+3 (two code bytes per row, read straight from
// global memory: the 32 lanes of a half-wave read 64 contiguous bytes of one
// row) over row block rb, decodes each value exactly (E2M1 magnitude times
// 2^(scale - 127); a 0xFF input scale makes the whole column block NaN) and
// quantizes the four 32x1 blocks.  Codes are staged for 128-byte row stores.
// blockIdx.z selects a matrix of a stack of equal [rows, cols] matrices (the
// experts' weights); stochastic rounding indexes the stacked logical tensor.
// Rows past a segment's end (segment padding) are zeros.
constexpr int kRqR = 256;
constexpr int kRqC = 128;

// One launch can requantize two matrices with the same cols (the backward
// layer's Q_D(W) and Q_D(X)): tile rows [0, ty0) of the grid belong to job 0,
// the rest to job 1.
struct RqJob {
  const uint8_t* codes_in;
  const uint8_t* scales_in;
  int64_t rows;
  uint64_t seed;
  uint8_t* codes;
  uint8_t* scales;
  int64_t s_pitch;  // bytes between output scale rows (at least the output row's blocks)
};

template <int ROUND>
__global__ __launch_bounds__(256) void k_requant(const RqJob j0, const RqJob j1, int ty0,
                                                 int64_t cols, const Segs segs) {
  constexpr int NRB = kRqR / 32;
  __shared__ uint4 s_codes[kRqC * NRB];
  __shared__ __align__(16) uint8_t s_scales[kRqC * NRB];

  const bool second = (int)blockIdx.y >= ty0;   // uniform over the workgroup
  const RqJob& job = second ? j1 : j0;
  const int ty = (int)blockIdx.y - (second ? ty0 : 0);
  const int64_t rows = job.rows;
  const uint64_t seed = job.seed;
  const int64_t z = blockIdx.z;
  const uint8_t* __restrict__ codes_in = job.codes_in + z * rows * (cols / 2);
  const uint8_t* __restrict__ scales_in = job.scales_in + z * rows * (cols / 32);
  uint8_t* __restrict__ codes = job.codes + z * rows * (cols / 2);
  uint8_t* __restrict__ scales = job.scales + z * cols * job.s_pitch;
  const int64_t col0 = (int64_t)blockIdx.x * kRqC;
  const TileRows tr = tile_rows(segs, kRqR, rows, ty);
  const int64_t row0 = tr.row0;
  const int ncols = (int)min<int64_t>(kRqC, cols - col0);   // multiple of 32
  const int nrb = tr.nrb;
  const int64_t ld_in = cols / 2, ld_sin = cols / 32;
  const int o = threadIdx.x % 32, rb = threadIdx.x / 32;

  if (rb < nrb && o * 4 < ncols) {
    const int64_t c0 = col0 + o * 4;
    // rows at or past nreal are padding: load the segment's last row instead (never
    // used) and zero it.  Row i's addresses step from row 0's by i pitches, a
    // product uniform over the workgroup.
    const int64_t r_first = row0 + rb * 32, r_last = row0 + tr.nreal - 1;
    const uint8_t* const cp0 = codes_in + r_first * ld_in + c0 / 2;
    const uint8_t* const cpl = codes_in + r_last * ld_in + c0 / 2;
    const uint8_t* const sp0 = scales_in + r_first * ld_sin + c0 / 32;
    const uint8_t* const spl = scales_in + r_last * ld_sin + c0 / 32;
    uint32_t cw[32], sw[32];
    if (rb * 32 + 32 <= tr.nreal) {  // a whole row block: no padding rows
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        cw[i] = *reinterpret_cast<const uint16_t*>(cp0 + i * ld_in);
        sw[i] = sp0[i * ld_sin];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const bool real = rb * 32 + i < tr.nreal;
        cw[i] = *reinterpret_cast<const uint16_t*>(real ? cp0 + i * ld_in : cpl);
        sw[i] = *(real ? sp0 + i * ld_sin : spl);
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (rb * 32 + i >= tr.nreal) {
          cw[i] = 0;     // code +0
          sw[i] = 127;   // any finite scale
        }
      }
    }
    // Row scales 2^(byte - 127) as floats (byte 0: the subnormal 2^-127; 0xFF: +Inf,
    // which makes every decoded value of the row NaN).
    float rs[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) rs[i] = __builtin_amdgcn_ldexpf(1.0f, (int)sw[i] - 127);
    // generator state of column 4o's block; column 4o + cc is cc elements on
    const uint64_t zc = ROUND == MX_SR ? sm64_state(seed, (uint64_t)(z * rows + row0 + rb * 32) *
                                                              (uint64_t)cols + (uint64_t)(col0 + o * 4))
                                       : 0;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {  // column 4o + cc: code byte cc / 2 of each row
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const mx_v2f r = cc < 2 ? decode_byte<0>(cw[i], rs[i]) : decode_byte<1>(cw[i], rs[i]);
        v[i] = (cc & 1) ? r.y : r.x;
      }
      const uint32_t m = amax_bits<32>(v);
      uint32_t byte;
      const int c = o * 4 + cc;
      s_codes[c * NRB + rb] =
          quant_col32_m<ROUND>(v, m, byte, zc + (uint64_t)cc * kGamma, (uint64_t)cols);
      s_scales[c * NRB + rb] = (uint8_t)byte;
    }
  }
  __syncthreads();
  store_col_tile<kRqC, NRB>(s_codes, s_scales, tr.out_len, job.s_pitch, col0, ncols, tr.out0, nrb, codes,
                            scales);
}

// ============================================================== rotated double quantization
// Input: Q_D of X rotated along cols (packed row-blocked [rows, cols], sign mask
// s).  Each row block is decoded exactly and rotated back (s * FWHT(y) * 2^-5,
// float32, the same quad FWHT as the rotated quantizer), the tile (128 rows x 64
// columns) is staged in LDS as float32, and each 32x1 column block is rotated
// along rows with the same signs and quantized (output transposed).
constexpr int kRhtR = 128;
constexpr int kRhtC = 64;

// One launch can take two matrices with the same cols and sign mask (the
// rotated backward's Q_D(H W) and Q_D(H X)): tile rows [0, ty0) of the grid
// belong to matrix 0.  Named fields, selected per workgroup.
struct RhtJobs {
  const uint8_t* codes_in0;
  const uint8_t* codes_in1;
  const uint8_t* scales_in0;
  const uint8_t* scales_in1;
  int64_t rows0, rows1;
  uint64_t seed0, seed1;
  uint8_t* codes0;
  uint8_t* codes1;
  uint8_t* scales0;
  uint8_t* scales1;
  int ty0;
};

template <int ROUND>
__global__ __launch_bounds__(256) void k_requant_rht(const RhtJobs jobs, int64_t cols,
                                                     uint32_t sign_mask) {
  constexpr int NRB = kRhtR / 32;
  __shared__ float s_x[kRhtR * kRhtC];  // [row][col]
  __shared__ uint4 s_codes[kRhtC * NRB];
  __shared__ __align__(16) uint8_t s_scales[kRhtC * NRB];

  const bool t = (int)blockIdx.y >= jobs.ty0;  // uniform over the workgroup
  const uint8_t* __restrict__ codes_in = t ? jobs.codes_in1 : jobs.codes_in0;
  const uint8_t* __restrict__ scales_in = t ? jobs.scales_in1 : jobs.scales_in0;
  const int64_t rows = t ? jobs.rows1 : jobs.rows0;
  const uint64_t seed = t ? jobs.seed1 : jobs.seed0;
  uint8_t* __restrict__ codes = t ? jobs.codes1 : jobs.codes0;
  uint8_t* __restrict__ scales = t ? jobs.scales1 : jobs.scales0;
  const int64_t col0 = (int64_t)blockIdx.x * kRhtC;
  const int64_t row0 = (int64_t)((int)blockIdx.y - (t ? jobs.ty0 : 0)) * kRhtR;
  const int ncols = (int)min<int64_t>(kRhtC, cols - col0);   // 32 or 64
  const int nrows = (int)min<int64_t>(kRhtR, rows - row0);   // multiple of 32
  const int nrb = nrows / 32;
  const int64_t ld_in = cols / 2, ld_sin = cols / 32;
  const int q = threadIdx.x & 3;

  // ---- decode and undo the row rotation: quad j takes row blocks j, j + 64, ...
  // The factor 2^-5 and the sign of element q*8+i are one exact multiply.
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = apply_sign(0.03125f, sign_mask, q * 8 + i);
  for (int blk = threadIdx.x >> 2; blk < kRhtR * (kRhtC / 32); blk += 64) {
    const int r = blk / (kRhtC / 32), kb = blk % (kRhtC / 32);
    if (r >= nrows || kb * 32 >= ncols) continue;  // whole quads drop out together
    const uint32_t wcodes = *reinterpret_cast<const uint32_t*>(
        codes_in + (row0 + r) * ld_in + (col0 + kb * 32) / 2 + q * 4);
    const uint32_t byte = scales_in[(row0 + r) * ld_sin + (col0 / 32 + kb)];
    float v[8];
    decode8(wcodes, byte, v);
    fwht32_quad(v, q);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= f[i];
    float* dst = &s_x[r * kRhtC + kb * 32 + q * 8];
    reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  __syncthreads();

  // ---- rotate and quantize the column blocks: thread (c, rb)
  {
    const int c = threadIdx.x % kRhtC, rb = threadIdx.x / kRhtC;
    if (rb < nrb && c < ncols) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = apply_sign(s_x[(rb * 32 + i) * kRhtC + c], sign_mask, i);
      fwht32_lane(v);
      uint32_t byte;
      const uint64_t idx0 = (uint64_t)(row0 + rb * 32) * (uint64_t)cols + (uint64_t)(col0 + c);
      s_codes[c * NRB + rb] =
          quant_col32<ROUND>(v, byte, ROUND == MX_SR ? sm64_state(seed, idx0) : 0, (uint64_t)cols);
      s_scales[c * NRB + rb] = (uint8_t)byte;
    }
  }
  __syncthreads();
  store_col_tile<kRhtC, NRB>(s_codes, s_scales, rows, rows / 32, col0, ncols, row0, nrb, codes,
                             scales);
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
    decode8(w, byte, v);
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
    for (int q = 0; q < 4; ++q) decode8(ws[q], byte, v + 8 * q);
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
static int grid_for_row(int64_t nblk) {
  // 64 kRowU blocks per 256-thread workgroup and iteration; at most 64 workgroups per CU
  const int64_t g = cdiv(nblk, 64 * kRowU);
  return (int)hmin(g, 256 * 64);
}
static int grid_for_blocks(int64_t nblk) {
  const int64_t g = cdiv(nblk, 64);
  return (int)hmin(g, 256 * 32);
}

template <typename T>
static int launch_quant_row_jobs(RowJobs<T> jobs, int round, int had, uint32_t mask,
                                 hipStream_t st) {
  const int64_t per = 64 * kRowU;  // blocks per window
  jobs.w0 = cdiv(jobs.n0, per);
  jobs.nwin = jobs.w0 + cdiv(jobs.n1, per);
  if (jobs.nwin == 0) return MX_OK;
  const dim3 grid(grid_for_row(jobs.nwin * per)), block(256);
  if (jobs.sld != 0) {  // one tensor, scale rows sld bytes apart
    if (round == MX_RNE) {
      if (had) k_quant_row<T, MX_RNE, true, false, true><<<grid, block, 0, st>>>(jobs, mask);
      else k_quant_row<T, MX_RNE, false, false, true><<<grid, block, 0, st>>>(jobs, mask);
    } else {
      if (had) k_quant_row<T, MX_SR, true, false, true><<<grid, block, 0, st>>>(jobs, mask);
      else k_quant_row<T, MX_SR, false, false, true><<<grid, block, 0, st>>>(jobs, mask);
    }
    return launch_status();
  }
  if (jobs.n1 > 0) {
    if (round == MX_RNE) {
      if (had) k_quant_row<T, MX_RNE, true, true><<<grid, block, 0, st>>>(jobs, mask);
      else k_quant_row<T, MX_RNE, false, true><<<grid, block, 0, st>>>(jobs, mask);
    } else {
      if (had) k_quant_row<T, MX_SR, true, true><<<grid, block, 0, st>>>(jobs, mask);
      else k_quant_row<T, MX_SR, false, true><<<grid, block, 0, st>>>(jobs, mask);
    }
  } else {  // one tensor: the selection compiles away
    if (round == MX_RNE) {
      if (had) k_quant_row<T, MX_RNE, true, false><<<grid, block, 0, st>>>(jobs, mask);
      else k_quant_row<T, MX_RNE, false, false><<<grid, block, 0, st>>>(jobs, mask);
    } else {
      if (had) k_quant_row<T, MX_SR, true, false><<<grid, block, 0, st>>>(jobs, mask);
      else k_quant_row<T, MX_SR, false, false><<<grid, block, 0, st>>>(jobs, mask);
    }
  }
  return launch_status();
}

template <typename T>
static int launch_quant_row(const T* x, int64_t rows, int64_t cols, int round, uint64_t seed,
                            int had, uint32_t mask, uint8_t* codes, uint8_t* scales,
                            hipStream_t st, int64_t sld = 0) {
  RowJobs<T> jobs{};
  if (sld != 0 && sld != cols / 32) {  // 0 or cols / 32: packed scale rows
    jobs.nbr = cols / 32;
    jobs.sld = sld;
  }
  jobs.x0 = jobs.x1 = x;
  jobs.codes0 = jobs.codes1 = reinterpret_cast<uint32_t*>(codes);
  jobs.scales0 = jobs.scales1 = scales;
  jobs.seed0 = jobs.seed1 = seed;
  jobs.n0 = rows * cols / 32;
  jobs.n1 = 0;
  return launch_quant_row_jobs(jobs, round, had, mask, st);
}

static Segs plain_segs() {
  Segs s{};
  s.n = 0;
  return s;
}

// Segments of tile height TR over the row offsets offs[0..groups] (host array).
static Segs make_segs(const int64_t* offs, int64_t groups, int TR, int64_t pad = kSegPad) {
  Segs s{};
  s.n = (int)groups;
  s.tile_start[0] = 0;
  s.out_off[0] = 0;
  for (int64_t g = 0; g < groups; ++g) {
    const int64_t n = offs[g + 1] - offs[g];
    s.row_off[g] = offs[g];
    s.tile_start[g + 1] = s.tile_start[g] + (int)cdiv(n, TR);
    s.out_off[g + 1] = s.out_off[g] + cdiv(n, pad) * pad;
  }
  s.row_off[groups] = offs[groups];
  s.out_len = s.out_off[groups];
  return s;
}

// Start of each segment on the padded row axis (out[0..groups], out[groups] = total).
// pad: segment spacing, a multiple of 256 rows when not kSegPad.
void segments_padded_offsets(const int64_t* offs, int64_t groups, int64_t* out,
                             int64_t pad = kSegPad) {
  out[0] = 0;
  for (int64_t g = 0; g < groups; ++g) out[g + 1] = out[g] + cdiv(offs[g + 1] - offs[g], pad) * pad;
}

int64_t segments_padded_rows(const int64_t* offs, int64_t groups, int64_t pad = kSegPad) {
  int64_t p = 0;
  for (int64_t g = 0; g < groups; ++g) p += cdiv(offs[g + 1] - offs[g], pad) * pad;
  return p;
}

// Column blocks (ROW = false) or both block shapes from one read (ROW = true).
template <typename T, bool ROW>
static int launch_quant_tile(const T* x, int64_t rows, int64_t cols, int round, uint64_t seed_row,
                             uint64_t seed_col, int had, uint32_t mask, uint8_t* codes_row,
                             uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                             hipStream_t st, const Segs& segs = plain_segs(),
                             int64_t sp_row = 0, int64_t sp_col = 0) {
  constexpr int TC = kTileRowBytes / sizeof(T);
  // scale row pitches of the two outputs: 0 = packed (blocks per row)
  if (sp_row == 0) sp_row = cols / 32;
  if (sp_col == 0) sp_col = (segs.n ? segs.out_len : rows) / 32;
  const unsigned ty = segs.n ? (unsigned)segs.tile_start[segs.n] : (unsigned)cdiv(rows, kTileR);
  if (ty == 0) return MX_OK;
  const dim3 grid((unsigned)cdiv(cols, TC), ty), block(256);
#define MX_TILE_ARGS x, rows, cols, seed_row, seed_col, mask, codes_row, scales_row, codes_col, scales_col, segs, sp_row, sp_col
  constexpr bool kHad = !ROW || sizeof(T) == 2;  // rotated row pass: bf16 only
  if (round == MX_RNE) {
    if (had && kHad) k_quant_tile<T, MX_RNE, ROW, kHad><<<grid, block, 0, st>>>(MX_TILE_ARGS);
    else k_quant_tile<T, MX_RNE, ROW, false><<<grid, block, 0, st>>>(MX_TILE_ARGS);
  } else {
    if (had && kHad) k_quant_tile<T, MX_SR, ROW, kHad><<<grid, block, 0, st>>>(MX_TILE_ARGS);
    else k_quant_tile<T, MX_SR, ROW, false><<<grid, block, 0, st>>>(MX_TILE_ARGS);
  }
#undef MX_TILE_ARGS
  return launch_status();
}

// sld: bytes between the output's scale rows (0: packed, blocks per row).
int quantize_impl(const void* x, int dtype, int64_t rows, int64_t cols, int axis, int round,
                  uint64_t seed, int had, uint32_t mask, uint8_t* codes, uint8_t* scales,
                  hipStream_t st, int64_t sld = 0) {
  if (rows == 0 || cols == 0) return MX_OK;
  if (axis == MX_ROW) {
    return dtype == MX_BF16
               ? launch_quant_row(static_cast<const uint16_t*>(x), rows, cols, round, seed, had,
                                  mask, codes, scales, st, sld)
               : launch_quant_row(static_cast<const float*>(x), rows, cols, round, seed, had, mask,
                                  codes, scales, st, sld);
  }
  return dtype == MX_BF16
             ? launch_quant_tile<uint16_t, false>(static_cast<const uint16_t*>(x), rows, cols, round,
                                                  0, seed, had, mask, nullptr, nullptr, codes,
                                                  scales, st, plain_segs(), 0, sld)
             : launch_quant_tile<float, false>(static_cast<const float*>(x), rows, cols, round, 0,
                                               seed, had, mask, nullptr, nullptr, codes, scales, st,
                                               plain_segs(), 0, sld);
}

static int launch_requant_jobs(const RqJob& j0, const RqJob& j1, int ty0, int ty1, int64_t cols,
                               int round, int64_t batch, const Segs& segs, hipStream_t st) {
  if (ty0 + ty1 == 0 || batch == 0) return MX_OK;
  const dim3 grid((unsigned)cdiv(cols, kRqC), (unsigned)(ty0 + ty1), (unsigned)batch), block(256);
  if (round == MX_RNE) k_requant<MX_RNE><<<grid, block, 0, st>>>(j0, j1, ty0, cols, segs);
  else k_requant<MX_SR><<<grid, block, 0, st>>>(j0, j1, ty0, cols, segs);
  return launch_status();
}

static int launch_requant(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                          int64_t cols, int round, uint64_t seed, uint8_t* codes, uint8_t* scales,
                          int64_t batch, const Segs& segs, hipStream_t st, int64_t s_pitch = 0) {
  const int ty = segs.n ? segs.tile_start[segs.n] : (int)cdiv(rows, kRqR);
  if (s_pitch == 0) s_pitch = (segs.n ? segs.out_len : rows) / 32;
  const RqJob j{codes_in, scales_in, rows, seed, codes, scales, s_pitch};
  return launch_requant_jobs(j, j, ty, 0, cols, round, batch, segs, st);
}

int requantize_impl(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows, int64_t cols,
                    int round, uint64_t seed, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return MX_OK;
  return launch_requant(codes_in, scales_in, rows, cols, round, seed, codes, scales, 1,
                        plain_segs(), st);
}

// Two packed row-blocked matrices [rows0, cols] and [rows1, cols] requantized
// (32x1, transposed outputs) by one launch, each with its own seed; the output
// scale rows are s_pitch0 / s_pitch1 bytes apart (0: packed).
int requantize_pair_impl(const uint8_t* codes_in0, const uint8_t* scales_in0, int64_t rows0,
                         const uint8_t* codes_in1, const uint8_t* scales_in1, int64_t rows1,
                         int64_t cols, int round, uint64_t seed0, uint64_t seed1,
                         uint8_t* codes0, uint8_t* scales0, uint8_t* codes1, uint8_t* scales1,
                         hipStream_t st, int64_t s_pitch0 = 0, int64_t s_pitch1 = 0) {
  if (cols == 0) return MX_OK;
  const RqJob j0{codes_in0, scales_in0, rows0, seed0, codes0, scales0,
                 s_pitch0 ? s_pitch0 : rows0 / 32};
  const RqJob j1{codes_in1, scales_in1, rows1, seed1, codes1, scales1,
                 s_pitch1 ? s_pitch1 : rows1 / 32};
  return launch_requant_jobs(j0, j1, (int)cdiv(rows0, kRqR), (int)cdiv(rows1, kRqR), cols, round,
                             1, plain_segs(), st);
}

// A stack of `batch` [rows, cols] matrices, each requantized on its own (the
// experts' weights); stochastic rounding indexes the stacked [batch*rows, cols].
int requantize_batched_impl(const uint8_t* codes_in, const uint8_t* scales_in, int64_t batch,
                            int64_t rows, int64_t cols, int round, uint64_t seed, uint8_t* codes,
                            uint8_t* scales, hipStream_t st, int64_t s_pitch = 0) {
  if (rows == 0 || cols == 0) return MX_OK;
  return launch_requant(codes_in, scales_in, rows, cols, round, seed, codes, scales, batch,
                        plain_segs(), st, s_pitch);
}

template <typename T>
static int launch_quant_rows2(const void* x0, int64_t n0, uint8_t* codes0, uint8_t* scales0,
                              uint64_t seed0, const void* x1, int64_t n1, uint8_t* codes1,
                              uint8_t* scales1, uint64_t seed1, int round, int had,
                              uint32_t mask, hipStream_t st) {
  RowJobs<T> jobs{};
  jobs.x0 = static_cast<const T*>(x0);
  jobs.x1 = static_cast<const T*>(x1);
  jobs.codes0 = reinterpret_cast<uint32_t*>(codes0);
  jobs.codes1 = reinterpret_cast<uint32_t*>(codes1);
  jobs.scales0 = scales0;
  jobs.scales1 = scales1;
  jobs.seed0 = seed0;
  jobs.seed1 = seed1;
  jobs.n0 = n0;
  jobs.n1 = n1;
  return launch_quant_row_jobs(jobs, round, had, mask, st);
}

// Row (1x32) quantization of two tensors of the same type and rounding in one
// launch: x0 [rows0, cols0] and x1 [rows1, cols1], each with its own outputs
// and seed (the logical indices of each start at 0).
int quantize_rows2_impl(const void* x0, int64_t rows0, int64_t cols0, uint8_t* codes0,
                        uint8_t* scales0, uint64_t seed0, const void* x1, int64_t rows1,
                        int64_t cols1, uint8_t* codes1, uint8_t* scales1, uint64_t seed1,
                        int dtype, int round, int had, uint32_t mask, hipStream_t st) {
  const int64_t n0 = rows0 * cols0 / 32, n1 = rows1 * cols1 / 32;
  if (n0 + n1 == 0) return MX_OK;
  return dtype == MX_BF16
             ? launch_quant_rows2<uint16_t>(x0, n0, codes0, scales0, seed0, x1, n1, codes1,
                                            scales1, seed1, round, had, mask, st)
             : launch_quant_rows2<float>(x0, n0, codes0, scales0, seed0, x1, n1, codes1, scales1,
                                         seed1, round, had, mask, st);
}

// 32x1 blocks per row segment (offs: host array of groups+1 row offsets).
int quantize_segments_impl(const void* x, int dtype, int64_t rows, int64_t cols,
                           const int64_t* offs, int64_t groups, int round, uint64_t seed,
                           uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return MX_OK;
  const Segs s = make_segs(offs, groups, kTileR);
  return dtype == MX_BF16
             ? launch_quant_tile<uint16_t, false>(static_cast<const uint16_t*>(x), rows, cols, round,
                                                  0, seed, 0, 0, nullptr, nullptr, codes, scales,
                                                  st, s)
             : launch_quant_tile<float, false>(static_cast<const float*>(x), rows, cols, round, 0,
                                               seed, 0, 0, nullptr, nullptr, codes, scales, st, s);
}

// Row (1x32) quantization of every row plus the per-segment column (32x1)
// quantization, from one read of x: the row pass of the tile kernel covers the
// segment's real rows only and writes them at their own rows, so the row output
// is the plain row quantization.
int quantize_dual_segments_impl(const void* x, int dtype, int64_t rows, int64_t cols,
                                const int64_t* offs, int64_t groups, int round, uint64_t seed_row,
                                uint64_t seed_col, uint8_t* codes_row, uint8_t* scales_row,
                                uint8_t* codes_col, uint8_t* scales_col, hipStream_t st,
                                int64_t sp_row = 0, int64_t sp_col = 0, int64_t pad = kSegPad) {
  if (rows == 0 || cols == 0) return MX_OK;
  const Segs s = make_segs(offs, groups, kTileR, pad);
  return dtype == MX_BF16
             ? launch_quant_tile<uint16_t, true>(static_cast<const uint16_t*>(x), rows, cols, round,
                                                 seed_row, seed_col, 0, 0, codes_row, scales_row,
                                                 codes_col, scales_col, st, s, sp_row, sp_col)
             : launch_quant_tile<float, true>(static_cast<const float*>(x), rows, cols, round,
                                              seed_row, seed_col, 0, 0, codes_row, scales_row,
                                              codes_col, scales_col, st, s, sp_row, sp_col);
}

int requantize_segments_impl(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                             int64_t cols, const int64_t* offs, int64_t groups, int round,
                             uint64_t seed, uint8_t* codes, uint8_t* scales, hipStream_t st,
                             int64_t s_pitch = 0, int64_t pad = kSegPad) {
  if (rows == 0 || cols == 0) return MX_OK;
  return launch_requant(codes_in, scales_in, rows, cols, round, seed, codes, scales, 1,
                        make_segs(offs, groups, kRqR, pad), st, s_pitch);
}

// sp_row / sp_col: bytes between scale rows of the row-blocked [rows][cols/32]
// and column-blocked [cols][rows/32] outputs (0: packed).
int quantize_dual_impl(const void* x, int dtype, int64_t rows, int64_t cols, int round,
                       uint64_t seed_row, uint64_t seed_col, int had, uint32_t mask,
                       uint8_t* codes_row, uint8_t* scales_row, uint8_t* codes_col,
                       uint8_t* scales_col, hipStream_t st, int64_t sp_row = 0,
                       int64_t sp_col = 0) {
  if (rows == 0 || cols == 0) return MX_OK;
  if (dtype == MX_BF16)
    return launch_quant_tile<uint16_t, true>(static_cast<const uint16_t*>(x), rows, cols, round,
                                             seed_row, seed_col, had, mask, codes_row, scales_row,
                                             codes_col, scales_col, st, plain_segs(), sp_row,
                                             sp_col);
  if (!had)
    return launch_quant_tile<float, true>(static_cast<const float*>(x), rows, cols, round,
                                          seed_row, seed_col, 0, 0, codes_row, scales_row,
                                          codes_col, scales_col, st, plain_segs(), sp_row, sp_col);
  if ((sp_row && sp_row != cols / 32) || (sp_col && sp_col != rows / 32)) return MX_ERR_SHAPE;
  // float32 with the rotation: a row block spans 8 lanes of the tile kernel, so
  // the two block shapes go through the row kernel and the column tile kernel
  const int s = quantize_impl(x, dtype, rows, cols, MX_ROW, round, seed_row, 1, mask, codes_row,
                              scales_row, st);
  if (s != MX_OK) return s;
  return quantize_impl(x, dtype, rows, cols, MX_COL, round, seed_col, 1, mask, codes_col,
                       scales_col, st);
}

static int launch_requant_rht(const RhtJobs& jobs, int ty1, int64_t cols, int round,
                              uint32_t mask, hipStream_t st) {
  if (jobs.ty0 + ty1 == 0 || cols == 0) return MX_OK;
  const dim3 grid((unsigned)cdiv(cols, kRhtC), (unsigned)(jobs.ty0 + ty1)), block(256);
  if (round == MX_RNE) k_requant_rht<MX_RNE><<<grid, block, 0, st>>>(jobs, cols, mask);
  else k_requant_rht<MX_SR><<<grid, block, 0, st>>>(jobs, cols, mask);
  return launch_status();
}

int requantize_rht_impl(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                        int64_t cols, int round, uint64_t seed, uint32_t mask, uint8_t* codes,
                        uint8_t* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return MX_OK;
  const RhtJobs j{codes_in, codes_in, scales_in, scales_in, rows, rows, seed, seed,
                  codes, codes, scales, scales, (int)cdiv(rows, kRhtR)};
  return launch_requant_rht(j, 0, cols, round, mask, st);
}

// Two rotated double quantizations (same cols and sign mask) in one launch.
int requantize_rht_pair_impl(const uint8_t* codes_in0, const uint8_t* scales_in0, int64_t rows0,
                             const uint8_t* codes_in1, const uint8_t* scales_in1, int64_t rows1,
                             int64_t cols, int round, uint64_t seed0, uint64_t seed1,
                             uint32_t mask, uint8_t* codes0, uint8_t* scales0, uint8_t* codes1,
                             uint8_t* scales1, hipStream_t st) {
  const RhtJobs j{codes_in0, codes_in1, scales_in0, scales_in1, rows0, rows1, seed0, seed1,
                  codes0, codes1, scales0, scales1, (int)cdiv(rows0, kRhtR)};
  return launch_requant_rht(j, (int)cdiv(rows1, kRhtR), cols, round, mask, st);
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

extern "C" int mx_quantize_ld(const void* x, int dtype, int64_t rows, int64_t cols, int axis,
                              int round, uint64_t seed, int hadamard, uint32_t sign_mask,
                              uint8_t* codes, uint8_t* scales, int64_t scale_ld, void* stream) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(axis == MX_ROW || axis == MX_COL, MX_ERR_ENUM);
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(hadamard == 0 || hadamard == 1, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0, MX_ERR_SHAPE);
  if (axis == MX_ROW) MX_REQUIRE(cols % 32 == 0, MX_ERR_SHAPE);
  else MX_REQUIRE(rows % 32 == 0 && cols % 8 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(scale_ld >= (axis == MX_ROW ? cols : rows) / 32, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && codes && scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(x) && aligned16(codes), MX_ERR_ALIGN);
  const int64_t nb = (axis == MX_ROW ? cols : rows) / 32;  // blocks per output row
  return quantize_impl(x, dtype, rows, cols, axis, round, seed, hadamard, sign_mask, codes, scales,
                       as_stream(stream), scale_ld == nb ? 0 : scale_ld);
}

extern "C" int mx_quantize_pair(const void* x0, int64_t rows0, const void* x1, int64_t rows1,
                                int64_t cols, int dtype, int round, uint64_t seed0,
                                uint64_t seed1, int hadamard, uint32_t sign_mask,
                                uint8_t* codes0, uint8_t* scales0, uint8_t* codes1,
                                uint8_t* scales1, void* stream) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(hadamard == 0 || hadamard == 1, MX_ERR_ENUM);
  MX_REQUIRE(rows0 >= 0 && rows1 >= 0 && cols >= 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (cols == 0 || rows0 + rows1 == 0) return MX_OK;
  if (rows0 > 0) {
    MX_REQUIRE(x0 && codes0 && scales0, MX_ERR_NULL);
    MX_REQUIRE(aligned16(x0) && aligned16(codes0), MX_ERR_ALIGN);
  }
  if (rows1 > 0) {
    MX_REQUIRE(x1 && codes1 && scales1, MX_ERR_NULL);
    MX_REQUIRE(aligned16(x1) && aligned16(codes1), MX_ERR_ALIGN);
  }
  return quantize_rows2_impl(x0, rows0, cols, codes0, scales0, seed0, x1, rows1, cols, codes1,
                             scales1, seed1, dtype, round, hadamard, sign_mask, as_stream(stream));
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
  return quantize_dual_impl(x, dtype, rows, cols, round, seed_row, seed_col, 0, 0, codes_row,
                            scales_row, codes_col, scales_col, as_stream(stream));
}

extern "C" int mx_quantize_dual_rht(const void* x, int dtype, int64_t rows, int64_t cols,
                                    int round, uint64_t seed_row, uint64_t seed_col,
                                    uint32_t sign_mask, uint8_t* codes_row, uint8_t* scales_row,
                                    uint8_t* codes_col, uint8_t* scales_col, void* stream) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0 && rows % 32 == 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && codes_row && scales_row && codes_col && scales_col, MX_ERR_NULL);
  MX_REQUIRE(aligned16(x) && aligned16(codes_row) && aligned16(codes_col), MX_ERR_ALIGN);
  return quantize_dual_impl(x, dtype, rows, cols, round, seed_row, seed_col, 1, sign_mask,
                            codes_row, scales_row, codes_col, scales_col, as_stream(stream));
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

extern "C" int mx_requantize_pair(const uint8_t* codes_in0, const uint8_t* scales_in0,
                                  int64_t rows0, const uint8_t* codes_in1,
                                  const uint8_t* scales_in1, int64_t rows1, int64_t cols,
                                  int round, uint64_t seed0, uint64_t seed1, uint8_t* codes_out0,
                                  uint8_t* scales_out0, uint8_t* codes_out1, uint8_t* scales_out1,
                                  void* stream) {
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(rows0 >= 0 && rows1 >= 0 && cols >= 0, MX_ERR_SHAPE);
  MX_REQUIRE(rows0 % 32 == 0 && rows1 % 32 == 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (cols == 0 || rows0 + rows1 == 0) return MX_OK;
  if (rows0 > 0) {
    MX_REQUIRE(codes_in0 && scales_in0 && codes_out0 && scales_out0, MX_ERR_NULL);
    MX_REQUIRE(aligned16(codes_in0) && aligned16(codes_out0), MX_ERR_ALIGN);
  }
  if (rows1 > 0) {
    MX_REQUIRE(codes_in1 && scales_in1 && codes_out1 && scales_out1, MX_ERR_NULL);
    MX_REQUIRE(aligned16(codes_in1) && aligned16(codes_out1), MX_ERR_ALIGN);
  }
  return requantize_pair_impl(codes_in0, scales_in0, rows0, codes_in1, scales_in1, rows1, cols,
                              round, seed0, seed1, codes_out0, scales_out0, codes_out1,
                              scales_out1, as_stream(stream));
}

extern "C" int mx_requantize_rht(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                                 int64_t cols, int round, uint64_t seed, uint32_t sign_mask,
                                 uint8_t* codes_out, uint8_t* scales_out, void* stream) {
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0 && rows % 32 == 0 && cols % 32 == 0, MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(codes_in && scales_in && codes_out && scales_out, MX_ERR_NULL);
  MX_REQUIRE(aligned16(codes_in) && aligned16(codes_out), MX_ERR_ALIGN);
  return requantize_rht_impl(codes_in, scales_in, rows, cols, round, seed, sign_mask, codes_out,
                             scales_out, as_stream(stream));
}

static bool valid_offsets(const int64_t* offs, int64_t groups, int64_t rows) {
  if (!offs || groups < 1 || groups > MX_MAX_GROUPS || offs[0] != 0 || offs[groups] != rows)
    return false;
  for (int64_t g = 0; g < groups; ++g)
    if (offs[g + 1] < offs[g]) return false;
  return true;
}

extern "C" int64_t mx_segments_padded_rows(const int64_t* offs, int64_t groups) {
  if (!offs || groups < 1 || groups > MX_MAX_GROUPS || offs[0] != 0) return -1;
  for (int64_t g = 0; g < groups; ++g)
    if (offs[g + 1] < offs[g]) return -1;
  return segments_padded_rows(offs, groups);
}

extern "C" int mx_quantize_segments(const void* x, int dtype, int64_t rows, int64_t cols,
                                    const int64_t* offs, int64_t groups, int round, uint64_t seed,
                                    uint8_t* codes, uint8_t* scales, void* stream) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0 && cols % 8 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(valid_offsets(offs, groups, rows), MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && codes && scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(x) && aligned16(codes), MX_ERR_ALIGN);
  return quantize_segments_impl(x, dtype, rows, cols, offs, groups, round, seed, codes, scales,
                                as_stream(stream));
}

extern "C" int mx_requantize_segments(const uint8_t* codes_in, const uint8_t* scales_in,
                                      int64_t rows, int64_t cols, const int64_t* offs,
                                      int64_t groups, int round, uint64_t seed,
                                      uint8_t* codes_out, uint8_t* scales_out, void* stream) {
  MX_REQUIRE(round == MX_RNE || round == MX_SR, MX_ERR_ENUM);
  MX_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(valid_offsets(offs, groups, rows), MX_ERR_SHAPE);
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(codes_in && scales_in && codes_out && scales_out, MX_ERR_NULL);
  MX_REQUIRE(aligned16(codes_in) && aligned16(codes_out), MX_ERR_ALIGN);
  return requantize_segments_impl(codes_in, scales_in, rows, cols, offs, groups, round, seed,
                                  codes_out, scales_out, as_stream(stream));
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
