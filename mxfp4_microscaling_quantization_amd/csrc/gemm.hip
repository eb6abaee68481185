// MXFP4 GEMM on CDNA4's block-scaled FP4 matrix cores.
//
// C[m][n] = alpha * sum_k deq(A)[m][k] * deq(B)[n][k], A [M, K] and B [N, K]
// both packed along K (E2M1 codes + one E8M0 scale per 32 elements): the
// (1x32) x (32x1) MXFP4 product of "Oscillation-Reduced MXFP4 Training for
// Vision Transformers" (rebuttal, Question 2 (1) and (2)).
//
// Each V_MFMA_SCALE_F32_32X32X64_F8F6F4 multiplies a 32x64 FP4 tile by a
// 64x32 FP4 tile and applies one E8M0 scale per 32 K-values of every row /
// column, so the block scales go straight to the instruction and the products
// are exact; only the fp32 accumulation rounds.  Per lane, an operand is 16
// bytes: row (lane % 32), K-values [32 (lane / 32), 32 (lane / 32) + 32) of the
// instruction's 64, and the scale operand holds that row's bytes (the scale
// op_sel picks the byte).
//
// The instruction is fed B as its first operand and A as its second, so it
// produces D[n][m]: a lane then holds 4 consecutive n of one output row m (one
// 16-byte piece); the epilogue stages the tile through LDS so that each store
// instruction writes whole row segments of C.
//
// Tiling: a workgroup of WM x WN waves owns a BM x BN tile of C (256 x 256 for
// large problems: 2 x 4 waves of 128 x 64 with 16-byte scale-group loads, else
// 2 x 2 waves of 128 x 128, 16 accumulator tiles; 128 x 128 for small ones) and walks K in steps of 128 (64 code bytes per row) through a 4-stage
// LDS ring.  Direct global-to-LDS loads fill a stage three steps ahead; each
// step reads the second K-half's fragments while the first half's MFMAs run,
// and the next step's first half while the second half's run, with one
// barrier per step.  A contraction of at most three steps takes a 3-stage ring
// (three workgroups per CU); two small products can share one launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_schedule.h"
#include "mx_host.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFmtFp4 = 4;  // cbsz / blgp operand format: FP4 E2M1

struct GemmGroups {
  int ngroups;
  int tiles_n;                              // tiles along N (same for every group)
  int64_t lds_a, lds_b;                     // bytes between scale rows of A and of B
  int tile_start[MX_MAX_GROUPS + 1];        // prefix sum of tiles per group
  int64_t row_off[MX_MAX_GROUPS + 1];       // rows of A / C per group
};

// Contraction ranges: split s of n covers K-values [kbeg[s], kbeg[s] + klen[s])
// (each start a multiple of 128, each length a multiple of 32) and writes its
// own output at C + s c_stride, alpha applied per split.  Used for split-K
// (partial sums added afterwards) and for the experts' weight gradients (each
// over its own token range; a range may end before the next one starts).
struct GemmSplit {
  int n;
  int stream_c;                       // 1: final outputs, stored non-temporally
  int64_t c_stride;                   // elements between the splits' outputs
  int64_t kbeg[MX_MAX_GROUPS + 1];
  int32_t klen[MX_MAX_GROUPS];        // range lengths (kbeg[s+1] - kbeg[s] when contiguous)
};

// Contiguous ranges: split s ends where split s+1 begins.
static void contiguous_ranges(GemmSplit& sp) {
  for (int s = 0; s < sp.n; ++s) sp.klen[s] = (int32_t)(sp.kbeg[s + 1] - sp.kbeg[s]);
}

// A second, plain problem in the same launch (one group, the whole contraction,
// a final output): workgroups past the first problem's take its tiles.  Two
// small products that each fill one partial round of the CUs (the backward
// layer's dX and dW at a few thousand tokens) then overlap instead of running
// one after the other.
struct GemmPlain {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  int64_t M, N, K;
  float alpha;
  float* C;
  int64_t ldc;
  int64_t lds_a, lds_b;  // bytes between scale rows of A and of B
  int tiles, tiles_n;
};

// 16-byte store of C.  Final outputs are written with non-temporal stores: the
// next kernel does not read them, and a GEMM's output (up to several hundred MB)
// left dirty in the Infinity Cache would otherwise be written back during the
// next kernel, slowing it (measured 1.6x on an HBM-bound quantizer after a
// 235 MB output).  Split-K partials, read back at once, use ordinary stores.
__device__ __forceinline__ void store_c4(float* p, float4 v, bool stream) {
  if (stream) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<v4f*>(p));
  } else {
    *reinterpret_cast<float4*>(p) = v;
  }
}

constexpr int kGroupM = 4;  // tile rows walked together (L2 reuse of B tiles)

__device__ __forceinline__ v8i as_v8i(uint4 u) {
  v8i r = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
  return r;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t lmax(int64_t a, int64_t b) { return a > b ? a : b; }

// Direct global -> LDS loads (no destination VGPRs): lane i's 16 bytes (or 1
// byte) land at LDS address M0 + 16 i (or M0 + i).  Written as asm so that the
// compiler does not track these writes itself: the kernel waits on vmcnt
// explicitly before each barrier, and the "memory" clobber keeps LDS reads
// from moving above an issue.  M0 is set in the same block.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is written on purpose, nothing else here uses it
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_addr(lds)), "v"(g)
               : "memory", "m0");
}
// The same load from an SGPR base plus a 32-bit per-lane offset: the wave
// hands the address unit half the address data, and the instruction issues
// in about a third of the cycles between MFMAs (measured interleaved with
// scaled FP4 MFMAs).
__device__ __forceinline__ void dma16s(const uint8_t* base, uint32_t voff, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr(lds)), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds_addr(lds)), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, off"
               :
               : "s"(lds_addr(lds)), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void dma1(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ubyte %1, off"
               :
               : "s"(lds_addr(lds)), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Operand tile in LDS, per stage: codes [rows][64 B] with the four 16-byte
// chunks of row r stored in the order c ^ ((r >> 2) & 3), so that the 16 lanes
// reading chunk c of 16 consecutive rows hit 16 different bank groups.  One
// direct-to-LDS load moves 16 rows (4 lanes per row, 64 contiguous bytes of
// global memory).
// Scales: a dword DMA puts lane i's 4 bytes at [4i, 4i+4); a ushort (byte) DMA
// puts lane i's 2 bytes (byte) zero-extended in dword i.  With 4-byte aligned scale rows
// (K/32 % 4 == 0) one dword per row carries the step's four scale bytes:
// layout [rows][4] bytes.  Otherwise one byte per dword: layout [4][rows] dwords.
// Scale modes: kScGroup -- K/32 % 16 == 0: one 16-byte load per row brings the
// scales of four K-steps into a separate double buffer [rows][16 B] once per
// four steps (a quarter of the cache lines a per-step load touches);
// kScDword -- K/32 % 4 == 0: one dword per row and step, layout [rows][4];
// kScShort -- K/32 % 2 == 0: two 2-byte loads per row and step, layout [2][rows]
// dwords (bytes 0-1 and 2-3 of the step);
// kScByte -- otherwise: one byte per row and step, layout [4][rows] dwords.
// (the mode constants kScGroup .. kScShort live in gemm_schedule.h)

template <int ROWS, int SC>
struct TileLds {
  uint4 codes[ROWS * 4];
  uint32_t scales[SC == kScGroup ? 1 : (SC == kScDword ? ROWS : (SC == kScShort ? ROWS * 2 : ROWS * 4))];
};

template <int BM, int BN, int SC>
struct StageLds {
  TileLds<BM, SC> a;
  TileLds<BN, SC> b;
};

template <int BM, int BN>
struct ScaleGroupLds {
  uint4 a[BM];
  uint4 b[BN];
};

// The work of one workgroup: which problem (first or paired second), group,
// contraction range and output tile, and where its operands and output live.
// The first problem's workgroups come first in dispatch order.  Within a
// problem, consecutive logical tiles are spread over one XCD (workgroups are
// dealt round-robin to the 8 XCDs), then tile rows are walked kGroupM at a time.
struct TileWork {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  float* C;
  int64_t N, ldc, ldk, lds_a, lds_b, a_last, m0, n0, k0, kc_bytes, kc_blocks;
  float alpha;
  bool stream_c;
  int rows_valid, cols_valid, KT, tail_kb;
};

template <int BM, int BN, bool PAIR>
__device__ __forceinline__ TileWork tile_work(const uint8_t* A0, const uint8_t* SA0,
                                              const uint8_t* B0, const uint8_t* SB0, int64_t N0,
                                              int64_t K0, float alpha0, float* C0, int64_t ldc0,
                                              int64_t b_stride_codes, int64_t b_stride_scales,
                                              const GemmGroups& gg, const GemmSplit& sp,
                                              const GemmPlain& p1) {
  const int tiles0 = gg.tile_start[gg.ngroups];
  const int total0 = tiles0 * sp.n;
  const bool second = PAIR && (int)blockIdx.x >= total0;  // uniform over the workgroup
  const int total = second ? p1.tiles : total0;
  int id = (int)blockIdx.x - (second ? total0 : 0);
  {
    const int q = total / 8, r = total % 8, x = id % 8;
    id = x * q + min(x, r) + id / 8;
  }
  int split = 0, g = 0, tiles_n = p1.tiles_n;
  int64_t grow0 = 0, grows = p1.M, a_last = p1.M - 1, k0 = 0, k1 = p1.K;
  if (!second) {
    split = id / tiles0;
    id -= split * tiles0;
    while (g + 1 < gg.ngroups && gg.tile_start[g + 1] <= id) ++g;
    id -= gg.tile_start[g];
    tiles_n = gg.tiles_n;
    grow0 = gg.row_off[g];
    grows = gg.row_off[g + 1] - grow0;
    a_last = gg.row_off[gg.ngroups] - 1;  // last row of A in memory
    k0 = sp.kbeg[split];
    k1 = k0 + sp.klen[split];
  }
  TileWork w;
  w.A = second ? p1.A : A0;
  w.SA = second ? p1.SA : SA0;
  w.N = second ? p1.N : N0;
  const int64_t K = second ? p1.K : K0;
  w.alpha = second ? p1.alpha : alpha0;
  w.ldc = second ? p1.ldc : ldc0;
  w.stream_c = second || sp.stream_c != 0;
  w.C = second ? p1.C : C0 + split * sp.c_stride;
  w.B = second ? p1.B : B0 + (int64_t)g * b_stride_codes;
  w.SB = second ? p1.SB : SB0 + (int64_t)g * b_stride_scales;
  const int lt = id;
  const int tiles_m = (int)((grows + BM - 1) / BM);
  const int span = kGroupM * tiles_n;
  const int first_m = (lt / span) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int tm_idx = first_m + (lt % span) % gm;
  const int tn_idx = (lt % span) / gm;

  w.m0 = grow0 + (int64_t)tm_idx * BM;
  w.rows_valid = (int)min<int64_t>(BM, grow0 + grows - w.m0);
  w.n0 = (int64_t)tn_idx * BN;
  w.cols_valid = (int)min<int64_t>(BN, w.N - w.n0);
  w.a_last = a_last;
  w.k0 = k0;
  w.ldk = K / 2;   // code bytes per row
  w.lds_a = second ? p1.lds_a : gg.lds_a;  // bytes between scale rows
  w.lds_b = second ? p1.lds_b : gg.lds_b;
  const int64_t kc_len = k1 - k0;  // K-values of this range
  w.kc_bytes = kc_len / 2;
  w.kc_blocks = kc_len / 32;
  w.KT = (int)((kc_len + 127) / 128);
  w.tail_kb = (int)(w.kc_blocks - (int64_t)(w.KT - 1) * 4);  // valid 32-blocks in the last step
  return w;
}

// Epilogue of a BM x BN tile held by WM x WN waves in acc[TN][TM] (lane holds
// D[n = 8 g + 4 lh + v][m = lr], g, v = 0..3, of each 32x32 tile).  The LDS ring
// is idle by then: each wave stages its sub-tile there, 64 rows per pass (32
// when the ring is too small for that; row pitch CH 16-byte chunks, chunk index
// XORed with row & 15, so the 16-row writes and the row reads are free of bank
// conflicts), and reads it back so that every store instruction writes whole
// row segments of C (two rows of 512 bytes for 256 x 256 tiles, four of 256 for
// 128 x 128) instead of 32-byte pieces of 32 rows.
template <int BM, int BN, int WM, int WN, int TM, int TN, int RING>
__device__ __forceinline__ void store_tile_impl(v16f (&acc)[TN][TM], char* ring,
                                                const TileWork& tw) {
  constexpr int NW = WM * WN;
  constexpr int CH = TN * 8;      // 16-byte chunks per staged row
  constexpr int RB = CH * 16;     // bytes per staged row
  constexpr int RPI = 64 / CH;    // rows per read (one chunk per lane)
  constexpr int PR = RING >= NW * 64 * RB ? 64 : 32;  // rows per pass
  constexpr int PB = PR / 32;     // 32-row MFMA tiles per pass
  static_assert(TM % PB == 0 && CH >= 16 && 64 % CH == 0, "staging shape");
  static_assert(RING >= NW * PR * RB, "staging space");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm_off = (wave / WN) * (BM / WM);
  const int wn_off = (wave % WN) * (BN / WN);
  const int lr = lane & 31, lh = lane >> 5;
  const float alpha = tw.alpha;
  __syncthreads();  // every wave is done reading the ring
  char* stg = ring + wave * PR * RB;
#pragma unroll
  for (int p = 0; p < TM / PB; ++p) {
#pragma unroll
    for (int bb = 0; bb < PB; ++bb) {
      const int b = PB * p + bb;
      const int rl = bb * 32 + lr;
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int ch = a * 8 + gq * 2 + lh;
          *reinterpret_cast<float4*>(stg + rl * RB + ((ch ^ (rl & 15)) * 16)) =
              make_float4(acc[a][b][4 * gq] * alpha, acc[a][b][4 * gq + 1] * alpha,
                          acc[a][b][4 * gq + 2] * alpha, acc[a][b][4 * gq + 3] * alpha);
        }
    }
#pragma unroll 4
    for (int it = 0; it < PR / RPI; ++it) {
      const int rl = it * RPI + lane / CH, ch = lane % CH;
      const float4 v = *reinterpret_cast<const float4*>(stg + rl * RB + ((ch ^ (rl & 15)) * 16));
      const int mrow = wm_off + p * PR + rl;
      const int ncol = wn_off + ch * 4;
      if (mrow < tw.rows_valid) {
        float* crow = tw.C + (tw.m0 + mrow) * tw.ldc + tw.n0;
        if (ncol + 3 < tw.cols_valid) {
          store_c4(crow + ncol, v, tw.stream_c);
        } else {
          if (ncol + 0 < tw.cols_valid) crow[ncol + 0] = v.x;
          if (ncol + 1 < tw.cols_valid) crow[ncol + 1] = v.y;
          if (ncol + 2 < tw.cols_valid) crow[ncol + 2] = v.z;
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int SC, bool PAIR>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm_mx(
    const uint8_t* __restrict__ A0, const uint8_t* __restrict__ SA0, const uint8_t* __restrict__ B0,
    const uint8_t* __restrict__ SB0, int64_t N0, int64_t K0, float alpha0, float* __restrict__ C0,
    int64_t ldc0, int64_t b_stride_codes, int64_t b_stride_scales, GemmGroups gg, GemmSplit sp,
    const GemmPlain p1) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32;  // 32-row MFMA tiles per wave along m
  constexpr int TN = BN / WN / 32;  // along n
  constexpr int LA = BM / 16 / NW;  // code DMAs per wave per step, A (16 rows each)
  constexpr int LB = BN / 16 / NW;
  constexpr int QG = (BM + BN) / 64;                 // 64-row groups of both operands
  constexpr int QJ = SC == kScByte ? 4 * QG : (SC == kScShort ? 2 * QG : QG);  // scale jobs
  constexpr int QW = QJ / NW;  // scale DMAs per wave per step (or group)
  constexpr int LC = LA + LB + (SC == kScGroup ? 0 : QW);  // per-step vector-memory instructions
  static_assert(LA * NW * 16 == BM && LB * NW * 16 == BN, "tile/wave mismatch");
  static_assert(QW * NW == QJ && BM % 64 == 0 && BN % 64 == 0, "scale jobs");
  // STAGES 4: the pipelined ring.  STAGES 3: a short contraction (at most three
  // K-steps, guaranteed by the host), whose loads are all issued up front: the
  // fourth stage is never used, and the smaller ring lets one more workgroup
  // share a CU.
  static_assert((STAGES == 4 || (STAGES == 3 && SC != kScGroup)) && 2 * LC + QW < 64,
                "pipeline depth");
  static_assert(mx_schedule_listed(BM, BN, NW, SC, LC, QW),
                "tile configuration missing from the schedule table of gemm_schedule.h");

  // The LDS ring (contiguous, reused by the epilogue); every access uses a
  // compile-time stage index (with three stages, index 3 is on paths a short
  // contraction never takes).
  __shared__ StageLds<BM, BN, SC> ring[STAGES];
  __shared__ ScaleGroupLds<(SC == kScGroup ? BM : 1), (SC == kScGroup ? BN : 1)> sg[2];
  auto stage = [&](auto S) -> StageLds<BM, BN, SC>& { return ring[decltype(S)::value % STAGES]; };
  auto bufA = [&](auto S) -> TileLds<BM, SC>& { return stage(S).a; };
  auto bufB = [&](auto S) -> TileLds<BN, SC>& { return stage(S).b; };

  const TileWork tw = tile_work<BM, BN, PAIR>(A0, SA0, B0, SB0, N0, K0, alpha0, C0, ldc0,
                                              b_stride_codes, b_stride_scales, gg, sp, p1);
  const uint8_t* __restrict__ A = tw.A;
  const uint8_t* __restrict__ SA = tw.SA;
  const uint8_t* Bg = tw.B;
  const uint8_t* SBg = tw.SB;
  const int64_t N = tw.N, ldk = tw.ldk, lds_a = tw.lds_a, lds_b = tw.lds_b, a_last = tw.a_last;
  const int64_t m0 = tw.m0, n0 = tw.n0, k0 = tw.k0, kc_bytes = tw.kc_bytes, kc_blocks = tw.kc_blocks;
  const int KT = tw.KT, tail_kb = tw.tail_kb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm_off = (wave / WN) * (BM / WM);
  const int wn_off = (wave % WN) * (BN / WN);
  const int lr = lane & 31;  // MFMA operand row of this lane
  const int lh = lane >> 5;  // which 32-block of the instruction's 64 K-values

  // Per-lane DMA sources for this wave's rows (row clamped into memory; rows
  // past the tile's valid range feed outputs that are never stored).
  const int dr = lane >> 2;                        // row within a 16-row group
  const int dc = (lane & 3) ^ ((dr >> 2) & 3);     // chunk this lane fetches
  const uint8_t* a_src[LA];
  const uint8_t* b_src[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int64_t row = lmin(m0 + (wave * LA + j) * 16 + dr, a_last);
    a_src[j] = A + row * ldk + k0 / 2 + dc * 16;
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int64_t row = lmin(n0 + (wave * LB + j) * 16 + dr, N - 1);
    b_src[j] = Bg + row * ldk + k0 / 2 + dc * 16;
  }
  // scale jobs: job q covers 64 rows (lane = row) of A (q % QG < BM/64) or B,
  // for all 32-blocks of a step (dword), of four steps (group), for 32-blocks
  // 2 (q / QG) and 2 (q / QG) + 1 (short mode) or for 32-block q / QG (byte mode)
  const uint8_t* s_src[QW];
  int s_dst[QW];  // dword / uint4 offset in the A or B scale area, B marked by +2^20
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int q = wave * QW + j;
    const int grp = q % QG, part = (SC == kScByte || SC == kScShort) ? q / QG : 0;
    const int kb = SC == kScShort ? 2 * part : part;  // first 32-block the job loads
    const bool isA = grp < BM / 64;
    const int r0 = (isA ? grp : grp - BM / 64) * 64;
    const int64_t row = isA ? lmin(m0 + r0 + lane, a_last) : lmin(n0 + r0 + lane, N - 1);
    s_src[j] = (isA ? SA : SBg) + row * (isA ? lds_a : lds_b) + k0 / 32 + kb;
    s_dst[j] = ((SC == kScByte || SC == kScShort) ? part * (isA ? BM : BN) + r0 : r0) +
               (isA ? 0 : (1 << 20));
  }

  auto issue = [&](int kt, auto S) {
    // the last step may have fewer than 4 valid 32-blocks: clamp the column so
    // the load stays inside the row; those blocks are masked before the MFMA.
    TileLds<BM, SC>& ta = bufA(S);
    TileLds<BN, SC>& tb = bufB(S);
    const int64_t kc = (int64_t)kt * 64;
    const int64_t coff = lmin(kc, lmax(kc_bytes - 16 - dc * 16, -dc * 16));
#pragma unroll
    for (int j = 0; j < LA; ++j) dma16(a_src[j] + coff, &ta.codes[((wave * LA + j) * 16) * 4]);
#pragma unroll
    for (int j = 0; j < LB; ++j) dma16(b_src[j] + coff, &tb.codes[((wave * LB + j) * 16) * 4]);
    if constexpr (SC != kScGroup) {
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        const bool isB = s_dst[j] >= (1 << 20);
        uint32_t* dst = isB ? &tb.scales[s_dst[j] - (1 << 20)] : &ta.scales[s_dst[j]];
        if (SC == kScDword) {
          dma4(s_src[j] + (int64_t)kt * 4, dst);
        } else if (SC == kScShort) {
          // bytes [4 kt + kb, 4 kt + kb + 2), clamped into the row (kc_blocks >= 2)
          const int kb = 2 * ((wave * QW + j) / QG);
          dma2(s_src[j] + lmin((int64_t)kt * 4, kc_blocks - 2 - kb), dst);
        } else {
          const int kb = (wave * QW + j) / QG;
          dma1(s_src[j] + lmin((int64_t)kt * 4, kc_blocks - 1 - kb), dst);
        }
      }
    }
  };
  // group mode: scales of steps 4 g .. 4 g + 3 (16 bytes per row) into sg[g & 1]
  auto issue_scales = [&](int grp) {
    if constexpr (SC == kScGroup) {
      ScaleGroupLds<(SC == kScGroup ? BM : 1), (SC == kScGroup ? BN : 1)>& t = sg[grp & 1];
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        const bool isB = s_dst[j] >= (1 << 20);
        uint4* dst = isB ? &t.b[s_dst[j] - (1 << 20)] : &t.a[s_dst[j]];
        dma16(s_src[j] + (int64_t)grp * 16, dst);
      }
    }
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // an empty contraction range (an expert without tokens) loads nothing and
  // writes zeros
  if (0 < KT) issue_scales(0);
  if (0 < KT) issue(0, I0{});
  if (1 < KT) issue(1, I1{});
  if (2 < KT) issue(2, I2{});

  // Fragment registers: f?[h] holds the lane's 16 code bytes for K-half h of
  // the current step; s?c the current step's scale dwords, s?n the next one's.
  uint4 fa[2][TM], fb[2][TN];
  uint32_t sac[TM], sbc[TN];

  // read scales of step kt (stage S) into sa/sb
  auto read_scales = [&](int kt, auto S, uint32_t (&sa)[TM], uint32_t (&sb)[TN]) {
    constexpr int P = decltype(S)::value;
    const uint8_t* sab = SC == kScGroup ? reinterpret_cast<const uint8_t*>(sg[(kt >> 2) & 1].a)
                                        : reinterpret_cast<const uint8_t*>(bufA(S).scales);
    const uint8_t* sbb = SC == kScGroup ? reinterpret_cast<const uint8_t*>(sg[(kt >> 2) & 1].b)
                                        : reinterpret_cast<const uint8_t*>(bufB(S).scales);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int row = wm_off + t * 32 + lr;
      if constexpr (SC == kScByte) {
        sa[t] = (uint32_t)sab[4 * (lh * BM + row)] | ((uint32_t)sab[4 * ((2 + lh) * BM + row)] << 16);
      } else if constexpr (SC == kScShort) {
        const uint32_t* s32 = reinterpret_cast<const uint32_t*>(sab);
        sa[t] = (s32[row] | (s32[BM + row] << 16)) >> (8 * lh);
      } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(
            sab + (SC == kScGroup ? row * 16 + P * 4 : row * 4));
        sa[t] = w >> (8 * lh);
      }
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int row = wn_off + t * 32 + lr;
      if constexpr (SC == kScByte) {
        sb[t] = (uint32_t)sbb[4 * (lh * BN + row)] | ((uint32_t)sbb[4 * ((2 + lh) * BN + row)] << 16);
      } else if constexpr (SC == kScShort) {
        const uint32_t* s32 = reinterpret_cast<const uint32_t*>(sbb);
        sb[t] = (s32[row] | (s32[BN + row] << 16)) >> (8 * lh);
      } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(
            sbb + (SC == kScGroup ? row * 16 + P * 4 : row * 4));
        sb[t] = w >> (8 * lh);
      }
    }
  };
  auto read_frags = [&](int h, auto S) {
    const TileLds<BM, SC>& ta = bufA(S);
    const TileLds<BN, SC>& tb = bufB(S);
    const int kb = 2 * h + lh;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int row = wm_off + t * 32 + lr;
      fa[h][t] = ta.codes[row * 4 + (kb ^ ((row >> 2) & 3))];
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int row = wn_off + t * 32 + lr;
      fb[h][t] = tb.codes[row * 4 + (kb ^ ((row >> 2) & 3))];
    }
  };
  // 32-blocks past K in the last step: zero A's codes, neutral scales (127)
  auto mask_tail = [&](int h, uint32_t (&sa)[TM], uint32_t (&sb)[TN]) {
    if (2 * h + lh >= tail_kb) {
      const uint32_t keep = h ? 0x0000FFFFu : 0xFFFF0000u;
      const uint32_t neutral = h ? 0x007F0000u : 0x0000007Fu;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        fa[h][t] = make_uint4(0, 0, 0, 0);
        sa[t] = (sa[t] & keep) | neutral;
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) sb[t] = (sb[t] & keep) | neutral;
    }
  };
  auto mfma_half = [&](auto H, const uint32_t (&sa)[TM], const uint32_t (&sb)[TN]) {
    constexpr int h = decltype(H)::value;
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            as_v8i(fb[h][a]), as_v8i(fa[h][b]), acc[a][b], kFmtFp4, kFmtFp4, h ? 2 : 0, (int)sb[a],
            h ? 2 : 0, (int)sa[b]);
  };

  // Barrier that also drains this wave's LDS reads, so a stage is never
  // refilled while a read of it is in flight, whatever order the compiler
  // gives the surrounding code.
  auto barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // stage 0 (and scale group 0) landed for every wave
  if (2 < KT) wait_vmcnt<2 * LC>();
  else if (1 < KT) wait_vmcnt<LC>();
  else wait_vmcnt<0>();
  barrier();
  read_scales(0, I0{}, sac, sbc);
  read_frags(0, I0{});

  // Step kt: read K-half 1 of stage kt; MFMAs of half 0; wait for stage kt+1
  // and barrier (every wave is then also done with stage kt-1); refill stage
  // kt-1 with step kt+3; read half 0 and the scales of step kt+1; MFMAs of
  // half 1.  LDS reads thus overlap the other half's MFMAs.  FULL steps have
  // kt + 7 < KT rounded down to a multiple of 4: every load is issued and no
  // K tail, so the step is straight-line code the scheduler keeps in order.
  auto step = [&](int kt, auto S, auto FULL) {
    constexpr int P = decltype(S)::value;  // kt % 4
    constexpr bool F = decltype(FULL)::value;
    using SN1 = std::integral_constant<int, (P + 1) % 4>;
    using SN3 = std::integral_constant<int, (P + 3) % 4>;
    // vector-memory instructions issued after step kt+1's loads may stay in
    // flight at the barrier: step kt+2's loads and, in group mode, a scale
    // group issued at step kt-2 (before them) or kt-1 (after them)
    constexpr int G2 = (SC == kScGroup && P == 2) ? QW : 0;
    constexpr int G1 = (SC == kScGroup && P == 1) ? QW : 0;
    uint32_t san[TM], sbn[TN];
    read_frags(1, S);
    if (!F && kt == KT - 1) mask_tail(0, sac, sbc);
    mfma_half(I0{}, sac, sbc);
    if constexpr (F) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<LC + G1 + G2>();
      barrier();
      issue(kt + 3, SN3{});
      if (P == 0) issue_scales((kt >> 2) + 1);
      read_scales(kt + 1, SN1{}, san, sbn);
      read_frags(0, SN1{});
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(I1{}, sac, sbc);
#pragma unroll
      for (int t = 0; t < TM; ++t) sac[t] = san[t];
#pragma unroll
      for (int t = 0; t < TN; ++t) sbc[t] = sbn[t];
    } else {
      if (kt + 1 < KT) {
        if (kt + 3 < KT) wait_vmcnt<LC + G1 + G2>();
        else if (kt + 2 < KT) wait_vmcnt<LC + G2>();
        else wait_vmcnt<0>();
        barrier();
        if (kt + 3 < KT) issue(kt + 3, SN3{});
        if (P == 0 && kt + 4 < KT) issue_scales((kt >> 2) + 1);
        read_scales(kt + 1, SN1{}, san, sbn);
      }
      if (kt == KT - 1) mask_tail(1, sac, sbc);
      mfma_half(I1{}, sac, sbc);
      if (kt + 1 < KT) {
        read_frags(0, SN1{});
#pragma unroll
        for (int t = 0; t < TM; ++t) sac[t] = san[t];
#pragma unroll
        for (int t = 0; t < TN; ++t) sbc[t] = sbn[t];
      }
    }
  };

  using Full = std::true_type;
  using Part = std::false_type;
  int kt = 0;
  for (; kt + 7 < KT; kt += 4) {
    step(kt, I0{}, Full{});
    step(kt + 1, I1{}, Full{});
    step(kt + 2, I2{}, Full{});
    step(kt + 3, I3{}, Full{});
  }
  for (; kt < KT; kt += 4) {
    step(kt, I0{}, Part{});
    if (kt + 1 < KT) step(kt + 1, I1{}, Part{});
    if (kt + 2 < KT) step(kt + 2, I2{}, Part{});
    if (kt + 3 < KT) step(kt + 3, I3{}, Part{});
  }

  store_tile_impl<BM, BN, WM, WN, TM, TN, (int)sizeof(ring)>(
      acc, reinterpret_cast<char*>(ring), tw);
}

// Ping-pong variant for 256 x 256 tiles with 16-byte scale-group loads: eight
// waves, two per SIMD (waves w and w + 4), in two groups: waves 0-3 own rows
// 0-127 of the tile, waves 4-7 rows 128-255, each wave 128 x 64 of C.  Every
// K-step is a load phase L (read the step's fragments of both K-halves and its
// scales into registers, wait for them) and a compute phase C (the step's 16
// MFMAs, with this wave's share of the global -> LDS loads three steps ahead
// issued between them, one per four MFMAs), each ended by a workgroup barrier.
// Group 1 starts one barrier late, so while one wave of a SIMD runs its MFMAs
// the other reads its fragments: the MFMA pipe alternates between the two
// waves' bursts, and no wave needs a second set of fragment registers.  The
// loads are spread over the MFMA bursts because the address unit moves about
// 64 bytes per clock per CU (a 1 KB load takes ~16 of the 32 clocks of an
// MFMA): issued all at once they stall the issuing waves for hundreds of
// clocks (measured), spread out they cost a few clocks each.
// Barriers: 0 ends the prologue; group 0's L(j) runs between barriers 2j and
// 2j+1 and its C(j) between 2j+1 and 2j+2, group 1 one barrier later.  Stage j
// of the ring is read in L(j) by both groups, so by barrier 2j+2; the load of
// step j+3 into the stage of step j-1 is issued in C(j), after barrier 2j+1.
// Each wave waits for its own share of step j+1 at the end of its L(j), by
// barrier 2j+2 at the latest, before any wave reads that stage.
// UNAL: scale rows whose groups are not 16-byte aligned (a packed operand with
// K / 32 not a multiple of 16, such as the 90-byte rows of K = 2880, or a
// contraction range starting off a 512 boundary).  A lane then fetches the two
// aligned 16-byte pieces holding its row's group (the second only when it holds
// a byte of the range, so no load leaves the 16-byte blocks that hold the
// row's bytes) into sg and sgx, and at the end of L(4g + 3), once they have
// landed, shifts the group into place in sg: the readers see the same layout
// as in the aligned case.
template <bool UNAL>
__global__ __launch_bounds__(512) void k_gemm_pp(
    const uint8_t* __restrict__ A0, const uint8_t* __restrict__ SA0, const uint8_t* __restrict__ B0,
    const uint8_t* __restrict__ SB0, int64_t N0, int64_t K0, float alpha0, float* __restrict__ C0,
    int64_t ldc0, int64_t b_stride_codes, int64_t b_stride_scales, GemmGroups gg, GemmSplit sp) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4, NW = 8;
  constexpr int TM = 4, TN = 2;  // 32 x 32 MFMA tiles per wave along m and n
  constexpr int LA = 2, LB = 2;  // code DMAs per wave per step (16 rows each)
  constexpr int LC = LA + LB;
  constexpr int GL = UNAL ? kPpGroupLoadsUnal : kPpGroupLoads;  // loads per scale group
  static_assert(LA * NW * 16 == BM && LB * NW * 16 == BN, "tile/wave mismatch");
  static_assert(kPpLoads == LC && kPpGroupLoads == 1 && kPpGroupLoadsUnal == 2 && kPpLead == 3 &&
                    kPpWaitNear == LC && kPpWaitFirst[0] == 0 && kPpWaitFirst[1] == LC &&
                    kPpWaitFirst[2] == 2 * LC,
                "schedule constants of gemm_schedule.h");
  __shared__ StageLds<BM, BN, kScGroup> ring[4];
  __shared__ ScaleGroupLds<BM, BN> sg[2];
  __shared__ ScaleGroupLds<UNAL ? BM : 1, UNAL ? BN : 1> sgx;  // second pieces (UNAL)

  const TileWork tw = tile_work<BM, BN, false>(A0, SA0, B0, SB0, N0, K0, alpha0, C0, ldc0,
                                               b_stride_codes, b_stride_scales, gg, sp,
                                               GemmPlain{});
  const int64_t kc_bytes = tw.kc_bytes;
  const int KT = tw.KT, tail_kb = tw.tail_kb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;           // 0: rows 0-127, 1: rows 128-255
  const int wm_off = grp * (BM / WM);
  const int wn_off = (wave & 3) * (BN / WN);
  const int lr = lane & 31;            // MFMA operand row of this lane
  const int lh = lane >> 5;            // which 32-block of the instruction's 64 K-values

  // DMA sources: rows clamped into memory (rows past the tile feed outputs
  // that are never stored)
  const int dr = lane >> 2;
  const int dc = (lane & 3) ^ ((dr >> 2) & 3);
  const uint8_t* a_src[LA];
  const uint8_t* b_src[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int64_t row = lmin(tw.m0 + (wave * LA + j) * 16 + dr, tw.a_last);
    a_src[j] = tw.A + row * tw.ldk + tw.k0 / 2 + dc * 16;
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int64_t row = lmin(tw.n0 + (wave * LB + j) * 16 + dr, tw.N - 1);
    b_src[j] = tw.B + row * tw.ldk + tw.k0 / 2 + dc * 16;
  }
  // the same sources as 32-bit offsets from the tile's first row at the range's
  // first K byte (the host guarantees 256 rows of either operand span < 2^31 B);
  // every load addresses through them, so no 64-bit per-lane pointer stays live
  // across the K loop (held there, they spilled in the unaligned-scale variant:
  // ~90 MB of scratch traffic per grouped MoE launch)
  const uint8_t* a_base = tw.A + tw.m0 * tw.ldk + tw.k0 / 2;
  const uint8_t* b_base = tw.B + tw.n0 * tw.ldk + tw.k0 / 2;
  uint32_t a_off[LA], b_off[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j)
    a_off[j] = (uint32_t)(a_src[j] - a_base);
#pragma unroll
  for (int j = 0; j < LB; ++j)
    b_off[j] = (uint32_t)(b_src[j] - b_base);
  // scale group job of this wave: 64 rows (lane = row) of A (waves 0-3) or B
  const bool s_isA = wave < 4;
  const int s_r0 = (wave & 3) * 64;
  const uint8_t* s_src =
      s_isA ? tw.SA + lmin(tw.m0 + s_r0 + lane, tw.a_last) * tw.lds_a + tw.k0 / 32
            : tw.SB + lmin(tw.n0 + s_r0 + lane, tw.N - 1) * tw.lds_b + tw.k0 / 32;
  // UNAL: offset of the row's first scale byte in its aligned 16-byte piece
  const uint32_t s_sh = (uint32_t)(reinterpret_cast<uintptr_t>(s_src) & 15);
  const int64_t kc_blocks = tw.kc_blocks;

  auto issue = [&](int kt, auto S) {
    constexpr int P = decltype(S)::value;
    const int64_t kc = (int64_t)kt * 64;
    const int64_t coff = lmin(kc, lmax(kc_bytes - 16 - dc * 16, -dc * 16));
#pragma unroll
    for (int j = 0; j < LA; ++j)
      dma16(a_base + a_off[j] + coff, &ring[P].a.codes[((wave * LA + j) * 16) * 4]);
#pragma unroll
    for (int j = 0; j < LB; ++j)
      dma16(b_base + b_off[j] + coff, &ring[P].b.codes[((wave * LB + j) * 16) * 4]);
  };
  auto issue_scales = [&](int g) {
    ScaleGroupLds<BM, BN>& t = sg[g & 1];
    if constexpr (UNAL) {
      // group g's bytes [s_src + 16 g, + 16) lie in the pieces at p0 and p0 + 16;
      // byte s_src + 16 g is in the range (16 g < kc_blocks for every group the
      // kernel loads), and the second piece is read only if it holds one too
      const uint8_t* p0 = s_src - s_sh + (int64_t)g * 16;
      const uint8_t* p1 = 16 * g + 16 < kc_blocks + s_sh ? p0 + 16 : p0;
      dma16(p0, s_isA ? &t.a[s_r0] : &t.b[s_r0]);
      dma16(p1, s_isA ? &sgx.a[s_r0] : &sgx.b[s_r0]);
    } else {
      dma16(s_src + (int64_t)g * 16, s_isA ? &t.a[s_r0] : &t.b[s_r0]);
    }
  };
  // UNAL: this lane's row of group g (both pieces landed) shifted into place:
  // bytes [s_sh, s_sh + 16) of the 32-byte pair become the row's 16 bytes in sg
  auto align_group = [&](int g) {
    if constexpr (UNAL) {
      uint4* row = s_isA ? &sg[g & 1].a[s_r0 + lane] : &sg[g & 1].b[s_r0 + lane];
      const uint4 lo = *row;
      const uint4 hi = s_isA ? sgx.a[s_r0 + lane] : sgx.b[s_r0 + lane];
      const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      // shift by s_sh >> 2 dwords with bit selects (a select written as an
      // index would be lowered to a private-memory array), then by s_sh & 3 bytes
      const uint32_t m2 = 0u - ((s_sh >> 3) & 1), m1 = 0u - ((s_sh >> 2) & 1), r = s_sh & 3;
      uint32_t t[6], u[5];
#pragma unroll
      for (int i = 0; i < 6; ++i) t[i] = (w[i + 2] & m2) | (w[i] & ~m2);
#pragma unroll
      for (int i = 0; i < 5; ++i) u[i] = (t[i + 1] & m1) | (t[i] & ~m1);
      // v_alignbyte: ({u[i + 1], u[i]} >> 8 r) [31:0]
      *row = make_uint4(__builtin_amdgcn_alignbyte(u[1], u[0], r),
                        __builtin_amdgcn_alignbyte(u[2], u[1], r),
                        __builtin_amdgcn_alignbyte(u[3], u[2], r),
                        __builtin_amdgcn_alignbyte(u[4], u[3], r));
    }
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // fragments of the current step (both K-halves), the scale groups of the
  // current four steps and the current step's scale dwords
  uint4 fa[2][TM], fb[2][TN], ga[TM], gb[TN];
  uint32_t sa[TM], sb[TN];

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  auto barrier_lds = [&]() {  // this wave's LDS reads landed, then barrier
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // phase L(j), j % 4 == P: fragments and scales of step j, then the waits
  auto load_phase = [&](int kt, auto S, auto FULL) {
    constexpr int P = decltype(S)::value;
    constexpr bool F = decltype(FULL)::value;
    if (P == 0) {
      const ScaleGroupLds<BM, BN>& t = sg[(kt >> 2) & 1];
#pragma unroll
      for (int i = 0; i < TM; ++i) ga[i] = t.a[wm_off + i * 32 + lr];
#pragma unroll
      for (int i = 0; i < TN; ++i) gb[i] = t.b[wn_off + i * 32 + lr];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = 2 * h + lh;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm_off + i * 32 + lr;
        fa[h][i] = ring[P].a.codes[row * 4 + (kb ^ ((row >> 2) & 3))];
      }
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int row = wn_off + i * 32 + lr;
        fb[h][i] = ring[P].b.codes[row * 4 + (kb ^ ((row >> 2) & 3))];
      }
    }
    // this wave's share of step kt + 1 (issued in C(kt - 2), or by the
    // prologue) has landed, and with it the scale group issued before it;
    // vector-memory instructions issued after it: the loads of step kt + 2
    // (in C(kt - 1)) and the scale groups issued in C(kt - 2) after that
    // step's loads and in C(kt - 1) (one per four steps)
    if constexpr (F) {
      constexpr int W = UNAL ? kPpWaitFullUnal[P] : kPpWaitFull[P];
      static_assert(W == LC + ((P == 1 || P == 2) ? GL : 0), "schedule constants");
      wait_vmcnt<W>();
    } else {
      if (kt + 2 < KT) wait_vmcnt<kPpWaitNear>();
      else wait_vmcnt<0>();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = reinterpret_cast<const uint32_t*>(&ga[i])[P] >> (8 * lh);
#pragma unroll
    for (int i = 0; i < TN; ++i) sb[i] = reinterpret_cast<const uint32_t*>(&gb[i])[P] >> (8 * lh);
    if (!F && kt == KT - 1) {
      // 32-blocks past K in the last step: zero A's codes, neutral scales (127)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (2 * h + lh >= tail_kb) {
          const uint32_t keep = h ? 0x0000FFFFu : 0xFFFF0000u;
          const uint32_t neutral = h ? 0x007F0000u : 0x0000007Fu;
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            fa[h][i] = make_uint4(0, 0, 0, 0);
            sa[i] = (sa[i] & keep) | neutral;
          }
#pragma unroll
          for (int i = 0; i < TN; ++i) sb[i] = (sb[i] & keep) | neutral;
        }
      }
    }
    // the next group, read from sg in L(kt + 1), has landed with step kt + 1
    // (after the scale dwords are taken, so the group registers are free)
    if (P == 3 && (F || kt + 1 < KT)) align_group((kt >> 2) + 1);
    barrier_lds();
  };
  // MFMA i of a step: K-half i / 8, tile (a, b) = ((i % 8) / TM, i % TM)
  auto mfma_i = [&](auto I) {
    constexpr int i = decltype(I)::value;
    constexpr int h = i / (TM * TN), a = (i % (TM * TN)) / TM, b = i % TM;
    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        as_v8i(fb[h][a]), as_v8i(fa[h][b]), acc[a][b], kFmtFp4, kFmtFp4, h ? 2 : 0,
        (int)sb[a], h ? 2 : 0, (int)sa[b]);
  };
  // phase C(j): the 16 MFMAs of step j with this wave's loads of step j + 3
  // after MFMAs 0, 4, 8 and 12 and, every four steps, its scale-group load
  // after MFMA 14.  FULL steps load at a uniform K offset from SGPR bases; the
  // last steps clamp each lane's column into the row.
  auto compute_phase = [&](int kt, auto S, auto FULL) {
    constexpr int P = decltype(S)::value;
    constexpr bool F = decltype(FULL)::value;
    constexpr int S3 = (P + 3) % 4;
    const bool load = F || kt + 3 < KT;
    const int64_t kc = (int64_t)(kt + 3) * 64;
    const int64_t coff = lmin(kc, lmax(kc_bytes - 16 - dc * 16, -dc * 16));
    const uint8_t* ak = a_base + kc;
    const uint8_t* bk = b_base + kc;
    auto load_a = [&](int j) {
      if (F) dma16s(ak, a_off[j], &ring[S3].a.codes[((wave * LA + j) * 16) * 4]);
      else if (load) dma16(a_base + a_off[j] + coff, &ring[S3].a.codes[((wave * LA + j) * 16) * 4]);
    };
    auto load_b = [&](int j) {
      if (F) dma16s(bk, b_off[j], &ring[S3].b.codes[((wave * LB + j) * 16) * 4]);
      else if (load) dma16(b_base + b_off[j] + coff, &ring[S3].b.codes[((wave * LB + j) * 16) * 4]);
    };
    auto one = [&](auto I) {
      constexpr int i = decltype(I)::value;
      mfma_i(I);
      if constexpr (i % 4 == 0 || i == 14) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (i == 0 || i == 4) load_a(i / 4);
        if constexpr (i == 8 || i == 12) load_b(i / 4 - 2);
        if constexpr (i == 14) {
          if (P == 0 && (F || kt + 4 < KT)) issue_scales((kt >> 2) + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    static_assert(TM * TN * 2 == 16 && LA == 2 && LB == 2, "load placement");
    using std::integral_constant;
    one(integral_constant<int, 0>{});
    one(integral_constant<int, 1>{});
    one(integral_constant<int, 2>{});
    one(integral_constant<int, 3>{});
    one(integral_constant<int, 4>{});
    one(integral_constant<int, 5>{});
    one(integral_constant<int, 6>{});
    one(integral_constant<int, 7>{});
    one(integral_constant<int, 8>{});
    one(integral_constant<int, 9>{});
    one(integral_constant<int, 10>{});
    one(integral_constant<int, 11>{});
    one(integral_constant<int, 12>{});
    one(integral_constant<int, 13>{});
    one(integral_constant<int, 14>{});
    one(integral_constant<int, 15>{});
    barrier();
  };

  // prologue: scale group 0 and steps 0-2 issued; step 0 and the group landed
  if (0 < KT) issue_scales(0);
  if (0 < KT) issue(0, I0{});
  if (1 < KT) issue(1, I1{});
  if (2 < KT) issue(2, I2{});
  if (2 < KT) wait_vmcnt<kPpWaitFirst[2]>();
  else if (1 < KT) wait_vmcnt<kPpWaitFirst[1]>();
  else wait_vmcnt<kPpWaitFirst[0]>();
  if (0 < KT) align_group(0);
  barrier_lds();
  if (grp == 1) barrier();  // group 1 runs one phase behind group 0

  using Full = std::true_type;
  using Part = std::false_type;
  int kt = 0;
  for (; kt + 7 < KT; kt += 4) {
    load_phase(kt, I0{}, Full{});
    compute_phase(kt, I0{}, Full{});
    load_phase(kt + 1, I1{}, Full{});
    compute_phase(kt + 1, I1{}, Full{});
    load_phase(kt + 2, I2{}, Full{});
    compute_phase(kt + 2, I2{}, Full{});
    load_phase(kt + 3, I3{}, Full{});
    compute_phase(kt + 3, I3{}, Full{});
  }
  for (; kt < KT; kt += 4) {
    load_phase(kt, I0{}, Part{});
    compute_phase(kt, I0{}, Part{});
    if (kt + 1 < KT) {
      load_phase(kt + 1, I1{}, Part{});
      compute_phase(kt + 1, I1{}, Part{});
    }
    if (kt + 2 < KT) {
      load_phase(kt + 2, I2{}, Part{});
      compute_phase(kt + 2, I2{}, Part{});
    }
    if (kt + 3 < KT) {
      load_phase(kt + 3, I3{}, Part{});
      compute_phase(kt + 3, I3{}, Part{});
    }
  }
  if (grp == 0) barrier();  // both groups have now passed 2 KT + 2 barriers

  store_tile_impl<BM, BN, WM, WN, TM, TN, (int)sizeof(ring)>(acc, reinterpret_cast<char*>(ring),
                                                              tw);
}

// ---------------------------------------------------------------- host side
template <int BM, int BN, int WM, int WN, int SC, int STAGES = 4>
static int launch_gemm(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                       const int64_t* offs, int64_t groups, int64_t N, int64_t K, float alpha,
                       float* c, int64_t ldc, int64_t b_stride_codes, int64_t b_stride_scales,
                       int64_t lds_a, int64_t lds_b, GemmSplit sp, const GemmPlain* p1,
                       hipStream_t st) {
  // a dispatch holds at most 2^32 - 1 work-items (and the kernel counts tiles
  // in int): a larger launch is rejected
  constexpr int64_t kMaxWg = 0xFFFFFFFFll / (WM * WN * 64);
  int64_t t64 = 0;
  for (int64_t g = 0; g < groups; ++g) t64 += cdiv(offs[g + 1] - offs[g], BM) * cdiv(N, BN);
  const int64_t p1_tiles = p1 ? cdiv(p1->M, BM) * cdiv(p1->N, BN) : 0;
  if (t64 * sp.n + p1_tiles > kMaxWg) return MX_ERR_SHAPE;
  GemmGroups gg;
  gg.ngroups = (int)groups;
  gg.tiles_n = (int)cdiv(N, BN);
  gg.lds_a = lds_a;
  gg.lds_b = lds_b;
  gg.tile_start[0] = 0;
  for (int64_t g = 0; g < groups; ++g) {
    gg.row_off[g] = offs[g];
    const int64_t rows = offs[g + 1] - offs[g];
    gg.tile_start[g + 1] = gg.tile_start[g] + (int)(cdiv(rows, BM) * gg.tiles_n);
  }
  gg.row_off[groups] = offs[groups];
  const int total = gg.tile_start[groups] * sp.n;
  if constexpr (BM == 128) {  // paired launches take 128 x 128 tiles only
    if (p1) {
      GemmPlain q = *p1;
      q.tiles = (int)p1_tiles;
      q.tiles_n = (int)cdiv(q.N, BN);
      if (total + q.tiles == 0) return MX_OK;
      k_gemm_mx<BM, BN, WM, WN, 4, SC, true><<<dim3(total + q.tiles), dim3(WM * WN * 64), 0, st>>>(
          a, sa, b, sb, N, K, alpha, c, ldc, b_stride_codes, b_stride_scales, gg, sp, q);
      return launch_status();
    }
  } else {
    if (p1) return MX_ERR_SHAPE;
  }
  if (total == 0) return MX_OK;
  k_gemm_mx<BM, BN, WM, WN, STAGES, SC, false><<<dim3(total), dim3(WM * WN * 64), 0, st>>>(
      a, sa, b, sb, N, K, alpha, c, ldc, b_stride_codes, b_stride_scales, gg, sp, GemmPlain{});
  return launch_status();
}

// The ping-pong kernel for 256 x 256 tiles (no paired second product); unal:
// scale groups not 16-byte aligned.
template <bool UNAL>
static int launch_gemm_pp(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                          const uint8_t* sb, const int64_t* offs, int64_t groups, int64_t N,
                          int64_t K, float alpha, float* c, int64_t ldc, int64_t b_stride_codes,
                          int64_t b_stride_scales, int64_t lds_a, int64_t lds_b, GemmSplit sp,
                          hipStream_t st) {
  constexpr int64_t kMaxWg = 0xFFFFFFFFll / 512;
  int64_t t64 = 0;
  for (int64_t g = 0; g < groups; ++g) t64 += cdiv(offs[g + 1] - offs[g], 256) * cdiv(N, 256);
  if (t64 * sp.n > kMaxWg) return MX_ERR_SHAPE;
  GemmGroups gg;
  gg.ngroups = (int)groups;
  gg.tiles_n = (int)cdiv(N, 256);
  gg.lds_a = lds_a;
  gg.lds_b = lds_b;
  gg.tile_start[0] = 0;
  for (int64_t g = 0; g < groups; ++g) {
    gg.row_off[g] = offs[g];
    gg.tile_start[g + 1] = gg.tile_start[g] + (int)(cdiv(offs[g + 1] - offs[g], 256) * gg.tiles_n);
  }
  gg.row_off[groups] = offs[groups];
  const int total = gg.tile_start[groups] * sp.n;
  if (total == 0) return MX_OK;
  k_gemm_pp<UNAL><<<dim3(total), dim3(512), 0, st>>>(a, sa, b, sb, N, K, alpha, c, ldc,
                                                      b_stride_codes, b_stride_scales, gg, sp);
  return launch_status();
}

// Scale-load mode of one product: 16-byte groups of four steps, one dword per
// step, two 2-byte loads or bytes, by what the scale rows' pitch (lds_a,
// lds_b: at least K / 32, padding past K / 32 is never used) and alignment
// allow.  A group of four steps may run past K / 32 into a row's padding but
// not past its pitch, since the pitch is then a multiple of 16.
static int scale_mode(const uint8_t* sa, const uint8_t* sb, int64_t lds_a, int64_t lds_b,
                      int64_t b_stride_scales, const GemmSplit& sp) {
  auto al = [&](uintptr_t m) {
    return (reinterpret_cast<uintptr_t>(sa) & (m - 1)) == 0 &&
           (reinterpret_cast<uintptr_t>(sb) & (m - 1)) == 0 && b_stride_scales % (int64_t)m == 0 &&
           lds_a % (int64_t)m == 0 && lds_b % (int64_t)m == 0;
  };
  // scale rows of every split must start aligned as well (group mode reads 16
  // bytes of four steps, dword mode 4 bytes of one; every split starts at a
  // multiple of 128 K-values, i.e. 4 scale bytes)
  bool k512 = true, k128 = true;
  for (int s = 0; s < sp.n; ++s) {
    k512 = k512 && sp.kbeg[s] % 512 == 0;
    k128 = k128 && sp.kbeg[s] % 128 == 0;
  }
  if (al(16) && k512) return kScGroup;
  if (al(4) && k128) return kScDword;
  if (al(2) && k128) return kScShort;
  return kScByte;
}

// The mode both products of a paired launch can use (the modes, weakest last:
// group, dword, short, byte).
static int common_scale_mode(int a, int b) {
  auto rank = [](int m) { return m == kScGroup ? 0 : (m == kScDword ? 1 : (m == kScShort ? 2 : 3)); };
  return rank(a) >= rank(b) ? a : b;
}

// Large tiles when they still give every CU a few tiles, else smaller ones;
// a paired launch (p1) always takes 128 x 128 tiles.
static int gemm_launch(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                       const int64_t* offs, int64_t groups, int64_t N, int64_t K, float alpha,
                       float* c, int64_t ldc, int64_t b_stride_codes, int64_t b_stride_scales,
                       int64_t lds_a, int64_t lds_b, GemmSplit sp, hipStream_t st,
                       const GemmPlain* p1 = nullptr) {
  if (K > INT32_MAX) return MX_ERR_SHAPE;  // range lengths are 32-bit
  int64_t tiles256 = 0;
  for (int64_t g = 0; g < groups; ++g) tiles256 += cdiv(offs[g + 1] - offs[g], 256) * cdiv(N, 256);
  int sc = scale_mode(sa, sb, lds_a, lds_b, b_stride_scales, sp);
  if (p1) {
    GemmSplit one{};
    one.n = 1;
    sc = common_scale_mode(sc, scale_mode(p1->SA, p1->SB, p1->lds_a, p1->lds_b, 0, one));
  }
  const bool big = !p1 && tiles256 * sp.n >= 512;
#define MX_GEMM_ARGS a, sa, b, sb, offs, groups, N, K, alpha, c, ldc, b_stride_codes, b_stride_scales, lds_a, lds_b, sp, p1, st
  if (big) {
    // the ping-pong kernel (eight waves, two per SIMD, 128 x 64 per wave: one
    // wave's LDS waits and barrier overlap the other's MFMAs) takes scale rows in
    // 16-byte groups, shifted into place when they are not 16-byte aligned; it
    // addresses 256 rows of an operand with 32-bit offsets
    if (256 * (K / 2) < ((int64_t)1 << 31)) {
      if (sc == kScGroup)
        return launch_gemm_pp<false>(a, sa, b, sb, offs, groups, N, K, alpha, c, ldc,
                                     b_stride_codes, b_stride_scales, lds_a, lds_b, sp, st);
      return launch_gemm_pp<true>(a, sa, b, sb, offs, groups, N, K, alpha, c, ldc, b_stride_codes,
                                  b_stride_scales, lds_a, lds_b, sp, st);
    }
    // the four-wave kernel with per-step scale loads otherwise (eight waves would
    // spill in its K loop)
    if (sc == kScGroup) return launch_gemm<256, 256, 2, 4, kScGroup>(MX_GEMM_ARGS);
    if (sc == kScDword) return launch_gemm<256, 256, 2, 2, kScDword>(MX_GEMM_ARGS);
    if (sc == kScShort) return launch_gemm<256, 256, 2, 2, kScShort>(MX_GEMM_ARGS);
    return launch_gemm<256, 256, 2, 2, kScByte>(MX_GEMM_ARGS);
  }
  // at most three K-steps in every range: the short-contraction variant (three
  // stages, three workgroups per CU); group-mode scales need K % 512 == 0
  int64_t klen = 0;
  for (int s = 0; s < sp.n; ++s) klen = klen > sp.klen[s] ? klen : sp.klen[s];
  if (!p1 && klen <= 3 * 128 && sc != kScGroup) {
    if (sc == kScDword) return launch_gemm<128, 128, 2, 2, kScDword, 3>(MX_GEMM_ARGS);
    if (sc == kScShort) return launch_gemm<128, 128, 2, 2, kScShort, 3>(MX_GEMM_ARGS);
    return launch_gemm<128, 128, 2, 2, kScByte, 3>(MX_GEMM_ARGS);
  }
  if (sc == kScGroup) return launch_gemm<128, 128, 2, 2, kScGroup>(MX_GEMM_ARGS);
  if (sc == kScDword) return launch_gemm<128, 128, 2, 2, kScDword>(MX_GEMM_ARGS);
  if (sc == kScShort) return launch_gemm<128, 128, 2, 2, kScShort>(MX_GEMM_ARGS);
  return launch_gemm<128, 128, 2, 2, kScByte>(MX_GEMM_ARGS);
#undef MX_GEMM_ARGS
}

// C[m][n] = 0 for m < M, n < N (row pitch ldc): the product of an empty
// contraction, written without touching the operands.
__global__ __launch_bounds__(256) void k_zero_c(float* __restrict__ c, int64_t M, int64_t N,
                                                int64_t ldc) {
  const int64_t n4 = (N + 3) / 4, total = M * n4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / n4, q = (i % n4) * 4;
    float* p = c + r * ldc + q;
    if (q + 3 < N) {
      store_c4(p, make_float4(0.f, 0.f, 0.f, 0.f), true);
    } else {
      for (int64_t j = q; j < N; ++j) c[r * ldc + j] = 0.f;
    }
  }
}

int zero_c_impl(float* c, int64_t M, int64_t N, int64_t ldc, hipStream_t st) {
  if (M == 0 || N == 0) return MX_OK;
  const int64_t n4 = M * ((N + 3) / 4);
  k_zero_c<<<dim3((unsigned)hmin(cdiv(n4, 256), 4096)), dim3(256), 0, st>>>(c, M, N, ldc);
  return launch_status();
}

// lds_a, lds_b: bytes between the scale rows of A and of B (K / 32 when
// packed; the backward layers pad their own operands' rows to 16 bytes).
// K == 0: C = 0 by a fill kernel; the operands are not read.
int gemm_impl(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
              const int64_t* offs, int64_t groups, int64_t N, int64_t K, float alpha, float* c,
              int64_t ldc, int64_t b_stride_codes, int64_t b_stride_scales, int64_t lds_a,
              int64_t lds_b, hipStream_t st) {
  if (K == 0) return zero_c_impl(c, offs[groups], N, ldc, st);
  GemmSplit one{};
  one.n = 1;
  one.stream_c = 1;
  one.kbeg[0] = 0;
  one.kbeg[1] = K;
  contiguous_ranges(one);
  return gemm_launch(a, sa, b, sb, offs, groups, N, K, alpha, c, ldc, b_stride_codes,
                     b_stride_scales, lds_a, lds_b, one, st);
}

// ---------------------------------------------------------------- split-K
// When an M x N output gives the CUs too few 128 x 128 tiles, the contraction
// is cut into chunks (multiples of 512, at least 1024 long) whose partial sums
// go to a caller workspace and are added in split order by a second kernel,
// so the result does not depend on timing.
SplitPlan gemm_split_plan(int64_t M, int64_t N, int64_t K) {
  SplitPlan p = {1, K};
  const int64_t tiles128 = cdiv(M, 128) * cdiv(N, 128);
  if (cdiv(M, 256) * cdiv(N, 256) >= 512 || tiles128 >= 256 || K < 2048) return p;
  int64_t n = hmin(hmin(cdiv(512, tiles128), K / 1024), 64);
  if (n < 2) return p;
  const int64_t chunk = cdiv(cdiv(K, n), 512) * 512;
  n = cdiv(K, chunk);
  if (n < 2) return p;
  p.n = (int)n;
  p.kchunk = chunk;
  return p;
}

__global__ __launch_bounds__(256) void k_splitk_sum(const float4* __restrict__ part, int n,
                                                    int64_t rows, int64_t cols4, float alpha,
                                                    float* __restrict__ c, int64_t ldc) {
  const int64_t total = rows * cols4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 s = part[i];
    for (int k = 1; k < n; ++k) {
      const float4 v = part[k * total + i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const int64_t r = i / cols4, q = i % cols4;
    store_c4(c + r * ldc + q * 4, make_float4(s.x * alpha, s.y * alpha, s.z * alpha, s.w * alpha),
             true);
  }
}

// C[M][N] (ldc) = alpha * A . B^T with the plan's splits; part: plan.n * M * N
// floats of workspace (16-byte aligned); N % 4 == 0.
int gemm_split_impl(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                    int64_t M, int64_t N, int64_t K, float alpha, float* c, int64_t ldc,
                    SplitPlan plan, float* part, int64_t lds_a, int64_t lds_b, hipStream_t st) {
  const int64_t offs[2] = {0, M};
  if (plan.n <= 1)
    return gemm_impl(a, sa, b, sb, offs, 1, N, K, alpha, c, ldc, 0, 0, lds_a, lds_b, st);
  GemmSplit sp{};
  sp.n = plan.n;
  sp.stream_c = 0;  // partial sums, read back by k_splitk_sum
  sp.c_stride = M * N;
  for (int i = 0; i <= plan.n; ++i) sp.kbeg[i] = hmin((int64_t)i * plan.kchunk, K);
  contiguous_ranges(sp);
  int s = gemm_launch(a, sa, b, sb, offs, 1, N, K, 1.0f, part, N, 0, 0, lds_a, lds_b, sp, st);
  if (s != MX_OK) return s;
  const int64_t n4 = M * (N / 4);
  k_splitk_sum<<<dim3((unsigned)hmin(cdiv(n4, 256), 4096)), dim3(256), 0, st>>>(
      reinterpret_cast<const float4*>(part), plan.n, M, N / 4, alpha, c, ldc);
  return launch_status();
}

// Whether two products are small enough to share a launch: neither would take
// 256 x 256 tiles, and the second needs no split.
bool gemm_pairable(int64_t M0, int64_t N0, SplitPlan plan0, int64_t M1, int64_t N1,
                   SplitPlan plan1) {
  return plan1.n == 1 && cdiv(M0, 256) * cdiv(N0, 256) * plan0.n < 512 &&
         cdiv(M1, 256) * cdiv(N1, 256) < 512;
}

// Two products in one launch: C0 [M0][N0] = alpha0 A0 . B0^T with plan0's
// splits (partial sums in part0, added afterwards) and the plain C1 [M1][N1] =
// alpha1 A1 . B1^T.  The first product's workgroups are dispatched first, so it
// should be the one with the longer contraction per workgroup.
int gemm_pair_impl(const uint8_t* a0, const uint8_t* sa0, const uint8_t* b0, const uint8_t* sb0,
                   int64_t M0, int64_t N0, int64_t K0, float alpha0, float* c0, int64_t ldc0,
                   SplitPlan plan0, float* part0, int64_t lds_a0, int64_t lds_b0,
                   const uint8_t* a1, const uint8_t* sa1, const uint8_t* b1, const uint8_t* sb1,
                   int64_t M1, int64_t N1, int64_t K1, float alpha1, float* c1, int64_t ldc1,
                   int64_t lds_a1, int64_t lds_b1, hipStream_t st) {
  const int64_t offs[2] = {0, M0};
  const GemmPlain p1{a1, sa1, b1, sb1, M1, N1, K1, alpha1, c1, ldc1, lds_a1, lds_b1, 0, 0};
  GemmSplit sp{};
  if (plan0.n <= 1) {
    sp.n = 1;
    sp.stream_c = 1;
    sp.kbeg[0] = 0;
    sp.kbeg[1] = K0;
    contiguous_ranges(sp);
    return gemm_launch(a0, sa0, b0, sb0, offs, 1, N0, K0, alpha0, c0, ldc0, 0, 0, lds_a0, lds_b0,
                       sp, st, &p1);
  }
  sp.n = plan0.n;
  sp.stream_c = 0;  // partial sums, read back by k_splitk_sum
  sp.c_stride = M0 * N0;
  for (int i = 0; i <= plan0.n; ++i) sp.kbeg[i] = hmin((int64_t)i * plan0.kchunk, K0);
  contiguous_ranges(sp);
  int s = gemm_launch(a0, sa0, b0, sb0, offs, 1, N0, K0, 1.0f, part0, N0, 0, 0, lds_a0, lds_b0,
                      sp, st, &p1);
  if (s != MX_OK) return s;
  const int64_t n4 = M0 * (N0 / 4);
  k_splitk_sum<<<dim3((unsigned)hmin(cdiv(n4, 256), 4096)), dim3(256), 0, st>>>(
      reinterpret_cast<const float4*>(part0), plan0.n, M0, N0 / 4, alpha0, c0, ldc0);
  return launch_status();
}

// C_s [M][N] = alpha * A[:, kbeg[s]:kbeg[s] + klen[s]] . B[:, same]^T for s < n,
// written at c + s * M * N (A [M, K], B [N, K] packed along K; each kbeg a
// multiple of 128, each klen a multiple of 32, klen null: the ranges end where
// the next begins; an empty range writes zeros).
int gemm_ranges_impl(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                     int64_t M, int64_t N, int64_t K, const int64_t* kbeg, const int64_t* klen,
                     int n, float alpha, float* c, int64_t lds_a, int64_t lds_b, hipStream_t st) {
  GemmSplit sp{};
  sp.n = n;
  sp.stream_c = 1;
  sp.c_stride = M * N;
  for (int i = 0; i <= n; ++i) sp.kbeg[i] = kbeg[i];
  contiguous_ranges(sp);
  if (klen)
    for (int i = 0; i < n; ++i) sp.klen[i] = (int32_t)klen[i];
  const int64_t offs[2] = {0, M};
  return gemm_launch(a, sa, b, sb, offs, 1, N, K, alpha, c, N, 0, 0, lds_a, lds_b, sp, st);
}

}  // namespace mx

using namespace mx;

extern "C" int mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                       const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float alpha,
                       float* c, int64_t ldc, void* stream) {
  MX_REQUIRE(M >= 0 && N >= 0 && K >= 0 && K % 32 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(ldc >= N && ldc % 4 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31 && K <= INT32_MAX, MX_ERR_SHAPE);
  if (M == 0 || N == 0) return MX_OK;
  MX_REQUIRE(c, MX_ERR_NULL);
  if (K > 0) MX_REQUIRE(a_codes && a_scales && b_codes && b_scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(c), MX_ERR_ALIGN);
  if (K > 0) MX_REQUIRE(aligned16(a_codes) && aligned16(b_codes), MX_ERR_ALIGN);
  const int64_t offs[2] = {0, M};
  return gemm_impl(a_codes, a_scales, b_codes, b_scales, offs, 1, N, K, alpha, c, ldc, 0, 0,
                   K / 32, K / 32, as_stream(stream));
}

extern "C" int mx_gemm_ld(const uint8_t* a_codes, const uint8_t* a_scales, int64_t a_scale_ld,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t b_scale_ld,
                          int64_t M, int64_t N, int64_t K, float alpha, float* c, int64_t ldc,
                          void* stream) {
  MX_REQUIRE(M >= 0 && N >= 0 && K >= 0 && K % 32 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(ldc >= N && ldc % 4 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(a_scale_ld >= K / 32 && b_scale_ld >= K / 32, MX_ERR_SHAPE);
  MX_REQUIRE(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31 && K <= INT32_MAX, MX_ERR_SHAPE);
  if (M == 0 || N == 0) return MX_OK;
  MX_REQUIRE(c, MX_ERR_NULL);
  if (K > 0) MX_REQUIRE(a_codes && a_scales && b_codes && b_scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(c), MX_ERR_ALIGN);
  if (K > 0) MX_REQUIRE(aligned16(a_codes) && aligned16(b_codes), MX_ERR_ALIGN);
  const int64_t offs[2] = {0, M};
  return gemm_impl(a_codes, a_scales, b_codes, b_scales, offs, 1, N, K, alpha, c, ldc, 0, 0,
                   a_scale_ld, b_scale_ld, as_stream(stream));
}

extern "C" int mx_gemm_grouped_ld(const uint8_t* a_codes, const uint8_t* a_scales,
                                  int64_t a_scale_ld, const uint8_t* b_codes,
                                  const uint8_t* b_scales, int64_t b_scale_ld,
                                  const int64_t* offs, int64_t groups, int64_t N, int64_t K,
                                  float alpha, float* c, void* stream) {
  MX_REQUIRE(offs, MX_ERR_NULL);
  MX_REQUIRE(groups >= 1 && groups <= MX_MAX_GROUPS, MX_ERR_SHAPE);
  MX_REQUIRE(N >= 0 && K >= 0 && K % 32 == 0 && N % 4 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(a_scale_ld >= K / 32 && b_scale_ld >= K / 32, MX_ERR_SHAPE);
  MX_REQUIRE(offs[0] == 0, MX_ERR_SHAPE);
  for (int64_t g = 0; g < groups; ++g) MX_REQUIRE(offs[g + 1] >= offs[g], MX_ERR_SHAPE);
  const int64_t M = offs[groups];
  MX_REQUIRE(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31 && K <= INT32_MAX, MX_ERR_SHAPE);
  if (M == 0 || N == 0) return MX_OK;
  MX_REQUIRE(c, MX_ERR_NULL);
  if (K > 0) MX_REQUIRE(a_codes && a_scales && b_codes && b_scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(c), MX_ERR_ALIGN);
  if (K > 0) MX_REQUIRE(aligned16(a_codes) && aligned16(b_codes), MX_ERR_ALIGN);
  return gemm_impl(a_codes, a_scales, b_codes, b_scales, offs, groups, N, K, alpha, c, N,
                   N * K / 2, N * b_scale_ld, a_scale_ld, b_scale_ld, as_stream(stream));
}

extern "C" int mx_gemm_grouped(const uint8_t* a_codes, const uint8_t* a_scales,
                               const uint8_t* b_codes, const uint8_t* b_scales,
                               const int64_t* offs, int64_t groups, int64_t N, int64_t K,
                               float alpha, float* c, void* stream) {
  MX_REQUIRE(offs, MX_ERR_NULL);
  MX_REQUIRE(groups >= 1 && groups <= MX_MAX_GROUPS, MX_ERR_SHAPE);
  MX_REQUIRE(N >= 0 && K >= 0 && K % 32 == 0 && N % 4 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(offs[0] == 0, MX_ERR_SHAPE);
  for (int64_t g = 0; g < groups; ++g) MX_REQUIRE(offs[g + 1] >= offs[g], MX_ERR_SHAPE);
  const int64_t M = offs[groups];
  MX_REQUIRE(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31 && K <= INT32_MAX, MX_ERR_SHAPE);
  if (M == 0 || N == 0) return MX_OK;
  MX_REQUIRE(c, MX_ERR_NULL);
  if (K > 0) MX_REQUIRE(a_codes && a_scales && b_codes && b_scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(c), MX_ERR_ALIGN);
  if (K > 0) MX_REQUIRE(aligned16(a_codes) && aligned16(b_codes), MX_ERR_ALIGN);
  return gemm_impl(a_codes, a_scales, b_codes, b_scales, offs, groups, N, K, alpha, c, N,
                   N * K / 2, N * K / 32, K / 32, K / 32, as_stream(stream));
}
