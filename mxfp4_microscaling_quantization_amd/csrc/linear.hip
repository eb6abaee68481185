// Quantized linear layer: forward and backward compositions of the quantizer
// and GEMM kernels ("Oscillation-Reduced MXFP4 Training for Vision
// Transformers", rebuttal, Question 2):
//   forward   Y  = Q_D^(1)(X) . Q_D^(2)(W)^T             (1x32 RNE along K)
//   backward  dX = Q_S^(3)(dY) . Q_S^(4)(Q_D^(2)(W))     (contraction over N)
//             dW = Q_S^(5)(dY)^T . Q_S^(6)(Q_D^(1)(X))   (contraction over M)
// Q^(4) and Q^(6) are the double quantizations that give the 32x1 group shape
// the backward products need; quantizer q draws its stochastic rounding from
// seed + q.  A backward product whose output has too few tiles for the chip
// (a short, wide contraction such as dW of a ViT MLP) is split along its
// contraction into the workspace.  All launches go to the caller's stream in
// order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>

#include "mx_host.h"

namespace mx {
int quantize_dual_impl(const void* x, int dtype, int64_t rows, int64_t cols, int round,
                       uint64_t seed_row, uint64_t seed_col, int had, uint32_t mask,
                       uint8_t* codes_row, uint8_t* scales_row, uint8_t* codes_col,
                       uint8_t* scales_col, hipStream_t st, int64_t sp_row, int64_t sp_col);
int quantize_rows2_impl(const void* x0, int64_t rows0, int64_t cols0, uint8_t* codes0,
                        uint8_t* scales0, uint64_t seed0, const void* x1, int64_t rows1,
                        int64_t cols1, uint8_t* codes1, uint8_t* scales1, uint64_t seed1,
                        int dtype, int round, int had, uint32_t mask, hipStream_t st);
int requantize_pair_impl(const uint8_t* codes_in0, const uint8_t* scales_in0, int64_t rows0,
                         const uint8_t* codes_in1, const uint8_t* scales_in1, int64_t rows1,
                         int64_t cols, int round, uint64_t seed0, uint64_t seed1,
                         uint8_t* codes0, uint8_t* scales0, uint8_t* codes1, uint8_t* scales1,
                         hipStream_t st, int64_t s_pitch0, int64_t s_pitch1);
int requantize_rht_pair_impl(const uint8_t* codes_in0, const uint8_t* scales_in0, int64_t rows0,
                             const uint8_t* codes_in1, const uint8_t* scales_in1, int64_t rows1,
                             int64_t cols, int round, uint64_t seed0, uint64_t seed1,
                             uint32_t mask, uint8_t* codes0, uint8_t* scales0, uint8_t* codes1,
                             uint8_t* scales1, hipStream_t st);
int zero_c_impl(float* c, int64_t M, int64_t N, int64_t ldc, hipStream_t st);
int gemm_impl(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
              const int64_t* offs, int64_t groups, int64_t N, int64_t K, float alpha, float* c,
              int64_t ldc, int64_t b_stride_codes, int64_t b_stride_scales, int64_t lds_a,
              int64_t lds_b, hipStream_t st);
SplitPlan gemm_split_plan(int64_t M, int64_t N, int64_t K);
int gemm_split_impl(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                    int64_t M, int64_t N, int64_t K, float alpha, float* c, int64_t ldc,
                    SplitPlan plan, float* part, int64_t lds_a, int64_t lds_b, hipStream_t st);
bool gemm_pairable(int64_t M0, int64_t N0, SplitPlan plan0, int64_t M1, int64_t N1,
                   SplitPlan plan1);

int gemm_pair_impl(const uint8_t* a0, const uint8_t* sa0, const uint8_t* b0, const uint8_t* sb0,
                   int64_t M0, int64_t N0, int64_t K0, float alpha0, float* c0, int64_t ldc0,
                   SplitPlan plan0, float* part0, int64_t lds_a0, int64_t lds_b0,
                   const uint8_t* a1, const uint8_t* sa1, const uint8_t* b1, const uint8_t* sb1,
                   int64_t M1, int64_t N1, int64_t K1, float alpha1, float* c1, int64_t ldc1,
                   int64_t lds_a1, int64_t lds_b1, hipStream_t st);
int gemm_ranges_impl(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                     int64_t M, int64_t N, int64_t K, const int64_t* kbeg, const int64_t* klen,
                     int n, float alpha, float* c, int64_t lds_a, int64_t lds_b, hipStream_t st);
int requantize_batched_impl(const uint8_t* codes_in, const uint8_t* scales_in, int64_t batch,
                            int64_t rows, int64_t cols, int round, uint64_t seed, uint8_t* codes,
                            uint8_t* scales, hipStream_t st, int64_t s_pitch);
int quantize_dual_segments_impl(const void* x, int dtype, int64_t rows, int64_t cols,
                                const int64_t* offs, int64_t groups, int round, uint64_t seed_row,
                                uint64_t seed_col, uint8_t* codes_row, uint8_t* scales_row,
                                uint8_t* codes_col, uint8_t* scales_col, hipStream_t st,
                                int64_t sp_row, int64_t sp_col, int64_t pad);
int requantize_segments_impl(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                             int64_t cols, const int64_t* offs, int64_t groups, int round,
                             uint64_t seed, uint8_t* codes, uint8_t* scales, hipStream_t st,
                             int64_t s_pitch, int64_t pad);
int64_t segments_padded_rows(const int64_t* offs, int64_t groups, int64_t pad);
void segments_padded_offsets(const int64_t* offs, int64_t groups, int64_t* out, int64_t pad);

static size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

// Finish time of list scheduling n0 jobs of length a, then n1 of length b, on
// `slots` machines (every job starts on the machine that frees first).
static double list_makespan(int64_t n0, double a, int64_t n1, double b, int64_t slots) {
  std::map<double, int64_t> free_at;  // finish time -> machines free from then on
  free_at[0.0] = slots;
  double end = 0.0;
  auto run = [&](int64_t n, double len) {
    while (n > 0) {
      auto it = free_at.begin();
      const double t = it->first;
      const int64_t k = hmin(it->second, n);
      n -= k;
      if (k == it->second) free_at.erase(it);
      else it->second -= k;
      free_at[t + len] += k;
      end = t + len > end ? t + len : end;
    }
  };
  run(n0, a);
  run(n1, b);
  return end;
}

// The split of the first product of a paired launch (C0 [M0][N0], contraction
// K0, at most most.n chunks: the workspace holds that many partial sums) that
// finishes the launch and the pass adding its partial sums soonest, next to the
// plain second product (C1 [M1][N1], contraction K1).  Both take 128 x 128
// tiles, two workgroups per CU; a workgroup costs a fixed kWgSteps plus one per
// K-step, dispatched first product first; the partial-sum pass costs
// kSumStepsPerMB per MB of partial sums read plus kSumSteps.  (Constants from
// the DeiT-S fc1 backward: ~0.5 us per K-step, ~3 us per workgroup outside its
// K loop, ~4 TB/s for the pass.)  Chunks are multiples of 512 K-values.
static SplitPlan gemm_paired_split_plan(int64_t M0, int64_t N0, int64_t K0, SplitPlan most, int64_t M1,
                                 int64_t N1, int64_t K1) {
  constexpr double kWgSteps = 6.0, kSumSteps = 4.0, kSumStepsPerMB = 0.5;
  const int64_t slots = 2 * (int64_t)device_cu_count();
  const int64_t t0 = cdiv(M0, 128) * cdiv(N0, 128), t1 = cdiv(M1, 128) * cdiv(N1, 128);
  const double b = (double)cdiv(K1, 128) + kWgSteps;
  const double mb = (double)M0 * N0 * 4 / 1e6;
  SplitPlan best = {1, K0};
  double best_cost = list_makespan(t0, (double)cdiv(K0, 128) + kWgSteps, t1, b, slots);
  for (int n = 2; n <= most.n; ++n) {
    const int64_t chunk = cdiv(cdiv(K0, n), 512) * 512;
    if (cdiv(K0, chunk) != n) continue;  // the same split as a smaller n
    const double cost = list_makespan(t0 * n, (double)cdiv(chunk, 128) + kWgSteps, t1, b, slots) +
                        kSumSteps + kSumStepsPerMB * mb * n;
    if (cost < best_cost) {
      best_cost = cost;
      best = SplitPlan{n, chunk};
    }
  }
  return best;
}


// Scale rows of the backward operands in the workspace are padded to a
// multiple of 16 bytes, so every product can load four steps' scales of a row
// with one 16-byte access (the padding is never read as data).
static int64_t pad16(int64_t v) { return (v + 15) / 16 * 16; }

// Workspace layout: four packed operands, each codes then scales (scale rows
// p3..p6 bytes apart), then the split-K partial sums of the dX / dW products
// when they are split (shared: the two products run one after the other, and a
// launch that pairs them splits only dW), all 256-byte aligned.
struct BwdLayout {
  size_t q3c, q3s, q4c, q4s, q5c, q5s, q6c, q6s, part, total;
  int64_t p3, p4, p5, p6;
  SplitPlan dx, dw;
};

static BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K) {
  BwdLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round256(bytes);
    return at;
  };
  L.p3 = L.p4 = pad16(N / 32);
  L.p5 = L.p6 = pad16(M / 32);
  L.q3c = take((size_t)M * N / 2);  L.q3s = take((size_t)(M * L.p3));   // dY rows   [M][N]
  L.q4c = take((size_t)K * N / 2);  L.q4s = take((size_t)(K * L.p4));   // W^T blocks [K][N]
  L.q5c = take((size_t)N * M / 2);  L.q5s = take((size_t)(N * L.p5));   // dY^T      [N][M]
  L.q6c = take((size_t)K * M / 2);  L.q6s = take((size_t)(K * L.p6));   // X^T blocks [K][M]
  L.dx = gemm_split_plan(M, K, N);   // dX [M][K], contraction over N
  L.dw = gemm_split_plan(N, K, M);   // dW [N][K], contraction over M
  const size_t px = L.dx.n > 1 ? (size_t)L.dx.n * M * K * 4 : 0;
  const size_t pw = L.dw.n > 1 ? (size_t)L.dw.n * N * K * 4 : 0;
  L.part = take(px > pw ? px : pw);
  L.total = o;
  return L;
}

// Grouped (mixture-of-experts) backward workspace: Q3 [R][N], the experts'
// Q4 [E][K][N], Q5 [N][P] and Q6 [K][P] packed, P = the padded token axis;
// scale rows p3..p6 bytes apart.  Each expert's token segment starts at a
// multiple of 512 positions of P, so its dW product loads the scales of four
// K-steps at once (16 bytes per row); the positions past the segment's rows
// rounded up to the quantizers' tile height are never written, and the product
// stops at its rows rounded up to 32.
constexpr int64_t kExpertSegPad = 512;

struct GroupedLayout {
  size_t q3c, q3s, q4c, q4s, q5c, q5s, q6c, q6s, total;
  int64_t P, p3, p4, p5, p6;
};

static GroupedLayout grouped_layout(const int64_t* offs, int64_t E, int64_t N, int64_t K) {
  GroupedLayout L;
  const int64_t R = offs[E];
  L.P = segments_padded_rows(offs, E, kExpertSegPad);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round256(bytes);
    return at;
  };
  L.p3 = L.p4 = pad16(N / 32);
  L.p5 = L.p6 = pad16(L.P / 32);
  L.q3c = take((size_t)R * N / 2);      L.q3s = take((size_t)(R * L.p3));
  L.q4c = take((size_t)E * K * N / 2);  L.q4s = take((size_t)(E * K * L.p4));
  L.q5c = take((size_t)N * L.P / 2);    L.q5s = take((size_t)(N * L.p5));
  L.q6c = take((size_t)K * L.P / 2);    L.q6s = take((size_t)(K * L.p6));
  L.total = o;
  return L;
}

static bool valid_offsets(const int64_t* offs, int64_t groups) {
  if (!offs || groups < 1 || groups > MX_MAX_GROUPS || offs[0] != 0) return false;
  for (int64_t g = 0; g < groups; ++g)
    if (offs[g + 1] < offs[g]) return false;
  return true;
}

// Two rotated operands carry a factor 32 (H H^T = 32 I): the product takes 2^-5.
constexpr float kHadamardAlpha = 0.03125f;

static int linear_fwd_impl(const void* x, const void* w, int dtype, int64_t M, int64_t N,
                           int64_t K, int had, uint32_t mask, float* y, uint8_t* xq_codes,
                           uint8_t* xq_scales, uint8_t* wq_codes, uint8_t* wq_scales,
                           hipStream_t st) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(M >= 0 && N >= 0 && K >= 0, MX_ERR_SHAPE);
  MX_REQUIRE(M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX, MX_ERR_SHAPE);  // GEMM bounds
  MX_REQUIRE(M % 32 == 0 && N % 32 == 0 && K % 32 == 0, MX_ERR_SHAPE);
  if (M == 0 || N == 0) return MX_OK;
  if (K == 0) {  // Y = 0; the packed operands are empty
    MX_REQUIRE(y, MX_ERR_NULL);
    MX_REQUIRE(aligned16(y), MX_ERR_ALIGN);
    return zero_c_impl(y, M, N, N, st);
  }
  MX_REQUIRE(x && w && y && xq_codes && xq_scales && wq_codes && wq_scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(x) && aligned16(w) && aligned16(y) && aligned16(xq_codes) &&
                 aligned16(wq_codes), MX_ERR_ALIGN);
  // Q_D(X) and Q_D(W) (1x32 along K, nearest) in one launch
  int s = quantize_rows2_impl(x, M, K, xq_codes, xq_scales, 0, w, N, K, wq_codes, wq_scales, 0,
                              dtype, MX_RNE, had, mask, st);
  if (s != MX_OK) return s;
  const int64_t offs[2] = {0, M};
  return gemm_impl(xq_codes, xq_scales, wq_codes, wq_scales, offs, 1, N, K,
                   had ? kHadamardAlpha : 1.0f, y, N, 0, 0, K / 32, K / 32, st);
}

static int linear_bwd_impl(const void* dy, int dtype, int64_t M, int64_t N, int64_t K,
                           const uint8_t* xq_codes, const uint8_t* xq_scales,
                           const uint8_t* wq_codes, const uint8_t* wq_scales, uint64_t seed,
                           int had, uint32_t mask, float* dx, float* dw, void* workspace,
                           size_t workspace_bytes, hipStream_t st) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(M >= 0 && N >= 0 && K >= 0, MX_ERR_SHAPE);
  MX_REQUIRE(M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX, MX_ERR_SHAPE);  // GEMM bounds
  MX_REQUIRE(M % 32 == 0 && N % 32 == 0 && K % 32 == 0, MX_ERR_SHAPE);
  if (K == 0) return MX_OK;  // dX [M][0] and dW [N][0] are empty
  if (M == 0 || N == 0) {
    // an empty contraction: dX = 0 (over N == 0) and dW = 0 (over M == 0)
    if (M > 0) MX_REQUIRE(dx && aligned16(dx), dx ? MX_ERR_ALIGN : MX_ERR_NULL);
    if (N > 0) MX_REQUIRE(dw && aligned16(dw), dw ? MX_ERR_ALIGN : MX_ERR_NULL);
    int s = zero_c_impl(dx, M, K, K, st);
    if (s != MX_OK) return s;
    return zero_c_impl(dw, N, K, K, st);
  }
  MX_REQUIRE(dy && xq_codes && xq_scales && wq_codes && wq_scales && dx && dw, MX_ERR_NULL);
  MX_REQUIRE(aligned16(dy) && aligned16(xq_codes) && aligned16(wq_codes) && aligned16(dx) &&
                 aligned16(dw), MX_ERR_ALIGN);
  const BwdLayout L = bwd_layout(M, N, K);
  MX_REQUIRE(workspace && workspace_bytes >= L.total, MX_ERR_WORKSPACE);
  MX_REQUIRE(aligned16(workspace), MX_ERR_ALIGN);
  uint8_t* ws = static_cast<uint8_t*>(workspace);

  // scale pitches of Q3..Q6: padded, except that the rotated kernels write
  // packed rows (into the same, larger, buffers)
  const int64_t p3 = had ? N / 32 : L.p3, p4 = had ? N / 32 : L.p4;
  const int64_t p5 = had ? M / 32 : L.p5, p6 = had ? M / 32 : L.p6;
  int s = quantize_dual_impl(dy, dtype, M, N, MX_SR, seed + 3, seed + 5, had, mask, ws + L.q3c,
                             ws + L.q3s, ws + L.q5c, ws + L.q5s, st, p3, p5);
  if (s != MX_OK) return s;
  if (had) {  // the rotated Q4 and Q6 in one launch
    s = requantize_rht_pair_impl(wq_codes, wq_scales, N, xq_codes, xq_scales, M, K, MX_SR,
                                 seed + 4, seed + 6, mask, ws + L.q4c, ws + L.q4s, ws + L.q6c,
                                 ws + L.q6s, st);
  } else {  // Q4 = Q_S(Q_D(W)) and Q6 = Q_S(Q_D(X)) in one launch
    s = requantize_pair_impl(wq_codes, wq_scales, N, xq_codes, xq_scales, M, K, MX_SR, seed + 4,
                             seed + 6, ws + L.q4c, ws + L.q4s, ws + L.q6c, ws + L.q6s, st, p4, p6);
  }
  if (s != MX_OK) return s;
  const float alpha = had ? kHadamardAlpha : 1.0f;
  float* part = reinterpret_cast<float*>(ws + L.part);
  if (gemm_pairable(N, K, L.dw, M, K, L.dx)) {  // small products: dW and dX in one launch
    // dW's split balanced against dX in the shared launch (at most the workspace's
    // partial sums)
    const SplitPlan pw = gemm_paired_split_plan(N, K, M, L.dw, M, K, N);
    return gemm_pair_impl(ws + L.q5c, ws + L.q5s, ws + L.q6c, ws + L.q6s, N, K, M, alpha, dw, K,
                          pw, part, p5, p6, ws + L.q3c, ws + L.q3s, ws + L.q4c, ws + L.q4s, M,
                          K, N, alpha, dx, K, p3, p4, st);
  }
  s = gemm_split_impl(ws + L.q3c, ws + L.q3s, ws + L.q4c, ws + L.q4s, M, K, N, alpha, dx, K, L.dx,
                      part, p3, p4, st);
  if (s != MX_OK) return s;
  return gemm_split_impl(ws + L.q5c, ws + L.q5s, ws + L.q6c, ws + L.q6s, N, K, M, alpha, dw, K,
                         L.dw, part, p5, p6, st);
}

// ---------------------------------------------------------------- no-allocation backward
// Workspace of mx_linear_bwd_noalloc: one file-scope device array, present on
// every GPU the library runs on from module load to process end.  Its name is a
// host-side stand-in in host code: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (nullptr and an error status
// when the runtime cannot give it).
static int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MX_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MX_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MX_OK;
}

}  // namespace mx

using namespace mx;

extern "C" size_t mx_linear_bwd_noalloc_max_workspace(void) { return kScratchBytes; }

extern "C" int mx_linear_bwd_noalloc(const void* dy, int dtype, int64_t M, int64_t N, int64_t K,
                                     const uint8_t* xq_codes, const uint8_t* xq_scales,
                                     const uint8_t* wq_codes, const uint8_t* wq_scales,
                                     uint64_t seed, float* dx, float* dw, void* stream) {
  // sizes first, so an oversized layer is rejected before any runtime call
  MX_REQUIRE(M >= 0 && N >= 0 && K >= 0, MX_ERR_SHAPE);
  MX_REQUIRE(M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX, MX_ERR_SHAPE);
  MX_REQUIRE(M % 32 == 0 && N % 32 == 0 && K % 32 == 0, MX_ERR_SHAPE);
  const size_t need = bwd_layout(M, N, K).total;
  MX_REQUIRE(need <= kScratchBytes, MX_ERR_WORKSPACE);
  void* ws = nullptr;
  const int s = scratch_for_current_device(&ws);
  if (s != MX_OK) return s;
  return linear_bwd_impl(dy, dtype, M, N, K, xq_codes, xq_scales, wq_codes, wq_scales, seed, 0,
                         0, dx, dw, ws, kScratchBytes, as_stream(stream));
}

extern "C" int mx_linear_fwd(const void* x, const void* w, int dtype, int64_t M, int64_t N,
                             int64_t K, float* y, uint8_t* xq_codes, uint8_t* xq_scales,
                             uint8_t* wq_codes, uint8_t* wq_scales, void* stream) {
  return linear_fwd_impl(x, w, dtype, M, N, K, 0, 0, y, xq_codes, xq_scales, wq_codes, wq_scales,
                         as_stream(stream));
}

extern "C" int mx_linear_fwd_rht(const void* x, const void* w, int dtype, int64_t M, int64_t N,
                                 int64_t K, uint32_t sign_mask, float* y, uint8_t* xq_codes,
                                 uint8_t* xq_scales, uint8_t* wq_codes, uint8_t* wq_scales,
                                 void* stream) {
  return linear_fwd_impl(x, w, dtype, M, N, K, 1, sign_mask, y, xq_codes, xq_scales, wq_codes,
                         wq_scales, as_stream(stream));
}

extern "C" size_t mx_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  return bwd_layout(M, N, K).total;
}

extern "C" int mx_linear_bwd(const void* dy, int dtype, int64_t M, int64_t N, int64_t K,
                             const uint8_t* xq_codes, const uint8_t* xq_scales,
                             const uint8_t* wq_codes, const uint8_t* wq_scales, uint64_t seed,
                             float* dx, float* dw, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return linear_bwd_impl(dy, dtype, M, N, K, xq_codes, xq_scales, wq_codes, wq_scales, seed, 0,
                         0, dx, dw, workspace, workspace_bytes, as_stream(stream));
}

extern "C" int mx_linear_bwd_rht(const void* dy, int dtype, int64_t M, int64_t N, int64_t K,
                                 const uint8_t* xq_codes, const uint8_t* xq_scales,
                                 const uint8_t* wq_codes, const uint8_t* wq_scales, uint64_t seed,
                                 uint32_t sign_mask, float* dx, float* dw, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return linear_bwd_impl(dy, dtype, M, N, K, xq_codes, xq_scales, wq_codes, wq_scales, seed, 1,
                         sign_mask, dx, dw, workspace, workspace_bytes, as_stream(stream));
}

extern "C" size_t mx_grouped_linear_bwd_workspace_size(const int64_t* offs, int64_t groups,
                                                       int64_t N, int64_t K) {
  if (!valid_offsets(offs, groups) || N < 0 || K < 0) return 0;
  return grouped_layout(offs, groups, N, K).total;
}

// Backward of the grouped layer: dX through the grouped product with each
// expert's double-quantized weight, dW_e over the expert's own tokens in one
// launch of contraction ranges (the padded token axis of Q5 and Q6).
extern "C" int mx_grouped_linear_bwd(const void* dy, int dtype, const int64_t* offs,
                                     int64_t groups, int64_t N, int64_t K,
                                     const uint8_t* xq_codes, const uint8_t* xq_scales,
                                     const uint8_t* wq_codes, const uint8_t* wq_scales,
                                     uint64_t seed, float* dx, float* dw, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  MX_REQUIRE(dtype == MX_F32 || dtype == MX_BF16, MX_ERR_ENUM);
  MX_REQUIRE(valid_offsets(offs, groups), MX_ERR_SHAPE);
  MX_REQUIRE(N >= 0 && K >= 0 && N % 32 == 0 && K % 32 == 0, MX_ERR_SHAPE);
  MX_REQUIRE(N <= INT32_MAX && K <= INT32_MAX, MX_ERR_SHAPE);
  const int64_t E = groups, R = offs[groups];
  if (N == 0 || K == 0) return MX_OK;
  MX_REQUIRE(dw, MX_ERR_NULL);
  MX_REQUIRE(aligned16(dw), MX_ERR_ALIGN);
  if (R > 0) {
    MX_REQUIRE(dy && xq_codes && xq_scales && dx, MX_ERR_NULL);
    MX_REQUIRE(aligned16(dy) && aligned16(xq_codes) && aligned16(dx), MX_ERR_ALIGN);
  }
  MX_REQUIRE(wq_codes && wq_scales, MX_ERR_NULL);
  MX_REQUIRE(aligned16(wq_codes), MX_ERR_ALIGN);
  const GroupedLayout L = grouped_layout(offs, E, N, K);
  MX_REQUIRE(L.P <= INT32_MAX, MX_ERR_SHAPE);  // the dW contraction axis
  MX_REQUIRE(workspace && workspace_bytes >= L.total, MX_ERR_WORKSPACE);
  MX_REQUIRE(aligned16(workspace), MX_ERR_ALIGN);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const hipStream_t st = as_stream(stream);

  int s = requantize_batched_impl(wq_codes, wq_scales, E, N, K, MX_SR, seed + 4, ws + L.q4c,
                                  ws + L.q4s, st, L.p4);
  if (s != MX_OK) return s;
  if (R > 0) {
    // Q3 (1x32 along N, every token) and Q5 (32x1 along each expert's tokens)
    // from one read of dY
    s = quantize_dual_segments_impl(dy, dtype, R, N, offs, E, MX_SR, seed + 3, seed + 5,
                                    ws + L.q3c, ws + L.q3s, ws + L.q5c, ws + L.q5s, st, L.p3,
                                    L.p5, kExpertSegPad);
    if (s != MX_OK) return s;
    s = requantize_segments_impl(xq_codes, xq_scales, R, K, offs, E, MX_SR, seed + 6, ws + L.q6c,
                                 ws + L.q6s, st, L.p6, kExpertSegPad);
    if (s != MX_OK) return s;
    s = gemm_impl(ws + L.q3c, ws + L.q3s, ws + L.q4c, ws + L.q4s, offs, E, K, N, 1.0f, dx, K,
                  K * N / 2, K * L.p4, L.p3, L.p4, st);
    if (s != MX_OK) return s;
  }
  int64_t kbeg[MX_MAX_GROUPS + 1], klen[MX_MAX_GROUPS];
  segments_padded_offsets(offs, E, kbeg, kExpertSegPad);
  for (int64_t e = 0; e < E; ++e) klen[e] = (offs[e + 1] - offs[e] + 31) / 32 * 32;
  return gemm_ranges_impl(ws + L.q5c, ws + L.q5s, ws + L.q6c, ws + L.q6s, N, K, L.P, kbeg, klen, (int)E,
                          1.0f, dw, L.p5, L.p6, st);
}

extern "C" const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: unsupported or inconsistent sizes";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case MX_ERR_ENUM: return "MX_ERR_ENUM: an enum or flag argument is out of range";
    case MX_ERR_WORKSPACE: return "MX_ERR_WORKSPACE: workspace missing or too small";
    case MX_ERR_HIP: return "MX_ERR_HIP: the HIP runtime rejected a launch";
    default: return "unknown mx_status";
  }
}
