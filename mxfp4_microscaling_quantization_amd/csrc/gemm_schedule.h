// Load / wait schedule constants of the MXFP4 GEMM kernels (gemm.hip).  The
// kernels take their vmcnt thresholds and load counts from here and check them
// against their own tile arithmetic at compile time; the CPU model of the
// schedule in the tests reads this file, so the model and the kernels cannot
// drift apart.  Plain integer literals only (the model parses them).
#pragma once

namespace mx {

// Scale-load modes: 16-byte groups of four K-steps, one dword per step, two
// 2-byte loads per step, bytes.
enum { kScGroup = 0, kScDword = 1, kScByte = 2, kScShort = 3 };

// k_gemm_mx (one barrier per K-step, loads three steps ahead): for each tile
// configuration the host launches, LC = vector-memory loads a wave issues per
// step (code loads, plus the step's scale loads in the per-step modes) and QW
// = scale loads per wave per scale job (per four steps in group mode).
struct MxSchedule {
  int bm, bn, waves, sc, lc, qw;
};
constexpr MxSchedule kMxSchedules[] = {
    {256, 256, 8, kScGroup, 4, 1},  {256, 256, 4, kScDword, 10, 2},
    {256, 256, 4, kScShort, 12, 4}, {256, 256, 4, kScByte, 16, 8},
    {128, 128, 4, kScGroup, 4, 1},  {128, 128, 4, kScDword, 5, 1},
    {128, 128, 4, kScShort, 6, 2},  {128, 128, 4, kScByte, 8, 4},
};
constexpr bool mx_schedule_listed(int bm, int bn, int waves, int sc, int lc, int qw) {
  for (const MxSchedule& s : kMxSchedules)
    if (s.bm == bm && s.bn == bn && s.waves == waves && s.sc == sc && s.lc == lc && s.qw == qw)
      return true;
  return false;
}

// k_gemm_pp (256 x 256 tiles, group scale loads, phases L(j) / C(j)): per step
// a wave issues kPpLoads code loads for step j + kPpLead in C(j), then, when
// j % 4 == 0, kPpGroupLoads scale-group loads for the next group; at the end of
// L(j) it waits with vmcnt(kPpWaitFull[j % 4]) on full steps, vmcnt(kPpWaitNear)
// on the last steps while j + 2 < KT (else 0), and after the prologue (group 0,
// steps 0-2) with vmcnt(kPpWaitFirst[min(KT, 3) - 1]).
constexpr int kPpLoads = 4;
constexpr int kPpGroupLoads = 1;
constexpr int kPpLead = 3;
constexpr int kPpWaitFull[4] = {4, 5, 5, 4};
constexpr int kPpWaitNear = 4;
constexpr int kPpWaitFirst[3] = {0, 4, 8};
// The same kernel on scale rows that are not 16-byte aligned (K / 32 not a
// multiple of 16, e.g. 90-byte rows at K = 2880): a scale group is fetched as
// the two aligned 16-byte pieces that hold it (kPpGroupLoadsUnal loads) and
// shifted into place in LDS at the end of L(j), j % 4 == 3.  Code loads, lead
// and the other waits are as above.
constexpr int kPpGroupLoadsUnal = 2;
constexpr int kPpWaitFullUnal[4] = {4, 6, 6, 4};

}  // namespace mx
