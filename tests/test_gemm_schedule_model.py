"""CPU model of the MXFP4 GEMM kernel's load / wait schedule in its 16-byte
scale-group mode (csrc/gemm.hip, k_gemm_mx: the prologue, the `step` lambda and
the two K loops).  Each step k waits with s_waitcnt vmcnt(n) before its barrier
and then reads stage k+1 and the scale group of step k+1; completion is in issue
order, so vmcnt(n) means every load except the last n issued has landed.  The
model replays the kernel's issue order and thresholds for every step count and
checks that no wait leaves data the following reads need in flight, including
contractions whose last scale group is partial (scale rows padded past K/32)."""
import pytest


def schedule_violation(KT, LC, QW, g2_extra=0, grouped=True):
    """None if the schedule is sound for KT steps; LC = loads per stage, QW =
    loads per scale group (per wave).  g2_extra plants a wrong allowance.
    grouped=False: the per-step scale modes (dword, short, byte), whose scale
    loads are part of each stage's LC loads and which issue no scale groups."""
    issued = []
    if not grouped:
        QW = 0

    def issue(kt):
        issued.extend([("stage", kt)] * LC)

    def issue_scales(g):
        if grouped:
            issued.extend([("group", g)] * QW)

    def wait(n, need):
        pending = issued[len(issued) - n:] if n else []
        done = issued[:len(issued) - n] if n else issued
        for item in need:
            if item in pending or item not in done:
                return f"KT={KT}: vmcnt({n}) leaves {item} in flight"
        return None

    issue_scales(0)                      # prologue: group 0, stages 0..2
    for k in range(min(3, KT)):
        issue(k)
    n = 2 * LC if KT > 2 else (LC if KT > 1 else 0)
    e = wait(n, [("stage", 0)] + ([("group", 0)] if grouped else []))
    if e:
        return e

    def step(kt, full):
        P = kt % 4
        G2 = QW if P == 2 else 0
        G1 = (QW if P == 1 else 0) + (g2_extra if P == 1 else 0)
        need = [("stage", kt + 1)] + ([("group", (kt + 1) >> 2)] if grouped else [])
        if full:                         # kt + 7 < KT rounded to a multiple of 4
            e = wait(LC + G1 + G2, need)
            if e:
                return e
            issue(kt + 3)
            if P == 0:
                issue_scales((kt >> 2) + 1)
        elif kt + 1 < KT:
            n = LC + G1 + G2 if kt + 3 < KT else (LC + G2 if kt + 2 < KT else 0)
            e = wait(n, need)
            if e:
                return e
            if kt + 3 < KT:
                issue(kt + 3)
            if P == 0 and kt + 4 < KT:
                issue_scales((kt >> 2) + 1)
        return None

    kt = 0
    while kt + 7 < KT:
        for d in range(4):
            e = step(kt + d, True)
            if e:
                return e
        kt += 4
    while kt < KT:
        for d in range(4):
            if kt + d < KT:
                e = step(kt + d, False)
                if e:
                    return e
        kt += 4
    return None


# (LC, QW) of the 256x256 tile with four waves (8 code loads, 2 scale-group loads
# per wave) and of the 128x128 tile and the 256x256 tile with eight waves (4, 1)
@pytest.mark.parametrize("LC,QW", [(8, 2), (4, 1)])
def test_every_step_count_waits_for_what_it_reads(LC, QW):
    bad = [e for KT in range(1, 65) if (e := schedule_violation(KT, LC, QW))]
    assert not bad, bad[:3]


def test_model_catches_a_short_wait():
    """A wait that allows one more scale group in flight at P == 1 must fail."""
    assert any(schedule_violation(KT, 8, 2, g2_extra=2) for KT in range(1, 65))


# per-step scale modes: LC = code loads + scale loads per wave and step (256x256
# tile, four waves: dword 8 + 2, short 8 + 4, byte 8 + 8; 128x128 tile: 4 + 1,
# 4 + 2, 4 + 4).  Step counts 1..3 also cover the three-stage short-contraction
# variant, which issues every load in the prologue.
@pytest.mark.parametrize("LC", [10, 12, 16, 5, 6, 8])
def test_per_step_scale_modes_wait_for_what_they_read(LC):
    bad = [e for KT in range(1, 65) if (e := schedule_violation(KT, LC, 0, grouped=False))]
    assert not bad, bad[:3]


def test_model_catches_a_short_wait_in_per_step_modes():
    """One more load left in flight at P == 1 must fail there too."""
    assert any(schedule_violation(KT, 10, 0, g2_extra=1, grouped=False) for KT in range(1, 65))
