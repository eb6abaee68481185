"""CPU model of the MXFP4 GEMM kernels' load / wait schedules, driven by the
constants the kernels themselves use (csrc/gemm_schedule.h, which the kernels
check against their own tile arithmetic at compile time).

Vector-memory loads complete in issue order, so s_waitcnt vmcnt(n) means every
load except the last n issued has landed.  The model replays each kernel's
issue order for every step count 1..64 and checks that no wait leaves data that
the following reads need in flight:
 - k_gemm_mx: each step waits before its barrier, then reads stage k+1 and the
   scale group of step k+1 (per-step scale modes: the scales are part of each
   stage's loads);
 - k_gemm_pp: phase L(j) ends with a wait after which stage j+1 and its scale
   group are read; phase C(j) issues stage j+3, then (j % 4 == 0) the next scale
   group.
"""
import os
import re

import pytest

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "mxfp4_microscaling_quantization_amd", "csrc", "gemm_schedule.h")


def header_constants():
    text = re.sub(r"//.*", "", open(HEADER).read())
    modes = dict((m, int(v)) for m, v in re.findall(r"(kSc\w+)\s*=\s*(\d+)", text))
    table = re.search(r"kMxSchedules\[\]\s*=\s*\{(.*?)\};", text, re.S).group(1)
    rows = []
    for bm, bn, waves, sc, lc, qw in re.findall(
            r"\{\s*(\d+),\s*(\d+),\s*(\d+),\s*(kSc\w+),\s*(\d+),\s*(\d+)\s*\}", table):
        rows.append(dict(bm=int(bm), bn=int(bn), waves=int(waves), sc=modes[sc], lc=int(lc),
                         qw=int(qw), mode=sc))

    def scalar(name):
        return int(re.search(rf"constexpr int {name}\s*=\s*(\d+);", text).group(1))

    def array(name):
        body = re.search(rf"constexpr int {name}\[\d+\]\s*=\s*\{{([^}}]*)\}};", text).group(1)
        return [int(v) for v in body.split(",")]

    pp = dict(loads=scalar("kPpLoads"), group_loads=scalar("kPpGroupLoads"),
              lead=scalar("kPpLead"), wait_full=array("kPpWaitFull"),
              wait_near=scalar("kPpWaitNear"), wait_first=array("kPpWaitFirst"))
    # unaligned scale rows: two loads per group, their own full-step waits
    pp_unal = dict(pp, group_loads=scalar("kPpGroupLoadsUnal"),
                   wait_full=array("kPpWaitFullUnal"))
    return modes, rows, pp, pp_unal


MODES, MX_ROWS, PP, PP_UNAL = header_constants()


class Issued:
    def __init__(self):
        self.items = []

    def add(self, item, n):
        self.items.extend([item] * n)

    def wait(self, n, need, KT, where):
        """vmcnt(n): everything but the last n loads landed; `need` must be landed."""
        pending = self.items[len(self.items) - n:] if n else []
        done = self.items[:len(self.items) - n] if n else self.items
        for item in need:
            if item in pending or item not in done:
                return f"KT={KT} {where}: vmcnt({n}) leaves {item} in flight"
        return None


def mx_violation(KT, LC, QW, grouped, extra=0):
    """k_gemm_mx; `extra` plants a wrong allowance at P == 1 (the model must catch it)."""
    q = Issued()
    if not grouped:
        QW = 0
    if grouped:
        q.add(("group", 0), QW)
    for k in range(min(3, KT)):
        q.add(("stage", k), LC)
    n = 2 * LC if KT > 2 else (LC if KT > 1 else 0)
    e = q.wait(n, [("stage", 0)] + ([("group", 0)] if grouped else []), KT, "prologue")
    if e:
        return e
    kt = 0
    while kt < KT:
        full = kt + 7 < KT
        for d in range(4):
            k = kt + d
            if k >= KT:
                break
            P = k % 4
            G2 = QW if P == 2 else 0
            G1 = (QW if P == 1 else 0) + (extra if P == 1 else 0)
            need = [("stage", k + 1)] + ([("group", (k + 1) >> 2)] if grouped else [])
            if full:
                e = q.wait(LC + G1 + G2, need, KT, f"step {k}")
                if e:
                    return e
                q.add(("stage", k + 3), LC)
                if P == 0 and grouped:
                    q.add(("group", (k >> 2) + 1), QW)
            elif k + 1 < KT:
                n = LC + G1 + G2 if k + 3 < KT else (LC + G2 if k + 2 < KT else 0)
                e = q.wait(n, need, KT, f"step {k}")
                if e:
                    return e
                if k + 3 < KT:
                    q.add(("stage", k + 3), LC)
                if P == 0 and grouped and k + 4 < KT:
                    q.add(("group", (k >> 2) + 1), QW)
        kt += 4
    return None


def pp_violation(KT, pp, extra=0):
    """k_gemm_pp (one wave's loads; every wave issues the same sequence)."""
    LC, QW, lead = pp["loads"], pp["group_loads"], pp["lead"]
    q = Issued()
    q.add(("group", 0), QW)
    for k in range(min(lead, KT)):
        q.add(("stage", k), LC)
    e = q.wait(pp["wait_first"][min(KT, 3) - 1], [("stage", 0), ("group", 0)], KT, "prologue")
    if e:
        return e
    kt = 0
    while kt < KT:
        full = kt + 7 < KT
        for d in range(4):
            j = kt + d
            if j >= KT:
                break
            P = j % 4
            # end of L(j): stage j+1 and its scale group are read next
            if j + 1 < KT:
                need = [("stage", j + 1), ("group", (j + 1) >> 2)]
                if full:
                    n = pp["wait_full"][P] + (extra if P == 1 else 0)
                else:
                    n = pp["wait_near"] if j + 2 < KT else 0
                e = q.wait(n, need, KT, f"L({j})")
                if e:
                    return e
            # C(j): stage j + lead, then the next scale group every four steps
            if full or j + lead < KT:
                q.add(("stage", j + lead), LC)
            if P == 0 and (full or j + 4 < KT):
                q.add(("group", (j >> 2) + 1), QW)
        kt += 4
    return None


def test_header_lists_the_launched_configurations():
    keys = {(r["bm"], r["bn"], r["waves"], r["mode"]) for r in MX_ROWS}
    assert (256, 256, 8, "kScGroup") in keys and (128, 128, 4, "kScByte") in keys
    assert len(keys) == len(MX_ROWS) == 8
    for r in MX_ROWS:   # the loads per step follow from the tile and the wave count
        codes = (r["bm"] + r["bn"]) // 16 // r["waves"]
        assert r["lc"] == codes + (0 if r["mode"] == "kScGroup" else r["qw"])


@pytest.mark.parametrize("row", MX_ROWS, ids=lambda r: f"{r['bm']}x{r['bn']}-{r['waves']}w-{r['mode']}")
def test_mx_kernel_waits_for_what_it_reads(row):
    grouped = row["mode"] == "kScGroup"
    bad = [e for KT in range(1, 65) if (e := mx_violation(KT, row["lc"], row["qw"], grouped))]
    assert not bad, bad[:3]


def test_pp_kernel_waits_for_what_it_reads():
    bad = [e for KT in range(1, 65) if (e := pp_violation(KT, PP))]
    assert not bad, bad[:3]


def test_pp_kernel_with_unaligned_scale_rows_waits_for_what_it_reads():
    """Two loads per scale group; the group is shifted into place at the end of
    L(j), j % 4 == 3, the same point where the model requires it landed."""
    assert PP_UNAL["group_loads"] == 2
    bad = [e for KT in range(1, 65) if (e := pp_violation(KT, PP_UNAL))]
    assert not bad, bad[:3]
    # waiting for more (the aligned thresholds) stays safe; one more load in
    # flight at P == 1 or 2 leaves a piece of the group in flight
    tight = dict(PP_UNAL, wait_full=PP["wait_full"])
    assert not any(pp_violation(KT, tight) for KT in range(1, 65))
    loose = dict(PP_UNAL, wait_full=[w + (1 if i in (1, 2) else 0)
                                     for i, w in enumerate(PP_UNAL["wait_full"])])
    assert any(pp_violation(KT, loose) for KT in range(1, 65))


def test_models_catch_a_wait_that_is_one_too_loose():
    """One more load allowed in flight at P == 1 must be caught in both models."""
    assert any(pp_violation(KT, PP, extra=1) for KT in range(1, 65))
    grp = next(r for r in MX_ROWS if r["mode"] == "kScGroup")
    assert any(mx_violation(KT, grp["lc"], grp["qw"], True, extra=grp["qw"]) for KT in range(1, 65))
    per = next(r for r in MX_ROWS if r["mode"] == "kScDword")
    assert any(mx_violation(KT, per["lc"], 0, False, extra=1) for KT in range(1, 65))
