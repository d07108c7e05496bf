"""Host check of the grouped GEMM's load accounting (gemm_schedule.h).

Each K stage waits with vmcnt(n), n = the loads issued after that stage's
last load. A count too small stalls; a count too large lets a wave read LDS
before its data has landed, a silent race. The closed forms of the header
are compared with a brute-force walk over the issue order the tile loop
follows, for every ring depth, load count and stage count in use and
around them.
"""
import os
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "top_routing_expert_02_amd", "csrc")

CASES = [(na, nw, la, lb) for na in (2, 3) for nw in (2, 3, 4) for la, lb in
         ((8, 8), (6, 8), (4, 8), (2, 8))]
NK = list(range(1, 12)) + [64, 224]


def issue_order(nk, NA, NW, LA, LB, t):
    """(kind, stage) of every load issued by the wait at the end of stage t;
    refills past the last stage are marked as reloads."""
    out = [("A", 0)] * LA + [("W", 0)] * LB
    for p in range(1, min(max(NA, NW), nk)):
        if p < NA:
            out += [("A", p)] * LA
        if p < NW:
            out += [("W", p)] * LB
    for j in range(0, min(t, max(0, nk - min(NA, NW)))):
        a, w = j + NA, j + NW
        out += [("A", a) if a < nk else ("reload", -1)] * LA
        out += [("W", w) if w < nk else ("reload", -1)] * LB
    return out


def brute(nk, NA, NW, LA, LB, t):
    seq = issue_order(nk, NA, NW, LA, LB, t)
    s = t + 1
    last = max(i for i, x in enumerate(seq) if x in (("A", s), ("W", s)))
    # every load of stages <= s is at or before the last one waited for
    assert all(not (x[0] in "AW" and 0 <= x[1] <= s) for x in seq[last + 1:])
    return len(seq) - 1 - last


@pytest.fixture(scope="module")
def closed_forms(tmp_path_factory):
    d = tmp_path_factory.mktemp("sched")
    src = d / "check.cpp"
    cases = ", ".join("{%d, %d, %d, %d}" % c for c in CASES)
    nks = ", ".join(str(n) for n in NK)
    # one loop over the cases (an unrolled call per case takes minutes to compile)
    lines = ['#include "gemm_schedule.h"', "#include <cstdio>", "int main() {",
             f"  const int cases[][4] = {{{cases}}};",
             f"  const int nks[] = {{{nks}}};",
             "  for (const auto& c : cases)",
             "    for (int nk : nks) {",
             '      std::printf("P %d %d %d %d %d %d\\n", c[0], c[1], c[2], c[3], nk,',
             "                  moe::sched_prologue_loads(nk, c[0], c[1], c[2], c[3]));",
             "      for (int t = 0; t < nk - 1; ++t)",
             '        std::printf("W %d %d %d %d %d %d %d\\n", c[0], c[1], c[2], c[3], nk, t,',
             "                    moe::sched_loads_after(t, nk, c[0], c[1], c[2], c[3]));",
             '      std::printf("S %d %d %d %d %d\\n", c[0], c[1], c[2], c[3],',
             "                  moe::sched_steady_loads(c[0], c[1], c[2], c[3]));",
             "    }"]
    lines.append("  return 0;\n}")
    src.write_text("\n".join(lines))
    exe = d / "check"
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return [line.split() for line in out.splitlines()]


def test_stage_waits_match_the_issue_order(closed_forms):
    n = 0
    for rec in closed_forms:
        if rec[0] != "W":
            continue
        na, nw, la, lb, nk, t, got = map(int, rec[1:])
        assert got == brute(nk, na, nw, la, lb, t), (na, nw, la, lb, nk, t)
        assert 0 <= got <= 63  # a vmcnt immediate
        n += 1
    assert n > 1000


def test_prologue_wait_matches_the_issue_order(closed_forms):
    for rec in closed_forms:
        if rec[0] != "P":
            continue
        na, nw, la, lb, nk, got = map(int, rec[1:])
        # stage 0 is the first entry: everything of the prologue after it
        seq = issue_order(nk, na, nw, la, lb, 0)
        assert got == len(seq) - (la + lb), (na, nw, la, lb, nk)


def test_xcd_plan_covers_every_tile_once(tmp_path):
    """sched_xcd_plan: every tile of a launch goes to exactly one block, each
    block takes slot b // 8 of its windows of G // 8 consecutive tiles, one
    window per round (interleaved: XCD b % 8 takes window 8 r + b % 8 in
    round r; otherwise a contiguous range of windows per XCD), and no block
    runs more rounds than ceil(total / G)."""
    src = tmp_path / "plan.cpp"
    src.write_text("\n".join([
        '#include "gemm_schedule.h"', "#include <cstdio>", "int main() {",
        "  const int grids[] = {256, 248, 64, 8, 7};",
        "  const int totals[] = {0, 1, 5, 8, 9, 63, 255, 256, 257, 511, 512, 513, 2800, 2816, 2992, 7488, 9856};",
        "  for (int rr = 0; rr < 2; ++rr)",
        "    for (int G : grids)",
        "      for (int total : totals)",
        "        for (int b = 0; b < G; ++b) {",
        "          int first, stride, end;",
        "          moe::sched_xcd_plan(b, G, total, rr != 0, first, stride, end);",
        '          std::printf("%d %d %d %d %d %d %d\\n", rr, G, total, b, first, stride, end);',
        "        }",
        "  return 0;\n}"]))
    exe = tmp_path / "plan"
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    runs = {}
    for line in out.splitlines():
        rr, G, total, b, first, stride, end = map(int, line.split())
        assert stride > 0 and end <= total
        runs.setdefault((rr, G, total), []).append((b, list(range(first, end, stride))))
    assert len(runs) == 2 * 5 * 17
    for (rr, G, total), blocks in runs.items():
        seen = [t for _, ts in blocks for t in ts]
        assert sorted(seen) == list(range(total)), (rr, G, total)
        rounds = -(-total // G)
        assert max(len(ts) for _, ts in blocks) <= max(rounds, 1), (rr, G, total)
        if G % 8 == 0 and total > G:
            S = G // 8
            for b, ts in blocks:
                assert all(t % S == b // 8 for t in ts), (rr, G, total, b)
                windows = [t // S for t in ts]
                if rr:
                    assert windows == [8 * r + b % 8 for r in range(len(ts))], (G, total, b)
                else:
                    assert all(w2 - w1 == 1 for w1, w2 in zip(windows, windows[1:])), (G, total, b)


def test_refilling_stages_wait_the_steady_count(closed_forms):
    """A stage t that refills (t + min(NA, NW) < nk) waits with the rings'
    fixed count sched_steady_loads, an immediate in the kernel's steady
    state: for rings with NA <= NW <= NA + 1 (the kernel's) it
    must equal the closed form (itself checked against the brute-force walk)
    at every such stage."""
    steady = {tuple(map(int, r[1:5])): int(r[5]) for r in closed_forms if r[0] == "S"}
    n = 0
    for rec in closed_forms:
        if rec[0] != "W":
            continue
        na, nw, la, lb, nk, t, got = map(int, rec[1:])
        if t + min(na, nw) < nk and na <= nw <= na + 1:
            assert got == steady[(na, nw, la, lb)], (na, nw, la, lb, nk, t)
            n += 1
    assert n > 500
    # the kernel's rings: 2+2, 2+3, 3+3, 3+4 buffers
    for na, nw in ((2, 2), (2, 3), (3, 3), (3, 4)):
        assert na <= nw <= na + 1


def refill_slots(nk, NA, NW, LA, LB):
    """(kind, stage, slot) of every refill load of a tile's K loop: the
    refill at stage j loads token stage j + NA into token slot j % NA and
    weight stage j + NW into weight slot j % NW (a stage past the last loads
    the last one again, marked stage -1)."""
    out = []
    for j in range(0, max(0, nk - min(NA, NW))):
        a, w = j + NA, j + NW
        out += [("A", a if a < nk else -1, j % NA)] * LA
        out += [("W", w if w < nk else -1, j % NW)] * LB
    return out


@pytest.mark.parametrize("na,nw,la,lb", [c for c in CASES if c[0] <= c[1] <= c[0] + 1])
def test_epilogue_lds_is_free(na, nw, la, lb):
    """After a tile's last stage, the loads issued after the last stage's own
    loads have not been waited for. None of them may land in the LDS the
    epilogue uses: the weight slot its outputs are staged in (slot 1, or 2
    when the K loop's last refill reloaded the last stage into slot 1, as
    the tile loop picks it) or the token slots the next tile's offsets park
    in (slot 1, and slot 2 for 64-row tiles, whose token offsets go there).
    Slot 0 is the next tile's stage 0."""
    tm = la // 2
    for nk in NK:
        seq = []
        for p in range(min(max(na, nw), nk)):  # the prologue: stage 0, then 1 ..
            seq += ([("A", p, p)] * la if p < na else []) + ([("W", p, p)] * lb if p < nw else [])
        seq += refill_slots(nk, na, nw, la, lb)
        last = max(i for i, x in enumerate(seq) if x[1] == nk - 1)
        pending = seq[last + 1:]
        ws = 2 if (nw > na and nk % nw == 1) else 1
        parked = {1, 2} if tm == 1 else {1}
        assert ws < nw
        for kind, stage, slot in pending:
            assert stage == -1, (nk, kind, stage)
            if kind == "W":
                assert slot != ws, (na, nw, nk)
            else:
                assert slot not in parked, (na, nw, nk)
