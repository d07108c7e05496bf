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
