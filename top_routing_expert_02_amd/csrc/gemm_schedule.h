// Load accounting of the grouped GEMM's stage rings (host and device).
//
// A tile of nk K stages keeps its token tiles in a ring of NA buffers and
// its weight tiles in a ring of NW buffers. Each wave issues its LDS-DMA
// loads in this order:
//   prologue entry 0:  token stage 0 (LA loads), weight stage 0 (LB loads)
//   prologue entries p = 1 .. min(max(NA, NW), nk) - 1:
//                      token stage p if p < NA, weight stage p if p < NW
//   refill group j, after stage j, for j < nk - min(NA, NW):
//                      token stage j + NA, weight stage j + NW (a stage past
//                      the last one loads the last one again, into a
//                      buffer no later stage reads: every group has
//                      LA + LB loads)
// Loads return in issue order, so "stage s has landed" is vmcnt(n) with n
// the number of loads issued after stage s's last one at the moment of the
// wait. The wait for stage t + 1 comes at the end of stage t, when groups
// 0 .. t - 1 have been issued.
#pragma once

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

// loads of prologue entries 0 .. p - 1
MOE_HD inline int sched_prefix(int p, int NA, int NW, int LA, int LB) {
  int n = 0;
  for (int q = 0; q < p; ++q) n += (q < NA ? LA : 0) + (q < NW ? LB : 0);
  return n;
}

// issue position (1-based count of loads up to and including it) of the
// last load of token stage s (weight = false) or weight stage s
MOE_HD inline int sched_pos(bool weight, int s, int nk, int NA, int NW, int LA, int LB) {
  const int nmax = NA > NW ? NA : NW;
  const int entries = nmax < nk ? nmax : nk;
  const int N = weight ? NW : NA;
  if (s < N) {
    // in prologue entry s: its token loads come first
    return sched_prefix(s, NA, NW, LA, LB) + (weight ? (s < NA ? LA : 0) + LB : LA);
  }
  const int j = s - N;  // refill group
  return sched_prefix(entries, NA, NW, LA, LB) + j * (LA + LB) + (weight ? LA + LB : LA);
}

// loads issued after stage t + 1's last load, at the wait at the end of stage t
MOE_HD inline int sched_loads_after(int t, int nk, int NA, int NW, int LA, int LB) {
  const int nmax = NA > NW ? NA : NW;
  const int nmin = NA < NW ? NA : NW;
  const int entries = nmax < nk ? nmax : nk;
  int groups = t < nk - nmin ? t : nk - nmin;
  if (groups < 0) groups = 0;
  const int issued = sched_prefix(entries, NA, NW, LA, LB) + groups * (LA + LB);
  const int a = sched_pos(false, t + 1, nk, NA, NW, LA, LB);
  const int w = sched_pos(true, t + 1, nk, NA, NW, LA, LB);
  return issued - (a > w ? a : w);
}

// loads of prologue entries 1 .. (issued after the previous tile's stores)
MOE_HD inline int sched_prologue_loads(int nk, int NA, int NW, int LA, int LB) {
  const int nmax = NA > NW ? NA : NW;
  const int entries = nmax < nk ? nmax : nk;
  return sched_prefix(entries, NA, NW, LA, LB) - (LA + LB);
}

}  // namespace moe
