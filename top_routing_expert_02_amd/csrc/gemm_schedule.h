// Scheduling arithmetic of the grouped GEMM, shared by the kernel and the
// host tests: the blocks' tile ranges and the load accounting of the stage
// rings.
//
// Load accounting.
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
MOE_HD constexpr int sched_prefix(int p, int NA, int NW, int LA, int LB) {
  int n = 0;
  for (int q = 0; q < p; ++q) n += (q < NA ? LA : 0) + (q < NW ? LB : 0);
  return n;
}

// issue position (1-based count of loads up to and including it) of the
// last load of token stage s (weight = false) or weight stage s
MOE_HD constexpr int sched_pos(bool weight, int s, int nk, int NA, int NW, int LA, int LB) {
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
MOE_HD constexpr int sched_loads_after(int t, int nk, int NA, int NW, int LA, int LB) {
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

// The same wait at any stage t that refills (t + min(NA, NW) < nk), for
// rings with NA <= NW <= NA + 1 (the kernel's): every refill
// group issues the same loads, so the count depends on the rings alone (a
// host test checks it against sched_loads_after at every such t). The
// kernel uses it as an immediate in its steady state. (With other depths
// the count changes over the first stages.)
MOE_HD constexpr int sched_steady_loads(int NA, int NW, int LA, int LB) {
  return sched_loads_after(0, 2 * (NA + NW) + 2, NA, NW, LA, LB);
}

// loads of prologue entries 1 .. (issued after the previous tile's stores)
MOE_HD inline int sched_prologue_loads(int nk, int NA, int NW, int LA, int LB) {
  const int nmax = NA > NW ? NA : NW;
  const int entries = nmax < nk ? nmax : nk;
  return sched_prefix(entries, NA, NW, LA, LB) - (LA + LB);
}

// Tiles of block b in a persistent launch of G blocks over `total` tiles:
// first, first + stride, ... below end. Blocks are dealt to the 8 XCDs
// round-robin (block b runs on XCD b mod 8), and the tiles one XCD runs
// together are consecutive: they share weight and token panels in its L2.
// A launch whose tiles fit in one round gives each XCD ceil(total / 8)
// consecutive tiles. Over several rounds:
//  * interleaved (reread): round r runs windows 8r .. 8r + 7 of G / 8
//    consecutive tiles, one per XCD, so the whole chip works on
//    neighbouring tiles: the weight panels of an expert whose M tiles come
//    in several groups (each group re-reads them) are read again while the
//    MALL still holds them;
//  * otherwise each XCD works through a contiguous range of its own, one
//    window per round. Experts read once (a few M tiles each) streamed
//    faster this way: the decode layer's first GEMM went from 204 to 170 µs
//    and the large-E layer's GEMMs from 914 and 966 to 868 and 932 µs,
//    while the 16384-token layer's (22 M tiles per expert, re-read) got 5%
//    slower, hence the choice.
// Block b takes slot b / 8 of each of its windows. Every tile below total
// goes to exactly one block.
MOE_HD inline void sched_xcd_plan(int b, int G, int total, bool reread, int& first, int& stride,
                                  int& end) {
  first = b;
  stride = G;
  end = total;
  if (G % 8 != 0) return;
  const int kk = b / 8, x = b % 8;
  const int S = G / 8;
  if (total <= G) {
    const int per = (total + 7) / 8;
    first = kk < per ? x * per + kk : total;
    return;
  }
  if (reread) {
    first = x * S + kk;
    return;
  }
  const int R = (total + G - 1) / G;
  first = x * R * S + kk;
  stride = S;
  end = total < (x + 1) * R * S ? total : (x + 1) * R * S;
}

}  // namespace moe
