// Dispatch under the general capacity rule: a priority order (token-major or
// rank-major) and rounds of overflow re-routing to each token's next
// candidate expert (page "MoE 模型原理：路由、专家负载、容量、通信与推理成本",
// wrblog.cn, §4.3, second overflow option: capacity allocated candidate by
// candidate; ai-master.cc EP engineering answer 001, §一: overflow moves to
// the next-best expert or is dropped).
//
// Assignment (t, r) has a priority position q: t*k + r (token order) or
// r*T + t (rank order). Each round is the first-come rule of the plain
// dispatch applied to the assignments still unplaced, in position order:
//   1. per 64-position tile, a histogram of the experts they are offered to;
//   2. per expert, an exclusive prefix over tiles (one block);
//   3. per tile, a 64-bit mask per expert: the popcount below a position is
//      its rank among the tile's arrivals at that expert. Its slot is the
//      expert's fill at the round's start + the tile base + that rank, and it
//      is placed while the slot is below C.
// Between rounds each token hands its unplaced assignments, in rank order,
// the next unused columns of its candidate list. At the end the kept rows
// are laid out expert-major in slot order. Integer work only: deterministic.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kRrTile = 64;  // positions per tile (one bit each in a 64-bit mask)

struct Order {
  int64_t T;
  int k;
  bool rank;
  __device__ __forceinline__ void at(int64_t q, int64_t& t, int& r) const {
    if (rank) {
      r = static_cast<int>(q / T);
      t = q - static_cast<int64_t>(r) * T;
    } else {
      t = q / k;
      r = static_cast<int>(q - t * k);
    }
  }
};

// expert the assignment at position q is offered to this round, or -1
__device__ __forceinline__ int offered(const Order& o, int64_t q, int64_t Q, const int32_t* cand,
                                       int n, const int32_t* col, const int32_t* served,
                                       int64_t& a) {
  if (q >= Q) return -1;
  int64_t t;
  int r;
  o.at(q, t, r);
  a = t * o.k + r;
  const int c = col[a];
  if (served[a] >= 0 || c < 0) return -1;
  return cand[t * n + c];
}

__global__ __launch_bounds__(256) void rr_init_kernel(int64_t T, int k, int E, int32_t* __restrict__ col,
                                                      int32_t* __restrict__ served,
                                                      int32_t* __restrict__ next_col,
                                                      int32_t* __restrict__ fill) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < T) {
    next_col[i] = k;
    for (int r = 0; r < k; ++r) {
      col[i * k + r] = r;
      served[i * k + r] = -1;
    }
  }
  if (i < E) fill[i] = 0;
}

// before round j >= 1: unplaced assignments take the token's next columns
__global__ __launch_bounds__(256) void rr_advance_kernel(int64_t T, int k, int n, int32_t* __restrict__ col,
                                                         const int32_t* __restrict__ served,
                                                         int32_t* __restrict__ next_col) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  int nc = next_col[t];
  for (int r = 0; r < k; ++r) {
    const int64_t a = t * k + r;
    if (served[a] >= 0 || col[a] < 0) continue;
    col[a] = (nc < n) ? nc++ : -1;
  }
  next_col[t] = nc;
}

__global__ __launch_bounds__(kRrTile) void rr_hist_kernel(Order o, int64_t Q, const int32_t* __restrict__ cand,
                                                          int n, int E, const int32_t* __restrict__ col,
                                                          const int32_t* __restrict__ served,
                                                          int32_t* __restrict__ hist) {
  __shared__ int s_hist[1024];
  for (int e = threadIdx.x; e < E; e += kRrTile) s_hist[e] = 0;
  __syncthreads();
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kRrTile + threadIdx.x;
  int64_t a = 0;
  const int e = offered(o, q, Q, cand, n, col, served, a);
  if (e >= 0) atomicAdd(&s_hist[e], 1);
  __syncthreads();
  int32_t* h = hist + static_cast<int64_t>(blockIdx.x) * E;
  for (int i = threadIdx.x; i < E; i += kRrTile) h[i] = s_hist[i];
}

// one block: P = 1024 / E (rounded down to a power of two) threads per
// expert, each owning a contiguous run of tiles; a first pass sums each run,
// an exclusive prefix over the runs (in LDS) gives each its starting base,
// a second pass writes the bases. Loads go out eight at a time (the passes
// are bound by load latency).
__global__ __launch_bounds__(1024) void rr_scan_kernel(const int32_t* __restrict__ hist, int ntiles, int E,
                                                       int C, int round, int32_t* __restrict__ base,
                                                       int32_t* __restrict__ fill,
                                                       int32_t* __restrict__ fill0,
                                                       int32_t* __restrict__ counts) {
  __shared__ int part[1024];
  int P = 1;
  while (P * 2 * E <= 1024) P *= 2;
  const int tid = threadIdx.x;
  const bool active = tid < P * E;
  const int e = tid % E;
  const int p = tid / E;
  const int chunk = (ntiles + P - 1) / P;
  const int t_begin = min(ntiles, p * chunk);
  const int t_end = min(ntiles, t_begin + chunk);
  int sum = 0;
  if (active) {
    int t = t_begin;
    for (; t + 8 <= t_end; t += 8) {
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = hist[static_cast<int64_t>(t + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += h[u];
    }
    for (; t < t_end; ++t) sum += hist[static_cast<int64_t>(t) * E + e];
    part[p * E + e] = sum;
  }
  __syncthreads();
  if (!active) return;
  int run = 0;
  for (int q = 0; q < p; ++q) run += part[q * E + e];
  int t = t_begin;
  for (; t + 8 <= t_end; t += 8) {
    int h[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) h[u] = hist[static_cast<int64_t>(t + u) * E + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      base[static_cast<int64_t>(t + u) * E + e] = run;
      run += h[u];
    }
  }
  for (; t < t_end; ++t) {
    const int64_t i = static_cast<int64_t>(t) * E + e;
    base[i] = run;
    run += hist[i];
  }
  if (p == P - 1) {  // run is now the expert's total over all tiles
    const int f = fill[e];
    fill0[e] = f;
    fill[e] = min(C, f + run);
    if (round == 0 && counts != nullptr) counts[e] = run;
  }
}

__global__ __launch_bounds__(kRrTile) void rr_place_kernel(Order o, int64_t Q, const int32_t* __restrict__ cand,
                                                           int n, int E, int C, const int32_t* __restrict__ col,
                                                           int32_t* __restrict__ served,
                                                           const int32_t* __restrict__ base,
                                                           const int32_t* __restrict__ fill0,
                                                           int32_t* __restrict__ slot) {
  __shared__ unsigned long long mask[1024];
  for (int e = threadIdx.x; e < E; e += kRrTile) mask[e] = 0ull;
  __syncthreads();
  const int i = threadIdx.x;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kRrTile + i;
  int64_t a = 0;
  const int e = offered(o, q, Q, cand, n, col, served, a);
  if (e >= 0) atomicOr(&mask[e], 1ull << i);
  __syncthreads();
  if (e < 0) return;
  const int rank = __popcll(mask[e] & ((1ull << i) - 1ull));
  const int s = fill0[e] + base[static_cast<int64_t>(blockIdx.x) * E + e] + rank;
  slot[a] = s;
  if (s < C) served[a] = col[a];
}

// offsets = exclusive prefix of the final fill (one block, E <= 1024)
__global__ __launch_bounds__(1024) void rr_offsets_kernel(const int32_t* __restrict__ fill, int E,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int s[1024];
  const int e = threadIdx.x;
  const int v = (e < E) ? fill[e] : 0;
  s[e] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (e >= off) ? s[e - off] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e] = s[e] - v;
  if (e == E - 1) offsets[E] = s[e];
}

__global__ __launch_bounds__(256) void rr_finalize_kernel(int64_t T, int k, int n,
                                                          const int32_t* __restrict__ cand,
                                                          const float* __restrict__ cand_gates,
                                                          const int32_t* __restrict__ served,
                                                          const int32_t* __restrict__ slot,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_of,
                                                          int32_t* __restrict__ row_token,
                                                          int32_t* __restrict__ served_ids,
                                                          float* __restrict__ combine_gates) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (a >= T * k) return;
  const int64_t t = a / k;
  const int c = served[a];
  if (c >= 0) {
    const int e = cand[t * n + c];
    const int row = offsets[e] + slot[a];
    row_of[a] = row;
    row_token[row] = static_cast<int32_t>(t);
    if (served_ids != nullptr) served_ids[a] = e;
    if (combine_gates != nullptr) combine_gates[a] = cand_gates[t * n + c];
  } else {
    row_of[a] = -1;
    if (served_ids != nullptr) served_ids[a] = -1;
    if (combine_gates != nullptr) combine_gates[a] = 0.f;
  }
}

unsigned blocks_of(int64_t n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

}  // namespace

int64_t reroute_tiles(int64_t T, int k) { return (T * k + kRrTile - 1) / kRrTile; }

hipError_t launch_dispatch_reroute(const void* x, const int32_t* cand, const float* cand_gates,
                                   int64_t T, int k, int n, int E, int C, bool rank_priority,
                                   int rounds, int row_bytes, const ReroutePlan& ws,
                                   int32_t* counts, int32_t* offsets, int32_t* slot,
                                   int32_t* row_of, int32_t* row_token, int32_t* served_ids,
                                   float* combine_gates, void* x_perm, hipStream_t s) {
  const int64_t Q = T * k;
  const int64_t ntiles = reroute_tiles(T, k);
  const Order o{T, k, rank_priority};
  klaunch(rr_init_kernel, blocks_of(T > E ? T : E, 256), 256, 0, s, T, k, E, ws.col, ws.served,
                                                                ws.next_col, ws.fill);
  for (int j = 0; j <= rounds; ++j) {
    if (j > 0)
      klaunch(rr_advance_kernel, blocks_of(T, 256), 256, 0, s, T, k, n, ws.col, ws.served, ws.next_col);
    klaunch(rr_hist_kernel, static_cast<unsigned>(ntiles), kRrTile, 0, s, o, Q, cand, n, E, ws.col,
                                                                     ws.served, ws.hist);
    klaunch(rr_scan_kernel, 1, 1024, 0, s, ws.hist, static_cast<int>(ntiles), E, C, j, ws.base, ws.fill,
                                      ws.fill0, counts);
    klaunch(rr_place_kernel, static_cast<unsigned>(ntiles), kRrTile, 0, s, o, Q, cand, n, E, C, ws.col,
                                                                      ws.served, ws.base, ws.fill0,
                                                                      slot);
  }
  klaunch(rr_offsets_kernel, 1, 1024, 0, s, ws.fill, E, offsets);
  klaunch(rr_finalize_kernel, blocks_of(Q, 256), 256, 0, s, T, k, n, cand, cand_gates, ws.served, slot,
                                                        offsets, row_of, row_token, served_ids,
                                                        combine_gates);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || x_perm == nullptr) return err;
  return launch_scatter_rows(x, row_of, T, k, row_bytes, x_perm, s);
}

}  // namespace moe
