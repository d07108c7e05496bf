// Capacity-limited dispatch: per-expert counts, prefix sums, first-come slots
// and the permutation of token rows into expert-contiguous buffers.
//
// Page "MoE 模型原理：路由、专家负载、容量、通信与推理成本" (wrblog.cn) §4.2 fixes
// the rule: each expert accepts tokens until its capacity C is used up, later
// tokens overflow, and spare capacity of one expert is not handed to another.
// §5 lists the metadata (expert ids, buffer positions, combine weights); the
// MiniMax gate/communication interview page (mianshidashi.cn, 深入解析 02 and
// 06) names the counting, packing and contiguous-buffer permutation.
//
// slot(t,e) = |{t' < t : e in S_t'}| makes the result unique and the layout
// deterministic, with no atomics deciding an order:
//   1. per 64-token tile, count each expert's tokens (histogram);
//   2. an exclusive prefix over tiles gives each tile its first slot per
//      expert; counts, n_e = min(count_e, C) and offsets follow;
//   3. inside a tile, a 64-bit mask per expert marks the tokens that chose it;
//      popcount of the mask below a token gives its rank in the tile.
// For small problems steps 2 and 3 run in one kernel (each tile block sums
// the histograms it needs itself), which saves a launch.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                   int k, int E, int32_t* __restrict__ hist) {
  __shared__ int h[1024];
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kTileTokens;
  const int nt = static_cast<int>(min<int64_t>(kTileTokens, T - t0));
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < nt * k; p += 256) atomicAdd(&h[ids[t0 * k + p]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[tile * E + e] = h[e];
}

// One block of 1024 threads. Experts are processed in chunks of up to 1024;
// each chunk's experts get 1024/pow2(chunk) segments of consecutive tiles.
// Segment sums -> exclusive prefix over segments -> per-tile bases.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ hist, int ntiles,
                                                    int E, int C, int32_t* __restrict__ base,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int part[1024];
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int ec = min(E - e0, 1024);
    int ecp = 1;
    while (ecp < ec) ecp <<= 1;
    const int segs = 1024 / ecp;
    const int el = tid & (ecp - 1);
    const int seg = tid / ecp;
    const int len = (ntiles + segs - 1) / segs;
    const int tb = min(ntiles, seg * len);
    const int te = min(ntiles, tb + len);
    const int e = e0 + el;
    const bool valid = el < ec;
    int sum = 0;
    if (valid)
      for (int t = tb; t < te; ++t) sum += hist[static_cast<int64_t>(t) * E + e];
    part[tid] = sum;
    __syncthreads();
    if (valid && seg == 0) {
      int run = 0;
      for (int s = 0; s < segs; ++s) {
        const int v = part[s * ecp + el];
        part[s * ecp + el] = run;
        run += v;
      }
      cnt[e] = run;
    }
    __syncthreads();
    if (valid) {
      int run = part[tid];
      for (int t = tb; t < te; ++t) {
        const int64_t i = static_cast<int64_t>(t) * E + e;
        const int v = hist[i];
        base[i] = run;
        run += v;
      }
    }
    __syncthreads();
  }
  // offsets: exclusive prefix of n_e = min(count_e, C) (Hillis-Steele in LDS)
  int v = (tid < E) ? min(cnt[tid], C) : 0;
  part[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  if (tid < E) {
    counts[tid] = cnt[tid];
    offsets[tid + 1] = part[tid];
  }
  if (tid == 0) offsets[0] = 0;
}

// One block per 64-token tile: slots, capacity test, rows.
__global__ __launch_bounds__(256) void permute_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int64_t T, int k, int E, int C,
    int32_t* __restrict__ slot, int32_t* __restrict__ row_of, int32_t* __restrict__ row_token) {
  __shared__ unsigned long long mask[1024];
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kTileTokens;
  const int nt = static_cast<int>(min<int64_t>(kTileTokens, T - t0));
  const int np = nt * k;
  for (int e = threadIdx.x; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  for (int p = threadIdx.x; p < np; p += 256)
    atomicOr(&mask[ids[t0 * k + p]], 1ull << (p / k));
  __syncthreads();
  for (int p = threadIdx.x; p < np; p += 256) {
    const int t = p / k;
    const int e = ids[t0 * k + p];
    const int rank = __popcll(mask[e] & ((1ull << t) - 1ull));
    const int s = base[tile * E + e] + rank;
    const int row = (s < C) ? offsets[e] + s : -1;
    slot[t0 * k + p] = s;
    row_of[t0 * k + p] = row;
    if (row >= 0) row_token[row] = static_cast<int32_t>(t0 + t);
  }
}

// The same, for small problems (ntiles * E <= kFusedScanLimit) without the
// separate scan: every block sums the per-tile histograms itself (the bases of
// its own tile and the totals), then derives n_e = min(count_e, C) and the
// exclusive prefix over experts. All blocks compute identical values; block 0
// writes counts and offsets.
constexpr int kFusedScanLimit = 32768;

// hist has hrows rows of 64 / rpt tokens each (rpt rows per 64-token tile).
// prob_sum (nullable): also the route's mean-probability sums, prob_sum[e] =
// sum over the prows rows of prob_part [prows, E] (one row per route block),
// in the order of prob_reduce_kernel (so the same bits): a layer call then
// needs no launch of its own for them. Each wavefront takes one expert at a
// time; a block-wide tree per expert (eight barriers each) took a decode
// batch's single block from 4.4 to 10.4 µs.
__global__ __launch_bounds__(256) void permute_scan_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ hist, int hrows, int rpt, int64_t T,
    int k, int E, int C, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot, int32_t* __restrict__ row_of, int32_t* __restrict__ row_token,
    const float* __restrict__ prob_part, int prows, float* __restrict__ prob_sum) {
  __shared__ unsigned long long mask[1024];
  __shared__ int s_base[1024];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_part[2][256];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kTileTokens;
  const int nt = static_cast<int>(min<int64_t>(kTileTokens, T - t0));
  const int np = nt * k;
  // s_base[e] = sum of hist[r][e] over the rows r of tiles before this one,
  // s_cnt[e] the sum over all rows. Rows first, first + stride, ...: eight
  // loads are issued before their sums (the loop is bound by load latency;
  // integer sums do not depend on the order).
  const int before = static_cast<int>(tile) * rpt;
  auto tile_sums = [&](int e, int first, int stride, int& b, int& c) {
    int t2 = first;
    for (; t2 + 7 * stride < hrows; t2 += 8 * stride) {
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = hist[static_cast<int64_t>(t2 + u * stride) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (t2 + u * stride < before) b += h[u];
        c += h[u];
      }
    }
    for (; t2 < hrows; t2 += stride) {
      const int h = hist[static_cast<int64_t>(t2) * E + e];
      if (t2 < before) b += h;
      c += h;
    }
  };
  if (256 % E == 0) {
    // E divides 256: read hist flat and coalesced; thread tid always meets
    // expert tid % E, in tiles tid / E, tid / E + 256 / E, ...
    const int P = 256 / E;
    const int e = tid % E;
    int b = 0, c = 0;
    tile_sums(e, tid / E, P, b, c);
    s_part[0][tid] = b;
    s_part[1][tid] = c;
    __syncthreads();
    if (tid < E) {
      b = 0;
      c = 0;
      for (int j = 0; j < P; ++j) {
        b += s_part[0][j * E + tid];
        c += s_part[1][j * E + tid];
      }
      s_base[tid] = b;
      s_cnt[tid] = c;
    }
  } else {
    for (int e = tid; e < E; e += 256) {
      int b = 0, c = 0;
      tile_sums(e, 0, 1, b, c);
      s_base[e] = b;
      s_cnt[e] = c;
    }
  }
  for (int e = tid; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  // kept rows n_e = min(count_e, C); thread tid sums experts 4 tid .. 4 tid + 3,
  // then an exclusive prefix over the 256 partial sums gives the offsets.
  int n_loc[4];
  int part = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    n_loc[j] = (e < E) ? min(s_cnt[e], C) : 0;
    part += n_loc[j];
  }
  s_part[0][tid] = part;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = (tid >= off) ? s_part[0][tid - off] : 0;
    __syncthreads();
    s_part[0][tid] += add;
    __syncthreads();
  }
  int run = s_part[0][tid] - part;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < E) s_off[e] = run;
    run += n_loc[j];
  }
  if (tid == 255) s_off[E] = run;  // the total: experts past E add nothing
  __syncthreads();
  if (tile == 0) {
    for (int e = tid; e < E; e += 256) counts[e] = s_cnt[e];
    for (int e = tid; e <= E; e += 256) offsets[e] = s_off[e];
  }
  for (int p = tid; p < np; p += 256) atomicOr(&mask[ids[t0 * k + p]], 1ull << (p / k));
  __syncthreads();
  for (int p = tid; p < np; p += 256) {
    const int t = p / k;
    const int e = ids[t0 * k + p];
    const int rank = __popcll(mask[e] & ((1ull << t) - 1ull));
    const int sl = s_base[e] + rank;
    const int row = (sl < C) ? s_off[e] + sl : -1;
    slot[t0 * k + p] = sl;
    row_of[t0 * k + p] = row;
    if (row >= 0) row_token[row] = static_cast<int32_t>(t0 + t);
  }
  if (prob_sum != nullptr) {
    // one wavefront per expert, no block barrier. Lane l forms the strided
    // sums of rows l, l+64, l+128, l+192 (each over r, r+256, ...), pairs
    // them as a 256-thread tree's first two levels would and finishes with
    // shuffle steps: the additions of prob_reduce_kernel in its order.
    const int lane = tid & 63;
    const int waves = static_cast<int>(gridDim.x) * 4;
    for (int e = static_cast<int>(blockIdx.x) * 4 + (tid >> 6); e < E; e += waves) {
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      for (int r0 = lane; r0 < prows; r0 += 1024) {
        // a chunk of 1024 rows: all 16 loads issued before the adds; a row
        // past the end adds +0, which leaves these non-negative sums unchanged
        float h[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = r0 + 64 * q + 256 * u;
            h[q][u] = r < prows ? prob_part[static_cast<int64_t>(r) * E + e] : 0.f;
          }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int u = 0; u < 4; ++u) a[q] += h[q][u];
      }
      float v = (a[0] + a[2]) + (a[1] + a[3]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_down(v, off, 64);
      if (lane == 0) prob_sum[e] = v;
    }
  }
}

// x_perm[r] = x[row_token[r]] for every kept row (rows read from offsets[E]
// on the device). One wave copies one row at a time, VEC bytes per lane and
// up to four loads in flight per lane before their stores.
template <int VEC>
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offsets, int E,
                                                          int row_bytes, char* __restrict__ x_perm) {
  typedef typename std::conditional<VEC == 16, uint4, uint32_t>::type V;
  const int64_t rows = offsets[E];
  const int lane = threadIdx.x & 63;
  const int64_t wave = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
  const int chunks = row_bytes / VEC;
  for (int64_t r = wave; r < rows; r += nwaves) {
    const V* src = reinterpret_cast<const V*>(x + static_cast<int64_t>(row_token[r]) * row_bytes);
    V* dst = reinterpret_cast<V*>(x_perm + r * row_bytes);
    int c = lane;
    for (; c + 192 < chunks; c += 256) {
      const V a = src[c], b = src[c + 64], d = src[c + 128], e = src[c + 192];
      dst[c] = a;
      dst[c + 64] = b;
      dst[c + 128] = d;
      dst[c + 192] = e;
    }
    for (; c < chunks; c += 64) dst[c] = src[c];
  }
}

// The same copy token by token: x_perm[row_of[t,j]] = x[t] for every kept
// assignment (t, j). One wave per token reads its row once, up to four
// VEC-byte loads in flight per lane, and writes it to each of its kept rows
// (a token kept by k experts is read once, not k times).
template <int VEC>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const char* __restrict__ x,
                                                           const int32_t* __restrict__ row_of,
                                                           int64_t T, int k, int row_bytes,
                                                           char* __restrict__ x_perm) {
  typedef typename std::conditional<VEC == 16, uint4, uint32_t>::type V;
  const int lane = threadIdx.x & 63;
  const int64_t wave = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
  const int chunks = row_bytes / VEC;
  for (int64_t t = wave; t < T; t += nwaves) {
    // this token's kept rows (wave-uniform loads)
    const int32_t* ro = row_of + t * k;
    bool any = false;
    for (int j = 0; j < k; ++j) any |= ro[j] >= 0;
    if (!any) continue;
    const V* src = reinterpret_cast<const V*>(x + t * row_bytes);
    int c = lane;
    for (; c + 192 < chunks; c += 256) {
      const V a = src[c], b = src[c + 64], d = src[c + 128], e = src[c + 192];
      for (int j = 0; j < k; ++j) {
        const int r = ro[j];
        if (r < 0) continue;
        V* dst = reinterpret_cast<V*>(x_perm + static_cast<int64_t>(r) * row_bytes);
        dst[c] = a;
        dst[c + 64] = b;
        dst[c + 128] = d;
        dst[c + 192] = e;
      }
    }
    for (; c < chunks; c += 64) {
      const V a = src[c];
      for (int j = 0; j < k; ++j) {
        const int r = ro[j];
        if (r >= 0) reinterpret_cast<V*>(x_perm + static_cast<int64_t>(r) * row_bytes)[c] = a;
      }
    }
  }
}

hipError_t launch_hist(const int32_t* ids, int64_t T, int k, int E, int32_t* hist,
                       hipStream_t s) {
  klaunch(hist_kernel, static_cast<unsigned>((T + kTileTokens - 1) / kTileTokens), 256, 0, s, ids, T, k, E, hist);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* hist, int ntiles, int E, int C, int32_t* base,
                       int32_t* counts, int32_t* offsets, hipStream_t s) {
  klaunch(scan_kernel, 1, 1024, 0, s, hist, ntiles, E, C, base, counts, offsets);
  return hipGetLastError();
}

bool fused_scan_fits(int64_t hist_rows, int E) {
  return hist_rows * E <= kFusedScanLimit;
}

hipError_t launch_permute_scan(const void* x, const int32_t* ids, const int32_t* hist, int hist_tokens,
                               int64_t T, int k, int E, int C, int row_bytes, int32_t* counts,
                               int32_t* offsets, int32_t* slot, int32_t* row_of,
                               int32_t* row_token, void* x_perm, const float* prob_part, int prows,
                               float* prob_sum, hipStream_t s) {
  const int ntiles = static_cast<int>((T + kTileTokens - 1) / kTileTokens);
  const int hrows = static_cast<int>((T + hist_tokens - 1) / hist_tokens);
  klaunch(permute_scan_kernel, ntiles, 256, 0, s, ids, hist, hrows, kTileTokens / hist_tokens, T, k, E, C,
          counts, offsets, slot, row_of, row_token, prob_part, prows, prob_sum);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || x_perm == nullptr) return err;
  return launch_scatter_rows(x, row_of, T, k, row_bytes, x_perm, s);
}

hipError_t launch_permute(const void* x, const int32_t* ids, const int32_t* base,
                          const int32_t* offsets, int64_t T, int k, int E, int C,
                          int row_bytes, int32_t* slot, int32_t* row_of, int32_t* row_token,
                          void* x_perm, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((T + kTileTokens - 1) / kTileTokens);
  klaunch(permute_kernel, grid, 256, 0, s, ids, base, offsets, T, k, E, C, slot, row_of, row_token);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || x_perm == nullptr) return err;
  return launch_scatter_rows(x, row_of, T, k, row_bytes, x_perm, s);
}

hipError_t launch_scatter_rows(const void* x, const int32_t* row_of, int64_t T, int k, int row_bytes,
                               void* x_perm, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // one wave per token in flight: enough blocks for every token up to 8 per CU
  const int64_t blocks = (T + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < 2048 ? blocks : 2048);
  if (row_bytes % 16 == 0)
    klaunch(scatter_rows_kernel<16>, grid, 256, 0, s, static_cast<const char*>(x), row_of, T, k, row_bytes,
            static_cast<char*>(x_perm));
  else
    klaunch(scatter_rows_kernel<4>, grid, 256, 0, s, static_cast<const char*>(x), row_of, T, k, row_bytes,
            static_cast<char*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* offsets,
                              int E, int64_t max_rows, int row_bytes, void* x_perm, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  // one wave per row in flight: enough blocks for every row up to 8 per CU
  const int64_t blocks = (max_rows + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < 2048 ? blocks : 2048);
  if (row_bytes % 16 == 0)
    klaunch(gather_rows_kernel<16>, grid, 256, 0, s, static_cast<const char*>(x), row_token, offsets, E,
            row_bytes, static_cast<char*>(x_perm));
  else
    klaunch(gather_rows_kernel<4>, grid, 256, 0, s, static_cast<const char*>(x), row_token, offsets, E,
            row_bytes, static_cast<char*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
