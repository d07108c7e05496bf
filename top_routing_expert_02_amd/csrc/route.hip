// Routing kernels: router scores, softmax, top-k and gates.
//
// Router scores s_t = W_r x_t + b_r, softmax over the E experts, top-k
// selection and renormalised gates follow page "MoE 模型原理：路由、专家负载、
// 容量、通信与推理成本" (wrblog.cn) §2.1 and §2.2. Top-k is taken on the fp32
// logits (softmax is strictly increasing), ids in descending score order,
// equal scores to the lower expert index.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

// ------------------------------------------------------------------ logits (bf16, MFMA)
//
// A block computes a (16*MT tokens) x (16*NT experts) tile of the logits with
// v_mfma_f32_16x16x32_bf16: x rows are the A operand, W_r rows the B operand.
// The four waves split the d axis (wave w takes the 64-wide K steps w, w+4,
// ...); their partial sums meet in LDS and are added in a fixed order.
// The kernel streams x once and re-reads W_r (E*d*2 bytes) from L2 per token
// tile.
//
// Operands pass through a per-wave LDS tile. The MFMA layout gives every
// lane of a quad a different row, and 16-byte loads in that layout touch 16
// cache lines per instruction, half of each: they ran at about a fifth of
// the per-CU load rate. So a wave loads whole lines instead (one instruction
// = 8 rows x 128 bytes, 8 lanes per row), writes them to its own tile of
// 128-byte rows with 16-byte chunks XOR-swizzled by (row / 2) & 7, and
// reads the fragments back conflict-free: in a 64-wide step, MFMA h takes
// k = 32h + 8g .. 32h + 8g + 7 for lane group g. A wave only reads what it
// wrote itself, and one wave's LDS operations run in order, so the tile
// needs no barrier.
//
// A wave keeps P K steps of loads in flight: a ring of P register slots,
// each refilled with the step P further on as soon as it is written to LDS.
// Refills past the wave's last step (when its step count is not a multiple
// of P) re-read that step and are never used. Each wave adds its steps in
// order, so neither P nor the pipelining changes the result. Rows past T
// and experts past E are clamped on load; their outputs are computed and
// never stored.
//
// zero (nullable): nzero ints the top-k kernel that follows accumulates into
// (its per-tile expert histograms), cleared here to save a launch.
template <int MT, int NT>
struct LogitsShape {
  static constexpr int NREG = MT * NT * 4;
  static constexpr int ROWS = 16 * (MT + NT);  // staged rows per wave and step: x rows, then W_r rows
  static constexpr int NLD = ROWS / 8;         // load instructions per step
  static_assert(4 * ROWS * 8 * 16 >= 3 * NREG * 64 * 4, "the partial sums reuse the tiles");
};

// This wave's partial sums of the block tile (tokens t0.., experts e0..)
// over its K steps, in acc; my is its staging tile.
template <int MT, int NT, int P>
__device__ __forceinline__ void logits_accumulate(const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ Wr, int64_t T, int d, int E,
                                                  int64_t t0, int e0,
                                                  u32x4_t (&my)[LogitsShape<MT, NT>::ROWS][8],
                                                  f32x4_t (&acc)[MT][NT]) {
  constexpr int NLD = LogitsShape<MT, NT>::NLD;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // whole-line loads: instruction j, lane l -> staged row 8j + l/8, chunk l%8
  const uint16_t* src[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int r = 8 * j + (lane >> 3);
    if (r < 16 * MT) {
      int64_t t = t0 + r;
      if (t >= T) t = T - 1;
      src[j] = x + t * d + 8 * (lane & 7);
    } else {
      int e = e0 + r - 16 * MT;
      if (e >= E) e = E - 1;
      src[j] = Wr + static_cast<int64_t>(e) * d + 8 * (lane & 7);
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = d >> 6;  // d is a multiple of 64
  const int nw = nsteps > wave ? (nsteps - wave + 3) >> 2 : 0;  // this wave's K steps
  if (nw > 0) {
    const int klast = wave * 64 + (nw - 1) * 256;
    u32x4_t slot[P][NLD];
    auto load = [&](u32x4_t (&v)[NLD], int i) {
      const int k0 = min(wave * 64 + i * 256, klast);
#pragma unroll
      for (int j = 0; j < NLD; ++j) v[j] = *reinterpret_cast<const u32x4_t*>(src[j] + k0);
    };
    auto put = [&](const u32x4_t (&v)[NLD]) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int r = 8 * j + (lane >> 3);
        my[r][(lane & 7) ^ ((r >> 1) & 7)] = v[j];
      }
    };
    // fragments of one half step (32 of the 64 k), double-buffered
    bf16x8_t fa[2][MT], fb[2][NT];
    auto read = [&](bf16x8_t (&a)[MT], bf16x8_t (&b)[NT], int h) {
      const int c = 4 * h + (lane >> 4);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = 16 * mt + (lane & 15);
        a[mt] = __builtin_bit_cast(bf16x8_t, my[r][c ^ ((r >> 1) & 7)]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * (MT + nt) + (lane & 15);
        b[nt] = __builtin_bit_cast(bf16x8_t, my[r][c ^ ((r >> 1) & 7)]);
      }
    };
    auto mma = [&](const bf16x8_t (&a)[MT], const bf16x8_t (&b)[NT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    };
    // Step s sits in ring slot s % P. While the MFMAs of one half step run,
    // the wave reads the next half step's fragments; step s + 1 goes into
    // the tile right behind the last fragment reads of step s. The main
    // loop has no branches (the compiler then counts the ring's loads in
    // flight exactly); the last P steps, whose data is already loaded, run
    // in the tail.
#pragma unroll
    for (int p = 0; p < P; ++p) load(slot[p], p);
    __builtin_amdgcn_sched_barrier(0);
    put(slot[0]);
    load(slot[0], P);
    __builtin_amdgcn_sched_barrier(0);
    read(fa[0], fb[0], 0);
    int s0 = 0;
    for (; s0 + P < nw; s0 += P) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        read(fa[1], fb[1], 1);  // step s0 + q, k 32..63
        mma(fa[0], fb[0]);      // step s0 + q, k 0..31
        put(slot[(q + 1) % P]);  // step s0 + q + 1 replaces step s0 + q in the tile
        load(slot[(q + 1) % P], s0 + q + 1 + P);
        __builtin_amdgcn_sched_barrier(0);
        read(fa[0], fb[0], 0);  // step s0 + q + 1, k 0..31
        mma(fa[1], fb[1]);      // step s0 + q, k 32..63
      }
    }
#pragma unroll
    for (int q = 0; q < P; ++q) {
      if (s0 + q < nw) {
        read(fa[1], fb[1], 1);
        mma(fa[0], fb[0]);
        if (s0 + q + 1 < nw) {
          put(slot[(q + 1) % P]);
          read(fa[0], fb[0], 0);
        }
        mma(fa[1], fb[1]);
      }
    }
  }
}

// Adds the four waves' partial sums in a fixed order: afterwards wave 0's acc
// holds the block tile (the other waves' acc are left as they were). tiles:
// the staging tiles of all waves, reused for the partials.
template <int MT, int NT>
__device__ __forceinline__ void logits_reduce(f32x4_t (&acc)[MT][NT], void* tiles) {
  constexpr int NREG = LogitsShape<MT, NT>::NREG;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // every wave is done with its tile: the partial sums reuse them
  float(&red)[3][NREG][64] = *reinterpret_cast<float(*)[3][NREG][64]>(tiles);
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][(mt * NT + nt) * 4 + i][lane] = acc[mt][nt][i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = (mt * NT + nt) * 4 + i;
          float v = acc[mt][nt][i];
          v += red[0][r][lane];
          v += red[1][r][lane];
          v += red[2][r][lane];
          acc[mt][nt][i] = v;
        }
  }
}

template <int MT, int NT, int P>
__global__ __launch_bounds__(256) void logits_bf16_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ Wr,
                                                          const float* __restrict__ br,
                                                          float* __restrict__ logits, int64_t T,
                                                          int d, int E, int32_t* __restrict__ zero,
                                                          int64_t nzero) {
  if (zero != nullptr) {
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * gridDim.y * 256;
    for (int64_t i = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * 256 + threadIdx.x;
         i < nzero; i += nthreads)
      zero[i] = 0;
  }
  __shared__ u32x4_t tile[4][LogitsShape<MT, NT>::ROWS][8];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * (16 * MT);
  const int e0 = blockIdx.y * (16 * NT);
  f32x4_t acc[MT][NT];
  logits_accumulate<MT, NT, P>(x, Wr, T, d, E, t0, e0, tile[wave], acc);
  logits_reduce<MT, NT>(acc, &tile[0][0][0]);
  if (wave != 0) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = e0 + nt * 16 + (lane & 15);
      const float bias = (br != nullptr && e < E) ? br[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // output layout of the 16x16 MFMA: lane holds rows 4*(lane/16)+i, column lane%16
        const int64_t t = t0 + mt * 16 + (lane >> 4) * 4 + i;
        if (t < T && e < E) logits[t * E + e] = acc[mt][nt][i] + bias;
      }
    }
}

// ------------------------------------------------------------------ logits (fp32)
// One wave per token; lanes split d; one wave-wide sum per expert.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(256) void logits_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ Wr,
                                                         const float* __restrict__ br,
                                                         float* __restrict__ logits, int64_t T,
                                                         int d, int E) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* xt = x + t * d;
  for (int e = 0; e < E; ++e) {
    const float* we = Wr + static_cast<int64_t>(e) * d;
    float s = 0.f;
    for (int m = lane; m < d; m += 64) s = fmaf(xt[m], we[m], s);
    s = wave_sum(s);
    if (lane == 0) logits[t * E + e] = s + (br != nullptr ? br[e] : 0.f);
  }
}

// ------------------------------------------------------------------ top-k, softmax, gates
//
// A block owns TB tokens: a whole 64-token tile, or a quarter of one when
// the layer has too few tiles to fill the chip. A token is handled by a
// group of G lanes (G a power of two, 4 <= G <= 64); lane g of the group
// holds the logits of experts g, g+G, ... (NV of them). A wave holds 64/G
// tokens at a time, and the block has enough waves (up to 16) that it takes
// as few passes as possible: the rounds below are chains of dependent
// cross-lane shuffles, so the kernel is latency-bound and wants many waves
// in flight.
//
// Round r of k picks the group-wide best (largest logit, then lowest index)
// among the experts not yet taken, by an xor butterfly over the group; the
// comparison is a strict total order, so every lane ends with the same
// winner. Lane r of the group keeps the winner of round r.
//
// p_{t,i} = exp(s_{t,i} - m) / sum_j exp(s_{t,j} - m) with m the top logit;
// gates are exp(s - m) of the chosen experts divided by their sum
// (renormalised) or by the full sum (plain softmax probability). Butterfly
// sums add the same two operands on both partner lanes, so every lane holds
// a bit-identical total and reruns are bit-exact.
//
// Side outputs: the expert histogram of each 64-token tile (integer
// atomics, order free: LDS per block, then, for quarter-tile blocks, added
// into the tile's row, which the logits kernel cleared) and sum_t p_{t,i}
// per block (fixed-order sums: lanes, then groups, then waves).
// Exchange with a partner lane inside a group of up to 16 lanes (one DPP
// row) without the LDS: the partner of lane i is i ^ 1 and i ^ 2 (quad
// permutes), i ^ 7 (mirror inside 8 lanes) and i ^ 15 (mirror inside 16)
// for OFF = 1, 2, 4, 8; larger OFF go through ds_bpermute as i ^ OFF. The
// masks 1, 2, 7, 15 are linearly independent over GF(2), so the four steps,
// in any order, combine every lane of a 16-lane group exactly once, as the
// xor butterfly 1, 2, 4, 8 does. Every lane of the wave must be active.
template <int OFF>
__device__ __forceinline__ int grp_xchg(int v) {
  if constexpr (OFF == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);       // quad_perm 1,0,3,2
  else if constexpr (OFF == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
  else if constexpr (OFF == 4) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true); // row_half_mirror
  else if constexpr (OFF == 8) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true); // row_mirror
  else return __shfl_xor(v, OFF, 64);
}
template <int OFF>
__device__ __forceinline__ float grp_xchg(float v) {
  return __builtin_bit_cast(float, grp_xchg<OFF>(__builtin_bit_cast(int, v)));
}
// (v, i) replaces (bv, bi) when ok and it ranks higher: the larger value,
// the lower index on a tie. Bitwise tests and selects, no branches: the
// exec-mask code the compiler makes for short-circuit tests cost several
// times the comparisons themselves (the skewed layer's selection ran about
// 1300 cycles per round that way).
__device__ __forceinline__ void keep_better(float v, int i, bool ok, float& bv, int& bi) {
  const bool take = ok & ((v > bv) | ((v == bv) & (i < bi)));
  bv = take ? v : bv;
  bi = take ? i : bi;
}

// step(integral_constant<OFF>) for OFF = G/2, G/4, ..., 1
template <int G, typename F>
__device__ __forceinline__ void grp_steps(F&& step) {
  if constexpr (G >= 64) step(std::integral_constant<int, 32>{});
  if constexpr (G >= 32) step(std::integral_constant<int, 16>{});
  if constexpr (G >= 16) step(std::integral_constant<int, 8>{});
  if constexpr (G >= 8) step(std::integral_constant<int, 4>{});
  if constexpr (G >= 4) step(std::integral_constant<int, 2>{});
  if constexpr (G >= 2) step(std::integral_constant<int, 1>{});
}

// One token's selection by its group of G lanes: v holds lane gl's logits
// of experts gl, gl + G, ... (bit j of `invalid` set where there is no
// expert or no token). Returns the lane's pick (round gl < nsel) and its
// gate, and each logit's exp(s - m) with their group-wide sum se (for the
// probabilities).
template <int G, int NV>
__device__ __forceinline__ void token_topk(const float (&v)[NV], uint32_t invalid, int gl, int E, int k,
                                           int nsel, int renormalize, int& my_id, float& my_gate,
                                           float (&ex)[NV], float& se) {
  uint32_t taken = invalid;
  float my_v = 0.f, top = 0.f;
  my_id = -1;
  for (int r = 0; r < nsel; ++r) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NV; ++j) keep_better(v[j], gl + j * G, !((taken >> j) & 1u), bv, bi);
    grp_steps<G>([&](auto o) {
      constexpr int OFF = decltype(o)::value;
      keep_better(grp_xchg<OFF>(bv), grp_xchg<OFF>(bi), true, bv, bi);
    });
    if (r == 0) top = bv;
    taken |= (((bi & (G - 1)) == gl) & (bi < E)) ? (1u << (bi / G)) : 0u;
    const bool mine_r = gl == r;
    my_v = mine_r ? bv : my_v;
    my_id = mine_r ? bi : my_id;
  }
  // softmax denominator
  se = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    ex[j] = ((invalid >> j) & 1u) ? 0.f : __expf(v[j] - top);
    se += ex[j];
  }
  grp_steps<G>([&](auto o) { se += grp_xchg<decltype(o)::value>(se); });
  const float mine = (gl < nsel) ? __expf(my_v - top) : 0.f;
  float den = se;
  if (renormalize) {
    den = (gl < k) ? mine : 0.f;  // the top-k sum, also for later candidates
    grp_steps<G>([&](auto o) { den += grp_xchg<decltype(o)::value>(den); });
  }
  my_gate = mine / den;
}

template <int G, int NV, int WAVES, int TB>
__global__ __launch_bounds__(64 * WAVES) void topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int E, int k, int nsel, int renormalize,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ gates,
                                                   float* __restrict__ prob_part,
                                                   int32_t* __restrict__ hist) {
  constexpr int TPW = 64 / G;                 // tokens per wave pass
  constexpr int PASSES = TB / (TPW * WAVES);  // passes per wave
  static_assert(TPW * WAVES * PASSES == TB, "TB tokens per block");
  static_assert(TB == 64 || TB == 16, "whole or quarter tiles");
  constexpr int NT = 64 * WAVES;              // threads
  __shared__ float s_prob[WAVES][1024];
  __shared__ int s_hist[1024];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane & (G - 1);   // lane inside the group
  const int grp = lane / G;        // group inside the wave
  const int64_t tile = blockIdx.x;
  const bool want_prob = prob_part != nullptr;
  const bool want_hist = hist != nullptr;

  if (want_hist)
    for (int e = threadIdx.x; e < E; e += NT) s_hist[e] = 0;
  __syncthreads();

  float psum[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) psum[j] = 0.f;

  for (int pass = 0; pass < PASSES; ++pass) {
    const int64_t t = tile * TB + (wave * PASSES + pass) * TPW + grp;
    const bool tv = t < T;
    const float* row = logits + (tv ? t : 0) * E;
    float v[NV];
    uint32_t invalid = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = gl + j * G;
      if (e < E && tv) {
        v[j] = row[e];
      } else {
        v[j] = 0.f;
        invalid |= 1u << j;  // not an expert: never chosen, not summed
      }
    }
    int my_id;
    float my_gate, ex[NV], se;
    token_topk<G, NV>(v, invalid, gl, E, k, nsel, renormalize, my_id, my_gate, ex, se);
    if (tv && gl < nsel) {
      ids[t * nsel + gl] = my_id;
      gates[t * nsel + gl] = my_gate;
      if (want_hist && gl < k) atomicAdd(&s_hist[my_id], 1);
    }
    if (want_prob && tv) {
      const float inv = 1.0f / se;
#pragma unroll
      for (int j = 0; j < NV; ++j) psum[j] += ex[j] * inv;
    }
  }

  if (want_prob) {
    // groups of the wave hold the same experts for different tokens
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int off = G; off < 64; off <<= 1) psum[j] += __shfl_xor(psum[j], off, 64);
    if (grp == 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int e = gl + j * G;
        if (e < E) s_prob[wave][e] = psum[j];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NT) {
    if (want_prob) {
      float sum = s_prob[0][e];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += s_prob[w][e];  // fixed order
      prob_part[tile * E + e] = sum;
    }
    if (want_hist) {
      if constexpr (TB == 64) hist[tile * E + e] = s_hist[e];
      else if (s_hist[e] != 0) atomicAdd(&hist[(tile * TB / 64) * E + e], s_hist[e]);
    }
  }
}

// ------------------------------------------------------------------ fused route (E <= 64)
//
// Router logits, softmax, top-k, gates and the block's expert histogram in
// one launch, for layers whose experts fit one logits tile (E <= 16 NT). A
// block computes its 16 MT tokens x all experts with the MFMA K loop above;
// the sums go to LDS instead of HBM, and the 256 threads then select per
// token as topk_kernel does (G lanes per token). Side outputs per block:
// the histogram row of its tokens' first k choices (rows of 16 MT tokens,
// plain stores) and its probability sums (fixed order: lanes, groups,
// waves), which prob_reduce adds in block order.
template <int MT, int NT, int P, int G, int NV>
__global__ __launch_bounds__(256) void route_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wr, const float* __restrict__ br,
    int64_t T, int d, int E, int k, int nsel, int renormalize, int32_t* __restrict__ ids,
    float* __restrict__ gates, float* __restrict__ prob_part, int32_t* __restrict__ hist) {
  constexpr int TB = 16 * MT;       // tokens per block
  constexpr int NE = 16 * NT;       // experts of the tile (E <= NE)
  constexpr int TPW = 64 / G;       // tokens per wave pass
  constexpr int PASSES = TB / (TPW * 4) > 0 ? TB / (TPW * 4) : 1;
  __shared__ u32x4_t tile[4][LogitsShape<MT, NT>::ROWS][8];
  __shared__ float s_log[TB][NE + 1];
  __shared__ float s_prob[4][NE];
  __shared__ int s_hist[NE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;

  f32x4_t acc[MT][NT];
  logits_accumulate<MT, NT, P>(x, Wr, T, d, E, t0, 0, tile[wave], acc);
  logits_reduce<MT, NT>(acc, &tile[0][0][0]);
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = nt * 16 + (lane & 15);
        const float bias = (br != nullptr && e < E) ? br[e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s_log[mt * 16 + (lane >> 4) * 4 + i][e] = acc[mt][nt][i] + bias;
      }
  }
  if (tid < NE) s_hist[tid] = 0;
  __syncthreads();

  const int gl = lane & (G - 1);
  const int grp = lane / G;
  float psum[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) psum[j] = 0.f;
  for (int pass = 0; pass < PASSES; ++pass) {
    const int tl = (wave * PASSES + pass) * TPW + grp;  // token within the block
    const int64_t t = t0 + tl;
    const bool tv = tl < TB && t < T;
    float v[NV];
    uint32_t invalid = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = gl + j * G;
      if (e < E && tv) {
        v[j] = s_log[tl][e];
      } else {
        v[j] = 0.f;
        invalid |= 1u << j;
      }
    }
    int my_id;
    float my_gate, ex[NV], se;
    token_topk<G, NV>(v, invalid, gl, E, k, nsel, renormalize, my_id, my_gate, ex, se);
    if (tv && gl < nsel) {
      ids[t * nsel + gl] = my_id;
      gates[t * nsel + gl] = my_gate;
      if (hist != nullptr && gl < k) atomicAdd(&s_hist[my_id], 1);
    }
    if (prob_part != nullptr && tv) {
      const float inv = 1.0f / se;
#pragma unroll
      for (int j = 0; j < NV; ++j) psum[j] += ex[j] * inv;
    }
  }
  if (prob_part != nullptr) {
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int off = G; off < 64; off <<= 1) psum[j] += __shfl_xor(psum[j], off, 64);
    if (grp == 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int e = gl + j * G;
        if (e < NE) s_prob[wave][e] = psum[j];
      }
    }
  }
  __syncthreads();
  if (tid < E) {
    if (prob_part != nullptr)
      prob_part[static_cast<int64_t>(blockIdx.x) * E + tid] =
          ((s_prob[0][tid] + s_prob[1][tid]) + s_prob[2][tid]) + s_prob[3][tid];
    if (hist != nullptr) hist[static_cast<int64_t>(blockIdx.x) * E + tid] = s_hist[tid];
  }
}

// One block per expert: thread i adds tiles i, i + 256, ... in order, then a
// fixed tree over the threads (the result is bit-reproducible).
__global__ __launch_bounds__(256) void prob_reduce_kernel(const float* __restrict__ part,
                                                          int ntiles, int E,
                                                          float* __restrict__ out) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int t = tid; t < ntiles; t += 256) s += part[static_cast<int64_t>(t) * E + e];
  red[tid] = s;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  if (tid == 0) out[e] = red[0];
}

// ------------------------------------------------------------------ launchers

hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* Wr, const float* br,
                              float* logits, int64_t T, int d, int E, int32_t* zero, int64_t nzero,
                              hipStream_t s) {
  // tiles: 16 tokens x all of E up to 64 experts (32 tokens once that still
  // gives 256 blocks), 64 x 64 beyond; the ring depth P keeps 32-48 KiB of
  // loads in flight per wave
  if (E <= 16) {
    dim3 grid(static_cast<unsigned>((T + 15) / 16), 1);
    klaunch(logits_bf16_kernel<1, 1, 4>, grid, 256, 0, s, x, Wr, br, logits, T, d, E, zero, nzero);
  } else if (E <= 32) {
    dim3 grid(static_cast<unsigned>((T + 15) / 16), 1);
    klaunch(logits_bf16_kernel<1, 2, 4>, grid, 256, 0, s, x, Wr, br, logits, T, d, E, zero, nzero);
  } else if (E <= 64 && T >= 32 * 256) {
    dim3 grid(static_cast<unsigned>((T + 31) / 32), 1);
    klaunch(logits_bf16_kernel<2, 4, 3>, grid, 256, 0, s, x, Wr, br, logits, T, d, E, zero, nzero);
  } else if (E <= 64) {
    dim3 grid(static_cast<unsigned>((T + 15) / 16), 1);
    klaunch(logits_bf16_kernel<1, 4, 4>, grid, 256, 0, s, x, Wr, br, logits, T, d, E, zero, nzero);
  } else {
    dim3 grid(static_cast<unsigned>((T + 63) / 64), static_cast<unsigned>((E + 63) / 64));
    klaunch(logits_bf16_kernel<4, 4, 3>, grid, 256, 0, s, x, Wr, br, logits, T, d, E, zero, nzero);
  }
  return hipGetLastError();
}

int route_fused_tokens(int64_t T, int E) {
  if (E > 64) return 0;
  return (E > 32 && T >= 32 * 256) ? 32 : 16;
}

hipError_t launch_route_fused_bf16(const uint16_t* x, const uint16_t* Wr, const float* br, int64_t T, int d,
                                   int E, int k, int nsel, int renormalize, int32_t* ids, float* gates,
                                   float* prob_part, int32_t* hist, hipStream_t s) {
  const int tb = route_fused_tokens(T, E);
  const dim3 grid(static_cast<unsigned>((T + tb - 1) / tb));
  // tile shapes and ring depths as the logits kernel; G lanes per token
  if (E <= 8)
    klaunch(route_fused_bf16_kernel<1, 1, 4, 8, 1>, grid, 256, 0, s, x, Wr, br, T, d, E, k, nsel, renormalize,
            ids, gates, prob_part, hist);
  else if (E <= 16)
    klaunch(route_fused_bf16_kernel<1, 1, 4, 16, 1>, grid, 256, 0, s, x, Wr, br, T, d, E, k, nsel,
            renormalize, ids, gates, prob_part, hist);
  else if (E <= 32)
    klaunch(route_fused_bf16_kernel<1, 2, 4, 16, 2>, grid, 256, 0, s, x, Wr, br, T, d, E, k, nsel,
            renormalize, ids, gates, prob_part, hist);
  else if (tb == 32)
    klaunch(route_fused_bf16_kernel<2, 4, 3, 16, 4>, grid, 256, 0, s, x, Wr, br, T, d, E, k, nsel,
            renormalize, ids, gates, prob_part, hist);
  else
    klaunch(route_fused_bf16_kernel<1, 4, 4, 16, 4>, grid, 256, 0, s, x, Wr, br, T, d, E, k, nsel,
            renormalize, ids, gates, prob_part, hist);
  return hipGetLastError();
}

hipError_t launch_logits_f32(const float* x, const float* Wr, const float* br, float* logits,
                             int64_t T, int d, int E, hipStream_t s) {
  klaunch(logits_f32_kernel, static_cast<unsigned>((T + 3) / 4), 256, 0, s, x, Wr, br, logits, T, d, E);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int nsel, int renormalize,
                       int32_t* ids, float* gates, float* prob_part, int32_t* hist, int tb,
                       hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((T + tb - 1) / tb);
  // whole tiles: up to 16 waves; quarter tiles: G/4 waves, one pass
#define MOE_TOPK(G, NV)                                                                           \
  do {                                                                                            \
    if (tb == 64)                                                                                 \
      klaunch(topk_kernel<G, NV, (G >= 16 ? 16 : G), 64>, grid, 64 * (G >= 16 ? 16 : G), 0, s,    \
              logits, T, E, k, nsel, renormalize, ids, gates, prob_part, hist);                   \
    else                                                                                          \
      klaunch(topk_kernel<G, NV, G / 4, 16>, grid, 16 * G, 0, s, logits, T, E, k, nsel,          \
              renormalize, ids, gates, prob_part, hist);                                          \
  } while (0)
  // groups of at least 16 lanes (k <= 16 results per token) holding up to 16
  // logits per lane: a wave runs 4 tokens' shuffle chains side by side, and
  // each round's butterfly has at most 4 levels below 256 experts
  if (E <= 4) MOE_TOPK(4, 1);
  else if (E <= 8) MOE_TOPK(8, 1);
  else if (E <= 16) MOE_TOPK(16, 1);
  else if (E <= 32) MOE_TOPK(16, 2);
  else if (E <= 64) MOE_TOPK(16, 4);
  else if (E <= 128) MOE_TOPK(16, 8);
  else if (E <= 256) MOE_TOPK(16, 16);
  else if (E <= 512) MOE_TOPK(32, 16);
  else MOE_TOPK(64, 16);
#undef MOE_TOPK
  return hipGetLastError();
}

hipError_t launch_prob_reduce(const float* part, int ntiles, int E, float* out, hipStream_t s) {
  klaunch(prob_reduce_kernel, E, 256, 0, s, part, ntiles, E, out);
  return hipGetLastError();
}

}  // namespace moe
