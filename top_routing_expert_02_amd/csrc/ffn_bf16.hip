// Grouped expert GEMMs for bf16 layers on gfx950 matrix cores.
//
// The expert FFN, FFN(x) = W2 sigma(W1 x + b1) + b2 (page "MoE 模型原理：路由、
// 专家负载、容量、通信与推理成本", wrblog.cn, §1), runs over the expert-
// contiguous rows as one grouped GEMM per layer: every expert is a group with
// its own row count (the "batched or grouped GEMM" of the MiniMax gate /
// communication interview page, mianshidashi.cn, and of page "Expert
// Parallelism：为什么让 Token 去找 Expert，而不是搬运参数？", section "Dropless
// MoE": groups of different M in one launch).
//
//   out[r, n] = epilogue( sum_k A[r, k] * W[e, n, k] + bias[e, n] ),  r in expert e's rows
//
// Both operands are K-contiguous (A row-major [rows, K]; W[e] row-major [N, K]).
//
// Design (gfx950, wave64, 160 KiB LDS per CU):
//  * Block tile BM tokens x BN=256 features with BM = 256, 192, 128 or 64;
//    four waves in a 2x2 grid; each wave owns BM/2 tokens x 128 features as 32x32
//    v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulators in AGPRs. The
//    weight tile is the MFMA A operand and the token tile the B operand, so a
//    lane's accumulators hold 4 consecutive features of one token: the
//    epilogue stores 8-byte (bf16) or 16-byte (fp32) vectors.
//  * The tile height is chosen on the device, per launch, from the actual
//    expert row counts (the cost model is at the schedule below): a group
//    count that leaves a mostly idle last round of 256-row tiles runs as
//    192-row tiles, and experts with a few dozen rows (decode batches) run
//    64-row tiles, which stream the same weights with a quarter of the
//    MFMAs. The host never learns the row counts.
//  * K advances in stages of BK=64: every LDS row is 128 bytes, one full
//    cache line of the source row, so each L1->L2 request moves a whole line.
//    The 16-byte chunks of a row are XOR-swizzled by (row/2)&7, which keeps
//    the fragment reads (16 lanes = 16 rows at one chunk) on distinct banks.
//  * Tiles move global -> LDS with gfx950's LDS-DMA loads
//    (global_load_lds_dwordx4: no staging registers, no ds_write); one
//    instruction fills 8 rows (1 KiB); each lane fetches the chunk that the
//    swizzle places at its LDS slot.
//  * Two stage buffers (three for tiles of 128 or 64 rows). A stage is four K16 steps; each step's MFMAs run with
//    the next step's fragment reads in flight, and the buffer a stage occupied
//    is refilled (with the stage after next) right after the barrier that
//    shows every wave has read it: half of the loads between the MFMAs of
//    that stage's last step, the other half between those of the next
//    stage's first step (a whole stage's loads at once back up the load
//    queue, and the wave stalls at an MFMA issue slot). The next tile's first
//    stages, and its bias slice, load during the current tile's last step and
//    epilogue.
//  * Persistent blocks, one per CU. The schedule is computed on the device
//    from expert_offsets (no host read-back): expert-major tiles, M tiles of
//    an expert innermost, so concurrent tiles share weight panels. Blocks are
//    renumbered so that consecutive tiles run on one XCD (blocks are dealt to
//    the 8 XCDs round-robin) and share its L2.
//  * Ragged M: rows past an expert's end read that expert's last row and are
//    never stored, so no tile reads outside [0, rows).
#include "moe_internal.h"

#include <hip/hip_ext.h>

#include <type_traits>

namespace moe {

namespace {

constexpr int BN = 256;       // features per tile
constexpr int BK = 64;        // K per LDS stage
constexpr int ROWB = BK * 2;  // bytes per LDS row (128)
constexpr int kWtRowB = BN * 2;  // bytes per row of a K-major weight stage (512)
// stage buffers: two for the 256- and 192-row tiles, three for the shorter
// ones (a tile of few rows streams weights, so more bytes in flight pay)
template <int TM>
constexpr int stages_for() { return TM <= 2 ? 3 : 2; }  // wait_loads allows at most 3
constexpr int kLdsBytes = 3 * (128 + BN) * ROWB;  // the largest of NST (BM + BN) rows
constexpr int TN = 4;         // 32-feature MFMA tiles per wave
constexpr int WN = BN / 2;    // features per wave
static_assert(kGemmBM == 256, "the taller of the two tile heights");

// Row r of a stage holds its 16-byte chunk c at position c ^ swz_key(r).
// A fragment read covers 32 rows at one chunk; the LDS serves 16 lanes per
// cycle, and with this key the 16 rows of a group land on 16 distinct
// 4-bank groups (rows 2j and 2j+1 differ in the bank half, rows 2j at j =
// 0..7 differ in the chunk position).
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }

// ---- hand-scheduled inline-asm blocks (mfma_steps.inc, generated)
//
// The matrix core holds one MFMA behind the one executing (32 cycles each
// for 32x32x16), so any other instruction a wave issues is free only while it
// fits in that shadow: a run of LDS reads issued before the MFMAs leaves the
// core idle. Each K16 step block therefore issues one fragment read (and, in
// the refill step, one or two LDS-DMA loads) after each MFMA. The compiler
// cannot place them there: its wait insertion treats any LDS read as
// dependent on every LDS-DMA load in flight and waits for all of them, which
// would serialise the stage pipeline. A block reads the next K16 step's
// fragments and waits for them before it ends: no read is in flight past a
// block. Stage order is explicit (wait_loads and a barrier before a stage is
// read).
//   acc[i][j] += W_i * T_j: W = weight fragments (MFMA A operand),
//   T = token fragments (B operand); next fragments from ta / wa, the 32-row
//   fragment tiles 4096 B apart.
// LDS-DMA loads take their LDS destination from M0 (lane L writes bytes
// 16L..16L+15 of a 1 KiB block); an instruction sits between each M0 write
// and the load that uses it. M0 is reserved by the compiler; the clobber
// orders its own uses against these blocks. The M0 sums also write SCC, which
// the compiler may hold a comparison in across a block: it is clobbered
// too. Every LDS-DMA load of this kernel
// is issued from asm, so the compiler tracks none of them: it would otherwise
// wait for all of them before reusing an address register or reading any
// LDS, which would stall each epilogue on the next tile's prefetch.
typedef short v4i16 __attribute__((ext_vector_type(4)));
#include "mfma_steps.inc"

template <int TM>
__device__ __forceinline__ void step(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                     const bf16x8_t (&t)[TM], bf16x8_t (&nw)[TN], bf16x8_t (&nt)[TM],
                                     uint32_t ta, uint32_t wa) {
  if constexpr (TM == 4) step_4x4(acc, w, t, nw, nt, ta, wa);
  else if constexpr (TM == 3) step_3x4(acc, w, t, nw, nt, ta, wa);
  else if constexpr (TM == 2) step_2x4(acc, w, t, nw, nt, ta, wa);
  else step_1x4(acc, w, t, nw, nt, ta, wa);
}

// HALF 0: the first half of a stage's LDS-DMA loads, 1: the rest
template <int TM, int HALF>
__device__ __forceinline__ void step_dma(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                         const bf16x8_t (&t)[TM], bf16x8_t (&nw)[TN],
                                         bf16x8_t (&nt)[TM], uint32_t ta, uint32_t wa,
                                         const uint32_t (&vo)[2 * TM + 2 * TN], uint32_t la, uint32_t lb,
                                         const char* ga, const char* gw) {
  if constexpr (HALF == 0) {
    if constexpr (TM == 4) step_dma0_4x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 3) step_dma0_3x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 2) step_dma0_2x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
    else step_dma0_1x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
  } else {
    if constexpr (TM == 4) step_dma1_4x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 3) step_dma1_3x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 2) step_dma1_2x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
    else step_dma1_1x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
  }
}

template <int TM>
__device__ __forceinline__ void last_step(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                          const bf16x8_t (&t)[TM]) {
  if constexpr (TM == 4) last_4x4(acc, w, t);
  else if constexpr (TM == 3) last_3x4(acc, w, t);
  else if constexpr (TM == 2) last_2x4(acc, w, t);
  else last_1x4(acc, w, t);
}

template <int TM>
__device__ __forceinline__ void read_frags(bf16x8_t (&nw)[TN], bf16x8_t (&nt)[TM], uint32_t ta,
                                           uint32_t wa) {
  if constexpr (TM == 4) frags_4x4(nw, nt, ta, wa);
  else if constexpr (TM == 3) frags_3x4(nw, nt, ta, wa);
  else if constexpr (TM == 2) frags_2x4(nw, nt, ta, wa);
  else frags_1x4(nw, nt, ta, wa);
}

// The same steps for a K-major weight stage (WT): the next weight fragments
// arrive as 64-bit halves (k 0..3 and 4..7 of each lane's 8), joined here.
__device__ __forceinline__ void join_halves(bf16x8_t (&nw)[TN], const v4i16 (&lo)[TN],
                                            const v4i16 (&hi)[TN]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
    nw[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo[i], hi[i], 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int TM>
__device__ __forceinline__ void step_t(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                       const bf16x8_t (&t)[TM], bf16x8_t (&nw)[TN], bf16x8_t (&nt)[TM],
                                       uint32_t ta, const uint32_t (&wa)[TN]) {
  v4i16 lo[TN], hi[TN];
  if constexpr (TM == 4) step_t_4x4(acc, w, t, nt, lo, hi, ta, wa);
  else if constexpr (TM == 3) step_t_3x4(acc, w, t, nt, lo, hi, ta, wa);
  else if constexpr (TM == 2) step_t_2x4(acc, w, t, nt, lo, hi, ta, wa);
  else step_t_1x4(acc, w, t, nt, lo, hi, ta, wa);
  join_halves(nw, lo, hi);
}

template <int TM, int HALF>
__device__ __forceinline__ void step_dma_t(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                           const bf16x8_t (&t)[TM], bf16x8_t (&nw)[TN],
                                           bf16x8_t (&nt)[TM], uint32_t ta, const uint32_t (&wa)[TN],
                                           const uint32_t (&vo)[2 * TM + 2 * TN], uint32_t la,
                                           uint32_t lb, const char* ga, const char* gw) {
  v4i16 lo[TN], hi[TN];
  if constexpr (HALF == 0) {
    if constexpr (TM == 4) step_dma0_t_4x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 3) step_dma0_t_3x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 2) step_dma0_t_2x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
    else step_dma0_t_1x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
  } else {
    if constexpr (TM == 4) step_dma1_t_4x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 3) step_dma1_t_3x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
    else if constexpr (TM == 2) step_dma1_t_2x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
    else step_dma1_t_1x4(acc, w, t, nt, lo, hi, ta, wa, vo, la, lb, ga, gw);
  }
  join_halves(nw, lo, hi);
}

template <int TM>
__device__ __forceinline__ void read_frags_t(bf16x8_t (&nw)[TN], bf16x8_t (&nt)[TM], uint32_t ta,
                                             const uint32_t (&wa)[TN]) {
  v4i16 lo[TN], hi[TN];
  if constexpr (TM == 4) frags_t_4x4(nt, lo, hi, ta, wa);
  else if constexpr (TM == 3) frags_t_3x4(nt, lo, hi, ta, wa);
  else if constexpr (TM == 2) frags_t_2x4(nt, lo, hi, ta, wa);
  else frags_t_1x4(nt, lo, hi, ta, wa);
  join_halves(nw, lo, hi);
}

template <int TM>
__device__ __forceinline__ void issue_stage(const uint32_t (&ao)[2 * TM], const uint32_t (&bo)[2 * TN],
                                            uint32_t la, uint32_t lb, const char* ga, const char* gw) {
  if constexpr (TM == 4) stage_4x4(ao, bo, la, lb, ga, gw);
  else if constexpr (TM == 3) stage_3x4(ao, bo, la, lb, ga, gw);
  else if constexpr (TM == 2) stage_2x4(ao, bo, la, lb, ga, gw);
  else stage_1x4(ao, bo, la, lb, ga, gw);
}

// The tile's bias slice (BN fp32 values, 1 KiB) goes to LDS with the tile's
// first stage: lane L loads features n0 + 4L .. n0 + 4L + 3 (clamped into
// [0, N); a clamped slot duplicates a value that is never stored).
__device__ __forceinline__ void issue_bias(const float* gsrc, uint32_t lds_dst) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gsrc), "s"(lds_dst)
      : "memory", "m0");
#pragma clang diagnostic pop
}

template <int ACT>
__device__ __forceinline__ float activate(float v) {
  if constexpr (ACT == kActRelu) return v > 0.f ? v : 0.f;
  else if constexpr (ACT == kActGeluTanh) return act_gelu_tanh_fast(v);
  else return v;
}

// One output tile: expert e, output rows [row0, row0 + rv) (rv valid of the
// tile's height), features from n0; operand A's first row arow and K range
// [k0, k0 + 64 nk); part: which K half (split launches write the second half's
// partial sums to their own buffer).
struct TileInfo {
  int e, row0, rv, n0, arow, k0, nk, part;
};

// Epilogue cost of an fp32 output tile in K-equivalents (its stores take
// about as long as 512 more K per row of MFMA work); weighs a K split, which
// doubles the stores, against the rounds it saves.
constexpr int kEpiK = 512;

constexpr int kGroupM = 4;  // M tiles per group of the tile order

// s_tiles[e]: exclusive prefix over experts of their M tiles of height BM;
// ntiles output tiles, each in K parts of nk stages (unit u covers tile
// u mod ntiles, part u / ntiles; at most two parts).
__device__ __forceinline__ TileInfo decode_tile(int u, const int* s_tiles, const int32_t* offsets,
                                                int E, int NT, int BM, int nk, int ntiles) {
  const int part = u >= ntiles ? 1 : 0;
  const int tile = u - part * ntiles;
  // expert: the largest e with s_tiles[e] * NT <= tile (experts with no
  // rows share their successor's prefix and are skipped)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tiles[mid] * NT <= tile) lo = mid;
    else hi = mid - 1;
  }
  TileInfo t;
  t.e = lo;
  const int mte = s_tiles[lo + 1] - s_tiles[lo];
  const int v = tile - s_tiles[lo] * NT;
  // grouped order inside an expert with many M tiles: groups of kGroupM M
  // tiles, each swept over all N tiles with its M tiles innermost, so the 32
  // consecutive tiles one XCD runs at a time share 4 token panels and 8
  // weight panels; up to 8 M tiles form one group (every weight panel is
  // then read once per expert)
  const int GM = mte <= 2 * kGroupM ? mte : kGroupM;
  const int g = v / (GM * NT);
  const int r = v - g * GM * NT;
  const int gm = min(GM, mte - g * GM);
  const int nt = r / gm;
  const int mt = g * kGroupM + (r - nt * gm);
  t.row0 = offsets[lo] + mt * BM;
  t.rv = min(BM, offsets[lo + 1] - t.row0);
  t.n0 = nt * BN;
  t.arow = t.row0;
  t.k0 = part * nk * BK;
  t.nk = nk;
  t.part = part;
  return t;
}

// Weight-gradient tiles: C[e] [M, N] = A_e^T B_e where the operands come
// transposed (A^T [M, lda], B^T [N, lda]) with expert e's rows padded to a
// multiple of 64 at columns [poff[e], poff[e+1]). s_tiles[e]: prefix of the
// experts' M tiles (MT for an expert with rows, 0 without); M tiles inner.
__device__ __forceinline__ TileInfo decode_tile_wg(int tile, const int* s_tiles,
                                                   const int32_t* poff, int E, int NT, int BM,
                                                   int M) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tiles[mid] * NT <= tile) lo = mid;
    else hi = mid - 1;
  }
  TileInfo t;
  t.e = lo;
  const int mte = s_tiles[lo + 1] - s_tiles[lo];
  const int u = tile - s_tiles[lo] * NT;
  // the grouped order of decode_tile
  const int GM = mte <= 2 * kGroupM ? mte : kGroupM;
  const int g = u / (GM * NT);
  const int r = u - g * GM * NT;
  const int gm = min(GM, mte - g * GM);
  const int nt = r / gm;
  const int mt = g * GM + (r - nt * gm);
  t.arow = mt * BM;
  t.row0 = lo * M + t.arow;  // C viewed as [E*M, N]
  t.rv = min(BM, M - t.arow);
  t.n0 = nt * BN;
  t.k0 = poff[lo];
  t.nk = (poff[lo + 1] - poff[lo]) / BK;
  t.part = 0;
  return t;
}

// Wait until the stage awaited has landed, with n (0 or 1) later stages of
// G loads each still allowed in flight (at most three stage buffers).
template <int G>
__device__ __forceinline__ void wait_loads(int n) {
  if (n >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(G) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Per-tile DMA sources: byte offsets (from the tile's token and weight bases)
// of the chunk each lane loads for every 1 KiB block it fills (lane L lands
// at row L/8, position L%8 of its block). Token rows past the expert's end
// read its last row; feature rows past N read row N-1. With row_idx, tile row
// r is row row_idx[row0 + r] of A (the token rows are gathered straight from
// x, so the permuted copy is never written).
// lda: elements between consecutive rows of A and of W (K for the expert
// FFN); w_estride: elements between experts' weight matrices (0 when W is
// one matrix).
template <int LA, int LB, bool WT>
__device__ __forceinline__ void tile_sources(const TileInfo& t, const uint16_t* A,
                                             const int32_t* __restrict__ row_idx, const uint16_t* W,
                                             int N, int lda, int64_t w_estride, int wave, int drow,
                                             int dpos, const char*& Abase, const char*& Wbase,
                                             uint32_t (&aoffs)[LA], uint32_t (&boffs)[LB]) {
  if constexpr (WT)  // W_e stored [K, N]: the tile's columns from its first K row
    Wbase = reinterpret_cast<const char*>(W + t.e * w_estride + static_cast<int64_t>(t.k0) * N + t.n0);
  else
    Wbase = reinterpret_cast<const char*>(W + t.e * w_estride + static_cast<int64_t>(t.n0) * lda + t.k0);
  if (row_idx != nullptr) {
    Abase = reinterpret_cast<const char*>(A + t.k0);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (wave * LA + i) * 8 + drow;
      const uint32_t src = static_cast<uint32_t>(row_idx[t.row0 + min(r, t.rv - 1)]);
      aoffs[i] = (src * static_cast<uint32_t>(lda) + (dpos ^ swz_key(r)) * 8) * 2;
    }
  } else {
    Abase = reinterpret_cast<const char*>(A + static_cast<int64_t>(t.arow) * lda + t.k0);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (wave * LA + i) * 8 + drow;
      aoffs[i] = static_cast<uint32_t>((min(r, t.rv - 1) * lda + (dpos ^ swz_key(r)) * 8) * 2);
    }
  }
  if constexpr (WT) {
    // K-major stage: block i of this wave is K rows kr, kr + 1 (512 bytes
    // each); lane L lands at byte 16 (L % 32) of row kr + L / 32, in 64-byte
    // segment p = (L % 32) / 4, which holds the row's segment p ^ (kr & 3).
    // Columns past N read column N - 8 onward (never stored).
    const int lane = drow * 8 + dpos;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int kr = (wave * LB + i) * 2 + (lane >> 5);
      const int p = (lane & 31) >> 2;
      const int col = min(t.n0 + 32 * (p ^ (kr & 3)) + 8 * (lane & 3), N - 8) - t.n0;
      boffs[i] = static_cast<uint32_t>((static_cast<int64_t>(kr) * N + col) * 2);
    }
  } else {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (wave * LB + i) * 8 + drow;
      boffs[i] = static_cast<uint32_t>(((min(t.n0 + r, N - 1) - t.n0) * lda + (dpos ^ swz_key(r)) * 8) * 2);
    }
  }
}

// Activation, conversion and stores of one wave's (32 TM) x 128 outputs (the
// accumulators started at the bias). FULL: every row and feature of the tile
// is in range (no per-lane checks).
template <int TM, bool OUT_F32, int ACT, bool FULL>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TN][TM], void* __restrict__ out,
                                         const TileInfo& t, int N, int wm, int wn, int l5, int hi) {
  constexpr int WM = 32 * TM;
  const int fb = wn * WN + hi * 4;  // this lane's first feature in the tile
  const int nb = t.n0 + fb;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = wm * WM + j * 32 + l5;
    if (!FULL && m >= t.rv) continue;
    const int64_t orow = static_cast<int64_t>(t.row0 + m) * N + nb;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!FULL && nb + i * 32 + q * 8 >= N) continue;
        const float v0 = activate<ACT>(acc[i][j][4 * q + 0]);
        const float v1 = activate<ACT>(acc[i][j][4 * q + 1]);
        const float v2 = activate<ACT>(acc[i][j][4 * q + 2]);
        const float v3 = activate<ACT>(acc[i][j][4 * q + 3]);
        const int64_t o = orow + i * 32 + q * 8;
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = make_float4(v0, v1, v2, v3);
        } else {
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
          const bf16x4_t h = {static_cast<__bf16>(v0), static_cast<__bf16>(v1), static_cast<__bf16>(v2),
                              static_cast<__bf16>(v3)};
          *reinterpret_cast<bf16x4_t*>(static_cast<uint16_t*>(out) + o) = h;
        }
      }
      // one 32x32 tile at a time: the scheduler may not hoist the next
      // tile's accumulator reads above these stores (that needs more VGPRs
      // than the next tile's prefetch state leaves free)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The persistent tile loop for tiles of BM = 64 TM rows. lds: NST stage
// buffers; s_tiles: the M-tile prefix for this height; s_bias: two slices.
// WG: weight-gradient tiles (decode_tile_wg; offsets holds the padded K
// offsets, M the rows of C per expert); else expert-FFN tiles of nkl stages
// each: ntiles output tiles, and total = ntiles (whole K) or 2 ntiles (two K
// halves; the second half's partial sums go to out2, without bias).
template <int TM, bool OUT_F32, int ACT, bool WG, bool WT = false>
__device__ __forceinline__ void tile_loop(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_idx,
                                          const uint16_t* __restrict__ W, const float* __restrict__ bias,
                                          void* __restrict__ out, void* __restrict__ out2,
                                          const int32_t* __restrict__ offsets,
                                          int E, int N, int nkl, int lda, int64_t w_estride, int M,
                                          char* lds, const int* s_tiles, float (*s_bias)[BN], int tile,
                                          int total, int ntiles, int NT) {
  constexpr int BM = 64 * TM;
  constexpr int WM = BM / 2;         // tokens per wave
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int LA = BM / 32;        // 1 KiB (8-row) DMA blocks of the token tile per wave
  constexpr int LB = BN / 32;        // 1 KiB DMA blocks of the weight tile per wave
  constexpr int G = LA + LB;         // DMA loads per wave per stage
  constexpr int NST = stages_for<TM>();
  static_assert(NST * STAGE <= kLdsBytes, "stage buffers exceed the LDS array");
  const int Gd = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // per-lane constants: fragment offsets of the four K16 steps of a stage
  // (lane (l5, hi) reads row l5, chunk 2s + hi) and the DMA source mapping
  const int l5 = lane & 31, hi = lane >> 5;
  const int key = swz_key(l5);  // equal for rows l5 + 32j
  uint32_t fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = l5 * ROWB + 16 * ((2 * s + hi) ^ key);
  const int drow = lane >> 3, dpos = lane & 7;
  auto decode = [&](int tl) {
    if constexpr (WG) return decode_tile_wg(tl, s_tiles, offsets, E, NT, BM, M);
    else return decode_tile(tl, s_tiles, offsets, E, NT, BM, nkl, ntiles);
  };
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const uint32_t trow = wm * WM * ROWB;            // this wave's token rows in a stage
  const uint32_t wrow = A_BYTES + wn * WN * ROWB;  // this wave's weight rows in a stage
  // WT: the weight stage is K-major, BK rows of BN features (kWtRowB bytes,
  // 64-byte segments at position seg ^ (row & 3)). Weight fragment tile i
  // of lane (l5, hi) in K16 step s: feature 32 i + l5 of this wave's 128,
  // k = 16 s + 8 hi .. + 7, as two transposing reads of 4 rows: a 16-lane
  // group g reads rows 8 (g / 2) + (lane % 16) / 4 at features
  // 16 (g % 2) + 4 (lane % 4) of the tile, and lane o of the group gets
  // feature 16 (g % 2) + o for those 4 rows.
  uint32_t wo[TN];
  if constexpr (WT) {
    const int key4 = (lane >> 2) & 3;
    const uint32_t rb = (8 * hi + ((lane & 15) >> 2)) * kWtRowB + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
#pragma unroll
    for (int i = 0; i < TN; ++i) wo[i] = A_BYTES + rb + 64 * ((4 * wn + i) ^ key4);
  }
  // bytes from one K stage of W to the next
  const int64_t wst = WT ? static_cast<int64_t>(BK) * N * 2 : ROWB;
  auto wadr = [&](uint32_t sbase, int s, uint32_t (&wa)[TN]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) wa[i] = sbase + wo[i] + s * 16 * kWtRowB;
  };

  uint32_t aoffs[LA], boffs[LB], vo[G];
  const char* Abase;
  const char* Wbase;
  // a tile's first stages and its bias slice (wave 0, one lane per 4 features)
  auto prologue = [&](const TileInfo& c, int par) {
    for (int p = 0; p < NST && p < (WG ? c.nk : nkl); ++p)
      issue_stage<TM>(aoffs, boffs, lds_base + p * STAGE + wave * LA * 1024,
                      lds_base + p * STAGE + A_BYTES + wave * LB * 1024, Abase + p * ROWB,
                      Wbase + p * wst);
    if (bias != nullptr && c.part == 0 && wave == 0)
      issue_bias(bias + static_cast<int64_t>(c.e) * N + min(c.n0 + 4 * lane, N - 4),
                 static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_bias[par][0])));
  };
  int par = 0;  // bias slice of the current tile
  TileInfo cur = decode(tile);
  tile_sources<LA, LB, WT>(cur, A, row_idx, W, N, lda, w_estride, wave, drow, dpos, Abase, Wbase, aoffs,
                           boffs);
  prologue(cur, par);

  for (;;) {
    // K stages of this tile (cur moves on before its epilogue); the same for
    // every expert-FFN tile
    const int nk = WG ? cur.nk : nkl;

    // the tile's first stages and bias slice (and, after an epilogue, its
    // stores)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // accumulators start at the bias: lane (l5, hi) holds features
    // fb + 32 i + 8 q + {0..3} of tile i (the same for every token tile j)
    f32x16_t acc[TN][TM];
    {
      const bool with_bias = bias != nullptr && cur.part == 0;
      const int fb = wn * WN + hi * 4;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 b = with_bias
                               ? *reinterpret_cast<const float4*>(&s_bias[par][fb + i * 32 + q * 8])
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int j = 0; j < TM; ++j) {
            acc[i][j][4 * q + 0] = b.x;
            acc[i][j][4 * q + 1] = b.y;
            acc[i][j][4 * q + 2] = b.z;
            acc[i][j][4 * q + 3] = b.w;
          }
        }
    }
    bf16x8_t wf0[TN], tf0[TM], wf1[TN], tf1[TM];
    if constexpr (WT) {
      uint32_t wa[TN];
      wadr(lds_base, 0, wa);
      read_frags_t<TM>(wf0, tf0, lds_base + trow + fo[0], wa);
    } else {
      read_frags<TM>(wf0, tf0, lds_base + trow + fo[0], lds_base + wrow + fo[0]);
    }

    TileInfo done = cur;
    const int next = tile + Gd;
#pragma unroll
    for (int i = 0; i < LA; ++i) vo[i] = aoffs[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) vo[LA + i] = boffs[i];
    int sc = 0;              // buffer holding K stage t
    uint32_t sb = lds_base;  // its LDS address
    int t = 0;
    // the second half of the last refill, issued with the next stage's first
    // K16 step: its LDS and global bases
    uint32_t pla = 0, plb = 0;
    const char* pga = nullptr;
    const char* pgw = nullptr;
    // one K16 step reading the fragments of step s of the stage at sbase
    auto kstep = [&](const bf16x8_t (&w)[TN], const bf16x8_t (&tk)[TM], bf16x8_t (&nw)[TN],
                     bf16x8_t (&nt)[TM], uint32_t sbase, int s) {
      if constexpr (WT) {
        uint32_t wa[TN];
        wadr(sbase, s, wa);
        step_t<TM>(acc, w, tk, nw, nt, sbase + trow + fo[s], wa);
      } else {
        step<TM>(acc, w, tk, nw, nt, sbase + trow + fo[s], sbase + wrow + fo[s]);
      }
    };
    // the same with half of a stage's LDS-DMA loads
    auto kstep_dma = [&](auto half, const bf16x8_t (&w)[TN], const bf16x8_t (&tk)[TM], bf16x8_t (&nw)[TN],
                         bf16x8_t (&nt)[TM], uint32_t sbase, int s) {
      constexpr int H = decltype(half)::value;
      if constexpr (WT) {
        uint32_t wa[TN];
        wadr(sbase, s, wa);
        step_dma_t<TM, H>(acc, w, tk, nw, nt, sbase + trow + fo[s], wa, vo, pla, plb, pga, pgw);
      } else {
        step_dma<TM, H>(acc, w, tk, nw, nt, sbase + trow + fo[s], sbase + wrow + fo[s], vo, pla, plb, pga,
                        pgw);
      }
    };
    // One K stage. D1: step 0 issues the second half of the previous stage's
    // refill; RF: stage t+NST is still to load (this stage's buffer takes it
    // once every wave has read the stage).
    auto stage = [&](auto d1, auto rf) {
      // K16 steps 0..2, each reading the next step's fragments
      if constexpr (decltype(d1)::value)
        kstep_dma(std::integral_constant<int, 1>{}, wf0, tf0, wf1, tf1, sb, 1);
      else
        kstep(wf0, tf0, wf1, tf1, sb, 1);
      kstep(wf1, tf1, wf0, tf0, sb, 2);
      kstep(wf0, tf0, wf1, tf1, sb, 3);
      // stage t+1 has landed and every wave has read its last fragments of
      // stage t
      if constexpr (decltype(rf)::value) wait_loads<G>(NST - 2);
      else wait_loads<G>(nk - 2 - t);
      __syncthreads();
      const int sn_i = (sc + 1 == NST) ? 0 : sc + 1;
      const uint32_t sn = lds_base + sn_i * STAGE;
      // K16 step 3; read step 0 of stage t+1
      if constexpr (decltype(rf)::value) {
        // the buffer of stage t takes stage t+NST: half of its loads now,
        // the rest with step 0 of stage t+1
        pla = sb + wave * LA * 1024;
        plb = sb + A_BYTES + wave * LB * 1024;
        pga = Abase + (t + NST) * ROWB;
        pgw = Wbase + (t + NST) * wst;
        kstep_dma(std::integral_constant<int, 0>{}, wf1, tf1, wf0, tf0, sn, 0);
      } else {
        kstep(wf1, tf1, wf0, tf0, sn, 0);
      }
      sc = sn_i;
      sb = sn;
    };
    using yes = std::true_type;
    using no = std::false_type;
    if (t + NST < nk) {
      // steady state; the first tail stage (there is one, as NST >= 2)
      // issues the last refill's second half
      stage(no{}, yes{});
      for (++t; t + NST < nk; ++t) stage(yes{}, yes{});
      stage(yes{}, no{});
      ++t;
    }
    // the last stages: nothing more to load
    for (; t + 1 < nk; ++t) stage(no{}, no{});
    // the last stage
    kstep(wf0, tf0, wf1, tf1, sb, 1);
    kstep(wf1, tf1, wf0, tf0, sb, 2);
    kstep(wf0, tf0, wf1, tf1, sb, 3);
    // every wave has read all of its fragments: all buffers are free, and the
    // next tile's first stages load during this tile's last MFMAs and epilogue
    __syncthreads();
    if (next < total) {
      cur = decode(next);
      tile_sources<LA, LB, WT>(cur, A, row_idx, W, N, lda, w_estride, wave, drow, dpos, Abase, Wbase,
                               aoffs, boffs);
      prologue(cur, par ^ 1);
    }
    last_step<TM>(acc, wf1, tf1);

    // ---- epilogue: lane holds token l5 of each 32-token tile j and
    // features 8q + 4*hi + {0..3} of each 32-feature tile i
    const bool full_tile = done.rv == BM && done.n0 + BN <= N;
    void* dst = done.part ? out2 : out;
    if (full_tile) epilogue<TM, OUT_F32, ACT, true>(acc, dst, done, N, wm, wn, l5, hi);
    else epilogue<TM, OUT_F32, ACT, false>(acc, dst, done, N, wm, wn, l5, hi);
    if (next >= total) break;
    tile = next;
    par ^= 1;
  }
}

}  // namespace

// SHORT selects the tile heights: 256 or 192 rows (experts that can fill
// tall tiles), or 192, 128 or 64 rows (every expert holds fewer than 256
// rows: decode batches, many experts). Two instantiations rather than one
// kernel with all four: each keeps its own register allocation.
// out2 (fp32 output without activation only, else null): with it, the
// schedule may split K in two halves when that fills more of the chip (few
// output tiles, long K); the first half (with bias) goes to out, the second
// to out2, and the number of parts (1 or 2) to *nsplit (when not null), so
// out = out + out2 holds the product only when *nsplit is 2.
// WT: each W_e is stored [K, N] (K-major, as W^T of the usual [N, K]); the
// weight stages are loaded row by row of K and read with transposing LDS
// reads.
template <bool OUT_F32, int ACT, bool SHORT, bool WT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_idx,
                              const uint16_t* __restrict__ W,
                              const float* __restrict__ bias, void* __restrict__ out,
                              void* __restrict__ out2, int32_t* __restrict__ nsplit,
                              const int32_t* __restrict__ offsets, int E, int N, int K) {
  // the body uses gfx950 builtins only: the host pass needs just the signature
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) char lds[SHORT ? kLdsBytes : 2 * (256 + BN) * ROWB];
  __shared__ int s_tiles[1025];  // exclusive prefix of M tiles per expert
  __shared__ int s_part[SHORT ? 3 : 2][256];
  __shared__ __attribute__((aligned(16))) float s_bias[2][BN];  // bias slices of this and the next tile

  const int tid = threadIdx.x;
  const int NT = (N + BN - 1) / BN;
  const int Gd = gridDim.x;
  const int per = (E + 255) / 256;
  const int eb = tid * per;
  const int b = blockIdx.x;
  // blocks are dealt to the 8 XCDs round-robin: renumber so that consecutive
  // tiles (which share weight and token panels) run on one XCD. A launch
  // whose tiles fit in one round spreads them evenly: ceil(tiles / 8) per
  // XCD (a permutation of the blocks either way, so later rounds, at a
  // stride of the grid, are unchanged).
  auto xcd_tile = [&](int total) {
    if (Gd % 8 != 0) return b;
    const int per = (min(total, Gd) + 7) / 8;
    const int kk = b / 8, x = b % 8;
    return kk < per ? x * per + kk : 8 * per + (kk - per) * 8 + x;
  };
  const int64_t wes = static_cast<int64_t>(N) * K;
  // K parts allowed: two when out2 is given and K splits into whole stages
  const int smax = (out2 != nullptr && (K / BK) % 2 == 0) ? 2 : 1;
  // work of one block: rounds of units x (rows x (K per part + epilogue))
  auto cost = [&](int64_t tiles, int rows, int S) {
    const int64_t rounds = (tiles * S + Gd - 1) / Gd;
    return rounds * rows * static_cast<int64_t>(K / S + kEpiK);
  };
  if constexpr (!SHORT) {
    // ---- device-side schedule. Both tile heights are counted, each whole
    // and (when allowed) split in K; the choice whose units need the least
    // block work (cost above) runs: the taller height, then the unsplit one,
    // on a tie.
    int c256 = 0, c192 = 0;
    for (int e = eb; e < min(E, eb + per); ++e) {
      const int n = offsets[e + 1] - offsets[e];
      c256 += (n + 255) / 256;
      c192 += (n + 191) / 192;
    }
    s_part[0][tid] = c256;
    s_part[1][tid] = c192;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int a0 = (tid >= off) ? s_part[0][tid - off] : 0;
      const int a1 = (tid >= off) ? s_part[1][tid - off] : 0;
      __syncthreads();
      s_part[0][tid] += a0;
      s_part[1][tid] += a1;
      __syncthreads();
    }
    bool tall = true;
    int S = 1;
    int64_t best = -1;
    for (int sp = 1; sp <= smax; ++sp)
      for (int q = 0; q < 2; ++q) {
        const int64_t c = cost(static_cast<int64_t>(s_part[q][255]) * NT, q == 0 ? 256 : 192, sp);
        if (best < 0 || c < best) {
          best = c;
          tall = q == 0;
          S = sp;
        }
      }
    const int BMs = tall ? 256 : 192;
    {
      const int sel = tall ? 0 : 1;
      int run = s_part[sel][tid] - (tall ? c256 : c192);
      for (int e = eb; e < min(E, eb + per); ++e) {
        s_tiles[e] = run;
        run += (offsets[e + 1] - offsets[e] + BMs - 1) / BMs;
      }
      if (tid == 255) s_tiles[E] = s_part[sel][255];
    }
    __syncthreads();
    if (nsplit != nullptr && b == 0 && tid == 0) *nsplit = S;
    const int ntiles = s_tiles[E] * NT;
    const int total = ntiles * S;
    const int nkl = K / BK / S;
    const int tile = xcd_tile(total);
    if (tile >= total) return;
    if (tall)
      tile_loop<4, OUT_F32, ACT, false, WT>(A, row_idx, W, bias, out, out2, offsets, E, N, nkl, K, wes, 0,
                                        lds, s_tiles, s_bias, tile, total, ntiles, NT);
    else
      tile_loop<3, OUT_F32, ACT, false, WT>(A, row_idx, W, bias, out, out2, offsets, E, N, nkl, K, wes, 0,
                                        lds, s_tiles, s_bias, tile, total, ntiles, NT);
  } else {
    // ---- the same with heights 192, 128 and 64, whole or split in K: the
    // least cost with h + 64 rows per tile of height h (its MFMA rows plus a
    // fixed share for its weight panel, which short tiles stream with fewer
    // MFMAs); the taller height, then the unsplit one, on a tie
    constexpr int kH[3] = {192, 128, 64};
    int c[3] = {0, 0, 0};
    for (int e = eb; e < min(E, eb + per); ++e) {
      const int n = offsets[e + 1] - offsets[e];
#pragma unroll
      for (int q = 0; q < 3; ++q) c[q] += (n + kH[q] - 1) / kH[q];
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) s_part[q][tid] = c[q];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int a[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) a[q] = (tid >= off) ? s_part[q][tid - off] : 0;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 3; ++q) s_part[q][tid] += a[q];
      __syncthreads();
    }
    int sel = 0, S = 1;
    int64_t best = -1;
    for (int sp = 1; sp <= smax; ++sp)
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int64_t c = cost(static_cast<int64_t>(s_part[q][255]) * NT, kH[q] + 64, sp);
        if (best < 0 || c < best) {
          best = c;
          sel = q;
          S = sp;
        }
      }
    const int BMs = sel == 0 ? 192 : (sel == 1 ? 128 : 64);
    {
      int run = s_part[sel][tid] - c[sel];
      for (int e = eb; e < min(E, eb + per); ++e) {
        s_tiles[e] = run;
        run += (offsets[e + 1] - offsets[e] + BMs - 1) / BMs;
      }
      if (tid == 255) s_tiles[E] = s_part[sel][255];
    }
    __syncthreads();
    if (nsplit != nullptr && b == 0 && tid == 0) *nsplit = S;
    const int ntiles = s_tiles[E] * NT;
    const int total = ntiles * S;
    const int nkl = K / BK / S;
    const int tile = xcd_tile(total);
    if (tile >= total) return;
    if (sel == 0)
      tile_loop<3, OUT_F32, ACT, false, WT>(A, row_idx, W, bias, out, out2, offsets, E, N, nkl, K, wes, 0,
                                        lds, s_tiles, s_bias, tile, total, ntiles, NT);
    else if (sel == 1)
      tile_loop<2, OUT_F32, ACT, false, WT>(A, row_idx, W, bias, out, out2, offsets, E, N, nkl, K, wes, 0,
                                        lds, s_tiles, s_bias, tile, total, ntiles, NT);
    else
      tile_loop<1, OUT_F32, ACT, false, WT>(A, row_idx, W, bias, out, out2, offsets, E, N, nkl, K, wes, 0,
                                        lds, s_tiles, s_bias, tile, total, ntiles, NT);
  }
#endif
}

// Weight gradients of the expert GEMMs on the same tile loop:
//   C[e] [M, N] = sum over expert e's rows r of A[r, m] B[r, n]
// with both operands given transposed and K-contiguous: At [M, lda],
// Bt [N, lda], expert e's rows at columns [poff[e], poff[e+1]) (a multiple
// of 64, zero-padded). Experts without rows get no tiles (their C is left
// to the caller). 256-row tiles, fp32 out, no bias.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_wgrad_bf16_kernel(const uint16_t* __restrict__ At, const uint16_t* __restrict__ Bt,
                               const int32_t* __restrict__ poff, int E, int M, int N, int lda,
                               float* __restrict__ C) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) char lds[2 * (256 + BN) * ROWB];
  __shared__ int s_tiles[1025];
  __shared__ int s_part[256];
  __shared__ __attribute__((aligned(16))) float s_bias[2][BN];
  const int tid = threadIdx.x;
  const int NT = (N + BN - 1) / BN;
  const int MT = (M + 255) / 256;
  const int per = (E + 255) / 256;
  const int eb = tid * per;
  int cnt = 0;
  for (int e = eb; e < min(E, eb + per); ++e) cnt += (poff[e + 1] > poff[e]) ? MT : 0;
  s_part[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int a0 = (tid >= off) ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += a0;
    __syncthreads();
  }
  {
    int run = s_part[tid] - cnt;
    for (int e = eb; e < min(E, eb + per); ++e) {
      s_tiles[e] = run;
      run += (poff[e + 1] > poff[e]) ? MT : 0;
    }
    if (tid == 255) s_tiles[E] = s_part[255];
  }
  __syncthreads();
  const int total = s_tiles[E] * NT;
  const int Gd = gridDim.x;
  const int b = blockIdx.x;
  const int tile = (Gd % 8 == 0) ? (b % 8) * (Gd / 8) + b / 8 : b;
  if (tile >= total) return;
  tile_loop<4, true, kActNone, true>(At, nullptr, Bt, nullptr, C, nullptr, poff, E, N, 0, lda, 0, M,
                                     lds, s_tiles, s_bias, tile, total, total, NT);
#endif
}

namespace {

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, const int32_t* row_idx, const uint16_t* W,
                            const float* bias, void* out, float* out2, int32_t* nsplit,
                            bool out_f32, int act, const int32_t* offsets, int E, int N, int K,
                            int64_t max_rows, int max_rows_per_expert, hipStream_t s,
                            hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (max_rows <= 0) {
    // nothing to launch: the events still mark this (empty) kernel's place
    for (hipEvent_t ev : {ev_start, ev_stop})
      if (ev != nullptr) {
        const hipError_t e = hipEventRecord(ev, s);
        if (e != hipSuccess) return e;
      }
    return hipSuccess;
  }
  if (!out_f32 || act != kActNone) out2 = nullptr;  // a split needs a linear fp32 output
  const int smax = (out2 != nullptr && (K / BK) % 2 == 0) ? 2 : 1;
  // short tiles when no expert can fill a 256-row tile
  const bool shorter = max_rows_per_expert < 256;
  // upper bound on tiles: sum_e ceil(n_e/h) <= max_rows/h + E for the shortest h
  const int64_t mt_bound = max_rows / (shorter ? 64 : 192) + E;
  const int slots = cu_count();
  const int64_t tiles = mt_bound * ((N + BN - 1) / BN) * smax;
  const unsigned grid = static_cast<unsigned>(tiles < slots ? tiles : slots);
  // with events, the dispatch records them at the kernel's start and end
  // (hipExtLaunchKernelGGL); without, a plain launch (the extended launch
  // measured several microseconds more launch gap per kernel)
  const bool timed = ev_start != nullptr || ev_stop != nullptr;
#define MOE_GEMM_ONE(OF, AC, SH)                                                                    \
  do {                                                                                             \
    if (timed)                                                                                     \
      hipExtLaunchKernelGGL(grouped_gemm_bf16_kernel<OF, AC, SH>, dim3(grid), dim3(256), 0, s,      \
                            ev_start, ev_stop, 0, A, row_idx, W, bias, out, static_cast<void*>(out2), \
                            nsplit, offsets, E, N, K);                                              \
    else                                                                                           \
      grouped_gemm_bf16_kernel<OF, AC, SH><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, out2,    \
                                                                nsplit, offsets, E, N, K);          \
  } while (0)
#define MOE_GEMM(OF, AC)            \
  do {                              \
    if (shorter)                    \
      MOE_GEMM_ONE(OF, AC, true);   \
    else                            \
      MOE_GEMM_ONE(OF, AC, false);  \
  } while (0)
  if (out_f32) MOE_GEMM(true, kActNone);
  else if (act == kActRelu) MOE_GEMM(false, kActRelu);
  else if (act == kActGeluTanh) MOE_GEMM(false, kActGeluTanh);
  else MOE_GEMM(false, kActNone);
#undef MOE_GEMM
#undef MOE_GEMM_ONE
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_wt(const uint16_t* A, const int32_t* row_idx, const uint16_t* W,
                               const float* bias, float* out, const int32_t* offsets, int E, int N,
                               int K, int64_t max_rows, int max_rows_per_expert, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  const bool shorter = max_rows_per_expert < 256;
  const int64_t mt_bound = max_rows / (shorter ? 64 : 192) + E;
  const int slots = cu_count();
  const int64_t tiles = mt_bound * ((N + BN - 1) / BN);
  const unsigned grid = static_cast<unsigned>(tiles < slots ? tiles : slots);
  if (shorter)
    grouped_gemm_bf16_kernel<true, kActNone, true, true><<<grid, 256, 0, s>>>(
        A, row_idx, W, bias, out, nullptr, nullptr, offsets, E, N, K);
  else
    grouped_gemm_bf16_kernel<true, kActNone, false, true><<<grid, 256, 0, s>>>(
        A, row_idx, W, bias, out, nullptr, nullptr, offsets, E, N, K);
  return hipGetLastError();
}

hipError_t launch_wgrad_bf16(const uint16_t* At, const uint16_t* Bt, const int32_t* poff, int E,
                             int M, int N, int lda, float* C, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>(E) * ((M + 255) / 256) * ((N + BN - 1) / BN);
  const int slots = cu_count();
  const unsigned grid = static_cast<unsigned>(tiles < slots ? tiles : slots);
  if (grid == 0) return hipSuccess;
  grouped_wgrad_bf16_kernel<<<grid, 256, 0, s>>>(At, Bt, poff, E, M, N, lda, C);
  return hipGetLastError();
}

}  // namespace moe
