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
//    lane's accumulators hold 4 consecutive features of one token. bf16
//    outputs go through LDS in 32-token slabs so that the stores write whole
//    cache lines (4 rows x 256 bytes per instruction); fp32 outputs store
//    16-byte vectors from the accumulators.
//  * Registers: the 256-row kernels use all 512 (256 of them accumulators).
//    Per-lane terms are recomputed from a fresh lane id where they are used
//    and the next tile's DMA offsets wait in LDS across the epilogue, so
//    that little is spilled: a scratch reload waits for every vector-memory
//    operation issued before it, the next tile's stage loads included.
//  * The tile height is chosen on the device, per launch, from the actual
//    expert row counts (the cost model is at the schedule below: rounds of
//    the persistent blocks times the K-loop work of a tile, its rows plus a
//    share for the weight panel every tile streams whole, plus its
//    epilogue): long-K layers with thousands of rows per expert run 256-row
//    tiles, ragged ones 192-row tiles, and experts with a few dozen rows
//    (decode batches) 64-row tiles, which stream the same weights with a
//    quarter of the MFMAs. The host never learns the row counts.
//  * K advances in stages of BK=64: every LDS row is 128 bytes, one full
//    cache line of the source row, so each L1->L2 request moves a whole line.
//    The 16-byte chunks of a row are XOR-swizzled by (row/2)&7, which keeps
//    the fragment reads (16 lanes = 16 rows at one chunk) on distinct banks.
//  * Tiles move global -> LDS with gfx950's LDS-DMA loads
//    (global_load_lds_dwordx4: no staging registers, no ds_write); one
//    instruction fills 8 rows (1 KiB); each lane fetches the chunk that the
//    swizzle places at its LDS slot.
//  * Token and weight stages sit in rings of their own (2 + 2 buffers for
//    256-row tiles, 2 + 3 for 192, 3 + 3 for 128, 3 + 4 for 64). A stage is
//    four K16 steps; each step's MFMAs run with the next step's fragment
//    reads in flight, and a buffer is refilled (with the stage NA or NW
//    ahead) right after the barrier that shows every wave has read it: half
//    of the loads between the MFMAs of that stage's last step, the other
//    half between those of the next stage's first step (a whole stage's
//    loads at once back up the load queue, and the wave stalls at an MFMA
//    issue slot). The next tile's first stage, and its bias slice, load
//    during the current tile's last step and epilogue; its later stages
//    after the epilogue's stores.
//  * Persistent blocks, one per CU. The schedule is computed on the device
//    from expert_offsets (no host read-back): expert-major tiles, and inside
//    an expert with many M tiles groups of kGroupM M tiles swept over the N
//    tiles, so concurrent tiles share token and weight panels. The tiles one
//    XCD runs at a time are consecutive (blocks are dealt to the 8 XCDs
//    round-robin) and share its L2 (sched_xcd_plan: interleaved rounds when
//    an expert's weights are re-read, else a contiguous range per XCD).
//  * Ragged M: rows past an expert's end read that expert's last row and are
//    never stored, so no tile reads outside [0, rows).
//  * With a second output buffer (the second expert GEMM), tiles may run as
//    K parts whose partial sums (bf16) the combine adds: all tiles in two
//    halves when the whole tiles fit in one round, or, after two or more
//    full rounds, only the tiles of a last, partly filled round, split so
//    that their parts fill it.
#include "moe_internal.h"

#include "gemm_schedule.h"

#include <hip/hip_ext.h>

#include <atomic>
#include <type_traits>
#include <utility>

namespace moe {

namespace {

constexpr int BN = 256;       // features per tile
constexpr int BK = 64;        // K per LDS stage
constexpr int ROWB = BK * 2;  // bytes per LDS row (128)
constexpr int kWtRowB = BN * 2;  // bytes per row of a K-major weight stage (512)
// Stage rings. The token (A) and weight (W) tiles of a K stage sit in two
// rings of their own: NA token buffers and NW weight buffers (NW >= NA). A
// buffer takes the stage NA (NW) ahead once every wave has read it, so the
// weight stream, which a tile of few rows is bound by, runs NW - 1 stages
// ahead: 256-row tiles 2 + 2 buffers (128 KiB), 192 rows 2 + 3 (144 KiB),
// 128 rows 3 + 3 (144 KiB), 64 rows 3 + 4 (152 KiB).
template <int TM>
constexpr int a_stages() { return TM == 1 || TM == 2 ? 3 : 2; }
template <int TM>
constexpr int w_stages() { return TM == 4 ? 2 : (TM == 1 ? 4 : 3); }
template <int TM>
constexpr int lds_bytes_for() { return a_stages<TM>() * 64 * TM * ROWB + w_stages<TM>() * BN * ROWB; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
[[maybe_unused]] constexpr int kLdsTall = cmax(lds_bytes_for<4>(), lds_bytes_for<3>());
[[maybe_unused]] constexpr int kLdsShort = cmax(cmax(lds_bytes_for<3>(), lds_bytes_for<2>()), lds_bytes_for<1>());
constexpr int TN = 4;         // 32-feature MFMA tiles per wave
// Output modes of the epilogue: bf16 (after the activation), fp32, or the
// second expert GEMM's y_perm: bf16, for whole tiles and for the partial
// sums of the K parts of a split tile alike (see TilePlan).
constexpr int kOutBf16 = kGemmOutBf16;
constexpr int kOutF32 = kGemmOutF32;
constexpr int kOutYperm = kGemmOutYperm;
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

template <int TM>
__device__ __forceinline__ void stage_a(const uint32_t (&ao)[2 * TM], uint32_t la, const char* ga) {
  if constexpr (TM == 4) stage_a_4x4(ao, la, ga);
  else if constexpr (TM == 3) stage_a_3x4(ao, la, ga);
  else if constexpr (TM == 2) stage_a_2x4(ao, la, ga);
  else stage_a_1x4(ao, la, ga);
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

// One output tile: expert e, rows [row0, row0 + rv) of the grouped problem
// (rv valid of the tile's height), features from n0; operand A's first row
// arow and K range [k0, k0 + 64 nk); part: which K part (part 0 carries the
// bias; parts 1.. go to the second output buffer); split: the tile is one K
// part of several (a partial sum); orow: the output row of row0 in its
// buffer.
struct TileInfo {
  int e, row0, rv, n0, arow, k0, nk, part, orow;
  bool split;
};

// The tiles of one launch: the first mcap M tiles (in expert-major order)
// run whole, as units [0, dp = mcap NT) in the grouped order below; the last
// mt M tiles (rows r_tail onward, tail_rows of them) run as p K parts of nkp
// stages each: part j of tail M tile m (0..mt-1) and feature panel n is
// unit dp + (j NT + n) mt + m, so the parts that share a weight panel slice
// are neighbours. Part 0 writes its partial sums (with the bias) at the
// rows' own places in out; part j >= 1 writes rows
// (j - 1) tail_rows + (row - r_tail) of out2. p = 1: no parts (mt = 0).
struct TilePlan {
  int mcap, nk, p, nkp, mt, r_tail, tail_rows;
};

// Epilogue cost of an fp32 output tile in K-equivalents (its stores take
// about as long as 512 more K per row of MFMA work); weighs a K split, which
// doubles the stores, against the rounds it saves.
[[maybe_unused]] constexpr int kEpiK = 512;

// The tall schedule's share of a tile for its weight panel, in rows of the
// K loop: 256-row and 192-row tiles stream the same 256 weight rows per K
// stage. With it the 16384-token layer takes 256-row tiles (30 and 9 rounds
// against 39 and 11 of 192 rows); its GEMMs ran 3336 and 3280 µs that way
// against 3522 and 3398 µs with 192-row tiles, which the bare row count
// preferred. Layers with a short K (1024: the skewed layers' second GEMM)
// keep 192-row tiles, whose epilogues are shorter (256-row tiles ran 216
// µs there against 181).
[[maybe_unused]] constexpr int kTallShare = 128;

constexpr int kGroupM = 6;  // M tiles per group of the tile order

// At most this many K parts per tail tile: the combine reads one partial
// row per part for each of the tail's rows, which the cost model does not
// see.
constexpr int kMaxParts = 4;

// s_tiles[e]: exclusive prefix over experts of their M tiles of height BM.
// PARTS: the kernel may run K parts (else every unit is a whole tile and
// pl.mcap is the M-tile count).
template <bool PARTS>
__device__ __forceinline__ TileInfo decode_tile(int u, const int* s_tiles, const int32_t* offsets,
                                                int E, int NT, int BM, const TilePlan& pl) {
  TileInfo t;
  const int dp = pl.mcap * NT;
  if (PARTS && u >= dp) {
    // a K part of a tail tile: parts outermost, then feature panels, M tiles
    // innermost
    const int tt = pl.mt * NT;
    const int v = u - dp;
    const int j = v / tt;
    const int r = v - j * tt;
    const int n = r / pl.mt;
    const int gm = pl.mcap + (r - n * pl.mt);
    // expert: the largest e with s_tiles[e] <= gm (experts with no rows
    // share their successor's prefix and are skipped)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tiles[mid] <= gm) lo = mid;
      else hi = mid - 1;
    }
    t.e = lo;
    t.row0 = offsets[lo] + (gm - s_tiles[lo]) * BM;
    t.rv = min(BM, offsets[lo + 1] - t.row0);
    t.n0 = n * BN;
    t.arow = t.row0;
    t.k0 = j * pl.nkp * BK;
    t.nk = pl.nkp;
    t.part = j;
    t.split = true;
    t.orow = j == 0 ? t.row0 : (j - 1) * pl.tail_rows + (t.row0 - pl.r_tail);
    return t;
  }
  // a whole tile. Expert: the largest e with min(s_tiles[e], mcap) NT <= u
  // (experts with no rows, or all rows in the tail, are skipped)
  auto pre = [&](int e) { return PARTS ? min(s_tiles[e], pl.mcap) : s_tiles[e]; };
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre(mid) * NT <= u) lo = mid;
    else hi = mid - 1;
  }
  t.e = lo;
  const int mte = pre(lo + 1) - s_tiles[lo];
  const int v = u - s_tiles[lo] * NT;
  // grouped order inside an expert with many M tiles: groups of kGroupM M
  // tiles, each swept over all N tiles with its M tiles innermost, so the
  // tiles one XCD runs at a time share a few token and weight panels; up to
  // 2 kGroupM M tiles form one group (every weight panel is then read once
  // per expert). The group size was picked by measurement on the
  // 16384-token layer (17 M tiles of 256 rows per expert): groups of 6 ran
  // its GEMMs 0.5% and 2.4% faster than groups of 5, and groups of 3, 4 and
  // 7 no better than 5
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
  t.k0 = 0;
  t.nk = pl.nk;
  t.part = 0;
  t.split = false;
  t.orow = t.row0;
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
  t.split = false;
  t.orow = t.row0;
  return t;
}

// s_waitcnt vmcnt(n) for a wave-uniform n (a jump over immediate forms).
template <int N>
__device__ __forceinline__ bool wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  return true;
}
template <int... N>
__device__ __forceinline__ void wait_vm_impl(int n, std::integer_sequence<int, N...>) {
  (void)(((n == N) && wait_vm_n<N>()) || ...);
}
__device__ __forceinline__ void wait_vm(int n) {
  wait_vm_impl(n < 63 ? n : 63, std::make_integer_sequence<int, 64>{});
}

// The loads a wave may leave in flight at each wait: gemm_schedule.h counts
// them from the issue order of the stage rings.
template <int NA, int NW, int LA, int LB>
__device__ __forceinline__ int loads_after(int t, int nk) {
  return sched_loads_after(t, nk, NA, NW, LA, LB);
}
template <int NA, int NW, int LA, int LB>
__device__ __forceinline__ int prologue_loads(int nk) {
  return sched_prologue_loads(nk, NA, NW, LA, LB);
}

// The lane id, read afresh. Per-lane values derived from it are then
// computed where they are used: derived from a lane id kept since the
// kernel's start, the compiler hoists them out of the tile loop and, with
// every register taken, spills them, and reloading a spilled value waits
// for every vector-memory operation issued before it (the next tile's
// stage loads included).
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
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
                                             int N, int lda, int64_t w_estride, int wave,
                                             const char*& Abase, const char*& Wbase,
                                             uint32_t (&aoffs)[LA], uint32_t (&boffs)[LB]) {
  const int lane = fresh_lane();
  const int drow = lane >> 3, dpos = lane & 7;
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
// is in range (no per-lane checks). A K part of a tile (t.split) stores
// partial sums; rows go to t.orow onward.
template <int TM, int OUT, int ACT, bool FULL>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TN][TM], void* __restrict__ out,
                                         const TileInfo& t, int N, int wm, int wn, int l5, int hi) {
  constexpr int WM = 32 * TM;
  const bool f32 = OUT == kOutF32;
  const int fb = wn * WN + hi * 4;  // this lane's first feature in the tile
  const int nb = t.n0 + fb;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = wm * WM + j * 32 + l5;
    if (!FULL && m >= t.rv) continue;
    const int64_t orow = static_cast<int64_t>(t.orow + m) * N + nb;
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
        if (f32) {
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

// Per-lane words parked in LDS while a tile's epilogue runs: word i of
// lane L at byte addr + 256 i + 4 L, written and read in pairs. Kept in
// registers, the next tile's DMA offsets were spilled to scratch around
// the epilogue, and each spill and reload waited for every vector-memory
// operation in flight (the next tile's stage 0, the epilogue's stores).
// N is even; unpark waits for its reads before it returns.
template <int N>
__device__ __forceinline__ void park_words(const uint32_t (&v)[N], uint32_t addr) {
  static_assert(N % 2 == 0 && N <= 8, "pairs, at most 8 words");
#pragma unroll
  for (int i = 0; i < N; i += 2)
    asm volatile("ds_write2st64_b32 %0, %1, %2 offset0:%3 offset1:%4"
                 :
                 : "v"(addr), "v"(v[i]), "v"(v[i + 1]), "i"(i), "i"(i + 1)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void unpark_words(uint32_t (&v)[N], uint32_t addr) {
  static_assert(N % 2 == 0 && N <= 8, "pairs, at most 8 words");
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t w[4];
  if constexpr (N == 2) {
    asm volatile("ds_read2st64_b32 %0, %1 offset0:0 offset1:1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(w[0]) : "v"(addr) : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read2st64_b32 %0, %2 offset0:0 offset1:1\n\tds_read2st64_b32 %1, %2 offset0:2 offset1:3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]) : "v"(addr) : "memory");
  } else if constexpr (N == 6) {
    asm volatile(
        "ds_read2st64_b32 %0, %3 offset0:0 offset1:1\n\tds_read2st64_b32 %1, %3 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %2, %3 offset0:4 offset1:5\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]) : "v"(addr) : "memory");
  } else {
    asm volatile(
        "ds_read2st64_b32 %0, %4 offset0:0 offset1:1\n\tds_read2st64_b32 %1, %4 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %2, %4 offset0:4 offset1:5\n\tds_read2st64_b32 %3, %4 offset0:6 offset1:7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]) : "v"(addr) : "memory");
  }
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = w[i / 2][i % 2];
}

// The same for a full tile with bf16 outputs, through LDS: the accumulator
// layout gives a store instruction 32 rows x 16 bytes (32 partial cache
// lines), so each 32-token slab of the wave's outputs (32 rows x 128
// features, 8 KiB) is written to the wave's staging area stg, 16-byte chunk
// c of row r at position c ^ (r & 15), and read back as whole rows: a store
// then writes 4 rows x 256 bytes (8 whole lines). Same values as epilogue().
// One wave's LDS operations run in order, so the slabs reuse stg without a
// wait, and the stores consume the reads before any later write to stg.
// FULL: every row and feature of the tile is in range; else slabs past the
// tile's rv rows are skipped and each lane stores only rows below rv and
// features below N (N and the tile's first feature are multiples of 64, so
// a lane's 8 features are all in range or all out).
template <int TM, int ACT, bool FULL>
__device__ __forceinline__ void epilogue_staged(const f32x16_t (&acc)[TN][TM], uint16_t* __restrict__ out,
                                                const TileInfo& t, int N, int wm, int wn,
                                                char* __restrict__ stg) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  constexpr int WM = 32 * TM;
  const int lane = fresh_lane();
  const int l5 = lane & 31, hi = lane >> 5;
  const int orow = __builtin_amdgcn_readfirstlane(t.orow);
  const int n0 = __builtin_amdgcn_readfirstlane(t.n0);
  const int rq = lane >> 4, rc = lane & 15;  // read-back: row 4g + rq, chunk rc
  char* wp = stg + l5 * 256 + 8 * hi;
  // rows of the wave's first slab still in range; features in range
  const int rleft = FULL ? WM : __builtin_amdgcn_readfirstlane(t.rv) - wm * WM;
  const bool col_ok = FULL || n0 + wn * WN + 8 * rc < N;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    if (!FULL && j * 32 >= rleft) break;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x4_t h = {static_cast<__bf16>(activate<ACT>(acc[i][j][4 * q + 0])),
                            static_cast<__bf16>(activate<ACT>(acc[i][j][4 * q + 1])),
                            static_cast<__bf16>(activate<ACT>(acc[i][j][4 * q + 2])),
                            static_cast<__bf16>(activate<ACT>(acc[i][j][4 * q + 3]))};
        *reinterpret_cast<bf16x4_t*>(wp + (((4 * i + q) ^ (l5 & 15)) << 4)) = h;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    uint16_t* o = out + static_cast<int64_t>(orow + wm * WM + j * 32 + rq) * N + n0 + wn * WN + 8 * rc;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int r = 4 * g + rq;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + r * 256 + ((rc ^ (r & 15)) << 4));
      if (FULL || (j * 32 + r < rleft && col_ok))
        *reinterpret_cast<u32x4_t*>(o + static_cast<int64_t>(4 * g) * N) = v;
      if (g % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The persistent tile loop for tiles of BM = 64 TM rows: units tile,
// tile + stride, ... below end, then tile2, tile2 + stride2, ... below end2.
// lds: the two stage rings; s_tiles: the M-tile prefix for this height;
// s_bias: two slices.
// WG: weight-gradient tiles (decode_tile_wg; offsets holds the padded K
// offsets, M the rows of C per expert); else expert-FFN units as the plan
// pl numbers them (decode_tile: whole tiles, then K parts of tail tiles,
// whose parts 1.. go to out2 without bias).
// SP: partly filled bf16 tiles also store through LDS (the short-tile
// kernel, where most tiles are partly filled: the large-E layer's second
// GEMM 900 -> 867 us); the tall-tile kernels keep the direct stores there,
// which need fewer registers (the staged path for partial tiles cost them
// 2-3 more spilled VGPRs and 0.5% on the 16384-token layer).
template <int TM, int OUT, int ACT, bool WG, bool WT = false, bool SP = false>
__device__ __forceinline__ void tile_loop(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_idx,
                                          const uint16_t* __restrict__ W, const float* __restrict__ bias,
                                          void* __restrict__ out, void* __restrict__ out2,
                                          const int32_t* __restrict__ offsets,
                                          int E, int N, const TilePlan& pl, int lda, int64_t w_estride, int M,
                                          char* lds, const int* s_tiles, float (*s_bias)[BN], int tile,
                                          int stride, int end, int tile2, int stride2, int end2, int NT) {
  constexpr int BM = 64 * TM;
  constexpr int WM = BM / 2;         // tokens per wave
  constexpr int A_BYTES = BM * ROWB;  // one token stage
  constexpr int W_BYTES = BN * ROWB;  // one weight stage (BK rows of kWtRowB bytes when WT)
  static_assert(W_BYTES == BK * kWtRowB, "both weight layouts fill the same stage size");
  constexpr int LA = BM / 32;        // 1 KiB (8-row) DMA blocks of the token tile per wave
  constexpr int LB = BN / 32;        // 1 KiB DMA blocks of the weight tile per wave
  static_assert(LB == 8, "stage_w_b8 issues a weight stage");
  constexpr int NA = a_stages<TM>();
  constexpr int NW = w_stages<TM>();
  // K parts only for y_perm outputs (the second expert GEMM): other kernels
  // keep the plain unit sequence and decode (fewer live registers)
  constexpr bool PARTS = !WG && OUT == kOutYperm;
  constexpr int NMIN = NA < NW ? NA : NW;  // refills run while stage t + NMIN exists
  constexpr int NMAX = NA > NW ? NA : NW;
  static_assert(NA <= NW && NW <= NA + 1, "sched_steady_loads holds for rings with NA <= NW <= NA + 1");
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
  // a unit's tile is the same for the whole wave: its fields go to scalar
  // registers (the DMA asm takes its base addresses as SGPRs)
  auto decode = [&](int tl) {
    TileInfo t;
    if constexpr (WG) t = decode_tile_wg(tl, s_tiles, offsets, E, NT, BM, M);
    else t = decode_tile<PARTS>(tl, s_tiles, offsets, E, NT, BM, pl);
    if constexpr (PARTS) {
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
    t.rv = __builtin_amdgcn_readfirstlane(t.rv);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    t.arow = __builtin_amdgcn_readfirstlane(t.arow);
    t.k0 = __builtin_amdgcn_readfirstlane(t.k0);
    t.nk = __builtin_amdgcn_readfirstlane(t.nk);
    t.part = __builtin_amdgcn_readfirstlane(t.part);
    t.orow = __builtin_amdgcn_readfirstlane(t.orow);
    }
    return t;
  };
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const uint32_t w_base = lds_base + NA * A_BYTES;
  auto a_slot = [&](int i) { return lds_base + static_cast<uint32_t>(i * A_BYTES); };
  auto w_slot = [&](int j) { return w_base + static_cast<uint32_t>(j * W_BYTES); };
  const uint32_t trow = wm * WM * ROWB;  // this wave's token rows in a token stage
  const uint32_t wrow = wn * WN * ROWB;  // this wave's weight rows in a weight stage
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
    for (int i = 0; i < TN; ++i) wo[i] = rb + 64 * ((4 * wn + i) ^ key4);
  }
  // bytes from one K stage of W to the next
  const int64_t wst = WT ? static_cast<int64_t>(BK) * N * 2 : ROWB;
  auto wadr = [&](uint32_t sbase, int s, uint32_t (&wa)[TN]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) wa[i] = sbase + wo[i] + s * 16 * kWtRowB;
  };

  uint32_t aoffs[LA], boffs[LB], vo[LA + LB];
  const char* Abase;
  const char* Wbase;
  // a tile's stage 0 and its bias slice (wave 0, one lane per 4 features):
  // issued before the previous tile's epilogue
  auto prologue0 = [&](const TileInfo& c, int par) {
    issue_stage<TM>(aoffs, boffs, a_slot(0) + wave * LA * 1024, w_slot(0) + wave * LB * 1024, Abase, Wbase);
    if (bias != nullptr && c.part == 0 && wave == 0)
      issue_bias(bias + static_cast<int64_t>(c.e) * N + min(c.n0 + 4 * fresh_lane(), N - 4),
                 static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_bias[par][0])));
  };
  // its stages 1 .. min(NW, nk) - 1 (token stage p only while p < NA):
  // issued after the previous tile's epilogue stores
  // Parking place of the next tile's DMA offsets during the epilogue: this
  // wave's own part of token slot 1 (of slots 2 and 1 for 64-row tiles,
  // whose part of a slot holds 8 words), free from the last stage's barrier
  // until prologue1 below refills it, after reading them back.
  static_assert(TM > 1 || NA >= 3, "64-row tiles park their token offsets in token slot 2");
  auto park_base = [&]() {
    return a_slot(1) + static_cast<uint32_t>(wave * LA * 1024 + 4 * fresh_lane());
  };
  auto park = [&]() {
    const uint32_t pb = park_base();
    park_words<LB>(boffs, pb);
    if constexpr (TM > 1) park_words<LA>(aoffs, pb + LB * 256);
    else park_words<LA>(aoffs, pb + A_BYTES);
  };
  auto unpark = [&]() {
    const uint32_t pb = park_base();
    unpark_words<LB>(boffs, pb);
    if constexpr (TM > 1) unpark_words<LA>(aoffs, pb + LB * 256);
    else unpark_words<LA>(aoffs, pb + A_BYTES);
  };
  auto prologue1 = [&](int nk) {
    for (int p = 1; p < NMAX && p < nk; ++p) {
      if (p < NA && p < NW)
        issue_stage<TM>(aoffs, boffs, a_slot(p) + wave * LA * 1024, w_slot(p) + wave * LB * 1024,
                        Abase + p * ROWB, Wbase + p * wst);
      else if (p < NW)
        stage_w_b8(boffs, w_slot(p) + wave * LB * 1024, Wbase + p * wst);
      else
        stage_a<TM>(aoffs, a_slot(p) + wave * LA * 1024, Abase + p * ROWB);
    }
  };
  int par = 0;  // bias slice of the current tile
  TileInfo cur = decode(tile);
  tile_sources<LA, LB, WT>(cur, A, row_idx, W, N, lda, w_estride, wave, Abase, Wbase, aoffs,
                           boffs);
  prologue0(cur, par);
  prologue1((WG || PARTS) ? cur.nk : pl.nk);

  for (;;) {
    // K stages of this tile (cur moves on before its epilogue)
    const int nk = (WG || PARTS) ? cur.nk : pl.nk;

    // stage 0 and the bias slice have landed (the later prologue stages may
    // still be in flight)
    wait_vm(prologue_loads<NA, NW, LA, LB>(nk));
    __syncthreads();
    // accumulators start at the bias: lane (l5, hi) holds features
    // fb + 32 i + 8 q + {0..3} of tile i (the same for every token tile j)
    f32x16_t acc[TN][TM];
    {
      const bool with_bias = bias != nullptr && cur.part == 0;
      const int fb = wn * WN + (fresh_lane() >> 5) * 4;
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
      wadr(w_slot(0), 0, wa);
      read_frags_t<TM>(wf0, tf0, a_slot(0) + trow + fo[0], wa);
    } else {
      read_frags<TM>(wf0, tf0, a_slot(0) + trow + fo[0], w_slot(0) + wrow + fo[0]);
    }

    TileInfo done = cur;
    // the next unit: on in this sequence, else the first of the second
    int next = tile + stride;
    const bool second = PARTS && next >= end;
    if (second) next = tile2;
    const bool more = second ? tile2 < end2 : next < end;
#pragma unroll
    for (int i = 0; i < LA; ++i) vo[i] = aoffs[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) vo[LA + i] = boffs[i];
    int ai = 0, wi = 0;  // ring slots of stage t
    int t = 0;
    // the second half of the last refill, issued with the next stage's first
    // K16 step: its LDS and global bases
    uint32_t pla = 0, plb = 0;
    const char* pga = nullptr;
    const char* pgw = nullptr;
    // one K16 step reading the fragments of step s of the stage in slots sa, sw
    auto kstep = [&](const bf16x8_t (&w)[TN], const bf16x8_t (&tk)[TM], bf16x8_t (&nw)[TN],
                     bf16x8_t (&nt)[TM], uint32_t sa, uint32_t sw, int s) {
      if constexpr (WT) {
        uint32_t wa[TN];
        wadr(sw, s, wa);
        step_t<TM>(acc, w, tk, nw, nt, sa + trow + fo[s], wa);
      } else {
        step<TM>(acc, w, tk, nw, nt, sa + trow + fo[s], sw + wrow + fo[s]);
      }
    };
    // the same with half of a refill's LDS-DMA loads
    auto kstep_dma = [&](auto half, const bf16x8_t (&w)[TN], const bf16x8_t (&tk)[TM], bf16x8_t (&nw)[TN],
                         bf16x8_t (&nt)[TM], uint32_t sa, uint32_t sw, int s) {
      constexpr int H = decltype(half)::value;
      if constexpr (WT) {
        uint32_t wa[TN];
        wadr(sw, s, wa);
        step_dma_t<TM, H>(acc, w, tk, nw, nt, sa + trow + fo[s], wa, vo, pla, plb, pga, pgw);
      } else {
        step_dma<TM, H>(acc, w, tk, nw, nt, sa + trow + fo[s], sw + wrow + fo[s], vo, pla, plb, pga, pgw);
      }
    };
    // One K stage. D1: step 0 issues the second half of the previous refill;
    // RF: refill this stage's buffers (token stage t + NA, weight stage
    // t + NW) once every wave has read the stage; a stage past the last one
    // loads the last one again, into a buffer no later stage reads, so every
    // refill has the same loads.
    auto stage = [&](auto d1, auto rf) {
      const uint32_t sa = a_slot(ai), sw = w_slot(wi);
      // K16 steps 0..2, each reading the next step's fragments
      if constexpr (decltype(d1)::value)
        kstep_dma(std::integral_constant<int, 1>{}, wf0, tf0, wf1, tf1, sa, sw, 1);
      else
        kstep(wf0, tf0, wf1, tf1, sa, sw, 1);
      kstep(wf1, tf1, wf0, tf0, sa, sw, 2);
      kstep(wf0, tf0, wf1, tf1, sa, sw, 3);
      // stage t+1 has landed and every wave has read its last fragments of
      // stage t (a refilling stage waits for the rings' fixed count)
      if constexpr (decltype(rf)::value)
        wait_vm_n<sched_steady_loads(NA, NW, LA, LB)>();
      else
        wait_vm(loads_after<NA, NW, LA, LB>(t, nk));
      __syncthreads();
      const int an = (ai + 1 == NA) ? 0 : ai + 1;
      const int wnx = (wi + 1 == NW) ? 0 : wi + 1;
      // K16 step 3; read step 0 of stage t+1
      if constexpr (decltype(rf)::value) {
        // half of the refill's loads now, the rest with step 0 of stage t+1
        pla = sa + wave * LA * 1024;
        plb = sw + wave * LB * 1024;
        pga = Abase + min(t + NA, nk - 1) * ROWB;
        pgw = Wbase + min(t + NW, nk - 1) * wst;
        kstep_dma(std::integral_constant<int, 0>{}, wf1, tf1, wf0, tf0, a_slot(an), w_slot(wnx), 0);
      } else {
        kstep(wf1, tf1, wf0, tf0, a_slot(an), w_slot(wnx), 0);
      }
      ai = an;
      wi = wnx;
    };
    using yes = std::true_type;
    using no = std::false_type;
    if (t + NMIN < nk) {
      // steady state; the first stage without a refill (there is one, as
      // NMIN >= 2) issues the last refill's second half
      stage(no{}, yes{});
      for (++t; t + NMIN < nk; ++t) stage(yes{}, yes{});
      stage(yes{}, no{});
      ++t;
    }
    // the last stages: nothing more to load
    for (; t + 1 < nk; ++t) stage(no{}, no{});
    // the last stage
    {
      const uint32_t sa = a_slot(ai), sw = w_slot(wi);
      kstep(wf0, tf0, wf1, tf1, sa, sw, 1);
      kstep(wf1, tf1, wf0, tf0, sa, sw, 2);
      kstep(wf0, tf0, wf1, tf1, sa, sw, 3);
    }
    // the last K16 step's MFMAs (fragments already in registers) run while
    // the wave meets the others and sets up the next tile
    last_step<TM>(acc, wf1, tf1);
    // every wave has read all of its fragments: all buffers are free, and the
    // next tile's stage 0 loads during this tile's epilogue
    __syncthreads();
    if (more) {
      cur = decode(next);
      tile_sources<LA, LB, WT>(cur, A, row_idx, W, N, lda, w_estride, wave, Abase, Wbase,
                               aoffs, boffs);
      prologue0(cur, par ^ 1);
      park();
    }

    // ---- epilogue: lane holds token l5 of each 32-token tile j and
    // features 8q + 4*hi + {0..3} of each 32-feature tile i
    const bool full_tile = done.rv == BM && done.n0 + BN <= N;
    void* dst = done.part ? out2 : out;
    if constexpr (OUT != kOutF32) {
      // Staging area: this wave's own 8 KiB of a weight slot other than 0
      // (the next tile's stage 0). The wave itself refills that region in
      // prologue1, after these reads. With NW = NA + 1 the last refill of
      // the K loop loaded a stage past the last one into weight slot
      // nk % NW and nothing has waited for it, so that slot is avoided.
      const int ws = (NW > NA && nk % NW == 1) ? 2 : 1;
      char* stg = lds + NA * A_BYTES + ws * W_BYTES + wave * LB * 1024;
      if (full_tile) {
        epilogue_staged<TM, ACT, true>(acc, static_cast<uint16_t*>(dst), done, N, wm, wn, stg);
      } else if constexpr (SP) {
        epilogue_staged<TM, ACT, false>(acc, static_cast<uint16_t*>(dst), done, N, wm, wn, stg);
      } else {
        const int fl = fresh_lane();
        epilogue<TM, OUT, ACT, false>(acc, dst, done, N, wm, wn, fl & 31, fl >> 5);
      }
    } else {
      const int fl = fresh_lane();
      if (full_tile) epilogue<TM, OUT, ACT, true>(acc, dst, done, N, wm, wn, fl & 31, fl >> 5);
      else epilogue<TM, OUT, ACT, false>(acc, dst, done, N, wm, wn, fl & 31, fl >> 5);
    }
    if (!more) break;
    // the next tile's later prologue stages, after this tile's stores
    unpark();
    prologue1((WG || PARTS) ? cur.nk : pl.nk);
    tile = next;
    if (second) {
      stride = stride2;
      end = end2;
      tile2 = end2;
    }
    par ^= 1;
  }
}

}  // namespace

// SHORT selects the tile heights: 256 or 192 rows (experts that can hold
// many tall tiles), or 192, 128 or 64 rows (every expert holds at most 512
// rows: decode batches, many experts). Two instantiations rather than one
// kernel with all four: each keeps its own register allocation.
// OUT: kOutBf16 (after ACT), kOutF32, or kOutYperm (no activation, bf16).
// out2 (kOutYperm only, else null; cap_rows bf16 rows of N): with it, the
// schedule may run tiles as K parts (TilePlan: all tiles in two halves, or
// the last M tiles in p parts). nsplit (when not null) receives p (1: no
// parts), the first row of the split tiles, r_tail, and their row count,
// tail_rows. A row r < r_tail of out is then a result, and a row
// r >= r_tail the sum, in order, of out's row r and out2's rows
// (j - 1) tail_rows + r - r_tail, j = 1 .. p - 1 (each part rounded to
// bf16).
// WT: each W_e is stored [K, N] (K-major, as W^T of the usual [N, K]); the
// weight stages are loaded row by row of K and read with transposing LDS
// reads.
template <int OUT, int ACT, bool SHORT, bool WT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_idx,
                              const uint16_t* __restrict__ W,
                              const float* __restrict__ bias, void* __restrict__ out,
                              void* __restrict__ out2, int32_t* __restrict__ nsplit,
                              const int32_t* __restrict__ offsets, int E, int N, int K, int cap_rows) {
  // the body uses gfx950 builtins only: the host pass needs just the signature
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) char lds[SHORT ? kLdsShort : kLdsTall];
  __shared__ int s_tiles[1025];  // exclusive prefix of M tiles per expert
  // the schedule's partial sums live in the stage rings, which no load
  // touches before the schedule is done (a barrier follows it)
  int (*s_part)[256] = reinterpret_cast<int (*)[256]>(lds);
  __shared__ __attribute__((aligned(16))) float s_bias[2][BN];  // bias slices of this and the next tile

  const int tid = threadIdx.x;
  const int NT = (N + BN - 1) / BN;
  const int Gd = gridDim.x;
  const int per = (E + 255) / 256;
  const int eb = tid * per;
  const int b = blockIdx.x;
  const int64_t wes = static_cast<int64_t>(N) * K;
  const int nks = K / BK;
  // ---- device-side schedule. Tile heights: 256 or 192 (tall), 192, 128 or
  // 64 (short). For each height the M tiles per expert are counted and
  // prefix-summed; then every plan is costed as the work of the busiest
  // block, in row-K units: rounds x (rows x K + rows x kEpiK), where rows
  // are the tile's MFMA rows plus a share for the weight panel it streams
  // whole (kTallShare, charged to the K loop only, in the tall kernel; 64
  // rows in the short one).
  constexpr int NQ = SHORT ? 3 : 2;
  constexpr int kH[3] = {SHORT ? 192 : 256, SHORT ? 128 : 192, 64};
  auto unit_cost = [&](int h, int p) {  // one tile of height h, K split in p parts
    if constexpr (SHORT)
      return static_cast<int64_t>(h + 64) * (nks / p * BK + kEpiK);
    else
      return static_cast<int64_t>(h + kTallShare) * (nks / p * BK) + static_cast<int64_t>(h) * kEpiK;
  };
  int c[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) c[q] = 0;
  for (int e = eb; e < min(E, eb + per); ++e) {
    const int n = offsets[e + 1] - offsets[e];
#pragma unroll
    for (int q = 0; q < NQ; ++q) c[q] += (n + kH[q] - 1) / kH[q];
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) s_part[q][tid] = c[q];
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int a[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) a[q] = (tid >= off) ? s_part[q][tid - off] : 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NQ; ++q) s_part[q][tid] += a[q];
    __syncthreads();
  }
  // Plans: whole tiles of one height (the taller first, so it wins a tie),
  // then, with out2, K parts:
  //  * every tile in two K halves, when the whole tiles fit in one round
  //    (few rows, long K: decode batches);
  //  * after at least two rounds of whole tiles, the last M tiles (enough
  //    of them, with all their feature panels, to hold the tiles that would
  //    run in a last, partly filled round) in p K parts, as many as still
  //    fit in one round, at most kMaxParts: the last round then runs short
  //    parts on most blocks instead of whole tiles on a few. On the
  //    16384-token layer's second GEMM (2144 tiles): 8 rounds of 256 whole
  //    tiles, and the 96 tiles left (6 M tiles) run as 192 half tiles.
  //  A split only to even out one round after a single round of whole
  //  tiles is not offered: on the skewed layer's second GEMM (352 tiles,
  //  K = 1024) the parts ran no faster and the combine, which adds their
  //  fp32 rows, took 25.8 µs instead of 12.7.
  int sel = 0, P = 1, MT = 0;
  int64_t best = -1;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t tiles = static_cast<int64_t>(s_part[q][255]) * NT;
    const int64_t cq = (tiles + Gd - 1) / Gd * unit_cost(kH[q], 1);
    if (best < 0 || cq < best) {
      best = cq;
      sel = q;
    }
  }
  if (OUT == kOutYperm && out2 != nullptr) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int mtq = s_part[q][255];
      const int64_t tiles = static_cast<int64_t>(mtq) * NT;
      int p = 1, mt = 0;
      int64_t cq = -1;
      if (tiles > 0 && tiles <= Gd) {
        if (nks % 2 == 0) {
          p = 2;
          mt = mtq;
          cq = (2 * tiles + Gd - 1) / Gd * unit_cost(kH[q], 2);
        }
      } else if (tiles > Gd) {
        const int64_t full = tiles / Gd, rest = tiles % Gd;
        if (full >= 2 && rest > 0) {
          mt = static_cast<int>((rest + NT - 1) / NT);
          for (int pp = min(Gd / (mt * NT), kMaxParts); pp >= 2; --pp)
            if (nks % pp == 0 && static_cast<int64_t>(pp - 1) * mt * kH[q] <= cap_rows) {
              p = pp;
              break;
            }
          if (p > 1) cq = full * unit_cost(kH[q], 1) + unit_cost(kH[q], p);
        }
      }
      if (cq >= 0 && cq < best) {
        best = cq;
        sel = q;
        P = p;
        MT = mt;
      }
    }
  }
  const int BMs = kH[sel];
  int many = 0;  // an expert of this thread has more than 2 kGroupM M tiles
  {
    int run = s_part[sel][tid] - c[sel];
    for (int e = eb; e < min(E, eb + per); ++e) {
      s_tiles[e] = run;
      const int mt = (offsets[e + 1] - offsets[e] + BMs - 1) / BMs;
      many |= mt > 2 * kGroupM;
      run += mt;
    }
    if (tid == 255) s_tiles[E] = s_part[sel][255];
  }
  // (also the barrier after s_tiles)
  const bool reread = __syncthreads_or(many) != 0;
  TilePlan pl;
  pl.mcap = s_tiles[E] - MT;
  pl.nk = nks;
  pl.p = P;
  pl.nkp = nks / P;
  pl.mt = MT;
  pl.r_tail = offsets[E];
  if (MT > 0) {
    int lo = 0, hi = E - 1;  // the expert of M tile mcap
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tiles[mid] <= pl.mcap) lo = mid;
      else hi = mid - 1;
    }
    pl.r_tail = offsets[lo] + (pl.mcap - s_tiles[lo]) * BMs;
  }
  pl.tail_rows = offsets[E] - pl.r_tail;
  if (nsplit != nullptr && b == 0 && tid == 0) {
    nsplit[0] = P;
    nsplit[1] = pl.r_tail;
    nsplit[2] = pl.tail_rows;
  }
  // this block's units (sched_xcd_plan; reread: some expert has more M
  // tiles than one group of the tile order holds, so its weight panels are
  // read more than once): whole tiles first, then tail parts
  const int dp = pl.mcap * NT;
  const int nparts = P > 1 ? P * MT * NT : 0;
  int first, stride, end, first2, stride2, end2;
  sched_xcd_plan(b, Gd, dp, reread, first, stride, end);
  sched_xcd_plan(b, Gd, nparts, reread, first2, stride2, end2);
  first2 += dp;
  end2 += dp;
  if (first >= end) {
    if (first2 >= end2) return;
    first = first2;
    stride = stride2;
    end = end2;
    first2 = end2;
  }
#define MOE_TILE_LOOP(TMV)                                                                                \
  tile_loop<TMV, OUT, ACT, false, WT, SHORT>(A, row_idx, W, bias, out, out2, offsets, E, N, pl, K, wes, 0, lds, \
                                      s_tiles, s_bias, first, stride, end, first2, stride2, end2, NT)
  // each kernel instantiates only its own heights (separate register
  // allocations)
  if constexpr (!SHORT) {
    if (BMs == 256) MOE_TILE_LOOP(4);
    else MOE_TILE_LOOP(3);
  } else {
    if (BMs == 192) MOE_TILE_LOOP(3);
    else if (BMs == 128) MOE_TILE_LOOP(2);
    else MOE_TILE_LOOP(1);
  }
#undef MOE_TILE_LOOP
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
  const TilePlan pl{};  // unused by weight-gradient tiles
  tile_loop<4, kOutF32, kActNone, true>(At, nullptr, Bt, nullptr, C, nullptr, poff, E, N, pl, lda, 0, M,
                                     lds, s_tiles, s_bias, tile, Gd, total, total, 1, total, NT);
#endif
}

namespace {

std::atomic<int> g_max_blocks{0};  // 0: no cap

// persistent blocks for one GEMM launch: one per CU, at most the cap
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  int n = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    if (cached[dev] == 0) {
      int c = 0;
      if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
        c = 256;
      cached[dev] = c;
    }
    n = cached[dev];
  }
  const int cap = g_max_blocks.load(std::memory_order_relaxed);
  return cap > 0 && cap < n ? cap : n;
}

}  // namespace

void set_gemm_max_blocks(int blocks) { g_max_blocks.store(blocks, std::memory_order_relaxed); }

hipError_t launch_gemm_bf16(const uint16_t* A, const int32_t* row_idx, const uint16_t* W,
                            const float* bias, void* out, void* out2, int32_t* nsplit,
                            int out_mode, int act, const int32_t* offsets, int E, int N, int K,
                            int64_t max_rows, int max_rows_per_expert, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  // K parts: y_perm outputs only (the combine adds the parts)
  if (out_mode != kGemmOutYperm) out2 = nullptr;
  const int smax = (out2 != nullptr && (K / BK) % 2 == 0) ? 2 : 1;
  // short tiles (192, 128, 64 rows) when no expert can hold more than two
  // 256-row tiles: ragged experts of a few hundred rows pad less with the
  // finer heights. The skewed layer (64 experts, capacity 512) ran its GEMMs
  // 44 / 54 µs that way against 50 / 60 µs with the tall heights; the small
  // layer (capacity 1280) did not gain.
  const bool shorter = max_rows_per_expert <= 512;
  // upper bound on tiles: sum_e ceil(n_e/h) <= max_rows/h + E for the shortest h
  const int64_t mt_bound = max_rows / (shorter ? 64 : 192) + E;
  const int slots = cu_count();
  const int64_t tiles = mt_bound * ((N + BN - 1) / BN) * smax;
  const unsigned grid = static_cast<unsigned>(tiles < slots ? tiles : slots);
  const int cap = static_cast<int>(max_rows < INT32_MAX ? max_rows : INT32_MAX);  // rows of out2
#define MOE_GEMM(OM, AC)                                                                              \
  do {                                                                                               \
    if (shorter)                                                                                     \
      klaunch(grouped_gemm_bf16_kernel<OM, AC, true>, dim3(grid), dim3(256), 0, s, A, row_idx, W, bias, \
              out, out2, nsplit, offsets, E, N, K, cap);                           \
    else                                                                                             \
      klaunch(grouped_gemm_bf16_kernel<OM, AC, false>, dim3(grid), dim3(256), 0, s, A, row_idx, W,     \
              bias, out, out2, nsplit, offsets, E, N, K, cap);                     \
  } while (0)
  if (out_mode == kGemmOutYperm) MOE_GEMM(kOutYperm, kActNone);
  else if (out_mode == kGemmOutF32) MOE_GEMM(kOutF32, kActNone);
  else if (act == kActRelu) MOE_GEMM(kOutBf16, kActRelu);
  else if (act == kActGeluTanh) MOE_GEMM(kOutBf16, kActGeluTanh);
  else MOE_GEMM(kOutBf16, kActNone);
#undef MOE_GEMM
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
    grouped_gemm_bf16_kernel<kOutF32, kActNone, true, true><<<grid, 256, 0, s>>>(
        A, row_idx, W, bias, out, nullptr, nullptr, offsets, E, N, K, 0);
  else
    grouped_gemm_bf16_kernel<kOutF32, kActNone, false, true><<<grid, 256, 0, s>>>(
        A, row_idx, W, bias, out, nullptr, nullptr, offsets, E, N, K, 0);
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
