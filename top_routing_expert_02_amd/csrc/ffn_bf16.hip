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
//  * Block tile BM=256 tokens x BN=256 features, K in steps of BK=32; four
//    waves in a 2x2 grid; each wave owns 128 tokens x 128 features as 32x32
//    v_mfma_f32_32x32x16_bf16 tiles (fp32 accumulators in AGPRs). The weight tile is the MFMA A operand and the token tile the B
//    operand, so a lane's accumulators hold 4 consecutive features of one
//    token: the epilogue stores 8-byte (bf16) or 16-byte (fp32) vectors.
//  * LDS holds four stages of both tiles (128 KiB at BN=256): tiles kt+1..kt+3
//    are in flight while kt computes. Rows are 64 B (32 bf16); the four
//    16-byte chunks of a row are XOR-swizzled by the row's 256-byte block,
//    which makes the fragment reads conflict-free.
//  * Tiles move global -> LDS with gfx950's LDS-DMA loads (global_load_lds_
//    dwordx4: no staging registers, no ds_write); each lane fetches the chunk
//    the swizzle places at its LDS slot; one barrier per stage. In the steady
//    state a stage's loads are spread between the MFMAs of the K16 step that
//    follows the barrier; the next tile's first stages load during the
//    current tile's last MFMAs and epilogue.
//  * Persistent blocks, one per CU. The schedule is computed on the device
//    from expert_offsets (no host read-back): expert-major tiles, M tiles of
//    an expert innermost, so concurrent tiles share weight panels. Blocks are
//    renumbered so that consecutive tiles run on one XCD (blocks are dealt to
//    the 8 XCDs round-robin) and share its L2.
//  * Ragged M: rows past an expert's end read that expert's last row and are
//    never stored, so no tile reads outside [0, rows).
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM;   // 256 token rows per tile
constexpr int BK = 32;        // K per LDS stage
[[maybe_unused]] constexpr int ROWB = BK * 2;  // bytes per LDS row (64)

// Row r of a stage holds its 16-byte chunk c at position c ^ swz_key(r): the
// key is the row's 256-byte block (mod 4). With it the MFMA fragment reads
// (32 consecutive rows at one chunk, per ds_read_b128) run at the LDS's full
// 256 B/clk (4 cycles per instruction); measured with SQ_LDS_BANK_CONFLICT,
// unswizzled rows take 16 cycles and keys r&3 or (r/2)&3 take 8.
__device__ __forceinline__ int swz_key(int row) { return (row >> 2) & 3; }

typedef __attribute__((address_space(3))) void lds_void_t;

// Queue one stage (BK columns of the token and weight tiles) with LDS-DMA
// loads. One global_load_lds_dwordx4 fills 1 KiB = 16 rows of 64 B; wave w's
// instruction i fills block w*L+i.
template <int LA, int LB, int A_BYTES>
__device__ __forceinline__ void issue_stage(const char* ak, const char* wk, char* sb,
                                            const uint32_t (&aoffs)[LA],
                                            const uint32_t (&boffs)[LB], int wave) {
#pragma unroll
  for (int i = 0; i < LA; ++i)
    __builtin_amdgcn_global_load_lds(ak + aoffs[i], (lds_void_t*)(sb + (wave * LA + i) * 1024), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < LB; ++i)
    __builtin_amdgcn_global_load_lds(wk + boffs[i], (lds_void_t*)(sb + A_BYTES + (wave * LB + i) * 1024),
                                     16, 0, 0);
}

// ---- hand-scheduled K16 steps
//
// A wave issues MFMAs one at a time (an MFMA waits for the matrix core), so
// LDS latency is hidden only by reads issued between MFMAs. The compiler
// cannot place them there: its wait insertion treats any LDS read as
// dependent on every LDS-DMA load in flight and waits for all of them, which
// would serialise the stage pipeline. Each block below therefore issues the
// MFMAs of one K16 step interleaved with the reads of the next step's
// fragments, and waits for those reads before it ends: no read is in flight
// past a block. Stage order is explicit (wait_stage and a barrier before a
// stage is read). Each block starts with two wait states (a VALU write of an
// MFMA source register needs them).
//   acc[i][j] += W_i * T_j: W = weight fragments (MFMA A operand),
//   T = token fragments (B operand); next fragments from ta / wa, tiles
//   2048 B apart.
#define MOE_MFMA(D, A, B) "v_mfma_f32_32x32x16_bf16 " D ", " A ", " B ", " D "\n\t"
#define MOE_RD(D, ADDR, OFF) "ds_read_b128 " D ", " ADDR " offset:" OFF "\n\t"

__device__ __forceinline__ void step_4x4(f32x16_t (&acc)[4][4], const bf16x8_t (&w)[4],
                                         const bf16x8_t (&t)[4], bf16x8_t (&nw)[4],
                                         bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa) {
  asm volatile(
      MOE_RD("%16", "%32", "0") MOE_RD("%17", "%32", "2048")
      MOE_RD("%18", "%32", "4096") MOE_RD("%19", "%32", "6144")
      MOE_RD("%20", "%33", "0") MOE_RD("%21", "%33", "2048")
      MOE_RD("%22", "%33", "4096") MOE_RD("%23", "%33", "6144")
      MOE_MFMA("%0", "%24", "%28") MOE_MFMA("%1", "%24", "%29")
      MOE_MFMA("%2", "%24", "%30") MOE_MFMA("%3", "%24", "%31")
      MOE_MFMA("%4", "%25", "%28") MOE_MFMA("%5", "%25", "%29")
      MOE_MFMA("%6", "%25", "%30") MOE_MFMA("%7", "%25", "%31")
      MOE_MFMA("%8", "%26", "%28") MOE_MFMA("%9", "%26", "%29")
      MOE_MFMA("%10", "%26", "%30") MOE_MFMA("%11", "%26", "%31")
      MOE_MFMA("%12", "%27", "%28") MOE_MFMA("%13", "%27", "%29")
      MOE_MFMA("%14", "%27", "%30") MOE_MFMA("%15", "%27", "%31")
      "s_waitcnt lgkmcnt(0)"
      : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
        "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
        "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
        "+a"(acc[3][3]), "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]), "=&v"(nt[3]), "=&v"(nw[0]),
        "=&v"(nw[1]), "=&v"(nw[2]), "=&v"(nw[3])
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]),
        "v"(ta), "v"(wa)
      : "memory");
}

__device__ __forceinline__ void last_4x4(f32x16_t (&acc)[4][4], const bf16x8_t (&w)[4],
                                         const bf16x8_t (&t)[4]) {
  asm volatile(
      "s_nop 1\n\t"
      MOE_MFMA("%0", "%16", "%20") MOE_MFMA("%1", "%16", "%21") MOE_MFMA("%2", "%16", "%22")
      MOE_MFMA("%3", "%16", "%23") MOE_MFMA("%4", "%17", "%20") MOE_MFMA("%5", "%17", "%21")
      MOE_MFMA("%6", "%17", "%22") MOE_MFMA("%7", "%17", "%23") MOE_MFMA("%8", "%18", "%20")
      MOE_MFMA("%9", "%18", "%21") MOE_MFMA("%10", "%18", "%22") MOE_MFMA("%11", "%18", "%23")
      MOE_MFMA("%12", "%19", "%20") MOE_MFMA("%13", "%19", "%21") MOE_MFMA("%14", "%19", "%22")
      MOE_MFMA("%15", "%19", "%23")
      // results are read by VALU next (accumulator moves): 24 wait states
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
        "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
        "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
        "+a"(acc[3][3])
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3])
      : "memory");
}

__device__ __forceinline__ void step_4x2(f32x16_t (&acc)[2][4], const bf16x8_t (&w)[2],
                                         const bf16x8_t (&t)[4], bf16x8_t (&nw)[2],
                                         bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa) {
  asm volatile(
      MOE_RD("%8", "%20", "0") MOE_RD("%9", "%20", "2048")
      MOE_RD("%10", "%20", "4096") MOE_RD("%11", "%20", "6144")
      MOE_RD("%12", "%21", "0") MOE_RD("%13", "%21", "2048")
      MOE_MFMA("%0", "%14", "%16") MOE_MFMA("%1", "%14", "%17")
      MOE_MFMA("%2", "%14", "%18") MOE_MFMA("%3", "%14", "%19")
      MOE_MFMA("%4", "%15", "%16") MOE_MFMA("%5", "%15", "%17")
      MOE_MFMA("%6", "%15", "%18") MOE_MFMA("%7", "%15", "%19")
      "s_waitcnt lgkmcnt(0)"
      : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
        "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]),
        "=&v"(nt[3]), "=&v"(nw[0]), "=&v"(nw[1])
      : "v"(w[0]), "v"(w[1]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(ta), "v"(wa)
      : "memory");
}

__device__ __forceinline__ void last_4x2(f32x16_t (&acc)[2][4], const bf16x8_t (&w)[2],
                                         const bf16x8_t (&t)[4]) {
  asm volatile(
      "s_nop 1\n\t"
      MOE_MFMA("%0", "%8", "%10") MOE_MFMA("%1", "%8", "%11") MOE_MFMA("%2", "%8", "%12")
      MOE_MFMA("%3", "%8", "%13") MOE_MFMA("%4", "%9", "%10") MOE_MFMA("%5", "%9", "%11")
      MOE_MFMA("%6", "%9", "%12") MOE_MFMA("%7", "%9", "%13")
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
        "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3])
      : "v"(w[0]), "v"(w[1]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3])
      : "memory");
}

// The same K16 steps with the next stage's LDS-DMA loads spread between the
// MFMAs (one load per one or two MFMAs). Issued as a burst right after the
// barrier, the four waves' loads queue at the address unit together and the
// waves stall behind them; spread out, they issue in the MFMA shadow. M0
// carries the LDS destination of each load (lane L writes bytes 16L..16L+15
// of a 1 KiB block); la / lb are this wave's first token / weight block of the
// stage being refilled, ga / gw the global bases of its K columns, vo the
// per-lane byte offsets (token blocks first, then weight blocks).
// M0 is reserved by the compiler, which sets it again before each LDS-DMA
// load of its own; the clobber below orders those against these blocks.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#define MOE_M0(BASE, OFF) "s_add_u32 m0, " BASE ", " OFF "\n\t"
#define MOE_DMA(V, G) "global_load_lds_dwordx4 " V ", " G "\n\t"

__device__ __forceinline__ void step_dma_4x4(f32x16_t (&acc)[4][4], const bf16x8_t (&w)[4],
                                             const bf16x8_t (&t)[4], bf16x8_t (&nw)[4],
                                             bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa,
                                             const uint32_t (&vo)[8], uint32_t la, uint32_t lb,
                                             const char* ga, const char* gw) {
  asm volatile(
      MOE_RD("%16", "%32", "0") MOE_RD("%17", "%32", "2048")
      MOE_RD("%18", "%32", "4096") MOE_RD("%19", "%32", "6144")
      MOE_RD("%20", "%33", "0") MOE_RD("%21", "%33", "2048")
      MOE_RD("%22", "%33", "4096") MOE_RD("%23", "%33", "6144")
      MOE_M0("%42", "0") MOE_MFMA("%0", "%24", "%28") MOE_DMA("%34", "%44")
      MOE_M0("%42", "0x400") MOE_MFMA("%1", "%24", "%29") MOE_MFMA("%2", "%24", "%30")
      MOE_DMA("%35", "%44")
      MOE_M0("%42", "0x800") MOE_MFMA("%3", "%24", "%31") MOE_MFMA("%4", "%25", "%28")
      MOE_DMA("%36", "%44")
      MOE_M0("%42", "0xc00") MOE_MFMA("%5", "%25", "%29") MOE_MFMA("%6", "%25", "%30")
      MOE_DMA("%37", "%44")
      MOE_M0("%43", "0") MOE_MFMA("%7", "%25", "%31") MOE_MFMA("%8", "%26", "%28")
      MOE_DMA("%38", "%45")
      MOE_M0("%43", "0x400") MOE_MFMA("%9", "%26", "%29") MOE_MFMA("%10", "%26", "%30")
      MOE_DMA("%39", "%45")
      MOE_M0("%43", "0x800") MOE_MFMA("%11", "%26", "%31") MOE_MFMA("%12", "%27", "%28")
      MOE_DMA("%40", "%45")
      MOE_M0("%43", "0xc00") MOE_MFMA("%13", "%27", "%29") MOE_MFMA("%14", "%27", "%30")
      MOE_DMA("%41", "%45")
      MOE_MFMA("%15", "%27", "%31")
      "s_waitcnt lgkmcnt(0)"
      : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
        "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
        "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
        "+a"(acc[3][3]), "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]), "=&v"(nt[3]), "=&v"(nw[0]),
        "=&v"(nw[1]), "=&v"(nw[2]), "=&v"(nw[3])
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]),
        "v"(ta), "v"(wa), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]), "v"(vo[5]),
        "v"(vo[6]), "v"(vo[7]), "s"(la), "s"(lb), "s"(ga), "s"(gw)
      : "memory", "m0");
}

__device__ __forceinline__ void step_dma_4x2(f32x16_t (&acc)[2][4], const bf16x8_t (&w)[2],
                                             const bf16x8_t (&t)[4], bf16x8_t (&nw)[2],
                                             bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa,
                                             const uint32_t (&vo)[6], uint32_t la, uint32_t lb,
                                             const char* ga, const char* gw) {
  asm volatile(
      MOE_RD("%8", "%20", "0") MOE_RD("%9", "%20", "2048")
      MOE_RD("%10", "%20", "4096") MOE_RD("%11", "%20", "6144")
      MOE_RD("%12", "%21", "0") MOE_RD("%13", "%21", "2048")
      MOE_M0("%28", "0") MOE_MFMA("%0", "%14", "%16") MOE_DMA("%22", "%30")
      MOE_M0("%28", "0x400") MOE_MFMA("%1", "%14", "%17") MOE_DMA("%23", "%30")
      MOE_M0("%28", "0x800") MOE_MFMA("%2", "%14", "%18") MOE_DMA("%24", "%30")
      MOE_M0("%28", "0xc00") MOE_MFMA("%3", "%14", "%19") MOE_DMA("%25", "%30")
      MOE_M0("%29", "0") MOE_MFMA("%4", "%15", "%16") MOE_DMA("%26", "%31")
      MOE_M0("%29", "0x400") MOE_MFMA("%5", "%15", "%17") MOE_DMA("%27", "%31")
      MOE_MFMA("%6", "%15", "%18") MOE_MFMA("%7", "%15", "%19")
      "s_waitcnt lgkmcnt(0)"
      : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
        "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]),
        "=&v"(nt[3]), "=&v"(nw[0]), "=&v"(nw[1])
      : "v"(w[0]), "v"(w[1]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(ta), "v"(wa),
        "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]), "v"(vo[5]), "s"(la), "s"(lb),
        "s"(ga), "s"(gw)
      : "memory", "m0");
}
#pragma clang diagnostic pop
#undef MOE_M0
#undef MOE_DMA

// Fragments only (the first K16 step of a tile).
template <int TM, int TN>
__device__ __forceinline__ void read_frags(bf16x8_t (&nw)[TN], bf16x8_t (&nt)[TM], uint32_t ta,
                                           uint32_t wa) {
  static_assert(TM == 4 && (TN == 4 || TN == 2), "wave tile is 128 tokens x 128 or 64 features");
  if constexpr (TN == 4) {
    asm volatile(
        MOE_RD("%0", "%8", "0") MOE_RD("%1", "%8", "2048") MOE_RD("%2", "%8", "4096")
        MOE_RD("%3", "%8", "6144") MOE_RD("%4", "%9", "0") MOE_RD("%5", "%9", "2048")
        MOE_RD("%6", "%9", "4096") MOE_RD("%7", "%9", "6144")
        "s_waitcnt lgkmcnt(0)"
        : "=v"(nt[0]), "=v"(nt[1]), "=v"(nt[2]), "=v"(nt[3]), "=v"(nw[0]), "=v"(nw[1]), "=v"(nw[2]),
          "=v"(nw[3])
        : "v"(ta), "v"(wa)
        : "memory");
  } else {
    asm volatile(
        MOE_RD("%0", "%6", "0") MOE_RD("%1", "%6", "2048") MOE_RD("%2", "%6", "4096")
        MOE_RD("%3", "%6", "6144") MOE_RD("%4", "%7", "0") MOE_RD("%5", "%7", "2048")
        "s_waitcnt lgkmcnt(0)"
        : "=v"(nt[0]), "=v"(nt[1]), "=v"(nt[2]), "=v"(nt[3]), "=v"(nw[0]), "=v"(nw[1])
        : "v"(ta), "v"(wa)
        : "memory");
  }
}

template <int TM, int TN>
__device__ __forceinline__ void step(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                     const bf16x8_t (&t)[TM], bf16x8_t (&nw)[TN], bf16x8_t (&nt)[TM],
                                     uint32_t ta, uint32_t wa) {
  if constexpr (TN == 4) step_4x4(acc, w, t, nw, nt, ta, wa);
  else step_4x2(acc, w, t, nw, nt, ta, wa);
}

template <int TM, int TN, int NV>
__device__ __forceinline__ void step_dma(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                         const bf16x8_t (&t)[TM], bf16x8_t (&nw)[TN],
                                         bf16x8_t (&nt)[TM], uint32_t ta, uint32_t wa,
                                         const uint32_t (&vo)[NV], uint32_t la, uint32_t lb,
                                         const char* ga, const char* gw) {
  if constexpr (TN == 4) step_dma_4x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
  else step_dma_4x2(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
}

template <int TM, int TN>
__device__ __forceinline__ void last_step(f32x16_t (&acc)[TN][TM], const bf16x8_t (&w)[TN],
                                          const bf16x8_t (&t)[TM]) {
  if constexpr (TN == 4) last_4x4(acc, w, t);
  else last_4x2(acc, w, t);
}
#undef MOE_MFMA
#undef MOE_RD

// tanh-GELU as u * sigmoid(2z), z = sqrt(2/pi) (u + 0.044715 u^3), with the
// hardware base-2 exponential and reciprocal (about 1 ulp each; the result is
// rounded to bf16 afterwards).
__device__ __forceinline__ float gelu_fast(float u) {
  // exp(-2z) = 2^x with x = u * (c0 + c1 u^2)
  constexpr float c0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float c1 = c0 * 0.044715f;
  const float x = u * fmaf(c1, u * u, c0);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}

template <int ACT>
__device__ __forceinline__ float activate(float v) {
  if constexpr (ACT == kActRelu) return v > 0.f ? v : 0.f;
  else if constexpr (ACT == kActGeluTanh) return gelu_fast(v);
  else return v;
}

struct TileInfo {
  int e, row0, rv, n0;
};

__device__ __forceinline__ TileInfo decode_tile(int tile, const int* s_tiles, const int32_t* offsets,
                                                int E, int NT, int BN) {
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
  const int u = tile - s_tiles[lo] * NT;
  const int nt = u / mte;  // M tiles of an expert are innermost
  const int mt = u - nt * mte;
  t.row0 = offsets[lo] + mt * BM;
  t.rv = min(BM, offsets[lo + 1] - t.row0);
  t.n0 = nt * BN;
  return t;
}

// Wait until at most min(n, MAXN) later stages (G loads each) of this wave
// are in flight.
template <int G, int MAXN>
__device__ __forceinline__ void wait_loads(int n) {
  if (MAXN >= 2 && n >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G) : "memory");
  else if (MAXN >= 1 && n >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(G) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Per-tile DMA sources: byte offsets (from the tile's token and weight bases)
// of the chunk each lane loads for every 1 KiB block it fills. Token rows past
// the expert's end read its last row; feature rows past N read row N-1.
// With row_idx, tile row r is row row_idx[row0 + r] of A (the token rows are
// gathered straight from x, so the permuted copy is never written).
template <int LA, int LB>
__device__ __forceinline__ void tile_sources(const TileInfo& t, const uint16_t* A,
                                             const int32_t* __restrict__ row_idx, const uint16_t* W,
                                             int N, int K, int wave, int drow, int dpos,
                                             const char*& Abase, const char*& Wbase,
                                             uint32_t (&aoffs)[LA], uint32_t (&boffs)[LB]) {
  Wbase = reinterpret_cast<const char*>(W + (static_cast<int64_t>(t.e) * N + t.n0) * K);
  if (row_idx != nullptr) {
    Abase = reinterpret_cast<const char*>(A);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (wave * LA + i) * 16 + drow;
      const uint32_t src = static_cast<uint32_t>(row_idx[t.row0 + min(r, t.rv - 1)]);
      aoffs[i] = (src * static_cast<uint32_t>(K) + (dpos ^ swz_key(r)) * 8) * 2;
    }
  } else {
    Abase = reinterpret_cast<const char*>(A + static_cast<int64_t>(t.row0) * K);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (wave * LA + i) * 16 + drow;
      aoffs[i] = static_cast<uint32_t>((min(r, t.rv - 1) * K + (dpos ^ swz_key(r)) * 8) * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wave * LB + i) * 16 + drow;
    boffs[i] = static_cast<uint32_t>(((min(t.n0 + r, N - 1) - t.n0) * K + (dpos ^ swz_key(r)) * 8) * 2);
  }
}


// Bias, activation, conversion and stores of one wave's 128 x WN outputs.
// FULL: every row and feature of the tile is in range (no per-lane checks).
template <int TM, int TN, int WM, int WN, bool OUT_F32, int ACT, bool FULL>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TN][TM], const float* __restrict__ bias,
                                         void* __restrict__ out, const TileInfo& t, int N, int wm,
                                         int wn, int l5, int hi) {
  const int nb = t.n0 + wn * WN + hi * 4;  // this lane's first feature
  float4 bq[TN][4];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = nb + i * 32 + q * 8;
      bq[i][q] = (bias != nullptr && (FULL || n < N))
                     ? *reinterpret_cast<const float4*>(bias + static_cast<int64_t>(t.e) * N + n)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
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
        const float v0 = activate<ACT>(acc[i][j][4 * q + 0] + bq[i][q].x);
        const float v1 = activate<ACT>(acc[i][j][4 * q + 1] + bq[i][q].y);
        const float v2 = activate<ACT>(acc[i][j][4 * q + 2] + bq[i][q].z);
        const float v3 = activate<ACT>(acc[i][j][4 * q + 3] + bq[i][q].w);
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
    }
  }
}

}  // namespace

template <int BN, int NST, int OCC, bool OUT_F32, int ACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_idx,
                              const uint16_t* __restrict__ W,
                              const float* __restrict__ bias, void* __restrict__ out,
                              const int32_t* __restrict__ offsets, int E, int N, int K) {
  // the body uses gfx950 builtins only: the host pass needs just the signature
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int WM = BM / 2;         // tokens per wave
  constexpr int WN = BN / 2;         // features per wave
  constexpr int TM = WM / 32;        // 32-token MFMA tiles per wave
  constexpr int TN = WN / 32;        // 32-feature MFMA tiles per wave
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int LA = BM / 64;        // 1 KiB DMA blocks of the token tile per wave
  constexpr int LB = BN / 64;        // 1 KiB DMA blocks of the weight tile per wave
  constexpr int G = LA + LB;         // DMA loads per wave per stage

  __shared__ __attribute__((aligned(1024))) char lds[NST * STAGE];
  __shared__ int s_tiles[1025];  // exclusive prefix of M tiles per expert
  __shared__ int s_part[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---- device-side schedule: M tiles per expert, exclusive prefix
  {
    const int per = (E + 255) / 256;
    const int eb = tid * per;
    int local = 0;
    for (int e = eb; e < min(E, eb + per); ++e) local += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    s_part[tid] = local;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = (tid >= off) ? s_part[tid - off] : 0;
      __syncthreads();
      s_part[tid] += add;
      __syncthreads();
    }
    int run = s_part[tid] - local;
    for (int e = eb; e < min(E, eb + per); ++e) {
      s_tiles[e] = run;
      run += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    }
    if (tid == 255) s_tiles[E] = s_part[255];
    __syncthreads();
  }
  const int NT = (N + BN - 1) / BN;
  const int total = s_tiles[E] * NT;
  const int Gd = gridDim.x;
  const int b = blockIdx.x;
  // blocks are dealt to the 8 XCDs round-robin: renumber so that consecutive
  // tiles (which share weight and token panels) run on one XCD
  int tile = (Gd % 8 == 0) ? (b % 8) * (Gd / 8) + b / 8 : b;
  if (tile >= total) return;

  // per-lane constants: fragment offsets (K16 step s of a stage) and the DMA
  // source mapping (lane L lands at row L/4, position L%4 of its 1 KiB block,
  // so it loads the chunk the swizzle places there)
  const int l5 = lane & 31, hi = lane >> 5;
  const uint32_t fo0 = l5 * ROWB + 16 * ((0 + hi) ^ swz_key(l5));
  const uint32_t fo1 = l5 * ROWB + 16 * ((2 + hi) ^ swz_key(l5));
  const int drow = lane >> 2, dpos = lane & 3;
  const int nk = K / BK;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const uint32_t trow = wm * WM * ROWB;            // this wave's token rows in a stage
  const uint32_t wrow = A_BYTES + wn * WN * ROWB;  // this wave's weight rows in a stage

  uint32_t aoffs[LA], boffs[LB], vo[G];
  const char* Abase;
  const char* Wbase;
  TileInfo cur = decode_tile(tile, s_tiles, offsets, E, NT, BN);
  tile_sources<LA, LB>(cur, A, row_idx, W, N, K, wave, drow, dpos, Abase, Wbase, aoffs, boffs);
  for (int p = 0; p < NST && p < nk; ++p)
    issue_stage<LA, LB, A_BYTES>(Abase + p * ROWB, Wbase + p * ROWB, lds + p * STAGE, aoffs, boffs, wave);

  for (;;) {
    f32x16_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // the tile's first stage (and, after an epilogue, its stores)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    bf16x8_t w0[TN], t0[TM], w1[TN], t1[TM];
    read_frags<TM, TN>(w0, t0, lds_base + trow + fo0, lds_base + wrow + fo0);

    TileInfo done = cur;
    const int next = tile + Gd;
#pragma unroll
    for (int i = 0; i < LA; ++i) vo[i] = aoffs[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) vo[LA + i] = boffs[i];
    int sc = 0;              // stage holding K tile t
    uint32_t sb = lds_base;  // its LDS address
    int t = 0;
    // steady state: K tile t+NST still to load
    for (; t + NST < nk; ++t) {
      const int sn_i = (sc + 1 == NST) ? 0 : sc + 1;
      const uint32_t sn = lds_base + sn_i * STAGE;
      // K16 step 0 of stage t; read step 1 of stage t
      step<TM, TN>(acc, w0, t0, w1, t1, sb + trow + fo1, sb + wrow + fo1);
      // stage t+1 ready (t+2 .. t+NST-1 may still load); every wave is done
      // with stage t, which then takes K tile t+NST
      wait_loads<G, NST - 2>(NST - 2);
      __syncthreads();
      // K16 step 1 of stage t; read step 0 of stage t+1; stage t (free after
      // the barrier) takes K tile t+NST
      {
        const uint32_t sl = lds_base + sc * STAGE;
        step_dma<TM, TN, G>(acc, w1, t1, w0, t0, sn + trow + fo0, sn + wrow + fo0, vo,
                            sl + wave * LA * 1024, sl + A_BYTES + wave * LB * 1024,
                            Abase + (t + NST) * ROWB, Wbase + (t + NST) * ROWB);
      }
      sc = sn_i;
      sb = sn;
    }
    // the last stages: nothing more to load
    for (; t + 1 < nk; ++t) {
      const int sn_i = (sc + 1 == NST) ? 0 : sc + 1;
      const uint32_t sn = lds_base + sn_i * STAGE;
      step<TM, TN>(acc, w0, t0, w1, t1, sb + trow + fo1, sb + wrow + fo1);
      wait_loads<G, NST - 2>(nk - 2 - t);
      __syncthreads();
      step<TM, TN>(acc, w1, t1, w0, t0, sn + trow + fo0, sn + wrow + fo0);
      sc = sn_i;
      sb = sn;
    }
    // the last stage
    step<TM, TN>(acc, w0, t0, w1, t1, sb + trow + fo1, sb + wrow + fo1);
    __syncthreads();
    if (next < total) {
      // all stages are free: the next tile's first stages load during this
      // tile's last MFMAs and epilogue
      cur = decode_tile(next, s_tiles, offsets, E, NT, BN);
      tile_sources<LA, LB>(cur, A, row_idx, W, N, K, wave, drow, dpos, Abase, Wbase, aoffs, boffs);
      for (int p = 0; p < NST && p < nk; ++p)
        issue_stage<LA, LB, A_BYTES>(Abase + p * ROWB, Wbase + p * ROWB, lds + p * STAGE, aoffs, boffs,
                                     wave);
    }
    last_step<TM, TN>(acc, w1, t1);

    // ---- epilogue: lane holds token l5 of each 32-token tile j and
    // features 8q + 4*hi + {0..3} of each 32-feature tile i
    const bool full_tile = done.rv == BM && done.n0 + BN <= N;
    if (full_tile) epilogue<TM, TN, WM, WN, OUT_F32, ACT, true>(acc, bias, out, done, N, wm, wn, l5, hi);
    else epilogue<TM, TN, WM, WN, OUT_F32, ACT, false>(acc, bias, out, done, N, wm, wn, l5, hi);
    if (next >= total) break;
    tile = next;
  }
#endif
}

#ifndef MOE_GEMM_NST
#define MOE_GEMM_NST 4
#endif
#ifndef MOE_GEMM_OCC
#define MOE_GEMM_OCC 1
#endif

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
                            const float* bias, void* out,
                            bool out_f32, int act, const int32_t* offsets, int E, int N, int K,
                            int64_t max_rows, int max_rows_per_expert, hipStream_t s) {
  (void)max_rows_per_expert;
  if (max_rows <= 0) return hipSuccess;
  // upper bound on tiles: sum_e ceil(n_e/BM) <= max_rows/BM + E
  const int64_t mt_bound = max_rows / BM + E;
  constexpr int BN = 256, NST = MOE_GEMM_NST, OCC = MOE_GEMM_OCC;
  const int slots = cu_count() * OCC;
  const int64_t tiles = mt_bound * ((N + BN - 1) / BN);
  const unsigned grid = static_cast<unsigned>(tiles < slots ? tiles : slots);
  if (out_f32) {
    grouped_gemm_bf16_kernel<BN, NST, OCC, true, kActNone><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
  } else {
    if (act == kActRelu)
      grouped_gemm_bf16_kernel<BN, NST, OCC, false, kActRelu><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
    else if (act == kActGeluTanh)
      grouped_gemm_bf16_kernel<BN, NST, OCC, false, kActGeluTanh><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
    else
      grouped_gemm_bf16_kernel<BN, NST, OCC, false, kActNone><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
  }
  return hipGetLastError();
}

}  // namespace moe
