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
//  * Block tile BM=256 tokens x BN (256 or 128) features; four waves in a 2x2
//    grid; each wave owns 128 tokens x BN/2 features as 32x32
//    v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulators in AGPRs. The
//    weight tile is the MFMA A operand and the token tile the B operand, so a
//    lane's accumulators hold 4 consecutive features of one token: the
//    epilogue stores 8-byte (bf16) or 16-byte (fp32) vectors.
//  * K advances in stages of BK=64: every LDS row is 128 bytes, one full
//    cache line of the source row, so each L1->L2 request moves a whole line
//    (32-element stages would request half lines and need twice the
//    requests for the same bytes). The 16-byte chunks of a row are XOR-
//    swizzled by (row/2)&7, which keeps the fragment reads (16 lanes = 16
//    rows at one chunk) on distinct banks.
//  * Tiles move global -> LDS with gfx950's LDS-DMA loads
//    (global_load_lds_dwordx4: no staging registers, no ds_write); one
//    instruction fills 8 rows (1 KiB); each lane fetches the chunk that the
//    swizzle places at its LDS slot.
//  * A stage is four K16 steps. Each step's MFMAs run with the next step's
//    fragment reads in flight. The buffer a stage occupied is refilled (with
//    the stage NST ahead) between the MFMAs of that stage's last step, right
//    after the barrier that shows every wave has read it; the next tile's
//    first stages load during the current tile's last step and epilogue.
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
constexpr int BK = 64;        // K per LDS stage
constexpr int ROWB = BK * 2;  // bytes per LDS row (128)

// Row r of a stage holds its 16-byte chunk c at position c ^ swz_key(r).
// A fragment read covers 32 rows at one chunk; the LDS serves 16 lanes per
// cycle, and with this key the 16 rows of a group land on 16 distinct
// 4-bank groups (rows 2j and 2j+1 differ in the bank half, rows 2j at j =
// 0..7 differ in the chunk position).
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }

typedef __attribute__((address_space(3))) void lds_void_t;

// Queue one stage (BK columns of the token and weight tiles) with LDS-DMA
// loads. One global_load_lds_dwordx4 fills 1 KiB = 8 rows of 128 B; wave w's
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
// The matrix core holds one MFMA behind the one executing (32 cycles each
// for 32x32x16), so any other instruction a wave issues is free only while it
// fits in that shadow: a run of LDS reads issued before the MFMAs leaves the
// core idle. Each block below therefore issues one fragment read (and, in the
// refill step, one LDS-DMA load) after each MFMA. The compiler cannot place
// them there: its wait insertion treats any LDS read as dependent on every
// LDS-DMA load in flight and waits for all of them, which would serialise the
// stage pipeline. A block reads the next K16 step's fragments and waits for
// them before it ends: no read is in flight past a block. Stage order is
// explicit (wait_loads and a barrier before a stage is read).
//   acc[i][j] += W_i * T_j: W = weight fragments (MFMA A operand),
//   T = token fragments (B operand); next fragments from ta / wa, the 32-row
//   fragment tiles 4096 B apart.
#define MOE_MFMA(D, A, B) "v_mfma_f32_32x32x16_bf16 " D ", " A ", " B ", " D "\n\t"
#define MOE_RD(D, ADDR, OFF) "ds_read_b128 " D ", " ADDR " offset:" OFF "\n\t"

// The last step of a stage also refills the stage buffer that became free:
// G LDS-DMA loads spread between the MFMAs. M0 carries the LDS destination of
// each load (lane L writes bytes 16L..16L+15 of a 1 KiB block); la / lb are
// this wave's first token / weight block of the buffer, ga / gw the global
// bases of the K columns being loaded, vo the per-lane byte offsets (token
// blocks first, then weight blocks). An instruction sits between each M0
// write and the load that uses it. M0 is reserved by the compiler, which sets
// it again before each LDS-DMA load of its own; the clobber orders those
// against these blocks.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// ---------------------------------------------------------------- 4x4 (wave 128 x 128)
#define MOE_ACC_4X4                                                                           \
  "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),        \
      "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),    \
      "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),    \
      "+a"(acc[3][3])
#define MOE_NEXT_4X4                                                                          \
  "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]), "=&v"(nt[3]), "=&v"(nw[0]), "=&v"(nw[1]),         \
      "=&v"(nw[2]), "=&v"(nw[3])
#define MOE_CUR_4X4 \
  "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3])

__device__ __forceinline__ void step_4x4(f32x16_t (&acc)[4][4], const bf16x8_t (&w)[4],
                                         const bf16x8_t (&t)[4], bf16x8_t (&nw)[4],
                                         bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %24, %28, %0\n\t"
      "ds_read_b128 %16, %32 offset:0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %24, %29, %1\n\t"
      "ds_read_b128 %17, %32 offset:4096\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %24, %30, %2\n\t"
      "ds_read_b128 %18, %32 offset:8192\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %24, %31, %3\n\t"
      "ds_read_b128 %19, %32 offset:12288\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %25, %28, %4\n\t"
      "ds_read_b128 %20, %33 offset:0\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %25, %29, %5\n\t"
      "ds_read_b128 %21, %33 offset:4096\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %25, %30, %6\n\t"
      "ds_read_b128 %22, %33 offset:8192\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %25, %31, %7\n\t"
      "ds_read_b128 %23, %33 offset:12288\n\t"
      "v_mfma_f32_32x32x16_bf16 %8, %26, %28, %8\n\t"
      "v_mfma_f32_32x32x16_bf16 %9, %26, %29, %9\n\t"
      "v_mfma_f32_32x32x16_bf16 %10, %26, %30, %10\n\t"
      "v_mfma_f32_32x32x16_bf16 %11, %26, %31, %11\n\t"
      "v_mfma_f32_32x32x16_bf16 %12, %27, %28, %12\n\t"
      "v_mfma_f32_32x32x16_bf16 %13, %27, %29, %13\n\t"
      "v_mfma_f32_32x32x16_bf16 %14, %27, %30, %14\n\t"
      "v_mfma_f32_32x32x16_bf16 %15, %27, %31, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : MOE_ACC_4X4, MOE_NEXT_4X4
      : MOE_CUR_4X4, "v"(ta), "v"(wa)
      : "memory");
}

__device__ __forceinline__ void step_dma_4x4(f32x16_t (&acc)[4][4], const bf16x8_t (&w)[4],
                                             const bf16x8_t (&t)[4], bf16x8_t (&nw)[4],
                                             bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa,
                                             const uint32_t (&vo)[16], uint32_t la, uint32_t lb,
                                             const char* ga, const char* gw) {
  asm volatile(
      "s_add_u32 m0, %50, 0x0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %24, %28, %0\n\t"
      "global_load_lds_dwordx4 %34, %52\n\t"
      "ds_read_b128 %16, %32 offset:0\n\t"
      "s_add_u32 m0, %50, 0x400\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %24, %29, %1\n\t"
      "global_load_lds_dwordx4 %35, %52\n\t"
      "ds_read_b128 %17, %32 offset:4096\n\t"
      "s_add_u32 m0, %50, 0x800\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %24, %30, %2\n\t"
      "global_load_lds_dwordx4 %36, %52\n\t"
      "ds_read_b128 %18, %32 offset:8192\n\t"
      "s_add_u32 m0, %50, 0xc00\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %24, %31, %3\n\t"
      "global_load_lds_dwordx4 %37, %52\n\t"
      "ds_read_b128 %19, %32 offset:12288\n\t"
      "s_add_u32 m0, %50, 0x1000\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %25, %28, %4\n\t"
      "global_load_lds_dwordx4 %38, %52\n\t"
      "ds_read_b128 %20, %33 offset:0\n\t"
      "s_add_u32 m0, %50, 0x1400\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %25, %29, %5\n\t"
      "global_load_lds_dwordx4 %39, %52\n\t"
      "ds_read_b128 %21, %33 offset:4096\n\t"
      "s_add_u32 m0, %50, 0x1800\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %25, %30, %6\n\t"
      "global_load_lds_dwordx4 %40, %52\n\t"
      "ds_read_b128 %22, %33 offset:8192\n\t"
      "s_add_u32 m0, %50, 0x1c00\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %25, %31, %7\n\t"
      "global_load_lds_dwordx4 %41, %52\n\t"
      "ds_read_b128 %23, %33 offset:12288\n\t"
      "s_add_u32 m0, %51, 0x0\n\t"
      "v_mfma_f32_32x32x16_bf16 %8, %26, %28, %8\n\t"
      "global_load_lds_dwordx4 %42, %53\n\t"
      "s_add_u32 m0, %51, 0x400\n\t"
      "v_mfma_f32_32x32x16_bf16 %9, %26, %29, %9\n\t"
      "global_load_lds_dwordx4 %43, %53\n\t"
      "s_add_u32 m0, %51, 0x800\n\t"
      "v_mfma_f32_32x32x16_bf16 %10, %26, %30, %10\n\t"
      "global_load_lds_dwordx4 %44, %53\n\t"
      "s_add_u32 m0, %51, 0xc00\n\t"
      "v_mfma_f32_32x32x16_bf16 %11, %26, %31, %11\n\t"
      "global_load_lds_dwordx4 %45, %53\n\t"
      "s_add_u32 m0, %51, 0x1000\n\t"
      "v_mfma_f32_32x32x16_bf16 %12, %27, %28, %12\n\t"
      "global_load_lds_dwordx4 %46, %53\n\t"
      "s_add_u32 m0, %51, 0x1400\n\t"
      "v_mfma_f32_32x32x16_bf16 %13, %27, %29, %13\n\t"
      "global_load_lds_dwordx4 %47, %53\n\t"
      "s_add_u32 m0, %51, 0x1800\n\t"
      "v_mfma_f32_32x32x16_bf16 %14, %27, %30, %14\n\t"
      "global_load_lds_dwordx4 %48, %53\n\t"
      "s_add_u32 m0, %51, 0x1c00\n\t"
      "v_mfma_f32_32x32x16_bf16 %15, %27, %31, %15\n\t"
      "global_load_lds_dwordx4 %49, %53\n\t"
      "s_waitcnt lgkmcnt(0)"
      : MOE_ACC_4X4, MOE_NEXT_4X4
      : MOE_CUR_4X4, "v"(ta), "v"(wa), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]),
        "v"(vo[4]), "v"(vo[5]), "v"(vo[6]), "v"(vo[7]), "v"(vo[8]), "v"(vo[9]), "v"(vo[10]),
        "v"(vo[11]), "v"(vo[12]), "v"(vo[13]), "v"(vo[14]), "v"(vo[15]), "s"(la), "s"(lb),
        "s"(ga), "s"(gw)
      : "memory", "m0");
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
      : MOE_ACC_4X4
      : MOE_CUR_4X4
      : "memory");
}

// ---------------------------------------------------------------- 4x2 (wave 128 tokens x 64 features)
#define MOE_ACC_4X2                                                                          \
  "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),       \
      "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3])
#define MOE_NEXT_4X2 \
  "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]), "=&v"(nt[3]), "=&v"(nw[0]), "=&v"(nw[1])
#define MOE_CUR_4X2 "v"(w[0]), "v"(w[1]), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3])

__device__ __forceinline__ void step_4x2(f32x16_t (&acc)[2][4], const bf16x8_t (&w)[2],
                                         const bf16x8_t (&t)[4], bf16x8_t (&nw)[2],
                                         bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %14, %16, %0\n\t"
      "ds_read_b128 %8, %20 offset:0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %14, %17, %1\n\t"
      "ds_read_b128 %9, %20 offset:4096\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %14, %18, %2\n\t"
      "ds_read_b128 %10, %20 offset:8192\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %14, %19, %3\n\t"
      "ds_read_b128 %11, %20 offset:12288\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %15, %16, %4\n\t"
      "ds_read_b128 %12, %21 offset:0\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %15, %17, %5\n\t"
      "ds_read_b128 %13, %21 offset:4096\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %15, %18, %6\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %15, %19, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : MOE_ACC_4X2, MOE_NEXT_4X2
      : MOE_CUR_4X2, "v"(ta), "v"(wa)
      : "memory");
}

// 12 loads (8 token blocks, 4 weight blocks) over 8 MFMAs
__device__ __forceinline__ void step_dma_4x2(f32x16_t (&acc)[2][4], const bf16x8_t (&w)[2],
                                             const bf16x8_t (&t)[4], bf16x8_t (&nw)[2],
                                             bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa,
                                             const uint32_t (&vo)[12], uint32_t la, uint32_t lb,
                                             const char* ga, const char* gw) {
  asm volatile(
      "s_add_u32 m0, %34, 0x0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %14, %16, %0\n\t"
      "global_load_lds_dwordx4 %22, %36\n\t"
      "s_add_u32 m0, %34, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %23, %36\n\t"
      "ds_read_b128 %8, %20 offset:0\n\t"
      "s_add_u32 m0, %34, 0x800\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %14, %17, %1\n\t"
      "global_load_lds_dwordx4 %24, %36\n\t"
      "s_add_u32 m0, %34, 0xc00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %25, %36\n\t"
      "ds_read_b128 %9, %20 offset:4096\n\t"
      "s_add_u32 m0, %34, 0x1000\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %14, %18, %2\n\t"
      "global_load_lds_dwordx4 %26, %36\n\t"
      "s_add_u32 m0, %34, 0x1400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %27, %36\n\t"
      "ds_read_b128 %10, %20 offset:8192\n\t"
      "s_add_u32 m0, %34, 0x1800\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %14, %19, %3\n\t"
      "global_load_lds_dwordx4 %28, %36\n\t"
      "s_add_u32 m0, %34, 0x1c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %29, %36\n\t"
      "ds_read_b128 %11, %20 offset:12288\n\t"
      "s_add_u32 m0, %35, 0x0\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %15, %16, %4\n\t"
      "global_load_lds_dwordx4 %30, %37\n\t"
      "ds_read_b128 %12, %21 offset:0\n\t"
      "s_add_u32 m0, %35, 0x400\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %15, %17, %5\n\t"
      "global_load_lds_dwordx4 %31, %37\n\t"
      "ds_read_b128 %13, %21 offset:4096\n\t"
      "s_add_u32 m0, %35, 0x800\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %15, %18, %6\n\t"
      "global_load_lds_dwordx4 %32, %37\n\t"
      "s_add_u32 m0, %35, 0xc00\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %15, %19, %7\n\t"
      "global_load_lds_dwordx4 %33, %37\n\t"
      "s_waitcnt lgkmcnt(0)"
      : MOE_ACC_4X2, MOE_NEXT_4X2
      : MOE_CUR_4X2, "v"(ta), "v"(wa), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]),
        "v"(vo[4]), "v"(vo[5]), "v"(vo[6]), "v"(vo[7]), "v"(vo[8]), "v"(vo[9]), "v"(vo[10]),
        "v"(vo[11]), "s"(la), "s"(lb), "s"(ga), "s"(gw)
      : "memory", "m0");
}

__device__ __forceinline__ void last_4x2(f32x16_t (&acc)[2][4], const bf16x8_t (&w)[2],
                                         const bf16x8_t (&t)[4]) {
  asm volatile(
      "s_nop 1\n\t"
      MOE_MFMA("%0", "%8", "%10") MOE_MFMA("%1", "%8", "%11") MOE_MFMA("%2", "%8", "%12")
      MOE_MFMA("%3", "%8", "%13") MOE_MFMA("%4", "%9", "%10") MOE_MFMA("%5", "%9", "%11")
      MOE_MFMA("%6", "%9", "%12") MOE_MFMA("%7", "%9", "%13")
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : MOE_ACC_4X2
      : MOE_CUR_4X2
      : "memory");
}
#pragma clang diagnostic pop

// Fragments only (the first K16 step of a tile). The outputs are early-
// clobber: a read's data may land before the later reads are issued, so no
// destination may share a register with the addresses.
template <int TN>
__device__ __forceinline__ void read_frags(bf16x8_t (&nw)[TN], bf16x8_t (&nt)[4], uint32_t ta,
                                           uint32_t wa) {
  static_assert(TN == 4 || TN == 2, "wave tile is 128 tokens x 128 or 64 features");
  if constexpr (TN == 4) {
    asm volatile(
        MOE_RD("%0", "%8", "0") MOE_RD("%1", "%8", "4096") MOE_RD("%2", "%8", "8192")
        MOE_RD("%3", "%8", "12288") MOE_RD("%4", "%9", "0") MOE_RD("%5", "%9", "4096")
        MOE_RD("%6", "%9", "8192") MOE_RD("%7", "%9", "12288")
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]), "=&v"(nt[3]), "=&v"(nw[0]), "=&v"(nw[1]),
          "=&v"(nw[2]), "=&v"(nw[3])
        : "v"(ta), "v"(wa)
        : "memory");
  } else {
    asm volatile(
        MOE_RD("%0", "%6", "0") MOE_RD("%1", "%6", "4096") MOE_RD("%2", "%6", "8192")
        MOE_RD("%3", "%6", "12288") MOE_RD("%4", "%7", "0") MOE_RD("%5", "%7", "4096")
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(nt[0]), "=&v"(nt[1]), "=&v"(nt[2]), "=&v"(nt[3]), "=&v"(nw[0]), "=&v"(nw[1])
        : "v"(ta), "v"(wa)
        : "memory");
  }
}

template <int TN>
__device__ __forceinline__ void step(f32x16_t (&acc)[TN][4], const bf16x8_t (&w)[TN],
                                     const bf16x8_t (&t)[4], bf16x8_t (&nw)[TN], bf16x8_t (&nt)[4],
                                     uint32_t ta, uint32_t wa) {
  if constexpr (TN == 4) step_4x4(acc, w, t, nw, nt, ta, wa);
  else step_4x2(acc, w, t, nw, nt, ta, wa);
}

template <int TN, int NV>
__device__ __forceinline__ void step_dma(f32x16_t (&acc)[TN][4], const bf16x8_t (&w)[TN],
                                         const bf16x8_t (&t)[4], bf16x8_t (&nw)[TN],
                                         bf16x8_t (&nt)[4], uint32_t ta, uint32_t wa,
                                         const uint32_t (&vo)[NV], uint32_t la, uint32_t lb,
                                         const char* ga, const char* gw) {
  if constexpr (TN == 4) step_dma_4x4(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
  else step_dma_4x2(acc, w, t, nw, nt, ta, wa, vo, la, lb, ga, gw);
}

template <int TN>
__device__ __forceinline__ void last_step(f32x16_t (&acc)[TN][4], const bf16x8_t (&w)[TN],
                                          const bf16x8_t (&t)[4]) {
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

// Wait until at most n (< 3) stages of G loads each, issued after the one
// awaited, are still in flight.
template <int G>
__device__ __forceinline__ void wait_loads(int n) {
  if (n >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G) : "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(G) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Per-tile DMA sources: byte offsets (from the tile's token and weight bases)
// of the chunk each lane loads for every 1 KiB block it fills (lane L lands
// at row L/8, position L%8 of its block). Token rows past the expert's end
// read its last row; feature rows past N read row N-1. With row_idx, tile row
// r is row row_idx[row0 + r] of A (the token rows are gathered straight from
// x, so the permuted copy is never written).
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
      const int r = (wave * LA + i) * 8 + drow;
      const uint32_t src = static_cast<uint32_t>(row_idx[t.row0 + min(r, t.rv - 1)]);
      aoffs[i] = (src * static_cast<uint32_t>(K) + (dpos ^ swz_key(r)) * 8) * 2;
    }
  } else {
    Abase = reinterpret_cast<const char*>(A + static_cast<int64_t>(t.row0) * K);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (wave * LA + i) * 8 + drow;
      aoffs[i] = static_cast<uint32_t>((min(r, t.rv - 1) * K + (dpos ^ swz_key(r)) * 8) * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wave * LB + i) * 8 + drow;
    boffs[i] = static_cast<uint32_t>(((min(t.n0 + r, N - 1) - t.n0) * K + (dpos ^ swz_key(r)) * 8) * 2);
  }
}

// Bias, activation, conversion and stores of one wave's 128 x WN outputs.
// FULL: every row and feature of the tile is in range (no per-lane checks).
template <int TN, int WN, bool OUT_F32, int ACT, bool FULL>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TN][4], const float* __restrict__ bias,
                                         void* __restrict__ out, const TileInfo& t, int N, int wm,
                                         int wn, int l5, int hi) {
  constexpr int WM = BM / 2;
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
  for (int j = 0; j < 4; ++j) {
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

template <int BN, int NST, bool OUT_F32, int ACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_idx,
                              const uint16_t* __restrict__ W,
                              const float* __restrict__ bias, void* __restrict__ out,
                              const int32_t* __restrict__ offsets, int E, int N, int K) {
  // the body uses gfx950 builtins only: the host pass needs just the signature
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int WM = BM / 2;         // tokens per wave
  constexpr int WN = BN / 2;         // features per wave
  constexpr int TN = WN / 32;        // 32-feature MFMA tiles per wave
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int LA = BM / 32;        // 1 KiB (8-row) DMA blocks of the token tile per wave
  constexpr int LB = BN / 32;        // 1 KiB DMA blocks of the weight tile per wave
  constexpr int G = LA + LB;         // DMA loads per wave per stage
  static_assert(NST >= 2 && NST <= 4, "2 to 4 stages");

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

  // per-lane constants: fragment offsets of the four K16 steps of a stage
  // (lane (l5, hi) reads row l5, chunk 2s + hi) and the DMA source mapping
  const int l5 = lane & 31, hi = lane >> 5;
  const int key = swz_key(l5);  // equal for rows l5 + 32j
  uint32_t fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = l5 * ROWB + 16 * ((2 * s + hi) ^ key);
  const int drow = lane >> 3, dpos = lane & 7;
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
    f32x16_t acc[TN][4];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // the tile's first stages (and, after an epilogue, its stores)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    bf16x8_t wf0[TN], tf0[4], wf1[TN], tf1[4];
    read_frags<TN>(wf0, tf0, lds_base + trow + fo[0], lds_base + wrow + fo[0]);

    TileInfo done = cur;
    const int next = tile + Gd;
#pragma unroll
    for (int i = 0; i < LA; ++i) vo[i] = aoffs[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) vo[LA + i] = boffs[i];
    int sc = 0;              // buffer holding K stage t
    uint32_t sb = lds_base;  // its LDS address
    int t = 0;
    // steady state: stage t+NST still to load
    for (; t + NST < nk; ++t) {
      // K16 steps 0..2 of stage t, each reading the next step's fragments
      step<TN>(acc, wf0, tf0, wf1, tf1, sb + trow + fo[1], sb + wrow + fo[1]);
      step<TN>(acc, wf1, tf1, wf0, tf0, sb + trow + fo[2], sb + wrow + fo[2]);
      step<TN>(acc, wf0, tf0, wf1, tf1, sb + trow + fo[3], sb + wrow + fo[3]);
      // stage t+1 has landed (stages t+2 .. t+NST-1 may still load) and every
      // wave has read its last fragments of stage t
      wait_loads<G>(NST - 2);
      __syncthreads();
      const int sn_i = (sc + 1 == NST) ? 0 : sc + 1;
      const uint32_t sn = lds_base + sn_i * STAGE;
      // K16 step 3 of stage t; read step 0 of stage t+1; the buffer of stage
      // t takes stage t+NST
      step_dma<TN, G>(acc, wf1, tf1, wf0, tf0, sn + trow + fo[0], sn + wrow + fo[0], vo,
                      sb + wave * LA * 1024, sb + A_BYTES + wave * LB * 1024,
                      Abase + (t + NST) * ROWB, Wbase + (t + NST) * ROWB);
      sc = sn_i;
      sb = sn;
    }
    // the last stages: nothing more to load
    for (; t + 1 < nk; ++t) {
      step<TN>(acc, wf0, tf0, wf1, tf1, sb + trow + fo[1], sb + wrow + fo[1]);
      step<TN>(acc, wf1, tf1, wf0, tf0, sb + trow + fo[2], sb + wrow + fo[2]);
      step<TN>(acc, wf0, tf0, wf1, tf1, sb + trow + fo[3], sb + wrow + fo[3]);
      wait_loads<G>(nk - 2 - t);
      __syncthreads();
      const int sn_i = (sc + 1 == NST) ? 0 : sc + 1;
      const uint32_t sn = lds_base + sn_i * STAGE;
      step<TN>(acc, wf1, tf1, wf0, tf0, sn + trow + fo[0], sn + wrow + fo[0]);
      sc = sn_i;
      sb = sn;
    }
    // the last stage
    step<TN>(acc, wf0, tf0, wf1, tf1, sb + trow + fo[1], sb + wrow + fo[1]);
    step<TN>(acc, wf1, tf1, wf0, tf0, sb + trow + fo[2], sb + wrow + fo[2]);
    step<TN>(acc, wf0, tf0, wf1, tf1, sb + trow + fo[3], sb + wrow + fo[3]);
    // every wave has read all of its fragments: all buffers are free, and the
    // next tile's first stages load during this tile's last MFMAs and epilogue
    __syncthreads();
    if (next < total) {
      cur = decode_tile(next, s_tiles, offsets, E, NT, BN);
      tile_sources<LA, LB>(cur, A, row_idx, W, N, K, wave, drow, dpos, Abase, Wbase, aoffs, boffs);
      for (int p = 0; p < NST && p < nk; ++p)
        issue_stage<LA, LB, A_BYTES>(Abase + p * ROWB, Wbase + p * ROWB, lds + p * STAGE, aoffs, boffs,
                                     wave);
    }
    last_step<TN>(acc, wf1, tf1);

    // ---- epilogue: lane holds token l5 of each 32-token tile j and
    // features 8q + 4*hi + {0..3} of each 32-feature tile i
    const bool full_tile = done.rv == BM && done.n0 + BN <= N;
    if (full_tile) epilogue<TN, WN, OUT_F32, ACT, true>(acc, bias, out, done, N, wm, wn, l5, hi);
    else epilogue<TN, WN, OUT_F32, ACT, false>(acc, bias, out, done, N, wm, wn, l5, hi);
    if (next >= total) break;
    tile = next;
  }
#endif
}

#ifndef MOE_GEMM_BN
#define MOE_GEMM_BN 256
#endif
#ifndef MOE_GEMM_NST
#define MOE_GEMM_NST 2
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

template <int BN, int NST>
hipError_t launch_cfg(const uint16_t* A, const int32_t* row_idx, const uint16_t* W, const float* bias,
                      void* out, bool out_f32, int act, const int32_t* offsets, int E, int N, int K,
                      int64_t max_rows, hipStream_t s) {
  // upper bound on tiles: sum_e ceil(n_e/BM) <= max_rows/BM + E
  const int64_t mt_bound = max_rows / BM + E;
  const int slots = cu_count();
  const int64_t tiles = mt_bound * ((N + BN - 1) / BN);
  const unsigned grid = static_cast<unsigned>(tiles < slots ? tiles : slots);
  if (out_f32) {
    grouped_gemm_bf16_kernel<BN, NST, true, kActNone><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
  } else if (act == kActRelu) {
    grouped_gemm_bf16_kernel<BN, NST, false, kActRelu><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
  } else if (act == kActGeluTanh) {
    grouped_gemm_bf16_kernel<BN, NST, false, kActGeluTanh><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
  } else {
    grouped_gemm_bf16_kernel<BN, NST, false, kActNone><<<grid, 256, 0, s>>>(A, row_idx, W, bias, out, offsets, E, N, K);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, const int32_t* row_idx, const uint16_t* W,
                            const float* bias, void* out,
                            bool out_f32, int act, const int32_t* offsets, int E, int N, int K,
                            int64_t max_rows, int max_rows_per_expert, hipStream_t s) {
  (void)max_rows_per_expert;
  if (max_rows <= 0) return hipSuccess;
  return launch_cfg<MOE_GEMM_BN, MOE_GEMM_NST>(A, row_idx, W, bias, out, out_f32, act, offsets, E, N, K,
                                              max_rows, s);
}

}  // namespace moe
