// Internal declarations shared by the host API and the kernel launchers of
// libmoe.so. Not part of the public ABI (that is include/moe.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- kernel timing
// Optional per-stage kernel timing of the layer forward. While a stage runs
// with events set, its first kernel dispatch records `start` when the kernel
// begins and every dispatch records `stop` when its kernel ends (the last
// one is what remains), so stop - start spans the stage's kernels without
// the launch gap in front of the first one. Plain launches otherwise (the
// extended launch adds a few microseconds of launch gap per kernel).
struct StageEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
extern thread_local StageEvents t_stage_events;

template <typename... KArgs, typename... Args>
inline void klaunch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                    Args... args) {
  StageEvents& ev = t_stage_events;
  if (ev.start == nullptr && ev.stop == nullptr) {
    kernel<<<grid, block, shmem, s>>>(static_cast<KArgs>(args)...);
  } else {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0u,
                          static_cast<KArgs>(args)...);
    ev.start = nullptr;
  }
}

// Tokens per dispatch tile: the unit of the per-tile expert histograms and of
// the permutation kernel (one 64-bit lane mask per expert and tile).
constexpr int kTileTokens = 64;

// M tile of the bf16 grouped GEMM (tokens per tile).
constexpr int kGemmBM = 256;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// sigma of the expert FFN. tanh-GELU written as u * sigmoid(2z) with
// z = sqrt(2/pi) (u + 0.044715 u^3), which equals 0.5 u (1 + tanh z).
__device__ __forceinline__ float act_relu(float u) { return u > 0.f ? u : 0.f; }
__device__ __forceinline__ float act_gelu_tanh(float u) {
  const float z = 0.7978845608028654f * (u + 0.044715f * u * u * u);
  return u / (1.0f + __expf(-2.0f * z));
}

// tanh-GELU of the bf16 expert GEMM epilogue: u * sigmoid(2z) with the
// hardware base-2 exponential and reciprocal (about 1 ulp each; the result is
// rounded to bf16 afterwards). The backward pass recomputes h with it.
// exp(-2z) = 2^x with x = u * (c0 + c1 u^2)
constexpr float kGeluExpC0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
constexpr float kGeluExpC1 = kGeluExpC0 * 0.044715f;
__device__ __forceinline__ float act_gelu_tanh_fast(float u) {
  const float x = u * fmaf(kGeluExpC1, u * u, kGeluExpC0);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}

// ---------------------------------------------------------------- launchers
// Each returns the first HIP error of its launches (hipSuccess if none).

// logits[t,e] = b_r[e] + sum_m x[t,m] W_r[e,m]  (fp32 result)
hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* Wr, const float* br,
                              float* logits, int64_t T, int d, int E, int32_t* zero, int64_t nzero,
                              hipStream_t s);
hipError_t launch_logits_f32(const float* x, const float* Wr, const float* br, float* logits,
                             int64_t T, int d, int E, hipStream_t s);

// softmax, top-nsel, gates; optional per-tile prob sums [ntiles,E] and expert
// histograms of the first k choices [ntiles,E] (tile = kTileTokens tokens).
// ids/gates are [T,nsel] (nsel >= k): the top-k then the next candidates;
// renormalised gates divide by the sum over the first k only.
hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int nsel, int renormalize,
                       int32_t* ids, float* gates, float* prob_part, int32_t* hist, int tb,
                       hipStream_t s);
// Router logits, softmax, top-nsel and gates in one launch for E <= 64
// (route_fused_tokens(T, E) > 0): blocks of route_fused_tokens tokens; per
// block one row of prob_part [blocks,E] (nullable) and of hist [blocks,E]
// (nullable): the counts of the first k choices of its tokens.
int route_fused_tokens(int64_t T, int E);
hipError_t launch_route_fused_bf16(const uint16_t* x, const uint16_t* Wr, const float* br, int64_t T, int d,
                                   int E, int k, int nsel, int renormalize, int32_t* ids, float* gates,
                                   float* prob_part, int32_t* hist, hipStream_t s);
// out[e] = sum over tiles of part[tile,e], tiles in order.
hipError_t launch_prob_reduce(const float* part, int ntiles, int E, float* out, hipStream_t s);

// per-tile expert histograms from topk ids
hipError_t launch_hist(const int32_t* ids, int64_t T, int k, int E, int32_t* hist,
                       hipStream_t s);
// column-wise exclusive prefix of hist over tiles (base), counts, offsets
hipError_t launch_scan(const int32_t* hist, int ntiles, int E, int C, int32_t* base,
                       int32_t* counts, int32_t* offsets, hipStream_t s);
// slots, capacity, row_of, row_token and (when x_perm is not null) the row
// copy into x_perm
hipError_t launch_permute(const void* x, const int32_t* ids, const int32_t* base,
                          const int32_t* offsets, int64_t T, int k, int E, int C,
                          int row_bytes, int32_t* slot, int32_t* row_of, int32_t* row_token,
                          void* x_perm, hipStream_t s);

// scan and permute in one launch, from histograms of hist_tokens (16, 32 or
// 64) tokens per row; valid when fused_scan_fits(rows of hist, E). With
// prob_sum (nullable) it also sums the route's probability partials
// (prob_part [prows, E]) as launch_prob_reduce would.
bool fused_scan_fits(int64_t hist_rows, int E);
hipError_t launch_permute_scan(const void* x, const int32_t* ids, const int32_t* hist, int hist_tokens,
                               int64_t T, int k, int E, int C, int row_bytes, int32_t* counts,
                               int32_t* offsets, int32_t* slot, int32_t* row_of,
                               int32_t* row_token, void* x_perm, const float* prob_part, int prows,
                               float* prob_sum, hipStream_t s);

// Dispatch with a priority order and overflow re-routing rounds. The plan's
// buffers live in the workspace: col/served [T*k], next_col [T], fill/fill0
// [E], hist/base [reroute_tiles(T,k) * E].
struct ReroutePlan {
  int32_t* col;
  int32_t* served;
  int32_t* next_col;
  int32_t* fill;
  int32_t* fill0;
  int32_t* hist;
  int32_t* base;
};
int64_t reroute_tiles(int64_t T, int k);
hipError_t launch_dispatch_reroute(const void* x, const int32_t* cand, const float* cand_gates,
                                   int64_t T, int k, int n, int E, int C, bool rank_priority,
                                   int rounds, int row_bytes, const ReroutePlan& ws,
                                   int32_t* counts, int32_t* offsets, int32_t* slot,
                                   int32_t* row_of, int32_t* row_token, int32_t* served_ids,
                                   float* combine_gates, void* x_perm, hipStream_t s);

// ---- backward (backward.hip)
// dst[g] = src[g]^T for groups of [R, Cc] matrices (2- or 4-byte elements)
hipError_t launch_transpose(const void* src, void* dst, int groups, int R, int Cc, bool bf16,
                            hipStream_t s);
// row_expert[row_of[a]] = ids[a], row_gate[row_of[a]] = gates[a] for kept a
hipError_t launch_row_info(const int32_t* ids, const float* gates, const int32_t* row_of, int64_t T,
                           int k, int32_t* row_expert, float* row_gate, hipStream_t s);
// per kept row: h = sigma(u) rounded as the forward, du = g Z sigma'(u),
// dY = g dy_t, dg_row = <Z, h> + <dy_t, b2_e>
hipError_t launch_bwd_rows(const float* u, const float* Z, const int32_t* row_token,
                           const float* row_gate, const int32_t* row_expert, const int32_t* offsets,
                           int E, const void* dy, const float* b2, int d, int d_ff, int64_t max_rows,
                           bool bf16, int act, void* h, void* du, void* dY, float* dg_row,
                           hipStream_t s);
// ds [T,E] and dsT [E,T]: softmax backward of dp (gates and L_aux terms)
hipError_t launch_router_bwd(const float* logits, const int32_t* ids, const int32_t* row_of,
                             const float* dg_row, const int32_t* counts, int64_t T, int E, int k,
                             int renormalize, float aux_coef, float* ds, float* dsT, hipStream_t s);
// router terms for a few experts (E <= kRouterDirectMaxE):
// dx[t] = sum over kept j of dxp[row_of[t,j]] + sum_e ds[t,e] W_r[e] (W_r
// nullable: the gather only)
constexpr int kRouterDirectMaxE = 16;
hipError_t launch_router_dx(const float* dxp, const int32_t* row_of, const float* ds, const void* W_r,
                            bool w_bf16, int64_t T, int k, int E, int d, float* dx, hipStream_t s);
// dW_r = ds^T x [E,d], db_r (nullable) = column sums of ds; splits > 1 token
// slices through part (splits*E*(d+1) floats), added in slice order
hipError_t launch_router_wgrad(const float* ds, const void* x, bool x_bf16, int64_t T, int E, int d,
                               int splits, float* part, float* dW, float* db, hipStream_t s);
// C[g] (+)= A_g^T B_g over the rows [offsets[g], offsets[g+1]); B rows through
// b_rows; dbias (nullable) gets the column sums of A_g. splits > 1 splits
// each group's rows; part then holds groups*splits*M*(N+1) floats.
hipError_t launch_wgrad(const void* A, bool a_bf16, const void* B, bool b_bf16, const int32_t* b_rows,
                        const int32_t* offsets, int groups, int M, int N, float* C, float* dbias,
                        bool accumulate, int splits, float* part, hipStream_t s);
// poff = exclusive prefix of the experts' row counts rounded up to 64
hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t s);
// dst [Cc, ld]: expert e's rows of src [*, Cc] (through row_idx when given)
// as columns [poff[e], poff[e] + n_e), zeros up to poff[e+1]; colsum_part
// (nullable, bf16 only): the column sums of each 64-row tile of the padded
// rows, [max_padded / 64, Cc]
hipError_t launch_padded_transpose(const void* src, const int32_t* row_idx, const int32_t* offsets,
                                   const int32_t* poff, int E, int Cc, int64_t max_padded, int ld,
                                   bool bf16, void* dst, float* colsum_part,
                                   hipStream_t s);
// out[e][c] = the column sums of expert e's rows from padded_transpose's
// per-tile sums (ascending tiles)
hipError_t launch_seg_colsum(const float* part, const int32_t* poff, int E, int Cc, float* out,
                             hipStream_t s);
// C[e] (MN floats each) = 0 for the experts without rows
hipError_t launch_zero_empty(const int32_t* offsets, int E, int64_t MN, float* C, hipStream_t s);
// C[e] = At_e Bt_e^T over expert e's padded K range (bf16 MFMA, fp32 out);
// experts without rows are skipped
hipError_t launch_wgrad_bf16(const uint16_t* At, const uint16_t* Bt, const int32_t* poff, int E,
                             int M, int N, int lda, float* C, hipStream_t s);
// o = {0, n}
hipError_t launch_range(int32_t* o, int32_t n, hipStream_t s);

// x_perm[row_of[t,j]] = x[t] for every kept assignment (row_of [T,k], -1 = dropped)
hipError_t launch_scatter_rows(const void* x, const int32_t* row_of, int64_t T, int k, int row_bytes,
                               void* x_perm, hipStream_t s);
// x_perm[r] = x[row_token[r]] for r < offsets[E] (rows bounded by max_rows)
hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* offsets,
                              int E, int64_t max_rows, int row_bytes, void* x_perm, hipStream_t s);

// grouped expert GEMMs
//   gemm1: h = act(A W1_e^T + b1_e)   A [rows,K=d], W1 [E,N=d_ff,K], h [rows,N]
//   gemm2: y = A W2_e^T + b2_e        A [rows,K=d_ff], W2 [E,N=d,K], y [rows,N]
// row_idx (nullable): row r of the grouped problem is row row_idx[r] of A.
// out_mode: kGemmOutBf16 (bf16 after act), kGemmOutF32 (fp32, no act), or
// kGemmOutYperm (no act; bf16 when the launch runs whole tiles).
// out2 (nullable; y_perm mode only): a second bf16 [max_rows,N] buffer
// that lets the kernel run tiles as K parts; nsplit (3 words) then receives
// p, r_tail and tail_rows: with p > 1, rows r >= r_tail of the result are
// the sum, in order j = 0 .. p-1, of part 0 = out's row r and part j =
// out2's row (j-1) tail_rows + r - r_tail, each part rounded to bf16.
// cap on the persistent GEMMs' grid (0: one block per CU)
void set_gemm_max_blocks(int blocks);
constexpr int kGemmOutBf16 = 0;
constexpr int kGemmOutF32 = 1;
constexpr int kGemmOutYperm = 2;
hipError_t launch_gemm_bf16(const uint16_t* A, const int32_t* row_idx, const uint16_t* W,
                            const float* bias, void* out, void* out2, int32_t* nsplit,
                            int out_mode, int act, const int32_t* offsets, int E, int N, int K,
                            int64_t max_rows, int max_rows_per_expert, hipStream_t s);
// The same product with each W_e stored [K, N] (the transposed layout, so
// that out = A W_e with W_e as given): fp32 out, no activation, no K split.
// N and K are multiples of 64.
hipError_t launch_gemm_bf16_wt(const uint16_t* A, const int32_t* row_idx, const uint16_t* W,
                               const float* bias, float* out, const int32_t* offsets, int E, int N,
                               int K, int64_t max_rows, int max_rows_per_expert, hipStream_t s);
hipError_t launch_gemm_f32(const float* A, const int32_t* row_idx, const float* W, const float* bias,
                           float* out,
                           int act, const int32_t* offsets, int E, int N, int K,
                           int max_rows_per_expert, hipStream_t s);

// y[t] = sum_j gates[t,j] y_perm[row_of[t,j]] (kept j only), rounded once;
// y_perm rows are bf16 (yperm_bf16) or fp32; with y_perm2 (nullable) and
// nsplit[0] = p > 1, rows r >= nsplit[1] are instead the sums of the second
// GEMM's p bf16 partial rows (launch_gemm_bf16), added first in fp32
hipError_t launch_combine(const void* y_perm, bool yperm_bf16, const void* y_perm2,
                          const int32_t* nsplit, const int32_t* row_of, const float* gates,
                          int64_t T, int k, int d, bool out_bf16, void* y, hipStream_t s);

// load statistics of one routing step (one block): kept [E] = rows per
// expert from offsets, dropped [E] = max(count - kept, 0) (both nullable);
// stats [kNumStats] fp64 in the order below (same values as MOE_STAT_*)
constexpr int kStatDropped = 0;
constexpr int kStatOverflowRatio = 1;
constexpr int kStatMaxOverMean = 2;
constexpr int kStatPaddingRatio = 3;
constexpr int kStatLoadEntropy = 4;
constexpr int kStatKeptVariance = 5;
constexpr int kStatAuxLoss = 6;
constexpr int kStatKeptRows = 7;
constexpr int kNumStats = 8;
hipError_t launch_load_stats(const int32_t* counts, const int32_t* offsets, const float* prob_sum, int E,
                             int C, int64_t T, int k, double alpha, int32_t* kept, int32_t* dropped,
                             double* stats, hipStream_t s);

// activation codes (same values as MOE_ACT_*)
constexpr int kActRelu = 0;
constexpr int kActGeluTanh = 1;
constexpr int kActNone = -1;

}  // namespace moe
