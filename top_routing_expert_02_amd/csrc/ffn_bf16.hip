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
//  * Block tile BM=256 tokens x BN features x BK=64, four waves in a 2x2 grid;
//    each wave owns 128 tokens x BN/2 features as 32x32 v_mfma_f32_32x32x16_bf16
//    tiles. The weight tile is the MFMA A operand and the token tile the B
//    operand, so a lane's accumulators hold 4 consecutive features of one
//    token: the epilogue stores 8-byte (bf16) or 16-byte (fp32) vectors.
//  * LDS holds two stages of both tiles (128 KiB at BN=256). Rows are 128 B
//    (64 bf16); the eight 16-byte chunks of a row are XOR-swizzled with
//    ((row + row/8) & 7) so that ds_read_b128 of 16 consecutive rows at one
//    chunk touches every bank once.
//  * Tiles move global -> LDS with gfx950's LDS-DMA loads (global_load_lds_
//    dwordx4: no staging registers, no ds_write); each lane fetches the chunk
//    the swizzle places at its LDS slot. Double buffered: the loads of K tile
//    kt+1 are in flight while tile kt feeds the matrix cores; one barrier per
//    K tile. Fragments of K16 step s+1 are read from LDS during step s.
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

constexpr int BM = kGemmBM;  // 256
constexpr int BK = 64;
constexpr int ROWB = BK * 2;  // bytes per LDS row

__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row + (row >> 3)) & 7);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Queue one K tile (BK columns) of the token and weight tiles into LDS stage
// `sb` with LDS-DMA loads: instruction i of wave w fills the 1 KiB block
// w*L+i, i.e. rows 8(w*L+i) .. 8(w*L+i)+7.
template <int LA, int LB, int A_BYTES>
__device__ __forceinline__ void issue_tile(const uint16_t* ak, const uint16_t* wk, char* sb,
                                           const int (&aoffs)[LA], const int (&boffs)[LB],
                                           int wave) {
#pragma unroll
  for (int i = 0; i < LA; ++i)
    __builtin_amdgcn_global_load_lds(ak + aoffs[i], (lds_void_t*)(sb + (wave * LA + i) * 1024), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < LB; ++i)
    __builtin_amdgcn_global_load_lds(wk + boffs[i], (lds_void_t*)(sb + A_BYTES + (wave * LB + i) * 1024),
                                     16, 0, 0);
}

// Fragments of K16 step s: tokens tile j (rows 32j..32j+31 of the wave's
// token rows) and weights tile i.
template <int TM, int TN>
__device__ __forceinline__ void load_frags(const char* tb, const char* wb, const int (&fo)[4], int s,
                                           bf16x8_t (&tf)[TM], bf16x8_t (&wf)[TN]) {
#pragma unroll
  for (int j = 0; j < TM; ++j)
    tf[j] = *reinterpret_cast<const bf16x8_t*>(tb + j * 32 * ROWB + fo[s ^ ((j & 1) * 2)]);
#pragma unroll
  for (int i = 0; i < TN; ++i)
    wf[i] = *reinterpret_cast<const bf16x8_t*>(wb + i * 32 * ROWB + fo[s ^ ((i & 1) * 2)]);
}

// One BK-wide K tile from LDS stage `st` into the accumulators; fragments of
// step s+1 are read while step s runs on the matrix cores.
template <int TM, int TN, int A_BYTES, int WM, int WN>
__device__ __forceinline__ void compute_tile(const char* st, const int (&fo)[4], int wm, int wn,
                                             f32x16_t (&acc)[TN][TM]) {
  const char* tb = st + wm * WM * ROWB;
  const char* wb = st + A_BYTES + wn * WN * ROWB;
  bf16x8_t tf0[TM], wf0[TN], tf1[TM], wf1[TN];
  load_frags<TM, TN>(tb, wb, fo, 0, tf0, wf0);
#pragma unroll
  for (int s = 0; s < BK / 16; s += 2) {
    load_frags<TM, TN>(tb, wb, fo, s + 1, tf1, wf1);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf0[i], tf0[j], acc[i][j], 0, 0, 0);
    if (s + 2 < BK / 16) load_frags<TM, TN>(tb, wb, fo, s + 2, tf0, wf0);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf1[i], tf1[j], acc[i][j], 0, 0, 0);
  }
}

}  // namespace

template <int BN, bool OUT_F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                              const float* __restrict__ bias, void* __restrict__ out,
                              const int32_t* __restrict__ offsets, int E, int N, int K,
                              int act) {
  constexpr int WM = BM / 2;   // tokens per wave
  constexpr int WN = BN / 2;   // features per wave
  constexpr int TM = WM / 32;  // 32-token MFMA tiles per wave
  constexpr int TN = WN / 32;  // 32-feature MFMA tiles per wave
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int LA = BM / 32;  // 1 KiB LDS-DMA blocks of the token tile per wave
  constexpr int LB = BN / 32;  // 1 KiB LDS-DMA blocks of the weight tile per wave

  // two stages as distinct objects, so that the compiler can tell the stage
  // being read from the stage the LDS-DMA loads are filling
  __shared__ __attribute__((aligned(1024))) char lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1[STAGE];
  __shared__ int s_tiles[1025];  // exclusive prefix of M tiles per expert
  __shared__ int s_part[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---- device-side schedule: M tiles per expert, exclusive prefix
  {
    const int per = (E + 255) / 256;
    const int eb = tid * per;
    int local = 0;
    for (int e = eb; e < min(E, eb + per); ++e) {
      const int ne = offsets[e + 1] - offsets[e];
      local += (ne + BM - 1) / BM;
    }
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
      const int ne = offsets[e + 1] - offsets[e];
      run += (ne + BM - 1) / BM;
    }
    if (tid == 255) s_tiles[E] = s_part[255];
    __syncthreads();
  }
  const int NT = (N + BN - 1) / BN;
  const int total = s_tiles[E] * NT;

  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int lb = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;

  // Fragment reads. Lane (l5 = lane%32, hi = lane/32) of a 32x32x16 MFMA reads
  // row l5 of a 32-row tile at chunk 2s+hi (K16 step s). With f = (row +
  // row/8) & 7, rows 32j+l5 have f = f0 for even j and f0^4 for odd j, and
  // (2s+hi) ^ (f0^4) = (2(s^2)+hi) ^ f0: four per-lane offsets cover all reads.
  const int l5 = lane & 31, hi = lane >> 5;
  const int f0 = (l5 + (l5 >> 3)) & 7;
  int fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = l5 * ROWB + 16 * (((2 * s) ^ (f0 & 6)) | (hi ^ (f0 & 1)));

  // LDS-DMA: one global_load_lds_dwordx4 fills 1 KiB = 8 rows of 128 B; lane L
  // lands at row L/8, position L%8, so it loads the chunk the swizzle puts
  // there: chunk = position ^ f(row).
  const int drow = lane >> 3, dpos = lane & 7;

  for (int tile = lb; tile < total; tile += G) {
    // expert of this tile: the largest e with s_tiles[e]*NT <= tile
    int lo = 0, hi_e = E - 1;
    while (lo < hi_e) {
      const int mid = (lo + hi_e + 1) >> 1;
      if (s_tiles[mid] * NT <= tile) lo = mid;
      else hi_e = mid - 1;
    }
    const int e = lo;
    const int mte = s_tiles[e + 1] - s_tiles[e];
    const int u = tile - s_tiles[e] * NT;
    const int nt = u / mte;
    const int mt = u - nt * mte;
    const int row0 = offsets[e] + mt * BM;
    const int rv = min(BM, offsets[e + 1] - row0);  // valid rows in this tile
    const int n0 = nt * BN;

    const uint16_t* Abase = A + static_cast<int64_t>(row0) * K;
    const uint16_t* Wbase = W + (static_cast<int64_t>(e) * N + n0) * K;
    int aoffs[LA], boffs[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (wave * LA + i) * 8 + drow;
      const int c = dpos ^ ((r + (r >> 3)) & 7);
      aoffs[i] = min(r, rv - 1) * K + c * 8;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (wave * LB + i) * 8 + drow;
      const int c = dpos ^ ((r + (r >> 3)) & 7);
      boffs[i] = (min(n0 + r, N - 1) - n0) * K + c * 8;
    }

    f32x16_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    const int nk = K / BK;
    issue_tile<LA, LB, A_BYTES>(Abase, Wbase, lds0, aoffs, boffs, wave);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // tile kt sits in lds0 at the top of each pair
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      issue_tile<LA, LB, A_BYTES>(Abase + (kt + 1) * BK, Wbase + (kt + 1) * BK, lds1, aoffs, boffs, wave);
      compute_tile<TM, TN, A_BYTES, WM, WN>(lds0, fo, wm, wn, acc);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 2 < nk)
        issue_tile<LA, LB, A_BYTES>(Abase + (kt + 2) * BK, Wbase + (kt + 2) * BK, lds0, aoffs, boffs, wave);
      compute_tile<TM, TN, A_BYTES, WM, WN>(lds1, fo, wm, wn, acc);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (kt < nk) {
      compute_tile<TM, TN, A_BYTES, WM, WN>(lds0, fo, wm, wn, acc);
      __syncthreads();
    }

    // ---- epilogue: lane holds token (lane%32) of each 32-token tile j and
    // features 8q + 4*(lane/32) + {0..3} of each 32-feature tile i.
    const float* be = bias != nullptr ? bias + static_cast<int64_t>(e) * N : nullptr;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = wm * WM + j * 32 + (lane & 31);
      if (m >= rv) continue;
      const int64_t orow = static_cast<int64_t>(row0 + m) * N;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WN + i * 32 + q * 8 + (lane >> 5) * 4;
          if (n >= N) continue;
          float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
          float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          if (be != nullptr) {
            const float4 bb = *reinterpret_cast<const float4*>(be + n);
            v0 += bb.x; v1 += bb.y; v2 += bb.z; v3 += bb.w;
          }
          if (act == kActRelu) {
            v0 = act_relu(v0); v1 = act_relu(v1); v2 = act_relu(v2); v3 = act_relu(v3);
          } else if (act == kActGeluTanh) {
            v0 = act_gelu_tanh(v0); v1 = act_gelu_tanh(v1);
            v2 = act_gelu_tanh(v2); v3 = act_gelu_tanh(v3);
          }
          if constexpr (OUT_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + n) = make_float4(v0, v1, v2, v3);
          } else {
            uint2 o;
            o.x = f32_to_bf16(v0) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16);
            o.y = f32_to_bf16(v2) | (static_cast<uint32_t>(f32_to_bf16(v3)) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow + n) = o;
          }
        }
      }
    }
  }
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

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* out,
                            bool out_f32, int act, const int32_t* offsets, int E, int N, int K,
                            int64_t max_rows, int max_rows_per_expert, hipStream_t s) {
  (void)max_rows_per_expert;
  if (max_rows <= 0) return hipSuccess;
  // upper bound on tiles: sum_e ceil(n_e/BM) <= max_rows/BM + E
  const int64_t mt_bound = max_rows / BM + E;
  const int cus = cu_count();
  if (out_f32) {
    constexpr int BN = 128;
    const int64_t tiles = mt_bound * ((N + BN - 1) / BN);
    const unsigned grid = static_cast<unsigned>(tiles < cus ? tiles : cus);
    grouped_gemm_bf16_kernel<BN, true><<<grid, 256, 0, s>>>(A, W, bias, out, offsets, E, N, K, act);
  } else {
    constexpr int BN = 256;
    const int64_t tiles = mt_bound * ((N + BN - 1) / BN);
    const unsigned grid = static_cast<unsigned>(tiles < cus ? tiles : cus);
    grouped_gemm_bf16_kernel<BN, false><<<grid, 256, 0, s>>>(A, W, bias, out, offsets, E, N, K, act);
  }
  return hipGetLastError();
}

}  // namespace moe
