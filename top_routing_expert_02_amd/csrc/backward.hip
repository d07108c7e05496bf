// Backward pass of the MoE layer: gradients of L = <dy, y> + L_aux with the
// routing and capacity decisions of the forward held fixed (page "MoE 模型原理：
// 路由、专家负载、容量、通信与推理成本", wrblog.cn: §2.4, a chosen expert gets its
// gradient through the combine weight; §3.2, L_aux = alpha E sum_i f_i pbar_i
// with f_i a count; §9.1 lists expert backward and combine backward among the
// training steps).
//
// Kernels here (the expert dgrad GEMMs reuse the forward's grouped GEMMs on
// transposed weights):
//   transpose        W[e] [R,C] -> Wt[e] [C,R]
//   row_info         per kept row: its gate and expert
//   bwd_rows         per kept row: h = sigma(u) (as the forward rounds it),
//                    du = g Z sigma'(u), dY = g dy_t, and the combine-weight
//                    gradient dg = <Z, h> + <dy_t, b2_e> (Z = dy_t W2_e)
//   router_bwd       per token: softmax probabilities from the logits, dp
//                    through the (renormalised) gates and L_aux, ds (softmax
//                    backward), in [T,E] and [E,T] layouts
//   dx_gather        dx_t = sum over kept j of dx_perm[row_of[t,j]]
//   wgrad            C[g] (+)= A_g^T B_g over the rows of group g (fp32
//                    accumulate, 64x64 tiles, optional split over rows with
//                    an in-order reduction), and the column sums of A_g as
//                    one extra column of ones: dW1/db1, dW2/db2, dW_r/db_r,
//                    and ds W_r
// Every reduction runs in a fixed order: results are deterministic.
#include "moe_internal.h"

namespace moe {

namespace {

template <typename TE>
__device__ __forceinline__ float ld(const TE* p, int64_t i) {
  if constexpr (sizeof(TE) == 2) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

template <typename TE>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (sizeof(TE) == 2) return static_cast<float>(static_cast<__bf16>(v));
  else return v;
}

template <typename TE>
__device__ __forceinline__ void st(TE* p, int64_t i, float v) {
  if constexpr (sizeof(TE) == 2) {
    const __bf16 b = static_cast<__bf16>(v);
    reinterpret_cast<__bf16*>(p)[i] = b;
  } else {
    reinterpret_cast<float*>(p)[i] = v;
  }
}

// dst[e][c][r] = src[e][r][c]; 64x64 tiles through LDS
template <typename TE>
__global__ __launch_bounds__(256) void transpose_kernel(const TE* __restrict__ src, TE* __restrict__ dst,
                                                        int R, int Cc) {
  __shared__ TE tile[64][65];
  const int64_t e = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const TE* s = src + e * R * static_cast<int64_t>(Cc);
  TE* d = dst + e * R * static_cast<int64_t>(Cc);
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < Cc) tile[i][tx] = s[static_cast<int64_t>(r) * Cc + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < R && c < Cc) d[static_cast<int64_t>(c) * R + r] = tile[tx][i];
  }
}

// bf16 transposes move 4-byte pairs: a thread reads the same two columns of
// two consecutive rows, repacks them into two (row, row+1) pairs of the
// transposed matrix and the tile goes through LDS in 32-bit words (pitch 33:
// conflict-free). row_ptr(i) gives source row i of the 64-row tile, or null
// for a row of zeros; the tile lands at dst[c][dcol0 + i].
// colsum (nullable): colsum[c0 + c] = the sum over the tile's 64 rows of
// column c0 + c (fp32, rows in ascending order within each thread's four
// pairs, then the four threads of a column in lane order)
template <typename RowPtr>
__device__ __forceinline__ void transpose_tile_bf16(RowPtr row_ptr, int c0, int Cc, uint16_t* dst,
                                                    int64_t ldd, int64_t dcol0,
                                                    float* colsum = nullptr) {
  __shared__ uint32_t t32[64][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rp = ty + 8 * i;  // row pair
    const uint16_t* ra = row_ptr(2 * rp);
    const uint16_t* rb = row_ptr(2 * rp + 1);
    const int c = c0 + 2 * tx;
    uint32_t a = 0, b = 0;
    if (c < Cc) {
      if (ra != nullptr) a = *reinterpret_cast<const uint32_t*>(ra + c);
      if (rb != nullptr) b = *reinterpret_cast<const uint32_t*>(rb + c);
    }
    t32[2 * tx][rp] = (a & 0xFFFFu) | (b << 16);
    t32[2 * tx + 1][rp] = (a >> 16) | (b & 0xFFFF0000u);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cl = ty + 8 * i;
    if (c0 + cl < Cc)
      *reinterpret_cast<uint32_t*>(dst + static_cast<int64_t>(c0 + cl) * ldd + dcol0 + 2 * tx) = t32[cl][tx];
  }
  if (colsum != nullptr) {
    // column cl = thread / 4; its 32 row pairs in four runs of 8
    const int cl = threadIdx.x >> 2, part = threadIdx.x & 3;
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t v = t32[cl][part * 8 + k];
      sum += __uint_as_float(v << 16);
      sum += __uint_as_float(v & 0xFFFF0000u);
    }
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    if (part == 0 && c0 + cl < Cc) colsum[c0 + cl] = sum;
  }
}

// dst[e][c][r] = src[e][r][c] for bf16, R and Cc even
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst, int R, int Cc) {
  const int64_t e = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const uint16_t* s = src + e * R * static_cast<int64_t>(Cc);
  uint16_t* d = dst + e * R * static_cast<int64_t>(Cc);
  transpose_tile_bf16([&](int i) -> const uint16_t* {
    return (r0 + i < R) ? s + static_cast<int64_t>(r0 + i) * Cc : nullptr;
  }, c0, Cc, d, R, r0);
}

__global__ __launch_bounds__(256) void row_info_kernel(const int32_t* __restrict__ ids,
                                                       const float* __restrict__ gates,
                                                       const int32_t* __restrict__ row_of,
                                                       int64_t Tk, int32_t* __restrict__ row_expert,
                                                       float* __restrict__ row_gate) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (a >= Tk) return;
  const int row = row_of[a];
  if (row < 0) return;
  row_expert[row] = ids[a];
  row_gate[row] = gates[a];
}

__device__ __forceinline__ float gelu_tanh_grad(float u) {
  // d/du 0.5 u (1 + tanh z), z = a (u + b u^3): 0.5 (1 + th) + 0.5 u (1 - th^2) a (1 + 3 b u^2)
  constexpr float a = 0.7978845608028654f, b = 0.044715f;
  const float z = a * fmaf(b * u * u, u, u);
  const float th = 1.0f - 2.0f / (1.0f + __expf(2.0f * z));
  return 0.5f * (1.0f + th) + 0.5f * u * (1.0f - th * th) * a * fmaf(3.0f * b, u * u, 1.0f);
}

template <typename TE, int ACT>
__device__ __forceinline__ float act_fwd(float u) {
  if constexpr (ACT == kActRelu) return act_relu(u);
  else if constexpr (sizeof(TE) == 2) return act_gelu_tanh_fast(u);  // as the bf16 GEMM epilogue
  else return act_gelu_tanh(u);                                     // as the fp32 GEMM
}

template <int ACT>
__device__ __forceinline__ float act_grad(float u) {
  if constexpr (ACT == kActRelu) return u > 0.f ? 1.f : 0.f;
  else return gelu_tanh_grad(u);
}

// bf16 layers: h and dh/du of the tanh-GELU from one exp2 and one rcp.
// With E = exp2(u (c1 u^2 + c0)) = exp(-2z) (the forward epilogue's form) and
// s = 1 / (1 + E): h = u s (bit-identical to the forward), tanh z = 2 s - 1,
// 1 - tanh^2 z = 4 s (1 - s), so dh/du = s + 2 a u s (1 - s) (1 + 3 b u^2).
__device__ __forceinline__ void gelu_tanh_fwd_grad_fast(float u, float& h, float& dh) {
  constexpr float a = 0.7978845608028654f, b3 = 3.0f * 0.044715f;
  const float uu = u * u;
  const float x = u * fmaf(kGeluExpC1, uu, kGeluExpC0);
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
  h = u * sg;
  dh = fmaf(2.0f * a * u * sg * (1.0f - sg), fmaf(b3, uu, 1.0f), sg);
}

// the activation (rounded as the layer stores it) and its derivative
template <typename TE, int ACT>
__device__ __forceinline__ void act_fwd_grad(float u, float& h, float& dh) {
  if constexpr (ACT == kActGeluTanh && sizeof(TE) == 2) {
    gelu_tanh_fwd_grad_fast(u, h, dh);
    h = round_to<TE>(h);
  } else {
    h = round_to<TE>(act_fwd<TE, ACT>(u));
    dh = act_grad<ACT>(u);
  }
}

// VEC consecutive elements i .. i + VEC - 1 of an fp32 or bf16 array
template <int VEC, typename TE>
__device__ __forceinline__ void st_vec(TE* p, int64_t i, const float (&v)[VEC]) {
  if constexpr (VEC == 4 && sizeof(TE) == 2) {
    uint2 o;
    o.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    o.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p) + i) = o;
  } else if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int q = 0; q < VEC; ++q) st(p, i + q, v[q]);
  }
}
template <int VEC, typename TE>
__device__ __forceinline__ void ld_vec(const TE* p, int64_t i, float (&v)[VEC]) {
  if constexpr (VEC == 4 && sizeof(TE) == 2) {
    const uint2 q = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
  } else if constexpr (VEC == 4) {
    const float4 q = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  } else {
#pragma unroll
    for (int q = 0; q < VEC; ++q) v[q] = ld(p, i + q);
  }
}

// one block per kept row; VEC consecutive elements per thread (d and d_ff
// multiples of VEC)
template <typename TE, int ACT, int VEC>
__global__ __launch_bounds__(256) void bwd_rows_kernel(
    const float* __restrict__ u, const float* __restrict__ Z, const int32_t* __restrict__ row_token,
    const float* __restrict__ row_gate, const int32_t* __restrict__ row_expert,
    const int32_t* __restrict__ offsets, int E, const TE* __restrict__ dy, const float* __restrict__ b2,
    int d, int d_ff, TE* __restrict__ h, TE* __restrict__ du, TE* __restrict__ dY,
    float* __restrict__ dg_row) {
  __shared__ float red[256];
  const int64_t r = blockIdx.x;
  if (r >= offsets[E]) return;
  const int64_t t = row_token[r];
  const float g = row_gate[r];
  const int e = row_expert[r];
  float dot = 0.f;
  for (int c = threadIdx.x * VEC; c < d_ff; c += 256 * VEC) {
    const int64_t i = r * d_ff + c;
    float uv[VEC], z[VEC], hv[VEC], dv[VEC];
    ld_vec<VEC>(u, i, uv);
    ld_vec<VEC>(Z, i, z);
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      float dh;
      act_fwd_grad<TE, ACT>(uv[q], hv[q], dh);
      dot = fmaf(z[q], hv[q], dot);
      dv[q] = g * z[q] * dh;
    }
    st_vec<VEC>(h, i, hv);
    st_vec<VEC>(du, i, dv);
  }
  for (int c = threadIdx.x * VEC; c < d; c += 256 * VEC) {
    float yv[VEC], o[VEC];
    ld_vec<VEC>(dy, t * d + c, yv);
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      if (b2 != nullptr) dot = fmaf(yv[q], b2[static_cast<int64_t>(e) * d + c + q], dot);
      o[q] = g * yv[q];
    }
    st_vec<VEC>(dY, r * d + c, o);
  }
  red[threadIdx.x] = dot;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) dg_row[r] = red[0];
}

// one wave per token
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ids, const int32_t* __restrict__ row_of,
    const float* __restrict__ dg_row, const int32_t* __restrict__ counts, int64_t T, int E, int k,
    int renormalize, float aux_coef, float* __restrict__ ds, float* __restrict__ dsT) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* s = logits + t * E;
  float mx = -__builtin_inff();
  for (int i = lane; i < E; i += 64) mx = fmaxf(mx, s[i]);
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  float se = 0.f;
  for (int i = lane; i < E; i += 64) se += __expf(s[i] - mx);
  for (int off = 32; off >= 1; off >>= 1) se += __shfl_xor(se, off, 64);
  const float inv = 1.0f / se;
  // the token's chosen experts: probabilities, their sum, dg and sum dg g
  float P = 0.f, dgg = 0.f;
  for (int j = 0; j < k; ++j) {
    const int i = ids[t * k + j];
    P += __expf(s[i] - mx) * inv;
  }
  for (int j = 0; j < k; ++j) {
    const int i = ids[t * k + j];
    const int row = row_of[t * k + j];
    const float dg = row >= 0 ? dg_row[row] : 0.f;
    const float pj = __expf(s[i] - mx) * inv;
    dgg += dg * (pj / P);
  }
  // dp_i and the softmax backward
  float pdp = 0.f;
  for (int i = lane; i < E; i += 64) {
    const float p = __expf(s[i] - mx) * inv;
    float dp = aux_coef * static_cast<float>(counts[i]);
    for (int j = 0; j < k; ++j) {
      if (ids[t * k + j] != i) continue;
      const int row = row_of[t * k + j];
      const float dg = row >= 0 ? dg_row[row] : 0.f;
      dp += renormalize ? (dg - dgg) / P : dg;
    }
    pdp += p * dp;
  }
  for (int off = 32; off >= 1; off >>= 1) pdp += __shfl_xor(pdp, off, 64);
  for (int i = lane; i < E; i += 64) {
    const float p = __expf(s[i] - mx) * inv;
    float dp = aux_coef * static_cast<float>(counts[i]);
    for (int j = 0; j < k; ++j) {
      if (ids[t * k + j] != i) continue;
      const int row = row_of[t * k + j];
      const float dg = row >= 0 ? dg_row[row] : 0.f;
      dp += renormalize ? (dg - dgg) / P : dg;
    }
    const float v = p * (dp - pdp);
    ds[t * E + i] = v;
    dsT[static_cast<int64_t>(i) * T + t] = v;
  }
}

// VEC consecutive values as floats (one 16- or 8-byte load for VEC = 4)
template <int VEC>
__device__ __forceinline__ void load_vec(const float* p, float (&o)[VEC]) {
  if constexpr (VEC == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    o[0] = q.x;
    o[1] = q.y;
    o[2] = q.z;
    o[3] = q.w;
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[v] = p[v];
  }
}
template <int VEC>
__device__ __forceinline__ void load_vec(const uint16_t* p, float (&o)[VEC]) {
  if constexpr (VEC == 4) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(q.x << 16);
    o[1] = __uint_as_float(q.x & 0xffff0000u);
    o[2] = __uint_as_float(q.y << 16);
    o[3] = __uint_as_float(q.y & 0xffff0000u);
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[v] = ld(p, v);
  }
}

// dx[t] = sum over kept j of dxp[row_of[t,j]], plus (W_r given) the router
// term sum_e ds[t,e] W_r[e], formed separately in expert order and added
// last; VEC consecutive columns per thread.
template <typename TW, int VEC>
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dxp,
                                                        const int32_t* __restrict__ row_of,
                                                        const float* __restrict__ ds,
                                                        const TW* __restrict__ W_r, int64_t T, int k,
                                                        int E, int d, float* __restrict__ dx) {
  const int chunks = d / VEC;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= T * chunks) return;
  const int64_t t = i / chunks;
  const int c = static_cast<int>(i - t * chunks) * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int row = row_of[t * k + j];
    if (row < 0) continue;
    const float* src = dxp + static_cast<int64_t>(row) * d + c;
    if constexpr (VEC == 4) {
      const float4 q = *reinterpret_cast<const float4*>(src);
      acc[0] += q.x;
      acc[1] += q.y;
      acc[2] += q.z;
      acc[3] += q.w;
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] += src[v];
    }
  }
  if (W_r != nullptr) {
    float r[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[v] = 0.f;
    for (int e = 0; e < E; ++e) {
      const float g = ds[t * E + e];
      float w[VEC];
      load_vec<VEC>(W_r + static_cast<int64_t>(e) * d + c, w);
#pragma unroll
      for (int v = 0; v < VEC; ++v) r[v] = fmaf(g, w[v], r[v]);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += r[v];
  }
  float* dst = dx + t * d + c;
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) dst[v] = acc[v];
  }
}

// Router weight gradient for a few experts (E <= EMAX <= kRouterDirectMaxE):
//   dW_r[e][n] = sum_t ds[t,e] x[t,n],  db_r[e] = sum_t ds[t,e].
// Block (bx, sl) takes columns [256 VEC bx, 256 VEC (bx + 1)) (VEC per
// thread, all E sums in registers) and the sl-th of S token slices, in chunks
// of 64 tokens whose ds rows wait in LDS (zero-padded to EMAX); x is read 8
// tokens at a time, the loads of a batch in flight together. S == 1 writes
// dW and db; else part[sl] [E, d+1] (column d: the bias sums) for
// wgrad_reduce_kernel, which adds the slices in order.
template <typename TX, int EMAX, int VEC>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* __restrict__ ds,
                                                           const TX* __restrict__ x, int64_t T, int E,
                                                           int d, int S, float* __restrict__ part,
                                                           float* __restrict__ dW,
                                                           float* __restrict__ db) {
  constexpr int kChunk = 64, kBatch = 8;
  __shared__ __attribute__((aligned(16))) float s_ds[kChunk * EMAX];
  const int c = (blockIdx.x * 256 + threadIdx.x) * VEC;
  const int sl = blockIdx.y;
  const int64_t t0 = T * sl / S, t1 = T * (sl + 1) / S;
  const bool bias_thread = blockIdx.x == 0 && static_cast<int>(threadIdx.x) < E;
  float acc[EMAX][VEC];
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[e][v] = 0.f;
  float bacc = 0.f;
  auto token = [&](const float (&xv)[VEC], const float* g) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[e][v] = fmaf(g[e], xv[v], acc[e][v]);
  };
  for (int64_t tb = t0; tb < t1; tb += kChunk) {
    const int nt = static_cast<int>(min(static_cast<int64_t>(kChunk), t1 - tb));
    __syncthreads();
    for (int q = threadIdx.x; q < nt * EMAX; q += 256) {
      const int tt = q / EMAX, e = q - tt * EMAX;
      s_ds[q] = e < E ? ds[(tb + tt) * E + e] : 0.f;
    }
    __syncthreads();
    if (c < d) {
      const TX* xc = x + tb * d + c;
      int b0 = 0;
      for (; b0 + kBatch <= nt; b0 += kBatch) {
        float xv[kBatch][VEC];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) load_vec<VEC>(xc + static_cast<int64_t>(b0 + u) * d, xv[u]);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) token(xv[u], s_ds + (b0 + u) * EMAX);
      }
      for (; b0 < nt; ++b0) {
        float xv[VEC];
        load_vec<VEC>(xc + static_cast<int64_t>(b0) * d, xv);
        token(xv, s_ds + b0 * EMAX);
      }
    }
    if (bias_thread)
      for (int tt = 0; tt < nt; ++tt) bacc += s_ds[tt * EMAX + threadIdx.x];
  }
  float* out = dW;
  int64_t ld_out = d;
  if (S > 1) {
    out = part + static_cast<int64_t>(sl) * E * (d + 1);
    ld_out = d + 1;
  }
  if (c < d)
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E)
#pragma unroll
        for (int v = 0; v < VEC; ++v) out[e * ld_out + c + v] = acc[e][v];
  if (bias_thread) {
    if (S > 1) out[threadIdx.x * ld_out + d] = bacc;
    else if (db != nullptr) db[threadIdx.x] = bacc;
  }
}

// C[g][m][n] (+)= sum over rows r of group g of A[r][m] * B[src(r)][n]
// (src(r) = b_rows[r] when given). Group g holds rows [offsets[g],
// offsets[g+1]). 64x64 output tiles, 16 rows per step, 4x4 per thread.
// With dbias, column N is a column of ones: dbias[g][m] = sum_r A[r][m].
// With splits > 1, block z = g * splits + s takes the s-th slice of the
// group's rows and writes its partial sums to part[z] ([M, N+1]); a second
// kernel adds the slices in order.
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void wgrad_kernel(const TA* __restrict__ A, const TB* __restrict__ B,
                                                    const int32_t* __restrict__ b_rows,
                                                    const int32_t* __restrict__ offsets, int M, int N,
                                                    int splits, float* __restrict__ C,
                                                    float* __restrict__ dbias, int accumulate,
                                                    float* __restrict__ part) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int64_t g = blockIdx.z / splits;
  const int sp = blockIdx.z - static_cast<int>(g) * splits;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int g_begin = offsets[g], g_end = offsets[g + 1];
  const int chunk = ((g_end - g_begin + splits - 1) / splits + 15) & ~15;
  const int r_begin = min(g_end, g_begin + sp * chunk);
  const int r_end = min(g_end, r_begin + chunk);
  const int NB = dbias != nullptr ? N + 1 : N;  // columns incl. the ones column
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int r0 = r_begin; r0 < r_end; r0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = threadIdx.x + q * 256;
      const int rr = idx >> 6, cc = idx & 63;
      const int r = r0 + rr;
      const bool rv = r < r_end;
      As[rr][cc] = (rv && m0 + cc < M) ? ld(A, static_cast<int64_t>(r) * M + m0 + cc) : 0.f;
      const int n = n0 + cc;
      float bv = 0.f;
      if (rv && n < N) {
        const int64_t src = b_rows != nullptr ? b_rows[r] : r;
        bv = ld(B, src * N + n);
      } else if (rv && n == N) {
        bv = 1.f;  // the ones column (only reached when dbias is given: NB = N + 1)
      }
      Bs[rr][cc] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= NB) continue;
      if (splits > 1) {
        part[(static_cast<int64_t>(blockIdx.z) * M + m) * NB + n] = acc[i][j];
      } else if (n < N) {
        const int64_t o = (g * M + m) * static_cast<int64_t>(N) + n;
        C[o] = accumulate ? C[o] + acc[i][j] : acc[i][j];
      } else {
        dbias[g * M + m] = acc[i][j];
      }
    }
  }
}

// C[g][m][n] (+)= sum over s of part[g*splits+s][m][n], s in order; column N
// of the partials (when present) goes to dbias.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ part, int groups,
                                                           int splits, int M, int N, int NB,
                                                           float* __restrict__ C,
                                                           float* __restrict__ dbias, int accumulate) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per = static_cast<int64_t>(M) * NB;
  if (i >= per * groups) return;
  const int64_t g = i / per;
  const int64_t mn = i - g * per;
  const int m = static_cast<int>(mn / NB);
  const int n = static_cast<int>(mn - static_cast<int64_t>(m) * NB);
  // the slices in order, their loads eight at a time
  float acc = 0.f;
  int sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = part[(g * splits + sp + q) * per + mn];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += v[q];
  }
  for (; sp < splits; ++sp) acc += part[(g * splits + sp) * per + mn];
  if (n < N) {
    const int64_t o = (g * M + m) * static_cast<int64_t>(N) + n;
    C[o] = accumulate ? C[o] + acc : acc;
  } else if (dbias != nullptr) {
    dbias[g * M + m] = acc;
  }
}

// poff = exclusive prefix of the experts' row counts rounded up to 64
// (one block, E <= 1024)
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int32_t* __restrict__ poff) {
  __shared__ int s[1024];
  const int e = threadIdx.x;
  const int v = (e < E) ? ((offsets[e + 1] - offsets[e] + 63) & ~63) : 0;
  s[e] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (e >= off) ? s[e - off] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  if (e < E) poff[e] = s[e] - v;
  if (e == E - 1) poff[E] = s[e];
}

// dst[c][poff[e] + i] = src[row(offsets[e] + i)][c] for i < n_e and 0 for
// n_e <= i < padded n_e (row(r) = row_idx[r] when given); 64x64 tiles, a
// tile never straddles experts (poff is a multiple of 64)
template <typename TE>
__global__ __launch_bounds__(256) void padded_transpose_kernel(const TE* __restrict__ src,
                                                               const int32_t* __restrict__ row_idx,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ poff, int E,
                                                               int Cc, int ldd, TE* __restrict__ dst) {
  __shared__ TE tile[64][65];
  const int p0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (p0 >= poff[E]) return;
  int lo = 0, hi = E - 1;  // the expert e with poff[e] <= p0 < poff[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= p0) lo = mid;
    else hi = mid - 1;
  }
  const int ne = offsets[lo + 1] - offsets[lo];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int local = p0 - poff[lo] + i;
    const int c = c0 + tx;
    TE v{};
    if (local < ne && c < Cc) {
      const int64_t r = offsets[lo] + local;
      const int64_t row = row_idx != nullptr ? row_idx[r] : r;
      v = src[row * Cc + c];
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i;
    if (c < Cc) dst[static_cast<int64_t>(c) * ldd + p0 + tx] = tile[tx][i];
  }
}

// the same for bf16 through 4-byte pairs (see transpose_tile_bf16)
// colsum_part (nullable): per 64-row tile of the padded rows, the column
// sums of that tile ([padded rows / 64, Cc])
__global__ __launch_bounds__(256) void padded_transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                                    const int32_t* __restrict__ row_idx,
                                                                    const int32_t* __restrict__ offsets,
                                                                    const int32_t* __restrict__ poff, int E,
                                                                    int Cc, int ldd,
                                                                    uint16_t* __restrict__ dst,
                                                                    float* __restrict__ colsum_part) {
  const int p0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (p0 >= poff[E]) return;
  int lo = 0, hi = E - 1;  // the expert e with poff[e] <= p0 < poff[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= p0) lo = mid;
    else hi = mid - 1;
  }
  const int ne = offsets[lo + 1] - offsets[lo];
  const int first = p0 - poff[lo];
  const int64_t rbase = offsets[lo];
  transpose_tile_bf16([&](int i) -> const uint16_t* {
    const int local = first + i;
    if (local >= ne) return nullptr;
    const int64_t r = rbase + local;
    const int64_t row = row_idx != nullptr ? row_idx[r] : r;
    return src + row * Cc;
  }, c0, Cc, dst, ldd, p0,
     colsum_part != nullptr ? colsum_part + static_cast<int64_t>(blockIdx.y) * Cc : nullptr);
}

// out[e][c] = sum over expert e's 64-row tiles pt (ascending) of
// part[pt][c]: the column sums of the expert's rows (zero without rows)
__global__ __launch_bounds__(256) void seg_colsum_kernel(const float* __restrict__ part,
                                                         const int32_t* __restrict__ poff, int E, int Cc,
                                                         float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(E) * Cc) return;
  const int e = static_cast<int>(i / Cc);
  const int c = static_cast<int>(i - static_cast<int64_t>(e) * Cc);
  const int t0 = poff[e] / 64, t1 = poff[e + 1] / 64;
  float acc = 0.f;
  int pt = t0;
  for (; pt + 8 <= t1; pt += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = part[static_cast<int64_t>(pt + q) * Cc + c];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += v[q];
  }
  for (; pt < t1; ++pt) acc += part[static_cast<int64_t>(pt) * Cc + c];
  out[i] = acc;
}

// C[e] = 0 for the experts without rows (block y = expert)
__global__ __launch_bounds__(256) void zero_empty_kernel(const int32_t* __restrict__ offsets, int64_t MN,
                                                         float* __restrict__ C) {
  const int64_t e = blockIdx.y;
  if (offsets[e + 1] > offsets[e]) return;
  float* Ce = C + e * MN;
  // 16-byte stores where the matrix starts 16-byte aligned, then the rest
  const int64_t n4 = (reinterpret_cast<uintptr_t>(Ce) & 15) == 0 ? MN / 4 : 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (int64_t i = i0; i < n4; i += stride)
    reinterpret_cast<float4*>(Ce)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = 4 * n4 + i0; i < MN; i += stride) Ce[i] = 0.f;
}

__global__ void range_kernel(int32_t* __restrict__ o, int32_t n) {
  if (threadIdx.x == 0) {
    o[0] = 0;
    o[1] = n;
  }
}

unsigned blocks(int64_t n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

}  // namespace

hipError_t launch_transpose(const void* src, void* dst, int groups, int R, int Cc, bool bf16,
                            hipStream_t s) {
  dim3 grid(blocks(Cc, 64), blocks(R, 64), groups);
  if (bf16)
    transpose_bf16_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src),
                                               static_cast<uint16_t*>(dst), R, Cc);
  else
    transpose_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(src),
                                                 static_cast<float*>(dst), R, Cc);
  return hipGetLastError();
}

hipError_t launch_row_info(const int32_t* ids, const float* gates, const int32_t* row_of, int64_t T,
                           int k, int32_t* row_expert, float* row_gate, hipStream_t s) {
  row_info_kernel<<<blocks(T * k, 256), 256, 0, s>>>(ids, gates, row_of, T * k, row_expert,
                                                      row_gate);
  return hipGetLastError();
}

hipError_t launch_bwd_rows(const float* u, const float* Z, const int32_t* row_token,
                           const float* row_gate, const int32_t* row_expert, const int32_t* offsets,
                           int E, const void* dy, const float* b2, int d, int d_ff, int64_t max_rows,
                           bool bf16, int act, void* h, void* du, void* dY, float* dg_row,
                           hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(max_rows);
#define MOE_BWD_ROWS(TE, ACT, V)                                                                        \
  bwd_rows_kernel<TE, ACT, V><<<grid, 256, 0, s>>>(u, Z, row_token, row_gate, row_expert, offsets, E, \
                                                   static_cast<const TE*>(dy), b2, d, d_ff,          \
                                                   static_cast<TE*>(h), static_cast<TE*>(du),        \
                                                   static_cast<TE*>(dY), dg_row)
  // bf16 layers have d and d_ff multiples of 64; fp32 layers take 4-wide
  // vectors when both are multiples of 4
  if (bf16) {
    if (act == kActRelu) MOE_BWD_ROWS(uint16_t, kActRelu, 4);
    else MOE_BWD_ROWS(uint16_t, kActGeluTanh, 4);
  } else if (d % 4 == 0 && d_ff % 4 == 0) {
    if (act == kActRelu) MOE_BWD_ROWS(float, kActRelu, 4);
    else MOE_BWD_ROWS(float, kActGeluTanh, 4);
  } else {
    if (act == kActRelu) MOE_BWD_ROWS(float, kActRelu, 1);
    else MOE_BWD_ROWS(float, kActGeluTanh, 1);
  }
#undef MOE_BWD_ROWS
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const int32_t* ids, const int32_t* row_of,
                             const float* dg_row, const int32_t* counts, int64_t T, int E, int k,
                             int renormalize, float aux_coef, float* ds, float* dsT, hipStream_t s) {
  router_bwd_kernel<<<blocks(T, 4), 256, 0, s>>>(logits, ids, row_of, dg_row, counts, T, E, k,
                                                  renormalize, aux_coef, ds, dsT);
  return hipGetLastError();
}

hipError_t launch_router_dx(const float* dxp, const int32_t* row_of, const float* ds, const void* W_r,
                            bool w_bf16, int64_t T, int k, int E, int d, float* dx, hipStream_t s) {
#define MOE_RDX(TW, V)                                                                          \
  router_dx_kernel<TW, V><<<blocks(T * (d / V), 256), 256, 0, s>>>(dxp, row_of, ds,             \
                                                                  static_cast<const TW*>(W_r), \
                                                                  T, k, E, d, dx)
  if (d % 4 == 0) {
    if (w_bf16) MOE_RDX(uint16_t, 4);
    else MOE_RDX(float, 4);
  } else {
    if (w_bf16) MOE_RDX(uint16_t, 1);
    else MOE_RDX(float, 1);
  }
#undef MOE_RDX
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const float* ds, const void* x, bool x_bf16, int64_t T, int E, int d,
                               int splits, float* part, float* dW, float* db, hipStream_t s) {
  if (E > kRouterDirectMaxE || splits < 1 || (splits > 1 && part == nullptr)) return hipErrorInvalidValue;
  const int vec = d % 4 == 0 ? 4 : 1;
  dim3 grid(blocks(d, 256 * vec), splits);
#define MOE_RWG(TX, EM, V)                                                                              \
  router_wgrad_kernel<TX, EM, V><<<grid, 256, 0, s>>>(ds, static_cast<const TX*>(x), T, E, d, splits, \
                                                      part, dW, db)
#define MOE_RWG_V(TX, EM)           \
  if (vec == 4) MOE_RWG(TX, EM, 4); \
  else MOE_RWG(TX, EM, 1)
#define MOE_RWG_E(TX)             \
  if (E <= 8) {                   \
    MOE_RWG_V(TX, 8);             \
  } else {                        \
    MOE_RWG_V(TX, 16);            \
  }
  if (x_bf16) {
    MOE_RWG_E(uint16_t);
  } else {
    MOE_RWG_E(float);
  }
#undef MOE_RWG_E
#undef MOE_RWG_V
#undef MOE_RWG
  if (splits > 1) {
    const int64_t n = static_cast<int64_t>(E) * (d + 1);
    wgrad_reduce_kernel<<<blocks(n, 256), 256, 0, s>>>(part, 1, splits, E, d, d + 1, dW, db, 0);
  }
  return hipGetLastError();
}

hipError_t launch_wgrad(const void* A, bool a_bf16, const void* B, bool b_bf16, const int32_t* b_rows,
                        const int32_t* offsets, int groups, int M, int N, float* C, float* dbias,
                        bool accumulate, int splits, float* part, hipStream_t s) {
  const int NB = dbias != nullptr ? N + 1 : N;
  if (splits < 1 || (splits > 1 && part == nullptr)) return hipErrorInvalidValue;
  dim3 grid(blocks(NB, 64), blocks(M, 64), groups * splits);
  const int acc = accumulate ? 1 : 0;
#define MOE_WGRAD(TA, TB)                                                                        \
  wgrad_kernel<TA, TB><<<grid, 256, 0, s>>>(static_cast<const TA*>(A), static_cast<const TB*>(B), \
                                            b_rows, offsets, M, N, splits, C, dbias, acc, part)
  if (a_bf16 && b_bf16) MOE_WGRAD(uint16_t, uint16_t);
  else if (!a_bf16 && b_bf16) MOE_WGRAD(float, uint16_t);
  else if (a_bf16 && !b_bf16) MOE_WGRAD(uint16_t, float);
  else MOE_WGRAD(float, float);
#undef MOE_WGRAD
  if (splits > 1) {
    const int64_t n = static_cast<int64_t>(groups) * M * NB;
    wgrad_reduce_kernel<<<blocks(n, 256), 256, 0, s>>>(part, groups, splits, M, N, NB, C, dbias, acc);
  }
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t s) {
  pad_offsets_kernel<<<1, 1024, 0, s>>>(offsets, E, poff);
  return hipGetLastError();
}

hipError_t launch_padded_transpose(const void* src, const int32_t* row_idx, const int32_t* offsets,
                                   const int32_t* poff, int E, int Cc, int64_t max_padded, int ld,
                                   bool bf16, void* dst, float* colsum_part, hipStream_t s) {
  if (max_padded <= 0) return hipSuccess;
  if (colsum_part != nullptr && !bf16) return hipErrorInvalidValue;
  dim3 grid(blocks(Cc, 64), blocks(max_padded, 64));
  if (bf16)
    padded_transpose_bf16_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), row_idx, offsets,
                                                      poff, E, Cc, ld, static_cast<uint16_t*>(dst),
                                                      colsum_part);
  else
    padded_transpose_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(src), row_idx, offsets,
                                                        poff, E, Cc, ld, static_cast<float*>(dst));
  return hipGetLastError();
}

hipError_t launch_seg_colsum(const float* part, const int32_t* poff, int E, int Cc, float* out,
                             hipStream_t s) {
  seg_colsum_kernel<<<blocks(static_cast<int64_t>(E) * Cc, 256), 256, 0, s>>>(part, poff, E, Cc, out);
  return hipGetLastError();
}


hipError_t launch_zero_empty(const int32_t* offsets, int E, int64_t MN, float* C, hipStream_t s) {
  // blocks of experts with rows exit at once, but each still has to be
  // dispatched: about 32K blocks in all (a million took 110 us)
  int64_t bx = (MN + 256 * 64 - 1) / (256 * 64);
  const int64_t cap = E < 32768 ? 32768 / E : 1;
  if (bx > cap) bx = cap;
  if (bx < 1) bx = 1;
  dim3 grid(static_cast<unsigned>(bx), E);
  zero_empty_kernel<<<grid, 256, 0, s>>>(offsets, MN, C);
  return hipGetLastError();
}

hipError_t launch_range(int32_t* o, int32_t n, hipStream_t s) {
  range_kernel<<<1, 64, 0, s>>>(o, n);
  return hipGetLastError();
}

}  // namespace moe
