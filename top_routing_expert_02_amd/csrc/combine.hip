// Combine: y_t = sum_{i in S_t} p~_{t,i} E_i(x_t) over the kept assignments
// (page "MoE 模型原理：路由、专家负载、容量、通信与推理成本", wrblog.cn, §2.2 output
// formula; §5: expert outputs go back in the original token order and are
// merged by the routing weights).
//
// Gather form: a thread owns VEC consecutive columns of one token, reads the
// token's k rows of y_perm (bf16 for bf16 layers, fp32 for fp32 layers),
// accumulates j = 0..k-1 in fp32 in that fixed order and rounds once. No
// atomics, so the result is deterministic; a token with every assignment
// dropped writes exact zeros. When the second GEMM ran some tiles as K parts
// (device words nsplit: parts p, first split row, split row count), each
// row from the first split row on is the sum of its p partial rows (bf16),
// in part order, formed before the gate multiplies it.
#include "moe_internal.h"

namespace moe {

// the VEC columns c.. of row `ro` (element offset) as fp32; rows bf16 or fp32
template <int VEC>
__device__ __forceinline__ void load_row(const void* __restrict__ yp, bool bf16, int64_t ro,
                                         float (&q)[VEC]) {
  if (bf16) {
    const uint16_t* src = static_cast<const uint16_t*>(yp) + ro;
    if constexpr (VEC % 8 == 0) {
      uint4 u[VEC / 8];
#pragma unroll
      for (int h = 0; h < VEC / 8; ++h) u[h] = reinterpret_cast<const uint4*>(src)[h];
#pragma unroll
      for (int h = 0; h < VEC / 8; ++h) {
        const uint32_t w[4] = {u[h].x, u[h].y, u[h].z, u[h].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          q[8 * h + 2 * i] = __uint_as_float(w[i] << 16);
          q[8 * h + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) q[v] = bf16_to_f32(src[v]);
    }
    return;
  }
  const float* src = static_cast<const float*>(yp) + ro;
  if constexpr (VEC % 4 == 0) {
#pragma unroll
    for (int v = 0; v < VEC; v += 4) {
      const float4 a = *reinterpret_cast<const float4*>(src + v);
      q[v] = a.x;
      q[v + 1] = a.y;
      q[v + 2] = a.z;
      q[v + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = src[v];
  }
}

// the same columns of a row split in K: part 0 from y_perm row r, part
// j >= 1 from y_perm2 row (j - 1) trows + r - r_tail (bf16 rows), added in
// fp32 in order j = 0, 1, ..
template <int VEC>
__device__ __forceinline__ void load_parts(const void* __restrict__ yp, const void* __restrict__ y2,
                                           int p, int64_t r, int64_t r_tail, int64_t trows, int d, int c,
                                           float (&q)[VEC]) {
  load_row<VEC>(yp, true, r * d + c, q);
  for (int j = 1; j < p; ++j) {
    float b[VEC];
    load_row<VEC>(y2, true, ((j - 1) * trows + r - r_tail) * d + c, b);
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] += b[v];
  }
}

// y_perm rows bf16 (rows_bf16) or fp32; with y_perm2, nsplit = {p, r_tail,
// trows}: rows r >= r_tail are sums of p bf16 parts when p > 1
template <int VEC, bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm, int rows_bf16,
                                                      const void* __restrict__ y_perm2,
                                                      const int32_t* __restrict__ nsplit,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gates, int64_t T,
                                                      int k, int d, void* __restrict__ y) {
  const int chunks = d / VEC;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= T * chunks) return;
  const int64_t t = gid / chunks;
  const int c = static_cast<int>(gid - t * chunks) * VEC;
  int p = 1, r_tail = 0, trows = 0;
  if (y_perm2 != nullptr) {
    p = nsplit[0];
    r_tail = nsplit[1];
    trows = nsplit[2];
  }
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int row = row_of[t * k + j];
    if (row < 0) continue;
    const float g = gates[t * k + j];
    float q[VEC];
    if (p > 1 && row >= r_tail)
      load_parts<VEC>(y_perm, y_perm2, p, row, r_tail, trows, d, c, q);
    else
      load_row<VEC>(y_perm, rows_bf16 != 0, static_cast<int64_t>(row) * d + c, q);
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = fmaf(g, q[v], acc[v]);
  }
  if constexpr (BF16) {
    static_assert(VEC % 8 == 0, "bf16 output stores 16-byte groups of 8 columns");
#pragma unroll
    for (int h = 0; h < VEC / 8; ++h) {
      const float* a = acc + 8 * h;
      uint4 o;
      o.x = f32_to_bf16(a[0]) | (static_cast<uint32_t>(f32_to_bf16(a[1])) << 16);
      o.y = f32_to_bf16(a[2]) | (static_cast<uint32_t>(f32_to_bf16(a[3])) << 16);
      o.z = f32_to_bf16(a[4]) | (static_cast<uint32_t>(f32_to_bf16(a[5])) << 16);
      o.w = f32_to_bf16(a[6]) | (static_cast<uint32_t>(f32_to_bf16(a[7])) << 16);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + t * d + c)[h] = o;
    }
  } else {
    float* dst = static_cast<float*>(y) + t * d + c;
#pragma unroll
    for (int v = 0; v < VEC; ++v) dst[v] = acc[v];
  }
}

hipError_t launch_combine(const void* y_perm, bool yperm_bf16, const void* y_perm2,
                          const int32_t* nsplit, const int32_t* row_of, const float* gates, int64_t T,
                          int k, int d, bool out_bf16, void* y, hipStream_t s) {
  if (nsplit == nullptr) y_perm2 = nullptr;
  const int rb = yperm_bf16 ? 1 : 0;
  if (out_bf16) {
    // d is a multiple of 64: 16 columns per thread, two 16-byte loads per
    // row and k rows in flight
    const int64_t n = T * (d / 16);
    klaunch(combine_kernel<16, true>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
            y_perm, rb, y_perm2, nsplit, row_of, gates, T, k, d, y);
  } else if (d % 4 == 0) {
    const int64_t n = T * (d / 4);
    klaunch(combine_kernel<4, false>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
            y_perm, rb, y_perm2, nsplit, row_of, gates, T, k, d, y);
  } else {
    const int64_t n = T * d;
    klaunch(combine_kernel<1, false>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
            y_perm, rb, y_perm2, nsplit, row_of, gates, T, k, d, y);
  }
  return hipGetLastError();
}

}  // namespace moe
