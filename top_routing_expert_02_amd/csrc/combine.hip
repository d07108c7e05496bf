// Combine: y_t = sum_{i in S_t} p~_{t,i} E_i(x_t) over the kept assignments
// (page "MoE 模型原理：路由、专家负载、容量、通信与推理成本", wrblog.cn, §2.2 output
// formula; §5: expert outputs go back in the original token order and are
// merged by the routing weights).
//
// Gather form: a thread owns VEC consecutive columns of one token, reads the
// token's k rows of y_perm (fp32), accumulates j = 0..k-1 in fp32 in that
// fixed order and rounds once. No atomics, so the result is deterministic; a
// token with every assignment dropped writes exact zeros. After a K-split
// second GEMM, a row is the sum of its two partial rows, formed before the
// gate multiplies it.
#include "moe_internal.h"

namespace moe {

template <int VEC, bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const float* __restrict__ y_perm2,
                                                      const int32_t* __restrict__ nsplit,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gates, int64_t T,
                                                      int k, int d, void* __restrict__ y) {
  const int chunks = d / VEC;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= T * chunks) return;
  const int64_t t = gid / chunks;
  const int c = static_cast<int>(gid - t * chunks) * VEC;
  const float* y2 = (y_perm2 != nullptr && *nsplit == 2) ? y_perm2 : nullptr;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int row = row_of[t * k + j];
    if (row < 0) continue;
    const float g = gates[t * k + j];
    const int64_t ro = static_cast<int64_t>(row) * d + c;
    const float* src = y_perm + ro;
    if constexpr (VEC % 4 == 0) {
#pragma unroll
      for (int v = 0; v < VEC; v += 4) {
        float4 q = *reinterpret_cast<const float4*>(src + v);
        if (y2 != nullptr) {
          const float4 q2 = *reinterpret_cast<const float4*>(y2 + ro + v);
          q.x += q2.x;
          q.y += q2.y;
          q.z += q2.z;
          q.w += q2.w;
        }
        acc[v + 0] = fmaf(g, q.x, acc[v + 0]);
        acc[v + 1] = fmaf(g, q.y, acc[v + 1]);
        acc[v + 2] = fmaf(g, q.z, acc[v + 2]);
        acc[v + 3] = fmaf(g, q.w, acc[v + 3]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = fmaf(g, y2 != nullptr ? src[v] + y2[ro + v] : src[v], acc[v]);
    }
  }
  if constexpr (BF16) {
    static_assert(VEC == 8, "bf16 output uses 8 columns per thread");
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + t * d + c) = o;
  } else {
    float* dst = static_cast<float*>(y) + t * d + c;
#pragma unroll
    for (int v = 0; v < VEC; ++v) dst[v] = acc[v];
  }
}

hipError_t launch_combine(const float* y_perm, const float* y_perm2, const int32_t* nsplit,
                          const int32_t* row_of, const float* gates, int64_t T, int k, int d,
                          bool out_bf16, void* y, hipStream_t s) {
  if (nsplit == nullptr) y_perm2 = nullptr;
  if (out_bf16) {
    const int64_t n = T * (d / 8);
    combine_kernel<8, true><<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(y_perm, y_perm2, nsplit, row_of, gates, T, k, d, y);
  } else if (d % 4 == 0) {
    const int64_t n = T * (d / 4);
    combine_kernel<4, false><<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(y_perm, y_perm2, nsplit, row_of, gates, T, k, d, y);
  } else {
    const int64_t n = T * d;
    combine_kernel<1, false><<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(y_perm, y_perm2, nsplit, row_of, gates, T, k, d, y);
  }
  return hipGetLastError();
}

}  // namespace moe
