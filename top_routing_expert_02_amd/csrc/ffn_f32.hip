// Grouped expert FFN GEMMs for fp32 layers (FFN(x) = W2 sigma(W1 x + b1) + b2,
// page "MoE 模型原理：路由、专家负载、容量、通信与推理成本", wrblog.cn, §1).
//
// The fp32 path exists for small layers that need fp32 results (token rows
// may be gathered through a row index, like the bf16 path); it uses
// vector FMA with 64x64 LDS tiles (each thread 4x4 outputs, strided by 16 so
// that LDS reads are conflict-free). The grid is (N tiles, M tiles of the
// largest possible expert, experts); tiles past an expert's rows exit.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const int32_t* __restrict__ row_idx,
                                                       const float* __restrict__ W,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ out,
                                                       const int32_t* __restrict__ offsets, int N,
                                                       int K, int act) {
  const int e = blockIdx.z;
  const int r0 = offsets[e];
  const int ne = offsets[e + 1] - r0;
  const int m0 = blockIdx.y * 64;
  if (m0 >= ne) return;
  const int n0 = blockIdx.x * 64;
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15;
  const int ty = threadIdx.x >> 4;
  const float* We = W + static_cast<int64_t>(e) * N * K;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + i * 256;
      const int m = idx >> 4;
      const int kk = idx & 15;
      const bool kv = k0 + kk < K;
      float a = 0.f;
      if (m0 + m < ne && kv) {
        const int64_t row = row_idx != nullptr ? row_idx[r0 + m0 + m] : r0 + m0 + m;
        a = A[row * K + k0 + kk];
      }
      As[kk][m] = a;
      Bs[kk][m] = (n0 + m < N && kv) ? We[static_cast<int64_t>(n0 + m) * K + k0 + kk] : 0.f;
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
    if (m >= ne) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= N) continue;
      float v = acc[i][j] + (bias != nullptr ? bias[static_cast<int64_t>(e) * N + n] : 0.f);
      if (act == kActRelu) v = act_relu(v);
      else if (act == kActGeluTanh) v = act_gelu_tanh(v);
      out[static_cast<int64_t>(r0 + m) * N + n] = v;
    }
  }
}

hipError_t launch_gemm_f32(const float* A, const int32_t* row_idx, const float* W, const float* bias,
                           float* out,
                           int act, const int32_t* offsets, int E, int N, int K,
                           int max_rows_per_expert, hipStream_t s) {
  if (max_rows_per_expert <= 0) return hipSuccess;
  dim3 grid((N + 63) / 64, (max_rows_per_expert + 63) / 64, E);
  klaunch(gemm_f32_kernel, grid, 256, 0, s, A, row_idx, W, bias, out, offsets, N, K, act);
  return hipGetLastError();
}

}  // namespace moe
