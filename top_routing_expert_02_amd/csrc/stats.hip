// Load statistics of one routing step, from the counts the dispatch returns.
//
// Page "MoE 模型原理：路由、专家负载、容量、通信与推理成本" (wrblog.cn) §3.3 asks a
// production system to log the tokens each expert receives, the tokens each
// expert drops and the max/mean load; §13 adds tokens per expert, the
// overflow ratio and the padding ratio; §3.2 defines the load-balance loss
// L_aux = alpha E sum_i f_i pbar_i. The ai-master.cc EP answer 001 (follow-up
// 2) judges balance by the entropy of the expert activation distribution and
// the variance of the tokens each expert actually processes.
//
// One block of 256 threads; thread t owns experts t, t + 256, ...; every sum
// is a fixed-order tree over the threads, so results are bit-reproducible.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kStatThreads = 256;

// sum over the block in a fixed order (every thread gets the total)
template <typename V>
__device__ V block_sum(V v, V* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int off = kStatThreads / 2; off >= 1; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const V total = red[0];
  __syncthreads();
  return total;
}

__device__ int block_max(int v, int* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int off = kStatThreads / 2; off >= 1; off >>= 1) {
    if (tid < off) red[tid] = max(red[tid], red[tid + off]);
    __syncthreads();
  }
  const int m = red[0];
  __syncthreads();
  return m;
}

}  // namespace

__global__ __launch_bounds__(kStatThreads) void load_stats_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const float* __restrict__ prob_sum, int E, int C, int64_t T, int k, double alpha,
    int32_t* __restrict__ kept_out, int32_t* __restrict__ dropped_out, double* __restrict__ stats) {
  __shared__ double dred[kStatThreads];
  __shared__ long long ired[kStatThreads];
  __shared__ int mred[kStatThreads];
  const int tid = threadIdx.x;
  long long csum = 0, ksum = 0;
  int cmax = 0;
  for (int e = tid; e < E; e += kStatThreads) {
    const int c = counts[e];
    const int kp = offsets[e + 1] - offsets[e];
    const int dr = c > kp ? c - kp : 0;
    if (kept_out != nullptr) kept_out[e] = kp;
    if (dropped_out != nullptr) dropped_out[e] = dr;
    csum += c;
    ksum += kp;
    cmax = max(cmax, c);
  }
  const long long total = block_sum<long long>(csum, ired);
  const long long rows = block_sum<long long>(ksum, ired);
  const int maxc = block_max(cmax, mred);
  const double kept_mean = static_cast<double>(rows) / E;
  double ent = 0.0, var = 0.0, aux = 0.0;
  for (int e = tid; e < E; e += kStatThreads) {
    const int c = counts[e];
    const int kp = offsets[e + 1] - offsets[e];
    if (c > 0 && total > 0) {
      const double f = static_cast<double>(c) / static_cast<double>(total);
      ent -= f * log(f);
    }
    const double dk = static_cast<double>(kp) - kept_mean;
    var += dk * dk;
    if (prob_sum != nullptr)
      aux += (static_cast<double>(c) / static_cast<double>(T)) * (static_cast<double>(prob_sum[e]) / T);
  }
  ent = block_sum<double>(ent, dred);
  var = block_sum<double>(var, dred);
  aux = block_sum<double>(aux, dred);
  if (tid == 0) {
    const double assigned = static_cast<double>(T) * k;
    const double dropped = assigned - static_cast<double>(rows);
    stats[kStatDropped] = dropped;
    stats[kStatOverflowRatio] = dropped / assigned;
    stats[kStatMaxOverMean] = total > 0 ? static_cast<double>(maxc) * E / static_cast<double>(total) : 0.0;
    stats[kStatPaddingRatio] = rows > 0 ? static_cast<double>(E) * C / static_cast<double>(rows) : 0.0;
    stats[kStatLoadEntropy] = ent;
    stats[kStatKeptVariance] = var / E;
    stats[kStatAuxLoss] = prob_sum != nullptr ? alpha * E * aux : __builtin_nan("");
    stats[kStatKeptRows] = static_cast<double>(rows);
  }
}

hipError_t launch_load_stats(const int32_t* counts, const int32_t* offsets, const float* prob_sum, int E,
                             int C, int64_t T, int k, double alpha, int32_t* kept, int32_t* dropped,
                             double* stats, hipStream_t s) {
  klaunch(load_stats_kernel, dim3(1), dim3(kStatThreads), 0, s, counts, offsets, prob_sum, E, C, T, k, alpha,
          kept, dropped, stats);
  return hipGetLastError();
}

}  // namespace moe
