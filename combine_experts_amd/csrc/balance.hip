// Load-balance statistics of one routed batch and the aux-loss-free bias step.
//
// EP-in-LLMs article, "Static Capacity Factors and Token Dropping": the auxiliary loss
// L_aux = alpha * E * sum_i f_i * P_i, with f_i the share of dispatched (token, expert) pairs that
// went to expert i and P_i the mean router probability of expert i. The same article ("Modern
// Dropless Dynamic Dispatch") and "Chapter 10: MoE parallelism" (section 4, load balancing) name the
// aux-loss-free alternative: a per-expert bias on the routing scores, moved against the load.
// The bias step used here is b_i += gamma * sign(mean load - load_i).
//
// One block does the whole reduction: its inputs are E counts and ceil(T/64) x E per-block sums
// of router probabilities that the router wrote, a few hundred KB at most. Every sum runs in a
// fixed order, so the outputs do not depend on thread scheduling.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kSplit = 4;  // threads per expert summing disjoint runs of the router's block partials

__global__ void __launch_bounds__(kThreads) load_balance_kernel(const int32_t* __restrict__ counts,
                                                                const float* __restrict__ partials, int n_part,
                                                                int T, int E, int k, float alpha,
                                                                float* __restrict__ stats, float gamma,
                                                                float* __restrict__ sbias) {
  __shared__ long long s_sum[kThreads / MOE_WAVE];
  __shared__ int s_max[kThreads / MOE_WAVE];
  __shared__ float s_part[kSplit][256];
  __shared__ float s_term[kThreads];
  const int tid = threadIdx.x, lane = tid % MOE_WAVE, wave = tid / MOE_WAVE;

  // total and largest load (integers: any order gives the same result)
  long long csum = 0;
  int cmax = 0;
  for (int e = tid; e < E; e += kThreads) {
    const int c = counts[e];
    csum += c;
    cmax = max(cmax, c);
  }
  for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) {
    csum += __shfl_xor(csum, off, MOE_WAVE);
    cmax = max(cmax, __shfl_xor(cmax, off, MOE_WAVE));
  }
  if (lane == 0) {
    s_sum[wave] = csum;
    s_max[wave] = cmax;
  }
  __syncthreads();
  csum = 0;
  cmax = 0;
  for (int w = 0; w < kThreads / MOE_WAVE; ++w) {
    csum += s_sum[w];
    cmax = max(cmax, s_max[w]);
  }

  const double n_pairs = (double)T * (double)k;
  float term = 0.f;  // this thread's share of sum_i f_i * P_i, in ascending expert order
  // experts in chunks of 256; each expert's partials are summed by kSplit threads over disjoint
  // runs, and the runs are then added in run order
  const int run = (n_part + kSplit - 1) / kSplit;
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int el = tid % 256, part = tid / 256;
    const int e = e0 + el;
    float acc = 0.f;
    if (e < E) {
      const int b0 = part * run, b1 = min(n_part, b0 + run);
      for (int b = b0; b < b1; ++b) acc += partials[(size_t)b * E + e];
    }
    s_part[part][el] = acc;
    __syncthreads();
    if (part == 0 && e < E) {
      float psum = s_part[0][el];
      for (int p = 1; p < kSplit; ++p) psum += s_part[p][el];
      const int c = counts[e];
      const float f = n_pairs > 0 ? (float)((double)c / n_pairs) : 0.f;
      const float P = T > 0 ? psum / (float)T : 0.f;
      stats[e] = f;
      stats[E + e] = P;
      term += f * P;
      if (sbias != nullptr) {
        // sign(mean - c) = sign(sum - E*c), compared exactly in integers
        const long long diff = csum - (long long)E * c;
        const float step = diff > 0 ? gamma : (diff < 0 ? -gamma : 0.f);
        sbias[e] = sbias[e] + step;
      }
    }
    __syncthreads();
  }
  // sum of the per-thread terms: a fixed tree over thread index
  s_term[tid] = term;
  __syncthreads();
  for (int w = kThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) s_term[tid] += s_term[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    stats[2 * E] = alpha * (float)E * s_term[0];
    stats[2 * E + 1] = csum > 0 ? (float)((double)cmax * E / (double)csum) : 0.f;
  }
}

}  // namespace

hipError_t launch_load_balance(const int32_t* expert_counts, const float* prob_partials, int32_t n_partials,
                               int32_t T, int32_t E, int32_t k, float alpha, float* stats, float gamma,
                               float* select_bias, hipStream_t s) {
  hipLaunchKernelGGL(load_balance_kernel, dim3(1), dim3(kThreads), 0, s, expert_counts, prob_partials, n_partials, T,
                     E, k, alpha, stats, gamma, select_bias);
  return hipGetLastError();
}

}  // namespace moe
