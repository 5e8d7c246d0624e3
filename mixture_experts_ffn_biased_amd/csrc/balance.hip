// One step of the auxiliary-loss-free balance update, on the GPU.
//
// "Mixture of Experts and Hybrid Architectures", "Aux-loss-free balance loop":
// the per-expert bias starts at zero, the target usage is tokens * top_k /
// experts, the experts that fired more often than the target in the last
// batch have their bias lowered by gamma, those that fired less raised by
// gamma, and the entropy of the usage rises toward ln(E) as the loop runs.
// "Sparse MoE FFN" (DeepSeek-V3), "How it works": the bias only moves
// selection (the gates never read it) and its update happens outside the
// forward pass.
//
// One block: an LDS histogram of the chosen experts (integer atomics, so the
// counts are exact), the update compared in integers (count * E against
// T * k), and the entropy summed in fp64 in expert order (deterministic).
#include "common.hpp"
#include "plan.hpp"  // kMaxExperts

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void balance_update(const int32_t *__restrict__ idx, int64_t S, int E,
                                                       float gamma, float *__restrict__ bias,
                                                       int32_t *__restrict__ counts,
                                                       float *__restrict__ entropy) {
  __shared__ int cnt[kMaxExperts];
  __shared__ double term[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int64_t s = tid; s < S; s += blockDim.x) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = cnt[e];
    const int64_t ce = static_cast<int64_t>(c) * E;  // c > S / E  <=>  c * E > S
    if (ce > S)
      bias[e] -= gamma;
    else if (ce < S)
      bias[e] += gamma;
    if (counts) counts[e] = c;
    const double p = S > 0 ? static_cast<double>(c) / static_cast<double>(S) : 0.0;
    term[e] = p > 0.0 ? -p * log(p) : 0.0;
  }
  __syncthreads();
  if (tid == 0 && entropy) {
    double h = 0.0;
    for (int e = 0; e < E; ++e) h += term[e];
    entropy[0] = static_cast<float>(h);
  }
}

}  // namespace

hipError_t launch_balance_update(const int32_t *topk_idx, int64_t S, int E, float gamma, float *bias,
                                 int32_t *counts, float *entropy, hipStream_t s) {
  hipLaunchKernelGGL(balance_update, dim3(1), dim3(1024), 0, s, topk_idx, S, E, gamma, bias, counts, entropy);
  return hipGetLastError();
}

}  // namespace moe
