// The whole layer of a small fp32 configuration in one kernel, one
// workgroup per token: its router logits, its selection (select.hpp), its k
// routed SwiGLU experts and the shared one, and their gate-weighted sum.
//
// Per token this is the definition itself ("Sparse MoE FFN" (DeepSeek-V3),
// "How it works", eq. 12 and the expert equation; "Mixture of Experts and
// Hybrid Architectures", "The router in code"): y = Z + sum_j g_j E_j(u) with
// E(u) = W2 (SiLU(W1 u) * (W3 u)), every product in fp32 FMA, the sum in the
// combine's order (the shared expert's output first, then j = 0 .. k-1), and
// the block's residual added last.  Small layers are bound by the number of
// dependent launches, not by bytes or FLOPs: one launch replaces the seven of
// the general path (router, three permutation kernels, two grouped GEMMs,
// combine), and each token reads its experts' few KiB of weights from L2
// instead of the experts running as grouped GEMMs over permuted rows.  The
// permutation is not needed for the output; moe_route_debug still runs it.
#include "common.hpp"
#include "plan.hpp"
#include "select.hpp"

namespace moe {
namespace {

// row . x over n values (n % 4 == 0), row from global memory 16 bytes at a
// time, x from LDS, fp32 FMA in index order.
__device__ __forceinline__ float dot_row(const float *__restrict__ row, const float *x, int n) {
  float acc = 0.f;
  for (int j = 0; j < n; j += 4) {
    const float4 w = *reinterpret_cast<const float4 *>(row + j);
    acc = fmaf(x[j], w.x, acc);
    acc = fmaf(x[j + 1], w.y, acc);
    acc = fmaf(x[j + 2], w.z, acc);
    acc = fmaf(x[j + 3], w.w, acc);
  }
  return acc;
}

// LDS: the token's row (d), its logits (E), one expert's hidden row (hmax).
// A thread owns output columns tid + 256 q, q < kSmallMaxD / 256.
template <bool HS, bool HR>
__global__ __launch_bounds__(256) void small_layer_f32(const float *__restrict__ u, const float *__restrict__ Wr,
                                                       SelArgs sel, const float *__restrict__ W1,
                                                       const float *__restrict__ W3, const float *__restrict__ W2,
                                                       const float *__restrict__ W1s, const float *__restrict__ W3s,
                                                       const float *__restrict__ W2s, int d, int F, int Fs, int hmax,
                                                       const float *__restrict__ R, float *__restrict__ y,
                                                       int32_t *__restrict__ topk_idx, float *__restrict__ gates) {
  extern __shared__ float sm[];
  float *x = sm;
  float *lg = x + d;
  float *h = lg + kMaxExperts;
  __shared__ int sel_idx[kMaxTopK];
  __shared__ float sel_g[kMaxTopK];
  constexpr int Q = kSmallMaxD / 256;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = sel.k;

  for (int j = tid; j < d; j += 256) x[j] = u[t * d + j];
  __syncthreads();
  for (int e = tid; e < sel.E; e += 256) lg[e] = dot_row(Wr + static_cast<int64_t>(e) * d, x, d);
  __syncthreads();
  if (tid < 64) select_token(lg, sel, sel_idx, sel_g);
  __syncthreads();
  if (tid < k) {
    topk_idx[t * k + tid] = sel_idx[tid];
    gates[t * k + tid] = sel_g[tid];
  }

  float acc[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) acc[q] = 0.f;
  // One expert: h = SiLU(W1 x) * (W3 x), then its output columns; the shared
  // expert's output starts the sum, a routed one is added with its gate.
  auto expert = [&](const float *w1, const float *w3, const float *w2, int Fe, bool first, float g) {
    for (int f = tid; f < Fe; f += 256) {
      const float a1 = dot_row(w1 + static_cast<int64_t>(f) * d, x, d);
      const float a3 = dot_row(w3 + static_cast<int64_t>(f) * d, x, d);
      h[f] = silu(a1) * a3;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = tid + 256 * q;
      if (i < d) {
        const float o = dot_row(w2 + static_cast<int64_t>(i) * Fe, h, Fe);
        acc[q] = first ? o : fmaf(g, o, acc[q]);
      }
    }
    __syncthreads();  // h is rewritten by the next expert
  };
  if (HS) expert(W1s, W3s, W2s, Fs, true, 1.f);
  for (int j = 0; j < k; ++j) {
    const int64_t e = sel_idx[j];
    const int64_t es = static_cast<int64_t>(F) * d;
    expert(W1 + e * es, W3 + e * es, W2 + e * es, F, false, sel_g[j]);
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = tid + 256 * q;
    if (i < d) y[t * d + i] = HR ? acc[q] + R[t * d + i] : acc[q];
  }
}

}  // namespace

bool small_layer_fits(const moe_cfg &c, int kind) {
  return c.dtype == MOE_F32 && kind == MOE_EXPERT_SWIGLU && c.T * c.k <= kSmallMaxSlots && c.d <= kSmallMaxD &&
         c.F <= kSmallMaxF && c.F_shared <= kSmallMaxF && c.E <= kMaxExperts;
}

hipError_t launch_small_layer(const Plan &p, const void *u, const void *W_router, const float *bias,
                              const Experts &x, const void *residual, void *y, int32_t *topk_idx, float *gates,
                              hipStream_t s) {
  const moe_cfg &c = p.cfg;
  SelArgs sel{c.E, c.k, c.score_fn, c.n_groups, c.topk_groups, c.route_scale, bias};
  const int hmax = c.F > c.F_shared ? c.F : c.F_shared;
  const size_t lds = sizeof(float) * (c.d + kMaxExperts + hmax);
  const bool hs = c.F_shared > 0, hr = residual != nullptr;
  auto kern = hs ? (hr ? small_layer_f32<true, true> : small_layer_f32<true, false>)
                 : (hr ? small_layer_f32<false, true> : small_layer_f32<false, false>);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(c.T)), dim3(256), lds, s, static_cast<const float *>(u),
                     static_cast<const float *>(W_router), sel, static_cast<const float *>(x.W1),
                     static_cast<const float *>(x.W3), static_cast<const float *>(x.W2),
                     static_cast<const float *>(x.W1s), static_cast<const float *>(x.W3s),
                     static_cast<const float *>(x.W2s), c.d, c.F, c.F_shared, hmax,
                     static_cast<const float *>(residual), static_cast<float *>(y), topk_idx, gates);
  return hipGetLastError();
}

}  // namespace moe
