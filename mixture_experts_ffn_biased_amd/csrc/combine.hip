// Stage 5: gate-weighted combine, y[t] = Z[t] + sum_j gates[t][j] * O[inv[t*k+j]]
// (+ R[t], the block input, in the pre-norm block form).  Z, O and R are in
// the layer dtype; the sum is accumulated in fp32, R added last.
//
// "Sparse MoE FFN" (DeepSeek-V3), eq. 12 and "Packed forward": the routed
// outputs are scaled by their gates and summed, the shared output is added
// unweighted, and every token receives all k routed outputs (no dropping).
// Instead of a scatter-add into a zero buffer, each token reads its k rows
// through the inverse permutation and sums them in a fixed order with fp32
// accumulation: no atomics, bitwise deterministic.
#include "common.hpp"
#include "plan.hpp"

#include <type_traits>

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte chunk with the non-temporal hint: O, Z and R are each read once
// here, so their lines need not displace anything in the caches.
__device__ __forceinline__ uint4 load_once(const uint16_t *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Widens 8 bf16 values (one 16-byte chunk) into acc += g * x, or acc = x.
__device__ __forceinline__ void fma8(float (&acc)[8], float g, const uint4 &o) {
  const uint32_t w[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(g, bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu)), acc[2 * i]);
    acc[2 * i + 1] = fmaf(g, bf16_to_f32(static_cast<uint16_t>(w[i] >> 16)), acc[2 * i + 1]);
  }
}

// One thread per 16-byte chunk of a token row: block (t, y) covers chunks
// y * kCombineThreads .. of token t, so every thread issues all its loads
// (Z, the k rows of O, R) before its first wait and no thread idles in a
// partial last pass over the row.
constexpr int kCombineThreads = 128;

// KB: the layer's k when it is one of the common values (every load of a
// chunk then goes out before the first wait); 0 for any other k, which runs
// in batches of 8.  HZ / HR: Z / R present.  The sum order is the same in
// every case: Z, then j = 0 .. k-1, then R.
template <int KB, bool HZ, bool HR>
__global__ __launch_bounds__(kCombineThreads) void combine_bf16(const uint16_t *__restrict__ O,
                                                                const uint16_t *__restrict__ Z,
                                                                const int32_t *__restrict__ inv,
                                                                const float *__restrict__ gates,
                                                                int d, int k, const uint16_t *__restrict__ R,
                                                                uint16_t *__restrict__ y) {
  const int64_t t = blockIdx.x;
  const int nchunk = d / 8;
  __shared__ int pos[kMaxTopK];
  __shared__ float gw[kMaxTopK];
  if (static_cast<int>(threadIdx.x) < k) {
    pos[threadIdx.x] = inv[t * k + threadIdx.x];
    gw[threadIdx.x] = gates[t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = static_cast<int>(blockIdx.y) * kCombineThreads + static_cast<int>(threadIdx.x);
  if (c >= nchunk) return;
  constexpr int NB = KB > 0 ? KB : 8;  // rows loaded together
  const int64_t col = static_cast<int64_t>(c) * 8;
  uint4 z = {0u, 0u, 0u, 0u}, r = {0u, 0u, 0u, 0u};
  if (HZ) z = load_once(Z + t * d + col);
  if (HR) r = load_once(R + t * d + col);
  float acc[8];
  {
    const uint32_t zw[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = bf16_to_f32(static_cast<uint16_t>(zw[i] & 0xffffu));
      acc[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(zw[i] >> 16));
    }
  }
  const int kk = KB > 0 ? KB : k;
  for (int j0 = 0; j0 < kk; j0 += NB) {
    uint4 o[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (KB > 0 || j0 + i < kk) o[i] = load_once(O + static_cast<int64_t>(pos[j0 + i]) * d + col);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (KB > 0 || j0 + i < kk) fma8(acc, gw[j0 + i], o[i]);
  }
  if (HR) {  // the block's residual, added last
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(static_cast<uint16_t>(rw[i] & 0xffffu));
      acc[2 * i + 1] += bf16_to_f32(static_cast<uint16_t>(rw[i] >> 16));
    }
  }
  uint4 out;
  out.x = pack_bf16x2(acc[0], acc[1]);
  out.y = pack_bf16x2(acc[2], acc[3]);
  out.z = pack_bf16x2(acc[4], acc[5]);
  out.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4 *>(y + t * d + col) = out;
}

__global__ __launch_bounds__(256) void combine_f32(const float *__restrict__ O,
                                                   const float *__restrict__ Z,
                                                   const int32_t *__restrict__ inv,
                                                   const float *__restrict__ gates, int d,
                                                   int k, const float *__restrict__ R, float *__restrict__ y) {
  const int64_t t = blockIdx.x;
  __shared__ int pos[kMaxTopK];
  __shared__ float gw[kMaxTopK];
  if (static_cast<int>(threadIdx.x) < k) {
    pos[threadIdx.x] = inv[t * k + threadIdx.x];
    gw[threadIdx.x] = gates[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d / 4; c += 256) {
    float4 acc = Z ? *reinterpret_cast<const float4 *>(Z + t * d + c * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 o = *reinterpret_cast<const float4 *>(O + static_cast<int64_t>(pos[j]) * d + c * 4);
      const float g = gw[j];
      acc.x = fmaf(g, o.x, acc.x);
      acc.y = fmaf(g, o.y, acc.y);
      acc.z = fmaf(g, o.z, acc.z);
      acc.w = fmaf(g, o.w, acc.w);
    }
    if (R) {  // the block's residual, added last
      const float4 r = *reinterpret_cast<const float4 *>(R + t * d + c * 4);
      acc.x += r.x;
      acc.y += r.y;
      acc.z += r.z;
      acc.w += r.w;
    }
    *reinterpret_cast<float4 *>(y + t * d + c * 4) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const Plan &p, const float *gates, const void *residual, void *y, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  const void *Z = c.F_shared > 0 ? p.Z : nullptr;
  const dim3 grid(static_cast<unsigned>(c.T));
  if (c.dtype == MOE_BF16) {
    const bool hz = Z != nullptr, hr = residual != nullptr;
    auto pick = [&](auto kb) {
      constexpr int KB = decltype(kb)::value;
      return hz ? (hr ? combine_bf16<KB, true, true> : combine_bf16<KB, true, false>)
                : (hr ? combine_bf16<KB, false, true> : combine_bf16<KB, false, false>);
    };
    auto kern = pick(std::integral_constant<int, 0>{});
    switch (c.k) {
      case 1: kern = pick(std::integral_constant<int, 1>{}); break;
      case 2: kern = pick(std::integral_constant<int, 2>{}); break;
      case 4: kern = pick(std::integral_constant<int, 4>{}); break;
      case 6: kern = pick(std::integral_constant<int, 6>{}); break;
      case 8: kern = pick(std::integral_constant<int, 8>{}); break;
      default: break;
    }
    const unsigned ny = static_cast<unsigned>((c.d / 8 + kCombineThreads - 1) / kCombineThreads);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(c.T), ny), dim3(kCombineThreads), 0, s,
                       static_cast<const uint16_t *>(p.O),
                       static_cast<const uint16_t *>(Z), p.inv, gates, c.d, c.k,
                       static_cast<const uint16_t *>(residual), static_cast<uint16_t *>(y));
  } else
    hipLaunchKernelGGL(combine_f32, grid, dim3(256), 0, s, static_cast<const float *>(p.O),
                       static_cast<const float *>(Z), p.inv, gates, c.d, c.k,
                       static_cast<const float *>(residual), static_cast<float *>(y));
  return hipGetLastError();
}

}  // namespace moe
