// Pre-norm of the MoE block: out[t] = h[t] / sqrt(mean_j h[t][j]^2 + eps) * g.
//
// "Lesson 2 -- From the Dense FFN to a Layer of Experts", section 2: the MoE
// layer replaces the FFN inside the same pre-norm residual block, H' = H~ +
// MoE(Norm(H~)); "Mixture of experts and architecture families": the norm is
// RMSNorm (no mean-centering).  The normalised rows are written once in the
// layer dtype and read by both the router and the gate/up GEMM, whose tiles
// are loaded from memory straight into LDS.
//
// One block of 256 threads per row; the sum of squares is accumulated in a
// fixed order (per thread, then a wave butterfly, then the four waves in
// order), so results are bitwise reproducible.
#include "common.hpp"
#include "plan.hpp"

namespace moe {
namespace {

__device__ __forceinline__ float block_sum_256(float v, float *red) {
  v = wave_sum_f32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

// bf16 rows, d % 8 == 0 and d <= 256 * 8 * 4.
__global__ __launch_bounds__(256) void rmsnorm_bf16(const uint16_t *__restrict__ h, const uint16_t *__restrict__ g,
                                                    float eps, int d, uint16_t *__restrict__ out) {
  __shared__ float red[4];
  constexpr int MAXC = 4;  // 16-byte chunks a thread holds
  const int64_t t = blockIdx.x;
  const int nchunk = d / 8;
  float x[MAXC][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nchunk) {
      const uint4 v = *reinterpret_cast<const uint4 *>(h + t * d + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[i][2 * j] = bf16_to_f32(static_cast<uint16_t>(w[j] & 0xffffu));
        x[i][2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(w[j] >> 16));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(x[i][j], x[i][j], ss);
    }
  }
  const float inv = 1.0f / sqrtf(block_sum_256(ss, red) / static_cast<float>(d) + eps);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nchunk) {
      const uint4 gv = *reinterpret_cast<const uint4 *>(g + c * 8);
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = pack_bf16x2(x[i][2 * j] * inv * bf16_to_f32(static_cast<uint16_t>(gw[j] & 0xffffu)),
                           x[i][2 * j + 1] * inv * bf16_to_f32(static_cast<uint16_t>(gw[j] >> 16)));
      *reinterpret_cast<uint4 *>(out + t * d + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// fp32 rows, d % 4 == 0 and d <= 256 * 4 * 8.
__global__ __launch_bounds__(256) void rmsnorm_f32(const float *__restrict__ h, const float *__restrict__ g,
                                                   float eps, int d, float *__restrict__ out) {
  __shared__ float red[4];
  constexpr int MAXC = 8;
  const int64_t t = blockIdx.x;
  const int nchunk = d / 4;
  float4 x[MAXC];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nchunk) {
      x[i] = *reinterpret_cast<const float4 *>(h + t * d + c * 4);
      ss = fmaf(x[i].x, x[i].x, ss);
      ss = fmaf(x[i].y, x[i].y, ss);
      ss = fmaf(x[i].z, x[i].z, ss);
      ss = fmaf(x[i].w, x[i].w, ss);
    }
  }
  const float inv = 1.0f / sqrtf(block_sum_256(ss, red) / static_cast<float>(d) + eps);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nchunk) {
      const float4 gv = *reinterpret_cast<const float4 *>(g + c * 4);
      *reinterpret_cast<float4 *>(out + t * d + c * 4) =
          make_float4(x[i].x * inv * gv.x, x[i].y * inv * gv.y, x[i].z * inv * gv.z, x[i].w * inv * gv.w);
    }
  }
}

}  // namespace

int rmsnorm_max_d() { return 8192; }

hipError_t launch_rmsnorm(const void *h, const void *g, float eps, int64_t T, int d, int dtype, void *out,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(T));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(rmsnorm_bf16, grid, dim3(256), 0, s, static_cast<const uint16_t *>(h),
                       static_cast<const uint16_t *>(g), eps, d, static_cast<uint16_t *>(out));
  else
    hipLaunchKernelGGL(rmsnorm_f32, grid, dim3(256), 0, s, static_cast<const float *>(h),
                       static_cast<const float *>(g), eps, d, static_cast<float *>(out));
  return hipGetLastError();
}

}  // namespace moe
