// Shared device helpers for the gfx950 MoE kernels: bf16 bit handling, vector
// types, the wave64 MFMA fragment types and an order key for top-k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));

// Round to nearest even in one gfx950 v_cvt_pk_bf16_f32 (two values per
// instruction for the packed form).
__device__ __forceinline__ uint16_t f32_to_bf16_hw(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Eight bf16 values times eight bf16 scales: each fp32 product (exact for
// two bf16 values) rounded once to bf16, nearest even.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, uint4 g) {
  const uint32_t a[4] = {v.x, v.y, v.z, v.w};
  const uint32_t b[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_to_f32(static_cast<uint16_t>(a[i])) * bf16_to_f32(static_cast<uint16_t>(b[i]));
    const float hi = bf16_to_f32(static_cast<uint16_t>(a[i] >> 16)) * bf16_to_f32(static_cast<uint16_t>(b[i] >> 16));
    o[i] = pack_bf16x2(lo, hi);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 4 x 4 transpose within each quad of lanes, to bf16.  Lane j = lane & 3
// holds f[b] = rows b = 0..3 of its own column (the four lanes of a quad hold
// four consecutive columns); it returns row (j & 1) * 2 + (j >> 1) of those
// four columns, packed as 4 bf16 (low column first), so that a quad writes
// four whole 8-byte row pieces instead of sixteen 2-byte values.
__device__ __forceinline__ uint2 quad_transpose_bf16(const float (&f)[4], int j) {
  const uint32_t p0 = pack_bf16x2_hw(f[0], f[1]);  // rows 0, 1 of my column
  const uint32_t p1 = pack_bf16x2_hw(f[2], f[3]);  // rows 2, 3
  const bool odd = j & 1;
  // lanes j, j^1: the even one gathers rows 0, 1 of both columns, the odd one
  // rows 2, 3
  const uint32_t got1 = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(odd ? p0 : p1), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  const uint32_t own = odd ? p1 : p0;
  const uint32_t lo = odd ? got1 : own, hi = odd ? own : got1;  // lower, higher column
  const uint32_t r0 = (lo & 0xffffu) | (hi << 16);              // first row of the pair, 2 columns
  const uint32_t r1 = (lo >> 16) | (hi & 0xffff0000u);          // second row
  // lanes j, j^2: swap halves so each lane holds one row of all 4 columns
  const bool upper = j & 2;
  const uint32_t got2 = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(upper ? r0 : r1), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  return upper ? make_uint2(got2, r1) : make_uint2(r0, got2);
}

// Row of the quad block that quad_transpose_bf16 leaves in lane j.
__device__ __forceinline__ int quad_transpose_row(int j) { return (j & 1) * 2 + (j >> 1); }

// SiLU for the bf16 epilogues: x * rcp(1 + 2^(-x log2 e)) on the hardware
// exp2 and reciprocal (about 1 ulp each, well inside the bf16 rounding that
// follows); x -> -inf gives -0, x -> +inf gives x, NaN stays NaN.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// GELU(x) = x Phi(x), Phi the standard normal CDF, through erf (exact form).
__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// Total order used by top-k: larger score first, then lower index; NaN ranks
// below every number; -0 and +0 tie.  The 64-bit key is compared as an
// unsigned integer; 0 is reserved for "no candidate".
__device__ __forceinline__ uint64_t rank_key(float v, int idx) {
  uint32_t k;
  if (v != v) {
    k = 0u;
  } else {
    uint32_t b = __float_as_uint(v + 0.0f);  // -0 -> +0
    k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  return (static_cast<uint64_t>(k) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}

__device__ __forceinline__ int key_index(uint64_t key) {
  return static_cast<int>(~static_cast<uint32_t>(key & 0xffffffffu));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t k = static_cast<uint32_t>(key >> 32);
  if (k == 0u) return __uint_as_float(0x7fc00000u);
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

// One DPP step of a wave-wide unsigned 64-bit maximum: every lane takes the
// larger of its value and the value of the lane dpp_ctrl names.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const int lo = static_cast<int>(static_cast<uint32_t>(v));
  const int hi = static_cast<int>(static_cast<uint32_t>(v >> 32));
  const uint32_t olo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false));
  const uint32_t ohi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false));
  const uint64_t o = (static_cast<uint64_t>(ohi) << 32) | olo;
  return o > v ? o : v;
}

// Maximum over the 64 lanes of a wave, returned wave-uniform.  Within each
// row of 16 lanes: swap neighbours, swap pairs (quad_perm), mirror halves
// of 8, mirror the row (DPP); then the four row maxima by readlane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_u64<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_u64<0x141>(v);  // row_half_mirror
  v = dpp_max_u64<0x140>(v);  // row_mirror
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 16 * r));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 16 * r));
    const uint64_t x = (static_cast<uint64_t>(hi) << 32) | lo;
    best = x > best ? x : best;
  }
  return best;
}

// Maximum over each half of the wave (lanes 0-31 and 32-63), returned in
// every lane of that half: the row maxima as in wave_max_u64, then the two
// rows of each half.
__device__ __forceinline__ uint64_t half_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1>(v);
  v = dpp_max_u64<0x4E>(v);
  v = dpp_max_u64<0x141>(v);
  v = dpp_max_u64<0x140>(v);
  uint64_t row[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 16 * r));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 16 * r));
    row[r] = (static_cast<uint64_t>(hi) << 32) | lo;
  }
  const uint64_t h0 = row[0] > row[1] ? row[0] : row[1];
  const uint64_t h1 = row[2] > row[3] ? row[2] : row[3];
  return (threadIdx.x & 32) ? h1 : h0;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace moe
