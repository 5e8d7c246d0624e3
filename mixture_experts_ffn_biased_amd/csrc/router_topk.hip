// Stage 1: router GEMM fused with the score function, the selection-only
// bias, the group limit and top-k, one wave per token for the selection.
//
// Router: l = u . W_router^T with fp32 accumulation ("Mixture of Experts and
// Hybrid Architectures", "The router in code"; "Sparse MoE FFN", Routing:
// u_t^T e_i).  bf16 inputs use the bf16 MFMA (products of bf16 values are
// exact in fp32); fp32 inputs use fp32 FMA.
//
// bf16 layers with d a multiple of 128 split the GEMM over K when few 64-token
// tiles exist or K is long (router_logits_split writes fp32 partial logits,
// router_select adds them in a fixed order and selects), else run
// router_topk_stream: 64 tokens per workgroup, tiles of the tokens and of all
// router rows staged through a 4-slot LDS ring by direct global-to-LDS loads
// (three stages in flight).  Other layers run router_topk_bf16 /
// router_topk_f32 (register staging).  The selection of a token (select.hpp)
// is the same in every kernel.
#include "common.hpp"
#include "pipeline.hpp"
#include "plan.hpp"
#include "select.hpp"

namespace moe {
namespace {

constexpr int kRows = 32;           // tokens per block
constexpr int kLogitStride = 257;   // floats per logits row in LDS

// LDS tile of rows x 64 bf16 (128 bytes a row) in 16-byte chunks, XOR
// swizzled so that 16 consecutive rows reading one chunk hit distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__global__ __launch_bounds__(256) void router_topk_bf16(
    const uint16_t *__restrict__ u, const uint16_t *__restrict__ Wr, int64_t T, int d,
    SelArgs sel, int32_t *__restrict__ topk_idx, float *__restrict__ gates) {
  // 32 x 64 bf16 A tile + 256 x 64 bf16 B tile; later reused for the logits.
  __shared__ __attribute__((aligned(16))) unsigned char smem[kRows * 128 + kMaxExperts * 128 + 256];
  unsigned char *As = smem;
  unsigned char *Bs = smem + kRows * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int E = sel.E;

  const int lrow = tid >> 3, lch = tid & 7;
  const int64_t at = t0 + lrow;
  const uint16_t *arow = at < T ? u + at * d + lch * 8 : nullptr;
  uint4 ra;
  uint4 rb[kMaxExperts / 32];
  const uint4 zero = make_uint4(0, 0, 0, 0);

  auto load = [&](int k0) {
    ra = arow ? *reinterpret_cast<const uint4 *>(arow + k0) : zero;
#pragma unroll
    for (int i = 0; i < kMaxExperts / 32; ++i) {
      const int e = lrow + 32 * i;
      rb[i] = e < E ? *reinterpret_cast<const uint4 *>(Wr + static_cast<int64_t>(e) * d + k0 + lch * 8)
                    : zero;
    }
  };
  auto store = [&]() {
    *reinterpret_cast<uint4 *>(As + swz(lrow, lch)) = ra;
#pragma unroll
    for (int i = 0; i < kMaxExperts / 32; ++i)
      *reinterpret_cast<uint4 *>(Bs + swz(lrow + 32 * i, lch)) = rb[i];
  };

  const bool active = wave * 64 < E;
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  load(0);
  store();
  __syncthreads();
  for (int k0 = 0; k0 < d; k0 += 64) {
    const bool more = k0 + 64 < d;
    if (more) load(k0 + 64);
    if (active) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(As + swz(lane & 31, ch));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const bf16x8 b = *reinterpret_cast<const bf16x8 *>(Bs + swz(wave * 64 + ni * 32 + (lane & 31), ch));
          acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[ni], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (more) {
      store();
      __syncthreads();
    }
  }

  float *lg = reinterpret_cast<float *>(smem);
  if (active) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wave * 64 + ni * 32 + (lane & 31);
        if (col < E) lg[row * kLogitStride + col] = acc[ni][r];
      }
  }
  __syncthreads();
  for (int row = wave; row < kRows; row += 4) {
    const int64_t t = t0 + row;
    if (t >= T) break;
    select_token(lg + row * kLogitStride, sel, topk_idx + t * sel.k, gates + t * sel.k);
  }
}

__global__ __launch_bounds__(256) void router_topk_f32(
    const float *__restrict__ u, const float *__restrict__ Wr, int64_t T, int d, SelArgs sel,
    int32_t *__restrict__ topk_idx, float *__restrict__ gates) {
  __shared__ float lg[kRows * kLogitStride];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int E = sel.E;
  for (int q = tid; q < kRows * E; q += 256) {
    const int row = q / E, e = q % E;
    const int64_t t = t0 + row;
    if (t >= T) continue;
    const float *x = u + t * d;
    const float *w = Wr + static_cast<int64_t>(e) * d;
    float acc = 0.f;
    for (int j = 0; j < d; ++j) acc = fmaf(x[j], w[j], acc);
    lg[row * kLogitStride + e] = acc;
  }
  __syncthreads();
  for (int row = wave; row < kRows; row += 4) {
    const int64_t t = t0 + row;
    if (t >= T) break;
    select_token(lg + row * kLogitStride, sel, topk_idx + t * sel.k, gates + t * sel.k);
  }
}


// ---- streamed router for bf16, d % 128 == 0 -----------------------------------

constexpr int kRowsS = 64;  // tokens per workgroup

// NB = experts / 64 rounded up (1..4): B tile of 64*NB router rows.
template <int NB>
__global__ __launch_bounds__(256, 1) void router_topk_stream(
    const uint16_t *__restrict__ u, const uint16_t *__restrict__ Wr, int64_t T, int d, SelArgs sel,
    int32_t *__restrict__ topk_idx, float *__restrict__ gates) {
  constexpr int A_B = kRowsS * 64;         // 64 rows x 32 bf16
  constexpr int B_B = NB * 64 * 64;        // 64*NB rows x 32 bf16
  constexpr int SLOT = A_B + B_B;
  constexpr int PER_STAGE = 1 + NB;        // DMA instructions per wave per stage
  __shared__ __attribute__((aligned(16))) unsigned char ring0[SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[SLOT];
  __shared__ float lg[kRowsS * kLogitStride];
  unsigned char *const ring[4] = {ring0, ring1, ring2, ring3};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRowsS;
  const int E = sel.E;

  // DMA sources: group g of 16 rows lands at g*1024 (A) or A_B + g*1024 (B);
  // lane l -> row +l/4, physical chunk l%4 = logical chunk ^ ((row>>2)&3).
  const int sub = lane >> 2;
  const uint16_t *ap;
  {
    const int r = wave * 16 + sub;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    int64_t t = t0 + r;
    if (t >= T) t = T - 1;
    ap = u + t * d + c * 8;
  }
  const uint16_t *bp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r = (wave * NB + j) * 16 + sub;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int e = r < E ? r : E - 1;
    bp[j] = Wr + static_cast<int64_t>(e) * d + c * 8;
  }
  auto issue = [&](unsigned char *st, int kt) {
    const int koff = kt * 32;
    dma16(ap + koff, st + wave * 1024);
#pragma unroll
    for (int j = 0; j < NB; ++j) dma16(bp[j] + koff, st + A_B + (wave * NB + j) * 1024);
  };

  const int sw = (lane >> 2) & 3;
  const int fo0 = (lane & 31) * 64 + (((0 + (lane >> 5)) ^ sw) << 4);
  const int fo1 = (lane & 31) * 64 + (((2 + (lane >> 5)) ^ sw) << 4);
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  const int wcol = wave < NB ? wave : 0;  // waves past the experts compute a copy, never stored
  auto compute = [&](const unsigned char *st) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int fo = kk ? fo1 : fo0;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) a[mi] = *reinterpret_cast<const bf16x8 *>(st + mi * 2048 + fo);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        b[ni] = *reinterpret_cast<const bf16x8 *>(st + A_B + (wcol * 64 + ni * 32) * 64 + fo);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  };

  const int KT = d / 32;  // multiple of 4, >= 4
  issue(ring[0], 0);
  issue(ring[1], 1);
  issue(ring[2], 2);
  for (int j = 0; j < KT / 4 - 1; ++j) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      wait_vmcnt<2 * PER_STAGE>();
      raw_barrier();
      issue(ring[(s4 + 3) & 3], j * 4 + s4 + 3);
      compute(ring[s4]);
    }
  }
  wait_vmcnt<2 * PER_STAGE>();
  raw_barrier();
  issue(ring[3], KT - 1);
  compute(ring[0]);
  wait_vmcnt<2 * PER_STAGE>();
  raw_barrier();
  compute(ring[1]);
  wait_vmcnt<PER_STAGE>();
  raw_barrier();
  compute(ring[2]);
  wait_vmcnt<0>();
  raw_barrier();
  compute(ring[3]);

  if (wave < NB) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wave * 64 + ni * 32 + (lane & 31);
          if (col < E) lg[row * kLogitStride + col] = acc[mi][ni][r];
        }
  }
  __syncthreads();
  for (int row = wave; row < kRowsS; row += 4) {
    const int64_t t = t0 + row;
    if (t >= T) break;
    select_token(lg + row * kLogitStride, sel, topk_idx + t * sel.k, gates + t * sel.k);
  }
}

// ---- split-K router for bf16, d % 128 == 0 ------------------------------------
//
// When few 64-token tiles exist (decode) or the K loop is long, the router
// GEMM is split over K: workgroup (m, s) computes the partial logits of 64
// tokens over K range s and stores them (fp32); router_select then adds the
// splits in a fixed order (deterministic) and selects.

//
// part_sq (fused pre-norm block; null otherwise): each workgroup also sums
// the squares of its 64 tokens' inputs over its K range, in fp32 from the
// same LDS fragments the MFMAs read (wave w squares fragment mi = w/2 of
// half kk = w%2, so every value is squared exactly once), and stores them
// at part_sq[split][t]; router_select turns the sums into 1/rms.
template <int NB>
__global__ __launch_bounds__(256, 2) void router_logits_split(
    const uint16_t *__restrict__ u, const uint16_t *__restrict__ Wr, int64_t T, int d, int E,
    int kt_per_split, float *__restrict__ part, float *__restrict__ part_sq) {
  constexpr int A_B = kRowsS * 64;
  constexpr int B_B = NB * 64 * 64;
  constexpr int SLOT = A_B + B_B;
  constexpr int PER_STAGE = 1 + NB;
  __shared__ __attribute__((aligned(16))) unsigned char ring0[SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[SLOT];
  unsigned char *const ring[4] = {ring0, ring1, ring2, ring3};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRowsS;
  const int split = blockIdx.y;
  const int k_begin = split * kt_per_split * 32;

  const int sub = lane >> 2;
  const uint16_t *ap;
  {
    const int r = wave * 16 + sub;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    int64_t t = t0 + r;
    if (t >= T) t = T - 1;
    ap = u + t * d + k_begin + c * 8;
  }
  const uint16_t *bp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r = (wave * NB + j) * 16 + sub;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int e = r < E ? r : E - 1;
    bp[j] = Wr + static_cast<int64_t>(e) * d + k_begin + c * 8;
  }
  auto issue = [&](unsigned char *st, int kt) {
    const int koff = kt * 32;
    dma16(ap + koff, st + wave * 1024);
#pragma unroll
    for (int j = 0; j < NB; ++j) dma16(bp[j] + koff, st + A_B + (wave * NB + j) * 1024);
  };
  const int sw = (lane >> 2) & 3;
  const int fo0 = (lane & 31) * 64 + (((0 + (lane >> 5)) ^ sw) << 4);
  const int fo1 = (lane & 31) * 64 + (((2 + (lane >> 5)) ^ sw) << 4);
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  const int wcol = wave < NB ? wave : 0;
  const bool want_sq = part_sq != nullptr;
  const int sq_mi = wave >> 1, sq_kk = wave & 1;
  float sq = 0.f;  // squares of row sq_mi * 32 + lane % 32, this lane's K values
  auto compute = [&](const unsigned char *st) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int fo = kk ? fo1 : fo0;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) a[mi] = *reinterpret_cast<const bf16x8 *>(st + mi * 2048 + fo);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        b[ni] = *reinterpret_cast<const bf16x8 *>(st + A_B + (wcol * 64 + ni * 32) * 64 + fo);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
      if (want_sq && kk == sq_kk) {
        const bf16x8 v = sq_mi ? a[1] : a[0];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = static_cast<float>(v[i]);
          sq = fmaf(x, x, sq);  // x * x is exact in fp32
        }
      }
    }
  };
  const int KT = kt_per_split;  // multiple of 4, >= 4
  issue(ring[0], 0);
  issue(ring[1], 1);
  issue(ring[2], 2);
  for (int j = 0; j < KT / 4 - 1; ++j) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      wait_vmcnt<2 * PER_STAGE>();
      raw_barrier();
      issue(ring[(s4 + 3) & 3], j * 4 + s4 + 3);
      compute(ring[s4]);
    }
  }
  wait_vmcnt<2 * PER_STAGE>();
  raw_barrier();
  issue(ring[3], KT - 1);
  compute(ring[0]);
  wait_vmcnt<2 * PER_STAGE>();
  raw_barrier();
  compute(ring[1]);
  wait_vmcnt<PER_STAGE>();
  raw_barrier();
  compute(ring[2]);
  wait_vmcnt<0>();
  raw_barrier();
  compute(ring[3]);

  // The partial logits are written once and read once, so both sides carry
  // the non-temporal hint: they need not displace u, which the gate/up
  // gathers read again right after.
  if (wave < NB) {
    float *out = part + (static_cast<int64_t>(split) * T) * E;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wave * 64 + ni * 32 + (lane & 31);
          const int64_t t = t0 + row;
          if (col < E && t < T) __builtin_nontemporal_store(acc[mi][ni][r], &out[t * E + col]);
        }
  }
  if (want_sq) {
    // Row r's squares: waves 2(r/32) and 2(r/32)+1 (the two K halves), lanes
    // r%32 and r%32+32 of each, added in that fixed order.  Ring slot 0 is
    // free: every wave has passed the barrier after its last read of it.
    float *sqs = reinterpret_cast<float *>(ring0);
    sqs[wave * 64 + lane] = sq;
    __syncthreads();
    if (tid < kRowsS) {
      const int mi = tid >> 5, l = tid & 31;
      const float *w0 = sqs + (2 * mi) * 64, *w1 = sqs + (2 * mi + 1) * 64;
      const float v = (w0[l] + w0[l + 32]) + (w1[l] + w1[l + 32]);
      const int64_t t = t0 + tid;
      if (t < T) part_sq[static_cast<int64_t>(split) * T + t] = v;
    }
  }
}

// One wave per token: logits = sum of the splits in order, then selection.
// One wave per token.  NSC = the split count rounded up to a multiple of 4:
// every partial of the wave's experts is loaded before any is added (loads
// past the last split re-read it and add +0, which changes nothing), so the
// partial sums cost one memory round trip, not one per split.  The sum order
// is fixed: four running sums over splits sp % 4, then (v0 + v1) + (v2 + v3).
//
// Fused pre-norm block (part_sq non-null): the token's sum of squares is the
// splits' partial sums added in order; rs = 1 / sqrt(sum / d + eps) (IEEE
// square root and division) scales the summed logits before selection, and
// is stored at rscale[t] for the gate/up epilogue.
template <int NSC>
__global__ __launch_bounds__(256) void router_select(const float *__restrict__ part, int nsplit,
                                                     int64_t T, SelArgs sel,
                                                     int32_t *__restrict__ topk_idx,
                                                     float *__restrict__ gates, const float *__restrict__ part_sq,
                                                     int d, float eps, float *__restrict__ rscale) {
  __shared__ float lg[4][kLogitStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = sel.E;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (t >= T) return;
  constexpr int P = kMaxExperts / 64;
  float x[P][NSC];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int e = lane + 64 * p < E ? lane + 64 * p : E - 1;
#pragma unroll
    for (int sp = 0; sp < NSC; ++sp) {
      const int spc = sp < nsplit ? sp : nsplit - 1;
      x[p][sp] = __builtin_nontemporal_load(&part[(static_cast<int64_t>(spc) * T + t) * E + e]);
    }
  }
  float rs = 1.f;
  if (part_sq) {
    float q = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) q += part_sq[static_cast<int64_t>(sp) * T + t];
    rs = 1.0f / sqrtf(q / static_cast<float>(d) + eps);
    if (lane == 0) rscale[t] = rs;
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int e = lane + 64 * p;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < NSC; ++sp) v[sp & 3] += sp < nsplit ? x[p][sp] : 0.f;
    const float l = (v[0] + v[1]) + (v[2] + v[3]);
    if (e < E) lg[wave][e] = part_sq ? rs * l : l;
  }
  select_token(lg[wave], sel, topk_idx + t * sel.k, gates + t * sel.k);
}

}  // namespace

int router_splits(int64_t T, int d) {
  // Split K so that about 2 workgroups per CU (512) run, each >= 4 stages.
  const int64_t mt = (T + kRowsS - 1) / kRowsS;
  const int q = d / 128;  // stage groups of 4
  int best = 1;
  for (int s = 1; s <= q && s <= 16; ++s)
    if (q % s == 0 && mt * s <= 512) best = s;
  return best;
}

hipError_t launch_router_topk(const Plan &p, const void *u, const void *Wr, const float *bias,
                              int32_t *topk_idx, float *gates, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  SelArgs sel{c.E, c.k, c.score_fn, c.n_groups, c.topk_groups, c.route_scale, bias};
  // The fused pre-norm block always takes the split-K pair (its logits
  // kernel also sums the squares of the token rows), with one split or more.
  if (c.dtype == MOE_BF16 && c.d % 128 == 0 && (p.router_splits > 1 || p.fused_norm)) {
    const int S = p.router_splits;
    const dim3 grid(static_cast<unsigned>((c.T + kRowsS - 1) / kRowsS), static_cast<unsigned>(S));
    const int ktps = c.d / 32 / S;
    auto *U = static_cast<const uint16_t *>(u);
    auto *W = static_cast<const uint16_t *>(Wr);
    const int nb = (c.E + 63) / 64;
    if (nb == 1)
      hipLaunchKernelGGL(router_logits_split<1>, grid, dim3(256), 0, s, U, W, c.T, c.d, c.E, ktps, p.router_part,
                         p.part_sq);
    else if (nb == 2)
      hipLaunchKernelGGL(router_logits_split<2>, grid, dim3(256), 0, s, U, W, c.T, c.d, c.E, ktps, p.router_part,
                         p.part_sq);
    else if (nb == 3)
      hipLaunchKernelGGL(router_logits_split<3>, grid, dim3(256), 0, s, U, W, c.T, c.d, c.E, ktps, p.router_part,
                         p.part_sq);
    else
      hipLaunchKernelGGL(router_logits_split<4>, grid, dim3(256), 0, s, U, W, c.T, c.d, c.E, ktps, p.router_part,
                         p.part_sq);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 sgrid(static_cast<unsigned>((c.T + 3) / 4));
    if (S <= 4)
      hipLaunchKernelGGL(router_select<4>, sgrid, dim3(256), 0, s, p.router_part, S, c.T, sel, topk_idx, gates,
                         p.part_sq, c.d, p.norm_eps, p.rscale);
    else if (S <= 8)
      hipLaunchKernelGGL(router_select<8>, sgrid, dim3(256), 0, s, p.router_part, S, c.T, sel, topk_idx, gates,
                         p.part_sq, c.d, p.norm_eps, p.rscale);
    else if (S <= 12)
      hipLaunchKernelGGL(router_select<12>, sgrid, dim3(256), 0, s, p.router_part, S, c.T, sel, topk_idx, gates,
                         p.part_sq, c.d, p.norm_eps, p.rscale);
    else
      hipLaunchKernelGGL(router_select<16>, sgrid, dim3(256), 0, s, p.router_part, S, c.T, sel, topk_idx, gates,
                         p.part_sq, c.d, p.norm_eps, p.rscale);
    return hipGetLastError();
  }
  if (c.dtype == MOE_BF16 && c.d % 128 == 0) {
    const dim3 grid(static_cast<unsigned>((c.T + kRowsS - 1) / kRowsS));
    const int nb = (c.E + 63) / 64;
    auto *U = static_cast<const uint16_t *>(u);
    auto *W = static_cast<const uint16_t *>(Wr);
    if (nb == 1)
      hipLaunchKernelGGL(router_topk_stream<1>, grid, dim3(256), 0, s, U, W, c.T, c.d, sel, topk_idx, gates);
    else if (nb == 2)
      hipLaunchKernelGGL(router_topk_stream<2>, grid, dim3(256), 0, s, U, W, c.T, c.d, sel, topk_idx, gates);
    else if (nb == 3)
      hipLaunchKernelGGL(router_topk_stream<3>, grid, dim3(256), 0, s, U, W, c.T, c.d, sel, topk_idx, gates);
    else
      hipLaunchKernelGGL(router_topk_stream<4>, grid, dim3(256), 0, s, U, W, c.T, c.d, sel, topk_idx, gates);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((c.T + kRows - 1) / kRows));
  if (c.dtype == MOE_BF16)
    hipLaunchKernelGGL(router_topk_bf16, grid, dim3(256), 0, s, static_cast<const uint16_t *>(u),
                       static_cast<const uint16_t *>(Wr), c.T, c.d, sel, topk_idx, gates);
  else
    hipLaunchKernelGGL(router_topk_f32, grid, dim3(256), 0, s, static_cast<const float *>(u),
                       static_cast<const float *>(Wr), c.T, c.d, sel, topk_idx, gates);
  return hipGetLastError();
}

}  // namespace moe
