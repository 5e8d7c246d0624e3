// Stages 3 and 4: the experts, as grouped GEMMs over the tile list.
//
// Each expert is SwiGLU, FFN(x) = W2 (SiLU(W1 x) * W3 x) ("Sparse MoE FFN"
// (DeepSeek-V3), "How it works", expert equation), or one of the other
// bodies the epilogue selects: GEGLU, or the biased GELU MLP W2 GELU(W1 x +
// b1) + b2 ("Lesson 2 -- From the Dense FFN to a Layer of Experts", section
// 2).  "Mixture of experts and architecture families", "The router and load
// balancing", notes that the per-expert loop is batched as grouped GEMMs;
// here one launch covers every expert plus the shared expert (an extra group
// whose rows are all tokens).
//
//   gate_up: H[row] = act(x W1^T) * (x W3^T), x = u[token of row]  (gather)
//            or GELU(x W1^T + b1) for the GELU MLP
//   down:    O[row] = H[row] W2^T (+ b2)   (routed rows, bf16 or fp32)
//            Z[t]   = Hs[t] W2s^T (+ b2s)  (shared rows)
//
// Both are C = A B^T with A [rows][K] and B [N][K] row-major (K contiguous),
// the layout in which the weights arrive.  bf16 runs on the gfx950 MFMA
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; fp32 runs on FMA.
#include "common.hpp"
#include "plan.hpp"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

struct GemmArgs {
  const Tile *tiles;
  const int32_t *tile_count;
  const int32_t *perm;  // gate_up: position -> slot (token = slot / k)
  int k;
  int E;
  // A rows: gate_up reads u (gathered for routed, direct for shared);
  // down reads H / Hs directly.
  const void *A_routed;
  const void *A_shared;
  int gather;
  // B: [E][N][K] routed, [N][K] shared; B1 only for gate_up.
  const void *B0_routed, *B1_routed, *B0_shared, *B1_shared;
  int N_routed, N_shared, K_routed, K_shared;
  void *C_routed;  // [rows][N]
  void *C_shared;  // [rows][N]
  int c_shared_f32;
  int epi;                   // Epi
  const void *bias_routed;   // [E][N] or null (EPI_BIAS, EPI_BIAS_GELU)
  const void *bias_shared;   // [N] or null
};

// The bias row of a tile's group, or null.
__device__ __forceinline__ const void *group_bias(const GemmArgs &g, bool shared, int group, int N, int es) {
  if (g.epi < EPI_BIAS) return nullptr;
  if (shared) return g.bias_shared;
  if (!g.bias_routed) return nullptr;
  return static_cast<const char *>(g.bias_routed) + static_cast<int64_t>(group) * N * es;
}

template <bool DUAL>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16(GemmArgs g) {
  const int tile_id = blockIdx.x;
  if (tile_id >= *g.tile_count) return;
  const Tile tl = g.tiles[tile_id];
  const bool shared = tl.group == g.E;
  const int N = shared ? g.N_shared : g.N_routed;
  const int K = shared ? g.K_shared : g.K_routed;
  const int n0 = blockIdx.y * BN;
  if (n0 >= N) return;

  __shared__ __attribute__((aligned(16))) unsigned char smem[(DUAL ? 3 : 2) * BM * 128];
  unsigned char *As = smem;
  unsigned char *Bs0 = smem + BM * 128;
  unsigned char *Bs1 = smem + 2 * BM * 128;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid >> 3, lch = tid & 7;

  const uint16_t *A = static_cast<const uint16_t *>(shared ? g.A_shared : g.A_routed);
  const uint16_t *B0 = static_cast<const uint16_t *>(shared ? g.B0_shared : g.B0_routed);
  const uint16_t *B1 = static_cast<const uint16_t *>(shared ? g.B1_shared : g.B1_routed);
  if (!shared) {
    const int64_t es = static_cast<int64_t>(N) * K;
    B0 += tl.group * es;
    if (DUAL) B1 += tl.group * es;
  }

  // Row pointers of the 4 A rows and 4 B rows this thread stages.
  const uint16_t *ap[4];
  const uint16_t *bp0[4];
  const uint16_t *bp1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 32 * i;
    ap[i] = nullptr;
    if (r < tl.nrows) {
      int64_t arow;
      if (g.gather && !shared)
        arow = g.perm[tl.row0 + r] / g.k;
      else
        arow = static_cast<int64_t>(tl.row0) + r;
      ap[i] = A + arow * K + lch * 8;
    }
    const int n = n0 + r;
    bp0[i] = n < N ? B0 + static_cast<int64_t>(n) * K + lch * 8 : nullptr;
    bp1[i] = (DUAL && n < N) ? B1 + static_cast<int64_t>(n) * K + lch * 8 : nullptr;
  }

  uint4 ra[4], rb0[4], rb1[4];
  const uint4 zero = make_uint4(0, 0, 0, 0);
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ap[i] ? *reinterpret_cast<const uint4 *>(ap[i] + k0) : zero;
      rb0[i] = bp0[i] ? *reinterpret_cast<const uint4 *>(bp0[i] + k0) : zero;
      if (DUAL) rb1[i] = bp1[i] ? *reinterpret_cast<const uint4 *>(bp1[i] + k0) : zero;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = swz(lrow + 32 * i, lch);
      *reinterpret_cast<uint4 *>(As + off) = ra[i];
      *reinterpret_cast<uint4 *>(Bs0 + off) = rb0[i];
      if (DUAL) *reinterpret_cast<uint4 *>(Bs1 + off) = rb1[i];
    }
  };

  constexpr int NM = DUAL ? 2 : 1;
  f32x16 acc[2][2][NM];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][m][r] = 0.f;

  const bool wave_rows = wm * 64 < tl.nrows;
  const bool hi_rows = wm * 64 + 32 < tl.nrows;

  load(0);
  store();
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) load(k0 + BK);
    if (wave_rows) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        bf16x8 a[2], b0[2], b1[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          a[mi] = *reinterpret_cast<const bf16x8 *>(As + swz(wm * 64 + mi * 32 + (lane & 31), ch));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int off = swz(wn * 64 + ni * 32 + (lane & 31), ch);
          b0[ni] = *reinterpret_cast<const bf16x8 *>(Bs0 + off);
          if (DUAL) b1[ni] = *reinterpret_cast<const bf16x8 *>(Bs1 + off);
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          if (mi == 1 && !hi_rows) continue;
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            acc[mi][ni][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b0[ni], acc[mi][ni][0], 0, 0, 0);
            if (DUAL)
              acc[mi][ni][NM - 1] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b1[ni], acc[mi][ni][NM - 1], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
    if (more) {
      store();
      __syncthreads();
    }
  }

  if (!wave_rows) return;
  const bool f32_out = shared && g.c_shared_f32;
  void *C = shared ? g.C_shared : g.C_routed;
  const uint16_t *bias = static_cast<const uint16_t *>(group_bias(g, shared, tl.group, N, 2));
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = n0 + wn * 64 + ni * 32 + (lane & 31);
        if (row >= tl.nrows || col >= N) continue;
        float v = acc[mi][ni][0][r];
        if (DUAL) {
          v = (g.epi == EPI_GELU_GLU ? gelu(v) : silu_fast(v)) * acc[mi][ni][NM - 1][r];
        } else {
          if (bias) v += bf16_to_f32(bias[col]);
          if (g.epi == EPI_BIAS_GELU) v = gelu(v);
        }
        const int64_t o = (static_cast<int64_t>(tl.row0) + row) * N + col;
        if (f32_out)
          static_cast<float *>(C)[o] = v;
        else
          static_cast<uint16_t *>(C)[o] = f32_to_bf16_hw(v);
      }
}

// fp32 path: LDS-tiled FMA, 32 rows x 64 columns per block, 8 rows a thread.
constexpr int FM = 32, FN = 64, FK = 16;

template <bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GemmArgs g) {
  const int tile_id = blockIdx.x;
  if (tile_id >= *g.tile_count) return;
  const Tile tl = g.tiles[tile_id];
  const bool shared = tl.group == g.E;
  const int N = shared ? g.N_shared : g.N_routed;
  const int K = shared ? g.K_shared : g.K_routed;
  const int n0 = blockIdx.y * FN;
  if (n0 >= N) return;
  __shared__ float As[FM][FK + 1];
  __shared__ float Bs0[FN][FK + 1];
  __shared__ float Bs1[DUAL ? FN : 1][FK + 1];

  const float *A = static_cast<const float *>(shared ? g.A_shared : g.A_routed);
  const float *B0 = static_cast<const float *>(shared ? g.B0_shared : g.B0_routed);
  const float *B1 = static_cast<const float *>(shared ? g.B1_shared : g.B1_routed);
  if (!shared) {
    const int64_t es = static_cast<int64_t>(N) * K;
    B0 += tl.group * es;
    if (DUAL) B1 += tl.group * es;
  }
  const int tid = threadIdx.x, tx = tid & 63, ty = tid >> 6;
  // A staging: 32 rows x 16 = 512 values, two per thread.
  const float *ap[2];
  int acol[2], arow_l[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    arow_l[i] = q / FK;
    acol[i] = q % FK;
    const int r = arow_l[i];
    ap[i] = nullptr;
    if (r < tl.nrows) {
      int64_t arow = (g.gather && !shared) ? g.perm[tl.row0 + r] / g.k : static_cast<int64_t>(tl.row0) + r;
      ap[i] = A + arow * K;
    }
  }
  float acc0[FM / 4], acc1[FM / 4];
#pragma unroll
  for (int i = 0; i < FM / 4; ++i) acc0[i] = acc1[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += FK) {
#pragma unroll
    for (int i = 0; i < 2; ++i) As[arow_l[i]][acol[i]] = ap[i] ? ap[i][k0 + acol[i]] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      const int n = q / FK, kk = q % FK;
      const bool ok = n0 + n < N;
      Bs0[n][kk] = ok ? B0[static_cast<int64_t>(n0 + n) * K + k0 + kk] : 0.f;
      if (DUAL) Bs1[n][kk] = ok ? B1[static_cast<int64_t>(n0 + n) * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      const float b0 = Bs0[tx][kk];
      const float b1 = DUAL ? Bs1[tx][kk] : 0.f;
#pragma unroll
      for (int i = 0; i < FM / 4; ++i) {
        const float a = As[ty + 4 * i][kk];
        acc0[i] = fmaf(a, b0, acc0[i]);
        if (DUAL) acc1[i] = fmaf(a, b1, acc1[i]);
      }
    }
    __syncthreads();
  }
  const int col = n0 + tx;
  if (col >= N) return;
  float *C = static_cast<float *>(shared ? g.C_shared : g.C_routed);
  const float *bias = static_cast<const float *>(group_bias(g, shared, tl.group, N, 4));
  const float bcol = bias ? bias[col] : 0.f;
#pragma unroll
  for (int i = 0; i < FM / 4; ++i) {
    const int row = ty + 4 * i;
    if (row >= tl.nrows) continue;
    float v;
    if (DUAL) {
      v = (g.epi == EPI_GELU_GLU ? gelu(acc0[i]) : silu(acc0[i])) * acc1[i];
    } else {
      v = bias ? acc0[i] + bcol : acc0[i];
      if (g.epi == EPI_BIAS_GELU) v = gelu(v);
    }
    C[(static_cast<int64_t>(tl.row0) + row) * N + col] = v;
  }
}

hipError_t launch_on(const Plan &p, const GemmArgs &g, bool dual, int n_max, hipStream_t s) {
  const bool bf16 = p.cfg.dtype == MOE_BF16;
  const int bn = bf16 ? BN : FN;
  const dim3 grid(static_cast<unsigned>(p.max_tiles), static_cast<unsigned>((n_max + bn - 1) / bn));
  if (bf16) {
    if (dual)
      hipLaunchKernelGGL(grouped_gemm_bf16<true>, grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL(grouped_gemm_bf16<false>, grid, dim3(256), 0, s, g);
  } else {
    if (dual)
      hipLaunchKernelGGL(grouped_gemm_f32<true>, grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL(grouped_gemm_f32<false>, grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace

int gemm_tile_m(int dtype) { return dtype == MOE_BF16 ? BM : FM; }

hipError_t launch_gate_up(const Plan &p, const void *u, const Experts &x, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  GemmArgs g{};
  g.tiles = p.tiles;
  g.tile_count = p.tile_count;
  g.perm = p.perm;
  g.k = c.k;
  g.E = c.E;
  g.A_routed = u;
  g.A_shared = u;
  g.gather = 1;
  g.epi = gate_up_epi(p.kind);
  const bool dual = epi_dual(g.epi);
  g.B0_routed = x.W1;
  g.B1_routed = dual ? x.W3 : nullptr;
  g.B0_shared = x.W1s;
  g.B1_shared = dual ? x.W3s : nullptr;
  g.bias_routed = x.b1;
  g.bias_shared = x.b1s;
  g.N_routed = c.F;
  g.N_shared = c.F_shared;
  g.K_routed = c.d;
  g.K_shared = c.d;
  g.C_routed = p.H;
  g.C_shared = p.Hs;
  g.c_shared_f32 = 0;
  const int n_max = c.F > c.F_shared ? c.F : c.F_shared;
  return launch_on(p, g, dual, n_max, s);
}

hipError_t launch_down(const Plan &p, const Experts &x, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  GemmArgs g{};
  g.tiles = p.tiles;
  g.tile_count = p.tile_count;
  g.perm = p.perm;
  g.k = c.k;
  g.E = c.E;
  g.A_routed = p.H;
  g.A_shared = p.Hs;
  g.gather = 0;
  g.epi = down_epi(p.kind);
  g.B0_routed = x.W2;
  g.B1_routed = nullptr;
  g.B0_shared = x.W2s;
  g.B1_shared = nullptr;
  g.bias_routed = x.b2;
  g.bias_shared = x.b2s;
  g.N_routed = c.d;
  g.N_shared = c.d;
  g.K_routed = c.F;
  g.K_shared = c.F_shared;
  g.C_routed = p.O;
  g.C_shared = p.Z;
  g.c_shared_f32 = 0;
  return launch_on(p, g, false, c.d, s);
}

}  // namespace moe
