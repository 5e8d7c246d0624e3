// Grouped expert GEMMs for prefill-sized groups (many rows per expert): a
// persistent, XCD-aware, weight-streaming kernel for gfx950.
//
// Same two products as grouped_gemm.hip (the SwiGLU expert of "Sparse MoE
// FFN" (DeepSeek-V3), "How it works", batched as grouped GEMMs as "Mixture of
// experts and architecture families", "The router and load balancing",
// suggests); only the schedule and the data movement differ:
//
//  * One 512-thread workgroup per CU loops over work items (tile, n-slab).
//    Items are kept in eight per-XCD lists: a chunk (up to two 256-row tiles
//    of one expert) goes to one XCD with all its n-slabs, the tiles of a
//    chunk adjacent.  Workgroups of an XCD take items from their list in
//    order through an atomic counter, so the workgroups running together on
//    an XCD share the expert's token rows and weight slabs in that XCD's L2,
//    and each weight byte is fetched from HBM about once.  A workgroup whose
//    list is empty takes items from the other XCDs' lists.
//  * Tiles of 256 rows x 256 weight rows x 32, staged by direct global-to-LDS
//    16-byte loads (global_load_lds_dwordx4) through a 4-stage ring, so three
//    stages (96 KB) are in flight while one is multiplied; no VGPR staging.
//  * Eight waves in a 2x4 grid (two per SIMD, one from each row half), each
//    128 x 64 of v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  A wave
//    multiplies only the 32-row blocks that hold rows of the tile (its K loop
//    is specialised on that count), so a SIMD's MFMA work follows the tile's
//    row count, and each SIMD has a second wave to cover waits.
//  * gate_up: the 256 weight rows of a slab are 32 rows of W1 then the same
//    32 of W3 per wave column, so SiLU(x W1^T) * (x W3^T) meets in the same
//    lane; the bf16 result goes through LDS to 16-byte stores.
#include "common.hpp"
#include "pipeline.hpp"
#include "plan.hpp"

namespace moe {
namespace {

constexpr int SBM = 256, SBN = 256, SBK = 32, NSTAGE = 4;
constexpr int NTHREADS = 512;  // 8 waves: 2 row halves x 4 column quarters
constexpr int A_BYTES = SBM * SBK * 2;
constexpr int B_BYTES = SBN * SBK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

struct StreamArgs {
  const Tile *tiles;
  const int2 *items;        // per-XCD segments of {tile id, n-slab}
  const int32_t *xcd_off;   // [8] segment starts
  const int32_t *xcd_cnt;   // [8] segment lengths
  int32_t *counters;        // [8] zero on entry
  const int32_t *perm;      // gate_up: position -> slot
  int k;
  int E;
  const void *A_routed, *A_shared;
  int gather;
  const void *B0_routed, *B1_routed, *B0_shared, *B1_shared;
  int N_routed, N_shared, K_routed, K_shared;
  void *C_routed, *C_shared;
};

// Ring slots of one workgroup (separate __shared__ arrays).
struct Ring {
  unsigned char *s[NSTAGE];
};

// The K loop of one item for a wave with NMI active 32-row blocks (0..4).
// Every wave runs the same loads and barriers whatever its NMI, so waves
// with different row counts stay in step.
template <bool DUAL, int NMI>
__device__ __forceinline__ void kloop(const Ring &ring, const uint16_t *const (&ap)[2],
                                      const uint16_t *const (&bp)[2], int KT, int wave, int wm,
                                      int wn, int fo0, int fo1, f32x16 (&acc)[4][2]) {
  auto issue = [&](unsigned char *st, int kt) {
    const int koff = kt * SBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(ap[i] + koff, st + (wave * 2 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(bp[i] + koff, st + A_BYTES + (wave * 2 + i) * 1024);
  };
  auto compute = [&](const unsigned char *st) {
    if (NMI == 0) return;
    const unsigned char *sa = st + wm * 128 * 64;
    const unsigned char *sb = st + A_BYTES + wn * 64 * 64;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int fo = kk ? fo1 : fo0;
      bf16x8 a[NMI > 0 ? NMI : 1], b[2];
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) a[mi] = *reinterpret_cast<const bf16x8 *>(sa + mi * 2048 + fo);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) b[ni] = *reinterpret_cast<const bf16x8 *>(sb + ni * 2048 + fo);
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  };
  constexpr int PS = 2 * 2;  // loads per wave per stage
  issue(ring.s[0], 0);
  issue(ring.s[1], 1);
  issue(ring.s[2], 2);
  // Stage kt lives in slot kt % 4 (unrolled by 4: static slot indices).  It
  // is complete once at most the two later stages are outstanding; after
  // the barrier, stage kt+3 refills the slot of stage kt-1.
  for (int j = 0; j < KT / NSTAGE - 1; ++j) {
#pragma unroll
    for (int s4 = 0; s4 < NSTAGE; ++s4) {
      wait_vmcnt<2 * PS>();
      raw_barrier();
      issue(ring.s[(s4 + 3) & 3], j * NSTAGE + s4 + 3);
      compute(ring.s[s4]);
    }
  }
  wait_vmcnt<2 * PS>();
  raw_barrier();
  issue(ring.s[3], KT - 1);
  compute(ring.s[0]);
  wait_vmcnt<2 * PS>();
  raw_barrier();
  compute(ring.s[1]);
  wait_vmcnt<PS>();
  raw_barrier();
  compute(ring.s[2]);
  wait_vmcnt<0>();
  raw_barrier();
  compute(ring.s[3]);
}

template <bool DUAL>
__device__ __forceinline__ void run_item(const StreamArgs &g, int2 item, const Ring &ring) {
  const Tile tl = g.tiles[item.x];
  const bool shared = tl.group == g.E;
  const int N = shared ? g.N_shared : g.N_routed;
  const int K = shared ? g.K_shared : g.K_routed;
  const int n0 = item.y * (DUAL ? SBN / 2 : SBN);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  const uint16_t *A = static_cast<const uint16_t *>(shared ? g.A_shared : g.A_routed);
  const uint16_t *B0 = static_cast<const uint16_t *>(shared ? g.B0_shared : g.B0_routed);
  const uint16_t *B1 = static_cast<const uint16_t *>(shared ? g.B1_shared : g.B1_routed);
  if (!shared) {
    const int64_t es = static_cast<int64_t>(N) * K;
    B0 += tl.group * es;
    if (DUAL) B1 += tl.group * es;
  }

  // DMA sources: load i of wave w fills LDS rows g*16 .. g*16+15 (g = 2w+i)
  // of the A and B tiles; lane l lands in row +l/4, physical chunk l%4,
  // which holds logical k-chunk (l%4) ^ ((row>>2)&3).  Rows past the tile's
  // count read its first row (never stored).
  const uint16_t *ap[2];
  const uint16_t *bp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave * 2 + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int rr = r < tl.nrows ? r : 0;
    int64_t arow;
    if (g.gather && !shared)
      arow = g.perm[tl.row0 + rr] / g.k;
    else
      arow = static_cast<int64_t>(tl.row0) + rr;
    ap[i] = A + arow * K + c * 8;
    int64_t brow;
    const uint16_t *bsrc = B0;
    if (DUAL) {
      // 64 rows per wave column: 32 of W1, then the same 32 of W3.
      const int q = r & 63;
      brow = n0 + (r >> 6) * 32 + (q & 31);
      if (q >= 32) bsrc = B1;
    } else {
      brow = n0 + r;
    }
    bp[i] = bsrc + brow * K + c * 8;
  }

  const int sw = (lane >> 2) & 3;
  const int fo0 = (lane & 31) * 64 + (((0 + (lane >> 5)) ^ sw) << 4);
  const int fo1 = (lane & 31) * 64 + (((2 + (lane >> 5)) ^ sw) << 4);

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // Active 32-row blocks of this wave's half (wave-uniform).
  int rows_here = tl.nrows - wm * 128;
  rows_here = rows_here < 0 ? 0 : (rows_here > 128 ? 128 : rows_here);
  const int nmi = __builtin_amdgcn_readfirstlane((rows_here + 31) >> 5);
  const int KT = K / SBK;

  // The previous item's stores and loads are complete before the ring refills.
  wait_vmcnt<0>();
  raw_barrier();
  switch (nmi) {
    case 0: kloop<DUAL, 0>(ring, ap, bp, KT, wave, wm, wn, fo0, fo1, acc); break;
    case 1: kloop<DUAL, 1>(ring, ap, bp, KT, wave, wm, wn, fo0, fo1, acc); break;
    case 2: kloop<DUAL, 2>(ring, ap, bp, KT, wave, wm, wn, fo0, fo1, acc); break;
    case 3: kloop<DUAL, 3>(ring, ap, bp, KT, wave, wm, wn, fo0, fo1, acc); break;
    default: kloop<DUAL, 4>(ring, ap, bp, KT, wave, wm, wn, fo0, fo1, acc); break;
  }
  // Every wave is done reading the ring before it is reused for the output.
  raw_barrier();

  const int row_lane = 4 * (lane >> 5);
  if (DUAL) {
    // H tile: 256 rows x 128 columns bf16 (256 bytes a row); rows 0..127 in
    // slot 0, rows 128..255 in slot 1.
    uint16_t *Ht = reinterpret_cast<uint16_t *>(wm ? ring.s[1] : ring.s[0]);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi >= nmi) break;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mi * 32 + 8 * (r >> 2) + row_lane + (r & 3);
        const int col = wn * 32 + (lane & 31);
        Ht[row * 128 + col] = f32_to_bf16(silu(acc[mi][0][r]) * acc[mi][1][r]);
      }
    }
    __syncthreads();
    uint16_t *C = static_cast<uint16_t *>(shared ? g.C_shared : g.C_routed);
#pragma unroll 4
    for (int j = 0; j < 8; ++j) {
      const int q = tid + NTHREADS * j;
      const int row = q >> 4, ch = q & 15;
      const uint16_t *H = reinterpret_cast<const uint16_t *>(row < 128 ? ring.s[0] : ring.s[1]);
      if (row < tl.nrows)
        *reinterpret_cast<uint4 *>(C + (static_cast<int64_t>(tl.row0) + row) * N + n0 + ch * 8) =
            *reinterpret_cast<const uint4 *>(H + (row & 127) * 128 + ch * 8);
    }
    __syncthreads();
  } else {
    // Output tile: 256 x 256 bf16 (512 bytes a row); rows 64*s .. 64*s+63 in slot s.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi >= nmi) break;
      uint16_t *Ot = reinterpret_cast<uint16_t *>(
          wm ? (mi < 2 ? ring.s[2] : ring.s[3]) : (mi < 2 ? ring.s[0] : ring.s[1]));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = (mi & 1) * 32 + 8 * (r >> 2) + row_lane + (r & 3);
          const int col = wn * 64 + ni * 32 + (lane & 31);
          Ot[row * 256 + col] = f32_to_bf16(acc[mi][ni][r]);
        }
    }
    __syncthreads();
    uint16_t *C = static_cast<uint16_t *>(shared ? g.C_shared : g.C_routed);
#pragma unroll 4
    for (int j = 0; j < 16; ++j) {
      const int q = tid + NTHREADS * j;
      const int row = q >> 5, ch = q & 31;
      const unsigned char *slot =
          row < 128 ? (row < 64 ? ring.s[0] : ring.s[1]) : (row < 192 ? ring.s[2] : ring.s[3]);
      if (row < tl.nrows)
        *reinterpret_cast<uint4 *>(C + (static_cast<int64_t>(tl.row0) + row) * N + n0 + ch * 8) =
            *reinterpret_cast<const uint4 *>(slot + (row & 63) * 512 + ch * 16);
    }
    __syncthreads();
  }
}

template <bool DUAL>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_gemm_stream(StreamArgs g) {
  // Four separate ring slots: the compiler can then tell the LDS loads into
  // one slot from the reads of another and adds no waits of its own.
  __shared__ __attribute__((aligned(16))) unsigned char ring0[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[STAGE_BYTES];
  __shared__ int item_sh;
  Ring ring;
  ring.s[0] = ring0;
  ring.s[1] = ring1;
  ring.s[2] = ring2;
  ring.s[3] = ring3;
  const int xcd = blockIdx.x & 7;
  for (int o = 0; o < 8; ++o) {
    const int x = (xcd + o) & 7;
    const int cnt = g.xcd_cnt[x];
    const int off = g.xcd_off[x];
    for (;;) {
      if (threadIdx.x == 0) item_sh = atomicAdd(&g.counters[x], 1);
      __syncthreads();
      const int it = item_sh;
      __syncthreads();
      if (it >= cnt) break;
      run_item<DUAL>(g, g.items[off + it], ring);
    }
  }
}

// ---- schedule: per-XCD item lists ------------------------------------------

constexpr int kMaxChunks = 4096;

// One block.  Rebuilds the tile numbering of perm_scan (experts in order,
// ceil(count/256) tiles each, then the shared expert's tiles), groups tiles
// into chunks of up to two per expert, deals chunks to XCDs round-robin and
// writes both GEMMs' item lists (tile fastest, then n-slab, within a chunk).
__global__ __launch_bounds__(256) void stream_schedule(
    const int32_t *__restrict__ counts, int E, int64_t T, int has_shared, int nt_gu_r, int nt_gu_s,
    int nt_dn_r, int nt_dn_s, int2 *__restrict__ items_gu, int2 *__restrict__ items_dn,
    int32_t *__restrict__ meta /* [2][3][8]: off, cnt, counter for gate_up, down */) {
  __shared__ int cfirst[kMaxChunks];
  __shared__ unsigned char cmt[kMaxChunks];
  __shared__ int cpos[2][kMaxChunks];
  __shared__ int buf[256];
  __shared__ int xtot[2][8];
  __shared__ int xoff[2][8];
  const int tid = threadIdx.x;
  const int e = tid;
  const int c = e < E ? counts[e] : 0;
  const int nt = (c + SBM - 1) / SBM;
  const int nch = (nt + 1) / 2;
  // exclusive scans of tiles and chunks
  buf[tid] = nt;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? buf[tid - o] : 0;
    __syncthreads();
    buf[tid] += v;
    __syncthreads();
  }
  const int tile_off = buf[tid] - nt;
  const int routed_tiles = buf[255];
  __syncthreads();
  buf[tid] = nch;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? buf[tid - o] : 0;
    __syncthreads();
    buf[tid] += v;
    __syncthreads();
  }
  const int chunk_off = buf[tid] - nch;
  const int routed_chunks = buf[255];
  __syncthreads();
  for (int j = 0; j < nch; ++j) {
    cfirst[chunk_off + j] = tile_off + 2 * j;
    cmt[chunk_off + j] = static_cast<unsigned char>(nt - 2 * j < 2 ? nt - 2 * j : 2);
  }
  int n_chunks = routed_chunks;
  if (has_shared) {
    const int ns = static_cast<int>((T + SBM - 1) / SBM);
    const int nsc = (ns + 1) / 2;
    for (int j = tid; j < nsc; j += 256) {
      cfirst[routed_chunks + j] = routed_tiles + 2 * j;
      cmt[routed_chunks + j] = static_cast<unsigned char>(ns - 2 * j < 2 ? ns - 2 * j : 2);
    }
    n_chunks += nsc;
  }
  __syncthreads();
  if (tid < 16) {
    const int x = tid & 7, list = tid >> 3;
    int pos = 0;
    for (int ch = x; ch < n_chunks; ch += 8) {
      cpos[list][ch] = pos;
      const bool sh = ch >= routed_chunks;
      const int ntl = list == 0 ? (sh ? nt_gu_s : nt_gu_r) : (sh ? nt_dn_s : nt_dn_r);
      pos += cmt[ch] * ntl;
    }
    xtot[list][x] = pos;
  }
  __syncthreads();
  if (tid < 2) {
    int run = 0;
    for (int x = 0; x < 8; ++x) {
      xoff[tid][x] = run;
      meta[tid * 24 + x] = run;
      meta[tid * 24 + 8 + x] = xtot[tid][x];
      meta[tid * 24 + 16 + x] = 0;
      run += xtot[tid][x];
    }
  }
  __syncthreads();
  for (int ch = tid; ch < n_chunks; ch += 256) {
    const bool sh = ch >= routed_chunks;
    const int mt = cmt[ch];
    for (int list = 0; list < 2; ++list) {
      const int ntl = list == 0 ? (sh ? nt_gu_s : nt_gu_r) : (sh ? nt_dn_s : nt_dn_r);
      int2 *out = (list == 0 ? items_gu : items_dn) + xoff[list][ch & 7] + cpos[list][ch];
      for (int n = 0; n < ntl; ++n)
        for (int m = 0; m < mt; ++m) out[n * mt + m] = make_int2(cfirst[ch] + m, n);
    }
  }
}

int g_num_cus = 0;

int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

StreamArgs base_args(const Plan &p, int list) {
  StreamArgs a{};
  a.tiles = p.tiles;
  a.items = list == 0 ? p.items_gu : p.items_dn;
  a.xcd_off = p.sched_meta + list * 24;
  a.xcd_cnt = p.sched_meta + list * 24 + 8;
  a.counters = p.sched_meta + list * 24 + 16;
  a.perm = p.perm;
  a.k = p.cfg.k;
  a.E = p.cfg.E;
  return a;
}

}  // namespace

int stream_tile_m() { return SBM; }
int stream_max_chunks() { return kMaxChunks; }
int stream_nslab_gate_up(int F) { return F / (SBN / 2); }
int stream_nslab_down(int d) { return d / SBN; }

hipError_t launch_stream_schedule(const Plan &p, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  hipLaunchKernelGGL(stream_schedule, dim3(1), dim3(256), 0, s, p.counts, c.E, c.T, c.F_shared > 0 ? 1 : 0,
                     c.F / (SBN / 2), c.F_shared / (SBN / 2), c.d / SBN, c.d / SBN, p.items_gu, p.items_dn,
                     p.sched_meta);
  return hipGetLastError();
}

hipError_t launch_stream_gate_up(const Plan &p, const void *u, const void *W1, const void *W3,
                                 const void *W1s, const void *W3s, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  StreamArgs a = base_args(p, 0);
  a.A_routed = u;
  a.A_shared = u;
  a.gather = 1;
  a.B0_routed = W1;
  a.B1_routed = W3;
  a.B0_shared = W1s;
  a.B1_shared = W3s;
  a.N_routed = c.F;
  a.N_shared = c.F_shared;
  a.K_routed = c.d;
  a.K_shared = c.d;
  a.C_routed = p.H;
  a.C_shared = p.Hs;
  hipLaunchKernelGGL(grouped_gemm_stream<true>, dim3(num_cus()), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_down(const Plan &p, const void *W2, const void *W2s, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  StreamArgs a = base_args(p, 1);
  a.A_routed = p.H;
  a.A_shared = p.Hs;
  a.gather = 0;
  a.B0_routed = W2;
  a.B1_routed = nullptr;
  a.B0_shared = W2s;
  a.B1_shared = nullptr;
  a.N_routed = c.d;
  a.N_shared = c.d;
  a.K_routed = c.F;
  a.K_shared = c.F_shared;
  a.C_routed = p.O;
  a.C_shared = p.Z;
  hipLaunchKernelGGL(grouped_gemm_stream<false>, dim3(num_cus()), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
