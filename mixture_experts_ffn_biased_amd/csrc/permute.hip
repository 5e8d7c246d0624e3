// Stage 2: expert-contiguous permutation of the T*k routed slots.
//
// "Sparse MoE FFN" (DeepSeek-V3), "Packed forward": each expert gathers the
// tokens whose selection contains it.  Here that gather is planned once for
// all experts: a per-expert histogram, an exclusive prefix scan in LDS, and a
// stable scatter (within an expert, slots keep ascending t*k + j order), so
// the grouped GEMMs read one contiguous row range per expert and the combine
// finds every slot's row through the inverse map.  Integer work only; the
// result is unique and deterministic.  The scan kernel also writes the tile
// list of the grouped GEMMs, so no count ever travels to the host.
#include "common.hpp"
#include "plan.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void perm_hist(const int32_t *__restrict__ idx, int64_t S, int E,
                                                 int32_t *__restrict__ blk_counts) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kPermChunk;
  const int64_t s1 = s0 + kPermChunk < S ? s0 + kPermChunk : S;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) atomicAdd(&h[idx[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk_counts[blockIdx.x * static_cast<int64_t>(E) + e] = h[e];
}

// Block-wide exclusive scan of one value per thread (256 threads).
__device__ int exclusive_scan_256(int v, int *buf, int *total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  *total = buf[255];
  __syncthreads();
  return incl - v;
}

// One block: totals per expert, offsets, per-block bases, and the GEMM tiles.
__global__ __launch_bounds__(256) void perm_scan(
    const int32_t *__restrict__ blk_counts, int nblk, int E, int64_t S, int64_t T, int has_shared,
    int tile_m, int balanced, int32_t *__restrict__ blk_base, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, Tile *__restrict__ tiles, int32_t *__restrict__ tile_count) {
  __shared__ int buf[256];
  const int e = threadIdx.x;
  // The per-block counts are read 16 at a time, so their loads overlap.
  constexpr int U = 16;
  int c = 0;
  if (e < E) {
    int b = 0;
    for (; b + U <= nblk; b += U) {
      int v[U];
#pragma unroll
      for (int i = 0; i < U; ++i) v[i] = blk_counts[static_cast<int64_t>(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < U; ++i) c += v[i];
    }
    for (; b < nblk; ++b) c += blk_counts[static_cast<int64_t>(b) * E + e];
  }
  const int nt = e < E ? (c + tile_m - 1) / tile_m : 0;
  int total_slots, total_tiles;
  const int off = exclusive_scan_256(e < E ? c : 0, buf, &total_slots);
  const int toff = exclusive_scan_256(nt, buf, &total_tiles);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    int run = off;
    int b = 0;
    for (; b + U <= nblk; b += U) {
      int v[U];
#pragma unroll
      for (int i = 0; i < U; ++i) v[i] = blk_counts[static_cast<int64_t>(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        blk_base[static_cast<int64_t>(b + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; b < nblk; ++b) {
      blk_base[static_cast<int64_t>(b) * E + e] = run;
      run += blk_counts[static_cast<int64_t>(b) * E + e];
    }
    for (int i = 0; i < nt; ++i) {
      int64_t r0;
      int n;
      tile_rows(c, nt, i, tile_m, balanced, &r0, &n);
      tiles[toff + i] = Tile{e, off + static_cast<int32_t>(r0), n, 0};
    }
  }
  if (e == 0) offsets[E] = static_cast<int32_t>(S);
  int ns = 0;
  if (has_shared) {
    ns = static_cast<int>((T + tile_m - 1) / tile_m);
    for (int i = e; i < ns; i += 256) {
      int64_t r0;
      int n;
      tile_rows(T, ns, i, tile_m, balanced, &r0, &n);
      tiles[total_tiles + i] = Tile{E, static_cast<int32_t>(r0), n, 0};
    }
  }
  if (e == 0) *tile_count = total_tiles + ns;
}

// Stable scatter: a block walks its chunk in rounds of 256 slots (4 waves of
// 64).  A slot's position is the running count of its expert, plus the
// slots of that expert in the earlier waves of the round, plus its rank
// among the lanes of its own wave holding the same expert.  The lanes with
// the same expert are found with one ballot per bit of the expert index.
// rscale (fused pre-norm block; null otherwise): the token's 1/rms is copied
// to its slot's position, rperm[pos] = rscale[slot / k].
__global__ __launch_bounds__(256) void perm_scatter(const int32_t *__restrict__ idx, int64_t S, int E,
                                                    const int32_t *__restrict__ blk_base,
                                                    int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                    const float *__restrict__ rscale, int k,
                                                    float *__restrict__ rperm) {
  static_assert(kMaxExperts <= 256, "expert index in 8 bits");
  __shared__ int run[kMaxExperts];
  __shared__ int wcnt[4][kMaxExperts];  // slots of each expert in each wave of the round
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) run[e] = blk_base[blockIdx.x * static_cast<int64_t>(E) + e];
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kPermChunk;
  const int64_t s1 = s0 + kPermChunk < S ? s0 + kPermChunk : S;
  const uint64_t lower = (1ull << lane) - 1;
  for (int64_t base = s0; base < s1; base += 256) {
    for (int i = tid; i < 4 * kMaxExperts; i += 256) (&wcnt[0][0])[i] = 0;
    const int64_t s = base + tid;
    const int e = s < s1 ? idx[s] : -1;
    uint64_t same = __ballot(e >= 0);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t b = __ballot(on);
      same &= on ? b : ~b;
    }
    const int rank = __popcll(same & lower);
    __syncthreads();  // wcnt cleared, run up to date
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (e >= 0) {
      int pos = run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      perm[pos] = static_cast<int32_t>(s);
      inv[s] = pos;
      if (rscale) rperm[pos] = rscale[s / k];
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += 256) run[ee] += wcnt[0][ee] + wcnt[1][ee] + wcnt[2][ee] + wcnt[3][ee];
    __syncthreads();  // wcnt is read above before the next round clears it
  }
}

}  // namespace

hipError_t launch_permute(const Plan &p, const int32_t *topk_idx, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  const unsigned nblk = static_cast<unsigned>(p.n_perm_blocks);
  hipLaunchKernelGGL(perm_hist, dim3(nblk), dim3(256), 0, s, topk_idx, p.S, c.E, p.blk_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(256), 0, s, p.blk_counts, static_cast<int>(nblk), c.E,
                     p.S, c.T, c.F_shared > 0 ? 1 : 0, p.tile_m, p.tile_balanced, p.blk_base, p.counts, p.offsets,
                     p.tiles, p.tile_count);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (streaming_path(p.path)) {
    err = launch_stream_schedule(p, s);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(perm_scatter, dim3(nblk), dim3(256), 0, s, topk_idx, p.S, c.E, p.blk_base,
                     p.perm, p.inv, p.rscale, c.k, p.rperm);
  return hipGetLastError();
}

}  // namespace moe
