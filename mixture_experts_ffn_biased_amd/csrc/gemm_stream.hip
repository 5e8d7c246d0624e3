// Grouped expert GEMMs on gfx950 for bf16 layers: persistent, XCD-aware,
// weight-streaming kernels.
//
// Same two products and epilogues as grouped_gemm.hip (the SwiGLU expert of
// "Sparse MoE FFN" (DeepSeek-V3), "How it works", or the GEGLU and biased
// GELU-MLP bodies, batched as grouped GEMMs as "Mixture of experts and
// architecture families", "The router and load balancing", suggests); only
// the schedule and the data movement differ:
//
//  * One workgroup per CU loops over work items (tile, n-slab).  Items are
//    kept in eight per-XCD lists: a chunk (up to eight tiles of one expert)
//    goes to one XCD with all its n-slabs, the tiles of a chunk adjacent.
//    Workgroups of an XCD take items from their list in order through an
//    atomic counter, so the workgroups running together on an XCD share the
//    expert's token rows and weight slabs in that XCD's L2, and each weight
//    byte is fetched from HBM about once.  A workgroup whose list is empty
//    takes items from the other XCDs' lists.
//  * Each stage is a K-slice of 32 of the tile's token rows and 256 weight
//    rows, staged by direct global-to-LDS 16-byte loads into rings of
//    separate LDS slots; three stages are in flight while one is multiplied;
//    no VGPR staging.
//  * Prefill variant: 256-row tiles, 8 waves in a 2x4 grid (two per SIMD, one
//    from each row half), each 128 x 64 of v_mfma_f32_32x32x16_bf16 with fp32
//    accumulators.  A wave multiplies only the 32-row blocks that hold rows
//    of the tile (its K loop is specialised on that count), so a SIMD's MFMA
//    work follows the tile's row count.
//    - First product (gathered token rows): the pair ring.  Token slots hold
//      two stages (64 K values, 128 B a row), so a 1 KiB load covers 8 rows
//      x 128 B, whole cache lines of the gathered rows; 3 token slots and 4
//      weight slots fill the 160 KiB of LDS.  Loads go through buffer
//      resources, so the K loop adds only scalar offsets; weight loads carry
//      the non-temporal hint.
//    - Second product: the stage ring (4 slots of 32 KiB) over H, which the
//      first product writes tile-blocked: a tile's rows K-slice by K-slice,
//      each slice's nrows x 32 values contiguous (same size as row-major),
//      so each 16-row token load is one contiguous KiB.
//  * Decode variant (few rows per expert): 32-row tiles, 4 waves each 32 x 64,
//    an 8-slot stage ring (7 x 16 KB of weights in flight): a weight stream
//    with a small MFMA on the side.  Each slab is read once there, so its
//    loads carry the non-temporal hint.
//  * gate_up of the gated bodies: each wave column's 64 weight rows are 32
//    rows of W1 then the same 32 of W3, so act(x W1^T) * (x W3^T) meets in
//    the same lane; the bf16 result goes through LDS to 16-byte stores.  The
//    GELU MLP's gate_up is a single product like down (256 W1 rows a slab),
//    with bias and GELU in the epilogue.
//  * Weights are read either in their plain [rows][K] layout or packed once
//    (moe_pack_weights) so that each stage's 16 KB weight tile is contiguous
//    in memory in exactly the order it lands in LDS.
#include "common.hpp"
#include "pipeline.hpp"
#include "plan.hpp"

#include <type_traits>

namespace moe {
namespace {

constexpr int SBK = 32;            // K per stage
constexpr int SBN = 256;           // weight rows per stage
constexpr int B_BYTES = SBN * SBK * 2;
constexpr int B_STAGE_ELEMS = SBN * SBK;  // packed: elements per weight stage block

template <int VAR>
struct V;
template <>
struct V<0> {  // prefill (stage ring: NSTAGE slots; pair ring: PA_LOADS token loads a pair)
  static constexpr int BM = 256, NT = 512, NSTAGE = 4, A_LOADS = 2, B_LOADS = 2, PA_LOADS = 4;
};
template <>
struct V<1> {  // decode
  static constexpr int BM = 32, NT = 256, NSTAGE = 8, A_LOADS = 1, B_LOADS = 4;
};
constexpr int SBKA = 64;                       // prefill: K of a token slot
constexpr int A_SLOT_BYTES = 256 * SBKA * 2;   // 32 KiB
template <int VAR>
constexpr int a_bytes() { return V<VAR>::BM * SBK * 2; }
template <int VAR>
constexpr int stage_bytes() { return a_bytes<VAR>() + B_BYTES; }

// The epilogue kind names the product: the gated or GELU first product
// (gathered token rows in, H out) or the plain or biased second one (H in).
// In the prefill variant the first product runs the pair ring (whole cache
// lines of the gathered rows) and writes H tile-blocked; the second reads
// that layout through the stage ring, one contiguous KiB a load.
template <int EPI, int VAR>
constexpr bool pair_ring() {
  return VAR == 0 && (EPI == EPI_SILU_GLU || EPI == EPI_GELU_GLU || EPI == EPI_BIAS_GELU);
}
template <int EPI, int VAR>
constexpr bool writes_blocked() {
  return pair_ring<EPI, VAR>();
}
template <int EPI, int VAR>
constexpr bool reads_blocked() {
  return VAR == 0 && (EPI == EPI_PLAIN || EPI == EPI_BIAS);
}
// Element offset of H[row][col] of a tile (first row row0, nrows rows) whose
// rows are `ld` values long, in the tile-blocked layout: K-slice by K-slice
// (32 values), each slice's nrows x 32 values contiguous.
__device__ __forceinline__ int64_t blocked_off(int64_t row0, int nrows, int ld, int row, int col) {
  return row0 * ld + static_cast<int64_t>(col / SBK) * nrows * SBK + row * SBK + (col % SBK);
}

struct StreamArgs {
  const Tile *tiles;
  const int2 *items;        // per-XCD segments of {tile id, n-slab}
  const int32_t *xcd_off;   // [8] segment starts
  const int32_t *xcd_cnt;   // [8] segment lengths
  int32_t *counters;        // [8] zero on entry
  const int32_t *perm;      // gate_up: position -> slot
  int64_t a_rows;           // rows of the (ungathered) token matrix: T for gate_up
  int k;
  int E;
  const void *A_routed, *A_shared;
  int gather;
  const void *B0_routed, *B1_routed, *B0_shared, *B1_shared;  // plain layout
  const void *Bp_routed, *Bp_shared;  // packed layout: stage blocks of each slab
  int N_routed, N_shared, K_routed, K_shared;
  void *C_routed, *C_shared;
  const void *bias_routed;  // [E][N] or null (EPI_BIAS, EPI_BIAS_GELU)
  const void *bias_shared;  // [N] or null
  // Row scales of the gated first product (fused pre-norm block): the 1/rms
  // of the row's token at each routed position ([S] + one tile of padding)
  // and of each token for the shared expert ([T] + padding); null: none.
  const float *rs_routed, *rs_shared;
};

template <int NS>
struct Ring {
  unsigned char *s[NS];
};

// Stage-ring DMA sources of one thread (scalar members, not arrays, so that
// no private array is ever demoted to memory).  The prefill variant (second
// product) reads its token operand, the tile's block of H, through a buffer
// resource: ar, lane offsets ao0/ao1, bytes a_ks from one stage to the next;
// the decode variant through the pointer a0.
struct Ptrs {
  const uint16_t *a0, *a1;
  int a_ks;   // token-operand elements (decode) or bytes (prefill) from one stage to the next
  __amdgpu_buffer_rsrc_t ar;
  uint32_t ao0, ao1;
  int alive;  // bit i: token load i has a row of the tile (wave-uniform)
  // Prefill weight operand: a buffer resource over the packed slab or the
  // expert's matrix, lane offsets bo0/bo1, bytes b_ks from one stage to the next.
  __amdgpu_buffer_rsrc_t br;
  uint32_t bo0, bo1;
  int b_ks;
  __device__ __forceinline__ uint32_t ao(int i) const { return i == 0 ? ao0 : ao1; }
  __device__ __forceinline__ uint32_t bo(int i) const { return i == 0 ? bo0 : bo1; }
  const uint16_t *b0, *b1, *b2, *b3;
  __device__ __forceinline__ const uint16_t *a(int i) const { return i == 0 ? a0 : a1; }
  __device__ __forceinline__ const uint16_t *b(int i) const {
    return i == 0 ? b0 : (i == 1 ? b1 : (i == 2 ? b2 : b3));
  }
  __device__ __forceinline__ void set_a(int i, const uint16_t *v) {
    if (i == 0) a0 = v; else a1 = v;
  }
  __device__ __forceinline__ void set_b(int i, const uint16_t *v) {
    if (i == 0) b0 = v; else if (i == 1) b1 = v; else if (i == 2) b2 = v; else b3 = v;
  }
};

// The last R stages of an item (R in [NS-1, 2NS-2]), all slot indices
// static: iteration i consumes slot i % NS, refills while stages remain, and
// waits until at most the later stages already issued are outstanding.
template <int NS, int PS, int R, int I>
struct Rem {
  template <class Issue, class Compute>
  __device__ __forceinline__ static void run(const Ring<NS> &ring, int base, Issue &issue, Compute &compute) {
    constexpr int LATER = (NS - 2) < (R - 1 - I) ? (NS - 2) : (R - 1 - I);
    wait_vmcnt<LATER * PS>();
    raw_barrier();
    if (I < R - NS + 1) issue(ring.s[(I + NS - 1) % NS], base + I + NS - 1);
    compute(ring.s[I % NS]);
    Rem<NS, PS, R, I + 1>::run(ring, base, issue, compute);
  }
};
template <int NS, int PS, int R>
struct Rem<NS, PS, R, R> {
  template <class Issue, class Compute>
  __device__ __forceinline__ static void run(const Ring<NS> &, int, Issue &, Compute &) {}
};

// The stage ring's K loop (the decode variant, and the prefill variant's
// second product): NS slots, each a whole stage (token rows and weight rows
// of one K-slice of 32).  Every wave issues the same loads and barriers
// whatever its NMI, so waves with different row counts stay in step.
template <bool PACKED, int VAR, int NMI>
__device__ __forceinline__ void kloop(const Ring<V<VAR>::NSTAGE> &ring, const Ptrs &p, int KT,
                                      int wave, int lane, int wm, int wn, int fo0, int fo1,
                                      f32x16 (&acc)[4][2]) {
  constexpr int NS = V<VAR>::NSTAGE;
  constexpr int PS = V<VAR>::A_LOADS + V<VAR>::B_LOADS;  // loads per wave per stage
  constexpr int AB = a_bytes<VAR>();
  auto issue = [&](unsigned char *st, int kt) __attribute__((always_inline)) {
    const int koff = kt * SBK;
    if (VAR == 0) {
      // A load whose 16 rows all lie past the tile's rows reads the
      // zero-length resource: the same count of loads, no memory traffic.
#pragma unroll
      for (int i = 0; i < V<VAR>::A_LOADS; ++i)
        dma16_buf(((p.alive >> i) & 1) ? p.ar : buffer_rsrc(nullptr, 0), p.ao(i), kt * p.a_ks,
                  st + (wave * 2 + i) * 1024);
    } else {
      // 32 rows: each wave loads 8 rows with its first 32 lanes.
      if (lane < 32) dma16(p.a(0) + koff, st + wave * 512);
    }
    if (VAR == 0) {
#pragma unroll
      for (int i = 0; i < V<VAR>::B_LOADS; ++i)
        dma16_buf(p.br, p.bo(i), kt * p.b_ks, st + AB + (wave * V<VAR>::B_LOADS + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < V<VAR>::B_LOADS; ++i) {
        const uint16_t *src = PACKED ? p.b(i) + static_cast<int64_t>(kt) * B_STAGE_ELEMS : p.b(i) + koff;
        // Each weight slab is read once at decode sizes: a non-temporal load
        // keeps the stream from evicting the token rows and the router's
        // operands (the weights of the layer exceed the last-level cache).
        dma16<kLoadNonTemporal>(src, st + AB + (wave * V<VAR>::B_LOADS + i) * 1024);
      }
    }
  };
  auto compute = [&](const unsigned char *st) __attribute__((always_inline)) {
    if (NMI == 0) return;
    const unsigned char *sa = st + wm * 128 * 64;
    const unsigned char *sb = st + AB + wn * 64 * 64;
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
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) issue(ring.s[i], i);
  // Stage kt lives in slot kt % NS (unrolled by NS: static slot indices).  It
  // is complete once at most the NS-2 later stages are outstanding; after
  // the barrier, stage kt+NS-1 refills the slot of stage kt-1.  G full turns
  // of the ring issue a stage every iteration; the last R stages follow.
  const int G = (KT - NS + 1) / NS;
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      wait_vmcnt<(NS - 2) * PS>();
      raw_barrier();
      issue(ring.s[(s + NS - 1) % NS], j * NS + s + NS - 1);
      compute(ring.s[s]);
    }
  }
  // K is a multiple of NS stages (the plan guarantees it), so R == NS.
  Rem<NS, PS, NS, 0>::run(ring, G * NS, issue, compute);
}

// ---- prefill K loop ----------------------------------------------------------

// Prefill DMA sources: buffer resources (scalar registers; stage offsets go
// in the scalar offset) plus 32-bit per-lane byte offsets, so the K loop
// does no per-lane address arithmetic.  Each resource spans exactly its
// operand, so no load can leave it.
struct PPtrs {
  __amdgpu_buffer_rsrc_t ar;  // token operand: the token matrix
  int astep;                  // bytes from one 64-wide K-slice to the next
  int alive;                  // bit j: token load j has a row of the tile (wave-uniform)
  uint32_t ao0, ao1, ao2, ao3;
  __amdgpu_buffer_rsrc_t br0, br1;  // weight operand, per load
  int bstep;                        // bytes from one stage to the next
  uint32_t bo0, bo1;
  __device__ __forceinline__ uint32_t ao(int j) const {
    return j == 0 ? ao0 : (j == 1 ? ao1 : (j == 2 ? ao2 : ao3));
  }
  __device__ __forceinline__ void set_ao(int j, uint32_t v) {
    if (j == 0) ao0 = v; else if (j == 1) ao1 = v; else if (j == 2) ao2 = v; else ao3 = v;
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t br(int i) const { return i == 0 ? br0 : br1; }
  __device__ __forceinline__ uint32_t bo(int i) const { return i == 0 ? bo0 : bo1; }
};

// Token load j of wave w fills rows (4w + j) * 8 + l/8 of a token slot, lane
// l in physical chunk l%8, which holds logical chunk (l%8) ^ ((row >> 1) & 7).  A
// weight load fills 16 rows of 64 B: lane l in row +l/4, physical chunk l%4,
// holding logical chunk (l%4) ^ ((row>>2)&3).
template <int EPI, bool PACKED>
__device__ __forceinline__ PPtrs prefill_ptrs(const StreamArgs &g, const Tile &tl, bool shared, int slab_y, int N,
                                              int K, int KT, int n0, int wave, int lane) {
  constexpr bool DUAL = epi_dual(EPI);
  PPtrs p{};
  const char *A = static_cast<const char *>(shared ? g.A_shared : g.A_routed);
  p.ar = buffer_rsrc(A, static_cast<uint32_t>(g.a_rows * K * 2));
  p.astep = SBKA * 2;
  p.alive = 0;
#pragma unroll
  for (int j = 0; j < V<0>::PA_LOADS; ++j)
    if ((wave * V<0>::PA_LOADS + j) * 8 < tl.nrows) p.alive |= 1 << j;
#pragma unroll
  for (int j = 0; j < V<0>::PA_LOADS; ++j) {
    const int r = (wave * V<0>::PA_LOADS + j) * 8 + (lane >> 3);
    const int rr = r < tl.nrows ? r : 0;  // rows past the count read row 0 (never stored)
    const uint32_t chunk = static_cast<uint32_t>(((lane & 7) ^ ((r >> 1) & 7)) * 16);
    const int64_t arow = (g.gather && !shared) ? g.perm[tl.row0 + rr] / g.k : static_cast<int64_t>(tl.row0) + rr;
    p.set_ao(j, static_cast<uint32_t>(arow * K * 2) + chunk);
  }
  if (PACKED) {
    // The slab's stage blocks are contiguous: block kt at kt * B_STAGE_ELEMS,
    // load i of wave w at (w * B_LOADS + i) KiB in the block, lane at 16 B.
    const char *Bp = static_cast<const char *>(shared ? g.Bp_shared : g.Bp_routed);
    const int nslab = DUAL ? N / (SBN / 2) : N / SBN;
    const int64_t slab = (shared ? 0 : static_cast<int64_t>(tl.group) * nslab) + slab_y;
    const uint32_t slab_bytes = static_cast<uint32_t>(KT * B_STAGE_ELEMS * 2);
    p.br0 = p.br1 = buffer_rsrc(Bp + slab * slab_bytes, slab_bytes);
    p.bo0 = static_cast<uint32_t>((wave * V<0>::B_LOADS + 0) * 1024 + lane * 16);
    p.bo1 = p.bo0 + 1024;
    p.bstep = B_STAGE_ELEMS * 2;
  } else {
    const char *B0 = static_cast<const char *>(shared ? g.B0_shared : g.B0_routed);
    const char *B1 = static_cast<const char *>(shared ? g.B1_shared : g.B1_routed);
    const int64_t es = static_cast<int64_t>(N) * K * 2;  // one expert's matrix
    if (!shared) {
      B0 += tl.group * es;
      if (DUAL) B1 += tl.group * es;
    }
#pragma unroll
    for (int i = 0; i < V<0>::B_LOADS; ++i) {
      // rb: the load's first row (uniform); its 16 rows lie in one 32-row
      // half of a wave column, so W1 or W3 is a per-load choice.
      const int rb = (wave * V<0>::B_LOADS + i) * 16;
      const int r = rb + (lane >> 2);
      const uint32_t c = static_cast<uint32_t>((lane & 3) ^ ((r >> 2) & 3));
      const char *base = B0;
      int brow;
      if (DUAL) {
        // 64 rows per wave column: 32 of W1, then the same 32 of W3.
        brow = n0 + (rb >> 6) * 32 + (rb & 31) + (lane >> 2);
        if ((rb & 63) >= 32) base = B1;
      } else {
        brow = n0 + r;
      }
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, static_cast<uint32_t>(es));
      const uint32_t off = static_cast<uint32_t>(static_cast<int64_t>(brow) * K * 2) + c * 16;
      if (i == 0) {
        p.br0 = rs;
        p.bo0 = off;
      } else {
        p.br1 = rs;
        p.bo1 = off;
      }
    }
    p.bstep = SBK * 2;
  }
  return p;
}

// Token slots hold 256 rows x 64 K values (128 B a row), so one 1 KiB load
// covers 8 rows x 128 B, whole cache lines of the gathered token rows, where
// 32-wide slices would cover 16 half lines; weight slots hold one stage, 256
// rows x 32 K values, as in the stage ring.  Row r of a token slot keeps its
// logical 16-byte chunk c in physical chunk c ^ ((r >> 1) & 7): the LDS's 64
// banks span 256 bytes, two slot rows, and a 16-byte read serves 16 lanes a
// cycle, so the 16 rows a fragment read's lane group touches (8 row pairs)
// must put one chunk in 8 different bank groups of each row parity.
struct PRing {
  unsigned char *a0, *a1, *a2;
  unsigned char *b0, *b1, *b2, *b3;
};
template <int I>
__device__ __forceinline__ unsigned char *pa(const PRing &r) {
  return I == 0 ? r.a0 : (I == 1 ? r.a1 : r.a2);
}
template <int I>
__device__ __forceinline__ unsigned char *pb(const PRing &r) {
  return I == 0 ? r.b0 : (I == 1 ? r.b1 : (I == 2 ? r.b2 : r.b3));
}

// Stages base + I .. base + 11 of one turn, statically unrolled: token slot
// (I/2) % 3, weight slot I % 4 (base is a multiple of 12), so every slot
// index is a constant.  Iteration t issues token pair t/2 + 2 when t is
// even, then weight stage t + 3: loads that would lie past K go to a
// zero-length buffer (they read zeros, touch no memory and land in a slot
// no later stage reads), so every iteration issues the same loads, the
// issue is never conditional, and the wait is the same 8 loads each time:
// stage t's weights were the last load of iteration t-3 (after its token
// pair), its token pair went out earlier still, and iterations t-2 and t-1
// issued 4 + 2 + 2 loads.  Whole turns run without a stage-count check, so
// their loop has a single back edge; the last, partial turn (GUARD) checks
// the count and otherwise runs the same code.
template <int I, bool GUARD>
struct PStep {
  template <class IA, class IB, class C>
  __device__ __forceinline__ static void run(const PRing &ring, int base, int KT, IA &ia, IB &ib, C &c) {
    const int t = base + I;
    if (GUARD && t >= KT) return;
    wait_vmcnt<8>();
    raw_barrier();
    if (I % 2 == 0) ia(pa<(I / 2 + 2) % 3>(ring), t / 2 + 2, t + 4 < KT);
    ib(pb<(I + 3) % 4>(ring), t + 3, t + 3 < KT);
    c(pa<(I / 2) % 3>(ring), I & 1, pb<I % 4>(ring));
    PStep<I + 1, GUARD>::run(ring, base, KT, ia, ib, c);
  }
};
template <bool GUARD>
struct PStep<12, GUARD> {
  template <class IA, class IB, class C>
  __device__ __forceinline__ static void run(const PRing &, int, int, IA &, IB &, C &) {}
};

// K loop of one first-product prefill item (pair ring) for a wave with NMI
// active 32-row blocks (KT a multiple of 4).  Every wave issues the same loads and barriers whatever its
// NMI, so waves with different row counts stay in step.
template <bool PACKED, int NMI>
__device__ __forceinline__ void kloop_prefill(const PRing &ring, const PPtrs &p, int KT, int wave, int wm,
                                              int wn, int xa, int fo0, int fo1, f32x16 (&acc)[4][2]) {
  const __amdgpu_buffer_rsrc_t none = buffer_rsrc(nullptr, 0);
  // A load whose 8 rows all lie past the tile's rows reads the zero-length
  // resource too: the same count of loads, no memory traffic.
  auto issue_a = [&](unsigned char *st, int q, bool real) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < V<0>::PA_LOADS; ++j)
      dma16_buf(real && ((p.alive >> j) & 1) ? p.ar : none, p.ao(j), q * p.astep,
                st + (wave * V<0>::PA_LOADS + j) * 1024);
  };
  // A weight slab is read by the tiles of its chunk (up to eight), close
  // together in time, while the gathered token rows are read again by the
  // other slab items of their tile and by other experts' tiles: the slab
  // loads carry the non-temporal hint so that the weight stream does not push
  // the token rows out of the cache.
  auto issue_b = [&](unsigned char *st, int kt, bool real) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < V<0>::B_LOADS; ++i)
      dma16_buf<kLoadNonTemporal>(real ? p.br(i) : none, p.bo(i), kt * p.bstep,
                                  st + (wave * V<0>::B_LOADS + i) * 1024);
  };
  // half: which 32 of the token slot's 64 K values this stage multiplies.
  auto compute = [&](const unsigned char *sta, int half, const unsigned char *stb) __attribute__((always_inline)) {
    if (NMI == 0) return;
    const unsigned char *sa = sta + wm * 128 * (SBKA * 2);
    const unsigned char *sb = stb + wn * 64 * (SBK * 2);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int foa = xa ^ ((half * 4 + kk * 2) << 4);
      const int fob = kk ? fo1 : fo0;
      bf16x8 a[NMI > 0 ? NMI : 1], b[2];
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) a[mi] = *reinterpret_cast<const bf16x8 *>(sa + mi * 32 * (SBKA * 2) + foa);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) b[ni] = *reinterpret_cast<const bf16x8 *>(sb + ni * 2048 + fob);
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  };
  // Iterations -4 .. -1 of the pattern: pairs 0 and 1, stages 0 .. 2 (KT >= 4).
  issue_a(ring.a0, 0, true);
  issue_b(ring.b0, 0, true);
  issue_a(ring.a1, 1, true);
  issue_b(ring.b1, 1, true);
  issue_b(ring.b2, 2, true);
  const int G = KT / 12;
  for (int j = 0; j < G; ++j) PStep<0, false>::run(ring, 12 * j, KT, issue_a, issue_b, compute);
  if (12 * G < KT) PStep<0, true>::run(ring, 12 * G, KT, issue_a, issue_b, compute);
  // The loads past K may still be landing in slots the epilogue stages in.
  wait_vmcnt<0>();
}

template <int EPI, bool PACKED, int VAR, class RingT>
__device__ __forceinline__ void run_item(const StreamArgs &g, int2 item, const RingT &ring) {
  constexpr int BM = V<VAR>::BM, NT = V<VAR>::NT;
  constexpr bool DUAL = epi_dual(EPI);
  const Tile tl = g.tiles[item.x];
  const bool shared = tl.group == g.E;
  const int N = shared ? g.N_shared : g.N_routed;
  const int K = shared ? g.K_shared : g.K_routed;
  const int KT = K / SBK;
  const int n0 = item.y * (DUAL ? SBN / 2 : SBN);
  const int tid = threadIdx.x, lane = tid & 63;
  // Wave-uniform by construction; readfirstlane lets the compiler keep it and
  // every LDS slot address derived from it in SGPRs (the DMA's M0 operand).
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = VAR == 0 ? wave >> 2 : 0, wn = VAR == 0 ? (wave & 3) : wave;

  // DMA sources: the pair ring's (PPtrs), or 64-bit pointers per lane for
  // the stage ring.
  constexpr bool PAIR = pair_ring<EPI, VAR>();
  Ptrs p{};
  PPtrs pp{};
  if constexpr (PAIR) {
    pp = prefill_ptrs<EPI, PACKED>(g, tl, shared, item.y, N, K, KT, n0, wave, lane);
  } else {
    const uint16_t *A = static_cast<const uint16_t *>(shared ? g.A_shared : g.A_routed);
    auto a_row = [&](int r) -> const uint16_t * {
      const int rr = r < tl.nrows ? r : 0;  // rows past the count read row 0 (never stored)
      if (reads_blocked<EPI, VAR>()) return A + blocked_off(tl.row0, tl.nrows, K, rr, 0);
      const int64_t arow =
          (g.gather && !shared) ? g.perm[tl.row0 + rr] / g.k : static_cast<int64_t>(tl.row0) + rr;
      return A + arow * K;
    };
    // A token load fills 16 rows (8 in the decode variant, its first 32
    // lanes) of 64 B: lane l in row +l/4, physical chunk l%4, holding logical
    // chunk (l%4) ^ ((row>>2)&3).
    if constexpr (VAR == 0) {
      static_assert(reads_blocked<EPI, VAR>(), "the prefill stage ring reads tile-blocked H");
      // The tile's block of H: stage kt at kt * nrows * 64 bytes, row r at r * 64.
      p.ar = buffer_rsrc(A + static_cast<int64_t>(tl.row0) * K, static_cast<uint32_t>(tl.nrows * K * 2));
      p.a_ks = tl.nrows * SBK * 2;
      p.alive = 0;
#pragma unroll
      for (int i = 0; i < V<VAR>::A_LOADS; ++i) {
        const int r = (wave * 2 + i) * 16 + (lane >> 2);
        const int rr = r < tl.nrows ? r : 0;  // rows past the count read row 0 (never stored)
        const uint32_t off = static_cast<uint32_t>(rr * SBK * 2 + (((lane & 3) ^ ((r >> 2) & 3)) << 4));
        if (i == 0) p.ao0 = off; else p.ao1 = off;
        if ((wave * 2 + i) * 16 < tl.nrows) p.alive |= 1 << i;
      }
    } else {
      p.a_ks = SBK;
      const int r = wave * 8 + ((lane & 31) >> 2);
      p.set_a(0, a_row(r) + ((lane & 3) ^ ((r >> 2) & 3)) * 8);
    }
    if constexpr (VAR == 0) {
      // The prefill second product (256 W2 rows a slab, no W3).
      static_assert(!DUAL, "the prefill stage ring runs the second product");
      if (PACKED) {
        const char *Bp = static_cast<const char *>(shared ? g.Bp_shared : g.Bp_routed);
        const int64_t slab = (shared ? 0 : static_cast<int64_t>(tl.group) * (N / SBN)) + item.y;
        const uint32_t slab_bytes = static_cast<uint32_t>(KT * B_STAGE_ELEMS * 2);
        p.br = buffer_rsrc(Bp + slab * slab_bytes, slab_bytes);
        p.bo0 = static_cast<uint32_t>((wave * V<VAR>::B_LOADS + 0) * 1024 + lane * 16);
        p.bo1 = p.bo0 + 1024;
        p.b_ks = B_STAGE_ELEMS * 2;
      } else {
        const int64_t es = static_cast<int64_t>(N) * K * 2;  // one expert's matrix, bytes
        const char *B0 = static_cast<const char *>(shared ? g.B0_shared : g.B0_routed);
        if (!shared) B0 += tl.group * es;
        p.br = buffer_rsrc(B0, static_cast<uint32_t>(es));
#pragma unroll
        for (int i = 0; i < V<VAR>::B_LOADS; ++i) {
          const int r = (wave * V<VAR>::B_LOADS + i) * 16 + (lane >> 2);
          const uint32_t off = static_cast<uint32_t>(static_cast<int64_t>(n0 + r) * K * 2 +
                                                     (((lane & 3) ^ ((r >> 2) & 3)) << 4));
          if (i == 0) p.bo0 = off; else p.bo1 = off;
        }
        p.b_ks = SBK * 2;
      }
    } else if (PACKED) {
      // The slab's stage blocks are contiguous: block kt at kt * B_STAGE_ELEMS,
      // load i of wave w at (w * B_LOADS + i) KiB in the block, lane at 16 B.
      const uint16_t *Bp = static_cast<const uint16_t *>(shared ? g.Bp_shared : g.Bp_routed);
      const int nslab = DUAL ? N / (SBN / 2) : N / SBN;
      const int64_t slab = (shared ? 0 : static_cast<int64_t>(tl.group) * nslab) + item.y;
      const uint16_t *blk = Bp + slab * KT * B_STAGE_ELEMS;
#pragma unroll
      for (int i = 0; i < V<VAR>::B_LOADS; ++i) p.set_b(i, blk + (wave * V<VAR>::B_LOADS + i) * 512 + lane * 8);
    } else {
      const uint16_t *B0 = static_cast<const uint16_t *>(shared ? g.B0_shared : g.B0_routed);
      const uint16_t *B1 = static_cast<const uint16_t *>(shared ? g.B1_shared : g.B1_routed);
      if (!shared) {
        const int64_t es = static_cast<int64_t>(N) * K;
        B0 += tl.group * es;
        if (DUAL) B1 += tl.group * es;
      }
#pragma unroll
      for (int i = 0; i < V<VAR>::B_LOADS; ++i) {
        const int r = (wave * V<VAR>::B_LOADS + i) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
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
        p.set_b(i, bsrc + brow * K + c * 8);
      }
    }
  }

  const int sw = (lane >> 2) & 3;
  const int fo0 = (lane & 31) * 64 + (((0 + (lane >> 5)) ^ sw) << 4);
  const int fo1 = (lane & 31) * 64 + (((2 + (lane >> 5)) ^ sw) << 4);
  // Prefill token fragment: row lane%32 (so (row >> 1) & 7 == (lane >> 1) & 7),
  // logical chunk 4 * half + 2 * kk + lane/32; the K loop XORs in the static part.
  const int xa = (lane & 31) * (SBKA * 2) + (((lane >> 5) ^ ((lane >> 1) & 7)) << 4);

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
  const int nmi = VAR == 0 ? __builtin_amdgcn_readfirstlane((rows_here + 31) >> 5) : 1;

  // Row scale of this thread's row of the tile (gated first product of the
  // fused pre-norm block), loaded now and staged for the epilogue after the
  // K loop; rows past the tile read the buffer's padding and are never stored.
  const float *rs_src = DUAL ? (shared ? g.rs_shared : g.rs_routed) : nullptr;
  float my_rs = 1.f;
  if (rs_src && tid < tl.nrows) my_rs = rs_src[tl.row0 + tid];

  // The previous item's stores and loads are complete before the ring refills.
  wait_vmcnt<0>();
  raw_barrier();
  if constexpr (PAIR) {
    switch (nmi) {
      case 0: kloop_prefill<PACKED, 0>(ring, pp, KT, wave, wm, wn, xa, fo0, fo1, acc); break;
      case 1: kloop_prefill<PACKED, 1>(ring, pp, KT, wave, wm, wn, xa, fo0, fo1, acc); break;
      case 2: kloop_prefill<PACKED, 2>(ring, pp, KT, wave, wm, wn, xa, fo0, fo1, acc); break;
      case 3: kloop_prefill<PACKED, 3>(ring, pp, KT, wave, wm, wn, xa, fo0, fo1, acc); break;
      default: kloop_prefill<PACKED, 4>(ring, pp, KT, wave, wm, wn, xa, fo0, fo1, acc); break;
    }
  } else if constexpr (VAR == 0) {
    switch (nmi) {
      case 0: kloop<PACKED, VAR, 0>(ring, p, KT, wave, lane, wm, wn, fo0, fo1, acc); break;
      case 1: kloop<PACKED, VAR, 1>(ring, p, KT, wave, lane, wm, wn, fo0, fo1, acc); break;
      case 2: kloop<PACKED, VAR, 2>(ring, p, KT, wave, lane, wm, wn, fo0, fo1, acc); break;
      case 3: kloop<PACKED, VAR, 3>(ring, p, KT, wave, lane, wm, wn, fo0, fo1, acc); break;
      default: kloop<PACKED, VAR, 4>(ring, p, KT, wave, lane, wm, wn, fo0, fo1, acc); break;
    }
  } else {
    kloop<PACKED, VAR, 1>(ring, p, KT, wave, lane, wm, wn, fo0, fo1, acc);
  }
  // Every wave is done reading the ring before it is reused for the output.
  raw_barrier();

  // Epilogue: each quad of lanes transposes its 4 x 4 blocks (rows 8a + b of
  // four consecutive columns) so that a lane writes 4 columns of one row, 8
  // bytes, into the staging slots; the 16-byte chunk index of a staged row is
  // XOR-swizzled with row & 7 so the rows of a block land in different banks.
  const int row_lane = 4 * (lane >> 5);
  const int jq = lane & 3;
  const int rq = quad_transpose_row(jq);
  const int cq = (lane & 31) & ~3;  // first of the quad's columns within a 32-column block
  auto staged = [](int row, int col, int row_bytes) {
    return row * row_bytes + (((col >> 3) ^ (row & 7)) << 4) + (col & 7) * 2;
  };
  uint16_t *C = static_cast<uint16_t *>(shared ? g.C_shared : g.C_routed);
  // Tile-blocked copy-out of rows staged RS to a slot, 512 / 256 bytes a row
  // (RB): a wave writes 16 rows x 64 B of one 32-column slice, one contiguous
  // KiB; the 8 lanes of a bank group read 8 different rows.
  const int bsub = lane >> 4;
  auto copy_blocked = [&](const unsigned char *slot, int rf, auto rs, auto rb) __attribute__((always_inline)) {
    constexpr int RS = decltype(rs)::value, RB = decltype(rb)::value;
    constexpr int NSL = RB / (SBK * 2);  // 32-column slices in a staged row
    constexpr int WPS = RS / 16;         // waves covering one slice of the slot
    constexpr int SPP = 8 / WPS;         // slices per pass
#pragma unroll
    for (int j = 0; j < NSL / SPP; ++j) {
      const int q = j * SPP + wave / WPS;
      const int rl = (wave % WPS) * 16 + (lane & 15);
      const int row = rf + rl;
      if (row < tl.nrows)
        *reinterpret_cast<uint4 *>(C + blocked_off(tl.row0, tl.nrows, N, row, n0 + q * SBK + bsub * 8)) =
            *reinterpret_cast<const uint4 *>(slot + staged(rl, q * SBK + bsub * 8, RB));
    }
  };
  // Row-major copy-out: TPR threads of 16 B a row.
  auto copy_rows = [&](const unsigned char *slot, int rf, auto rs, auto rb) __attribute__((always_inline)) {
    constexpr int RS = decltype(rs)::value, RB = decltype(rb)::value;
    constexpr int TPR = RB / 16, RPP = NT / TPR;  // threads a row, rows a pass
#pragma unroll
    for (int j = 0; j < RS / RPP; ++j) {
      const int rl = j * RPP + tid / TPR, ch = tid % TPR;
      const int row = rf + rl;
      if (row < tl.nrows)
        *reinterpret_cast<uint4 *>(C + (static_cast<int64_t>(tl.row0) + row) * N + n0 + ch * 8) =
            *reinterpret_cast<const uint4 *>(slot + staged(rl, ch * 8, RB));
    }
  };
  using I32 = std::integral_constant<int, 32>;
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using I256 = std::integral_constant<int, 256>;
  using I512 = std::integral_constant<int, 512>;
  if (DUAL) {
    // H tile: BM rows x 128 columns bf16 (256 bytes a row), 128 rows a slot
    // (pair ring: token slots 0 and 1; stage ring: slots 0 and 1, the
    // decode tile's 32 rows in slot 0).  Row scales: weight slot 0 (pair
    // ring) or slot 2 (stage ring).
    unsigned char *Ht;
    float *rs_lds;
    if constexpr (PAIR) {
      Ht = wm ? ring.a1 : ring.a0;
      rs_lds = reinterpret_cast<float *>(ring.b0);
    } else {
      Ht = wm ? ring.s[1] : ring.s[0];
      rs_lds = reinterpret_cast<float *>(ring.s[2]);
    }
    if (rs_src) {
      if (tid < BM) rs_lds[tid] = my_rs;
      __syncthreads();
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi >= nmi) break;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float f[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float a1 = acc[mi][0][4 * a + b];
          float a3 = acc[mi][1][4 * a + b];
          if (rs_src) {
            // accumulator 4a + b is row 8a + 4 (lane / 32) + b of block mi of
            // this wave's half of the tile (rows wm * 128 ..)
            const float r = rs_lds[wm * 128 + mi * 32 + 8 * a + row_lane + b];
            a1 *= r;
            a3 *= r;
          }
          f[b] = (EPI == EPI_GELU_GLU ? gelu(a1) : silu_fast(a1)) * a3;
        }
        const int row = mi * 32 + 8 * a + row_lane + rq;
        *reinterpret_cast<uint2 *>(Ht + staged(row, wn * 32 + cq, 256)) = quad_transpose_bf16(f, jq);
      }
    }
    __syncthreads();
    if constexpr (PAIR) {
      copy_blocked(ring.a0, 0, I128{}, I256{});
      copy_blocked(ring.a1, 128, I128{}, I256{});
    } else {
      copy_rows(ring.s[0], 0, std::integral_constant<int, (BM < 128 ? BM : 128)>{}, I256{});
      if (BM > 128) copy_rows(ring.s[1], 128, I128{}, I256{});
    }
    __syncthreads();
  } else {
    // Output tile: BM x 256 bf16 (512 bytes a row).  Pair ring: 32-row
    // blocks 0-1, 2-3 and 4-5 in token slots 0, 1 and 2 (64 rows each),
    // blocks 6 and 7 in weight slots 0 and 1.  Stage ring: 64 rows a slot
    // (the decode tile's 32 rows in slot 0).
    float bv[2] = {0.f, 0.f};
    if (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) {
      const uint16_t *bias = static_cast<const uint16_t *>(shared ? g.bias_shared : g.bias_routed);
      if (bias) {
        if (!shared) bias += static_cast<int64_t>(tl.group) * N;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) bv[ni] = bf16_to_f32(bias[n0 + wn * 64 + ni * 32 + (lane & 31)]);
      }
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi >= nmi) break;
      unsigned char *Ot;
      int rbase = (mi & 1) * 32;
      if constexpr (PAIR) {
        if (wm == 0) {
          Ot = mi < 2 ? ring.a0 : ring.a1;
        } else {
          Ot = mi < 2 ? ring.a2 : (mi == 2 ? ring.b0 : ring.b1);
          if (mi >= 2) rbase = 0;
        }
      } else {
        Ot = wm ? (mi < 2 ? ring.s[2] : ring.s[3]) : (mi < 2 ? ring.s[0] : ring.s[1]);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float f[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            float v = acc[mi][ni][4 * a + b];
            if (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) v += bv[ni];
            if (EPI == EPI_BIAS_GELU) v = gelu(v);
            f[b] = v;
          }
          const int row = rbase + 8 * a + row_lane + rq;
          *reinterpret_cast<uint2 *>(Ot + staged(row, wn * 64 + ni * 32 + cq, 512)) = quad_transpose_bf16(f, jq);
        }
    }
    __syncthreads();
    // Copy-out region by region, each slot named statically (a runtime
    // choice among the slot pointers would make the compiler keep them in
    // memory).
    if constexpr (PAIR) {
      copy_blocked(ring.a0, 0, I64{}, I512{});
      copy_blocked(ring.a1, 64, I64{}, I512{});
      copy_blocked(ring.a2, 128, I64{}, I512{});
      copy_blocked(ring.b0, 192, I32{}, I512{});
      copy_blocked(ring.b1, 224, I32{}, I512{});
    } else if constexpr (BM > 64) {
      copy_rows(ring.s[0], 0, I64{}, I512{});
      copy_rows(ring.s[1], 64, I64{}, I512{});
      copy_rows(ring.s[2], 128, I64{}, I512{});
      copy_rows(ring.s[3], 192, I64{}, I512{});
    } else {
      copy_rows(ring.s[0], 0, std::integral_constant<int, BM>{}, I512{});
    }
    __syncthreads();
  }
}

// The ring is idle between items, so the fetched item index is broadcast
// through the first word of a slot.
template <int EPI, bool PACKED, int VAR, class RingT>
__device__ __forceinline__ void item_loop(const StreamArgs &g, const RingT &ring, int *item_sh) {
  const int xcd = blockIdx.x & 7;
  for (int o = 0; o < 8; ++o) {
    const int x = (xcd + o) & 7;
    const int cnt = g.xcd_cnt[x];
    const int off = g.xcd_off[x];
    for (;;) {
      if (threadIdx.x == 0) *item_sh = atomicAdd(&g.counters[x], 1);
      __syncthreads();
      const int it = __builtin_amdgcn_readfirstlane(*item_sh);
      __syncthreads();
      if (it >= cnt) break;
      run_item<EPI, PACKED, VAR>(g, g.items[off + it], ring);
    }
  }
}

// Separate __shared__ ring slots: the compiler can then tell the LDS loads
// into one slot from the reads of another and adds no waits of its own.
template <int EPI, bool PACKED>
__global__ __launch_bounds__(512, 1) void gemm_stream_prefill(StreamArgs g) {
  if constexpr (pair_ring<EPI, 0>()) {
    // 3 x 32 KiB token slots + 4 x 16 KiB weight slots: the whole 160 KiB.
    __shared__ __attribute__((aligned(16))) unsigned char a0[A_SLOT_BYTES], a1[A_SLOT_BYTES], a2[A_SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char b0[B_BYTES], b1[B_BYTES], b2[B_BYTES], b3[B_BYTES];
    PRing ring{a0, a1, a2, b0, b1, b2, b3};
    item_loop<EPI, PACKED, 0>(g, ring, reinterpret_cast<int *>(a0));
  } else {
    constexpr int SB = stage_bytes<0>();
    __shared__ __attribute__((aligned(16))) unsigned char r0[SB], r1[SB], r2[SB], r3[SB];
    Ring<4> ring;
    ring.s[0] = r0;
    ring.s[1] = r1;
    ring.s[2] = r2;
    ring.s[3] = r3;
    item_loop<EPI, PACKED, 0>(g, ring, reinterpret_cast<int *>(r0));
  }
}

template <int EPI, bool PACKED>
__global__ __launch_bounds__(256, 1) void gemm_stream_decode(StreamArgs g) {
  constexpr int SB = stage_bytes<1>();
  __shared__ __attribute__((aligned(16))) unsigned char r0[SB], r1[SB], r2[SB], r3[SB], r4[SB], r5[SB],
      r6[SB], r7[SB];
  Ring<8> ring;
  ring.s[0] = r0;
  ring.s[1] = r1;
  ring.s[2] = r2;
  ring.s[3] = r3;
  ring.s[4] = r4;
  ring.s[5] = r5;
  ring.s[6] = r6;
  ring.s[7] = r7;
  item_loop<EPI, PACKED, 1>(g, ring, reinterpret_cast<int *>(r0));
}

// ---- one-time weight packing -------------------------------------------------

// Packed layout, for one matrix kind (gate_up: W1 and W3 together; down: W2)
// of one expert: slabs of 256 weight rows in order, each slab its K/32 stage
// blocks in order, each block 256 rows x 64 bytes exactly as the rows land in
// LDS: row r, physical 16-byte chunk p holds k-chunk p ^ ((r>>2)&3) of the
// K-slice; for gate_up, row r is W1 row slab*128 + (r/64)*32 + r%32 when
// r%64 < 32 and the same row of W3 otherwise.
// g (the fused pre-norm block's RMSNorm weight, [K]; null: none): each value
// is multiplied by g of its column, the fp32 product (exact for two bf16
// values) rounded once to bf16, nearest even.
__global__ __launch_bounds__(256) void pack_weights(const uint16_t *__restrict__ W1,
                                                    const uint16_t *__restrict__ W3, int dual,
                                                    int64_t n_mats, int rows, int K,
                                                    const uint16_t *__restrict__ g,
                                                    uint16_t *__restrict__ out) {
  const int KT = K / SBK;
  const int nslab = dual ? rows / (SBN / 2) : rows / SBN;
  const int64_t per_mat = static_cast<int64_t>(nslab) * KT * (B_BYTES / 16);
  const int64_t total = n_mats * per_mat;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < total;
       q += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t e = q / per_mat;
    int64_t rem = q - e * per_mat;
    const int chunk = static_cast<int>(rem % (B_BYTES / 16));  // 16-byte chunk in the block
    rem /= (B_BYTES / 16);
    const int kt = static_cast<int>(rem % KT);
    const int slab = static_cast<int>(rem / KT);
    const int r = chunk >> 2, pch = chunk & 3;
    const int c = pch ^ ((r >> 2) & 3);
    const uint16_t *src;
    int64_t row;
    if (dual) {
      const int qq = r & 63;
      row = static_cast<int64_t>(slab) * 128 + (r >> 6) * 32 + (qq & 31);
      src = qq < 32 ? W1 : W3;
    } else {
      row = static_cast<int64_t>(slab) * SBN + r;
      src = W1;
    }
    const int k0 = kt * SBK + c * 8;
    const uint16_t *from = src + (e * rows + row) * K + k0;
    uint4 v = *reinterpret_cast<const uint4 *>(from);
    if (g) v = scale_bf16x8(v, *reinterpret_cast<const uint4 *>(g + k0));
    *reinterpret_cast<uint4 *>(out + q * 8) = v;
  }
}

// Router rows folded with the RMSNorm weight for the fused pre-norm block:
// out[e][j] = bf16(W[e][j] * g[j]), as in pack_weights; 8 values a thread.
__global__ __launch_bounds__(256) void fold_rows(const uint16_t *__restrict__ W, const uint16_t *__restrict__ g,
                                                 int64_t rows, int K, uint16_t *__restrict__ out) {
  const int64_t n = rows * K / 8;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < n;
       q += static_cast<int64_t>(gridDim.x) * 256) {
    const int k0 = static_cast<int>((q * 8) % K);
    const uint4 v = *reinterpret_cast<const uint4 *>(W + q * 8);
    *reinterpret_cast<uint4 *>(out + q * 8) = scale_bf16x8(v, *reinterpret_cast<const uint4 *>(g + k0));
  }
}

// ---- schedule: per-XCD item lists ------------------------------------------

constexpr int kMaxChunks = 4096;
// Tiles of one expert a chunk holds at most.  Whole experts of up to 8 tiles
// on one XCD: each slab is fetched once and read by all their tiles together.
constexpr int kChunkTiles = 8;
constexpr int kScheduleBlocks = 64;  // blocks of stream_schedule: 256 waves share out the chunks

// Rebuilds the tile numbering of perm_scan (experts in order, ceil(count /
// tile_m) tiles each, then the shared expert's tiles), groups tiles into
// chunks of up to kChunkTiles per expert, deals chunks to XCDs round-robin and writes
// both GEMMs' item lists (tile fastest, then n-slab, within a chunk).  Every
// block derives the same chunk table from the counts; the waves of all blocks
// then share out the chunks, a wave writing one chunk's run of items with
// contiguous stores, and block 0 writes the list offsets and counters.
__global__ __launch_bounds__(256) void stream_schedule(
    const int32_t *__restrict__ counts, int E, int64_t T, int has_shared, int tile_m, int nt_gu_r,
    int nt_gu_s,
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
  const int nt = (c + tile_m - 1) / tile_m;
  const int nch = (nt + kChunkTiles - 1) / kChunkTiles;
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
    cfirst[chunk_off + j] = tile_off + kChunkTiles * j;
    cmt[chunk_off + j] = static_cast<unsigned char>(nt - kChunkTiles * j < kChunkTiles ? nt - kChunkTiles * j : kChunkTiles);
  }
  int n_chunks = routed_chunks;
  if (has_shared) {
    const int ns = static_cast<int>((T + tile_m - 1) / tile_m);
    const int nsc = (ns + kChunkTiles - 1) / kChunkTiles;
    for (int j = tid; j < nsc; j += 256) {
      cfirst[routed_chunks + j] = routed_tiles + kChunkTiles * j;
      cmt[routed_chunks + j] = static_cast<unsigned char>(ns - kChunkTiles * j < kChunkTiles ? ns - kChunkTiles * j : kChunkTiles);
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
      if (blockIdx.x == 0) {
        meta[tid * 24 + x] = run;
        meta[tid * 24 + 8 + x] = xtot[tid][x];
        meta[tid * 24 + 16 + x] = 0;
      }
      run += xtot[tid][x];
    }
  }
  __syncthreads();
  // Item q = n * mt + m of a chunk is its tile m at n-slab n (mt is 1 or 2).
  const int lane = tid & 63;
  const int nwaves = static_cast<int>(gridDim.x) * 4;
  for (int ch = static_cast<int>(blockIdx.x) * 4 + (tid >> 6); ch < n_chunks; ch += nwaves) {
    const bool sh = ch >= routed_chunks;
    const int mt = cmt[ch];
    const int first = cfirst[ch];
    for (int list = 0; list < 2; ++list) {
      const int ntl = list == 0 ? (sh ? nt_gu_s : nt_gu_r) : (sh ? nt_dn_s : nt_dn_r);
      int2 *out = (list == 0 ? items_gu : items_dn) + xoff[list][ch & 7] + cpos[list][ch];
      for (int q = lane; q < ntl * mt; q += 64)
        out[q] = make_int2(first + q % mt, q / mt);
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

int stream_tile_m(int path) { return path == PATH_STREAM_DECODE ? V<1>::BM : V<0>::BM; }
// Prefill tiles of one expert get equal row counts (same tile count), so the
// tiles of a chunk, which share its weight slabs, run for the same time and
// read each slab together.
int stream_tile_balanced(int path) { return path == PATH_STREAM ? 1 : 0; }
int stream_max_chunks() { return kMaxChunks; }
// Gated bodies: 128 columns of W1 and W3 a slab; the GELU MLP: 256 of W1.
int stream_nslab_gate_up(int F, int kind) { return kind == MOE_EXPERT_GELU_MLP ? F / SBN : F / (SBN / 2); }
int stream_nslab_down(int d) { return d / SBN; }

// Packed regions: routed gate/up, routed down, shared gate/up, shared down.
// The gated bodies pack W1 and W3 together (2 F rows a matrix), the GELU MLP
// W1 alone (F rows, 256-row slabs like down).
size_t packed_weights_bytes(const moe_cfg &c, int kind) {
  const size_t g = kind == MOE_EXPERT_GELU_MLP ? 1 : 2;
  return 2ull * (g * c.E * c.F * c.d + static_cast<size_t>(c.E) * c.d * c.F + g * c.F_shared * c.d +
                 static_cast<size_t>(c.d) * c.F_shared);
}

PackedView packed_view(const moe_cfg &c, int kind, const void *base) {
  const size_t g = kind == MOE_EXPERT_GELU_MLP ? 1 : 2;
  const char *b = static_cast<const char *>(base);
  PackedView v;
  v.gu = b;
  v.dn = b + 2ull * g * c.E * c.F * c.d;
  v.gu_s = static_cast<const char *>(v.dn) + 2ull * c.E * c.d * c.F;
  v.dn_s = static_cast<const char *>(v.gu_s) + 2ull * g * c.F_shared * c.d;
  return v;
}

hipError_t launch_pack_weights(const moe_cfg &c, int kind, const void *W1, const void *W3, const void *W2,
                               const void *W1s, const void *W3s, const void *W2s, void *packed,
                               hipStream_t s, const void *norm_weight) {
  const PackedView v = packed_view(c, kind, packed);
  const int dual = kind == MOE_EXPERT_GELU_MLP ? 0 : 1;
  const uint16_t *g = static_cast<const uint16_t *>(norm_weight);
  auto run = [&](const void *a, const void *b, int du, int64_t n, int rows, int K, const uint16_t *gk,
                 const void *out) {
    const int64_t chunks = n * static_cast<int64_t>(rows) * K * (du ? 2 : 1) / 8;
    const unsigned blocks = static_cast<unsigned>(chunks / 256 < 65536 ? (chunks + 255) / 256 : 65536);
    hipLaunchKernelGGL(pack_weights, dim3(blocks), dim3(256), 0, s, static_cast<const uint16_t *>(a),
                       static_cast<const uint16_t *>(b), du, n, rows, K, gk,
                       static_cast<uint16_t *>(const_cast<void *>(out)));
    return hipGetLastError();
  };
  // The norm weight scales the inputs of the first product only (K = d).
  hipError_t e = run(W1, dual ? W3 : nullptr, dual, c.E, c.F, c.d, g, v.gu);
  if (e == hipSuccess) e = run(W2, nullptr, 0, c.E, c.d, c.F, nullptr, v.dn);
  if (e == hipSuccess && c.F_shared > 0)
    e = run(W1s, dual ? W3s : nullptr, dual, 1, c.F_shared, c.d, g, v.gu_s);
  if (e == hipSuccess && c.F_shared > 0) e = run(W2s, nullptr, 0, 1, c.d, c.F_shared, nullptr, v.dn_s);
  return e;
}

hipError_t launch_fold_rows(const void *W, const void *norm_weight, int64_t rows, int K, void *out, hipStream_t s) {
  const int64_t chunks = rows * K / 8;
  const unsigned blocks = static_cast<unsigned>(chunks / 256 < 65536 ? (chunks + 255) / 256 : 65536);
  hipLaunchKernelGGL(fold_rows, dim3(blocks), dim3(256), 0, s, static_cast<const uint16_t *>(W),
                     static_cast<const uint16_t *>(norm_weight), rows, K, static_cast<uint16_t *>(out));
  return hipGetLastError();
}

hipError_t launch_stream_schedule(const Plan &p, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  hipLaunchKernelGGL(stream_schedule, dim3(kScheduleBlocks), dim3(256), 0, s, p.counts, c.E, c.T,
                     c.F_shared > 0 ? 1 : 0,
                     p.tile_m, stream_nslab_gate_up(c.F, p.kind), stream_nslab_gate_up(c.F_shared, p.kind),
                     c.d / SBN, c.d / SBN, p.items_gu,
                     p.items_dn, p.sched_meta);
  return hipGetLastError();
}

typedef void (*stream_kernel_t)(StreamArgs);

// The kernel of one variant for an epilogue and weight layout.
template <int VAR>
static stream_kernel_t pick_kernel(int epi, bool packed) {
#define MOE_STREAM_K(E, P) (VAR == 0 ? gemm_stream_prefill<E, P> : gemm_stream_decode<E, P>)
  if (packed) {
    switch (epi) {
      case EPI_SILU_GLU: return MOE_STREAM_K(EPI_SILU_GLU, true);
      case EPI_GELU_GLU: return MOE_STREAM_K(EPI_GELU_GLU, true);
      case EPI_PLAIN: return MOE_STREAM_K(EPI_PLAIN, true);
      case EPI_BIAS: return MOE_STREAM_K(EPI_BIAS, true);
      case EPI_BIAS_GELU: return MOE_STREAM_K(EPI_BIAS_GELU, true);
      default: return nullptr;
    }
  }
  switch (epi) {
    case EPI_SILU_GLU: return MOE_STREAM_K(EPI_SILU_GLU, false);
    case EPI_GELU_GLU: return MOE_STREAM_K(EPI_GELU_GLU, false);
    case EPI_PLAIN: return MOE_STREAM_K(EPI_PLAIN, false);
    case EPI_BIAS: return MOE_STREAM_K(EPI_BIAS, false);
    case EPI_BIAS_GELU: return MOE_STREAM_K(EPI_BIAS_GELU, false);
    default: return nullptr;
  }
#undef MOE_STREAM_K
}

static hipError_t launch_stream(const Plan &p, const StreamArgs &a, int epi, bool packed, hipStream_t s) {
  const bool decode = p.path == PATH_STREAM_DECODE;
  const stream_kernel_t k = decode ? pick_kernel<1>(epi, packed) : pick_kernel<0>(epi, packed);
  if (!k) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(num_cus())), dim3(decode ? V<1>::NT : V<0>::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_gate_up(const Plan &p, const void *u, const Experts &x, const PackedView *pk,
                                 hipStream_t s) {
  const moe_cfg &c = p.cfg;
  const int epi = gate_up_epi(p.kind);
  const bool dual = epi_dual(epi);
  StreamArgs a = base_args(p, 0);
  a.A_routed = u;
  a.A_shared = u;
  a.a_rows = c.T;
  a.gather = 1;
  a.B0_routed = x.W1;
  a.B1_routed = dual ? x.W3 : nullptr;
  a.B0_shared = x.W1s;
  a.B1_shared = dual ? x.W3s : nullptr;
  a.Bp_routed = pk ? pk->gu : nullptr;
  a.Bp_shared = pk ? pk->gu_s : nullptr;
  a.bias_routed = x.b1;
  a.bias_shared = x.b1s;
  a.N_routed = c.F;
  a.N_shared = c.F_shared;
  a.K_routed = c.d;
  a.K_shared = c.d;
  a.C_routed = p.H;
  a.C_shared = p.Hs;
  a.rs_routed = p.rperm;  // null unless the plan is the fused pre-norm block's
  a.rs_shared = p.rscale;
  return launch_stream(p, a, epi, pk != nullptr, s);
}

hipError_t launch_stream_down(const Plan &p, const Experts &x, const PackedView *pk, hipStream_t s) {
  const moe_cfg &c = p.cfg;
  StreamArgs a = base_args(p, 1);
  a.A_routed = p.H;
  a.A_shared = p.Hs;
  a.gather = 0;
  a.B0_routed = x.W2;
  a.B1_routed = nullptr;
  a.B0_shared = x.W2s;
  a.B1_shared = nullptr;
  a.Bp_routed = pk ? pk->dn : nullptr;
  a.Bp_shared = pk ? pk->dn_s : nullptr;
  a.bias_routed = x.b2;
  a.bias_shared = x.b2s;
  a.N_routed = c.d;
  a.N_shared = c.d;
  a.K_routed = c.F;
  a.K_shared = c.F_shared;
  a.C_routed = p.O;
  a.C_shared = p.Z;
  return launch_stream(p, a, down_epi(p.kind), pk != nullptr, s);
}

}  // namespace moe
