// Host-side plan of one layer call: validated sizes, the carve-up of the
// caller's workspace, and the launchers of the five stages.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// One row block of the grouped GEMMs: `nrows` consecutive rows starting at
// row `row0` of expert `group` (group == E: the shared expert, whose rows are
// the tokens themselves).
struct Tile {
  int32_t group;
  int32_t row0;
  int32_t nrows;
  int32_t pad;
};

// Row range of tile i of the nt = ceil(c / tile_m) tiles over c rows.
// balanced 0: tiles of tile_m rows, the last one ragged; balanced 1: the rows
// spread evenly (sizes differ by at most one), so tiles that share weight
// slabs carry the same work.
__host__ __device__ inline void tile_rows(int64_t c, int nt, int i, int tile_m, int balanced, int64_t *r0,
                                          int *n) {
  if (!balanced) {
    *r0 = static_cast<int64_t>(i) * tile_m;
    *n = static_cast<int>(c - *r0 < tile_m ? c - *r0 : tile_m);
  } else {
    const int64_t base = c / nt, rem = c % nt;
    *r0 = i * base + (i < rem ? i : rem);
    *n = static_cast<int>(base + (i < rem ? 1 : 0));
  }
}

constexpr int kPermChunk = 1024;  // slots per block in the permutation kernels
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 32;
constexpr int kMaxGroups = 64;

// Which grouped-GEMM kernels run the experts.
enum GemmPath {
  PATH_TILED = 0,          // grouped_gemm.hip: 128-row tiles (fp32 too), any size multiple of 64
  PATH_STREAM = 1,         // gemm_stream.hip prefill variant: 256-row tiles
  PATH_STREAM_DECODE = 2,  // gemm_stream.hip decode variant: 32-row tiles, deep weight ring
  PATH_SMALL = 3,          // small_layer.hip: the whole small fp32 SwiGLU layer in one kernel
};

inline bool streaming_path(int path) { return path == PATH_STREAM || path == PATH_STREAM_DECODE; }

// Limits of the one-kernel small layer (fp32, SwiGLU): routed slots, d, F and F_shared.
constexpr int kSmallMaxSlots = 512;
constexpr int kSmallMaxD = 1024;
constexpr int kSmallMaxF = 1024;

// Expert weights of one call in the plain layout and the body they form
// (moe_expert_kind).  W3 / W3s are unused by the GELU MLP; b1, b2, b1s, b2s
// are its biases in the layer dtype (null: zero) and null for the gated kinds.
struct Experts {
  int kind;
  const void *W1, *W3, *W2, *b1, *b2;
  const void *W1s, *W3s, *W2s, *b1s, *b2s;
};

// Epilogue of a grouped-GEMM tile.  The gated gate_up products hold two
// accumulators (W1 and W3 rows); the others one, plus an optional bias row
// of the group ([N] in the layer dtype, null: zero).
enum Epi {
  EPI_SILU_GLU = 0,   // SiLU(a1) * a3
  EPI_GELU_GLU = 1,   // GELU(a1) * a3
  EPI_PLAIN = 2,      // a
  EPI_BIAS = 3,       // a + bias[col]
  EPI_BIAS_GELU = 4,  // GELU(a + bias[col])
};
__host__ __device__ constexpr bool epi_dual(int epi) { return epi <= EPI_GELU_GLU; }
inline int gate_up_epi(int kind) {
  return kind == MOE_EXPERT_GELU_MLP ? EPI_BIAS_GELU : (kind == MOE_EXPERT_GEGLU ? EPI_GELU_GLU : EPI_SILU_GLU);
}
inline int down_epi(int kind) { return kind == MOE_EXPERT_GELU_MLP ? EPI_BIAS : EPI_PLAIN; }

// Device views of the four regions of a packed weight buffer.
struct PackedView {
  const void *gu;    // routed W1/W3 stage blocks
  const void *dn;    // routed W2
  const void *gu_s;  // shared W1/W3
  const void *dn_s;  // shared W2
};

struct Plan {
  moe_cfg cfg;
  int kind;         // moe_expert_kind
  int path;         // GemmPath
  int64_t S;        // routed slots, T*k
  int tile_m;       // rows per grouped-GEMM tile (at most)
  int tile_balanced;  // tile_rows rule
  int router_splits;    // K splits of the router GEMM (1 = fused with selection)
  float *router_part;   // [router_splits][T][E] partial logits when router_splits > 1
  int64_t n_perm_blocks;
  int64_t max_tiles;
  // workspace carve-up (device pointers; null when only sizing)
  int32_t *blk_counts;  // [n_perm_blocks][E]
  int32_t *blk_base;    // [n_perm_blocks][E]
  int32_t *counts;      // [E]
  int32_t *offsets;     // [E+1]
  int32_t *perm;        // [S]  slot at each expert-contiguous position
  int32_t *inv;         // [S]  position of each slot
  Tile *tiles;          // [max_tiles]
  int32_t *tile_count;  // [1]
  int2 *items_gu;       // PATH_STREAM: per-XCD work lists of the gate/up GEMM
  int2 *items_dn;       //              and of the down GEMM
  int32_t *sched_meta;  //              [2][3][8] list offsets, lengths, counters
  int64_t max_items_gu, max_items_dn;
  void *H;              // [S][F]        hidden activations of each routed slot
  void *Hs;             // [T][F_shared] same for the shared expert
  void *O;              // [S][d]        expert output of each routed slot
  void *Z;              // [T][d]        shared expert output (layer dtype)
  // Fused pre-norm block (fused_norm): the router sums each token's squares
  // (part_sq), router_select stores 1/rms (rscale), the permutation copies it
  // to each routed row's position (rperm), and the gate/up epilogue scales
  // the accumulators of that row by it.  Null otherwise.
  int fused_norm;
  float norm_eps;
  float *part_sq;       // [router_splits][T]
  float *rscale;        // [T] (+ one tile of padding)
  float *rperm;         // [S] (+ one tile of padding)
  size_t bytes;
};

moe_status validate(const moe_cfg *c);
int router_splits(int64_t T, int d);
// Fills *p for experts of the given kind; base == nullptr computes only the
// size.  fused_norm: the plan of the fused pre-norm block (its router always
// takes the split-K pair and the plan carries the row-scale buffers).
void make_plan(const moe_cfg &c, int kind, void *base, Plan *p, int fused_norm = 0, float norm_eps = 0.f);

bool small_layer_fits(const moe_cfg &c, int kind);
hipError_t launch_small_layer(const Plan &p, const void *u, const void *W_router, const float *bias,
                              const Experts &x, const void *residual, void *y, int32_t *topk_idx, float *gates,
                              hipStream_t s);
hipError_t launch_router_topk(const Plan &p, const void *u, const void *Wr, const float *bias,
                              int32_t *topk_idx, float *gates, hipStream_t s);
hipError_t launch_permute(const Plan &p, const int32_t *topk_idx, hipStream_t s);
hipError_t launch_gate_up(const Plan &p, const void *u, const Experts &x, hipStream_t s);
hipError_t launch_down(const Plan &p, const Experts &x, hipStream_t s);
// residual: optional [T][d] in the layer dtype, added to y last (the block form).
hipError_t launch_combine(const Plan &p, const float *gates, const void *residual, void *y, hipStream_t s);
int rmsnorm_max_d();
hipError_t launch_rmsnorm(const void *h, const void *g, float eps, int64_t T, int d, int dtype, void *out,
                          hipStream_t s);

int stream_tile_m(int path);
int stream_max_chunks();
int stream_tile_balanced(int path);
int stream_nslab_gate_up(int F, int kind);
int stream_nslab_down(int d);
size_t packed_weights_bytes(const moe_cfg &c, int kind);
PackedView packed_view(const moe_cfg &c, int kind, const void *base);
// norm_weight (bf16 [d]; null: none): the fused pre-norm block's RMSNorm
// weight, folded into the first product's weights (W1, W3, W1s, W3s).
hipError_t launch_pack_weights(const moe_cfg &c, int kind, const void *W1, const void *W3, const void *W2,
                               const void *W1s, const void *W3s, const void *W2s, void *packed,
                               hipStream_t s, const void *norm_weight = nullptr);
// out [rows][K] = bf16(W * norm_weight[col]) (bf16, rows * K % 8 == 0).
hipError_t launch_fold_rows(const void *W, const void *norm_weight, int64_t rows, int K, void *out, hipStream_t s);
hipError_t launch_stream_schedule(const Plan &p, hipStream_t s);
// pk == nullptr: the plain weights of x; else the packed buffer's regions
// (x's weight pointers are not read; its biases are).
hipError_t launch_stream_gate_up(const Plan &p, const void *u, const Experts &x, const PackedView *pk,
                                 hipStream_t s);
hipError_t launch_stream_down(const Plan &p, const Experts &x, const PackedView *pk, hipStream_t s);

}  // namespace moe
