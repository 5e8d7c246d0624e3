// The C ABI of libmoe (declared in include/moe.h): validation, workspace
// carve-up, the five-stage launch sequence and optional per-stage timing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "plan.hpp"

namespace moe {

int gemm_tile_m(int dtype);
// balance.hip
hipError_t launch_balance_update(const int32_t *topk_idx, int64_t S, int E, float gamma, float *bias,
                                 int32_t *counts, float *entropy, hipStream_t s);

moe_status validate(const moe_cfg *c) {
  if (!c) return MOE_ERR_NULL;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_DTYPE;
  if (c->T < 0) return MOE_ERR_SHAPE;
  if (c->d <= 0 || c->d % 64 != 0) return MOE_ERR_SHAPE;
  if (c->F <= 0 || c->F % 64 != 0) return MOE_ERR_SHAPE;
  if (c->F_shared < 0 || c->F_shared % 64 != 0) return MOE_ERR_SHAPE;
  if (c->E < 1 || c->E > kMaxExperts) return MOE_ERR_SHAPE;
  if (c->k < 1 || c->k > c->E || c->k > kMaxTopK) return MOE_ERR_CFG;
  if (c->n_groups < 1 || c->n_groups > kMaxGroups || c->E % c->n_groups != 0) return MOE_ERR_CFG;
  if (c->topk_groups < 1 || c->topk_groups > c->n_groups) return MOE_ERR_CFG;
  if (c->n_groups > 1) {
    const int per = c->E / c->n_groups;
    if (per < 2 || c->k > c->topk_groups * per) return MOE_ERR_CFG;
  }
  if (!std::isfinite(c->route_scale)) return MOE_ERR_CFG;
  if (c->T * static_cast<int64_t>(c->k) > 0x7fffffffLL - 1024) return MOE_ERR_SHAPE;
  return MOE_OK;
}

static size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The streaming kernels need bf16 and whole 256-row weight slabs
// (d % 256, F % 128, F_shared % 128; the GELU MLP's single gate_up product
// F % 256, F_shared % 256).  With at least 64 routed rows per expert on
// average they run 256-row tiles (prefill); with fewer, 32-row tiles with a
// deeper weight ring (decode), which also needs F % 256 and F_shared % 256.
// Everything else takes the tiled kernels, except small fp32 SwiGLU layers,
// which run whole in one kernel (small_layer.hip).
static int choose_path(const moe_cfg &c, int kind) {
  if (small_layer_fits(c, kind)) return PATH_SMALL;
  if (c.dtype != MOE_BF16) return PATH_TILED;
  if (c.d % 256 != 0 || c.F % 128 != 0 || c.F_shared % 128 != 0) return PATH_TILED;
  if (kind == MOE_EXPERT_GELU_MLP && (c.F % 256 != 0 || c.F_shared % 256 != 0)) return PATH_TILED;
  const int64_t S = c.T * c.k;
  int path = PATH_STREAM;
  if (S < 64LL * c.E) {
    if (c.F % 256 != 0 || c.F_shared % 256 != 0) return PATH_TILED;
    path = PATH_STREAM_DECODE;
  }
  // The prefill variant addresses the token matrix and one expert's weight
  // matrix with 32-bit byte offsets from their starts.
  const int64_t f_max = c.F > c.F_shared ? c.F : c.F_shared;
  if (path == PATH_STREAM && (c.T * c.d * 2 >= (1LL << 32) || f_max * c.d * 2 >= (1LL << 32))) return PATH_TILED;
  // A conservative bound on the schedule's chunks (the count chunks of at
  // most two tiles would reach; larger chunks make fewer).
  const int64_t m = stream_tile_m(path);
  const int64_t chunks = S / (2 * m) + c.E + c.T / (2 * m) + 4;
  if (chunks > stream_max_chunks()) return PATH_TILED;
  return path;
}

// Packed weights serve every T: both streaming variants read them.
static bool packable(const moe_cfg &c) {
  return c.dtype == MOE_BF16 && c.d % 256 == 0 && c.F % 256 == 0 && c.F_shared % 256 == 0;
}

static bool valid_kind(int kind) {
  return kind == MOE_EXPERT_SWIGLU || kind == MOE_EXPERT_GEGLU || kind == MOE_EXPERT_GELU_MLP;
}

void make_plan(const moe_cfg &c, int kind, void *base, Plan *p, int fused_norm, float norm_eps) {
  p->cfg = c;
  p->kind = kind;
  p->fused_norm = fused_norm;
  p->norm_eps = norm_eps;
  p->S = c.T * c.k;
  p->path = choose_path(c, kind);
  const bool streaming = streaming_path(p->path);
  p->tile_m = streaming ? stream_tile_m(p->path) : gemm_tile_m(c.dtype);
  p->tile_balanced = streaming ? stream_tile_balanced(p->path) : 0;
  p->router_splits = (c.dtype == MOE_BF16 && c.d % 128 == 0) ? router_splits(c.T, c.d) : 1;
  const bool split_pair = p->router_splits > 1 || fused_norm;  // logits kernel + router_select
  p->n_perm_blocks = (p->S + kPermChunk - 1) / kPermChunk;
  p->max_tiles = (p->S + p->tile_m - 1) / p->tile_m + c.E +
                 (c.F_shared > 0 ? (c.T + p->tile_m - 1) / p->tile_m : 0);
  const size_t es = c.dtype == MOE_BF16 ? 2 : 4;
  char *b = static_cast<char *>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void * {
    void *ptr = b ? b + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  p->router_part = static_cast<float *>(
      take(split_pair ? sizeof(float) * p->router_splits * c.T * c.E : 0));
  p->blk_counts = static_cast<int32_t *>(take(sizeof(int32_t) * p->n_perm_blocks * c.E));
  p->blk_base = static_cast<int32_t *>(take(sizeof(int32_t) * p->n_perm_blocks * c.E));
  p->counts = static_cast<int32_t *>(take(sizeof(int32_t) * c.E));
  p->offsets = static_cast<int32_t *>(take(sizeof(int32_t) * (c.E + 1)));
  p->perm = static_cast<int32_t *>(take(sizeof(int32_t) * p->S));
  p->inv = static_cast<int32_t *>(take(sizeof(int32_t) * p->S));
  p->tiles = static_cast<Tile *>(take(sizeof(Tile) * p->max_tiles));
  p->tile_count = static_cast<int32_t *>(take(sizeof(int32_t)));
  p->max_items_gu = p->max_items_dn = 0;
  if (streaming) {
    const int64_t nslab = stream_nslab_gate_up(c.F > c.F_shared ? c.F : c.F_shared, kind);
    p->max_items_gu = p->max_tiles * nslab;
    p->max_items_dn = p->max_tiles * stream_nslab_down(c.d);
  }
  p->items_gu = static_cast<int2 *>(take(sizeof(int2) * p->max_items_gu));
  p->items_dn = static_cast<int2 *>(take(sizeof(int2) * p->max_items_dn));
  p->sched_meta = static_cast<int32_t *>(take(sizeof(int32_t) * 48));
  p->H = take(es * p->S * c.F);
  p->Hs = take(es * c.T * c.F_shared);
  p->O = take(es * p->S * c.d);
  p->Z = take(c.F_shared > 0 ? es * c.T * c.d : 0);
  p->part_sq = p->rscale = p->rperm = nullptr;
  if (fused_norm) {
    p->part_sq = static_cast<float *>(take(sizeof(float) * p->router_splits * c.T));
    p->rscale = static_cast<float *>(take(sizeof(float) * (c.T + 256)));
    p->rperm = static_cast<float *>(take(sizeof(float) * (p->S + 256)));
  }
  p->bytes = off;
}

// ---- optional per-stage timing ----------------------------------------------

namespace {
struct Record {
  hipEvent_t ev[MOE_N_STAGES + 1];
};
std::mutex g_mu;
bool g_timing = false;
std::vector<Record> g_records;
constexpr size_t kMaxRecords = 100000;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_cfg *cfg) { return moe_workspace_bytes_ex(cfg, MOE_EXPERT_SWIGLU); }

size_t moe_workspace_bytes_ex(const moe_cfg *cfg, int32_t kind) {
  if (validate(cfg) != MOE_OK || !valid_kind(kind)) return 0;
  Plan p;
  make_plan(*cfg, kind, nullptr, &p);
  return p.bytes;
}

moe_status moe_check_cfg(const moe_cfg *cfg) { return validate(cfg); }

moe_status moe_plan_describe(const moe_cfg *cfg, int32_t *gemm_path, int32_t *tile_rows) {
  return moe_plan_describe_ex(cfg, MOE_EXPERT_SWIGLU, gemm_path, tile_rows);
}

moe_status moe_plan_describe_ex(const moe_cfg *cfg, int32_t kind, int32_t *gemm_path, int32_t *tile_rows) {
  const moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!valid_kind(kind)) return MOE_ERR_DTYPE;
  Plan p;
  make_plan(*cfg, kind, nullptr, &p);
  if (gemm_path) *gemm_path = p.path;
  if (tile_rows) *tile_rows = p.tile_m;
  return MOE_OK;
}

const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of the supported range";
    case MOE_ERR_CFG: return "inconsistent routing configuration";
    case MOE_ERR_DTYPE: return "unknown dtype or score function";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    default: return "unknown status";
  }
}

static moe_status prepare(const moe_cfg *cfg, int kind, void *workspace, size_t workspace_bytes, Plan *p) {
  Plan probe;
  make_plan(*cfg, kind, nullptr, &probe);
  if (!workspace) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < probe.bytes) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_ALIGN;
  make_plan(*cfg, kind, workspace, p);
  return MOE_OK;
}

// The token input and the outputs of a forward call.
static moe_status check_io(const void *u, const void *W_router, const moe_cfg *cfg, const void *y,
                           const int32_t *topk_idx, const float *gates) {
  if (!u || !W_router || !y || !topk_idx || !gates) return MOE_ERR_NULL;
  if (!aligned16(u) || !aligned16(W_router) || !aligned16(y)) return MOE_ERR_ALIGN;
  const size_t bytes = static_cast<size_t>(cfg->T) * cfg->d * (cfg->dtype == MOE_BF16 ? 2 : 4);
  const char *a = static_cast<const char *>(u);
  const char *b = static_cast<const char *>(y);
  if (a < b + bytes && b < a + bytes) return MOE_ERR_SHAPE;  // y aliases u
  return MOE_OK;
}

// Validation shared by the forward entry points; *p is filled on success.
static moe_status check_forward(const void *u, const void *W_router, const moe_cfg *cfg, int kind, const void *y,
                                const int32_t *topk_idx, const float *gates, void *workspace,
                                size_t workspace_bytes, Plan *p) {
  const moe_status st = check_io(u, W_router, cfg, y, topk_idx, gates);
  if (st != MOE_OK) return st;
  return prepare(cfg, kind, workspace, workspace_bytes, p);
}

// The SwiGLU experts of the plain entry points (shared may be null).
static Experts swiglu_experts(const void *W1, const void *W3, const void *W2, const moe_shared *shared) {
  Experts x{};
  x.kind = MOE_EXPERT_SWIGLU;
  x.W1 = W1;
  x.W3 = W3;
  x.W2 = W2;
  if (shared) {
    x.W1s = shared->W1;
    x.W3s = shared->W3;
    x.W2s = shared->W2;
  }
  return x;
}

// residual: nullptr for the layer, the block input h for the block form.
// pk: the packed buffer's regions (SwiGLU), or null for x's plain weights.
// timing: the per-stage timing hooks may run (they create HIP events while
// timing is enabled); the allocation-free entry point passes false.
static moe_status run_layer(const Plan &p, const void *u, const void *W_router, const float *bias,
                            const Experts &x, const PackedView *pk, void *y, int32_t *topk_idx, float *gates,
                            hipStream_t s, const void *residual = nullptr, bool timing = true) {
  (void)hipGetLastError();  // report only errors of the launches below
  Record rec{};
  bool timed = false;
  if (timing) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_timing && g_records.size() < kMaxRecords) {
      int made = 0;
      for (auto &e : rec.ev) {
        if (hipEventCreate(&e) != hipSuccess) break;
        ++made;
      }
      if (made != MOE_N_STAGES + 1) {
        for (int i = 0; i < made; ++i) (void)hipEventDestroy(rec.ev[i]);
        return MOE_ERR_HIP;
      }
      timed = true;
    }
  }
  auto mark = [&](int i) {
    if (timed) (void)hipEventRecord(rec.ev[i], s);
  };
  auto fail = [&]() {
    if (timed) {
      (void)hipStreamSynchronize(s);
      for (auto &e : rec.ev) (void)hipEventDestroy(e);
    }
    return MOE_ERR_HIP;
  };
  mark(0);
  if (p.path == PATH_SMALL) {
    // one kernel: its whole time is the first stage's
    if (launch_small_layer(p, u, W_router, bias, x, residual, y, topk_idx, gates, s) != hipSuccess) return fail();
    for (int i = 1; i <= MOE_N_STAGES; ++i) mark(i);
    if (timed) {
      std::lock_guard<std::mutex> lk(g_mu);
      g_records.push_back(rec);
    }
    return MOE_OK;
  }
  if (launch_router_topk(p, u, W_router, bias, topk_idx, gates, s) != hipSuccess) return fail();
  mark(1);
  if (launch_permute(p, topk_idx, s) != hipSuccess) return fail();
  mark(2);
  hipError_t err = p.path == PATH_TILED ? launch_gate_up(p, u, x, s) : launch_stream_gate_up(p, u, x, pk, s);
  if (err != hipSuccess) return fail();
  mark(3);
  err = p.path == PATH_TILED ? launch_down(p, x, s) : launch_stream_down(p, x, pk, s);
  if (err != hipSuccess) return fail();
  mark(4);
  if (launch_combine(p, gates, residual, y, s) != hipSuccess) return fail();
  mark(5);
  if (timed) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_records.push_back(rec);
  }
  return MOE_OK;
}

}  // extern "C"

// The plain SwiGLU weights of moe_layer_forward and its allocation-free twin
// (checked after cfg, for T > 0).
static moe_status check_plain_weights(const void *W1, const void *W3, const void *W2, const moe_shared *shared) {
  if (!W1 || !W3 || !W2) return MOE_ERR_NULL;
  if (shared && (!shared->W1 || !shared->W3 || !shared->W2)) return MOE_ERR_NULL;
  const void *ptrs[] = {W1, W3, W2, shared ? shared->W1 : W1, shared ? shared->W3 : W1,
                        shared ? shared->W2 : W1};
  for (const void *q : ptrs)
    if (!aligned16(q)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

extern "C" {

moe_status moe_layer_forward(const void *u, const void *W_router, const float *bias, const void *W1,
                             const void *W3, const void *W2, const moe_shared *shared,
                             const moe_cfg *cfg, void *y, int32_t *topk_idx, float *gates,
                             void *workspace, size_t workspace_bytes, void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if ((cfg->F_shared > 0) != (shared != nullptr)) return MOE_ERR_CFG;
  if (cfg->T == 0) return MOE_OK;
  st = check_plain_weights(W1, W3, W2, shared);
  if (st != MOE_OK) return st;
  Plan p;
  st = check_forward(u, W_router, cfg, MOE_EXPERT_SWIGLU, y, topk_idx, gates, workspace, workspace_bytes, &p);
  if (st != MOE_OK) return st;
  return run_layer(p, u, W_router, bias, swiglu_experts(W1, W3, W2, shared), nullptr, y, topk_idx, gates,
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- allocation-free forward -------------------------------------------------

namespace {
// The workspace of moe_layer_forward_noalloc: a fixed array in device memory,
// one copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only the
// address hipGetSymbolAddress returns for the current device is ever passed
// to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
moe_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const void *u, const void *W_router, const float *bias, const void *W1,
                                     const void *W3, const void *W2, const moe_shared *shared,
                                     const moe_cfg *cfg, void *y, int32_t *topk_idx, float *gates,
                                     void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if ((cfg->F_shared > 0) != (shared != nullptr)) return MOE_ERR_CFG;
  if (cfg->T == 0) return MOE_OK;
  st = check_plain_weights(W1, W3, W2, shared);
  if (st == MOE_OK) st = check_io(u, W_router, cfg, y, topk_idx, gates);
  if (st != MOE_OK) return st;
  // Argument errors and sizes beyond the array are reported before any HIP call.
  Plan probe;
  make_plan(*cfg, MOE_EXPERT_SWIGLU, nullptr, &probe);
  if (probe.bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  Plan p;
  st = check_forward(u, W_router, cfg, MOE_EXPERT_SWIGLU, y, topk_idx, gates, ws, MOE_NOALLOC_SCRATCH_BYTES, &p);
  if (st != MOE_OK) return st;
  // Every buffer the kernels read from the scratch is written earlier in the
  // same call (the GEMM work counters by the schedule kernel), so nothing is
  // cleared and nothing from an earlier call is read.
  return run_layer(p, u, W_router, bias, swiglu_experts(W1, W3, W2, shared), nullptr, y, topk_idx, gates,
                   static_cast<hipStream_t>(stream), nullptr, /*timing=*/false);
}

}  // extern "C"

// Checks an expert description against cfg and fills *x.  weights: its weight
// pointers are read (plain layout, or the source of a packing); otherwise
// only the kind and the biases are.
static moe_status check_experts(const moe_experts *experts, const moe_cfg *cfg, bool weights, Experts *x) {
  if (!experts) return MOE_ERR_NULL;
  const moe_experts &e = *experts;
  if (!valid_kind(e.kind)) return MOE_ERR_DTYPE;
  const bool gated = e.kind != MOE_EXPERT_GELU_MLP;
  const bool has_shared = cfg->F_shared > 0;
  if (weights && has_shared != (e.W1s || e.W3s || e.W2s)) return MOE_ERR_CFG;
  if (gated && (e.b1 || e.b2 || e.b1s || e.b2s)) return MOE_ERR_CFG;
  if (!has_shared && (e.b1s || e.b2s)) return MOE_ERR_CFG;
  *x = Experts{};
  x->kind = e.kind;
  x->b1 = e.b1;
  x->b2 = e.b2;
  x->b1s = e.b1s;
  x->b2s = e.b2s;
  if (weights) {
    if (!e.W1 || !e.W2 || (gated && !e.W3)) return MOE_ERR_NULL;
    if (has_shared && (!e.W1s || !e.W2s || (gated && !e.W3s))) return MOE_ERR_NULL;
    x->W1 = e.W1;
    x->W3 = gated ? e.W3 : nullptr;
    x->W2 = e.W2;
    x->W1s = e.W1s;
    x->W3s = gated ? e.W3s : nullptr;
    x->W2s = e.W2s;
  }
  const void *ptrs[] = {x->W1, x->W2, x->W3, x->b1, x->b2, x->W1s, x->W2s, x->W3s, x->b1s, x->b2s};
  for (const void *q : ptrs)
    if (q && !aligned16(q)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

extern "C" {

moe_status moe_layer_forward_ex(const void *u, const void *W_router, const float *bias,
                                const moe_experts *experts, const moe_cfg *cfg, void *y, int32_t *topk_idx,
                                float *gates, void *workspace, size_t workspace_bytes, void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  Experts x;
  st = check_experts(experts, cfg, cfg->T > 0, &x);
  if (st != MOE_OK || cfg->T == 0) return st;
  Plan p;
  st = check_forward(u, W_router, cfg, x.kind, y, topk_idx, gates, workspace, workspace_bytes, &p);
  if (st != MOE_OK) return st;
  return run_layer(p, u, W_router, bias, x, nullptr, y, topk_idx, gates, static_cast<hipStream_t>(stream));
}

moe_status moe_pack_weights_ex(const moe_cfg *cfg, const moe_experts *experts, void *packed, size_t packed_bytes,
                               void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  Experts x;
  st = check_experts(experts, cfg, true, &x);
  if (st != MOE_OK) return st;
  if (!packable(*cfg)) return MOE_ERR_SHAPE;
  if (!packed) return MOE_ERR_NULL;
  if (!aligned16(packed)) return MOE_ERR_ALIGN;
  if (packed_bytes < packed_weights_bytes(*cfg, x.kind)) return MOE_ERR_WORKSPACE;
  (void)hipGetLastError();
  if (launch_pack_weights(*cfg, x.kind, x.W1, x.W3, x.W2, x.W1s, x.W3s, x.W2s, packed,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_layer_forward_packed_ex(const void *u, const void *W_router, const float *bias,
                                       const moe_experts *experts, const void *packed, const moe_cfg *cfg, void *y,
                                       int32_t *topk_idx, float *gates, void *workspace, size_t workspace_bytes,
                                       void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  Experts x;
  st = check_experts(experts, cfg, false, &x);
  if (st != MOE_OK) return st;
  if (!packable(*cfg)) return MOE_ERR_SHAPE;
  if (cfg->T == 0) return MOE_OK;
  if (!packed) return MOE_ERR_NULL;
  if (!aligned16(packed)) return MOE_ERR_ALIGN;
  Plan p;
  st = check_forward(u, W_router, cfg, x.kind, y, topk_idx, gates, workspace, workspace_bytes, &p);
  if (st != MOE_OK) return st;
  if (!streaming_path(p.path)) return MOE_ERR_SHAPE;  // beyond the streaming kernels' limits
  const PackedView pk = packed_view(*cfg, x.kind, packed);
  return run_layer(p, u, W_router, bias, x, &pk, y, topk_idx, gates, static_cast<hipStream_t>(stream));
}

size_t moe_packed_weights_bytes(const moe_cfg *cfg) { return moe_packed_weights_bytes_ex(cfg, MOE_EXPERT_SWIGLU); }

size_t moe_packed_weights_bytes_ex(const moe_cfg *cfg, int32_t kind) {
  if (validate(cfg) != MOE_OK || !valid_kind(kind) || !packable(*cfg)) return 0;
  return packed_weights_bytes(*cfg, kind);
}

moe_status moe_pack_weights(const moe_cfg *cfg, const void *W1, const void *W3, const void *W2,
                            const moe_shared *shared, void *packed, size_t packed_bytes, void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!packable(*cfg)) return MOE_ERR_SHAPE;
  if ((cfg->F_shared > 0) != (shared != nullptr)) return MOE_ERR_CFG;
  if (!W1 || !W3 || !W2 || !packed) return MOE_ERR_NULL;
  if (shared && (!shared->W1 || !shared->W3 || !shared->W2)) return MOE_ERR_NULL;
  if (packed_bytes < packed_weights_bytes(*cfg, MOE_EXPERT_SWIGLU)) return MOE_ERR_WORKSPACE;
  const void *ptrs[] = {W1, W3, W2, packed, shared ? shared->W1 : W1, shared ? shared->W3 : W1,
                        shared ? shared->W2 : W1};
  for (const void *q : ptrs)
    if (!aligned16(q)) return MOE_ERR_ALIGN;
  (void)hipGetLastError();
  if (launch_pack_weights(*cfg, MOE_EXPERT_SWIGLU, W1, W3, W2, shared ? shared->W1 : nullptr,
                          shared ? shared->W3 : nullptr,
                          shared ? shared->W2 : nullptr, packed, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_layer_forward_packed(const void *u, const void *W_router, const float *bias,
                                    const void *packed, const moe_cfg *cfg, void *y, int32_t *topk_idx,
                                    float *gates, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!packable(*cfg)) return MOE_ERR_SHAPE;
  if (cfg->T == 0) return MOE_OK;
  if (!packed) return MOE_ERR_NULL;
  if (!aligned16(packed)) return MOE_ERR_ALIGN;
  Plan p;
  st = check_forward(u, W_router, cfg, MOE_EXPERT_SWIGLU, y, topk_idx, gates, workspace, workspace_bytes, &p);
  if (st != MOE_OK) return st;
  if (!streaming_path(p.path)) return MOE_ERR_SHAPE;  // beyond the streaming kernels' limits
  const PackedView pk = packed_view(*cfg, MOE_EXPERT_SWIGLU, packed);
  // The shared expert is present iff F_shared > 0 (the kernels read pk).
  return run_layer(p, u, W_router, bias, swiglu_experts(nullptr, nullptr, nullptr, nullptr), &pk, y, topk_idx,
                   gates, static_cast<hipStream_t>(stream));
}

// ---- pre-norm residual block ----------------------------------------------

static size_t elem_bytes(const moe_cfg &c) { return c.dtype == MOE_BF16 ? 2 : 4; }

// The larger of the two block forms' needs: the layer's buffers plus the
// normalised rows (unfused), or the layer's buffers with the row-scale
// buffers of the fused form.
size_t moe_block_workspace_bytes(const moe_cfg *cfg) {
  if (validate(cfg) != MOE_OK || cfg->d > rmsnorm_max_d()) return 0;
  Plan p, f;
  make_plan(*cfg, MOE_EXPERT_SWIGLU, nullptr, &p);
  make_plan(*cfg, MOE_EXPERT_SWIGLU, nullptr, &f, 1);
  const size_t unfused = p.bytes + align_up(static_cast<size_t>(cfg->T) * cfg->d * elem_bytes(*cfg));
  return unfused > f.bytes ? unfused : f.bytes;
}

moe_status moe_rmsnorm(const void *h, const void *norm_weight, float eps, int64_t T, int32_t d, int32_t dtype,
                       void *out, void *stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T < 0 || d <= 0 || d % 64 != 0 || d > rmsnorm_max_d()) return MOE_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.f) return MOE_ERR_CFG;
  if (T == 0) return MOE_OK;
  if (!h || !norm_weight || !out) return MOE_ERR_NULL;
  if (!aligned16(h) || !aligned16(norm_weight) || !aligned16(out)) return MOE_ERR_ALIGN;
  (void)hipGetLastError();
  if (launch_rmsnorm(h, norm_weight, eps, T, d, dtype, out, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

// Checks the norm arguments and the larger workspace of the block; *un is
// the normalised rows' place in the workspace (after the layer's buffers).
static moe_status block_setup(const void *norm_weight, float eps, const moe_cfg *cfg, const Plan &p,
                              void *workspace, size_t workspace_bytes, void **un) {
  if (!norm_weight) return MOE_ERR_NULL;
  if (!aligned16(norm_weight)) return MOE_ERR_ALIGN;
  if (!std::isfinite(eps) || eps < 0.f) return MOE_ERR_CFG;
  if (cfg->d > rmsnorm_max_d()) return MOE_ERR_SHAPE;
  if (workspace_bytes < moe_block_workspace_bytes(cfg)) return MOE_ERR_WORKSPACE;
  *un = static_cast<char *>(workspace) + p.bytes;
  return MOE_OK;
}

moe_status moe_block_forward(const void *h, const void *norm_weight, float norm_eps, const void *W_router,
                             const float *bias, const void *W1, const void *W3, const void *W2,
                             const moe_shared *shared, const moe_cfg *cfg, void *y, int32_t *topk_idx,
                             float *gates, void *workspace, size_t workspace_bytes, void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if ((cfg->F_shared > 0) != (shared != nullptr)) return MOE_ERR_CFG;
  if (cfg->T == 0) return MOE_OK;
  if (!W1 || !W3 || !W2) return MOE_ERR_NULL;
  if (shared && (!shared->W1 || !shared->W3 || !shared->W2)) return MOE_ERR_NULL;
  const void *ptrs[] = {W1, W3, W2, shared ? shared->W1 : W1, shared ? shared->W3 : W1,
                        shared ? shared->W2 : W1};
  for (const void *q : ptrs)
    if (!aligned16(q)) return MOE_ERR_ALIGN;
  Plan p;
  st = check_forward(h, W_router, cfg, MOE_EXPERT_SWIGLU, y, topk_idx, gates, workspace, workspace_bytes, &p);
  if (st != MOE_OK) return st;
  void *un = nullptr;
  st = block_setup(norm_weight, norm_eps, cfg, p, workspace, workspace_bytes, &un);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (launch_rmsnorm(h, norm_weight, norm_eps, cfg->T, cfg->d, cfg->dtype, un, s) != hipSuccess)
    return MOE_ERR_HIP;
  return run_layer(p, un, W_router, bias, swiglu_experts(W1, W3, W2, shared), nullptr, y, topk_idx, gates, s, h);
}

moe_status moe_block_forward_packed(const void *h, const void *norm_weight, float norm_eps, const void *W_router,
                                    const float *bias, const void *packed, const moe_cfg *cfg, void *y,
                                    int32_t *topk_idx, float *gates, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!packable(*cfg)) return MOE_ERR_SHAPE;
  if (cfg->T == 0) return MOE_OK;
  if (!packed) return MOE_ERR_NULL;
  if (!aligned16(packed)) return MOE_ERR_ALIGN;
  Plan p;
  st = check_forward(h, W_router, cfg, MOE_EXPERT_SWIGLU, y, topk_idx, gates, workspace, workspace_bytes, &p);
  if (st != MOE_OK) return st;
  if (!streaming_path(p.path)) return MOE_ERR_SHAPE;
  void *un = nullptr;
  st = block_setup(norm_weight, norm_eps, cfg, p, workspace, workspace_bytes, &un);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (launch_rmsnorm(h, norm_weight, norm_eps, cfg->T, cfg->d, cfg->dtype, un, s) != hipSuccess)
    return MOE_ERR_HIP;
  const PackedView pk = packed_view(*cfg, MOE_EXPERT_SWIGLU, packed);
  return run_layer(p, un, W_router, bias, swiglu_experts(nullptr, nullptr, nullptr, nullptr), &pk, y, topk_idx,
                   gates, s, h);
}

// ---- pre-norm block with the normalisation fused -----------------------------

size_t moe_block_packed_bytes(const moe_cfg *cfg) {
  if (validate(cfg) != MOE_OK || !packable(*cfg)) return 0;
  return packed_weights_bytes(*cfg, MOE_EXPERT_SWIGLU) + static_cast<size_t>(cfg->E) * cfg->d * 2;
}

moe_status moe_pack_block_weights(const moe_cfg *cfg, const void *norm_weight, const void *W_router, const void *W1,
                                  const void *W3, const void *W2, const moe_shared *shared, void *packed,
                                  size_t packed_bytes, void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!packable(*cfg)) return MOE_ERR_SHAPE;
  if ((cfg->F_shared > 0) != (shared != nullptr)) return MOE_ERR_CFG;
  if (!norm_weight || !W_router || !packed) return MOE_ERR_NULL;
  st = check_plain_weights(W1, W3, W2, shared);
  if (st != MOE_OK) return st;
  if (!aligned16(norm_weight) || !aligned16(W_router) || !aligned16(packed)) return MOE_ERR_ALIGN;
  if (packed_bytes < moe_block_packed_bytes(cfg)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (launch_pack_weights(*cfg, MOE_EXPERT_SWIGLU, W1, W3, W2, shared ? shared->W1 : nullptr,
                          shared ? shared->W3 : nullptr, shared ? shared->W2 : nullptr, packed, s,
                          norm_weight) != hipSuccess)
    return MOE_ERR_HIP;
  void *router = static_cast<char *>(packed) + packed_weights_bytes(*cfg, MOE_EXPERT_SWIGLU);
  if (launch_fold_rows(W_router, norm_weight, cfg->E, cfg->d, router, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_block_forward_fused(const void *h, float norm_eps, const float *bias, const void *packed,
                                   const moe_cfg *cfg, void *y, int32_t *topk_idx, float *gates, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if (!packable(*cfg)) return MOE_ERR_SHAPE;
  if (!std::isfinite(norm_eps) || norm_eps < 0.f) return MOE_ERR_CFG;
  if (cfg->T == 0) return MOE_OK;
  if (!packed) return MOE_ERR_NULL;
  if (!aligned16(packed)) return MOE_ERR_ALIGN;
  const void *router = static_cast<const char *>(packed) + packed_weights_bytes(*cfg, MOE_EXPERT_SWIGLU);
  st = check_io(h, router, cfg, y, topk_idx, gates);
  if (st != MOE_OK) return st;
  Plan probe;
  make_plan(*cfg, MOE_EXPERT_SWIGLU, nullptr, &probe, 1, norm_eps);
  if (!streaming_path(probe.path)) return MOE_ERR_SHAPE;  // beyond the streaming kernels' limits
  if (!workspace) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < probe.bytes) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_ALIGN;
  Plan p;
  make_plan(*cfg, MOE_EXPERT_SWIGLU, workspace, &p, 1, norm_eps);
  const PackedView pk = packed_view(*cfg, MOE_EXPERT_SWIGLU, packed);
  // The router and the gate/up GEMM read h itself; the norm weight is in the
  // packed weights and each token's 1/rms comes from the router's pass over h.
  return run_layer(p, h, router, bias, swiglu_experts(nullptr, nullptr, nullptr, nullptr), &pk, y, topk_idx,
                   gates, static_cast<hipStream_t>(stream), h);
}

moe_status moe_balance_update(const int32_t *topk_idx, int64_t T, int32_t k, int32_t E, float gamma,
                              float *bias, int32_t *counts, float *entropy, void *stream) {
  if (T < 0 || k < 1 || k > kMaxTopK || E < 1 || E > kMaxExperts) return MOE_ERR_SHAPE;
  if (T * static_cast<int64_t>(k) > 0x7fffffffLL - 1024) return MOE_ERR_SHAPE;
  if (!std::isfinite(gamma)) return MOE_ERR_CFG;
  if (!bias || (T > 0 && !topk_idx)) return MOE_ERR_NULL;
  auto al4 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 3u) == 0; };
  if (!al4(bias) || !al4(topk_idx) || !al4(counts) || !al4(entropy)) return MOE_ERR_ALIGN;
  (void)hipGetLastError();
  if (launch_balance_update(topk_idx, T * k, E, gamma, bias, counts, entropy, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_route_debug(const void *u, const void *W_router, const float *bias, const moe_cfg *cfg,
                           int32_t *topk_idx, float *gates, int32_t *counts, int32_t *offsets,
                           int32_t *perm, int32_t *inv, void *workspace, size_t workspace_bytes,
                           void *stream) {
  moe_status st = validate(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!u || !W_router || !topk_idx || !gates) return MOE_ERR_NULL;
  if (!aligned16(u) || !aligned16(W_router)) return MOE_ERR_ALIGN;
  Plan p;
  st = prepare(cfg, MOE_EXPERT_SWIGLU, workspace, workspace_bytes, &p);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (launch_router_topk(p, u, W_router, bias, topk_idx, gates, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_permute(p, topk_idx, s) != hipSuccess) return MOE_ERR_HIP;
  const int E = cfg->E;
  if (counts && hipMemcpyAsync(counts, p.counts, sizeof(int32_t) * E, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (offsets &&
      hipMemcpyAsync(offsets, p.offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (perm && hipMemcpyAsync(perm, p.perm, sizeof(int32_t) * p.S, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (inv && hipMemcpyAsync(inv, p.inv, sizeof(int32_t) * p.S, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_timing = on != 0;
  return MOE_OK;
}

moe_status moe_timing_read(double *ms, int64_t *calls, int reset) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (ms)
    for (int i = 0; i < MOE_N_STAGES; ++i) ms[i] = 0.0;
  moe_status st = MOE_OK;
  for (auto &r : g_records) {
    if (hipEventSynchronize(r.ev[MOE_N_STAGES]) != hipSuccess) {
      st = MOE_ERR_HIP;
      continue;
    }
    for (int i = 0; i < MOE_N_STAGES; ++i) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, r.ev[i], r.ev[i + 1]) != hipSuccess) st = MOE_ERR_HIP;
      if (ms) ms[i] += t;
    }
  }
  if (calls) *calls = static_cast<int64_t>(g_records.size());
  if (reset) {
    for (auto &r : g_records)
      for (auto &e : r.ev) (void)hipEventDestroy(e);
    g_records.clear();
  }
  return st;
}

}  // extern "C"
