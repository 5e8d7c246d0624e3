/*
 * moe.h -- C ABI of libmoe, the forward pass of one sparse mixture-of-experts
 * (MoE) feed-forward layer on an AMD Instinct MI355X (gfx950).
 *
 * The layer (sources: the web pages "Mixture of Experts and Hybrid
 * Architectures" (cheat sheet), "Mixture of experts and architecture
 * families", "Sparse MoE FFN" (DeepSeek-V3) and "Lesson 2 -- From the Dense
 * FFN to a Layer of Experts"):
 *
 *   l[t][e]  = u[t] . W_router[e]                      router, fp32 accumulate
 *   s        = l            (MOE_SCORE_SOFTMAX)        select on raw scores
 *            = sigmoid(l)   (MOE_SCORE_SIGMOID)        affinities
 *   sb       = s + bias                                selection only
 *   groups   : n_groups contiguous blocks of E/n_groups experts; group score
 *              = sum of its two largest sb; keep the topk_groups best groups
 *   topk_idx = the k largest sb among eligible experts, descending, ties to
 *              the lower index; NaN ranks below every number
 *   gates    = route_scale * softmax(l over the k chosen)      (SOFTMAX)
 *            = route_scale * s / sum(s over the k chosen)      (SIGMOID)
 *   y[t]     = sum_j gates[t][j] * FFN_{topk_idx[t][j]}(u[t]) + FFN_shared(u[t])
 *   FFN(x)   = W2 (SiLU(W1 x) * W3 x),  SiLU(x) = x sigmoid(x)
 *
 * "The router in code" (cheat sheet) fixes selection on score + bias, the
 * stable descending sort, and the softmax over the chosen raw scores.  "Sparse
 * MoE FFN", "How it works" (Routing, eq. 12, Packed forward) fixes sigmoid
 * affinities, group masking (8 groups keep 4, group score = sum of top-2),
 * renormalised gates times route_scale 2.5, the SwiGLU expert, the always-on
 * unweighted shared expert, and that no token is dropped.  The module returns
 * shared + routed; the residual is added by the caller.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are device memory owned by the caller, row-major and
 *     contiguous, 16-byte aligned.  The library never allocates device memory
 *     at run time.  Host state kept between calls: the optional timing
 *     records, the CU count of the device (read once), and the device
 *     address of each GPU's fixed scratch array of moe_layer_forward_noalloc
 *     (static device storage, looked up once per GPU).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL for
 *     the default stream); calls return after enqueueing and never
 *     synchronise.  Device faults surface at the caller's next sync.
 *   - Arguments are validated before anything is launched.  On a negative
 *     status nothing was launched and no output was written.
 *   - T == 0 is a valid no-op.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,      /* a required pointer is NULL                      */
    MOE_ERR_SHAPE = -2,     /* a size is out of the supported range            */
    MOE_ERR_CFG = -3,       /* inconsistent routing configuration              */
    MOE_ERR_DTYPE = -4,     /* unknown dtype or score function                 */
    MOE_ERR_WORKSPACE = -5, /* workspace missing or smaller than required      */
    MOE_ERR_HIP = -6,       /* a HIP launch or runtime call failed             */
    MOE_ERR_ALIGN = -7      /* a pointer is not 16-byte aligned                */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

typedef struct {
    int64_t T;           /* tokens (rows of u), >= 0                               */
    int32_t d;           /* hidden size, multiple of 64                            */
    int32_t E;           /* routed experts, 1..256                                 */
    int32_t k;           /* experts per token, 1..min(E, 32)                       */
    int32_t F;           /* routed expert inner width, multiple of 64              */
    int32_t F_shared;    /* shared expert inner width (N_s * F fused), 0 = none    */
    int32_t dtype;       /* moe_dtype of u, y and every weight matrix              */
    int32_t score_fn;    /* moe_score_fn                                           */
    int32_t n_groups;    /* expert groups (1 = no group limit); divides E, <= 64   */
    int32_t topk_groups; /* groups kept per token, 1..n_groups                     */
    float route_scale;   /* gate multiplier: 1.0 for softmax, 2.5 for DeepSeek-V3  */
} moe_cfg;

/* Shared (always-on) expert weights: W1, W3 [F_shared][d], W2 [d][F_shared]. */
typedef struct {
    const void *W1;
    const void *W3;
    const void *W2;
} moe_shared;

/* Bytes of device workspace moe_layer_forward and moe_route_debug need for
 * cfg, or 0 when cfg is invalid.  The buffer is scratch: its contents on
 * entry do not matter and are overwritten. */
size_t moe_workspace_bytes(const moe_cfg *cfg);

/* Checks cfg without touching the GPU; MOE_OK or the status the entry points
 * would return for it. */
moe_status moe_check_cfg(const moe_cfg *cfg);

/*
 * The whole layer forward.
 *   u        [T][d]       cfg->dtype   token inputs (pre-normed by the caller)
 *   W_router [E][d]       cfg->dtype   router rows e_i
 *   bias     [E]          fp32         selection-only bias; NULL == all zeros
 *   W1, W3   [E][F][d]    cfg->dtype   expert gate / up projections
 *   W2       [E][d][F]    cfg->dtype   expert down projections
 *   shared   NULL == no shared expert (then cfg->F_shared must be 0)
 *   y        [T][d]       cfg->dtype   out: shared + routed (no residual);
 *                                      overwritten, must not alias u
 *   topk_idx [T][k]       int32        out: chosen experts, descending sb
 *   gates    [T][k]       fp32         out: gate of each chosen expert
 *   workspace, workspace_bytes          >= moe_workspace_bytes(cfg)
 * Internally: fp32 accumulation everywhere; for bf16 the SwiGLU activations
 * and the per-slot expert outputs are stored as bf16 and y is rounded to
 * bf16 (nearest even).  The result is bitwise deterministic: there are no
 * floating-point atomics.
 */
moe_status moe_layer_forward(const void *u, const void *W_router, const float *bias,
                             const void *W1, const void *W3, const void *W2,
                             const moe_shared *shared, const moe_cfg *cfg, void *y,
                             int32_t *topk_idx, float *gates, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments and results as moe_layer_forward
 * (bitwise), minus the workspace: the library keeps one fixed device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU (its static storage, held until the
 * process ends) and uses it as the workspace.  The call itself allocates
 * nothing and enqueues no memset or copy.
 *   - Limit: configurations whose workspace (moe_workspace_bytes) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE before any HIP call
 *     (64 MiB covers, e.g., the DeepSeek-V3 layer shape up to T = 256).
 *   - The array of the current device is used; the stream must belong to it.
 *     Its address is looked up once per device, at the first call there.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other threads) race and must be
 *     serialised by the caller.  Nothing from an earlier call is read.
 *   - Per-stage timing (moe_timing_enable) does not record these calls.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const void *u, const void *W_router, const float *bias,
                                     const void *W1, const void *W3, const void *W2,
                                     const moe_shared *shared, const moe_cfg *cfg, void *y,
                                     int32_t *topk_idx, float *gates, void *stream);

/*
 * Packed weights (bf16 layers with d, F and F_shared multiples of 256).
 *
 * The expert weights are static, so they may be re-laid out once (model
 * load) into the order the streaming GEMM kernels consume them: for each
 * expert, slabs of 256 weight rows (gate/up: 128 columns of W1 and the same
 * 128 of W3, 32 rows of each alternating; down: 256 rows of W2), each slab as
 * its K/32 stage blocks of 16 KiB, each block the 256 rows x 32 values in the
 * order they land in LDS.  Every weight tile a kernel stage needs is then one
 * contiguous 16 KiB read.  The computation is unchanged: moe_layer_forward
 * and moe_layer_forward_packed give bitwise identical results.
 *
 * moe_packed_weights_bytes: size of the packed buffer for cfg's shapes (T is
 *   ignored), or 0 when cfg cannot be packed.
 * moe_pack_weights: fills packed (caller-owned device memory, >= that size,
 *   16-byte aligned) from the plain W1, W3, W2 and shared weights of
 *   moe_layer_forward; enqueued on stream.
 * moe_layer_forward_packed: moe_layer_forward with the packed buffer in
 *   place of W1, W3, W2 and shared (the shared expert is used iff
 *   cfg->F_shared > 0).  Returns MOE_ERR_SHAPE when cfg cannot be packed or
 *   is beyond the streaming kernels (moe_plan_describe then reports the
 *   tiled kernels): T too large for the streaming schedule, or a token
 *   matrix u of 4 GiB or more.
 */
size_t moe_packed_weights_bytes(const moe_cfg *cfg);
moe_status moe_pack_weights(const moe_cfg *cfg, const void *W1, const void *W3, const void *W2,
                            const moe_shared *shared, void *packed, size_t packed_bytes, void *stream);
moe_status moe_layer_forward_packed(const void *u, const void *W_router, const float *bias,
                                    const void *packed, const moe_cfg *cfg, void *y, int32_t *topk_idx,
                                    float *gates, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * Other expert bodies.  "Lesson 2 -- From the Dense FFN to a Layer of
 * Experts", section 2, writes each expert as the dense FFN it replaces, an
 * activation between two affine maps with biases, GELU or a gated unit; the
 * cheat sheet ("Mixture of Experts and Hybrid Architectures", "Calculator
 * defaults") takes GELU as the default activation and names SwiGLU and GEGLU
 * as the gated ones, which add the third matrix W3.
 * GELU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, the exact form (erff in
 * fp32).
 *
 *   MOE_EXPERT_SWIGLU    FFN(x) = W2 (SiLU(W1 x) * W3 x)     (= moe_layer_forward)
 *   MOE_EXPERT_GEGLU     FFN(x) = W2 (GELU(W1 x) * W3 x)
 *   MOE_EXPERT_GELU_MLP  FFN(x) = W2 GELU(W1 x + b1) + b2
 *
 * The gate weights the whole expert output, b2 included; the shared expert,
 * of the same body with its own biases, is added unweighted.
 *
 * moe_experts (every tensor device memory in cfg->dtype, 16-byte aligned):
 *   W1, W3 [E][F][d], W2 [E][d][F]; b1 [E][F], b2 [E][d]
 *   W1s, W3s [F_shared][d], W2s [d][F_shared]; b1s [F_shared], b2s [d]
 *   W3 / W3s are not read by the GELU MLP (may be NULL); the biases belong to
 *   the GELU MLP only (NULL there == zero; non-NULL with a gated kind is
 *   MOE_ERR_CFG).  The shared pointers must be NULL iff cfg->F_shared == 0
 *   (else MOE_ERR_CFG), biases aside.
 * moe_workspace_bytes_ex: workspace for cfg with experts of the given kind,
 *   0 when cfg or kind is invalid (for SwiGLU, moe_workspace_bytes(cfg)).
 * moe_plan_describe_ex: moe_plan_describe for the given kind.  The GELU MLP
 *   takes the streaming kernels only with F % 256 == 0 and F_shared % 256 == 0.
 * moe_layer_forward_ex: moe_layer_forward with these experts (plain layout).
 *   For bf16 the hidden activations after the activation (and the bias b1)
 *   and the per-slot expert outputs (with b2) are stored as bf16.
 *   MOE_ERR_DTYPE for an unknown kind.
 *
 * Packed weights for these bodies (the layout of moe_pack_weights; the GELU
 * MLP's gate/up region holds W1 alone, in 256-row slabs like W2):
 * moe_packed_weights_bytes_ex: size for cfg and kind, 0 when cfg cannot be
 *   packed (d, F, F_shared multiples of 256, bf16) or kind is unknown.
 * moe_pack_weights_ex: packs the weight pointers of *experts (its biases are
 *   not packed and not read) into packed, enqueued on stream.
 * moe_layer_forward_packed_ex: moe_layer_forward_ex with the packed buffer in
 *   place of the weights: experts->kind and its bias pointers are read (the
 *   kind must be the one packed), its weight pointers are not.  The result is
 *   bitwise that of moe_layer_forward_ex.  MOE_ERR_SHAPE when cfg cannot be
 *   packed or T is too large for the streaming schedule.
 */
typedef enum { MOE_EXPERT_SWIGLU = 0, MOE_EXPERT_GEGLU = 1, MOE_EXPERT_GELU_MLP = 2 } moe_expert_kind;

typedef struct {
    int32_t kind;     /* moe_expert_kind */
    const void *W1;
    const void *W3;
    const void *W2;
    const void *b1;
    const void *b2;
    const void *W1s;
    const void *W3s;
    const void *W2s;
    const void *b1s;
    const void *b2s;
} moe_experts;

size_t moe_workspace_bytes_ex(const moe_cfg *cfg, int32_t kind);
moe_status moe_plan_describe_ex(const moe_cfg *cfg, int32_t kind, int32_t *gemm_path, int32_t *tile_rows);
moe_status moe_layer_forward_ex(const void *u, const void *W_router, const float *bias,
                                const moe_experts *experts, const moe_cfg *cfg, void *y,
                                int32_t *topk_idx, float *gates, void *workspace,
                                size_t workspace_bytes, void *stream);
size_t moe_packed_weights_bytes_ex(const moe_cfg *cfg, int32_t kind);
moe_status moe_pack_weights_ex(const moe_cfg *cfg, const moe_experts *experts, void *packed,
                               size_t packed_bytes, void *stream);
moe_status moe_layer_forward_packed_ex(const void *u, const void *W_router, const float *bias,
                                       const moe_experts *experts, const void *packed,
                                       const moe_cfg *cfg, void *y, int32_t *topk_idx, float *gates,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Routing and permutation only (the first two stages of moe_layer_forward,
 * same kernels; the small fp32 layers that moe_layer_forward runs in one
 * kernel make the same selection there), for tests and tools.  Outputs, all
 * int32 device arrays:
 *   counts [E]       slots that chose expert e
 *   offsets [E+1]    exclusive prefix sum of counts; offsets[E] = T*k
 *   perm [T*k]       slot (t*k + j) at each expert-contiguous position; within
 *                    an expert, slots ascend (stable)
 *   inv [T*k]        position of each slot
 * Any of counts/offsets/perm/inv may be NULL (not copied out).
 */
moe_status moe_route_debug(const void *u, const void *W_router, const float *bias,
                           const moe_cfg *cfg, int32_t *topk_idx, float *gates,
                           int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * The layer inside its pre-norm residual block: y = h + MoE(RMSNorm(h)).
 * "Lesson 2 -- From the Dense FFN to a Layer of Experts", section 2: the MoE
 * layer takes the FFN's place in the pre-norm block, H' = H~ + MoE(Norm(H~));
 * "Sparse MoE FFN" (DeepSeek-V3), eq. 12 and "How it works": the skip adds
 * the block input outside the MoE module; "Mixture of experts and
 * architecture families": the norm is RMSNorm (no mean-centering).
 *
 * moe_rmsnorm: out[t][j] = h[t][j] / sqrt(mean_j h[t][j]^2 + eps) * g[j],
 *   h, out [T][d] and g [d] in dtype (device, 16-byte aligned; out may be h);
 *   fp32 arithmetic, one rounding to dtype.  d % 64 == 0, d <= 8192,
 *   0 <= eps finite.  T == 0 is a no-op.
 * moe_block_workspace_bytes: workspace of the block entry points (the
 *   layer's plus room for the normalised rows), 0 when cfg is invalid.
 * moe_block_forward, moe_block_forward_packed: moe_layer_forward and
 *   moe_layer_forward_packed on u = moe_rmsnorm(h, norm_weight, norm_eps)
 *   (computed into the workspace, read by the router and the expert GEMMs),
 *   with h added to y last in fp32 before the rounding to dtype:
 *     y[t] = h[t] + shared(u[t]) + sum_j gates[t][j] * expert_j(u[t]).
 *   h [T][d] and norm_weight [d] in cfg->dtype; y must not alias h;
 *   workspace_bytes >= moe_block_workspace_bytes(cfg).  Errors as for the
 *   layer entry points, plus MOE_ERR_CFG for a bad norm_eps.
 */
moe_status moe_rmsnorm(const void *h, const void *norm_weight, float eps, int64_t T, int32_t d, int32_t dtype,
                       void *out, void *stream);
size_t moe_block_workspace_bytes(const moe_cfg *cfg);
moe_status moe_block_forward(const void *h, const void *norm_weight, float norm_eps, const void *W_router,
                             const float *bias, const void *W1, const void *W3, const void *W2,
                             const moe_shared *shared, const moe_cfg *cfg, void *y, int32_t *topk_idx,
                             float *gates, void *workspace, size_t workspace_bytes, void *stream);
moe_status moe_block_forward_packed(const void *h, const void *norm_weight, float norm_eps, const void *W_router,
                                    const float *bias, const void *packed, const moe_cfg *cfg, void *y,
                                    int32_t *topk_idx, float *gates, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * The same block with the normalisation fused into the router and the first
 * expert product (no pass that writes normalised rows):
 *   RMSNorm(h)_j = rs * h_j * g_j,  rs = 1 / sqrt(mean_j h_j^2 + eps)
 * g is static, so it is folded once into the weights that multiply the
 * normalised rows: W_router, W1, W3, W1s, W3s (each product w * g[j]
 * rounded once to bf16, nearest even); rs is a per-token scalar, so the
 * router sums each token's squares in its pass over h (fp32, fixed order),
 * scales the token's logits by rs before the score function, and the gate/up
 * GEMM scales its accumulators of that token's rows by rs before SiLU.
 * Routing decisions are thus taken on rs * (h . bf16(W_router * g)).
 *
 * moe_block_packed_bytes: size of the fused block's packed buffer: the
 *   packed SwiGLU weights (moe_packed_weights_bytes) followed by the folded
 *   router rows [E][d]; 0 when cfg cannot be packed (bf16, d, F and F_shared
 *   multiples of 256).
 * moe_pack_block_weights: fills it from norm_weight [d], W_router and the
 *   plain expert weights of moe_block_forward (enqueued on stream).
 * moe_block_forward_fused: y = h + MoE(RMSNorm(h)) from that buffer, as
 *   moe_block_forward, with workspace_bytes >= moe_block_workspace_bytes(cfg).
 *   MOE_ERR_SHAPE when cfg cannot be packed or is beyond the streaming
 *   kernels (see moe_layer_forward_packed); MOE_ERR_CFG for a bad norm_eps.
 */
size_t moe_block_packed_bytes(const moe_cfg *cfg);
moe_status moe_pack_block_weights(const moe_cfg *cfg, const void *norm_weight, const void *W_router,
                                  const void *W1, const void *W3, const void *W2, const moe_shared *shared,
                                  void *packed, size_t packed_bytes, void *stream);
moe_status moe_block_forward_fused(const void *h, float norm_eps, const float *bias, const void *packed,
                                   const moe_cfg *cfg, void *y, int32_t *topk_idx, float *gates,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * One step of the auxiliary-loss-free balance update ("Mixture of Experts and
 * Hybrid Architectures", "Aux-loss-free balance loop"; the bias moves only
 * selection, "Sparse MoE FFN", "How it works", Routing), from the routing of
 * one batch:
 *   counts[e] = number of the T*k entries of topk_idx equal to e
 *   target    = T*k / E
 *   bias[e]  -= gamma  if counts[e] > target   (compared exactly: counts*E vs T*k)
 *   bias[e]  += gamma  if counts[e] < target   (fp32 add; an expert on target keeps its bias)
 *   *entropy  = -sum_e p_e ln p_e, p = counts / (T*k) (0 when T == 0; max ln E)
 *   topk_idx [T][k] int32   device, as written by moe_layer_forward; entries
 *                           outside [0, E) are not counted; may be NULL if T == 0
 *   bias     [E]    fp32    device, updated in place
 *   counts   [E]    int32   device out, may be NULL
 *   entropy  [1]    fp32    device out, may be NULL (computed in fp64)
 * Enqueued on stream as one kernel; allocates nothing and needs no workspace.
 * Returns MOE_ERR_SHAPE for T < 0, k outside 1..32 or E outside 1..256,
 * MOE_ERR_CFG for a non-finite gamma, MOE_ERR_NULL, MOE_ERR_ALIGN (4 bytes).
 */
moe_status moe_balance_update(const int32_t *topk_idx, int64_t T, int32_t k, int32_t E, float gamma,
                              float *bias, int32_t *counts, float *entropy, void *stream);

/*
 * Which grouped-GEMM kernels moe_layer_forward uses for cfg (host only, no
 * GPU call): *gemm_path = 0 for the tiled kernels (any size, fp32 or bf16),
 * 1 for the persistent weight-streaming kernels with 256-row tiles (bf16,
 * d % 256 == 0, F % 128 == 0, F_shared % 128 == 0, at least 64 routed rows
 * per expert on average, T * d * 2 and max(F, F_shared) * d * 2 below 2^32
 * bytes, which they address with 32-bit offsets), 2 for their decode variant
 * with 32-row tiles (fewer rows per expert; also F % 256 == 0,
 * F_shared % 256 == 0; T * d * 2 below 2^32 too); both also need T within
 * the streaming schedule; 3 for the one-kernel small layer (fp32 SwiGLU,
 * T * k <= 512, d, F and F_shared <= 1024: one workgroup per token computes
 * its routing, experts and sum without the permutation or grouped GEMMs);
 * *tile_rows = rows per GEMM tile.  Either pointer may be NULL.
 */
moe_status moe_plan_describe(const moe_cfg *cfg, int32_t *gemm_path, int32_t *tile_rows);

/* Human-readable text of a status code (static storage). */
const char *moe_status_str(int status);

/*
 * Optional per-stage GPU timing.  While enabled, every moe_layer_forward call
 * records a HIP event before and after each stage on its stream.
 * moe_timing_read synchronises on the recorded events, adds the elapsed
 * milliseconds of each stage into ms[MOE_N_STAGES], stores the number of
 * calls measured in *calls, and (reset != 0) clears the records.
 * Stages: 0 router+top-k, 1 permutation, 2 gate/up projections with the
 * activation, 3 down projections, 4 gate-weighted combine.
 */
#define MOE_N_STAGES 5
moe_status moe_timing_enable(int on);
moe_status moe_timing_read(double *ms, int64_t *calls, int reset);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
