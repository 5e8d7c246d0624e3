/*
 * moe_oracle.c -- CPU oracle for the forward pass of one sparse
 * mixture-of-experts (MoE) feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg call it; the product path never does.  It shares no code,
 * header, table or constant with the GPU library.
 *
 * What it computes (sources are the five web pages this project follows):
 *   - router logits l[t][e] = u_t . W_router[e]
 *       ["Mixture of Experts and Hybrid Architectures", "The router in code"]
 *       ["Sparse MoE FFN" (DeepSeek-V3), "How it works", Routing: u_t^T e_i]
 *   - selection score: the raw logit (softmax mode) or the sigmoid affinity
 *       s = 1/(1+exp(-l)) (sigmoid mode) ["Sparse MoE FFN", Routing]
 *   - biased score sb = s + b, used for selection only
 *       ["Mixture of Experts and Hybrid Architectures", "The router in code",
 *        "Troubleshooting", "Questions": bias touches selection only]
 *   - optional group limit: contiguous groups, group score = sum of the two
 *       largest sb in the group, keep the best M groups, then top-k inside
 *       them ["Sparse MoE FFN", Routing: 8 groups, keep 4, sum of top-2]
 *   - top-k by a stable descending sort (ties -> lower index)
 *       ["Mixture of Experts and Hybrid Architectures", "The router in code"]
 *   - gates from the raw scores of the chosen experts: max-subtracted
 *       softmax (softmax mode) or s / sum(s) (sigmoid mode), times
 *       route_scale ["The router in code"; "Sparse MoE FFN", Routing]
 *   - each expert is SwiGLU, W2 (SiLU(W1 u) * W3 u), SiLU(x) = x sigmoid(x)
 *       ["Sparse MoE FFN", "How it works", expert equation]; the generic
 *       expert of "Lesson 2 -- From the Dense FFN to a Layer of Experts",
 *       section 2, W2 phi(W1 u + b1) + b2 with phi = GELU, and the gated unit
 *       with GELU in place of SiLU (GEGLU, named beside SwiGLU in the cheat
 *       sheet's "Calculator defaults") are the other two bodies
 *       (oracle_forward_ex); GELU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2
 *       ["Sparse MoE FFN", "How it works", expert equation]
 *   - y = sum_j g_j FFN_{i_j}(u) + FFN_shared(u), no residual, no dropping
 *       ["Sparse MoE FFN", eq. 12 and "Packed forward"]
 *   - the expert-contiguous permutation of the (token, slot) pairs, stable
 *       in slot order ("gather the tokens where indices == i",
 *       ["Sparse MoE FFN", "Packed forward"]).
 *
 * Arithmetic is fp64 throughout.  Inputs are read as fp32, fp64 or bf16 bit
 * patterns (widened exactly), so the oracle sees exactly the values a GPU
 * run received.  Tokens are independent, so work is split over POSIX threads
 * by token; nothing else is reordered, blocked or fused.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2

#define ORC_SOFTMAX 0
#define ORC_SIGMOID 1

#define ORC_SWIGLU 0
#define ORC_GEGLU 1
#define ORC_GELU_MLP 2

/* ---- element access ------------------------------------------------------ */

static double elem(const void *p, int64_t i, int dtype)
{
    if (dtype == ORC_F64) return ((const double *)p)[i];
    if (dtype == ORC_F32) return (double)((const float *)p)[i];
    /* bf16 is the top half of an IEEE binary32: widen by a 16-bit shift. */
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---- ranking ------------------------------------------------------------- */

/* 1 when score a must be ranked strictly ahead of score b.  Larger first; NaN
 * ranks below every number, so indices stay valid and distinct. */
static int ahead(double a, double b)
{
    if (isnan(a)) return 0;
    if (isnan(b)) return 1;
    return a > b;
}

/* Stable descending sort of order[0..n) by key[order[i]] (insertion sort):
 * elements that tie keep their input order, which is ascending index. */
static void stable_sort_desc(int32_t *order, int n, const double *key)
{
    for (int i = 1; i < n; ++i) {
        int32_t v = order[i];
        int j = i - 1;
        while (j >= 0 && ahead(key[v], key[order[j]])) {
            order[j + 1] = order[j];
            --j;
        }
        order[j + 1] = v;
    }
}

static double rel_gap(double a, double b)
{
    double m = fabs(a);
    if (fabs(b) > m) m = fabs(b);
    if (m < 1.0) m = 1.0;
    return fabs(a - b) / m;
}

/* ---- problem description --------------------------------------------------- */

typedef struct {
    int64_t T;
    int d, E, k, F, Fs;
    int score_fn, n_groups, topk_groups;
    double route_scale;
    const void *u;
    int u_dtype;
    const void *Wr;
    int w_dtype; /* W_router, W1, W3, W2 and the shared weights */
    const double *bias;      /* [E] or NULL (= zeros) */
    const void *W1, *W3, *W2;    /* [E][F][d], [E][F][d], [E][d][F] */
    const void *W1s, *W3s, *W2s; /* [Fs][d], [Fs][d], [d][Fs] or NULL */
    int kind;                    /* ORC_SWIGLU, ORC_GEGLU, ORC_GELU_MLP */
    const void *b1, *b2;         /* GELU MLP: [E][F], [E][d] or NULL (zero) */
    const void *b1s, *b2s;       /* [Fs], [d] or NULL */
} problem;

/* ---- step 1: router logits ---------------------------------------------------- */

static void logits_of_token(const problem *P, int64_t t, double *l)
{
    for (int e = 0; e < P->E; ++e) {
        double acc = 0.0;
        for (int j = 0; j < P->d; ++j)
            acc += elem(P->u, t * P->d + j, P->u_dtype) *
                   elem(P->Wr, (int64_t)e * P->d + j, P->w_dtype);
        l[e] = acc;
    }
}

/* ---- steps 2-6: scores, biased group-limited top-k, gates ---------------------- */

typedef struct {
    int E, k, score_fn, n_groups, topk_groups;
    double route_scale;
    const double *bias;
} select_cfg;

/* scratch: 4*E doubles + 2*E ints, provided by the caller. */
static void select_token(const select_cfg *S, const double *l, int32_t *idx,
                         double *gates, double *gap_expert, double *gap_group,
                         double *scratch, int32_t *iscratch)
{
    const int E = S->E, k = S->k;
    double *s = scratch, *sb = scratch + E, *gscore = scratch + 2 * E;
    double *key = scratch + 3 * E;
    int32_t *order = iscratch, *eligible = iscratch + E;

    /* score and biased score */
    for (int e = 0; e < E; ++e) {
        s[e] = (S->score_fn == ORC_SIGMOID) ? 1.0 / (1.0 + exp(-l[e])) : l[e];
        sb[e] = s[e] + (S->bias ? S->bias[e] : 0.0);
        eligible[e] = 1;
    }

    /* group limit */
    *gap_group = INFINITY;
    if (S->n_groups > 1) {
        const int G = S->n_groups, per = E / G, M = S->topk_groups;
        for (int g = 0; g < G; ++g) {
            for (int i = 0; i < per; ++i) order[i] = g * per + i;
            stable_sort_desc(order, per, sb);
            gscore[g] = sb[order[0]] + sb[order[1]];
        }
        for (int g = 0; g < G; ++g) order[g] = g;
        stable_sort_desc(order, G, gscore);
        for (int e = 0; e < E; ++e) eligible[e] = 0;
        for (int r = 0; r < M; ++r)
            for (int i = 0; i < per; ++i) eligible[order[r] * per + i] = 1;
        if (M < G) *gap_group = rel_gap(gscore[order[M - 1]], gscore[order[M]]);
    }

    /* top-k over eligible experts by a stable descending sort of sb */
    int n = 0;
    for (int e = 0; e < E; ++e)
        if (eligible[e]) order[n++] = e;
    stable_sort_desc(order, n, sb);
    for (int j = 0; j < k; ++j) idx[j] = order[j];
    *gap_expert = (k < n) ? rel_gap(sb[order[k - 1]], sb[order[k]]) : INFINITY;

    /* gates from the raw scores of the chosen experts; the bias is not read */
    if (S->score_fn == ORC_SIGMOID) {
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += s[idx[j]];
        for (int j = 0; j < k; ++j) gates[j] = S->route_scale * s[idx[j]] / sum;
    } else {
        double m = l[idx[0]];
        for (int j = 1; j < k; ++j)
            if (l[idx[j]] > m) m = l[idx[j]];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) {
            key[j] = exp(l[idx[j]] - m);
            sum += key[j];
        }
        for (int j = 0; j < k; ++j) gates[j] = S->route_scale * key[j] / sum;
    }
}

/* ---- step 7/8: SwiGLU expert ------------------------------------------------- */

static double silu(double x) { return x / (1.0 + exp(-x)); }

static double gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

/* One expert of the given body:
 *   SwiGLU   h = SiLU(W1 x) * (W3 x)
 *   GEGLU    h = GELU(W1 x) * (W3 x)
 *   GELU MLP h = GELU(W1 x + b1)           (b1 NULL: zero)
 * out[0..d) += scale * (W2 h + b2)          (b2 only for the GELU MLP)
 * W1, W3 [F][d], W2 [d][F] at element offsets off13 / off2; b1, b2 at
 * offsets offb1 / offb2.  hbuf holds F doubles. */
static void expert_accumulate(const double *x, int d, int F, int kind, const void *W1,
                              const void *W3, const void *W2, const void *b1,
                              const void *b2, int64_t off13, int64_t off2,
                              int64_t offb1, int64_t offb2, int dtype, double scale,
                              double *out, double *hbuf)
{
    for (int f = 0; f < F; ++f) {
        double a = 0.0, c = 0.0;
        for (int j = 0; j < d; ++j) {
            a += elem(W1, off13 + (int64_t)f * d + j, dtype) * x[j];
            if (kind != ORC_GELU_MLP) c += elem(W3, off13 + (int64_t)f * d + j, dtype) * x[j];
        }
        if (kind == ORC_SWIGLU)
            hbuf[f] = silu(a) * c;
        else if (kind == ORC_GEGLU)
            hbuf[f] = gelu(a) * c;
        else
            hbuf[f] = gelu(a + (b1 ? elem(b1, offb1 + f, dtype) : 0.0));
    }
    for (int n = 0; n < d; ++n) {
        double o = 0.0;
        for (int f = 0; f < F; ++f)
            o += elem(W2, off2 + (int64_t)n * F + f, dtype) * hbuf[f];
        if (kind == ORC_GELU_MLP && b2) o += elem(b2, offb2 + n, dtype);
        out[n] += scale * o;
    }
}

/* ---- threading --------------------------------------------------------------- */

typedef struct job job;
typedef void (*token_fn)(job *, int64_t, double *, int32_t *);
struct job {
    const problem *P;
    const select_cfg *S;
    const int64_t *tokens; /* NULL = 0..n-1 */
    int64_t n;
    const double *logits_in;   /* oracle_select: [T][E] */
    const int32_t *forced_idx; /* oracle_forward: [n][k] or NULL */
    const double *forced_gates;
    double *logits_out;
    int32_t *idx;
    double *gates, *gap_e, *gap_g, *y;
    token_fn fn;
    int nthreads, tid;
    size_t dscratch, iscratch;
};

static void *worker(void *arg)
{
    job *J = (job *)arg;
    double *ds = (double *)malloc(J->dscratch * sizeof(double));
    int32_t *is = (int32_t *)malloc((J->iscratch + 1) * sizeof(int32_t));
    for (int64_t i = J->tid; i < J->n; i += J->nthreads) J->fn(J, i, ds, is);
    free(ds);
    free(is);
    return NULL;
}

static void run_jobs(job *proto, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    job jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *proto;
        jobs[i].nthreads = nthreads;
        jobs[i].tid = i;
    }
    if (nthreads == 1) {
        worker(&jobs[0]);
        return;
    }
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &jobs[i]);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* ---- exported: router logits ---------------------------------------------------- */

static void logits_task(job *J, int64_t i, double *ds, int32_t *is)
{
    (void)ds;
    (void)is;
    int64_t t = J->tokens ? J->tokens[i] : i;
    logits_of_token(J->P, t, J->logits_out + i * J->P->E);
}

/* logits[i][e] for the n tokens listed in tokens (NULL: tokens 0..n-1). */
int oracle_router_logits(int64_t n, const int64_t *tokens, int d, int E,
                         const void *u, int u_dtype, const void *Wr,
                         int w_dtype, double *logits, int nthreads)
{
    if (n < 0 || d <= 0 || E <= 0 || !u || !Wr || !logits) return -1;
    problem P = {0};
    P.d = d;
    P.E = E;
    P.u = u;
    P.u_dtype = u_dtype;
    P.Wr = Wr;
    P.w_dtype = w_dtype;
    job J = {0};
    J.P = &P;
    J.tokens = tokens;
    J.n = n;
    J.logits_out = logits;
    J.fn = logits_task;
    J.dscratch = 1;
    J.iscratch = 1;
    run_jobs(&J, nthreads);
    return 0;
}

/* ---- exported: selection from logits ------------------------------------------- */

static int check_select(int E, int k, int score_fn, int G, int M)
{
    if (E <= 0 || k <= 0 || k > E) return -1;
    if (score_fn != ORC_SOFTMAX && score_fn != ORC_SIGMOID) return -1;
    if (G < 1 || M < 1 || M > G || E % G != 0) return -1;
    if (G > 1 && (E / G < 2 || k > M * (E / G))) return -1;
    return 0;
}

static void select_task(job *J, int64_t i, double *ds, int32_t *is)
{
    const int E = J->S->E, k = J->S->k;
    double ge, gg;
    select_token(J->S, J->logits_in + i * E, J->idx + i * k, J->gates + i * k,
                 &ge, &gg, ds, is);
    if (J->gap_e) J->gap_e[i] = ge;
    if (J->gap_g) J->gap_g[i] = gg;
}

/* Steps 2-6 for n tokens given their logits [n][E]; bias [E] or NULL. */
int oracle_select(int64_t n, int E, int k, int score_fn, int n_groups,
                  int topk_groups, double route_scale, const double *bias,
                  const double *logits, int32_t *idx, double *gates,
                  double *gap_expert, double *gap_group, int nthreads)
{
    if (check_select(E, k, score_fn, n_groups, topk_groups)) return -1;
    if (n < 0 || !logits || !idx || !gates) return -1;
    select_cfg S = {E, k, score_fn, n_groups, topk_groups, route_scale, bias};
    job J = {0};
    J.S = &S;
    J.n = n;
    J.logits_in = logits;
    J.idx = idx;
    J.gates = gates;
    J.gap_e = gap_expert;
    J.gap_g = gap_group;
    J.fn = select_task;
    J.dscratch = 4 * (size_t)E;
    J.iscratch = 2 * (size_t)E;
    run_jobs(&J, nthreads);
    return 0;
}

/* ---- exported: whole-layer forward for a list of tokens -------------------------- */

static void forward_task(job *J, int64_t i, double *ds, int32_t *is)
{
    const problem *P = J->P;
    const int E = P->E, k = P->k, d = P->d;
    int64_t t = J->tokens ? J->tokens[i] : i;
    double *x = ds, *l = ds + d, *h = l + E, *sel = h + (P->F > P->Fs ? P->F : P->Fs);
    double *y = J->y + i * d;
    int32_t *idx = J->idx + i * k;
    double *gates = J->gates + i * k;

    for (int j = 0; j < d; ++j) x[j] = elem(P->u, t * d + j, P->u_dtype);
    if (J->forced_idx) {
        /* Selection supplied by the caller; gates recomputed from the raw
         * scores of that selection exactly as in the routed case. */
        logits_of_token(P, t, l);
        for (int j = 0; j < k; ++j) idx[j] = J->forced_idx[i * k + j];
        double *s = sel;
        for (int e = 0; e < E; ++e)
            s[e] = (P->score_fn == ORC_SIGMOID) ? 1.0 / (1.0 + exp(-l[e])) : l[e];
        if (P->score_fn == ORC_SIGMOID) {
            double sum = 0.0;
            for (int j = 0; j < k; ++j) sum += s[idx[j]];
            for (int j = 0; j < k; ++j) gates[j] = P->route_scale * s[idx[j]] / sum;
        } else {
            double m = l[idx[0]], sum = 0.0;
            for (int j = 1; j < k; ++j)
                if (l[idx[j]] > m) m = l[idx[j]];
            for (int j = 0; j < k; ++j) sum += exp(l[idx[j]] - m);
            for (int j = 0; j < k; ++j)
                gates[j] = P->route_scale * exp(l[idx[j]] - m) / sum;
        }
        if (J->gap_e) J->gap_e[i] = INFINITY;
        if (J->gap_g) J->gap_g[i] = INFINITY;
    } else {
        double ge, gg;
        logits_of_token(P, t, l);
        select_token(J->S, l, idx, gates, &ge, &gg, sel, is);
        if (J->gap_e) J->gap_e[i] = ge;
        if (J->gap_g) J->gap_g[i] = gg;
    }

    for (int n = 0; n < d; ++n) y[n] = 0.0;
    for (int j = 0; j < k; ++j) {
        int64_t e = idx[j];
        expert_accumulate(x, d, P->F, P->kind, P->W1, P->W3, P->W2, P->b1, P->b2,
                          e * P->F * d, e * d * P->F, e * P->F, e * d, P->w_dtype,
                          gates[j], y, h);
    }
    if (P->Fs > 0)
        expert_accumulate(x, d, P->Fs, P->kind, P->W1s, P->W3s, P->W2s, P->b1s, P->b2s,
                          0, 0, 0, 0, P->w_dtype, 1.0, y, h);
}

/*
 * y[i][0..d), idx[i][0..k), gates[i][0..k) for the n tokens listed in tokens
 * (NULL: 0..n-1).  forced_idx [n][k] (or NULL) replaces steps 2-5.
 * Fs == 0 means no shared expert (W1s, W3s, W2s ignored).  kind selects the
 * expert body (ORC_SWIGLU, ORC_GEGLU, ORC_GELU_MLP); W3 / W3s are unused and
 * b1, b2, b1s, b2s (NULL: zero) used only by the GELU MLP.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_forward_ex(int64_t n, const int64_t *tokens, int d, int E, int k,
                      int F, int Fs, int score_fn, int n_groups, int topk_groups,
                      double route_scale, const void *u, int u_dtype,
                      const void *Wr, const double *bias, int kind, const void *W1,
                      const void *W3, const void *W2, const void *b1, const void *b2,
                      const void *W1s, const void *W3s, const void *W2s, const void *b1s,
                      const void *b2s, int w_dtype, const int32_t *forced_idx, double *y,
                      int32_t *idx, double *gates, double *gap_expert, double *gap_group,
                      int nthreads)
{
    const int gated = kind == ORC_SWIGLU || kind == ORC_GEGLU;
    if (kind != ORC_SWIGLU && kind != ORC_GEGLU && kind != ORC_GELU_MLP) return -1;
    if (check_select(E, k, score_fn, n_groups, topk_groups)) return -1;
    if (n < 0 || d <= 0 || F <= 0 || Fs < 0) return -1;
    if (!u || !Wr || !W1 || (gated && !W3) || !W2 || !y || !idx || !gates) return -1;
    if (Fs > 0 && (!W1s || (gated && !W3s) || !W2s)) return -1;
    if (forced_idx)
        for (int64_t i = 0; i < n * k; ++i)
            if (forced_idx[i] < 0 || forced_idx[i] >= E) return -1;
    problem P = {0};
    P.d = d;
    P.E = E;
    P.k = k;
    P.F = F;
    P.Fs = Fs;
    P.score_fn = score_fn;
    P.n_groups = n_groups;
    P.topk_groups = topk_groups;
    P.route_scale = route_scale;
    P.u = u;
    P.u_dtype = u_dtype;
    P.Wr = Wr;
    P.w_dtype = w_dtype;
    P.bias = bias;
    P.W1 = W1;
    P.W3 = W3;
    P.W2 = W2;
    P.W1s = W1s;
    P.W3s = W3s;
    P.W2s = W2s;
    P.kind = kind;
    P.b1 = b1;
    P.b2 = b2;
    P.b1s = b1s;
    P.b2s = b2s;
    select_cfg S = {E, k, score_fn, n_groups, topk_groups, route_scale, bias};
    job J = {0};
    J.P = &P;
    J.S = &S;
    J.tokens = tokens;
    J.n = n;
    J.forced_idx = forced_idx;
    J.y = y;
    J.idx = idx;
    J.gates = gates;
    J.gap_e = gap_expert;
    J.gap_g = gap_group;
    J.fn = forward_task;
    int fmax = F > Fs ? F : Fs;
    J.dscratch = (size_t)d + E + fmax + 4 * (size_t)E;
    J.iscratch = 2 * (size_t)E;
    run_jobs(&J, nthreads);
    return 0;
}

/* The SwiGLU layer: oracle_forward_ex with kind ORC_SWIGLU. */
int oracle_forward(int64_t n, const int64_t *tokens, int d, int E, int k,
                   int F, int Fs, int score_fn, int n_groups, int topk_groups,
                   double route_scale, const void *u, int u_dtype,
                   const void *Wr, const double *bias, const void *W1,
                   const void *W3, const void *W2, const void *W1s,
                   const void *W3s, const void *W2s, int w_dtype,
                   const int32_t *forced_idx, double *y, int32_t *idx,
                   double *gates, double *gap_expert, double *gap_group,
                   int nthreads)
{
    return oracle_forward_ex(n, tokens, d, E, k, F, Fs, score_fn, n_groups, topk_groups,
                             route_scale, u, u_dtype, Wr, bias, ORC_SWIGLU, W1, W3, W2, NULL,
                             NULL, W1s, W3s, W2s, NULL, NULL, w_dtype, forced_idx, y, idx,
                             gates, gap_expert, gap_group, nthreads);
}

/* ---- exported: expert-contiguous permutation ---------------------------------------- */

/*
 * For n_slots = T*k slots (slot = t*k + j holds expert idx[slot]):
 *   counts[e]   = number of slots choosing expert e
 *   offsets[e]  = sum of counts[0..e)          (offsets[E] = n_slots)
 *   perm[p]     = the slot at position p, experts in ascending order and,
 *                 within an expert, slots in ascending order
 *   inv[slot]   = the position of slot
 * Returns -1 if an index is out of range.
 */
int oracle_permutation(int64_t n_slots, int E, const int32_t *idx,
                       int32_t *counts, int32_t *offsets, int32_t *perm,
                       int32_t *inv)
{
    for (int64_t s = 0; s < n_slots; ++s)
        if (idx[s] < 0 || idx[s] >= E) return -1;
    int64_t pos = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)pos;
        for (int64_t s = 0; s < n_slots; ++s)
            if (idx[s] == e) {
                perm[pos] = (int32_t)s;
                inv[s] = (int32_t)pos;
                ++pos;
            }
        counts[e] = (int32_t)(pos - offsets[e]);
    }
    offsets[E] = (int32_t)pos;
    return 0;
}
