/*
 * LatentMoE layer forward pass: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU library.
 *
 * Sources (cited by page title and the part of the page):
 *   [EXPL]   "LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through
 *            Equations, Architecture, Code and ..." (wpnews.pro).
 *   [README] "Latent-MoE" (GitHub README of kyegomez/Latent-MoE).
 *
 * What is computed, per token t (tokens are independent):
 *   1. router scores s = x_t W_r (+ b)                 [EXPL, Figure 3; Figure 8 top path]
 *   2. p = softmax(s) over all N' experts              [EXPL, Figure 3]
 *   3. the K' experts with the largest scores, slot k being the k-th in the
 *      order (score descending, expert index ascending)
 *                                                     [EXPL, Figure 3; LatentMoE code block]
 *   4. gate_k = p[sel_k] / sum_j p[sel_j]              [EXPL, MoE code block: the K weights
 *                                                      are renormalised to sum to 1]
 *   5. z = x_t W_down (width l)                        [EXPL, Figure 6 upper half]
 *   6. u = sum_k gate_k * W2_e relu(W1_e z)^2, e = sel_k  (experts run in l)
 *                                                     [EXPL, Figure 9; LatentMoE code block]
 *   7. y_t = u W_up + sum_s W2_s relu(W1_s x_t)^2      [EXPL, Figure 6 lower half; Figure 8
 *                                                      bottom path; shared experts unweighted]
 *   8. dispatch order: a stable counting sort of the (token, slot) pairs by
 *      expert, then token                             [EXPL, Figure 12 reading: one GPU]
 *
 * Readings where the pages are silent: selection is taken on the scores
 * (softmax is strictly increasing, so the set is the same in exact
 * arithmetic); ties go to the lower expert index; there is no residual
 * inside the layer, no bias other than the optional router bias (added to the
 * scores before softmax), no capacity limit and no token dropping.
 *
 * Arithmetic: every stored value (bf16 bits or float32) is widened exactly
 * to double and all sums are in double in plain index order.  No blocking,
 * fusion or reordering beyond the definition above.
 *
 * FP8 expert banks (the explainer's byte-count section prices expert weights
 * in FP8 and gives no scale convention; the reading taken here): W1 and W2
 * may be stored as OCP 8-bit floats of the E4M3 kind (1 sign bit, 4 exponent
 * bits of bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
 * 2^-6 * mantissa/8; exponent 15 with mantissa 7 is NaN; no infinities; the
 * largest finite value is 448) with one float32 scale per expert and output
 * column: W_e[i][j] = decode(q_e[i][j]) * scale_e[j], formed exactly in
 * double.
 *
 * Gated experts: the explainer notes (its feed-forward section) that a
 * gated activation such as SwiGLU adds a gate matrix next to W1 and changes
 * nothing else; the shaping paper's rank tables name an expert's three
 * matrices W_g, W_u, W_o.  The reading taken: a gated expert computes
 *   h = silu(W_g a) * (W1 a),  silu(v) = v / (1 + exp(-v)),  out = W2 h,
 * with W_g of W1's shape (W1 playing W_u, W2 playing W_o), for the routed
 * experts (input z, width l) and the shared experts (input x, width d) alike.
 * An FP8 bank holds W_g like W1, with its own per-column scales.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t d, l, m, m_s, n_shared, n_experts, top_k;
    int32_t bf16;       /* 1: tensors hold bf16 bit patterns, 0: float32 */
    int32_t has_bias;   /* 1: b_router is used */
    int32_t expert_fp8; /* 1: w1 and w2 hold E4M3 bytes with per-column scales */
    int32_t gated;      /* 1: gated (SwiGLU) experts, gate matrices w1g and w1g_s */
} orc_shape;

typedef struct {
    const void *x;        /* [T, d] */
    const void *w_router; /* [d, N'] */
    const float *b_router;/* [N'] or NULL */
    const void *w_down;   /* [d, l] */
    const void *w1;       /* [N', l, m] */
    const void *w2;       /* [N', m, l] */
    const void *w_up;     /* [l, d] */
    const void *w1_s;     /* [S, d, m_s] */
    const void *w2_s;     /* [S, m_s, d] */
    const float *w1_scale;/* [N', m]  (FP8 expert banks only) */
    const float *w2_scale;/* [N', l]  (FP8 expert banks only) */
    const void *w1g;      /* [N', l, m]  gate matrices (gated experts) */
    const void *w1g_s;    /* [S, d, m_s] shared gate matrices (gated experts) */
    const float *w1g_scale;/* [N', m] (gated FP8 expert banks only) */
} orc_tensors;

/* Optional per-token outputs; any pointer may be NULL.  Row r of each array
 * belongs to tokens[r]. */
typedef struct {
    double *logits;  /* [n, N'] */
    int32_t *idx;    /* [n, K'] */
    double *gate;    /* [n, K'] */
    double *z;       /* [n, l] */
    double *h;       /* [n, K', m]  relu(W1_e z)^2 (gated: silu(W_g z) * W1_e z) per slot */
    double *o;       /* [n, K', l]  W2_e h per slot (before the gate) */
    double *u;       /* [n, l] */
    double *hs;      /* [n, S*m_s]  relu(W1_s x)^2 (gated: silu(W_g,s x) * W1_s x) */
    double *y;       /* [n, d] */
} orc_outputs;

static double ld_elem(const void *base, int64_t i, int bf16)
{
    if (bf16) {
        uint32_t u = ((uint32_t)((const uint16_t *)base)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

/* Value of an E4M3 byte (see the header). */
static double fp8_e4m3(uint8_t q)
{
    const int sign = q >> 7, e = (q >> 3) & 15, mant = q & 7;
    double v;
    if (e == 15 && mant == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)mant / 8.0, -6);
    else
        v = ldexp(1.0 + (double)mant / 8.0, e - 7);
    return sign ? -v : v;
}

/* The decode alone, for pinning it: out[i] = value of q[i]. */
int orc_fp8_decode(const uint8_t *q, int64_t n, double *out)
{
    if (!q || !out || n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = fp8_e4m3(q[i]);
    return 0;
}

/* out[j] = sum_i in[i] * (decode(Q[off + i*cols + j]) * scale[j]) */
static void matvec_fp8(const double *in, const uint8_t *Q, int64_t off, int64_t rows,
                       int64_t cols, const float *scale, double *out)
{
    for (int64_t j = 0; j < cols; ++j)
        out[j] = 0.0;
    for (int64_t i = 0; i < rows; ++i) {
        const double a = in[i];
        const int64_t row = off + i * cols;
        for (int64_t j = 0; j < cols; ++j)
            out[j] += a * (fp8_e4m3(Q[row + j]) * (double)scale[j]);
    }
}

/* out[j] = sum_i in[i] * W[off + i*cols + j]  (W row-major [rows, cols]) */
static void matvec(const double *in, const void *W, int64_t off, int64_t rows,
                   int64_t cols, int bf16, double *out)
{
    for (int64_t j = 0; j < cols; ++j)
        out[j] = 0.0;
    for (int64_t i = 0; i < rows; ++i) {
        const double a = in[i];
        const int64_t row = off + i * cols;
        for (int64_t j = 0; j < cols; ++j)
            out[j] += a * ld_elem(W, row + j, bf16);
    }
}

static double sq_relu(double a) { return a > 0.0 ? a * a : 0.0; }

/* silu(v) = v * sigmoid(v) = v / (1 + e^-v); for v -> -inf the quotient
 * tends to -0, which the IEEE division gives once e^-v overflows. */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/* The K' indices with the largest s, ordered by (s descending, index
 * ascending).  Plain repeated selection. */
static int select_topk(const double *s, int64_t n, int64_t k, int32_t *idx,
                       unsigned char *taken)
{
    memset(taken, 0, (size_t)n);
    for (int64_t r = 0; r < k; ++r) {
        int64_t best = -1;
        for (int64_t e = 0; e < n; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || s[e] > s[best])
                best = e;
        }
        if (best < 0)
            return -1;
        taken[best] = 1;
        idx[r] = (int32_t)best;
    }
    return 0;
}

/* gate_k = p[idx_k] / sum_j p[idx_j] with p = softmax(s) over all n. */
static void gates(const double *s, int64_t n, const int32_t *idx, int64_t k,
                  double *g)
{
    double mx = s[0];
    for (int64_t e = 1; e < n; ++e)
        if (s[e] > mx)
            mx = s[e];
    double zsum = 0.0;
    for (int64_t e = 0; e < n; ++e)
        zsum += exp(s[e] - mx);
    double gsum = 0.0;
    for (int64_t r = 0; r < k; ++r) {
        g[r] = exp(s[idx[r]] - mx) / zsum;
        gsum += g[r];
    }
    for (int64_t r = 0; r < k; ++r)
        g[r] /= gsum;
}

static int check_shape(const orc_shape *c)
{
    if (!c || c->d <= 0 || c->l <= 0 || c->m <= 0 || c->n_experts <= 0 ||
        c->top_k <= 0 || c->top_k > c->n_experts || c->n_shared < 0 ||
        (c->n_shared > 0 && c->m_s <= 0))
        return -1;
    return 0;
}

/* Forward pass for the listed tokens.  idx_in (NULL or [n, K']) forces the
 * routing: those experts are used, with gates from this oracle's own
 * scores.  Returns 0 on success. */
int orc_forward(const orc_shape *c, const orc_tensors *w, int64_t T,
                const int64_t *tokens, int64_t n_tok, const int32_t *idx_in,
                const orc_outputs *out, int n_threads)
{
    if (check_shape(c) || !w || !tokens || !out)
        return -1;
    if (c->expert_fp8 && (!w->w1_scale || !w->w2_scale))
        return -1;
    if (c->gated && (!w->w1g || (c->n_shared > 0 && !w->w1g_s) || (c->expert_fp8 && !w->w1g_scale)))
        return -1;
    for (int64_t r = 0; r < n_tok; ++r)
        if (tokens[r] < 0 || tokens[r] >= T)
            return -2;
    const int64_t d = c->d, l = c->l, m = c->m, ms = c->m_s, S = c->n_shared;
    const int64_t N = c->n_experts, K = c->top_k;
    const int bf = c->bf16;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel reduction(| : err)
    {
        double *x = malloc(sizeof(double) * (size_t)d);
        double *s = malloc(sizeof(double) * (size_t)N);
        int32_t *sel = malloc(sizeof(int32_t) * (size_t)K);
        double *g = malloc(sizeof(double) * (size_t)K);
        unsigned char *taken = malloc((size_t)N);
        double *z = malloc(sizeof(double) * (size_t)l);
        double *a = malloc(sizeof(double) * (size_t)(m > ms ? m : ms));
        double *gv = malloc(sizeof(double) * (size_t)(m > ms ? m : ms));
        double *o = malloc(sizeof(double) * (size_t)(l > d ? l : d));
        double *u = malloc(sizeof(double) * (size_t)l);
        double *y = malloc(sizeof(double) * (size_t)d);
        double *tmp = malloc(sizeof(double) * (size_t)d);
        if (!x || !s || !sel || !g || !taken || !z || !a || !gv || !o || !u || !y || !tmp)
            err |= 1;

#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_tok; ++r) {
            if (err)
                continue;
            const int64_t t = tokens[r];
            for (int64_t i = 0; i < d; ++i)
                x[i] = ld_elem(w->x, t * d + i, bf);

            /* 1. router scores */
            matvec(x, w->w_router, 0, d, N, bf, s);
            if (c->has_bias && w->b_router)
                for (int64_t e = 0; e < N; ++e)
                    s[e] += (double)w->b_router[e];
            if (out->logits)
                memcpy(out->logits + r * N, s, sizeof(double) * (size_t)N);

            /* 3. selection (or forced routing) */
            if (idx_in) {
                for (int64_t k = 0; k < K; ++k) {
                    sel[k] = idx_in[r * K + k];
                    if (sel[k] < 0 || sel[k] >= N)
                        err |= 2;
                }
            } else if (select_topk(s, N, K, sel, taken)) {
                err |= 4;
            }
            if (err)
                continue;
            /* 2 + 4. softmax and renormalised gates */
            gates(s, N, sel, K, g);
            if (out->idx)
                memcpy(out->idx + r * K, sel, sizeof(int32_t) * (size_t)K);
            if (out->gate)
                memcpy(out->gate + r * K, g, sizeof(double) * (size_t)K);

            /* Routing outputs only: the remaining steps are skipped. */
            if (!out->z && !out->h && !out->o && !out->u && !out->hs && !out->y)
                continue;

            /* 5. shared down-projection */
            matvec(x, w->w_down, 0, d, l, bf, z);
            if (out->z)
                memcpy(out->z + r * l, z, sizeof(double) * (size_t)l);

            /* 6. latent experts and weighted combine in l */
            for (int64_t j = 0; j < l; ++j)
                u[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t e = sel[k];
                if (c->expert_fp8)
                    matvec_fp8(z, (const uint8_t *)w->w1, e * l * m, l, m, w->w1_scale + e * m, a);
                else
                    matvec(z, w->w1, e * l * m, l, m, bf, a);
                if (c->gated) {
                    if (c->expert_fp8)
                        matvec_fp8(z, (const uint8_t *)w->w1g, e * l * m, l, m, w->w1g_scale + e * m, gv);
                    else
                        matvec(z, w->w1g, e * l * m, l, m, bf, gv);
                    for (int64_t j = 0; j < m; ++j)
                        a[j] = silu(gv[j]) * a[j];
                } else {
                    for (int64_t j = 0; j < m; ++j)
                        a[j] = sq_relu(a[j]);
                }
                if (out->h)
                    memcpy(out->h + (r * K + k) * m, a, sizeof(double) * (size_t)m);
                if (c->expert_fp8)
                    matvec_fp8(a, (const uint8_t *)w->w2, e * m * l, m, l, w->w2_scale + e * l, o);
                else
                    matvec(a, w->w2, e * m * l, m, l, bf, o);
                if (out->o)
                    memcpy(out->o + (r * K + k) * l, o, sizeof(double) * (size_t)l);
                for (int64_t j = 0; j < l; ++j)
                    u[j] += g[k] * o[j];
            }
            if (out->u)
                memcpy(out->u + r * l, u, sizeof(double) * (size_t)l);

            /* 7. up-projection once, plus the unweighted shared experts */
            matvec(u, w->w_up, 0, l, d, bf, y);
            for (int64_t sh = 0; sh < S; ++sh) {
                matvec(x, w->w1_s, sh * d * ms, d, ms, bf, a);
                if (c->gated) {
                    matvec(x, w->w1g_s, sh * d * ms, d, ms, bf, gv);
                    for (int64_t j = 0; j < ms; ++j)
                        a[j] = silu(gv[j]) * a[j];
                } else {
                    for (int64_t j = 0; j < ms; ++j)
                        a[j] = sq_relu(a[j]);
                }
                if (out->hs)
                    memcpy(out->hs + r * S * ms + sh * ms, a, sizeof(double) * (size_t)ms);
                matvec(a, w->w2_s, sh * ms * d, ms, d, bf, tmp);
                for (int64_t i = 0; i < d; ++i)
                    y[i] += tmp[i];
            }
            if (out->y)
                memcpy(out->y + r * d, y, sizeof(double) * (size_t)d);
        }
        free(x); free(s); free(sel); free(g); free(taken); free(z);
        free(a); free(gv); free(o); free(u); free(y); free(tmp);
    }
    return err ? -3 : 0;
}

/* Step 3 on given scores (for example a GPU's float32 logits widened to
 * double): idx[t, :] for every row of s[T, N']. */
int orc_select(const double *s, int64_t T, int64_t N, int64_t K, int32_t *idx)
{
    if (!s || !idx || N <= 0 || K <= 0 || K > N)
        return -1;
    unsigned char *taken = malloc((size_t)N);
    if (!taken)
        return -1;
    int err = 0;
    for (int64_t t = 0; t < T && !err; ++t)
        err = select_topk(s + t * N, N, K, idx + t * K, taken);
    free(taken);
    return err;
}

/* Steps 2 + 4 on given scores and indices. */
int orc_gates(const double *s, int64_t T, int64_t N, const int32_t *idx,
              int64_t K, double *g)
{
    if (!s || !idx || !g || N <= 0 || K <= 0 || K > N)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        gates(s + t * N, N, idx + t * K, K, g + t * K);
    return 0;
}

/* Step 8: counts[e], offsets[e] (exclusive scan, offsets[N] = T*K),
 * pos[t, k] = offsets[e] + #{t' < t : e in idx[t']} and perm[pos] = t.
 * Fails on an index out of range or an expert repeated within a token. */
int orc_dispatch(const int32_t *idx, int64_t T, int64_t K, int64_t N,
                 int32_t *counts, int32_t *offsets, int32_t *pos, int32_t *perm)
{
    if (!idx || !counts || !offsets || !pos || !perm || N <= 0 || K <= 0)
        return -1;
    for (int64_t e = 0; e < N; ++e)
        counts[e] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t k = 0; k < K; ++k) {
            const int32_t e = idx[t * K + k];
            if (e < 0 || e >= N)
                return -2;
            for (int64_t j = 0; j < k; ++j)
                if (idx[t * K + j] == e)
                    return -3;
            counts[e] += 1;
        }
    int64_t run = 0;
    for (int64_t e = 0; e < N; ++e) {
        offsets[e] = (int32_t)run;
        run += counts[e];
    }
    offsets[N] = (int32_t)run;
    int32_t *fill = malloc(sizeof(int32_t) * (size_t)N);
    if (!fill)
        return -1;
    for (int64_t e = 0; e < N; ++e)
        fill[e] = offsets[e];
    for (int64_t t = 0; t < T; ++t)
        for (int64_t k = 0; k < K; ++k) {
            const int32_t e = idx[t * K + k];
            const int32_t p = fill[e]++;
            pos[t * K + k] = p;
            perm[p] = (int32_t)t;
        }
    free(fill);
    return 0;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Backward pass (the gradient of a scalar loss L through the layer, given
 * dy = dL/dy).  The routing is piecewise constant in the scores, so no
 * gradient flows through the top-K' choice; it flows through the gates,
 * g_k = exp(s_k) / sum_{j in sel} exp(s_j) (the renormalised softmax of
 * steps 2 and 4), whose Jacobian on the selected experts is
 * dg_k / ds_j = g_k (delta_kj - g_j) and zero elsewhere:
 *   ds_j = g_j (dg_j - sum_k g_k dg_k) for j in sel, 0 otherwise.
 * Every other step is a matrix product or an elementwise map:
 *   relu(a)^2 has derivative 2 relu(a);
 *   silu(g) v has partials silu'(g) v and silu(g), with
 *   silu'(g) = sigma(g) (1 + g (1 - sigma(g))), sigma(g) = 1 / (1 + e^-g).
 * Products and sums in double in plain index order; expert-bank gradients
 * are computed for a listed set of experts (their full size would not fit a
 * test's memory at the named widths).  FP8 banks are not differentiated.
 * ------------------------------------------------------------------------ */
typedef struct {
    double *dx;        /* [T, d] */
    double *dw_router; /* [d, N'] */
    double *db_router; /* [N'] */
    double *dw_down;   /* [d, l] */
    double *dw1;       /* [n_ex, l, m] for the listed experts */
    double *dw2;       /* [n_ex, m, l] */
    double *dw1g;      /* [n_ex, l, m] gated only */
    double *dw_up;     /* [l, d] */
    double *dw1_s;     /* [S, d, m_s] */
    double *dw2_s;     /* [S, m_s, d] */
    double *dw1g_s;    /* [S, d, m_s] gated only */
} orc_grads;

/* out[i] = sum_j W[off + i*cols + j] v[j]  (the product with W transposed) */
static void matvec_t(const double *v, const void *W, int64_t off, int64_t rows, int64_t cols, int bf16,
                     double *out)
{
    for (int64_t i = 0; i < rows; ++i) {
        double acc = 0.0;
        const int64_t row = off + i * cols;
        for (int64_t j = 0; j < cols; ++j)
            acc += ld_elem(W, row + j, bf16) * v[j];
        out[i] = acc;
    }
}

static double sigm(double v) { return 1.0 / (1.0 + exp(-v)); }

/* The expert's hidden layer and its input gradient for one input vector.
 * relu^2: pre holds a = in W1; gated: pre holds a_g = in W_g and a_v = in W1.
 * Given dh (gradient of the hidden layer), writes da (gradient of a, or of
 * a_g and a_v). */
static void act_forward(int gated, const double *a, const double *ag, int64_t n, double *h)
{
    for (int64_t j = 0; j < n; ++j)
        h[j] = gated ? silu(ag[j]) * a[j] : sq_relu(a[j]);
}

static void act_backward(int gated, const double *a, const double *ag, const double *dh, int64_t n, double *da,
                         double *dag)
{
    for (int64_t j = 0; j < n; ++j) {
        if (gated) {
            const double sg = sigm(ag[j]);
            da[j] = dh[j] * silu(ag[j]);
            dag[j] = dh[j] * a[j] * sg * (1.0 + ag[j] * (1.0 - sg));
        } else {
            da[j] = a[j] > 0.0 ? dh[j] * 2.0 * a[j] : 0.0;
        }
    }
}

int orc_backward(const orc_shape *c, const orc_tensors *w, int64_t T, const double *dy, const int32_t *experts,
                 int64_t n_ex, const orc_grads *out, int n_threads)
{
    if (check_shape(c) || !w || !dy || !out || T <= 0 || c->expert_fp8 || (n_ex > 0 && !experts))
        return -1;
    if (c->gated && (!w->w1g || (c->n_shared > 0 && !w->w1g_s)))
        return -1;
    const int64_t d = c->d, l = c->l, m = c->m, ms = c->m_s, S = c->n_shared;
    const int64_t N = c->n_experts, K = c->top_k;
    const int bf = c->bf16, gated = c->gated;
    for (int64_t r = 0; r < n_ex; ++r)
        if (experts[r] < 0 || experts[r] >= N)
            return -2;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    /* per-token quantities kept for the weight gradients */
    double *X = malloc(sizeof(double) * (size_t)(T * d));
    double *Z = malloc(sizeof(double) * (size_t)(T * l));
    double *U = malloc(sizeof(double) * (size_t)(T * l));
    double *DU = malloc(sizeof(double) * (size_t)(T * l));
    double *DS = malloc(sizeof(double) * (size_t)(T * N));
    double *DZ = malloc(sizeof(double) * (size_t)(T * l));
    double *HS = malloc(sizeof(double) * (size_t)(T * (S * ms + 1)));
    double *DAS = malloc(sizeof(double) * (size_t)(T * (S * ms + 1)));
    double *DAGS = malloc(sizeof(double) * (size_t)(T * (S * ms + 1)));
    int32_t *SEL = malloc(sizeof(int32_t) * (size_t)(T * K));
    double *G = malloc(sizeof(double) * (size_t)(T * K));
    int err = (!X || !Z || !U || !DU || !DS || !DZ || !HS || !DAS || !DAGS || !SEL || !G);

    /* phase 1: per token */
#pragma omp parallel reduction(| : err)
    {
        const int64_t wmax = m > ms ? m : ms;
        double *s = malloc(sizeof(double) * (size_t)N);
        unsigned char *taken = malloc((size_t)N);
        double *a = malloc(sizeof(double) * (size_t)wmax);
        double *ag = malloc(sizeof(double) * (size_t)wmax);
        double *h = malloc(sizeof(double) * (size_t)wmax);
        double *dh = malloc(sizeof(double) * (size_t)wmax);
        double *da = malloc(sizeof(double) * (size_t)wmax);
        double *dag = malloc(sizeof(double) * (size_t)wmax);
        double *o = malloc(sizeof(double) * (size_t)(K * l));
        double *dg = malloc(sizeof(double) * (size_t)K);
        double *tmp = malloc(sizeof(double) * (size_t)(d > l ? d : l));
        if (!s || !taken || !a || !ag || !h || !dh || !da || !dag || !o || !dg || !tmp)
            err |= 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            if (err)
                continue;
            double *x = X + t * d, *z = Z + t * l, *u = U + t * l, *du = DU + t * l, *dz = DZ + t * l;
            const double *dyt = dy + t * d;
            int32_t *sel = SEL + t * K;
            double *g = G + t * K;
            for (int64_t i = 0; i < d; ++i)
                x[i] = ld_elem(w->x, t * d + i, bf);
            matvec(x, w->w_router, 0, d, N, bf, s);
            if (c->has_bias && w->b_router)
                for (int64_t e = 0; e < N; ++e)
                    s[e] += (double)w->b_router[e];
            if (select_topk(s, N, K, sel, taken)) {
                err |= 4;
                continue;
            }
            gates(s, N, sel, K, g);
            matvec(x, w->w_down, 0, d, l, bf, z);
            /* forward of the routed experts, keeping each slot's output */
            for (int64_t j = 0; j < l; ++j)
                u[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t e = sel[k];
                matvec(z, w->w1, e * l * m, l, m, bf, a);
                if (gated)
                    matvec(z, w->w1g, e * l * m, l, m, bf, ag);
                act_forward(gated, a, ag, m, h);
                matvec(h, w->w2, e * m * l, m, l, bf, o + k * l);
                for (int64_t j = 0; j < l; ++j)
                    u[j] += g[k] * o[k * l + j];
            }
            /* y = u W_up + shared: du = dy W_up^T */
            matvec_t(dyt, w->w_up, 0, l, d, bf, du);
            /* gates and scores */
            double gdg = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int64_t j = 0; j < l; ++j)
                    acc += du[j] * o[k * l + j];
                dg[k] = acc;
                gdg += g[k] * acc;
            }
            double *ds = DS + t * N;
            for (int64_t e = 0; e < N; ++e)
                ds[e] = 0.0;
            for (int64_t k = 0; k < K; ++k)
                ds[sel[k]] = g[k] * (dg[k] - gdg);
            /* back through the routed experts into z */
            for (int64_t j = 0; j < l; ++j)
                dz[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t e = sel[k];
                matvec(z, w->w1, e * l * m, l, m, bf, a);
                if (gated)
                    matvec(z, w->w1g, e * l * m, l, m, bf, ag);
                for (int64_t j = 0; j < l; ++j)
                    tmp[j] = g[k] * du[j]; /* gradient of slot k's output */
                matvec_t(tmp, w->w2, e * m * l, m, l, bf, dh);
                act_backward(gated, a, ag, dh, m, da, dag);
                matvec_t(da, w->w1, e * l * m, l, m, bf, tmp);
                for (int64_t j = 0; j < l; ++j)
                    dz[j] += tmp[j];
                if (gated) {
                    matvec_t(dag, w->w1g, e * l * m, l, m, bf, tmp);
                    for (int64_t j = 0; j < l; ++j)
                        dz[j] += tmp[j];
                }
            }
            /* dx = ds W_r^T + dz W_down^T + shared */
            double *dx = out->dx ? out->dx + t * d : NULL;
            if (dx) {
                matvec_t(ds, w->w_router, 0, d, N, bf, dx);
                matvec_t(dz, w->w_down, 0, d, l, bf, tmp);
                for (int64_t i = 0; i < d; ++i)
                    dx[i] += tmp[i];
            }
            for (int64_t sh = 0; sh < S; ++sh) {
                double *hs = HS + t * S * ms + sh * ms, *das = DAS + t * S * ms + sh * ms;
                double *dags = DAGS + t * S * ms + sh * ms;
                matvec(x, w->w1_s, sh * d * ms, d, ms, bf, a);
                if (gated)
                    matvec(x, w->w1g_s, sh * d * ms, d, ms, bf, ag);
                act_forward(gated, a, ag, ms, hs);
                matvec_t(dyt, w->w2_s, sh * ms * d, ms, d, bf, dh);
                act_backward(gated, a, ag, dh, ms, das, dags);
                if (dx) {
                    matvec_t(das, w->w1_s, sh * d * ms, d, ms, bf, tmp);
                    for (int64_t i = 0; i < d; ++i)
                        dx[i] += tmp[i];
                    if (gated) {
                        matvec_t(dags, w->w1g_s, sh * d * ms, d, ms, bf, tmp);
                        for (int64_t i = 0; i < d; ++i)
                            dx[i] += tmp[i];
                    }
                }
            }
        }
        free(s); free(taken); free(a); free(ag); free(h); free(dh); free(da); free(dag); free(o); free(dg);
        free(tmp);
    }

    /* phase 2: dense weight gradients, sums over tokens in token order */
    if (!err) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < d; ++i) {
            for (int64_t e = 0; e < N && out->dw_router; ++e) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    acc += X[t * d + i] * DS[t * N + e];
                out->dw_router[i * N + e] = acc;
            }
            for (int64_t j = 0; j < l && out->dw_down; ++j) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    acc += X[t * d + i] * DZ[t * l + j];
                out->dw_down[i * l + j] = acc;
            }
            for (int64_t sh = 0; sh < S; ++sh)
                for (int64_t j = 0; j < ms; ++j) {
                    double acc = 0.0, accg = 0.0;
                    for (int64_t t = 0; t < T; ++t) {
                        acc += X[t * d + i] * DAS[t * S * ms + sh * ms + j];
                        accg += X[t * d + i] * DAGS[t * S * ms + sh * ms + j];
                    }
                    if (out->dw1_s)
                        out->dw1_s[(sh * d + i) * ms + j] = acc;
                    if (gated && out->dw1g_s)
                        out->dw1g_s[(sh * d + i) * ms + j] = accg;
                }
        }
        if (out->db_router)
            for (int64_t e = 0; e < N; ++e) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    acc += DS[t * N + e];
                out->db_router[e] = acc;
            }
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < l; ++i)
            for (int64_t j = 0; j < d && out->dw_up; ++j) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    acc += U[t * l + i] * dy[t * d + j];
                out->dw_up[i * d + j] = acc;
            }
        if (out->dw2_s) {
#pragma omp parallel for schedule(dynamic, 4)
            for (int64_t r = 0; r < S * ms; ++r) {
                const int64_t sh = r / ms, j = r % ms;
                for (int64_t i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < T; ++t)
                        acc += HS[t * S * ms + sh * ms + j] * dy[t * d + i];
                    out->dw2_s[(sh * ms + j) * d + i] = acc;
                }
            }
        }
    }

    /* phase 3: expert-bank gradients of the listed experts, tokens in order */
    if (!err && n_ex > 0 && (out->dw1 || out->dw2 || (gated && out->dw1g))) {
#pragma omp parallel reduction(| : err)
        {
            double *a = malloc(sizeof(double) * (size_t)m), *ag = malloc(sizeof(double) * (size_t)m);
            double *h = malloc(sizeof(double) * (size_t)m), *dh = malloc(sizeof(double) * (size_t)m);
            double *da = malloc(sizeof(double) * (size_t)m), *dag = malloc(sizeof(double) * (size_t)m);
            double *go = malloc(sizeof(double) * (size_t)l);
            if (!a || !ag || !h || !dh || !da || !dag || !go)
                err |= 1;
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_ex; ++r) {
                if (err)
                    continue;
                const int64_t e = experts[r];
                double *w1g_out = (gated && out->dw1g) ? out->dw1g + r * l * m : NULL;
                if (out->dw1)
                    memset(out->dw1 + r * l * m, 0, sizeof(double) * (size_t)(l * m));
                if (out->dw2)
                    memset(out->dw2 + r * m * l, 0, sizeof(double) * (size_t)(m * l));
                if (w1g_out)
                    memset(w1g_out, 0, sizeof(double) * (size_t)(l * m));
                for (int64_t t = 0; t < T; ++t)
                    for (int64_t k = 0; k < K; ++k) {
                        if (SEL[t * K + k] != e)
                            continue;
                        const double *z = Z + t * l;
                        matvec(z, w->w1, e * l * m, l, m, bf, a);
                        if (gated)
                            matvec(z, w->w1g, e * l * m, l, m, bf, ag);
                        act_forward(gated, a, ag, m, h);
                        for (int64_t j = 0; j < l; ++j)
                            go[j] = G[t * K + k] * DU[t * l + j];
                        if (out->dw2)
                            for (int64_t i = 0; i < m; ++i)
                                for (int64_t j = 0; j < l; ++j)
                                    out->dw2[(r * m + i) * l + j] += h[i] * go[j];
                        matvec_t(go, w->w2, e * m * l, m, l, bf, dh);
                        act_backward(gated, a, ag, dh, m, da, dag);
                        for (int64_t i = 0; i < l; ++i)
                            for (int64_t j = 0; j < m; ++j) {
                                if (out->dw1)
                                    out->dw1[(r * l + i) * m + j] += z[i] * da[j];
                                if (w1g_out)
                                    w1g_out[i * m + j] += z[i] * dag[j];
                            }
                    }
            }
            free(a); free(ag); free(h); free(dh); free(da); free(dag); free(go);
        }
    }
    free(X); free(Z); free(U); free(DU); free(DS); free(DZ); free(HS); free(DAS); free(DAGS); free(SEL); free(G);
    return err ? -3 : 0;
}
