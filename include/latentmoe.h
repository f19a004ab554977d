/*
 * latentmoe.h -- C ABI of the LatentMoE layer forward pass on MI355X (gfx950).
 *
 * The layer (page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained
 * Through Equations, Architecture, Code and ..." (wpnews.pro), Figures 3, 6,
 * 8 and 9 and its LatentMoE code block; same interface as the layer of the
 * "Latent-MoE" README, "Usage" section):
 *
 *   s      = x W_r (+ b)                      router in the model width d
 *   sel    = the K' experts of largest s       ties: lower expert index first
 *   gate_k = softmax(s)[sel_k] / sum_j softmax(s)[sel_j]
 *   z      = x W_down                         shared down-projection to l = d/alpha
 *   u      = sum_k gate_k W2_{sel_k}^T relu(W1_{sel_k}^T z)^2   (experts run in l)
 *   y      = u W_up + sum_s relu(x W1_s)^2 W2_s                (one up-projection,
 *                                                              unweighted shared experts)
 *
 * Layouts: every matrix is row-major and stored [in, out], so a vector times
 * the matrix is the layer's product (x[T,d] W_r[d,N'] -> s[T,N']).  (batch,
 * seq) is flattened into T tokens.  All pointers except the config, weight,
 * debug and cost structs themselves are DEVICE pointers unless stated.
 *
 * Errors: every call returns a latentmoe_status.  Arguments are validated on
 * the host before any GPU work; a HIP runtime error is reported as
 * LATENTMOE_ERR_HIP and its hipError_t is kept for latentmoe_last_hip_error().
 * Nothing is thrown across the ABI.  Inputs must be finite.
 */
#ifndef LATENTMOE_H
#define LATENTMOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum latentmoe_status {
    LATENTMOE_OK = 0,
    LATENTMOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, inconsistent shape, T out of range */
    LATENTMOE_ERR_UNSUPPORTED = 2,      /* valid layer, but outside what the kernels handle */
    LATENTMOE_ERR_OUT_OF_MEMORY = 3,    /* device allocation failed */
    LATENTMOE_ERR_HIP = 4,              /* a HIP runtime call failed */
    LATENTMOE_ERR_EXCEEDS_SCRATCH = 5   /* latentmoe_forward_noalloc: T needs more workspace
                                           than the library's static scratch holds */
} latentmoe_status;

/* Two ways to spend the saving of the latent projection (README "Two
 * flavors"; explainer Figure 13): acc keeps the baseline's cost with
 * K' = alpha K, eff keeps K' = K.  K' is always passed explicitly in top_k;
 * the variant only tells latentmoe_cost which baseline to compare with. */
typedef enum latentmoe_variant { LATENTMOE_VARIANT_ACC = 0, LATENTMOE_VARIANT_EFF = 1 } latentmoe_variant;

/* Storage and compute type.  BF16: bf16 tensors, fp32 accumulation, bf16
 * intermediates.  F32: fp32 tensors and intermediates throughout. */
typedef enum latentmoe_dtype { LATENTMOE_DTYPE_F32 = 0, LATENTMOE_DTYPE_BF16 = 1 } latentmoe_dtype;

/* Storage of the routed-expert banks W1 and W2.  AS_DTYPE: the config dtype.
 * FP8_E4M3 (bf16 configs only; the explainer's byte-count section prices
 * expert weights in FP8): OCP E4M3 bytes (bias 7, subnormals at exponent 0,
 * NaN at exponent 15 / mantissa 7, no infinities) with one fp32 scale per
 * expert and output column, W[e][i][j] = value(q[e][i][j]) * scale[e][j].
 * Expert GEMMs then read half the bytes; the values are widened exactly to
 * bf16 for the matrix cores and the scale is applied to the fp32 sums. */
typedef enum latentmoe_expert_format {
    LATENTMOE_EXPERT_AS_DTYPE = 0,
    LATENTMOE_EXPERT_FP8_E4M3 = 1
} latentmoe_expert_format;

/* Expert activation.  RELU2: out = W2 relu(W1 a)^2 (the explainer's Expert
 * class and Figure 9).  SWIGLU: the gated form the explainer's feed-forward
 * section allows, which adds a gate matrix next to W1 (the shaping paper's
 * W_g, W_u, W_o): out = W2 (silu(W_g a) * (W1 a)), silu(v) = v / (1 + e^-v), for the
 * routed experts (a = z) and the shared experts (a = x) alike; the gate
 * matrices come in w1_gate and w1_shared_gate. */
typedef enum latentmoe_expert_act { LATENTMOE_ACT_RELU2 = 0, LATENTMOE_ACT_SWIGLU = 1 } latentmoe_expert_act;

typedef struct latentmoe_config {
    int64_t d;          /* model width */
    int64_t l;          /* latent width; l * alpha == d */
    int64_t m;          /* routed-expert hidden width */
    int64_t m_shared;   /* shared-expert hidden width (ignored when n_shared == 0) */
    int64_t n_shared;   /* S >= 0 shared experts */
    int64_t n_experts;  /* N' routed experts (already alpha * N) */
    int64_t top_k;      /* K' experts per token */
    int64_t alpha;      /* compression factor */
    int32_t variant;    /* latentmoe_variant */
    int32_t dtype;      /* latentmoe_dtype */
    int64_t max_tokens; /* largest T a forward call may pass; sizes the workspace */
    int32_t has_router_bias; /* 1: b_router is added to the scores before softmax */
    int32_t expert_format;   /* latentmoe_expert_format */
    int32_t expert_act;      /* latentmoe_expert_act */
} latentmoe_config;

/* Device pointers, in the config's dtype except b_router and the scales
 * (always fp32) and W1/W2 under LATENTMOE_EXPERT_FP8_E4M3 (one byte per
 * weight).  latentmoe_create copies and repacks them; the caller may free or
 * change them once it returns. */
typedef struct latentmoe_weights {
    const void *w_router;   /* [d, N'] */
    const float *b_router;  /* [N'] or NULL */
    const void *w_down;     /* [d, l] */
    const void *w1;         /* [N', l, m] */
    const void *w2;         /* [N', m, l] */
    const void *w_up;       /* [l, d] */
    const void *w1_shared;  /* [S, d, m_shared] (NULL when S == 0) */
    const void *w2_shared;  /* [S, m_shared, d] (NULL when S == 0) */
    const float *w1_scale;  /* [N', m] FP8 expert banks only, else NULL */
    const float *w2_scale;  /* [N', l] FP8 expert banks only, else NULL */
    const void *w1_gate;         /* [N', l, m] SWIGLU only (E4M3 bytes in an FP8 bank), else NULL */
    const void *w1_shared_gate;  /* [S, d, m_shared] SWIGLU with S > 0 only, else NULL */
    const float *w1_gate_scale;  /* [N', m] SWIGLU FP8 expert banks only, else NULL */
} latentmoe_weights;

/* Optional device buffers that a forward call fills with its intermediate
 * results (any member may be NULL).  P = T * K'.  "E" is the config dtype. */
typedef struct latentmoe_debug {
    float *logits;       /* [T, N'] router scores (fp32, bias included) */
    int32_t *idx;        /* [T, K'] selected experts, slot order */
    float *gate;         /* [T, K'] renormalised weights */
    int32_t *counts;     /* [N'] (token, slot) pairs per expert */
    int32_t *offsets;    /* [N'+1] exclusive scan of counts */
    int32_t *perm_token; /* [P] token of each dispatch row (expert-major, token-ascending) */
    int32_t *pos;        /* [T, K'] dispatch row of each (token, slot) */
    void *z;             /* [T, l] E, x W_down */
    void *h_shared;      /* [T, S*m_shared] E, relu(x W1_s)^2 */
    void *h;             /* [P, m] E, relu(z W1_e)^2 per dispatch row */
    void *y_perm;        /* [P, l] E, h W2_e per dispatch row (no gate) */
    void *u;             /* [T, l] E, gate-weighted sum in l */
} latentmoe_debug;

/* Closed-form cost counts (README "Inspect the asymptotic cost quantities
 * from Table 1" section; every worked count of the explainer reproduces).
 * The baseline is the standard MoE with N = N'/alpha experts of width d and
 * K = K'/alpha (acc) or K' (eff).  FLOPs count 2 per multiply-add.  The
 * "2" of each expert term below is the number of expert matrices: 3 for
 * LATENTMOE_ACT_SWIGLU (routed, shared and baseline experts alike). */
typedef struct latentmoe_cost_out {
    double latent_expert_params;        /* 2 l m */
    double routed_pool_params;          /* N' 2 l m */
    double projection_params;           /* 2 d l */
    double router_params;               /* d N' */
    double shared_params;               /* S 2 d m_s */
    double layer_params_excl_router;    /* pool + shared + projections */
    double active_params_per_token;     /* K' 2 l m + shared + projections */
    double expert_bytes_per_token_fp8;  /* K' 2 l m, one byte per weight */
    double expert_bytes_per_token_bf16; /* K' 2 l m * 2 */
    double a2a_bytes_per_token;         /* K' l (0.5 + 2): fp4 out, bf16 back */
    double flops_per_token;             /* 2 (d N' + 2 d l + 2 K' l m + 2 S d m_s) */
    double log10_combinations;          /* log10 C(N', K') */
    double baseline_n_experts, baseline_top_k;
    double baseline_expert_params;      /* 2 d m */
    double baseline_layer_params_excl_router;
    double baseline_active_params_per_token;
    double baseline_a2a_bytes_per_token;
    double baseline_log10_combinations;
    double log10_combination_bound;     /* alpha log10 C(N, K) */
} latentmoe_cost_out;

typedef struct latentmoe_handle latentmoe_handle;

/* Validate cfg and w, allocate the workspace for cfg->max_tokens, and copy
 * the weights into the kernels' layout on `hip_stream` (a hipStream_t, or
 * NULL for the default stream).  Returns when the copies are complete.
 * On success *out owns the handle; on failure *out is NULL.  A weight that
 * the config needs and w leaves NULL (the scales of an FP8 bank, the gate
 * matrices of a SWIGLU layer) is LATENTMOE_ERR_INVALID_ARGUMENT. */
int latentmoe_create(const latentmoe_config *cfg, const latentmoe_weights *w,
                     void *hip_stream, latentmoe_handle **out);

/* y[T, d] = layer(x[T, d]).  x and y are device buffers of the config dtype
 * and must not overlap.  1 <= T <= max_tokens.  Asynchronous on hip_stream
 * (no host synchronisation); one forward in flight per handle.  dbg may be
 * NULL.  Routing and dispatch are deterministic; a given input always gives
 * the same bits. */
int latentmoe_forward(latentmoe_handle *h, const void *x, void *y, int64_t T,
                      void *hip_stream, const latentmoe_debug *dbg);

/* latentmoe_forward without device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same layer, same kernels, same arguments (no
 * debug outputs); the forward's workspace for T tokens (scores, routing,
 * dispatch order, tile table, z/u and h_s, H, Y, split-K partial sums) lives
 * in a static device array of LATENTMOE_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing, neither does anything it launches.  The bits equal
 * latentmoe_forward's whenever the split-K GEMMs of 65..256 rows get as
 * many partial sums as there (always true when T <= 64 or T > 256); else
 * they differ by the fp32 summation order only.  Every call on one GPU
 * shares that GPU's array and leaves its contents behind: calls that
 * overlap on one GPU (two streams, two handles, two host threads) race and
 * must be serialised by the caller -- a race can also leave the arrival
 * counters of the few-row split GEMMs (at the start of the array, zeroed
 * once when the first handle on the GPU is created, and left at zero by
 * every call) nonzero, which makes the later calls on that GPU wrong.
 * Nothing in the array needs clearing between calls.  The workspace needed is about T (K' (4 + 2 (m + l)) +
 * 4 N' + 2 (l + S m_s)) bytes for bf16 layers (e.g. readme widths: about 100
 * KB per token, about 650 tokens fit).  Errors: as latentmoe_forward, and
 * LATENTMOE_ERR_EXCEEDS_SCRATCH when T tokens need more than the array. */
#define LATENTMOE_NOALLOC_SCRATCH_BYTES (64ll << 20)
int latentmoe_forward_noalloc(latentmoe_handle *h, const void *x, void *y, int64_t T, void *hip_stream);

/* Gradients of a scalar loss L through the layer (device pointers; NULL
 * skips that gradient).  Weight gradients are fp32 in the weights' own
 * [in, out] layouts and are written, not accumulated; dx has the config
 * dtype.  P = T * K'. */
typedef struct latentmoe_grads {
    void *dx;               /* [T, d] E */
    float *dw_router;       /* [d, N'] */
    float *db_router;       /* [N'] (layers with a router bias) */
    float *dw_down;         /* [d, l] */
    float *dw1;             /* [N', l, m] */
    float *dw2;             /* [N', m, l] */
    float *dw_up;           /* [l, d] */
    float *dw1_shared;      /* [S, d, m_shared] */
    float *dw2_shared;      /* [S, m_shared, d] */
    float *dw1_gate;        /* [N', l, m] SWIGLU only */
    float *dw1_shared_gate; /* [S, d, m_shared] SWIGLU only */
} latentmoe_grads;

/* The layer's backward pass at input x[T, d] for dy = dL/dy [T, d] (both
 * device buffers of the config dtype): dx and the weight gradients.  The
 * top-K' choice is piecewise constant in the scores and passes no gradient;
 * it flows through the gates, the softmax renormalised over the selected
 * experts (explainer, MoE code block), and through every matrix product and
 * activation of the forward.  The forward is recomputed inside the call.
 * Asynchronous on hip_stream like latentmoe_forward, and deterministic.  The
 * first call on a handle allocates its backward workspace and the weight
 * layouts the backward products read (about one more copy of the weights).
 * Errors: LATENTMOE_ERR_UNSUPPORTED for FP8 expert banks;
 * LATENTMOE_ERR_INVALID_ARGUMENT for null handle/x/dy/g, T out of range, or
 * a router-bias gradient asked of a layer without one. */
int latentmoe_backward(latentmoe_handle *h, const void *x, const void *dy, int64_t T, void *hip_stream,
                       const latentmoe_grads *g);

/* Free the handle and everything it owns (NULL is a no-op).  The caller
 * must ensure no forward is still running on it. */
int latentmoe_destroy(latentmoe_handle *h);

/* Check a config without touching the GPU (the same checks as create). */
int latentmoe_validate_config(const latentmoe_config *cfg);

/* Bytes of device workspace create would allocate for cfg (host only). */
int latentmoe_workspace_bytes(const latentmoe_config *cfg, int64_t *bytes);

/* Host-only cost counts of cfg; `out` is a host pointer. */
int latentmoe_cost(const latentmoe_config *cfg, latentmoe_cost_out *out);

/* Static description of a status code. */
const char *latentmoe_status_string(int status);

/* hipError_t of the last LATENTMOE_ERR_HIP returned on this thread (0 if none). */
int latentmoe_last_hip_error(void);

/* Per-stage kernel timing with HIP events recorded on the forward's stream.
 * profile_begin reserves events for up to max_forwards forward calls and
 * times the stages whose bit is set in stage_mask (bit s = stage s; each
 * timed stage costs two event records per forward, so a caller measuring
 * throughput times only the stage it needs); profile_end waits for them and
 * writes, for each stage s < *n_stages, the total milliseconds in ms[s] and
 * the number of timed launches in launches[s] (host arrays of length
 * LATENTMOE_MAX_STAGES), and the stage names via latentmoe_stage_name.
 * Errors: LATENTMOE_ERR_INVALID_ARGUMENT for a null handle, max_forwards
 * outside [1, 100000] or an empty mask. */
#define LATENTMOE_MAX_STAGES 16
int latentmoe_profile_begin(latentmoe_handle *h, int max_forwards, uint32_t stage_mask);
int latentmoe_profile_end(latentmoe_handle *h, double *ms, int32_t *launches, int32_t *n_stages);
const char *latentmoe_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* LATENTMOE_H */
