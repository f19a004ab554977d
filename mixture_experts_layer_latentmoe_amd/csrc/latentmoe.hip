// LatentMoE layer on MI355X (gfx950): host plan, forward and backward
// launch sequences, and the C ABI.
//
// The layer is the one of the explainer page "LatentMoE: NVIDIA's Latent
// Mixture of Experts Explained Through Equations, Architecture, Code and
// ..." (Figures 3, 6, 8, 9; LatentMoE code block); see include/latentmoe.h.
//
// One forward is a fixed sequence of launches on the caller's stream, with
// no host synchronisation (the grouped GEMMs read their tile tables from
// device memory):
//   0 gemm_x            [s | z | h_s] = x [W_r | W_down | W1_s]: router scores
//                       in fp32 (+ bias), z, and the squared-ReLU hidden layer of
//                       the shared experts -- one MFMA pass over x
//   1 router_select     top-K', gates, chunk ranks / counts
//   2 dispatch_scan     per-expert scan over 16-token chunks, counts
//   3 dispatch_finalize offsets, grouped-GEMM tile table, pos[t,k], perm_token[p]
//                       (up to 64 chunks: 2 and 3 in one workgroup, one launch)
//   4 grouped_gemm1     H = relu(z[perm] W1_e)^2 per expert
//   5 grouped_gemm2     Y = H W2_e per expert
//     (4 + 5 fused: expert_mlp, Y = relu(z[perm] W1_e)^2 W2_e with H kept on
//     chip, for bf16 layers with bf16 banks at l = 512 and prefill-sized
//     row counts; expert_mlp.hpp)
//   6 combine           u[t] = sum_k gate[t,k] Y[pos[t,k]], written over z
//   7 gemm_up_shared2   y = [u | h_s] [W_up ; W2_s]
// Stages 0 and 7 fold the router and the always-on shared experts into the
// down- and up-projection GEMMs: all of them read x (resp. produce y) at
// width d, so one pass over x and one output write serve every path.  Up to
// 64 tokens, stages 0 and 7 run the few-row kernel (skinny.hpp).
//
// The backward (backward_impl) recomputes the forward with raw outputs and
// then runs the data-gradient and weight-gradient products (backward.hpp,
// gemm_tn.hpp).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "latentmoe.h"

#include "combine.hpp"
#include "common.hpp"
#include "dispatch.hpp"
#include "expert_mlp.hpp"
#include "gemm.hpp"
#include "gemm_tn.hpp"
#include "repack.hpp"
#include "route_tiny.hpp"
#include "router.hpp"
#include "skinny.hpp"
#include "backward.hpp"

using namespace lmoe;

namespace {

thread_local int g_last_hip_error = 0;

// Every device allocation of the library goes through here.  Test hook:
// with LATENTMOE_FAIL_ALLOC_AT=n in the environment, the n-th allocation of
// the process (counting from 1) fails as if the device were out of memory,
// so that tests can reach the clean-up paths of create and of the backward's
// first call.
std::atomic<long long> g_alloc_count{0};

hipError_t device_alloc(void **p, size_t bytes)
{
    const long long n = ++g_alloc_count;
    if (const char *f = std::getenv("LATENTMOE_FAIL_ALLOC_AT")) {
        if (std::atoll(f) == n) {
            *p = nullptr;
            return hipErrorOutOfMemory;
        }
    }
    return hipMalloc(p, bytes);
}

enum Stage {
    ST_GEMM_X = 0,
    ST_SELECT,
    ST_SCAN,
    ST_FINALIZE,
    ST_GEMM1,
    ST_GEMM2,
    ST_COMBINE,
    ST_GEMM_UP,
    ST_MLP,
    ST_COUNT
};

const char *kStageNames[ST_COUNT] = {"gemm_x_router_down_shared1", "router_select", "dispatch_scan",
                                     "dispatch_finalize", "grouped_gemm1_relu2", "grouped_gemm2",
                                     "combine", "gemm_up_shared2", "expert_mlp"};

struct HipError {
    hipError_t e;
};

inline void hip_check(hipError_t e)
{
    if (e != hipSuccess)
        throw HipError{e};
}

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct Plan {
    int64_t d, l, m, ms, S, N, K, alpha, Tmax;
    int dtype;      // latentmoe_dtype
    int esize;      // bytes per element
    bool fp8;       // routed-expert banks W1/W2 as E4M3 bytes + per-column scales
    int wesize;     // bytes per W1/W2 element
    int bk_b;       // elements per k-tile of the W1/W2 B tiles (128 bytes, 64 for E4M3)
    bool glu;       // gated (SwiGLU) experts: gate and value columns interleaved in the B operands
    int64_t nb1;    // B columns of grouped GEMM 1: m, or 2m when gated
    int64_t ld_zh;  // l + S*ms: row of [z|u , h_s]
    int64_t n_x;    // N' + l + S*ms (gated: N' + l + 2 S*ms): B columns of the pass over x
    int64_t P_max;
};

// The forward's workspace for up to T tokens: routing, dispatch order, the
// grouped GEMMs' tile table, scores, [z|u, h_s], H, Y and split-K partials.
// Rows of expert e sit in [offsets[e], offsets[e+1]) of H and Y.
struct Workspace {
    int *idx, *rank, *pos, *perm;
    float *gate, *logits;
    int *chunk_counts, *chunk_base, *counts, *offsets;
    int4 *tile_info;
    int *tile_rows;  // [tiles + 8][32]: 32-row tables of batches of at most kTinyTokens tokens
    int *n_mtiles;
    void *zh, *H, *Yp;
    float *partial;
    int64_t partial_cap;  // floats at `partial`
    int64_t ld_chunks;    // row length of the expert-major chunk arrays
    int *counters;        // [kSplitCounters] arrival counters of fewrow_split_kernel: zero when
                          // the workspace is made, and each launch leaves them at zero
};

constexpr int kGroupBM = 128, kGroupBMBig = 256, kGroupBMSmall = 32, kMinGroupBM = 32;
constexpr int kGroupSlack = 64;  // extra rows the 256-row tiles take (the kernel's XR)
constexpr int kNoColumn = 1 << 30;  // relu2_from / glu_from: no such columns
constexpr int kSplitKMaxRows = 256, kSplitKMax = 16;
constexpr int kSplitCounters = 4096;  // column groups of 32 of the widest few-row split GEMM
constexpr int kRouteCounter = kSplitCounters - 1;  // route_tiny_kernel's arrival counter

int64_t max_mtiles_for(int64_t P, int64_t N, int bm) { return (P + bm - 1) / bm + std::min<int64_t>(N, P); }

}  // namespace

struct latentmoe_handle {
    latentmoe_config cfg;
    Plan plan;
    int device = 0;
    // repacked weights (one allocation)
    void *wbuf = nullptr;
    void *wcat1T = nullptr, *w1T = nullptr, *w2T = nullptr, *wcat2T = nullptr;
    void *frag1 = nullptr, *frag2 = nullptr;  // fragment-major copies of wcat1T, wcat2T
    float *s1 = nullptr, *s2 = nullptr;  // E4M3 column scales [N', m], [N', l]
    float *bias = nullptr;
    // workspace (one allocation, sized for max_tokens)
    void *ws = nullptr;
    Workspace wk{};
    // this device's address of the static scratch array (latentmoe_forward_noalloc)
    void *scratch = nullptr;
    hipError_t scratch_err = hipSuccess;
    // profiling
    bool prof = false;
    int prof_cap = 0, prof_used = 0;
    uint32_t prof_mask = 0;  // stages timed
    std::vector<hipEvent_t> ev;  // [prof_cap][ST_COUNT][2]
    std::vector<int> ev_used;    // [prof_cap][ST_COUNT]
    // backward pass (allocated by its first call)
    void *bwbuf = nullptr;  // weight layouts of the backward products
    void *bws = nullptr;    // backward workspace
    void *wx_o = nullptr, *wx_of = nullptr;  // [d, n_x] = Wx (rows K = n_x contiguous) + fragment-major copy
    void *wu_o = nullptr, *wu_of = nullptr;  // [l + S m_s, d] = [W_up ; W2_s] + fragment-major copy
    void *w1b = nullptr, *w2b = nullptr;     // per expert [nb1 / bk][l][bk], [l / bk][m][bk]
    void *XA = nullptr;   // [Tmax, l + g S m_s] raw x-pass output (z, shared pre-activations)
    float *Apre = nullptr;  // [Pmax, nb1] routed pre-activations
    void *dUH = nullptr, *dYp = nullptr, *dA = nullptr, *dzp = nullptr, *dX = nullptr;
    void *xT = nullptr, *dXT = nullptr, *zhT = nullptr, *dyT = nullptr;
    void *HT = nullptr, *dYpT = nullptr, *zpT = nullptr, *dAT = nullptr;
    int *koff = nullptr;
    float *dWx = nullptr, *dWu = nullptr, *dW1g = nullptr;
    int64_t Tpad = 0, Ppad = 0;
};

namespace {

int validate(const latentmoe_config *c)
{
    if (!c)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->d <= 0 || c->l <= 0 || c->m <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->alpha <= 0 ||
        c->n_shared < 0 || c->max_tokens <= 0)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->l * c->alpha != c->d)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->n_experts % c->alpha != 0 || c->top_k > c->n_experts)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->variant != LATENTMOE_VARIANT_ACC && c->variant != LATENTMOE_VARIANT_EFF)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->variant == LATENTMOE_VARIANT_ACC && c->top_k % c->alpha != 0)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->dtype != LATENTMOE_DTYPE_F32 && c->dtype != LATENTMOE_DTYPE_BF16)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->has_router_bias != 0 && c->has_router_bias != 1)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->n_shared > 0 && c->m_shared <= 0)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->expert_format != LATENTMOE_EXPERT_AS_DTYPE && c->expert_format != LATENTMOE_EXPERT_FP8_E4M3)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (c->expert_act != LATENTMOE_ACT_RELU2 && c->expert_act != LATENTMOE_ACT_SWIGLU)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    // kernel support
    if (c->expert_format == LATENTMOE_EXPERT_FP8_E4M3 && c->dtype != LATENTMOE_DTYPE_BF16)
        return LATENTMOE_ERR_UNSUPPORTED;
    if (c->d % 64 || c->l % 64 || c->m % 64 || (c->n_shared > 0 && c->m_shared % 64))
        return LATENTMOE_ERR_UNSUPPORTED;
    if (c->n_experts % 16 || c->n_experts > 1024 || c->top_k > 64)
        return LATENTMOE_ERR_UNSUPPORTED;
    const int64_t ms = c->n_shared > 0 ? c->m_shared : 0;
    const int64_t P = c->max_tokens * c->top_k;
    const int64_t widest = std::max<int64_t>({c->d, c->m, c->l + c->n_shared * ms});
    if (P >= (int64_t(1) << 31) || c->max_tokens * widest >= (int64_t(1) << 40) || P * c->m >= (int64_t(1) << 40))
        return LATENTMOE_ERR_UNSUPPORTED;
    // every GEMM operand is addressed through a buffer descriptor with 32-bit
    // offsets: each must stay below 2 GiB
    const int64_t es = c->dtype == LATENTMOE_DTYPE_BF16 ? 2 : 4;
    const int64_t ld_zh = c->l + c->n_shared * ms;
    const int64_t gm = c->expert_act == LATENTMOE_ACT_SWIGLU ? 2 : 1;  // gated: gate beside W1
    const int64_t n_x = c->n_experts + c->l + gm * c->n_shared * ms;
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (c->max_tokens * c->d * es > lim || c->max_tokens * ld_zh * es > lim || P * c->m * es > lim ||
        (n_x + 31) * c->d * es > lim || c->d * ld_zh * es > lim || c->max_tokens * c->n_experts * 4 > lim ||
        gm * c->l * c->m * es > lim)  // one expert's GEMM 1 bank ([W_g | W1] when gated) or W2;
                                       // x-pass rows padded to 32 in the fragment-major copy
        return LATENTMOE_ERR_UNSUPPORTED;
    return LATENTMOE_OK;
}

Plan make_plan(const latentmoe_config *c)
{
    Plan p;
    p.d = c->d;
    p.l = c->l;
    p.m = c->m;
    p.S = c->n_shared;
    p.ms = c->n_shared > 0 ? c->m_shared : 0;
    p.N = c->n_experts;
    p.K = c->top_k;
    p.alpha = c->alpha;
    p.Tmax = c->max_tokens;
    p.dtype = c->dtype;
    p.esize = c->dtype == LATENTMOE_DTYPE_BF16 ? 2 : 4;
    p.fp8 = c->expert_format == LATENTMOE_EXPERT_FP8_E4M3;
    p.wesize = p.fp8 ? 1 : p.esize;
    p.bk_b = p.fp8 ? 64 : 128 / p.esize;
    p.glu = c->expert_act == LATENTMOE_ACT_SWIGLU;
    p.nb1 = p.glu ? 2 * p.m : p.m;
    p.ld_zh = p.l + p.S * p.ms;
    p.n_x = p.N + p.l + p.S * p.ms * (p.glu ? 2 : 1);
    p.P_max = p.Tmax * p.K;
    return p;
}

// fp32 partial sums of split-K GEMMs: up to kSplitKMax splits of the widest
// dense output, for up to kSplitKMaxRows rows of T, and at least the
// kFewRowMaxSplits tiles of 32 x 64 per column group of the few-row split
// kernel (so that its split count does not depend on T)
int64_t split_partial_floats(const Plan &p, int64_t T)
{
    const int64_t wide = std::max(p.n_x, p.d);
    return std::max<int64_t>((int64_t)kSplitKMax * std::min<int64_t>(T, kSplitKMaxRows) * wide,
                             (int64_t)kFewRowMaxSplits * ((wide + 31) / 32) * 2048);
}

struct Layout {
    int64_t off_cnt, off_idx, off_gate, off_rank, off_pos, off_perm, off_cc, off_cb, off_counts, off_offsets, off_ti,
        off_trows, off_nmt, off_logits, off_zh, off_H, off_Yp, off_part, total;
    int64_t ld_chunks, partial_floats;
};

// Byte offsets of a workspace for T tokens with room for `partial_floats`
// split-K partial sums (256-byte aligned pieces).  The split counters come
// first, at the same place for every T.
Layout ws_layout(const Plan &p, int64_t T, int64_t partial_floats)
{
    Layout L;
    int64_t o = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    const int64_t P = T * p.K;
    L.ld_chunks = align_up((T + kRouterTokens - 1) / kRouterTokens, 4);
    L.partial_floats = partial_floats;
    const int64_t mt = max_mtiles_for(P, p.N, kMinGroupBM);
    L.off_cnt = take(4 * kSplitCounters);
    L.off_idx = take(4 * P);
    L.off_gate = take(4 * P);
    L.off_rank = take(4 * P);
    L.off_pos = take(4 * P);
    L.off_perm = take(4 * P);
    L.off_cc = take(4 * L.ld_chunks * p.N);
    L.off_cb = take(4 * L.ld_chunks * p.N);
    L.off_counts = take(4 * p.N);
    L.off_offsets = take(4 * (p.N + 1));
    L.off_ti = take(16 * (mt + 8));  // a decode tile grid reads up to 8 entries past the table
    // the row table serves batches of at most kTinyTokens tokens
    L.off_trows = take(4 * 32 * (max_mtiles_for(std::min<int64_t>(T, kTinyTokens) * p.K, p.N, kMinGroupBM) + 8));
    L.off_nmt = take(4);
    L.off_logits = take(4 * T * p.N);
    L.off_zh = take((int64_t)p.esize * T * p.ld_zh);
    L.off_H = take((int64_t)p.esize * P * p.m);
    L.off_Yp = take((int64_t)p.esize * P * p.l);
    L.off_part = take(4 * partial_floats);
    L.total = o;
    return L;
}

Workspace carve_ws(void *base, const Layout &L)
{
    char *b = static_cast<char *>(base);
    Workspace w;
    w.idx = reinterpret_cast<int *>(b + L.off_idx);
    w.gate = reinterpret_cast<float *>(b + L.off_gate);
    w.rank = reinterpret_cast<int *>(b + L.off_rank);
    w.pos = reinterpret_cast<int *>(b + L.off_pos);
    w.perm = reinterpret_cast<int *>(b + L.off_perm);
    w.chunk_counts = reinterpret_cast<int *>(b + L.off_cc);
    w.chunk_base = reinterpret_cast<int *>(b + L.off_cb);
    w.counts = reinterpret_cast<int *>(b + L.off_counts);
    w.offsets = reinterpret_cast<int *>(b + L.off_offsets);
    w.tile_info = reinterpret_cast<int4 *>(b + L.off_ti);
    w.tile_rows = reinterpret_cast<int *>(b + L.off_trows);
    w.n_mtiles = reinterpret_cast<int *>(b + L.off_nmt);
    w.logits = reinterpret_cast<float *>(b + L.off_logits);
    w.zh = b + L.off_zh;
    w.H = b + L.off_H;
    w.Yp = b + L.off_Yp;
    w.partial = reinterpret_cast<float *>(b + L.off_part);
    w.partial_cap = L.partial_floats;
    w.ld_chunks = L.ld_chunks;
    w.counters = reinterpret_cast<int *>(b + L.off_cnt);
    return w;
}

struct WLayout {
    int64_t off_c1, off_w1, off_w2, off_c2, off_bias, off_s1, off_s2, off_f1, off_f2, total;
};

WLayout w_layout(const Plan &p)
{
    WLayout L;
    int64_t o = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    const int64_t es = p.esize;
    L.off_c1 = take(es * p.n_x * p.d);
    L.off_w1 = take(p.wesize * p.N * p.nb1 * p.l);
    L.off_w2 = take(p.wesize * p.N * p.l * p.m);
    L.off_c2 = take(es * p.d * p.ld_zh);
    L.off_bias = take(4 * p.N);
    L.off_s1 = take(p.fp8 ? 4 * p.N * p.nb1 : 0);
    L.off_s2 = take(p.fp8 ? 4 * p.N * p.l : 0);
    L.off_f1 = take(es * align_up(p.n_x, 32) * p.d);
    L.off_f2 = take(es * align_up(p.d, 32) * p.ld_zh);
    L.total = o;
    return L;
}

template <typename E>
void launch_transpose(const void *src, int64_t R, int64_t C, int64_t batch, int64_t src_bstride, void *dst,
                      int64_t dst_ld, int64_t dst_bstride, hipStream_t s, int glu_off = -1)
{
    constexpr int64_t kMaxZ = 32768;  // grid z stays below the 65535 limit
    for (int64_t b0 = 0; b0 < batch; b0 += kMaxZ) {
        dim3 grid((unsigned)((C + 31) / 32), (unsigned)((R + 31) / 32), (unsigned)std::min(kMaxZ, batch - b0));
        transpose_kernel<E><<<grid, dim3(256), 0, s>>>(static_cast<const E *>(src) + b0 * src_bstride, R, C,
                                                       src_bstride, static_cast<E *>(dst) + b0 * dst_bstride,
                                                       dst_ld, dst_bstride, glu_off);
        hip_check(hipGetLastError());
    }
}

void launch_fragmajor(const void *src, int64_t N, int64_t row_bytes, void *dst, hipStream_t s)
{
    const int64_t units = ((N + 31) / 32) * 32 * (row_bytes / 32) * 2;
    const int64_t blocks = std::min<int64_t>((units + 255) / 256, 65536);
    fragmajor_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(static_cast<const char *>(src), N, row_bytes,
                                                                  static_cast<char *>(dst));
    hip_check(hipGetLastError());
}

template <typename E>
void repack_weights(latentmoe_handle *h, const latentmoe_weights *w, hipStream_t s)
{
    const Plan &p = h->plan;
    char *base = static_cast<char *>(h->wbuf);
    const WLayout L = w_layout(p);
    E *c1 = reinterpret_cast<E *>(base + L.off_c1);
    char *w1 = base + L.off_w1;
    char *w2 = base + L.off_w2;
    E *c2 = reinterpret_cast<E *>(base + L.off_c2);
    // [W_r | W_down | W1_s] [d, N' + l + S m_s] -> K-contiguous rows:
    // W_r^T (N' rows), W_down^T (l rows), then W1_s[j]^T (m_s rows each;
    // gated: 2 m_s rows each, 8 gate rows then 8 value rows per 8 outputs)
    launch_transpose<E>(w->w_router, p.d, p.N, 1, 0, c1, p.d, 0, s);
    launch_transpose<E>(w->w_down, p.d, p.l, 1, 0, c1 + p.N * p.d, p.d, 0, s);
    if (p.S > 0 && p.glu) {
        E *sh = c1 + (p.N + p.l) * p.d;
        launch_transpose<E>(w->w1_shared_gate, p.d, p.ms, p.S, p.d * p.ms, sh, p.d, 2 * p.ms * p.d, s, 0);
        launch_transpose<E>(w->w1_shared, p.d, p.ms, p.S, p.d * p.ms, sh, p.d, 2 * p.ms * p.d, s, 8);
    } else if (p.S > 0) {
        launch_transpose<E>(w->w1_shared, p.d, p.ms, p.S, p.d * p.ms, c1 + (p.N + p.l) * p.d, p.d, p.ms * p.d, s);
    }
    // W1 [N', l, m] -> [N', l / bk, nb1, bk];  W2 [N', m, l] -> [N', m / bk, l, bk]:
    // per expert, k-tile t of B column n sits at (t * cols + n) * bk, so that
    // the B tile of one k-step is one contiguous run.  Gated: nb1 = 2m, the
    // gate matrix and W1 interleaved by 8 columns (transpose_kernel's row
    // map).  E4M3 banks: the same moves of bytes; the scales follow their
    // columns (gated: 8 gate scales, then 8 value scales).
    const int64_t bk = p.bk_b, nb1 = p.nb1;
    auto bank1 = [&](auto tag, const void *src, int glu_off) {
        using T = decltype(tag);
        launch_transpose<T>(src, bk, p.m, p.N * (p.l / bk), bk * p.m, w1, bk, bk * nb1, s, glu_off);
    };
    if (p.fp8) {
        bank1(uint8_t{}, w->w1, p.glu ? 8 : -1);
        if (p.glu)
            bank1(uint8_t{}, w->w1_gate, 0);
        launch_transpose<uint8_t>(w->w2, bk, p.l, p.N * (p.m / bk), bk * p.l, w2, bk, bk * p.l, s);
        h->s1 = reinterpret_cast<float *>(base + L.off_s1);
        h->s2 = reinterpret_cast<float *>(base + L.off_s2);
        if (p.glu) {
            // rows of 8 scales: gate rows to the even 32-byte slots, value rows to the odd ones
            hip_check(hipMemcpy2DAsync(h->s1, 64, w->w1_gate_scale, 32, 32, p.N * p.m / 8, hipMemcpyDeviceToDevice, s));
            hip_check(hipMemcpy2DAsync(reinterpret_cast<char *>(h->s1) + 32, 64, w->w1_scale, 32, 32, p.N * p.m / 8,
                                       hipMemcpyDeviceToDevice, s));
        } else {
            hip_check(hipMemcpyAsync(h->s1, w->w1_scale, 4 * p.N * p.m, hipMemcpyDeviceToDevice, s));
        }
        hip_check(hipMemcpyAsync(h->s2, w->w2_scale, 4 * p.N * p.l, hipMemcpyDeviceToDevice, s));
    } else {
        bank1(E{}, w->w1, p.glu ? 8 : -1);
        if (p.glu)
            bank1(E{}, w->w1_gate, 0);
        launch_transpose<E>(w->w2, bk, p.l, p.N * (p.m / bk), bk * p.l, w2, bk, bk * p.l, s);
    }
    // [W_up ; W2_s] -> [d, l + S m_s]: row i holds W_up[:, i] then W2_s[j][:, i]
    launch_transpose<E>(w->w_up, p.l, p.d, 1, 0, c2, p.ld_zh, 0, s);
    if (p.S > 0)
        launch_transpose<E>(w->w2_shared, p.ms, p.d, p.S, p.ms * p.d, c2 + p.l, p.ld_zh, p.ms, s);
    h->frag1 = base + L.off_f1;
    h->frag2 = base + L.off_f2;
    launch_fragmajor(c1, p.n_x, (int64_t)sizeof(E) * p.d, h->frag1, s);
    launch_fragmajor(c2, p.d, (int64_t)sizeof(E) * p.ld_zh, h->frag2, s);
    h->wcat1T = c1;
    h->w1T = w1;
    h->w2T = w2;
    h->wcat2T = c2;
    h->bias = reinterpret_cast<float *>(base + L.off_bias);
    if (h->cfg.has_router_bias)
        hip_check(hipMemcpyAsync(h->bias, w->b_router, 4 * p.N, hipMemcpyDeviceToDevice, s));
}

// ---- kernel launch helpers -------------------------------------------------

// GEMM stage tags (one kernel symbol per layer stage)
constexpr int kTagX = 0, kTagG1 = 1, kTagG2 = 2, kTagUp = 3;
// backward: data gradients, dense weight gradients, expert-bank weight gradients
constexpr int kTagDgrad = 4, kTagWgrad = 5, kTagWgradE = 6;
// the backward's forward recompute: x-pass and grouped GEMM 1 with raw outputs
constexpr int kTagXRaw = 7, kTagG1Raw = 8;

template <typename E, int BM, int BN, int WM, int WN, int NS, int TAG>
void launch_dense(const GemmParams &gp, hipStream_t s)
{
    const int64_t ntm = (gp.M + BM - 1) / BM, ntn = (gp.N + BN - 1) / BN;
    const int64_t grid = align_up(ntm * ntn, 8);
    gemm_kernel<E, BM, BN, WM, WN, NS, false, 1, TAG><<<dim3((unsigned)grid), dim3(64 * WM * WN), 0, s>>>(gp);
    hip_check(hipGetLastError());
}

template <typename E, int BM, int BN, int WM, int WN, int NS, int TAG, bool BQ8, int ACT = ACT_NONE, int XR = 0>
void launch_grouped(const GemmParams &gp, int64_t max_mtiles, hipStream_t s)
{
    const int64_t ntn = (gp.N + BN - 1) / BN;
    const int64_t grid = align_up(max_mtiles * ntn, 8);
    gemm_kernel<E, BM, BN, WM, WN, NS, true, 1, TAG, BQ8, ACT, XR><<<dim3((unsigned)grid), dim3(64 * WM * WN), 0, s>>>(gp);
    hip_check(hipGetLastError());
}

template <typename E, int TAG>
void launch_splitk(GemmParams gp, float *partial, int64_t cap_floats, hipStream_t s);

template <typename E, int MT, int NW, int COLS, int TAG>
void launch_skinny(const GemmParams &gp, hipStream_t s)
{
    const int64_t grid = (gp.N + COLS - 1) / COLS;
    skinny_gemm_kernel<E, MT, NW, COLS, TAG><<<dim3((unsigned)grid), dim3(64 * NW), 0, s>>>(gp);
    hip_check(hipGetLastError());
}

// Few-row GEMMs with K split over workgroups (fewrow_split_kernel) when the
// 16-column kernel would leave more than a quarter of the CUs without a
// workgroup (N < 3072 columns): 32-column groups, S splits so that about one
// workgroup per CU runs.  Measured at 64 rows: N = 2048, K = 3328 (the decode
// up-projection) 9.9 us with S = 4 against 12.1 us for the 16-column kernel;
// N = 3584, K = 2048 (the decode x-pass) 9.9 us with S = 2 against 9.2 us.
// Returns false (nothing launched) when it does not apply.
template <typename E, int TAG>
bool launch_fewrow(GemmParams gp, float *partial, int64_t cap_floats, int *counters, hipStream_t s)
{
    const int ncg = (gp.N + 31) / 32;
    if (ncg > 96 || ncg > kSplitCounters || !counters)
        return false;
    const int MT = gp.M <= 32 ? 1 : 2;
    const int64_t tile = (int64_t)MT * 1024;  // floats of one split's tile
    const int nkt = gp.K / (128 / (int)sizeof(E));
    int S = std::min(std::min(kFewRowMaxSplits, 256 / ncg), nkt);
    S = (int)std::min<int64_t>(S, cap_floats / (ncg * tile));
    if (S < 2)
        return false;
    const int per = (nkt + S - 1) / S;
    gp.splitk = (nkt + per - 1) / per;  // every split gets at least one k-tile
    gp.partial = partial;
    gp.counters = counters;
    const dim3 grid((unsigned)(ncg * gp.splitk));
    if (MT == 1)
        fewrow_split_kernel<E, 1, 1, 8, TAG><<<grid, dim3(512), 0, s>>>(gp);
    else
        fewrow_split_kernel<E, 2, 1, 8, TAG><<<grid, dim3(512), 0, s>>>(gp);
    hip_check(hipGetLastError());
    return true;
}

// Dense GEMMs: 256x256 tiles (8 waves) when they come close to filling the
// 256 CUs once, else 128x256 (8 waves, three LDS stages) when those fill it,
// else 128x128 (4 waves, two workgroups per CU) when those do; up to
// 64 rows (decode) the few-row kernels (K split over the waves of a
// workgroup, and over workgroups for narrow outputs); otherwise up to
// kSplitKMaxRows rows 64x128 tiles with K split so that ~512 workgroups
// stream the weights, followed by a fixed-order reduce that applies the
// epilogue.
template <typename E, int TAG>
void dense_gemm(const GemmParams &gp, float *partial, int64_t cap_floats, int *counters, hipStream_t s)
{
    const int64_t big = ((gp.M + 255) / 256) * ((gp.N + 255) / 256);
    const int64_t mid = ((gp.M + 127) / 128) * ((gp.N + 127) / 128);
    if (gp.M <= 64 && mid < 256) {
        if (launch_fewrow<E, TAG>(gp, partial, cap_floats, counters, s))
            return;
        if (gp.M <= 32)
            launch_skinny<E, 1, 8, 16, TAG>(gp, s);
        else
            launch_skinny<E, 2, 8, 16, TAG>(gp, s);
        return;
    }
    const int64_t wide = ((gp.M + 127) / 128) * ((gp.N + 255) / 256);
    if (big >= 192) {
        // one 256x256 or 256x320 workgroup per CU: 256x320 when its rounds of
        // 256 tiles times its width come out smaller (zipf_skew's x-pass and
        // up-projection: 3 rounds of 256 columns -> 2 of 320)
        const int64_t ntm = (gp.M + 255) / 256;
        const int64_t r256 = (ntm * ((gp.N + 255) / 256) + 255) / 256, r320 = (ntm * ((gp.N + 319) / 320) + 255) / 256;
        if constexpr (sizeof(E) == 2) {
            if (r320 * 320 < r256 * 256) {
                launch_dense<E, 256, 320, 4, 2, 2, TAG>(gp, s);
                return;
            }
        }
        launch_dense<E, 256, 256, 4, 2, 2, TAG>(gp, s);
    } else if (sizeof(E) == 2 && wide >= 256)
        launch_dense<E, 128, 256, 2, 4, 3, TAG>(gp, s);
    else if (mid >= 256 || gp.M > kSplitKMaxRows)
        launch_dense<E, 128, 128, 2, 2, 2, TAG>(gp, s);
    else
        launch_splitk<E, TAG>(gp, partial, cap_floats, s);
}

template <typename E, int TAG>
void launch_splitk(GemmParams gp, float *partial, int64_t cap_floats, hipStream_t s)
{
    constexpr int BM = 64, BN = 128;
    const int nk = gp.K / (128 / (int)sizeof(E));
    const int64_t tiles = ((gp.M + BM - 1) / BM) * ((gp.N + BN - 1) / BN);
    int S = (int)std::min<int64_t>((512 + tiles - 1) / tiles, kSplitKMax);
    S = std::max(1, std::min(S, nk / 2));
    while (S > 1 && (int64_t)S * gp.M * gp.N > cap_floats)
        --S;
    if (S <= 1) {
        gp.splitk = 1;
        launch_dense<E, BM, BN, 2, 2, 3, TAG>(gp, s);
        return;
    }
    const int per = (nk + S - 1) / S;
    gp.splitk = (nk + per - 1) / per;  // every split gets at least one k-tile
    gp.partial = partial;
    const int64_t grid = align_up(tiles * gp.splitk, 8);
    gemm_kernel<E, BM, BN, 2, 2, 3, false, 1, TAG><<<dim3((unsigned)grid), dim3(256), 0, s>>>(gp);
    hip_check(hipGetLastError());
    const int64_t groups = (int64_t)gp.M * (gp.N / 4);
    splitk_reduce_kernel<E><<<dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s>>>(gp);
    hip_check(hipGetLastError());
}

// Grouped GEMMs: the forward of a bf16 layer with bf16 expert banks takes
// 256x256 tiles (8 waves, two LDS stages) on a 256-row tile table (bm =
// kGroupBMBig) -- 256x320 for grouped GEMM 2 when N = l is a multiple of 320
// but not of 256 and the table has no extra rows (l = 640: two tiles per row
// block instead of three with the third half empty; measured at zipf_skew
// 252-256 -> 234-236 us); otherwise 128x256 tiles (8 waves, three LDS stages, one
// workgroup per CU) when N is a multiple of 256, else 128x128 (two
// workgroups per CU); when experts average few rows (decode), 32x128 tiles
// with four LDS stages so that more weight bytes are in flight, and for
// grouped GEMM 2 (N = l columns) 32x64 tiles of two waves, also four stages:
// 48 KiB of LDS, three workgroups per CU, twice the tiles on 1.5x the slots,
// so a shorter ragged last round (measured at decode_eff: 56.5-57.1 us
// against 57.9-58.8 us with 32x128; grouped GEMM 1 is slower with them,
// 53.2-53.9 -> 55.6-55.9 us).
// fp8: the weights (B) are E4M3 bytes with column scales in gp.scaleB; for few
// rows, 32x64 tiles of two waves and two stages (small LDS footprint, many
// workgroups per CU) stream the half-size weights fastest.
template <typename E, int TAG, int ACT = ACT_NONE>
void grouped_gemm(const GemmParams &gp, int64_t max_mtiles, int bm, bool fp8, hipStream_t s, int slack = 0)
{
    if constexpr (sizeof(E) == 2 && ACT == ACT_NONE) {
        if (bm == kGroupBMBig && !fp8) {
            if (TAG == kTagG2 && slack == 0 && gp.N % 320 == 0 && gp.N % 256 != 0)
                launch_grouped<E, kGroupBMBig, 320, 4, 2, 2, TAG, false>(gp, max_mtiles, s);
            else if (slack == kGroupSlack)
                launch_grouped<E, kGroupBMBig, 256, 4, 2, 2, TAG, false, ACT_NONE, kGroupSlack>(gp, max_mtiles, s);
            else if (slack == 0)
                launch_grouped<E, kGroupBMBig, 256, 4, 2, 2, TAG, false>(gp, max_mtiles, s);
            else
                throw HipError{hipErrorInvalidValue};
            return;
        }
        if (fp8) {
            if (bm == kGroupBMSmall)
                launch_grouped<E, kGroupBMSmall, 64, 1, 2, 2, TAG, true>(gp, max_mtiles, s);
            else
                launch_grouped<E, kGroupBM, 128, 2, 2, 2, TAG, true>(gp, max_mtiles, s);
            return;
        }
    }
    if ((bm != kGroupBMSmall && bm != kGroupBM) || slack != 0)  // a tile table these kernels cannot walk
        throw HipError{hipErrorInvalidValue};
    if (bm == kGroupBMSmall && TAG == kTagG2)
        launch_grouped<E, kGroupBMSmall, 64, 1, 2, 4, TAG, false, ACT>(gp, max_mtiles, s);
    else if (bm == kGroupBMSmall)
        launch_grouped<E, kGroupBMSmall, 128, 1, 4, 4, TAG, false, ACT>(gp, max_mtiles, s);
    else if (sizeof(E) == 2 && gp.N % 256 == 0)
        launch_grouped<E, kGroupBM, 256, 2, 4, 3, TAG, false, ACT>(gp, max_mtiles, s);
    else
        launch_grouped<E, kGroupBM, 128, 2, 2, 2, TAG, false, ACT>(gp, max_mtiles, s);
}

// Rows per tile of the grouped GEMMs' tile table: 32 when experts average
// fewer than 32 rows; else 256 where the 256x256 kernel serves both grouped
// GEMMs (big: the forward of a bf16 layer with bf16 banks; measured on the
// layer at t_exp = 256..512 rows per expert, its lower cost per row outweighs
// the longer padding of each expert's last tile), else 128.
int group_bm_for(int64_t P, int64_t N, bool big = false)
{
    return (P / N < 32) ? kGroupBMSmall : big ? kGroupBMBig : kGroupBM;
}

// Fused routed-expert MLP (expert_mlp.hpp): Y = act(z[perm] W1_e) W2_e with
// H kept on chip, for bf16 forwards with bf16 banks and prefill-sized row
// counts.  Rows per tile (the tile table's BM) and the wave layouts depend
// on l, which sets the register tile of Y [BM, l]: l = 512 takes 128-row
// tiles (64 x 128 of Y per wave).  At l = 1024 only 64-row tiles fit, which
// streams each expert's weights twice as often; measured slower than the two
// grouped GEMMs there, so that width keeps the unfused path.  Returns 0 where
// no instance serves the layer.
constexpr int kMlpMC = 128;  // hidden columns per chunk

int mlp_bm_for(const Plan &p, int64_t P, bool train)
{
    if (train || p.fp8 || p.esize != 2 || p.glu || P / p.N < 32 || p.m % kMlpMC)
        return 0;
    if (p.l == 512)
        return 128;
    return 0;
}

template <int BM, int LW, int KS2, int NS, int WM1, int WN1, int WM2, int WN2>
void launch_mlp_n(const MlpParams &mp, int64_t max_mtiles, hipStream_t s)
{
    using K = MlpShape<BM, LW, kMlpMC, KS2, NS, WM1, WN1, WM2, WN2, false>;
    static_assert(K::lds_bytes() <= 160 * 1024, "LDS");
    expert_mlp_kernel<BM, LW, kMlpMC, KS2, NS, WM1, WN1, WM2, WN2, false, 0>
        <<<dim3((unsigned)align_up(max_mtiles, 8)), dim3(512), 0, s>>>(mp);
    hip_check(hipGetLastError());
}

void launch_mlp(const Plan &p, const MlpParams &mp, int64_t max_mtiles, hipStream_t s)
{
    if (p.l == 512)  // four 32 KiB slots: three steps in flight
        launch_mlp_n<128, 512, 32, 4, 4, 2, 2, 4>(mp, max_mtiles, s);
    else
        throw HipError{hipErrorInvalidValue};
}

// Selection: kRouterTokens tokens per workgroup with the chunk counts and
// ranks of the chunked dispatch; batches of at most kTinyTokens tokens take
// kTinySelectWaves tokens per workgroup and the mask dispatch instead.
template <int NPL, int TOK, bool CHUNKS>
void launch_select_n(const Plan &p, const Workspace &w, int T, hipStream_t s)
{
    const int blocks = (T + TOK - 1) / TOK;
    router_select_kernel<NPL, TOK, CHUNKS>
        <<<dim3(blocks), dim3(64 * TOK), router_select_smem_bytes((int)p.N, (int)p.K, TOK, CHUNKS), s>>>(
            w.logits, T, (int)p.N, (int)p.K, w.idx, w.gate, w.rank, w.chunk_counts, (int)w.ld_chunks);
    hip_check(hipGetLastError());
}

template <int NPL>
void launch_select_tok(const Plan &p, const Workspace &w, int T, hipStream_t s)
{
    if (T <= kTinyTokens)
        launch_select_n<NPL, kTinySelectWaves, false>(p, w, T, s);
    else
        launch_select_n<NPL, kRouterTokens, true>(p, w, T, s);
}

// Decode batches: selection and dispatch order in one launch (route_tiny.hpp).
template <int NPL>
void launch_route_tiny_n(const TinyRouteParams &rp, hipStream_t s)
{
    const int blocks = (rp.T + kTinySelectWaves - 1) / kTinySelectWaves;
    route_tiny_kernel<NPL><<<dim3(blocks), dim3(kRouteTinyThreads), route_tiny_smem_bytes(rp.K), s>>>(rp);
    hip_check(hipGetLastError());
}

void launch_route_tiny(const Plan &p, const Workspace &w, int T, int bm, int slack, bool row_table, hipStream_t s)
{
    TinyRouteParams rp{};
    rp.scores = w.logits;
    rp.T = T;
    rp.N = (int)p.N;
    rp.K = (int)p.K;
    rp.idx = w.idx;
    rp.gate = w.gate;
    rp.counter = w.counters + kRouteCounter;
    rp.BM = bm;
    rp.slack = slack;
    rp.counts = w.counts;
    rp.offsets = w.offsets;
    rp.tile_info = w.tile_info;
    rp.n_mtiles = w.n_mtiles;
    rp.pos = w.pos;
    rp.perm = w.perm;
    rp.tile_rows = row_table ? w.tile_rows : nullptr;
    const int64_t npl = (p.N + 63) / 64;
    if (npl <= 1)
        launch_route_tiny_n<1>(rp, s);
    else if (npl <= 2)
        launch_route_tiny_n<2>(rp, s);
    else if (npl <= 4)
        launch_route_tiny_n<4>(rp, s);
    else if (npl <= 8)
        launch_route_tiny_n<8>(rp, s);
    else
        launch_route_tiny_n<16>(rp, s);
}

void launch_select(const Plan &p, const Workspace &w, int T, hipStream_t s)
{
    const int64_t npl = (p.N + 63) / 64;
    if (npl <= 1)
        launch_select_tok<1>(p, w, T, s);
    else if (npl <= 2)
        launch_select_tok<2>(p, w, T, s);
    else if (npl <= 4)
        launch_select_tok<4>(p, w, T, s);
    else if (npl <= 8)
        launch_select_tok<8>(p, w, T, s);
    else
        launch_select_tok<16>(p, w, T, s);
}

// ---- the forward -----------------------------------------------------------

struct StageTimer {
    latentmoe_handle *h;
    hipStream_t s;
    int slot;
    void begin(int st)
    {
        if (slot >= 0 && ((h->prof_mask >> st) & 1u))
            hip_check(hipEventRecord(h->ev[((size_t)slot * ST_COUNT + st) * 2], s));
    }
    void end(int st)
    {
        if (slot >= 0 && ((h->prof_mask >> st) & 1u)) {
            hip_check(hipEventRecord(h->ev[((size_t)slot * ST_COUNT + st) * 2 + 1], s));
            h->ev_used[(size_t)slot * ST_COUNT + st] = 1;
        }
    }
};

void copy2d(void *dst, int64_t dst_pitch, const void *src, int64_t src_pitch, int64_t width, int64_t rows,
            hipStream_t s)
{
    hip_check(hipMemcpy2DAsync(dst, dst_pitch, src, src_pitch, width, rows, hipMemcpyDeviceToDevice, s));
}

// train: the forward the backward pass recomputes.  The x-pass writes its
// raw output (z and the shared pre-activations) to XA and grouped GEMM 1 its
// pre-activations in fp32 to Apre; small kernels then form h_s and H.  u
// ends in zh beside h_s; y is not formed.
template <typename E>
void forward_impl(latentmoe_handle *h, const Workspace &w, const void *x, void *y, int T, hipStream_t s,
                  const latentmoe_debug *dbg, bool train = false)
{
    const Plan &p = h->plan;
    const int N = (int)p.N, K = (int)p.K;
    const int64_t P = (int64_t)T * K;
    const int nchunks = (T + kRouterTokens - 1) / kRouterTokens;
    const int es = p.esize;
    const int mlp_bm = mlp_bm_for(p, P, train);
    const int gbm = mlp_bm ? mlp_bm : group_bm_for(P, N, !train && !p.fp8 && es == 2);
    // 256-row tiles: when experts average at most 256 + kGroupSlack rows, an
    // expert's last tile takes up to kGroupSlack more rows, so an expert a few
    // rows past 256 streams its weights once (measured: wide_prefill's grouped
    // GEMMs -7 %); with more rows per expert (zipf_skew: 512 on average) the
    // larger A stage of those tiles costs more than the tails it saves (+3 %)
    const int slack = (gbm == kGroupBMBig && P <= (int64_t)N * (kGroupBMBig + kGroupSlack)) ? kGroupSlack : 0;
    const int64_t max_mt = max_mtiles_for(P, N, gbm);
    StageTimer tm{h, s, -1};
    if (h->prof && h->prof_used < h->prof_cap)
        tm.slot = h->prof_used++;

    // 0: [s | z | h_s] = x [W_r | W_down | W1_s]
    GemmParams g{};
    g.A = x;
    g.lda = p.d;
    g.a_bytes = (int64_t)T * p.d * es;
    g.B = h->wcat1T;
    g.Bfrag = h->frag1;
    g.ldb = p.d;
    g.C32 = w.logits;
    g.ldc32 = p.N;
    g.bias32 = h->cfg.has_router_bias ? h->bias : nullptr;
    g.c_split = N;
    g.C = w.zh;
    g.ldc = p.ld_zh;
    g.M = T;
    g.N = (int)p.n_x;
    g.K = (int)p.d;
    g.relu2_from = p.glu ? kNoColumn : (int)p.l;
    g.glu_from = p.glu ? (int)(p.N + p.l) : kNoColumn;
    g.group_m = 8;
    const int64_t ld_xa = p.n_x - p.N;  // l + g S m_s
    if (train) {
        g.C = h->XA;
        g.ldc = ld_xa;
        g.relu2_from = kNoColumn;
        g.glu_from = kNoColumn;
    }
    tm.begin(ST_GEMM_X);
    if (train)
        dense_gemm<E, kTagXRaw>(g, w.partial, w.partial_cap, w.counters, s);
    else
        dense_gemm<E, kTagX>(g, w.partial, w.partial_cap, w.counters, s);
    if (train) {
        const int64_t n = (int64_t)T * p.ld_zh;
        xpass_act_kernel<E><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
            static_cast<const E *>(h->XA), ld_xa, T, (int)p.l, (int)(p.S * p.ms), p.glu ? 1 : 0,
            static_cast<E *>(w.zh), p.ld_zh);
        hip_check(hipGetLastError());
    }
    tm.end(ST_GEMM_X);
    if (dbg && dbg->logits)
        hip_check(hipMemcpyAsync(dbg->logits, w.logits, 4 * (size_t)T * N, hipMemcpyDeviceToDevice, s));
    if (dbg && dbg->z)
        copy2d(dbg->z, es * p.l, w.zh, es * p.ld_zh, es * p.l, T, s);
    if (dbg && dbg->h_shared && p.S > 0)
        copy2d(dbg->h_shared, es * (p.ld_zh - p.l), static_cast<char *>(w.zh) + es * p.l, es * p.ld_zh,
               es * (p.ld_zh - p.l), T, s);

    // per-tile A-row table for 32-row tiles of decode batches: the first
    // grouped GEMM's workgroups load their A rows together with the tile record
    // (measured: bf16 experts -2.9 us in that GEMM, +0.6 us in the dispatch;
    // E4M3 experts gain nothing there, so they go through perm)
    const bool row_table = T <= kTinyTokens && gbm == kGroupBMSmall && !p.fp8;
    if (T <= kTinyTokens) {
        // 1-4 for decode batches in one launch: selection, and in its last
        // workgroup the dispatch order (measured at decode_eff: -2 us)
        tm.begin(ST_SELECT);
        launch_route_tiny(p, w, T, gbm, slack, row_table, s);
        tm.end(ST_SELECT);
    } else {
        // 1: top-K', gates, chunk ranks
        tm.begin(ST_SELECT);
        launch_select(p, w, T, s);
        tm.end(ST_SELECT);
    }
    // 2-4: dispatch order of larger batches (up to 64 chunks: one workgroup,
    // one launch)
    if (T > kTinyTokens && nchunks <= 64) {
        tm.begin(ST_FINALIZE);
        dispatch_small_kernel<<<dim3(1), dim3(1024), 0, s>>>(
            w.chunk_counts, nchunks, w.idx, w.rank, T, K, N, kRouterTokens, (int)w.ld_chunks, gbm, slack, w.chunk_base,
            w.counts, w.offsets, w.tile_info, w.n_mtiles, w.pos, w.perm);
        hip_check(hipGetLastError());
        tm.end(ST_FINALIZE);
    } else if (T > kTinyTokens) {
        tm.begin(ST_SCAN);
        chunk_scan_kernel<<<dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s>>>(w.chunk_counts, nchunks,
                                                                              (int)w.ld_chunks, N, w.chunk_base,
                                                                              w.counts);
        hip_check(hipGetLastError());
        tm.end(ST_SCAN);
        tm.begin(ST_FINALIZE);
        const int64_t blocks = std::min<int64_t>((P + 1023) / 1024, 256);
        finalize_kernel<<<dim3((unsigned)blocks), dim3(1024), 0, s>>>(
            w.idx, w.rank, w.chunk_base, w.counts, T, K, N, kRouterTokens, (int)w.ld_chunks, gbm, slack,
            w.offsets, w.tile_info, w.n_mtiles, w.pos, w.perm);
        hip_check(hipGetLastError());
        tm.end(ST_FINALIZE);
    }

    // 5: H = relu(z[perm] W1_e)^2
    GemmParams g1{};
    g1.A = w.zh;
    g1.lda = p.ld_zh;
    g1.a_bytes = (int64_t)T * p.ld_zh * es;
    g1.B = h->w1T;
    g1.ldb = p.bk_b;
    g1.b_kstep = p.nb1 * p.bk_b * p.wesize;
    g1.strideB = p.nb1 * p.l;
    g1.C = w.H;
    g1.ldc = p.m;
    g1.N = (int)p.nb1;
    g1.K = (int)p.l;
    g1.relu2_from = p.glu ? kNoColumn : 0;
    g1.glu_from = p.glu ? 0 : kNoColumn;
    g1.gather = w.perm;
    g1.tile_info = w.tile_info;
    g1.tile_rows = row_table ? w.tile_rows : nullptr;
    g1.n_mtiles = w.n_mtiles;
    g1.offsets = w.offsets;
    g1.scaleB = h->s1;
    if (train) {  // raw pre-activations in fp32 beside H
        g1.C32 = h->Apre;
        g1.ldc32 = p.nb1;
        g1.c_split = (int)p.nb1;
        g1.relu2_from = kNoColumn;
        g1.glu_from = kNoColumn;
    }
    if (mlp_bm) {
        // 5 + 6 fused: Y = relu(z[perm] W1_e)^2 W2_e, H on chip
        MlpParams mp{};
        mp.Z = w.zh;
        mp.ldz = p.ld_zh;
        mp.z_bytes = (int64_t)T * p.ld_zh * es;
        mp.gather = w.perm;
        mp.W1 = h->w1T;
        mp.W2 = h->w2T;
        mp.Y = w.Yp;
        mp.l = (int)p.l;
        mp.m = (int)p.m;
        mp.nb1 = (int)p.nb1;
        mp.tile_info = w.tile_info;
        mp.n_mtiles = w.n_mtiles;
        mp.offsets = w.offsets;
        tm.begin(ST_MLP);
        launch_mlp(p, mp, max_mt, s);
        tm.end(ST_MLP);
        // H exists only as a debug output here: the grouped GEMM forms it.
        // On a 64-row tile table its 128-row tiles start at each entry's
        // first row, so some rows are written twice, with identical bits.
        if (dbg && dbg->h)
            grouped_gemm<E, kTagG1>(g1, max_mt, kGroupBM, false, s);
    } else {
    tm.begin(ST_GEMM1);
    if (train && p.glu)
        grouped_gemm<E, kTagG1Raw, ACT_GLU>(g1, max_mt, gbm, false, s);
    else if (train)
        grouped_gemm<E, kTagG1Raw, ACT_RELU2>(g1, max_mt, gbm, false, s);
    else
        grouped_gemm<E, kTagG1>(g1, max_mt, gbm, p.fp8, s, slack);
    tm.end(ST_GEMM1);

    // 6: Y = H W2_e
    GemmParams g2 = g1;
    g2.tile_rows = nullptr;  // A = H in dispatch order
    g2.A = w.H;
    g2.lda = p.m;
    g2.a_bytes = P * p.m * es;
    g2.B = h->w2T;
    g2.ldb = p.bk_b;
    g2.b_kstep = p.l * p.bk_b * p.wesize;
    g2.strideB = p.l * p.m;
    g2.C = w.Yp;
    g2.ldc = p.l;
    g2.N = (int)p.l;
    g2.K = (int)p.m;
    g2.relu2_from = kNoColumn;
    g2.glu_from = kNoColumn;
    g2.gather = nullptr;
    g2.scaleB = h->s2;
    g2.C32 = nullptr;
    g2.c_split = 0;
    tm.begin(ST_GEMM2);
    grouped_gemm<E, kTagG2>(g2, max_mt, gbm, p.fp8, s, slack);
    tm.end(ST_GEMM2);
    }

    // 7: u = sum_k gate Y[pos], written over z (z is dead after stage 5)
    tm.begin(ST_COMBINE);
    // decode batches: all of a chunk's slot loads in flight at once (measured at
    // decode_eff: 0.1250 -> 0.1239 ms per step; even or slower for prefill)
    if (T <= kTinyTokens)
        combine_kernel<E, true><<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s>>>(
            static_cast<const E *>(w.Yp), w.pos, w.gate, T, K, (int)p.l, static_cast<E *>(w.zh), p.ld_zh);
    else
        combine_kernel<E><<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s>>>(
            static_cast<const E *>(w.Yp), w.pos, w.gate, T, K, (int)p.l, static_cast<E *>(w.zh), p.ld_zh);
    hip_check(hipGetLastError());
    tm.end(ST_COMBINE);
    if (train)
        return;

    // 8: y = [u | h_s] [W_up ; W2_s]
    GemmParams g3{};
    g3.A = w.zh;
    g3.lda = p.ld_zh;
    g3.a_bytes = (int64_t)T * p.ld_zh * es;
    g3.B = h->wcat2T;
    g3.Bfrag = h->frag2;
    g3.ldb = p.ld_zh;
    g3.C = y;
    g3.ldc = p.d;
    g3.M = T;
    g3.N = (int)p.d;
    g3.K = (int)p.ld_zh;
    g3.relu2_from = kNoColumn;
    g3.glu_from = kNoColumn;
    g3.group_m = 8;
    tm.begin(ST_GEMM_UP);
    dense_gemm<E, kTagUp>(g3, w.partial, w.partial_cap, w.counters, s);
    tm.end(ST_GEMM_UP);

    if (dbg) {
        if (dbg->idx)
            hip_check(hipMemcpyAsync(dbg->idx, w.idx, 4 * P, hipMemcpyDeviceToDevice, s));
        if (dbg->gate)
            hip_check(hipMemcpyAsync(dbg->gate, w.gate, 4 * P, hipMemcpyDeviceToDevice, s));
        if (dbg->counts)
            hip_check(hipMemcpyAsync(dbg->counts, w.counts, 4 * p.N, hipMemcpyDeviceToDevice, s));
        if (dbg->offsets)
            hip_check(hipMemcpyAsync(dbg->offsets, w.offsets, 4 * (p.N + 1), hipMemcpyDeviceToDevice, s));
        if (dbg->perm_token)
            hip_check(hipMemcpyAsync(dbg->perm_token, w.perm, 4 * P, hipMemcpyDeviceToDevice, s));
        if (dbg->pos)
            hip_check(hipMemcpyAsync(dbg->pos, w.pos, 4 * P, hipMemcpyDeviceToDevice, s));
        if (dbg->h)
            hip_check(hipMemcpyAsync(dbg->h, w.H, (size_t)es * P * p.m, hipMemcpyDeviceToDevice, s));
        if (dbg->y_perm)
            hip_check(hipMemcpyAsync(dbg->y_perm, w.Yp, (size_t)es * P * p.l, hipMemcpyDeviceToDevice, s));
        if (dbg->u)
            copy2d(dbg->u, es * p.l, w.zh, es * p.ld_zh, es * p.l, T, s);
    }
}

const Workspace &handle_ws(const latentmoe_handle *h) { return h->wk; }

// ---- workspace of latentmoe_forward_noalloc ---------------------------------

// The forward's workspace for callers that cannot allocate: a static array in
// the code object, one copy on each GPU the library runs on, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address is looked up with hipGetSymbolAddress
// (once per device, with that device current, from latentmoe_create) and only
// that address is ever handed to kernels.
constexpr int64_t kScratchBytes = LATENTMOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxScratchDevices] = {};

// Device address of `scratch` on `device` (which must be current).
hipError_t scratch_address(int device, void **out)
{
    *out = nullptr;
    if (device < 0 || device >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[device]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return e != hipSuccess ? e : hipErrorInvalidSymbol;
        // the split counters at the start of every workspace layout start at
        // zero (the kernels leave them so)
        e = hipMemset(ptr, 0, sizeof(int) * kSplitCounters);
        if (e == hipSuccess)
            e = hipDeviceSynchronize();
        if (e != hipSuccess)
            return e;
        g_scratch_addr[device] = ptr;
    }
    *out = g_scratch_addr[device];
    return hipSuccess;
}

void free_handle(latentmoe_handle *h)
{
    if (!h)
        return;
    for (hipEvent_t e : h->ev)
        if (e)
            (void)hipEventDestroy(e);
    if (h->wbuf)
        (void)hipFree(h->wbuf);
    if (h->ws)
        (void)hipFree(h->ws);
    if (h->bwbuf)
        (void)hipFree(h->bwbuf);
    if (h->bws)
        (void)hipFree(h->bws);
    delete h;
}

double log10_comb(double n, double k) { return (std::lgamma(n + 1) - std::lgamma(k + 1) - std::lgamma(n - k + 1)) / std::log(10.0); }

// ---- backward pass -----------------------------------------------------

// Weight gradients from MN-major bf16 operands (gemm_tn.hpp): 128x128 tiles,
// one grid over every batch.
template <int TAG>
void launch_tn(const GemmParams &gp, hipStream_t s)
{
    const int64_t per = ((gp.M + 127) / 128) * ((gp.N + 127) / 128);
    const int64_t tiles = (gp.k_offsets ? gp.n_batches : 1) * per;
    gemm_tn_kernel<TAG><<<dim3((unsigned)align_up(tiles, 8)), dim3(256), 0, s>>>(gp);
    hip_check(hipGetLastError());
}

// z_perm[p] = z[perm[p]] (the first l columns of the recompute's raw x-pass
// output XA), 16 bytes per thread.
template <typename E>
__global__ __launch_bounds__(256) void gather_rows_kernel(const E *__restrict__ src, int64_t ld_src,
                                                          const int *__restrict__ perm, int64_t P, int cols,
                                                          E *__restrict__ dst)
{
    constexpr int VEC = 16 / (int)sizeof(E);
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per = cols / VEC;
    if (q >= P * per)
        return;
    const int64_t r = q / per;
    const int c = (int)(q - r * per) * VEC;
    *reinterpret_cast<uint4 *>(dst + r * cols + c) = *reinterpret_cast<const uint4 *>(src + perm[r] * ld_src + c);
}

template <typename E, int TAG>
void launch_batched_k(const GemmParams &gp, hipStream_t s)
{
    constexpr int BM = 128, BN = 128;
    const int64_t tiles = (int64_t)gp.n_batches * ((gp.M + BM - 1) / BM) * ((gp.N + BN - 1) / BN);
    gemm_kernel<E, BM, BN, 2, 2, 2, false, 1, TAG><<<dim3((unsigned)align_up(tiles, 8)), dim3(256), 0, s>>>(gp);
    hip_check(hipGetLastError());
}

template <typename E>
void launch_pad_transpose(const void *src, int64_t ld_src, int rows, int C, const int *gather, const int *offs,
                          const int *koff, int nseg, void *dst, int64_t ld_dst, hipStream_t s)
{
    constexpr int VEC = 16 / (int)sizeof(E);
    if (reinterpret_cast<uintptr_t>(src) % 16 == 0 && ld_src % VEC == 0 && C % VEC == 0 && ld_dst % 64 == 0) {
        dim3 grid((unsigned)((C + 63) / 64), (unsigned)(ld_dst / 64));
        pad_transpose64_kernel<E><<<grid, dim3(256), 0, s>>>(static_cast<const E *>(src), ld_src, rows, C, gather,
                                                             offs, koff, nseg, static_cast<E *>(dst), ld_dst);
        hip_check(hipGetLastError());
        return;
    }
    dim3 grid((unsigned)((C + 31) / 32), (unsigned)(ld_dst / 32));
    pad_transpose_kernel<E><<<grid, dim3(256), 0, s>>>(static_cast<const E *>(src), ld_src, rows, C, gather, offs,
                                                       koff, nseg, static_cast<E *>(dst), ld_dst);
    hip_check(hipGetLastError());
}

int64_t n_x_padded(const Plan &p) { return align_up(p.n_x, 64); }

// Bytes of the backward's weight layouts and workspace.
struct BwdLayout {
    int64_t off_wx, off_wxf, off_wu, off_wuf, off_w1b, off_w2b, wtotal;
    int64_t off_xa, off_apre, off_duh, off_dyp, off_da, off_dzp, off_dx, off_xt, off_dxt, off_zht, off_dyt,
        off_ht, off_dypt, off_zpt, off_dat, off_koff, off_dwx, off_dwu, off_dw1g, total;
    int64_t Tpad, Ppad;
};

BwdLayout bwd_layout(const Plan &p)
{
    BwdLayout L{};
    const int64_t es = p.esize, nxp = n_x_padded(p), ldxa = p.n_x - p.N;
    int64_t o = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    L.off_wx = take(es * p.d * nxp);
    L.off_wxf = take(es * align_up(p.d, 32) * nxp);
    L.off_wu = take(es * p.ld_zh * p.d);
    L.off_wuf = take(es * align_up(p.ld_zh, 32) * p.d);
    L.off_w1b = take(es * p.N * p.l * p.nb1);
    L.off_w2b = take(es * p.N * p.m * p.l);
    L.wtotal = o;
    o = 0;
    L.Tpad = align_up(p.Tmax, 64);
    L.Ppad = align_up(p.P_max + 64 * p.N, 64);  // >= sum over experts of their rows rounded up to 64
    L.off_xa = take(es * p.Tmax * ldxa);
    L.off_apre = take(4 * p.P_max * p.nb1);
    L.off_duh = take(es * p.Tmax * p.ld_zh);
    L.off_dyp = take(es * p.P_max * p.l);
    L.off_da = take(es * p.P_max * p.nb1);
    L.off_dzp = take(es * p.P_max * p.l);
    L.off_dx = take(es * p.Tmax * nxp);
    // transposed, zero-padded operands of the fp32 layers' weight gradients;
    // bf16 layers read the activations in place (gemm_tn.hpp) and need only
    // z_perm (P x l, in the zpT area)
    const bool tr = es == 4;
    L.off_xt = take(tr ? es * p.d * L.Tpad : 0);
    L.off_dxt = take(tr ? es * nxp * L.Tpad : 0);
    L.off_zht = take(tr ? es * p.ld_zh * L.Tpad : 0);
    L.off_dyt = take(tr ? es * p.d * L.Tpad : 0);
    L.off_ht = take(tr ? es * p.m * L.Ppad : 0);
    L.off_dypt = take(tr ? es * p.l * L.Ppad : 0);
    L.off_zpt = take(tr ? es * p.l * L.Ppad : es * p.P_max * p.l);
    L.off_dat = take(tr ? es * p.nb1 * L.Ppad : 0);
    L.off_koff = take(4 * (p.N + 1));
    L.off_dwx = take(4 * p.d * p.n_x);
    L.off_dwu = take(4 * p.ld_zh * p.d);
    L.off_dw1g = take(p.glu ? 4 * p.N * p.l * p.nb1 : 0);
    L.total = o;
    return L;
}

// Every operand the backward reads through a buffer descriptor stays below
// 2 GiB (32-bit offsets).
bool bwd_fits(const Plan &p)
{
    const BwdLayout L = bwd_layout(p);
    const int64_t es = p.esize, lim = (int64_t(1) << 31) - 1;
    const int64_t sizes[] = {es * p.d * n_x_padded(p), es * p.ld_zh * p.d, es * p.l * p.nb1, es * p.m * p.l,
                             4 * p.P_max * p.nb1, es * p.P_max * p.nb1, es * p.Tmax * n_x_padded(p),
                             es * p.P_max * p.m, es * p.P_max * p.l};
    for (int64_t v : sizes)
        if (v > lim)
            return false;
    if (es == 4) {  // the transposed operands of the fp32 layers' weight gradients
        const int64_t tr[] = {es * n_x_padded(p) * L.Tpad, es * p.d * L.Tpad, es * p.ld_zh * L.Tpad,
                              es * p.m * L.Ppad, es * p.l * L.Ppad, es * p.nb1 * L.Ppad};
        for (int64_t v : tr)
            if (v > lim)
                return false;
    }
    return true;
}

// The first backward call on a handle: the weight layouts of the backward
// products (from the handle's own repacked copies) and the workspace.
template <typename E>
void backward_setup(latentmoe_handle *h, hipStream_t s)
{
    const Plan &p = h->plan;
    const BwdLayout L = bwd_layout(p);
    const int64_t es = p.esize, nxp = n_x_padded(p);
    if (device_alloc(&h->bwbuf, L.wtotal) != hipSuccess)
        throw HipError{hipErrorOutOfMemory};
    if (device_alloc(&h->bws, L.total) != hipSuccess)
        throw HipError{hipErrorOutOfMemory};
    char *w = static_cast<char *>(h->bwbuf);
    char *b = static_cast<char *>(h->bws);
    h->wx_o = w + L.off_wx;
    h->wx_of = w + L.off_wxf;
    h->wu_o = w + L.off_wu;
    h->wu_of = w + L.off_wuf;
    h->w1b = w + L.off_w1b;
    h->w2b = w + L.off_w2b;
    h->XA = b + L.off_xa;
    h->Apre = reinterpret_cast<float *>(b + L.off_apre);
    h->dUH = b + L.off_duh;
    h->dYp = b + L.off_dyp;
    h->dA = b + L.off_da;
    h->dzp = b + L.off_dzp;
    h->dX = b + L.off_dx;
    h->xT = b + L.off_xt;
    h->dXT = b + L.off_dxt;
    h->zhT = b + L.off_zht;
    h->dyT = b + L.off_dyt;
    h->HT = b + L.off_ht;
    h->dYpT = b + L.off_dypt;
    h->zpT = b + L.off_zpt;
    h->dAT = b + L.off_dat;
    h->koff = reinterpret_cast<int *>(b + L.off_koff);
    h->dWx = reinterpret_cast<float *>(b + L.off_dwx);
    h->dWu = reinterpret_cast<float *>(b + L.off_dwu);
    h->dW1g = p.glu ? reinterpret_cast<float *>(b + L.off_dw1g) : nullptr;
    h->Tpad = L.Tpad;
    h->Ppad = L.Ppad;
    // columns n_x .. n_xp of Wx and of dX stay zero (the dx product runs over
    // the padded width, a multiple of the k-tile)
    hip_check(hipMemsetAsync(h->wx_o, 0, es * p.d * nxp, s));
    hip_check(hipMemsetAsync(h->dX, 0, es * p.Tmax * nxp, s));
    // Wx [d, n_x]: the transpose of the x-pass's [n_x, d] rows (same column
    // order, gated pairs included); [W_up ; W2_s] [l + S m_s, d] likewise
    launch_transpose<E>(h->wcat1T, p.n_x, p.d, 1, 0, h->wx_o, nxp, 0, s);
    launch_transpose<E>(h->wcat2T, p.d, p.ld_zh, 1, 0, h->wu_o, p.d, 0, s);
    launch_fragmajor(h->wx_o, p.d, es * nxp, h->wx_of, s);
    launch_fragmajor(h->wu_o, p.ld_zh, es * p.d, h->wu_of, s);
    // expert banks with rows and K swapped: dH = dY W2^T reads W2 with rows
    // m and K = l; dz = dA W1^T reads W1 with rows l and K = nb1
    constexpr int BK = 128 / (int)sizeof(E);
    retile_kernel<E, BK><<<dim3((unsigned)(p.nb1 / BK), (unsigned)(p.l / BK), (unsigned)p.N), dim3(256), 0, s>>>(
        static_cast<const E *>(h->w1T), (int)p.l, (int)p.nb1, static_cast<E *>(h->w1b));
    hip_check(hipGetLastError());
    retile_kernel<E, BK><<<dim3((unsigned)(p.l / BK), (unsigned)(p.m / BK), (unsigned)p.N), dim3(256), 0, s>>>(
        static_cast<const E *>(h->w2T), (int)p.m, (int)p.l, static_cast<E *>(h->w2b));
    hip_check(hipGetLastError());
}

// Weight gradients of a bf16 layer, read straight from the row-major
// activations by the MN-major GEMM: dW_x = x^T [ds | dz | d pre_s],
// [dW_up ; dW2_s] = [u | h_s]^T dy, and per expert dW2 = H^T dY_perm and
// [dW_g | dW1] = z_perm^T dA over the expert's dispatch rows.
void weight_grads_tn(latentmoe_handle *h, const void *x, const void *dy, int T, hipStream_t s,
                     const latentmoe_grads *gr)
{
    const Plan &p = h->plan;
    const int N = (int)p.N;
    const int64_t P = (int64_t)T * p.K, es = 2, nxp = n_x_padded(p), ldxa = p.n_x - p.N;
    auto tn = [&](const void *A, int64_t lda, int64_t a_rows, const void *B, int64_t ldb, int M, int Nn, float *C) {
        GemmParams g{};
        g.A = A;
        g.lda = lda;
        g.a_bytes = a_rows * lda * es;
        g.B = B;
        g.ldb = ldb;
        g.b_bytes = a_rows * ldb * es;
        g.M = M;
        g.N = Nn;
        g.K = (int)a_rows;
        g.C32 = C;
        g.ldc32 = Nn;
        g.c_split = Nn;
        g.group_m = 8;
        return g;
    };
    if (gr->dw_router || gr->dw_down || gr->dw1_shared || gr->dw1_shared_gate) {
        launch_tn<kTagWgrad>(tn(x, p.d, T, h->dX, nxp, (int)p.d, (int)p.n_x, h->dWx), s);
        auto split = [&](float *dst, int rows, int col0, int nb, int w, int sel) {
            const int64_t n = (int64_t)nb * rows * w;
            split_cols_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(h->dWx, p.n_x, rows, col0, nb,
                                                                                    w, sel, dst);
            hip_check(hipGetLastError());
        };
        if (gr->dw_router)
            split(gr->dw_router, (int)p.d, 0, 1, N, -1);
        if (gr->dw_down)
            split(gr->dw_down, (int)p.d, N, 1, (int)p.l, -1);
        if (p.S > 0 && gr->dw1_shared)
            split(gr->dw1_shared, (int)p.d, (int)(p.N + p.l), (int)p.S, (int)p.ms, p.glu ? 1 : -1);
        if (p.S > 0 && p.glu && gr->dw1_shared_gate)
            split(gr->dw1_shared_gate, (int)p.d, (int)(p.N + p.l), (int)p.S, (int)p.ms, 0);
    }
    if (gr->dw_up || gr->dw2_shared) {
        launch_tn<kTagWgrad>(tn(h->wk.zh, p.ld_zh, T, dy, p.d, (int)p.ld_zh, (int)p.d, h->dWu), s);
        if (gr->dw_up)
            hip_check(hipMemcpyAsync(gr->dw_up, h->dWu, 4 * p.l * p.d, hipMemcpyDeviceToDevice, s));
        if (p.S > 0 && gr->dw2_shared)
            hip_check(hipMemcpyAsync(gr->dw2_shared, h->dWu + p.l * p.d, 4 * p.S * p.ms * p.d,
                                     hipMemcpyDeviceToDevice, s));
    }
    if (h->cfg.has_router_bias && gr->db_router) {
        col_sum_kernel<bf16><<<dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s>>>(
            static_cast<const bf16 *>(h->dX), nxp, T, N, gr->db_router);
        hip_check(hipGetLastError());
    }
    if (gr->dw2) {
        GemmParams g = tn(h->wk.H, p.m, P, h->dYp, p.l, (int)p.m, (int)p.l, gr->dw2);
        g.k_offsets = h->wk.offsets;
        g.n_batches = N;
        launch_tn<kTagWgradE>(g, s);
    }
    if (gr->dw1 || (p.glu && gr->dw1_gate)) {
        const int64_t n = P * p.l / 8;
        gather_rows_kernel<bf16><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
            static_cast<const bf16 *>(h->XA), ldxa, h->wk.perm, P, (int)p.l, static_cast<bf16 *>(h->zpT));
        hip_check(hipGetLastError());
        float *dst = p.glu ? h->dW1g : gr->dw1;
        GemmParams g = tn(h->zpT, p.l, P, h->dA, p.nb1, (int)p.l, (int)p.nb1, dst);
        g.k_offsets = h->wk.offsets;
        g.n_batches = N;
        launch_tn<kTagWgradE>(g, s);
        if (p.glu) {  // [N' l, 2m] gated pairs -> W1 (value) and W_g (gate)
            const int64_t nn = p.N * p.l * p.m;
            for (int sel = 0; sel < 2; ++sel) {
                float *out = sel ? gr->dw1 : gr->dw1_gate;
                if (!out)
                    continue;
                split_cols_kernel<<<dim3((unsigned)((nn + 255) / 256)), dim3(256), 0, s>>>(
                    h->dW1g, p.nb1, (int)(p.N * p.l), 0, 1, (int)p.m, sel, out);
                hip_check(hipGetLastError());
            }
        }
    }
}

template <typename E>
void backward_impl(latentmoe_handle *h, const void *x, const void *dy, int T, hipStream_t s,
                   const latentmoe_grads *gr)
{
    const Plan &p = h->plan;
    const int N = (int)p.N, K = (int)p.K;
    const int64_t P = (int64_t)T * K, es = p.esize, nxp = n_x_padded(p), ldxa = p.n_x - p.N;
    const int gbm = group_bm_for(P, N);
    const int64_t max_mt = max_mtiles_for(P, N, gbm);
    const int64_t Tp = align_up(T, 64);
    const int gl = p.glu ? 1 : 0;
    const int sms = (int)(p.S * p.ms);

    forward_impl<E>(h, handle_ws(h), x, nullptr, T, s, nullptr, true);

    // [du | dh_s] = dy [W_up ; W2_s]^T
    GemmParams ga{};
    ga.A = dy;
    ga.lda = p.d;
    ga.a_bytes = (int64_t)T * p.d * es;
    ga.B = h->wu_o;
    ga.Bfrag = h->wu_of;
    ga.ldb = p.d;
    ga.C = h->dUH;
    ga.ldc = p.ld_zh;
    ga.M = T;
    ga.N = (int)p.ld_zh;
    ga.K = (int)p.d;
    ga.group_m = 8;
    dense_gemm<E, kTagDgrad>(ga, h->wk.partial, h->wk.partial_cap, h->wk.counters, s);
    // shared experts: the gradient of their pre-activations -> dX[:, N' + l ..]
    if (sms > 0) {
        const int64_t n = (int64_t)T * sms;
        shared_act_grad_kernel<E><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
            static_cast<const E *>(h->XA), ldxa, static_cast<const E *>(h->dUH), p.ld_zh, T, (int)p.l, sms, gl,
            static_cast<E *>(h->dX), nxp, (int)(p.N + p.l));
        hip_check(hipGetLastError());
    }
    // gates and combine: dY_perm, and ds -> dX[:, 0 .. N')
    gate_combine_grad_kernel<E><<<dim3((unsigned)T), dim3(256), 0, s>>>(
        static_cast<const E *>(h->dUH), p.ld_zh, static_cast<const E *>(h->wk.Yp), h->wk.pos, h->wk.idx, h->wk.gate, K,
        (int)p.l, N, static_cast<E *>(h->dYp), static_cast<E *>(h->dX), nxp);
    hip_check(hipGetLastError());
    // dH = dY_perm W2_e^T; its epilogue writes the gradient of the routed
    // pre-activations dA = dH act'(A) instead of dH
    GemmParams gb{};
    gb.A = h->dYp;
    gb.lda = p.l;
    gb.a_bytes = P * p.l * es;
    gb.B = h->w2b;
    gb.ldb = p.bk_b;
    gb.b_kstep = p.m * p.bk_b * es;
    gb.strideB = p.m * p.l;
    gb.C = h->dA;
    gb.ldc = p.nb1;
    gb.act_pre = h->Apre;
    gb.ld_pre = p.nb1;
    gb.N = (int)p.m;
    gb.K = (int)p.l;
    gb.tile_info = h->wk.tile_info;
    gb.n_mtiles = h->wk.n_mtiles;
    gb.offsets = h->wk.offsets;
    if (p.glu)
        grouped_gemm<E, kTagDgrad, ACT_GLU_GRAD>(gb, max_mt, gbm, false, s);
    else
        grouped_gemm<E, kTagDgrad, ACT_RELU2_GRAD>(gb, max_mt, gbm, false, s);
    // dz_perm = dA W1_e^T; dz[t] = sum over t's slots -> dX[:, N' .. N' + l)
    GemmParams gc = gb;
    gc.act_pre = nullptr;
    gc.A = h->dA;
    gc.lda = p.nb1;
    gc.a_bytes = P * p.nb1 * es;
    gc.B = h->w1b;
    gc.b_kstep = p.l * p.bk_b * es;
    gc.strideB = p.l * p.nb1;
    gc.C = h->dzp;
    gc.ldc = p.l;
    gc.N = (int)p.l;
    gc.K = (int)p.nb1;
    grouped_gemm<E, kTagDgrad>(gc, max_mt, gbm, false, s);
    {
        const int64_t n = (int64_t)T * p.l / 8;
        gather_sum8_kernel<E><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
            static_cast<const E *>(h->dzp), h->wk.pos, T, K, (int)p.l, static_cast<E *>(h->dX), nxp, N);
        hip_check(hipGetLastError());
    }
    // dx = [ds | dz | d pre_s] Wx^T
    if (gr->dx) {
        GemmParams gd{};
        gd.A = h->dX;
        gd.lda = nxp;
        gd.a_bytes = (int64_t)T * nxp * es;
        gd.B = h->wx_o;
        gd.Bfrag = h->wx_of;
        gd.ldb = nxp;
        gd.C = gr->dx;
        gd.ldc = p.d;
        gd.M = T;
        gd.N = (int)p.d;
        gd.K = (int)nxp;
        gd.group_m = 8;
        dense_gemm<E, kTagDgrad>(gd, h->wk.partial, h->wk.partial_cap, h->wk.counters, s);
    }

    // ---- weight gradients (fp32), sums over tokens / an expert's rows ----
    if constexpr (sizeof(E) == 2) {
        weight_grads_tn(h, x, dy, T, s, gr);
        return;
    }
    auto wgrad = [&](const void *A, int64_t M, const void *B, int64_t Nn, int64_t lda, float *C) {
        GemmParams g{};
        g.A = A;
        g.lda = lda;
        g.a_bytes = M * lda * es;
        g.B = B;
        g.ldb = lda;
        g.C32 = C;
        g.ldc32 = Nn;
        g.c_split = (int)Nn;
        g.M = (int)M;
        g.N = (int)Nn;
        g.K = (int)lda;
        g.group_m = 8;
        return g;
    };
    // tokens padded to 64 with zero columns
    launch_pad_transpose<E>(x, p.d, T, (int)p.d, nullptr, nullptr, nullptr, 0, h->xT, Tp, s);
    launch_pad_transpose<E>(h->dX, nxp, T, (int)p.n_x, nullptr, nullptr, nullptr, 0, h->dXT, Tp, s);
    launch_pad_transpose<E>(h->wk.zh, p.ld_zh, T, (int)p.ld_zh, nullptr, nullptr, nullptr, 0, h->zhT, Tp, s);
    launch_pad_transpose<E>(dy, p.d, T, (int)p.d, nullptr, nullptr, nullptr, 0, h->dyT, Tp, s);
    if (gr->dw_router || gr->dw_down || gr->dw1_shared || gr->dw1_shared_gate) {
        GemmParams g = wgrad(h->xT, p.d, h->dXT, p.n_x, Tp, h->dWx);
        launch_dense<E, 128, 128, 2, 2, 2, kTagWgrad>(g, s);
        auto split = [&](float *dst, int rows, int col0, int nb, int w, int sel) {
            const int64_t n = (int64_t)nb * rows * w;
            split_cols_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(h->dWx, p.n_x, rows, col0, nb,
                                                                                    w, sel, dst);
            hip_check(hipGetLastError());
        };
        if (gr->dw_router)
            split(gr->dw_router, (int)p.d, 0, 1, N, -1);
        if (gr->dw_down)
            split(gr->dw_down, (int)p.d, N, 1, (int)p.l, -1);
        if (p.S > 0 && gr->dw1_shared)
            split(gr->dw1_shared, (int)p.d, (int)(p.N + p.l), (int)p.S, (int)p.ms, p.glu ? 1 : -1);
        if (p.S > 0 && p.glu && gr->dw1_shared_gate)
            split(gr->dw1_shared_gate, (int)p.d, (int)(p.N + p.l), (int)p.S, (int)p.ms, 0);
    }
    if (gr->dw_up || gr->dw2_shared) {
        GemmParams g = wgrad(h->zhT, p.ld_zh, h->dyT, p.d, Tp, h->dWu);
        launch_dense<E, 128, 128, 2, 2, 2, kTagWgrad>(g, s);
        if (gr->dw_up)
            hip_check(hipMemcpyAsync(gr->dw_up, h->dWu, 4 * p.l * p.d, hipMemcpyDeviceToDevice, s));
        if (p.S > 0 && gr->dw2_shared)
            hip_check(hipMemcpyAsync(gr->dw2_shared, h->dWu + p.l * p.d, 4 * p.S * p.ms * p.d,
                                     hipMemcpyDeviceToDevice, s));
    }
    if (h->cfg.has_router_bias && gr->db_router) {
        col_sum_kernel<E><<<dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s>>>(static_cast<const E *>(h->dX), nxp,
                                                                                  T, N, gr->db_router);
        hip_check(hipGetLastError());
    }
    // expert banks: per expert a sum over its rows, padded to 64 per expert
    const bool need1 = gr->dw1 || (p.glu && gr->dw1_gate);
    if (gr->dw2 || need1) {
        padded_offsets_kernel<<<dim3(1), dim3(1024), 0, s>>>(h->wk.counts, N, 64, h->koff);
        hip_check(hipGetLastError());
    }
    if (gr->dw2) {
        launch_pad_transpose<E>(h->wk.H, p.m, (int)P, (int)p.m, nullptr, h->wk.offsets, h->koff, N, h->HT, h->Ppad, s);
        launch_pad_transpose<E>(h->dYp, p.l, (int)P, (int)p.l, nullptr, h->wk.offsets, h->koff, N, h->dYpT, h->Ppad, s);
        GemmParams g = wgrad(h->HT, p.m, h->dYpT, p.l, h->Ppad, gr->dw2);
        g.k_offsets = h->koff;
        g.n_batches = N;
        launch_batched_k<E, kTagWgradE>(g, s);
    }
    if (need1) {
        launch_pad_transpose<E>(h->XA, ldxa, (int)P, (int)p.l, h->wk.perm, h->wk.offsets, h->koff, N, h->zpT, h->Ppad, s);
        launch_pad_transpose<E>(h->dA, p.nb1, (int)P, (int)p.nb1, nullptr, h->wk.offsets, h->koff, N, h->dAT, h->Ppad,
                                s);
        float *dst = p.glu ? h->dW1g : gr->dw1;
        GemmParams g = wgrad(h->zpT, p.l, h->dAT, p.nb1, h->Ppad, dst);
        g.k_offsets = h->koff;
        g.n_batches = N;
        launch_batched_k<E, kTagWgradE>(g, s);
        if (p.glu) {  // [N' l, 2m] gated pairs -> W1 (value) and W_g (gate)
            const int64_t n = p.N * p.l * p.m;
            for (int sel = 0; sel < 2; ++sel) {
                float *out = sel ? gr->dw1 : gr->dw1_gate;
                if (!out)
                    continue;
                split_cols_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
                    h->dW1g, p.nb1, (int)(p.N * p.l), 0, 1, (int)p.m, sel, out);
                hip_check(hipGetLastError());
            }
        }
    }
}

}  // namespace

extern "C" {

const char *latentmoe_status_string(int status)
{
    switch (status) {
    case LATENTMOE_OK: return "ok";
    case LATENTMOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LATENTMOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LATENTMOE_ERR_OUT_OF_MEMORY: return "out of device memory";
    case LATENTMOE_ERR_HIP: return "HIP runtime error";
    case LATENTMOE_ERR_EXCEEDS_SCRATCH: return "token count needs more workspace than the static scratch array holds";
    default: return "unknown status";
    }
}

int latentmoe_last_hip_error(void) { return g_last_hip_error; }

int latentmoe_validate_config(const latentmoe_config *cfg) { return validate(cfg); }

int latentmoe_workspace_bytes(const latentmoe_config *cfg, int64_t *bytes)
{
    const int st = validate(cfg);
    if (st != LATENTMOE_OK)
        return st;
    if (!bytes)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    const Plan p = make_plan(cfg);
    *bytes = ws_layout(p, p.Tmax, split_partial_floats(p, p.Tmax)).total + w_layout(p).total;
    return LATENTMOE_OK;
}

int latentmoe_cost(const latentmoe_config *c, latentmoe_cost_out *o)
{
    const int st = validate(c);
    if (st != LATENTMOE_OK)
        return st;
    if (!o)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    const double d = (double)c->d, l = (double)c->l, m = (double)c->m, N = (double)c->n_experts,
                 K = (double)c->top_k, a = (double)c->alpha, S = (double)c->n_shared,
                 ms = c->n_shared > 0 ? (double)c->m_shared : 0.0;
    // expert matrices: two, or three for gated experts (a gate beside W1)
    const double em = c->expert_act == LATENTMOE_ACT_SWIGLU ? 3.0 : 2.0;
    std::memset(o, 0, sizeof *o);
    o->latent_expert_params = em * l * m;
    o->routed_pool_params = N * em * l * m;
    o->projection_params = 2 * d * l;
    o->router_params = d * N;
    o->shared_params = S * em * d * ms;
    o->layer_params_excl_router = o->routed_pool_params + o->shared_params + o->projection_params;
    o->active_params_per_token = K * em * l * m + o->shared_params + o->projection_params;
    o->expert_bytes_per_token_fp8 = K * em * l * m;
    o->expert_bytes_per_token_bf16 = K * em * l * m * 2;
    o->a2a_bytes_per_token = K * l * (0.5 + 2.0);
    o->flops_per_token = 2 * (d * N + 2 * d * l + em * K * l * m + em * S * d * ms);
    o->log10_combinations = log10_comb(N, K);
    const double Nb = N / a, Kb = c->variant == LATENTMOE_VARIANT_ACC ? K / a : K;
    o->baseline_n_experts = Nb;
    o->baseline_top_k = Kb;
    o->baseline_expert_params = em * d * m;
    o->baseline_layer_params_excl_router = Nb * em * d * m + o->shared_params;
    o->baseline_active_params_per_token = Kb * em * d * m + o->shared_params;
    o->baseline_a2a_bytes_per_token = Kb * d * (0.5 + 2.0);
    o->baseline_log10_combinations = log10_comb(Nb, Kb);
    o->log10_combination_bound = a * o->baseline_log10_combinations;
    return LATENTMOE_OK;
}

int latentmoe_create(const latentmoe_config *cfg, const latentmoe_weights *w, void *hip_stream,
                     latentmoe_handle **out)
{
    if (!out)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    const int st = validate(cfg);
    if (st != LATENTMOE_OK)
        return st;
    if (!w || !w->w_router || !w->w_down || !w->w1 || !w->w2 || !w->w_up)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (cfg->n_shared > 0 && (!w->w1_shared || !w->w2_shared))
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (cfg->has_router_bias && !w->b_router)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (cfg->expert_format == LATENTMOE_EXPERT_FP8_E4M3 && (!w->w1_scale || !w->w2_scale))
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (cfg->expert_act == LATENTMOE_ACT_SWIGLU &&
        (!w->w1_gate || (cfg->n_shared > 0 && !w->w1_shared_gate) ||
         (cfg->expert_format == LATENTMOE_EXPERT_FP8_E4M3 && !w->w1_gate_scale)))
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    latentmoe_handle *h = new (std::nothrow) latentmoe_handle();
    if (!h)
        return LATENTMOE_ERR_OUT_OF_MEMORY;
    h->cfg = *cfg;
    h->plan = make_plan(cfg);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    try {
        hip_check(hipGetDevice(&h->device));
        h->scratch_err = scratch_address(h->device, &h->scratch);
        if (h->scratch_err != hipSuccess)
            (void)hipGetLastError();  // only latentmoe_forward_noalloc needs it; it reports the error
        const Plan &p = h->plan;
        const WLayout WL = w_layout(p);
        const Layout L = ws_layout(p, p.Tmax, split_partial_floats(p, p.Tmax));
        if (device_alloc(&h->wbuf, WL.total) != hipSuccess) {
            (void)hipGetLastError();
            free_handle(h);
            return LATENTMOE_ERR_OUT_OF_MEMORY;
        }
        if (device_alloc(&h->ws, L.total) != hipSuccess) {
            (void)hipGetLastError();
            free_handle(h);
            return LATENTMOE_ERR_OUT_OF_MEMORY;
        }
        h->wk = carve_ws(h->ws, L);
        hip_check(hipMemsetAsync(h->wk.counters, 0, sizeof(int) * kSplitCounters, s));
        if (p.dtype == LATENTMOE_DTYPE_BF16)
            repack_weights<bf16>(h, w, s);
        else
            repack_weights<float>(h, w, s);
        hip_check(hipStreamSynchronize(s));
    } catch (const HipError &e) {
        g_last_hip_error = (int)e.e;
        free_handle(h);
        return LATENTMOE_ERR_HIP;
    } catch (const std::bad_alloc &) {
        free_handle(h);
        return LATENTMOE_ERR_OUT_OF_MEMORY;
    }
    *out = h;
    return LATENTMOE_OK;
}

int latentmoe_backward(latentmoe_handle *h, const void *x, const void *dy, int64_t T, void *hip_stream,
                       const latentmoe_grads *g)
{
    if (!h || !x || !dy || !g || T < 1 || T > h->plan.Tmax)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (g->db_router && !h->cfg.has_router_bias)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (h->plan.fp8)
        return LATENTMOE_ERR_UNSUPPORTED;
    if (!bwd_fits(h->plan))
        return LATENTMOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    try {
        if (!h->bwbuf) {
            if (h->plan.dtype == LATENTMOE_DTYPE_BF16)
                backward_setup<bf16>(h, s);
            else
                backward_setup<float>(h, s);
        }
        if (h->plan.dtype == LATENTMOE_DTYPE_BF16)
            backward_impl<bf16>(h, x, dy, (int)T, s, g);
        else
            backward_impl<float>(h, x, dy, (int)T, s, g);
    } catch (const HipError &e) {
        g_last_hip_error = (int)e.e;
        if (e.e == hipErrorOutOfMemory && !h->bws) {  // setup failed: the next call tries again
            (void)hipGetLastError();
            (void)hipFree(h->bwbuf);
            h->bwbuf = nullptr;
            return LATENTMOE_ERR_OUT_OF_MEMORY;
        }
        return LATENTMOE_ERR_HIP;
    }
    return LATENTMOE_OK;
}

int latentmoe_forward(latentmoe_handle *h, const void *x, void *y, int64_t T, void *hip_stream,
                      const latentmoe_debug *dbg)
{
    if (!h || !x || !y || T < 1 || T > h->plan.Tmax)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    const int64_t bytes = T * h->plan.d * h->plan.esize;
    const char *xb = static_cast<const char *>(x);
    const char *yb = static_cast<const char *>(y);
    if (xb < yb + bytes && yb < xb + bytes)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    try {
        if (h->plan.dtype == LATENTMOE_DTYPE_BF16)
            forward_impl<bf16>(h, handle_ws(h), x, y, (int)T, s, dbg);
        else
            forward_impl<float>(h, handle_ws(h), x, y, (int)T, s, dbg);
    } catch (const HipError &e) {
        g_last_hip_error = (int)e.e;
        return LATENTMOE_ERR_HIP;
    }
    return LATENTMOE_OK;
}

int latentmoe_forward_noalloc(latentmoe_handle *h, const void *x, void *y, int64_t T, void *hip_stream)
{
    if (!h || !x || !y || T < 1 || T > h->plan.Tmax)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    const Plan &p = h->plan;
    const int64_t bytes = T * p.d * p.esize;
    const char *xb = static_cast<const char *>(x);
    const char *yb = static_cast<const char *>(y);
    if (xb < yb + bytes && yb < xb + bytes)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    if (!h->scratch) {
        g_last_hip_error = (int)h->scratch_err;
        return LATENTMOE_ERR_HIP;
    }
    // the workspace for T tokens; split-K partial sums take what is left
    const Layout base = ws_layout(p, T, 0);
    if (base.total > kScratchBytes)
        return LATENTMOE_ERR_EXCEEDS_SCRATCH;
    const int64_t room = (kScratchBytes - base.total) / 4;
    const Layout L = ws_layout(p, T, std::min(split_partial_floats(p, T), room));
    if (L.total > kScratchBytes)
        return LATENTMOE_ERR_EXCEEDS_SCRATCH;
    const Workspace w = carve_ws(h->scratch, L);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    try {
        if (p.dtype == LATENTMOE_DTYPE_BF16)
            forward_impl<bf16>(h, w, x, y, (int)T, s, nullptr);
        else
            forward_impl<float>(h, w, x, y, (int)T, s, nullptr);
    } catch (const HipError &e) {
        g_last_hip_error = (int)e.e;
        return LATENTMOE_ERR_HIP;
    }
    return LATENTMOE_OK;
}

int latentmoe_destroy(latentmoe_handle *h)
{
    free_handle(h);
    return LATENTMOE_OK;
}

int latentmoe_profile_begin(latentmoe_handle *h, int max_forwards, uint32_t stage_mask)
{
    if (!h || max_forwards < 1 || max_forwards > 100000 || (stage_mask & ((1u << ST_COUNT) - 1u)) == 0)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    try {
        for (hipEvent_t e : h->ev)
            if (e)
                hip_check(hipEventDestroy(e));
        h->ev.assign((size_t)max_forwards * ST_COUNT * 2, nullptr);
        h->ev_used.assign((size_t)max_forwards * ST_COUNT, 0);
        for (auto &e : h->ev)
            hip_check(hipEventCreate(&e));
    } catch (const HipError &e) {
        g_last_hip_error = (int)e.e;
        return LATENTMOE_ERR_HIP;
    }
    h->prof = true;
    h->prof_mask = stage_mask & ((1u << ST_COUNT) - 1u);
    h->prof_cap = max_forwards;
    h->prof_used = 0;
    return LATENTMOE_OK;
}

int latentmoe_profile_end(latentmoe_handle *h, double *ms, int32_t *launches, int32_t *n_stages)
{
    if (!h || !ms || !launches || !n_stages || !h->prof)
        return LATENTMOE_ERR_INVALID_ARGUMENT;
    for (int s = 0; s < LATENTMOE_MAX_STAGES; ++s) {
        ms[s] = 0.0;
        launches[s] = 0;
    }
    try {
        for (int f = 0; f < h->prof_used; ++f)
            for (int s = 0; s < ST_COUNT; ++s) {
                if (!h->ev_used[(size_t)f * ST_COUNT + s])
                    continue;
                hipEvent_t a = h->ev[((size_t)f * ST_COUNT + s) * 2], b = h->ev[((size_t)f * ST_COUNT + s) * 2 + 1];
                hip_check(hipEventSynchronize(b));
                float t = 0.f;
                hip_check(hipEventElapsedTime(&t, a, b));
                ms[s] += t;
                launches[s] += 1;
            }
    } catch (const HipError &e) {
        g_last_hip_error = (int)e.e;
        return LATENTMOE_ERR_HIP;
    }
    *n_stages = ST_COUNT;
    h->prof = false;
    return LATENTMOE_OK;
}

const char *latentmoe_stage_name(int stage)
{
    if (stage < 0 || stage >= ST_COUNT)
        return "";
    return kStageNames[stage];
}

}  // extern "C"
