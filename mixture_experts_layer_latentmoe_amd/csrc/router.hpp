// Router selection: top-K' of the scores, renormalised gates, and the first
// step of the dispatch histogram, fused in one kernel.
//
// Page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through
// Equations, Architecture, Code and ...": Figure 3 (one score per expert,
// softmax, keep the K largest), Figure 8 (the router reads x at the full
// width d, before the down-projection) and the MoE code block (the K kept
// weights are renormalised to sum to one).
//
// The scores s = x W_r (+ b) come from the same MFMA pass over x that
// produces z and the shared-expert hidden layer (their weights are one
// concatenated matrix), stored in fp32.  This kernel owns 16 tokens (one
// dispatch chunk), 16 waves, one token per wave -- small chunks keep every
// CU busy at a few thousand tokens.  Batches of at most kTinyTokens tokens
// take workgroups of 4 tokens (one wave per SIMD: the selection is a chain of
// dependent wave operations, and four waves sharing a SIMD take four times as
// long) and skip step 4 (route_tiny.hpp orders them by token masks):
//   1. scores become order-preserving 32-bit keys (-0.0 folded into +0.0, so
//      signed zeros tie); a 32-round radix search, counting with wave ballots,
//      finds the K'-th largest key; every key above it is selected, and of the
//      keys equal to it the lowest expert indices fill the remaining slots;
//   2. the selected keys are ranked (score descending, index ascending) by
//      comparing each against the others through LDS;
//   3. gate_k = exp(s_k - s_max) / sum_j exp(s_j - s_max) over the selected
//      set, which is the renormalised softmax (its denominator cancels); s_k
//      and s_max come back from the keys, the sum is a fixed-order DPP
//      reduction;
//   4. a bit mask per expert marks which tokens of the chunk chose it;
//      popcounts give each (token, slot) its rank inside the chunk and the
//      chunk's count per expert -- integer-exact, independent of the order of
//      the atomic ORs.  Counts are stored expert-major: [N'][ld_chunks].
#pragma once

#include "common.hpp"

namespace lmoe {

constexpr int kRouterTokens = 16;  // tokens per workgroup = one dispatch chunk
constexpr int kSelectWaves = 16;
constexpr int kTinyTokens = 64;    // batches up to this size: mask dispatch (64-bit token masks)
constexpr int kTinySelectWaves = 4;

__device__ __forceinline__ unsigned ordered_key(float v)
{
    v = (v == 0.f) ? 0.f : v;  // -0.0 and +0.0 tie
    const unsigned u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // > 0 for every finite v
}

__device__ __forceinline__ float key_value(unsigned k)
{
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__device__ __forceinline__ int wave_count(bool pred) { return __popcll(__ballot(pred)); }

// Sum over the 64 lanes in a fixed order with DPP moves (no LDS round trips):
// swaps inside quads, mirrors inside half-rows and rows (every lane then holds
// its row's sum), row 0 into row 1 and row 2 into row 3, then rows 0-1 into
// row 3; the total is lane 63's.
__device__ __forceinline__ float wave_sum_dpp(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// A token's scores in registers: expert e = lane + 64 j in val[j] (0 past N').
template <int NPL>
__device__ __forceinline__ void load_scores(const float *__restrict__ row, int N, int lane, float (&val)[NPL])
{
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int e = lane + 64 * j;
        val[j] = (e < N) ? row[e] : 0.f;
    }
}

// Steps 1-3 for one token (one wave) from its scores in registers: the K'
// selected experts, each selected lane's rank and renormalised gate (lanes <
// K' hold slot `lane`).  wkey, wexp: this wave's K'-entry LDS scratch.
template <int NPL>
__device__ __forceinline__ void select_token_vals(const float (&val)[NPL], int N, int K, int lane, unsigned *wkey,
                                                  int *wexp, int &me_out, int &rank_out, float &gate_out)
{
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    unsigned key[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int e = lane + 64 * j;
        key[j] = (e < N) ? ordered_key(val[j]) : 0u;
    }
    // 1. the K'-th largest key: largest th with #{key >= th} >= K'.  Once a
    // candidate has exactly K' keys at or above it, those keys are the
    // selection (every key equal to th is among them, so step 1's tie rule
    // takes all of them) and the lower bits need not be resolved.
    unsigned th = 0u;
    for (int b = 31; b >= 0; --b) {
        const unsigned cand = th | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j)
            cnt += wave_count(key[j] >= cand);
        if (cnt >= K) {
            th = cand;
            if (cnt == K)
                break;
        }
    }
    int need = K;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
        need -= wave_count(key[j] > th);
    // selection, compacted into LDS slots in (j, lane) order
    int base = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const bool tie = key[j] == th;
        const unsigned long long tmask = __ballot(tie);
        const int tie_rank = __popcll(tmask & lt_mask);   // among this j's ties, lower lanes first
        const bool sel = key[j] > th || (tie && tie_rank < need);
        need -= min(need, (int)__popcll(tmask));
        const unsigned long long smask = __ballot(sel);
        if (sel) {
            const int slot = base + __popcll(smask & lt_mask);
            wkey[slot] = key[j];
            wexp[slot] = lane + 64 * j;
        }
        base += __popcll(smask);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // 2. rank of slot `lane` by (key descending, index ascending); the
    // largest selected key on the way
    unsigned mk = 0u, top = 0u;
    int me = 0x7fffffff, rank = 0;
    if (lane < K) {
        mk = wkey[lane];
        me = wexp[lane];
        for (int q = 0; q < K; ++q) {
            const unsigned ok = wkey[q];
            const int oe = wexp[q];
            rank += (ok > mk || (ok == mk && oe < me)) ? 1 : 0;
            top = max(top, ok);
        }
    }
    // 3. gates from the scores the keys encode (a key maps back to its score
    // exactly, -0.0 as +0.0, which changes no difference)
    const float g = (lane < K) ? expf(key_value(mk) - key_value(top)) : 0.f;
    const float gsum = wave_sum_dpp(g);
    me_out = me;
    rank_out = rank;
    gate_out = g / gsum;
}

template <int NPL>
__device__ __forceinline__ void select_token(const float *__restrict__ row, int N, int K, int lane, unsigned *wkey,
                                             int *wexp, int &me_out, int &rank_out, float &gate_out)
{
    float val[NPL];
    load_scores<NPL>(row, N, lane, val);
    select_token_vals<NPL>(val, N, K, lane, wkey, wexp, me_out, rank_out, gate_out);
}

// NPL = ceil(N' / 64) scores held per lane (expert e = lane + 64 j); TOK
// tokens per workgroup, one per wave; CHUNKS: also step 4 (a workgroup's
// tokens are one dispatch chunk).
template <int NPL, int TOK, bool CHUNKS>
__global__ __launch_bounds__(64 * TOK) void router_select_kernel(
    const float *__restrict__ scores, int T, int N, int K, int *__restrict__ idx_out, float *__restrict__ gate_out,
    int *__restrict__ rank_out, int *__restrict__ chunk_counts, int ld_chunks)
{
    static_assert(TOK >= 1 && TOK <= 32, "token mask per chunk");
    extern __shared__ int rsmem[];
    unsigned *s_key = reinterpret_cast<unsigned *>(rsmem);  // [TOK waves][K]
    int *s_exp = rsmem + TOK * K;                           // [TOK waves][K]
    int *s_idx = s_exp + TOK * K;                           // [TOK][K]    (CHUNKS)
    unsigned *s_mask = reinterpret_cast<unsigned *>(s_idx + TOK * K);  // [N] (CHUNKS)
    const int tid = threadIdx.x, lane = tid & 63, r = tid >> 6;
    const int t0 = blockIdx.x * TOK, t = t0 + r;
    if constexpr (CHUNKS)
        for (int e = tid; e < N; e += 64 * TOK)
            s_mask[e] = 0u;

    if (t < T) {
        int me, rank;
        float gate;
        select_token<NPL>(scores + (int64_t)t * N, N, K, lane, s_key + r * K, s_exp + r * K, me, rank, gate);
        if (lane < K) {
            idx_out[(int64_t)t * K + rank] = me;
            gate_out[(int64_t)t * K + rank] = gate;
            if constexpr (CHUNKS)
                s_idx[r * K + rank] = me;
        }
    }
    if constexpr (CHUNKS) {
        __syncthreads();
        for (int q = tid; q < TOK * K; q += 64 * TOK) {
            const int rq = q / K;
            if (t0 + rq < T)
                atomicOr(&s_mask[s_idx[q]], 1u << rq);
        }
        __syncthreads();
        for (int q = tid; q < TOK * K; q += 64 * TOK) {
            const int rq = q / K;
            if (t0 + rq < T)
                rank_out[(int64_t)t0 * K + q] = __popc(s_mask[s_idx[q]] & ((1u << rq) - 1u));
        }
        for (int e = tid; e < N; e += 64 * TOK)
            chunk_counts[(int64_t)e * ld_chunks + blockIdx.x] = __popc(s_mask[e]);
    }
}

inline size_t router_select_smem_bytes(int N, int K, int tok, bool chunks)
{
    return sizeof(int) * (2 * (size_t)tok * K + (chunks ? (size_t)tok * K + N : 0));
}

}  // namespace lmoe
