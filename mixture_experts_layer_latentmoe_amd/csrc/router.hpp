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
// concatenated matrix), stored in fp32.  This kernel owns 32 tokens (one
// dispatch chunk) with 8 waves:
//   1. each wave selects the top K' of a row with K' rounds of a wave-wide
//      maximum over 64-bit keys (order-preserving bits of the score, then the
//      complemented expert index, so equal scores go to the lower index);
//      -0.0 is folded into +0.0 first, so signed zeros tie;
//   2. gate_k = exp(s_k - s_max) / sum_j exp(s_j - s_max) over the selected
//      set, which is the renormalised softmax (its denominator cancels);
//   3. a 32-bit mask per expert marks which tokens of the chunk chose it;
//      popcounts give each (token, slot) its rank inside the chunk and the
//      chunk's count per expert -- integer-exact, independent of the order of
//      the atomic ORs.
#pragma once

#include "common.hpp"

namespace lmoe {

constexpr int kRouterTokens = 32;
constexpr int kSelectWaves = 8;

__device__ __forceinline__ unsigned long long score_key(float v, int e)
{
    v = (v == 0.f) ? 0.f : v;  // -0.0 and +0.0 tie
    unsigned u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (unsigned)(~(unsigned)e);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long q = __shfl_xor(k, o, 64);
        k = q > k ? q : k;
    }
    return k;
}

__device__ __forceinline__ float wave_sum_f32(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// NPL = ceil(N' / 64) scores held per lane.
template <int NPL>
__global__ __launch_bounds__(64 * kSelectWaves) void router_select_kernel(
    const float *__restrict__ scores, int T, int N, int K, int *__restrict__ idx_out, float *__restrict__ gate_out,
    int *__restrict__ rank_out, int *__restrict__ chunk_counts)
{
    extern __shared__ int rsmem[];
    int *s_idx = rsmem;                                            // [32][K]
    unsigned *s_mask = reinterpret_cast<unsigned *>(rsmem + kRouterTokens * K);  // [N]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kRouterTokens;
    for (int e = tid; e < N; e += 64 * kSelectWaves)
        s_mask[e] = 0u;

    for (int r = wave; r < kRouterTokens; r += kSelectWaves) {
        const int t = t0 + r;
        if (t >= T)
            break;
        const float *row = scores + (int64_t)t * N;
        unsigned long long key[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int e = lane + 64 * j;
            key[j] = (e < N) ? score_key(row[e], e) : 0ull;
        }
        unsigned long long mine = 0ull;
        for (int k = 0; k < K; ++k) {
            unsigned long long best = key[0];
#pragma unroll
            for (int j = 1; j < NPL; ++j)
                best = key[j] > best ? key[j] : best;
            best = wave_max_u64(best);
            if (lane == k)
                mine = best;
            const int e = (int)(~(unsigned)(best & 0xffffffffull));
            if ((e & 63) == lane) {
#pragma unroll
                for (int j = 0; j < NPL; ++j)
                    if (j == (e >> 6))
                        key[j] = 0ull;
            }
        }
        const int e_mine = (int)(~(unsigned)(mine & 0xffffffffull));
        const float s_mine = (lane < K) ? row[e_mine] : 0.f;
        const float s_top = __shfl(s_mine, 0, 64);
        const float g = (lane < K) ? expf(s_mine - s_top) : 0.f;
        const float gsum = wave_sum_f32(g);
        if (lane < K) {
            idx_out[(int64_t)t * K + lane] = e_mine;
            gate_out[(int64_t)t * K + lane] = g / gsum;
            s_idx[r * K + lane] = e_mine;
        }
    }
    __syncthreads();

    for (int q = tid; q < kRouterTokens * K; q += 64 * kSelectWaves) {
        const int r = q / K;
        if (t0 + r < T)
            atomicOr(&s_mask[s_idx[q]], 1u << r);
    }
    __syncthreads();
    for (int q = tid; q < kRouterTokens * K; q += 64 * kSelectWaves) {
        const int r = q / K;
        if (t0 + r < T)
            rank_out[(int64_t)t0 * K + q] = __popc(s_mask[s_idx[q]] & ((1u << r) - 1u));
    }
    for (int e = tid; e < N; e += 64 * kSelectWaves)
        chunk_counts[(int64_t)blockIdx.x * N + e] = __popc(s_mask[e]);
}

inline size_t router_select_smem_bytes(int N, int K)
{
    return sizeof(int) * (size_t)kRouterTokens * K + sizeof(unsigned) * (size_t)N;
}

}  // namespace lmoe
