// Router: scores, top-K' selection, renormalised gates, and the first step
// of the dispatch histogram, fused in one kernel.
//
// Page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through
// Equations, Architecture, Code and ...": Figure 3 (router row per expert,
// softmax, keep the K largest), Figure 8 (the router reads x at the full
// width d, before the down-projection), and the MoE code block (the K kept
// weights are renormalised to sum to one).
//
// One workgroup owns RT = 32 tokens and ALL N' experts:
//   1. s[32, N'] = x W_r (+ b) on MFMA, fp32 accumulation; operands come
//      straight from global memory (W_r is a few MB and stays in L2).
//   2. s goes to LDS; each wave selects the top K' of a row with K' rounds of
//      a wave-wide maximum over 64-bit keys (order-preserving bits of the
//      score, then the complemented expert index, so equal scores go to the
//      lower index).  -0.0 is folded into +0.0 first, so signed zeros tie.
//   3. gate_k = exp(s_k - s_max) / sum_j exp(s_j - s_max) over the selected
//      set, the renormalised softmax (the softmax denominator cancels).
//   4. The 32 tokens form one dispatch chunk: a 32-bit mask per expert marks
//      which of them chose it; popcounts give each (token, slot) its rank
//      inside the chunk and the chunk's count per expert.  Integer-exact and
//      independent of atomic ordering (OR is order-free).
#pragma once

#include "common.hpp"

namespace lmoe {

constexpr int kRouterTokens = 32;

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

// NSW: n-subtiles (16 experts each) per wave; waves (w & 1) own token rows
// 16*(w&1) .. +15 and subtiles (w >> 1) + 2 q, q < NSW.
// NPL: score slots per lane in the selection (ceil(N'/64)).
template <typename E, int NSW, int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const E *__restrict__ x, const E *__restrict__ wrT, const float *__restrict__ bias,
    int T, int d, int N, int K, float *__restrict__ logits_out, int *__restrict__ idx_out,
    float *__restrict__ gate_out, int *__restrict__ rank_out, int *__restrict__ chunk_counts)
{
    constexpr int VEC = 16 / (int)sizeof(E);
    constexpr int KSTEP = 4 * VEC;  // elements of K per MFMA step
    extern __shared__ float rsmem[];
    const int ldl = N + 1;                       // padded LDS row of scores
    float *s_log = rsmem;                        // [32][N + 1]
    int *s_idx = reinterpret_cast<int *>(rsmem + kRouterTokens * ldl);  // [32][K]
    unsigned *s_mask = reinterpret_cast<unsigned *>(s_idx + kRouterTokens * K);  // [N]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kRouterTokens;
    const int mi = wave & 1;
    const int nsub = N / 16;

    // ---- 1. scores on MFMA -------------------------------------------------
    const int arow = t0 + mi * 16 + (lane & 15);
    const bool a_ok = arow < T;
    const E *a_ptr = x + (int64_t)(a_ok ? arow : 0) * d + (lane >> 4) * VEC;
    const E *b_ptr[NSW];
    bool b_ok[NSW];
#pragma unroll
    for (int q = 0; q < NSW; ++q) {
        const int nj = (wave >> 1) + 2 * q;
        b_ok[q] = nj < nsub;
        b_ptr[q] = wrT + (int64_t)(b_ok[q] ? nj * 16 + (lane & 15) : 0) * d + (lane >> 4) * VEC;
    }
    f32x4 acc[NSW];
#pragma unroll
    for (int q = 0; q < NSW; ++q)
        acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint4 zero = make_uint4(0, 0, 0, 0);
    uint4 a_cur = a_ok ? *reinterpret_cast<const uint4 *>(a_ptr) : zero;
    uint4 b_cur[NSW];
#pragma unroll
    for (int q = 0; q < NSW; ++q)
        b_cur[q] = b_ok[q] ? *reinterpret_cast<const uint4 *>(b_ptr[q]) : zero;
    for (int k0 = 0; k0 < d; k0 += KSTEP) {
        const bool more = k0 + KSTEP < d;
        uint4 a_nxt = zero, b_nxt[NSW];
        if (more && a_ok)
            a_nxt = *reinterpret_cast<const uint4 *>(a_ptr + k0 + KSTEP);
#pragma unroll
        for (int q = 0; q < NSW; ++q)
            b_nxt[q] = (more && b_ok[q]) ? *reinterpret_cast<const uint4 *>(b_ptr[q] + k0 + KSTEP) : zero;
#pragma unroll
        for (int q = 0; q < NSW; ++q)
            acc[q] = Mfma<E>::run(a_cur, b_cur[q], acc[q]);  // rows = tokens, cols = experts
        a_cur = a_nxt;
#pragma unroll
        for (int q = 0; q < NSW; ++q)
            b_cur[q] = b_nxt[q];
    }
    // lane l holds s[16 mi + 4 (l/16) + r][16 nj + l % 16]
#pragma unroll
    for (int q = 0; q < NSW; ++q) {
        const int nj = (wave >> 1) + 2 * q;
        if (nj < nsub) {
            const int col = nj * 16 + (lane & 15);
            const float bb = bias ? bias[col] : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s_log[(mi * 16 + 4 * (lane >> 4) + r) * ldl + col] = acc[q][r] + bb;
        }
    }
    for (int e = tid; e < N; e += 256)
        s_mask[e] = 0u;
    __syncthreads();

    if (logits_out) {
        for (int q = tid; q < kRouterTokens * N; q += 256) {
            const int r = q / N, e = q - r * N;
            if (t0 + r < T)
                logits_out[(int64_t)(t0 + r) * N + e] = s_log[r * ldl + e];
        }
    }

    // ---- 2 + 3. top-K' and gates, one row per wave at a time ---------------
    for (int r = wave; r < kRouterTokens; r += 4) {
        const int t = t0 + r;
        if (t >= T)
            break;
        unsigned long long key[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int e = lane + 64 * j;
            key[j] = (e < N) ? score_key(s_log[r * ldl + e], e) : 0ull;
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
        const float s_mine = (lane < K) ? s_log[r * ldl + e_mine] : 0.f;
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

    // ---- 4. chunk masks, ranks and counts ----------------------------------
    for (int q = tid; q < kRouterTokens * K; q += 256) {
        const int r = q / K;
        if (t0 + r < T)
            atomicOr(&s_mask[s_idx[q]], 1u << r);
    }
    __syncthreads();
    for (int q = tid; q < kRouterTokens * K; q += 256) {
        const int r = q / K;
        if (t0 + r < T)
            rank_out[(int64_t)t0 * K + q] = __popc(s_mask[s_idx[q]] & ((1u << r) - 1u));
    }
    for (int e = tid; e < N; e += 256)
        chunk_counts[(int64_t)blockIdx.x * N + e] = __popc(s_mask[e]);
}

inline size_t router_smem_bytes(int N, int K)
{
    return sizeof(float) * (size_t)kRouterTokens * (N + 1) + sizeof(int) * (size_t)kRouterTokens * K +
           sizeof(unsigned) * (size_t)N;
}

}  // namespace lmoe
