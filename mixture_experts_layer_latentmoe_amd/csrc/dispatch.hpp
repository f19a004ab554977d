// Dispatch order on one GPU: histogram, exclusive scans and the permutation.
//
// On several GPUs the explainer page ("LatentMoE: NVIDIA's Latent Mixture of
// Experts Explained Through Equations, Architecture, Code and ...", Figure
// 12 and the expert-parallel paragraphs) ships every token to its experts
// with an all-to-all; on one GPU that exchange becomes this on-chip
// permutation.  The order is a stable counting sort of the (token, slot)
// pairs by expert, then token:
//
//   counts[e]     = #{(t, k) : idx[t, k] = e}
//   offsets[e]    = sum_{e' < e} counts[e'],   offsets[N'] = T K'
//   pos[t, k]     = offsets[e] + #{t' < t : e in idx[t']}
//   perm_token[pos[t, k]] = t
//
// The router kernel already left, per 32-token chunk c, the count of every
// expert (chunk_counts[c][e]) and each pair's rank inside its chunk.  Here:
//   chunk_scan_kernel      chunk_base[c][e] = sum_{c' < c} chunk_counts[c'][e], counts[e]
//   expert_offsets_kernel  offsets, and the tile table of the grouped GEMMs
//   finalize_kernel        pos = offsets[e] + chunk_base[c][e] + rank; perm_token
// All integer, no atomics: the same idx always gives the same bits.
#pragma once

#include "common.hpp"

namespace lmoe {

// Workgroup of 256 threads per 64 experts; wave w scans a quarter of the chunks.
__global__ __launch_bounds__(256) void chunk_scan_kernel(const int *__restrict__ chunk_counts, int nchunks,
                                                         int N, int *__restrict__ chunk_base,
                                                         int *__restrict__ counts)
{
    __shared__ int part[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int per = (nchunks + 3) / 4;
    const int c_begin = min(nchunks, wave * per), c_end = min(nchunks, c_begin + per);
    int sum = 0;
    if (e < N)
        for (int c = c_begin; c < c_end; ++c)
            sum += chunk_counts[(int64_t)c * N + e];
    part[wave][lane] = sum;
    __syncthreads();
    int run = 0;
    for (int w = 0; w < wave; ++w)
        run += part[w][lane];
    if (e < N) {
        for (int c = c_begin; c < c_end; ++c) {
            const int64_t o = (int64_t)c * N + e;
            const int v = chunk_counts[o];
            chunk_base[o] = run;
            run += v;
        }
        if (wave == 3)
            counts[e] = run;
    }
}

// One workgroup of 1024 threads (N' <= 1024): exclusive scans of the counts
// and of the BM-row tile counts, then the (expert, first row) tile table.
__global__ __launch_bounds__(1024) void expert_offsets_kernel(const int *__restrict__ counts, int N, int BM,
                                                              int *__restrict__ offsets,
                                                              int *__restrict__ tile_expert,
                                                              int *__restrict__ tile_row0,
                                                              int *__restrict__ n_mtiles)
{
    __shared__ int sc[1024];
    __shared__ int st[1024];
    const int e = threadIdx.x;
    const int c = (e < N) ? counts[e] : 0;
    const int nt = (c + BM - 1) / BM;
    sc[e] = c;
    st[e] = nt;
    __syncthreads();
    // Hillis-Steele inclusive scans
    for (int o = 1; o < 1024; o <<= 1) {
        const int a = (e >= o) ? sc[e - o] : 0;
        const int b = (e >= o) ? st[e - o] : 0;
        __syncthreads();
        sc[e] += a;
        st[e] += b;
        __syncthreads();
    }
    const int excl_c = sc[e] - c, excl_t = st[e] - nt;
    if (e < N) {
        offsets[e] = excl_c;
        for (int j = 0; j < nt; ++j) {
            tile_expert[excl_t + j] = e;
            tile_row0[excl_t + j] = j * BM;
        }
    }
    if (e == 0) {
        offsets[N] = sc[1023];
        *n_mtiles = st[1023];
    }
}

__global__ __launch_bounds__(256) void finalize_kernel(const int *__restrict__ idx, const int *__restrict__ rank,
                                                       const int *__restrict__ chunk_base,
                                                       const int *__restrict__ offsets, int T, int K, int N,
                                                       int chunk_tokens, int *__restrict__ pos,
                                                       int *__restrict__ perm)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)T * K)
        return;
    const int t = (int)(q / K);
    const int e = idx[q];
    const int p = offsets[e] + chunk_base[(int64_t)(t / chunk_tokens) * N + e] + rank[q];
    pos[q] = p;
    perm[p] = t;
}

}  // namespace lmoe
