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
// The selection kernel already left, per chunk c of 16 tokens, the count of every
// expert (chunk_counts[e][c], expert-major) and each pair's rank inside its
// chunk.  Here:
//   chunk_scan_kernel  one wave per expert: chunk_base[e][c] = sum_{c' < c}
//                      chunk_counts[e][c'] (wave prefix sums), counts[e]
//   finalize_kernel    every workgroup scans counts into offsets in LDS, then
//                      pos = offsets[e] + chunk_base[e][c] + rank and
//                      perm_token[pos] = t; workgroup 0 also publishes offsets
//                      and the tile table of the grouped GEMMs
//   dispatch_small_kernel  both in one workgroup when a batch has at most 64
//                      chunks
//   (batches of at most 64 tokens: route_tiny.hpp, straight from idx)
// All integer, no ordering atomics: the same idx always gives the same bits.
#pragma once

#include "common.hpp"

namespace lmoe {

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o)
            v += u;
    }
    return v;
}

// 4 waves per workgroup, one expert per wave; a wave walks the expert's row
// of chunk counts 256 at a time (4 per lane, 16-byte loads).
__global__ __launch_bounds__(256) void chunk_scan_kernel(const int *__restrict__ chunk_counts, int nchunks,
                                                         int ld_chunks, int N, int *__restrict__ chunk_base,
                                                         int *__restrict__ counts)
{
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= N)
        return;
    const int *src = chunk_counts + (int64_t)e * ld_chunks;
    int *dst = chunk_base + (int64_t)e * ld_chunks;
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 256) {
        const int c = c0 + lane * 4;
        int4 v = make_int4(0, 0, 0, 0);
        if (c < nchunks)  // ld_chunks is a multiple of 4; entries past nchunks are ignored
            v = *reinterpret_cast<const int4 *>(src + c);
        if (c + 1 >= nchunks) v.y = 0;
        if (c + 2 >= nchunks) v.z = 0;
        if (c + 3 >= nchunks) v.w = 0;
        const int tot = v.x + v.y + v.z + v.w;
        const int incl = wave_incl_scan(tot, lane);
        const int ex = carry + incl - tot;
        if (c < nchunks)
            *reinterpret_cast<int4 *>(dst + c) = make_int4(ex, ex + v.x, ex + v.x + v.y, ex + v.x + v.y + v.z);
        carry += __shfl(incl, 63, 64);
    }
    if (lane == 0)
        counts[e] = carry;
}

// Exclusive scan of the counts (c = counts[threadIdx.x], 0 past N') into
// s_off; `lead` also publishes offsets and the tile table of the grouped
// GEMMs: per tile (expert, first dispatch row, rows of the expert from that
// row on, 0), so that a kernel finds its tile with one load.  Tiles are BM rows from each expert's first row,
// except that the last one may hold up to BM + slack rows: max(1, ceil((c -
// slack) / BM)) tiles for an expert with c > 0 rows (slack 0: ceil(c / BM)).
// 1024 threads, N' <= 1024; every thread calls it.  s_off is complete on return.
__device__ __forceinline__ void block_offsets(int c, bool lead, int N, int BM, int slack, int *__restrict__ offsets,
                                              int4 *__restrict__ tile_info,
                                              int *__restrict__ n_mtiles, int *s_off, int *s_wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int incl = wave_incl_scan(c, lane);
    if (lane == 63)
        s_wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w)
        before += s_wsum[w];
    const int excl = before + incl - c;
    s_off[tid] = excl;
    __syncthreads();

    if (lead) {
        if (tid < N)
            offsets[tid] = excl;
        if (tid == N - 1)
            offsets[N] = excl + c;
        // tile table: same scan over the tile counts
        const int nt = c > 0 ? max(1, (c - slack + BM - 1) / BM) : 0;
        const int tincl = wave_incl_scan(nt, lane);
        if (lane == 63)
            s_wsum[wave] = tincl;
        __syncthreads();
        int tbefore = 0;
        for (int w = 0; w < wave; ++w)
            tbefore += s_wsum[w];
        const int texcl = tbefore + tincl - nt;
        for (int j = 0; j < nt; ++j)
            tile_info[texcl + j] = make_int4(tid, excl + j * BM, c - j * BM, 0);
        if (tid == 1023)
            *n_mtiles = texcl + nt;
    }
}

// The part of the chunked order every workgroup computes: the offsets (and,
// if lead, the tile table), then pos/perm for the pairs q = q0, q0 + qs, ...
__device__ __forceinline__ void finalize_block(int c, bool lead, int64_t q0, int64_t qs, const int *__restrict__ idx,
                                               const int *__restrict__ rank, const int *__restrict__ chunk_base, int T,
                                               int K, int N, int chunk_tokens, int ld_chunks, int BM, int slack,
                                               int *__restrict__ offsets, int4 *__restrict__ tile_info,
                                               int *__restrict__ n_mtiles,
                                               int *__restrict__ pos, int *__restrict__ perm, int *s_off, int *s_wsum)
{
    block_offsets(c, lead, N, BM, slack, offsets, tile_info, n_mtiles, s_off, s_wsum);
    const int64_t P = (int64_t)T * K;
    for (int64_t q = q0; q < P; q += qs) {
        const int t = (int)(q / K);
        const int e = idx[q];
        const int p = s_off[e] + chunk_base[(int64_t)e * ld_chunks + t / chunk_tokens] + rank[q];
        pos[q] = p;
        perm[p] = t;
    }
}

// 1024 threads; N' <= 1024.  Every workgroup scans the counts; workgroup 0
// publishes offsets and the tile table; all share the pairs.
__global__ __launch_bounds__(1024) void finalize_kernel(const int *__restrict__ idx, const int *__restrict__ rank,
                                                       const int *__restrict__ chunk_base,
                                                       const int *__restrict__ counts, int T, int K, int N,
                                                       int chunk_tokens, int ld_chunks, int BM, int slack,
                                                       int *__restrict__ offsets, int4 *__restrict__ tile_info,
                                                       int *__restrict__ n_mtiles,
                                                       int *__restrict__ pos, int *__restrict__ perm)
{
    __shared__ int s_off[1024];
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x;
    const int c = (tid < N) ? counts[tid] : 0;
    finalize_block(c, blockIdx.x == 0, (int64_t)blockIdx.x * 1024 + tid, (int64_t)gridDim.x * 1024, idx, rank,
                   chunk_base, T, K, N, chunk_tokens, ld_chunks, BM, slack, offsets, tile_info, n_mtiles,
                   pos, perm, s_off, s_wsum);
}

// Small batches (at most 64 chunks): the chunk scan and finalize in one
// workgroup of 1024 threads -- one launch instead of two.  Thread e scans
// expert e's row of chunk counts in registers (every load of the row issued
// first); the chunk bases it writes are read back by other threads of this
// workgroup after the barriers of the offsets scan.
__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int *__restrict__ chunk_counts, int nchunks,
                                                             const int *__restrict__ idx, const int *__restrict__ rank,
                                                             int T, int K, int N, int chunk_tokens, int ld_chunks,
                                                             int BM, int slack, int *__restrict__ chunk_base,
                                                             int *__restrict__ counts, int *__restrict__ offsets,
                                                             int4 *__restrict__ tile_info,
                                                             int *__restrict__ n_mtiles, int *__restrict__ pos,
                                                             int *__restrict__ perm)
{
    __shared__ int s_off[1024];
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x;
    int c = 0;
    if (tid < N) {
        // ld_chunks is a multiple of 4; entries past nchunks are not counts
        const int4 *row = reinterpret_cast<const int4 *>(chunk_counts + (int64_t)tid * ld_chunks);
        int4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            v[u] = 4 * u < nchunks ? row[u] : make_int4(0, 0, 0, 0);
        int4 *out = reinterpret_cast<int4 *>(chunk_base + (int64_t)tid * ld_chunks);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (4 * u >= nchunks)
                break;
            const int n = nchunks - 4 * u;
            int4 b;
            b.x = c;
            c += v[u].x;
            b.y = c;
            c += n > 1 ? v[u].y : 0;
            b.z = c;
            c += n > 2 ? v[u].z : 0;
            b.w = c;
            c += n > 3 ? v[u].w : 0;
            out[u] = b;
        }
        counts[tid] = c;
    }
    finalize_block(c, true, tid, 1024, idx, rank, chunk_base, T, K, N, chunk_tokens, ld_chunks, BM, slack, offsets,
                   tile_info, n_mtiles, pos, perm, s_off, s_wsum);
}

}  // namespace lmoe
