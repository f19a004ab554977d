// Routing of decode batches (T <= kTinyTokens) in one launch: the selection
// of router.hpp -- four tokens per workgroup, one wave per token -- and, in
// the last workgroup to finish, the dispatch order.
//
// Page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through
// Equations, Architecture, Code and ...": Figure 3 and the MoE code block
// (top-K' of the scores, renormalised gates), and the grouping of the
// (token, slot) pairs by expert that the expert FFNs of Figure 9 consume.
//
// The workgroups' expert choices cross workgroups, and XCDs with their own
// L2, through device-coherent stores; each workgroup waits for its stores to
// complete, then counts itself in on a relaxed device-scope counter.  The
// workgroup that counts last resets the counter (so every launch starts from
// zero) and reads every choice back with device-coherent loads.  It then
// forms the order with its 256 threads: per expert a 64-bit mask of the
// tokens that chose it (LDS atomic ORs, whose order does not matter),
// counts[e] = popc(mask[e]), exclusive scans of the counts and of the tile
// counts (the tile table of the grouped GEMMs, as block_offsets forms it),
// and pos[t, k] = offsets[e] + popc(mask[e] & (2^t - 1)).  All integer: the
// same scores always give the same bits.  With 32-row tiles and a row table
// it also writes the token of each dispatch row at [tile][row in tile] (rows
// past an expert's last row stay unwritten), so that a grouped GEMM
// workgroup loads its A rows together with its tile record instead of
// through perm after it.
#pragma once

#include "dispatch.hpp"
#include "gemm.hpp"
#include "router.hpp"

namespace lmoe {

struct TinyRouteParams {
    const float *scores;  // [T][N'] fp32
    int T, N, K;
    int *idx;             // [T][K'] experts by rank
    float *gate;          // [T][K'] renormalised gates by rank
    int *counter;         // arrival counter, zero between launches
    int BM, slack;        // tile table: rows per tile, extra rows of an expert's last tile
    int *counts, *offsets;
    int4 *tile_info;
    int *n_mtiles, *pos, *perm;
    int *tile_rows;       // nullable: [tiles][32] token of each row of the 32-row tiles
};

constexpr int kRouteTinyThreads = 64 * kTinySelectWaves;

template <int NPL>
__global__ __launch_bounds__(kRouteTinyThreads) void route_tiny_kernel(const TinyRouteParams p)
{
    constexpr int NT = kRouteTinyThreads;
    constexpr int EPT = 1024 / NT;  // experts per thread (N' <= 1024)
    constexpr int PPT = 4096 / NT;  // pairs per thread (T K' <= 4096)
    extern __shared__ int rsmem[];
    unsigned *s_key = reinterpret_cast<unsigned *>(rsmem);  // [waves][K']
    int *s_exp = rsmem + kTinySelectWaves * p.K;           // [waves][K']
    __shared__ unsigned long long s_mask[1024];
    __shared__ int s_off[1024], s_toff[1024];
    __shared__ int s_wsum[2][NT / 64];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.x * kTinySelectWaves + wave;
    const int K = p.K, N = p.N;
    if (t < p.T) {
        int me, rank;
        float g;
        select_token<NPL>(p.scores + (int64_t)t * N, N, K, lane, s_key + wave * K, s_exp + wave * K, me, rank, g);
        if (lane < K) {
            __hip_atomic_store(p.idx + (int64_t)t * K + rank, me, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            p.gate[(int64_t)t * K + rank] = g;
        }
    }
    wait_vm_lgkm0<0>();  // this thread's choices are stored
    __syncthreads();     // ... and every thread's
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(p.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (int)gridDim.x - 1;
        if (old == (int)gridDim.x - 1)
            __hip_atomic_store(p.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last)
        return;

    // the last workgroup: every pair's expert, up front
    const int P = p.T * K;
    int e_q[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int q = tid + NT * j;
        e_q[j] = q < P ? __hip_atomic_load(p.idx + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -1;
    }
    for (int e = tid; e < 1024; e += NT)
        s_mask[e] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PPT; ++j)
        if (e_q[j] >= 0)
            atomicOr(&s_mask[e_q[j]], 1ull << ((tid + NT * j) / K));
    __syncthreads();

    // experts tid * EPT .. + EPT - 1: counts, tile counts, exclusive scans
    int c[EPT], nt[EPT], csum = 0, tsum = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        c[i] = e < N ? __popcll(s_mask[e]) : 0;
        nt[i] = c[i] > 0 ? max(1, (c[i] - p.slack + p.BM - 1) / p.BM) : 0;
        csum += c[i];
        tsum += nt[i];
    }
    const int ic = wave_incl_scan(csum, lane), it = wave_incl_scan(tsum, lane);
    if (lane == 63) {
        s_wsum[0][wave] = ic;
        s_wsum[1][wave] = it;
    }
    __syncthreads();
    int xc = ic - csum, xt = it - tsum;
    for (int w = 0; w < wave; ++w) {
        xc += s_wsum[0][w];
        xt += s_wsum[1][w];
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < N) {
            p.counts[e] = c[i];
            p.offsets[e] = xc;
            s_off[e] = xc;
            s_toff[e] = xt;
            for (int j = 0; j < nt[i]; ++j)
                p.tile_info[xt + j] = make_int4(e, xc + j * p.BM, c[i] - j * p.BM, 0);
        }
        xc += c[i];
        xt += nt[i];
    }
    if (tid == NT - 1) {
        p.offsets[N] = xc;
        *p.n_mtiles = xt;
    }
    __syncthreads();

    // each pair's dispatch row; with 32-row tiles (no extra rows) its token in
    // the row table as well
    const bool rows = p.BM == 32 && p.slack == 0 && p.tile_rows;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int e = e_q[j];
        if (e < 0)
            continue;
        const int q = tid + NT * j, tk = q / K;
        const int r = __popcll(s_mask[e] & ((1ull << tk) - 1ull));  // row within the expert
        const int row = s_off[e] + r;
        p.pos[q] = row;
        p.perm[row] = tk;
        if (rows)
            p.tile_rows[(s_toff[e] + (r >> 5)) * 32 + (r & 31)] = tk;
    }
}

inline size_t route_tiny_smem_bytes(int K) { return sizeof(int) * 2 * (size_t)kTinySelectWaves * K; }

}  // namespace lmoe
