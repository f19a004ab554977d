// Dense and grouped GEMMs on MFMA with LDS-staged, double-buffered tiles.
//
//   C[rows, N] = epilogue( A[rows, K] * B[K, N] ),  fp32 accumulation
//
// B is held transposed (B^T[N, K], K contiguous), the layout the weights are
// repacked into once at create time, so A and B tiles are loaded the same way:
// 16-byte chunks of K-contiguous rows.  A k-tile is 128 bytes of K (64 bf16 or
// 32 fp32 elements); in LDS a tile row is 8 chunks of 16 bytes, chunk c stored
// at position c ^ (row & 7) so that both the 16-byte writes of a row and the
// 16-row fragment reads of one chunk column hit distinct banks.
//
// Dense mode: rows = M; tiles walk grouped-by-M order inside each XCD.
// Grouped mode (routed experts): the dispatch rows of expert e are the
// contiguous range [offsets[e], offsets[e+1]); a device-built tile table
// lists (expert, first row) for every BM-row tile, so no host round trip is
// needed.  A rows may be gathered through `gather` (dispatch row -> token).
//
// Epilogue: columns >= relu2_from get relu(v)^2 (squared-ReLU expert
// activation), then the result is rounded to E and stored.
#pragma once

#include "common.hpp"

namespace lmoe {

struct GemmParams {
    const void *A;
    int64_t lda;        // elements
    const void *B;      // B^T rows: [N][ldb]
    int64_t ldb;        // elements
    int64_t strideB;    // elements between experts (grouped)
    void *C;
    int64_t ldc;        // elements
    int M, N, K;        // M: dense rows (unused in grouped mode)
    int relu2_from;     // first column that gets relu^2 (>= N: none)
    int group_m;        // dense: tiles of this many M-tiles are walked together
    // grouped mode
    const int *gather;       // dispatch row -> A row, or nullptr (A rows = dispatch rows)
    const int *tile_expert;  // [tiles]
    const int *tile_row0;    // [tiles] first row of the tile inside its expert
    const int *n_mtiles;     // device scalar: number of valid M tiles
    const int *offsets;      // [N'+1] first dispatch row of each expert
};

template <typename E, int BM, int BN, int WM, int WN, bool GROUPED>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p)
{
    static_assert(WM * WN == 4, "four waves per workgroup");
    constexpr int VEC = 16 / (int)sizeof(E);    // elements per 16-byte chunk
    constexpr int BK = 8 * VEC;                 // elements per k-tile
    constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile
    constexpr int TM = WTM / 16, TN = WTN / 16; // 16x16 MFMA tiles per wave
    constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;
    static_assert(TM >= 1 && TN >= 1 && ACH >= 1 && BCH >= 1, "tile shape");

    extern __shared__ uint4 smem[];
    uint4 *sA = smem;                 // [2][BM * 8]
    uint4 *sB = smem + 2 * BM * 8;    // [2][BN * 8]

    const int ntn = (p.N + BN - 1) / BN;
    int tm, tn, rows_valid, expert = 0;
    int64_t row_base; // first output row (dense: M row; grouped: dispatch row)
    if constexpr (GROUPED) {
        const int total = *p.n_mtiles * ntn;
        const int t = xcd_logical_tile(blockIdx.x, total);
        if (t < 0)
            return;
        tm = t / ntn;
        tn = t - tm * ntn;
        expert = p.tile_expert[tm];
        const int r0 = p.tile_row0[tm];
        const int start = p.offsets[expert];
        const int cnt = p.offsets[expert + 1] - start;
        rows_valid = min(BM, cnt - r0);
        row_base = (int64_t)start + r0;
    } else {
        const int ntm = (p.M + BM - 1) / BM;
        const int t = xcd_logical_tile(blockIdx.x, ntm * ntn);
        if (t < 0)
            return;
        const int gm = p.group_m;
        const int in_group = gm * ntn;
        const int g = t / in_group;
        const int first = g * gm;
        const int gsize = min(ntm - first, gm);
        const int r = t - g * in_group;
        tm = first + r % gsize;
        tn = r / gsize;
        rows_valid = min(BM, p.M - tm * BM);
        row_base = (int64_t)tm * BM;
    }
    const int n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave - (wave / WN) * WN;

    // Source addresses of this thread's chunks (fixed for the whole K loop).
    const char *a_src[ACH];
    const char *b_src[BCH];
    const char *Abase = static_cast<const char *>(p.A);
    const char *Bbase = static_cast<const char *>(p.B) + (int64_t)expert * p.strideB * (int64_t)sizeof(E);
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int q = tid + i * 256, r = q >> 3, c = q & 7;
        a_src[i] = nullptr;
        if (r < rows_valid) {
            int64_t arow = row_base + r;
            if (GROUPED && p.gather)
                arow = p.gather[arow];
            a_src[i] = Abase + (arow * p.lda) * (int64_t)sizeof(E) + c * 16;
        }
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        const int q = tid + i * 256, r = q >> 3, c = q & 7;
        b_src[i] = nullptr;
        if (n0 + r < p.N)
            b_src[i] = Bbase + ((int64_t)(n0 + r) * p.ldb) * (int64_t)sizeof(E) + c * 16;
    }

    uint4 ra[ACH], rb[BCH];
    const uint4 zero = make_uint4(0, 0, 0, 0);
    auto gload = [&](int kt) {
        const int64_t off = (int64_t)kt * 128;
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            ra[i] = a_src[i] ? *reinterpret_cast<const uint4 *>(a_src[i] + off) : zero;
#pragma unroll
        for (int i = 0; i < BCH; ++i)
            rb[i] = b_src[i] ? *reinterpret_cast<const uint4 *>(b_src[i] + off) : zero;
    };
    auto sstore = [&](int st) {
        uint4 *a = sA + st * BM * 8;
        uint4 *b = sB + st * BN * 8;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int q = tid + i * 256, r = q >> 3, c = q & 7;
            a[r * 8 + (c ^ (r & 7))] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int q = tid + i * 256, r = q >> 3, c = q & 7;
            b[r * 8 + (c ^ (r & 7))] = rb[i];
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = p.K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
        const uint4 *a = sA + st * BM * 8;
        const uint4 *b = sB + st * BN * 8;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = s * 4 + (lane >> 4);
            uint4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 16 + (lane & 15);
                af[i] = a[r * 8 + (c ^ (r & 7))];
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 16 + (lane & 15);
                bfr[j] = b[r * 8 + (c ^ (r & 7))];
            }
            // B fragment first: lane l then owns 4 consecutive output columns
            // (4*(l/16) + 0..3) of output row (l % 16).
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = Mfma<E>::run(bfr[j], af[i], acc[i][j]);
        }
        if (kt + 1 < nk)
            sstore(st ^ 1);
        __syncthreads();
    }

    E *C = static_cast<E *>(p.C);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int rl = wm * WTM + i * 16 + (lane & 15);
        if (rl >= rows_valid)
            continue;
        E *crow = C + (row_base + rl) * p.ldc;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + 4 * (lane >> 4);
            if (col >= p.N)
                continue;
            float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (col + r >= p.relu2_from) {
                    const float t = fmaxf(v[r], 0.f);
                    v[r] = t * t;
                }
            store4(crow + col, v[0], v[1], v[2], v[3]);
        }
    }
}

template <typename E, int BM, int BN>
constexpr size_t gemm_smem_bytes()
{
    return (size_t)2 * (BM + BN) * 8 * 16;
}

}  // namespace lmoe
