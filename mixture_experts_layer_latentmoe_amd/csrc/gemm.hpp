// Dense and grouped GEMMs on MFMA with LDS-staged, double-buffered tiles.
//
//   C[rows, N] = epilogue( A[rows, K] * B[K, N] ),  fp32 accumulation
//
// B is held transposed (B^T[N, K], K contiguous), the layout the weights are
// repacked into once at create time, so A and B tiles are loaded the same way:
// 16-byte chunks of K-contiguous rows.  A k-tile is 128 bytes of K (64 bf16 or
// 32 fp32 elements); in LDS a tile row is 8 chunks of 16 bytes, chunk c of row
// r stored at position c ^ ((r >> 1) & 7).  A 16-lane group of a fragment read
// touches 16 consecutive rows at one chunk column; with 64 banks of 4 bytes,
// row parity and the swizzled position then give 16 distinct 16-byte bank
// groups (the plain c ^ (r & 7) maps rows r and r + 8 to the same banks).
//
// Global loads are buffer loads with the LDS bit (HBM/L2 straight into the
// LDS stage, no staging registers): a row outside the valid range gets an
// offset beyond the buffer's size, and the hardware returns zeros for it, so
// the main loop has no branches.  With NS stages, k-tiles j + 1 .. j + NS - 1
// are in flight while k-tile j is multiplied; one barrier per k-tile.  Inside
// a k-tile, where registers allow, the MFMA fragments of the next 16-wide
// k-step are read from LDS while the current one multiplies (tile_mma_pipe).
//
// Dense mode: rows = M; tiles walk grouped-by-M order inside each XCD.
// Grouped mode (routed experts): the dispatch rows of expert e are the
// contiguous range [offsets[e], offsets[e+1]); a device-built tile table
// lists (expert, first row) for every BM-row tile, so no host round trip is
// needed.  A rows may be gathered through `gather` (dispatch row -> token).
// Batched-K mode: products that differ only in their K range (k_offsets).
// Split-K (dense, few rows): fp32 partials and a fixed-order reduce kernel.
//
// Epilogue: the first c_split columns (router scores) are stored in fp32 with
// a per-column bias; the rest go to C, where columns >= relu2_from get
// relu(v)^2 (squared-ReLU expert activation) and, from glu_from on, gated
// pairs give silu(gate) * value, rounded to E.  Whole tiles of E outputs and
// all-fp32 outputs are staged through LDS and written as whole rows with
// non-temporal stores; the compile-time ACT variants add the expert
// activation beside fp32 sums, or replace dH by the activation gradient.
//
// E4M3 expert weights (grouped GEMMs of a bf16 layer): B tiles hold the bytes
// (64 per row and k-tile), fragments are widened to bf16 in registers (exact:
// every E4M3 value is a bf16 value) and the per-column fp32 scale multiplies
// the fp32 sums before the epilogue, which equals multiplying the weights.
#pragma once

#include "common.hpp"

namespace lmoe {

struct GemmParams {
    const void *A;
    int64_t lda;        // elements
    int64_t a_bytes;    // size of the A buffer in bytes (range of the loads)
    const void *B;      // B^T rows: [N][ldb]
    int64_t ldb;        // elements
    int64_t b_kstep;    // bytes from one k-tile of a B row to the next; 0: rows are
                        // K-contiguous (one k-tile = 128 bytes, 64 for E4M3).  The
                        // k-tiled layout [K / BK][N][BK] has ldb = BK and
                        // b_kstep = N * BK * bytes per element
    int64_t strideB;    // elements between experts (grouped)
    void *C;            // columns [c_split, N) go to C[row][col - c_split]
    int64_t ldc;        // elements
    float *C32;         // columns [0, c_split) go to C32[row][col] in fp32 (+ bias32)
    int64_t ldc32;
    const float *bias32;  // nullable
    int c_split;        // multiple of 4; 0: no fp32 part
    int M, N, K;        // M: dense rows (unused in grouped mode)
    int relu2_from = 1 << 30;  // first column of C (after the split) that gets relu^2
    int glu_from = 1 << 30;    // first B column of gated pairs: from it on, in blocks of 16 B columns,
                        // 8 gate columns then the 8 value columns of the same outputs; each
                        // block gives 8 C columns silu(gate) * value (>= N: none).  A multiple
                        // of 16, at or after c_split.
    int group_m;        // dense: tiles of this many M-tiles are walked together
    int splitk;         // dense: > 1 splits K into this many contiguous k-tile ranges;
                        // raw fp32 sums go to partial[split][M][N] and a reduce
                        // kernel applies the epilogue
    float *partial;
    int *counters;      // dense, few rows, splitk > 1: one arrival counter per column group,
                        // zero between launches (fewrow_split_kernel)
    // grouped mode
    const int *gather;       // dispatch row -> A row, or nullptr (A rows = dispatch rows)
    const int4 *tile_info;   // [tiles] expert, first dispatch row, rows of the expert from it on, 0
    const int *tile_rows;    // 32-row tiles, nullable: [tiles][32] A row (after the gather) of each tile
                             // row; undefined past the expert's rows
    const int *n_mtiles;     // device scalar: number of valid M tiles
    const int *offsets;      // [N'+1] first dispatch row of each expert
    const float *scaleB;     // grouped, E4M3 B: [N'][N] scale of each expert's output column
    // dense, few rows: B again in fragment-major 1 KiB blocks (fragmajor_kernel)
    const void *Bfrag;
    // dense, batched K (weight gradients of the experts): n_batches products
    // share A and B and differ in their K range: batch e sums over
    // [k_offsets[e], k_offsets[e + 1]) (elements, multiples of the k-tile;
    // an empty range gives zeros) and writes output rows e M .. e M + M - 1
    const int *k_offsets;
    int n_batches;
    // MN-major GEMM (gemm_tn.hpp): size of the B buffer in bytes
    int64_t b_bytes;
    // pre-activations (fp32, row stride ld_pre) read by the gradient
    // epilogues (gemm_kernel's ACT 3 and 4)
    const float *act_pre;
    int64_t ld_pre;
};

// Epilogues of the fp32 staged store (template parameter ACT of gemm_kernel):
//  ACT_NONE      the sums to C32;
//  ACT_RELU2     the sums to C32 and relu(sum)^2 to C (N columns);
//  ACT_GLU       the sums to C32 and, for the gated pairs (16-column blocks:
//                8 gates, then their 8 values), silu(gate) * value to C (N / 2
//                columns);
//  ACT_RELU2_GRAD instead of the sums dH, dA = dH * 2 relu(a) to C (N columns),
//                a from act_pre;
//  ACT_GLU_GRAD  for output column j, gate column g = 16 (j / 8) + j % 8 and
//                value column g + 8 of act_pre: dH * v * silu'(gate) to C
//                column g and dH * silu(gate) to C column g + 8 (2 N columns).
enum { ACT_NONE = 0, ACT_RELU2 = 1, ACT_GLU = 2, ACT_RELU2_GRAD = 3, ACT_GLU_GRAD = 4 };

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over `bytes` bytes at p (loads past the end read 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes)
{
    const int n = bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

constexpr unsigned kOOB = 0x80000000u;  // offset that is always out of range
constexpr int kLoadNonTemporal = 2;     // cache policy of a buffer load: nt (streamed)

// 16-byte store of a staged epilogue, marked non-temporal (streamed through
// L2 without displacing the operands other tiles still read).
__device__ __forceinline__ void store16_stream(void *base, int64_t byte_off, uint4 v)
{
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(v4u, v),
                                reinterpret_cast<v4u *>(static_cast<char *>(base) + byte_off));
}

#define LMOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// vmcnt <= N and lgkmcnt == 0 (gfx9 s_waitcnt: vmcnt[3:0] + vmcnt[15:14],
// expcnt[6:4] left at 7 = no wait, lgkmcnt[11:8])
template <int N> __device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Output tile of one workgroup.  Dense: rows [row_base, row_base +
// rows_valid) of M; grouped: dispatch rows of one expert.  split: the K range
// of a split-K workgroup.
struct TileInfo {
    int n0, rows_valid, expert, split;
    int64_t row_base;
    int64_t c_row0;  // added to the output rows (batched K: e M)
};

// Logical tile t (no split-K) -> output tile.  Grouped: t walks the device
// tile table, N-tiles fastest.  Dense: tiles are walked in groups of group_m
// M-tiles, so that tiles in flight together share A and B panels.
// XR: grouped tiles whose expert has at most BM + XR rows left take them all
// (the tile table gives an expert's last tile up to BM + XR rows).
template <int BM, int BN, bool GROUPED, int XR = 0>
__device__ __forceinline__ void tile_coords(const GemmParams &p, int t, int ntn, TileInfo &ti)
{
    int tm, tn;
    ti.expert = 0;
    ti.split = 0;
    ti.c_row0 = 0;
    if constexpr (GROUPED) {
        tm = t / ntn;
        tn = t - tm * ntn;
        const int4 rec = p.tile_info[tm];
        ti.expert = rec.x;
        ti.rows_valid = (rec.z <= BM + XR) ? rec.z : BM;
        ti.row_base = rec.y;
    } else {
        const int ntm = (p.M + BM - 1) / BM;
        const int gm = p.group_m;
        const int in_group = gm * ntn;
        const int g = t / in_group;
        const int first = g * gm;
        const int gsize = min(ntm - first, gm);
        const int r = t - g * in_group;
        tm = first + r % gsize;
        tn = r / gsize;
        ti.rows_valid = min(BM, p.M - tm * BM);
        ti.row_base = (int64_t)tm * BM;
    }
    ti.n0 = tn * BN;
}

// The tile of this workgroup (one tile per workgroup, split-K aware).
template <int BM, int BN, bool GROUPED, int XR = 0>
__device__ __forceinline__ bool locate_tile(const GemmParams &p, TileInfo &ti)
{
    const int ntn = (p.N + BN - 1) / BN;
    if constexpr (GROUPED && BM == 32) {
        // decode-sized tile tables: tiles in grid order (tiles of one expert
        // share only a few A rows, nothing to keep in one L2), so that the
        // tile record and the tile count load together; the record of a
        // workgroup past the table is read (the table has room) but not used
        const int t = blockIdx.x;
        const int nmt = *p.n_mtiles;
        tile_coords<BM, BN, true, XR>(p, t, ntn, ti);
        __builtin_amdgcn_sched_barrier(0);  // both loads go out before either is waited for
        if (t >= nmt * ntn || ti.expert < 0)  // (testing the record keeps its load above the branch)
            return false;
    } else if constexpr (GROUPED) {
        const int t = xcd_logical_tile(blockIdx.x, *p.n_mtiles * ntn);
        if (t < 0)
            return false;
        tile_coords<BM, BN, true, XR>(p, t, ntn, ti);
    } else if (p.k_offsets) {
        const int ntm = (p.M + BM - 1) / BM, per = ntm * ntn;
        const int t = xcd_logical_tile(blockIdx.x, p.n_batches * per);
        if (t < 0)
            return false;
        const int e = t / per;
        tile_coords<BM, BN, false>(p, t - e * per, ntn, ti);
        ti.expert = e;
        ti.c_row0 = (int64_t)e * p.M;
    } else {
        const int ntm = (p.M + BM - 1) / BM;
        const int S = p.splitk > 1 ? p.splitk : 1;
        const int t2 = xcd_logical_tile(blockIdx.x, ntm * ntn * S);
        if (t2 < 0)
            return false;
        const int t = t2 / S;
        tile_coords<BM, BN, false>(p, t, ntn, ti);
        ti.split = t2 - t * S;
    }
    return true;
}

// Multiply one LDS k-tile (128 bytes of K: four k-steps of 32 bytes) into the
// wave's 32x32 accumulator tiles.
// Eight E4M3 bytes (K order) -> eight bf16 (exact: every E4M3 value is a
// bf16 value), element 0 in the low half of the first word.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 v)
{
    uint4 r;
    r.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, false));
    r.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, true));
    r.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, false));
    r.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, true));
    return r;
}

// BQ8: the B tile holds E4M3 bytes, 64 per row and k-tile (4 chunks of 16,
// chunk c of row r at c ^ ((r >> 2) & 3)); a fragment is 8 bytes, widened to
// bf16 in registers.
template <typename E, int TM, int TN, int WTM, int WTN, bool BQ8 = false, int XM = 0, int BM = 0>
__device__ __forceinline__ void tile_mma(f32x16 (&acc)[TM][TN], const uint4 *a, const uint4 *b, int wm, int wn, int lane,
                                         f32x16 (*accx)[XM > 0 ? XM : 1][1] = nullptr, bool xlive = false)
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int c = s * 2 + (lane >> 5);
        uint4 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WTM + i * 32 + (lane & 31);
            af[i] = a[r * 8 + (c ^ ((r >> 1) & 7))];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int r = wn * WTN + j * 32 + (lane & 31);
            if constexpr (BQ8)
                bfr[j] = e4m3x8_to_bf16(reinterpret_cast<const uint2 *>(b + r * 4 + (s ^ ((r >> 2) & 3)))[lane >> 5]);
            else
                bfr[j] = b[r * 8 + (c ^ ((r >> 1) & 7))];
        }
        // B fragment first: the tile's rows are output columns, so a lane
        // owns runs of 4 consecutive output columns of output row lane % 32.
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = Mfma32<E>::run(bfr[j], af[i], acc[i][j]);
        if constexpr (XM > 0) {
            // the extra rows BM .. BM + 32 XM - 1, times the wave's 32 columns
            // wn WTN + 32 wm .. (one B fragment, read again); skipped (uniform
            // branch) when the tile has no extra rows
            if (!xlive)
                continue;
            const int rb = wn * WTN + wm * 32 + (lane & 31);
            const uint4 bx = b[rb * 8 + (c ^ ((rb >> 1) & 7))];
#pragma unroll
            for (int i = 0; i < XM; ++i) {
                const int r = BM + i * 32 + (lane & 31);
                (*accx)[i][0] = Mfma32<E>::run(bx, a[r * 8 + (c ^ ((r >> 1) & 7))], (*accx)[i][0]);
            }
        }
    }
}

// The same product (bf16 operands in LDS, no extra rows) with the fragment
// reads software-pipelined: the fragments of k-step s + 1 go into a second
// register set, one LDS read between consecutive MFMAs of k-step s, so a
// k-step's LDS latency hides behind the previous one's multiplies instead of
// stalling the matrix pipe (left to itself, the compiler reads each k-step's
// fragments just before its first MFMA and waits for them there).  Each
// k-step is its own scheduling region; the group barriers fix the
// interleave inside it.  Same MFMAs in the same order: the sums are
// bit-identical.  Measured at wide_prefill: x-pass 346 -> 333-337 us,
// up-projection 291-293 -> 281-283 us; zipf_skew grouped GEMM 1 226-228 ->
// 218-222 us.
// (the accumulators and two fragment sets fit beside the addresses, and a
// k-step has at least as many MFMAs as fragment reads to interleave)
template <int TM, int TN>
constexpr bool kPipeFits = TM * TN * 16 + 8 * (TM + TN) <= 176 && TM * TN >= TM + TN;

template <typename E, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void tile_mma_pipe(f32x16 (&acc)[TM][TN], const uint4 *a, const uint4 *b, int wm, int wn,
                                              int lane)
{
    uint4 af[2][TM], bfr[2][TN];
    auto load = [&](int s, uint4(&fa)[TM], uint4(&fb)[TN]) {
        const int c = s * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WTM + i * 32 + (lane & 31);
            fa[i] = a[r * 8 + (c ^ ((r >> 1) & 7))];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int r = wn * WTN + j * 32 + (lane & 31);
            fb[j] = b[r * 8 + (c ^ ((r >> 1) & 7))];
        }
    };
    load(0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cur = s & 1;
        if (s < 3)
            load(s + 1, af[cur ^ 1], bfr[cur ^ 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = Mfma32<E>::run(bfr[cur][j], af[cur][i], acc[i][j]);
        if (s < 3) {
#pragma unroll
            for (int q = 0; q < TM + TN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Epilogue of four consecutive output columns col .. col + 3 of one row.
// Columns below c_split go to C32 in fp32 (+ bias32), the rest to C, with
// relu^2 from relu2_from on.  c_split is a multiple of 4, so a group never
// straddles it.
template <typename E>
__device__ __forceinline__ void store_out4(const GemmParams &p, int64_t row, int col, float (&v)[4])
{
    if (col < p.c_split) {
        if (p.bias32) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] += p.bias32[col + r];
        }
        store4(p.C32 + row * p.ldc32 + col, v[0], v[1], v[2], v[3]);
        return;
    }
    const int mc = col - p.c_split;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (mc + r >= p.relu2_from) {
            const float t = fmaxf(v[r], 0.f);
            v[r] = t * t;
        }
    store4(static_cast<E *>(p.C) + row * p.ldc + mc, v[0], v[1], v[2], v[3]);
}

// Epilogue straight from the accumulators: each lane stores runs of four
// output columns (times the column scales cs, if any).
// silu(g) * v for a gated pair; silu(g) = g / (1 + e^-g) (for g -> -inf
// the quotient tends to -0: e^-g overflows to +inf first).
__device__ __forceinline__ float glu_value(float g, float v) { return g / (1.f + expf(-g)) * v; }

// C column of the output that the gate group starting at B column `col`
// (col >= glu_from, (col - glu_from) % 16 < 8) feeds.
__device__ __forceinline__ int glu_out_col(const GemmParams &p, int col)
{
    const int rel = col - p.glu_from;
    return p.glu_from - p.c_split + (rel >> 4) * 8 + (rel & 15);
}

template <typename E, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_tile_direct(const GemmParams &p, const f32x16 (&acc)[TM][TN], int64_t row_base,
                                                  int rows_valid, int n0, int wm, int wn, int lane,
                                                  const float *cs = nullptr)
{
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int rl = wm * WTM + i * 32 + (lane & 31);
        if (rl >= rows_valid)
            continue;
        const int64_t row = row_base + rl;
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * WTN + jn * 32 + 8 * g + 4 * (lane >> 5);
                if (col >= p.N)
                    continue;
                float v[4] = {acc[i][jn][4 * g], acc[i][jn][4 * g + 1], acc[i][jn][4 * g + 2], acc[i][jn][4 * g + 3]};
                if (cs) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] *= cs[col + r];
                }
                if (col >= p.glu_from) {
                    // tiles start at multiples of 32 and glu_from is a multiple
                    // of 16, so the gate groups are the even g and their value
                    // groups (8 columns on) the next register group
                    if (g & 1)
                        continue;
                    float u[4] = {acc[i][jn][4 * g + 4], acc[i][jn][4 * g + 5], acc[i][jn][4 * g + 6],
                                  acc[i][jn][4 * g + 7]};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = glu_value(v[r], cs ? u[r] * cs[col + 8 + r] : u[r]);
                    store4(static_cast<E *>(p.C) + row * p.ldc + glu_out_col(p, col), v[0], v[1], v[2], v[3]);
                    continue;
                }
                store_out4<E>(p, row, col, v);
            }
        }
    }
}

// Epilogue through LDS: each wave converts its block 32 rows at a time into
// its own area `stg` (32 rows x WTN elements of E), then writes whole
// 16-byte chunks of output rows -- a store instruction covers a few full
// rows instead of 16 bytes in each of 32 rows.  Same arithmetic as
// store_tile_direct; for tiles without fp32 router columns (n0 >= c_split).
// Chunk c of staged row r sits at position c ^ (r % CPR).
template <typename E, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_tile_staged(const GemmParams &p, const f32x16 (&acc)[TM][TN], int64_t row_base,
                                                  int rows_valid, int n0, int wm, int wn, int lane, uint4 *stg,
                                                  const float *cs = nullptr)
{
    constexpr int ES = (int)sizeof(E);
    constexpr int CPR = WTN * ES / 16;  // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPR;       // staged rows per store instruction
    // chunk c of staged row r sits at c ^ (r % CPR), or, for a CPR that is not
    // a power of two (160-column wave tiles), at (c + r) % CPR
    constexpr bool P2 = (CPR & (CPR - 1)) == 0;
    static_assert(CPR >= 1 && CPR <= 64, "staged row");
    auto spos = [](int r, int c) { return P2 ? (c ^ (r & (CPR - 1))) : (c + r) % CPR; };
    const int lr = lane & 31, lc = lane >> 5;
    const int cbase = n0 + wn * WTN - p.c_split;  // first C column of this wave
    const int rows_here = rows_valid - wm * WTM;
    const int cw = lane % CPR;
    const bool col_ok = n0 + wn * WTN + cw * (16 / ES) < p.N;
    E *C = static_cast<E *>(p.C);
    char *sb = reinterpret_cast<char *>(stg);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i * 32 >= rows_here)  // uniform: nothing left to store
            break;
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cc = jn * 32 + 8 * g + 4 * lc;  // column inside the wave block
                float v[4] = {acc[i][jn][4 * g], acc[i][jn][4 * g + 1], acc[i][jn][4 * g + 2], acc[i][jn][4 * g + 3]};
                if (cs) {
                    const int col = n0 + wn * WTN + cc;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] *= (col + r < p.N) ? cs[col + r] : 0.f;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (cbase + cc + r >= p.relu2_from) {
                        const float t = fmaxf(v[r], 0.f);
                        v[r] = t * t;
                    }
                const int byte = cc * ES, ch = byte / 16;
                store4(reinterpret_cast<E *>(sb + (lr * CPR + spos(lr, ch)) * 16 + byte % 16), v[0], v[1], v[2],
                       v[3]);
            }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r0 = 0; r0 < 32; r0 += RPI) {
            const int rl = r0 + lane / CPR;
            // P2: the 64 lanes cover RPI whole rows and 32 % RPI == 0; otherwise
            // the lanes past RPI rows, and rows past 32, have nothing to store
            if (!P2 && (lane >= RPI * CPR || rl >= 32))
                continue;
            const uint4 v = stg[rl * CPR + spos(rl, cw)];
            if (col_ok && i * 32 + rl < rows_here)
                store16_stream(C, ((row_base + wm * WTM + i * 32 + rl) * p.ldc + cbase + cw * (16 / ES)) * ES, v);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

// The staged epilogue of an all-fp32 output (c_split >= N: every column
// goes to C32, no bias, no scales): each wave stages 32 rows x WTN floats,
// then writes whole 16-byte chunks of output rows (chunk c of staged row r
// at position c ^ (r % CPR)).
template <typename E, int TM, int TN, int WTM, int WTN, int ACT>
__device__ __forceinline__ void store_tile_staged_f32(const GemmParams &p, const f32x16 (&acc)[TM][TN],
                                                      int64_t row_base, int rows_valid, int n0, int wm, int wn,
                                                      int lane, uint4 *stg)
{
    constexpr int CPR = WTN * 4 / 16;  // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPR;      // staged rows per store instruction
    static_assert(CPR >= 1 && CPR <= 64 && (CPR & (CPR - 1)) == 0, "staged row");
    const int lr = lane & 31, lc = lane >> 5;
    const int cbase = n0 + wn * WTN;  // first output column of this wave
    const int rows_here = rows_valid - wm * WTM;
    const int cw = lane % CPR;
    const bool col_ok = cbase + cw * 4 < p.N;
    constexpr int NQ = 32 / RPI;  // store instructions per 32 staged rows
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i * 32 >= rows_here)  // uniform: nothing left to store
            break;
        // gradient epilogues: this block's pre-activations, all loads in flight before
        // the staging (gate chunk, and for gated pairs the value chunk)
        float4 pg[ACT >= ACT_RELU2_GRAD ? NQ : 1], pv[ACT == ACT_GLU_GRAD ? NQ : 1];
        if constexpr (ACT >= ACT_RELU2_GRAD) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int rl = q * RPI + lane / CPR;
                const int col = cbase + cw * 4;
                const int pc = ACT == ACT_GLU_GRAD ? 16 * (col >> 3) + (col & 7) : col;
                pg[q] = make_float4(0.f, 0.f, 0.f, 0.f);
                if constexpr (ACT == ACT_GLU_GRAD)
                    pv[q] = pg[q];
                if (col_ok && i * 32 + rl < rows_here) {
                    const float *src = p.act_pre + (row_base + wm * WTM + i * 32 + rl) * p.ld_pre + pc;
                    pg[q] = *reinterpret_cast<const float4 *>(src);
                    if constexpr (ACT == ACT_GLU_GRAD)
                        pv[q] = *reinterpret_cast<const float4 *>(src + 8);
                }
            }
        }
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ch = jn * 8 + 2 * g + lc;  // 16-byte chunk of columns jn 32 + 8 g + 4 lc ..
                stg[lr * CPR + (ch ^ (lr & (CPR - 1)))] =
                    make_uint4(__float_as_uint(acc[i][jn][4 * g]), __float_as_uint(acc[i][jn][4 * g + 1]),
                               __float_as_uint(acc[i][jn][4 * g + 2]), __float_as_uint(acc[i][jn][4 * g + 3]));
            }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int rl = q * RPI + lane / CPR;
            const uint4 v = stg[rl * CPR + (cw ^ (rl & (CPR - 1)))];
            if (!col_ok || i * 32 + rl >= rows_here)
                continue;
            const int64_t row = row_base + wm * WTM + i * 32 + rl;
            const int col = cbase + cw * 4;
            float s4[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
            if constexpr (ACT < ACT_RELU2_GRAD)
                store16_stream(p.C32, (row * p.ldc32 + col) * 4, v);
            if constexpr (ACT == ACT_RELU2) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float t = fmaxf(s4[r], 0.f);
                    s4[r] = t * t;
                }
                store4(static_cast<E *>(p.C) + row * p.ldc + col, s4[0], s4[1], s4[2], s4[3]);
            } else if constexpr (ACT == ACT_GLU) {
                if ((cw & 3) >= 2)  // value chunk: written with its gate chunk
                    continue;
                // gate chunk: its values are two chunks on in the staged row
                const uint4 u = stg[rl * CPR + ((cw + 2) ^ (rl & (CPR - 1)))];
                const float u4[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                     __uint_as_float(u.w)};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s4[r] = glu_value(s4[r], u4[r]);
                store4(static_cast<E *>(p.C) + row * p.ldc + (col >> 4) * 8 + (col & 15), s4[0], s4[1], s4[2], s4[3]);
            } else if constexpr (ACT == ACT_RELU2_GRAD) {
                const float a4[4] = {pg[q].x, pg[q].y, pg[q].z, pg[q].w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s4[r] = a4[r] > 0.f ? 2.f * a4[r] * s4[r] : 0.f;
                store4(static_cast<E *>(p.C) + row * p.ldc + col, s4[0], s4[1], s4[2], s4[3]);
            } else if constexpr (ACT == ACT_GLU_GRAD) {
                const int gc = 16 * (col >> 3) + (col & 7);
                const float g4[4] = {pg[q].x, pg[q].y, pg[q].z, pg[q].w}, v4[4] = {pv[q].x, pv[q].y, pv[q].z, pv[q].w};
                float dg[4], dv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sg = 1.f / (1.f + expf(-g4[r]));
                    dg[r] = s4[r] * v4[r] * sg * (1.f + g4[r] * (1.f - sg));
                    dv[r] = s4[r] * g4[r] * sg;
                }
                store4(static_cast<E *>(p.C) + row * p.ldc + gc, dg[0], dg[1], dg[2], dg[3]);
                store4(static_cast<E *>(p.C) + row * p.ldc + gc + 8, dv[0], dv[1], dv[2], dv[3]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

// The staged epilogue of a wave block whose B columns are all gated pairs
// (bcol0 = n0 + wn WTN >= glu_from): the wave stages 32 rows x WTN / 2
// outputs silu(gate) * value, then writes whole 16-byte chunks of output
// rows.  bcol0 - glu_from is a multiple of 16, so the gate groups are the even
// register groups g, their values sit in group g + 1, and the outputs of gate
// group g of MFMA tile jn are staged columns 16 jn + 4 g + 4 (lane / 32).
template <typename E, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_tile_staged_glu(const GemmParams &p, const f32x16 (&acc)[TM][TN],
                                                      int64_t row_base, int rows_valid, int n0, int wm, int wn,
                                                      int lane, uint4 *stg, const float *cs = nullptr)
{
    constexpr int ES = (int)sizeof(E);
    constexpr int CPR = (WTN / 2) * ES / 16;  // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPR;             // staged rows per store instruction
    static_assert(CPR >= 1 && CPR <= 64 && (CPR & (CPR - 1)) == 0, "staged row");
    const int lr = lane & 31, lc = lane >> 5;
    const int bcol0 = n0 + wn * WTN;
    const int cbase = glu_out_col(p, bcol0);  // C column of the wave's first output
    const int rows_here = rows_valid - wm * WTM;
    const int cw = lane % CPR;
    const bool col_ok = bcol0 + cw * 2 * (16 / ES) < p.N;  // a chunk's outputs come from 2 x its width of B
    E *C = static_cast<E *>(p.C);
    char *sb = reinterpret_cast<char *>(stg);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i * 32 >= rows_here)  // uniform: nothing left to store
            break;
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
            for (int g = 0; g < 4; g += 2) {
                float v[4] = {acc[i][jn][4 * g], acc[i][jn][4 * g + 1], acc[i][jn][4 * g + 2], acc[i][jn][4 * g + 3]};
                float u[4] = {acc[i][jn][4 * g + 4], acc[i][jn][4 * g + 5], acc[i][jn][4 * g + 6],
                              acc[i][jn][4 * g + 7]};
                if (cs) {
                    const int col = bcol0 + jn * 32 + 8 * g + 4 * lc;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        v[r] *= (col + r < p.N) ? cs[col + r] : 0.f;
                        u[r] *= (col + 8 + r < p.N) ? cs[col + 8 + r] : 0.f;
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] = glu_value(v[r], u[r]);
                const int cc = jn * 16 + 4 * g + 4 * lc;  // output column inside the wave block
                const int byte = cc * ES, ch = byte / 16;
                store4(reinterpret_cast<E *>(sb + (lr * CPR + (ch ^ (lr & (CPR - 1)))) * 16 + byte % 16), v[0], v[1],
                       v[2], v[3]);
            }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r0 = 0; r0 < 32; r0 += RPI) {
            const int rl = r0 + lane / CPR;
            const uint4 v = stg[rl * CPR + (cw ^ (rl & (CPR - 1)))];
            if (col_ok && i * 32 + rl < rows_here)
                store16_stream(C, ((row_base + wm * WTM + i * 32 + rl) * p.ldc + cbase + cw * (16 / ES)) * ES, v);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

// k-tile kt of A and B straight into the LDS stages na, nb (buffer loads with
// the LDS bit: lane l of a wave writes 16 bytes at the wave's base + 16 l;
// rows out of range read as zeros).  Position P of an A tile holds row
// r = P / 8, chunk (P % 8) ^ ((r / 2) % 8); of a B tile row P / CHB, chunk
// (P % CHB) ^ the B swizzle; instruction i of wave w fills positions
// (i * NW + w) * 64 .. +63.  With issue false every load is out of range and
// reads nothing: the instructions still go out, so that the number of loads
// in flight after a tile does not depend on the data.
template <int NIA, int NIB, int NW, int BPOL = 0>
__device__ __forceinline__ void tile_dma(uint4 *na, uint4 *nb, bool issue, unsigned kt, __amdgpu_buffer_rsrc_t ra,
                                         __amdgpu_buffer_rsrc_t rb, const unsigned (&a_off)[NIA],
                                         const unsigned (&b_off)[NIB], unsigned bks, int wave)
{
#pragma unroll
    for (int i = 0; i < NIA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LMOE_LDS(na + (i * NW + wave) * 64), 16,
                                                 issue ? a_off[i] + kt * 128u : kOOB, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NIB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LMOE_LDS(nb + (i * NW + wave) * 64), 16,
                                                 issue ? b_off[i] + kt * bks : kOOB, 0, 0, BPOL);
}

// One k-step: the refill of stages na, nb with tile kt, then (if live) the
// tile held in sa, sb into the accumulators.  The four stages are different
// LDS arrays; the restrict qualifiers tell the compiler so, which keeps it
// from making the reads of sa, sb wait for the DMA into na, nb.
template <typename E, int TM, int TN, int WTM, int WTN, bool BQ8, int NIA, int NIB, int NW, int XM = 0, int BM = 0,
          int BPOL = 0>
__device__ __forceinline__ void dma_mma(uint4 *__restrict__ na, uint4 *__restrict__ nb, const uint4 *__restrict__ sa,
                                        const uint4 *__restrict__ sb, bool issue, unsigned kt,
                                        __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                        const unsigned (&a_off)[NIA], const unsigned (&b_off)[NIB], unsigned bks,
                                        int wave, bool live, f32x16 (&acc)[TM][TN], int wm, int wn, int lane,
                                        f32x16 (*accx)[XM > 0 ? XM : 1][1] = nullptr, bool xlive = false)
{
    tile_dma<NIA, NIB, NW, BPOL>(na, nb, issue, kt, ra, rb, a_off, b_off, bks, wave);
    if (live) {
        if constexpr (!BQ8 && XM == 0 && sizeof(E) == 2 && kPipeFits<TM, TN>)
            tile_mma_pipe<E, TM, TN, WTM, WTN>(acc, sa, sb, wm, wn, lane);
        else
            tile_mma<E, TM, TN, WTM, WTN, BQ8, XM, BM>(acc, sa, sb, wm, wn, lane, accx, xlive);
    }
}

// NT = 64 * WM * WN threads; NS LDS stages (2 or 3), one barrier per k-tile;
// tiles kt+1 .. kt+NS-1 are in flight while tile kt is multiplied.  STAGE only
// names the layer stage, so that each stage is its own kernel symbol in
// profiles.  BQ8: B holds E4M3 bytes (grouped, bf16 only; see tile_mma) with
// per-column scales p.scaleB.
//
// XR > 0 (grouped, bf16 B, no ACT): a tile holds up to BM + XR rows; the
// extra rows BM .. BM + XR - 1 are a second block of XR / 32 MFMA row tiles
// per wave, over the wave's 32 columns wn WTN + 32 wm .. (WM 32 = WTN), read
// from the same A and B k-tiles -- an expert a few rows past a multiple of
// BM then streams its weights once instead of twice.
template <typename E, int BM, int BN, int WM, int WN, int NS, bool GROUPED, int MINB = 1, int STAGE = 0,
          bool BQ8 = false, int ACT = ACT_NONE, int XR = 0>
__global__ __launch_bounds__(64 * WM * WN, MINB) void gemm_kernel(const GemmParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int NW = WM * WN, NT = 64 * NW;
    constexpr int VEC = 16 / (int)sizeof(E);    // elements per 16-byte chunk
    constexpr int BK = 8 * VEC;                 // elements per k-tile
    constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32; // 32x32 MFMA tiles per wave
    constexpr int CHB = BQ8 ? 4 : 8;           // 16-byte chunks per B row and k-tile
    constexpr int EB = BQ8 ? 1 : (int)sizeof(E); // bytes per B element
    constexpr int BMA = BM + XR;                // A rows per tile (the extra block included)
    constexpr int XM = XR / 32;                 // extra MFMA row tiles per wave
    constexpr int NIA = BMA * 8 / NT, NIB = BN * CHB / NT;  // LDS-DMA instructions per thread
    static_assert(TM >= 1 && TN >= 1 && NIA >= 1 && NIB >= 1, "tile shape");
    static_assert(NIA * NT == BMA * 8 && NIB * NT == BN * CHB, "tile shape");
    static_assert(XR == 0 || (GROUPED && !BQ8 && ACT == ACT_NONE && XR % 32 == 0 && WM * 32 == WTN),
                  "extra rows: grouped bf16 tiles, one 32-column block per wave row");
    static_assert(NS >= 2 && NS <= 4, "stages");
    // Expert weights that one M-tile uses alone -- decode's 32-row tiles, and
    // 256-row tables with extra rows, whose experts average at most 320 rows --
    // load non-temporally, so that streaming them does not evict the gathered
    // A rows the expert's N-tiles share in L2.  Measured: decode_eff grouped
    // GEMMs 53.9 / 56.0 -> 48.9 / 50.5 us, wide_prefill 354 / 358 -> 342 / 355
    // us; with zipf_skew's 512 rows per expert (weights shared by the
    // expert's M-tiles) they lost 3-4 %, so those tables keep the default.
    constexpr int BPOL = (GROUPED && (BM == 32 || XR > 0)) ? kLoadNonTemporal : 0;
    static_assert(!BQ8 || (GROUPED && sizeof(E) == 2), "E4M3 B operands: grouped bf16 GEMMs");

    __shared__ uint4 sA0[BMA * 8], sA1[BMA * 8], sA2[NS > 2 ? BMA * 8 : 1], sA3[NS > 3 ? BMA * 8 : 1];
    __shared__ uint4 sB0[BN * CHB], sB1[BN * CHB], sB2[NS > 2 ? BN * CHB : 1], sB3[NS > 3 ? BN * CHB : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // decode-sized tile tables with a row table: this thread's A rows load
    // together with the tile record (both are indexed by the grid position),
    // instead of after it through the gather
    int pre_row[NIA];
    if constexpr (GROUPED && BM == 32) {
        if (p.tile_rows) {
            const int tm = blockIdx.x / ((p.N + BN - 1) / BN);
#pragma unroll
            for (int i = 0; i < NIA; ++i)
                pre_row[i] = p.tile_rows[tm * 32 + (((i * NW + wave) * 64 + lane) >> 3)];
        }
    }
    TileInfo ti;
    if (!locate_tile<BM, BN, GROUPED, XR>(p, ti))
        return;
    const int rows_valid = ti.rows_valid, expert = ti.expert, split = ti.split;
    const int64_t row_base = ti.row_base;
    const int n0 = ti.n0;

    const int wm = wave / WN, wn = wave - (wave / WN) * WN;

    // Buffer descriptors and this thread's source offsets (fixed for the K loop).
    const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(p.A, p.a_bytes);
    const char *Bexp = static_cast<const char *>(p.B) + (int64_t)expert * p.strideB * EB;
    const unsigned bks = p.b_kstep ? (unsigned)p.b_kstep : CHB * 16u;  // bytes per k-tile step of B
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        make_rsrc(Bexp, p.b_kstep ? (int64_t)(p.K / BK) * p.b_kstep : (int64_t)p.N * p.ldb * EB);
    unsigned a_off[NIA], b_off[NIB];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int P = (i * NW + wave) * 64 + lane, r = P >> 3, c = (P & 7) ^ ((r >> 1) & 7);
        a_off[i] = kOOB;
        if (r < rows_valid) {
            int64_t arow = row_base + r;
            if (GROUPED && BM == 32 && p.tile_rows)
                arow = pre_row[i];
            else if (GROUPED && p.gather)
                arow = p.gather[arow];
            a_off[i] = (unsigned)(arow * p.lda * (int64_t)sizeof(E)) + c * 16;
        }
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
        const int P = (i * NW + wave) * 64 + lane, r = P / CHB;
        const int c = BQ8 ? (P % CHB) ^ ((r >> 2) & 3) : (P & 7) ^ ((r >> 1) & 7);
        b_off[i] = (n0 + r < p.N) ? (unsigned)((int64_t)(n0 + r) * p.ldb * EB) + c * 16 : kOOB;
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc[i][j][q] = 0.f;
    f32x16 accx[XM > 0 ? XM : 1][1];  // the extra rows' block (XR > 0)
#pragma unroll
    for (int i = 0; i < (XM > 0 ? XM : 1); ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            accx[i][0][q] = 0.f;

    // A wave whose whole tile is padding (rows past the valid range or
    // columns past N) still loads and syncs but skips its MFMAs, leaving the
    // SIMD's matrix pipe to the other wave on it.
    const bool wave_live = (wm * WTM < rows_valid) && (n0 + wn * WTN < p.N);
    constexpr int NI = NIA + NIB;
    // this workgroup's k-tiles: [kt0, kt0 + nkl)
    int kt0 = 0, nkl = p.K / BK;
    if (!GROUPED && p.splitk > 1) {
        const int per = (nkl + p.splitk - 1) / p.splitk;
        kt0 = split * per;
        nkl = min(per, nkl - kt0);
    }
    if (!GROUPED && p.k_offsets) {
        kt0 = p.k_offsets[expert] / BK;
        nkl = p.k_offsets[expert + 1] / BK - kt0;
    }
    const int64_t c_row_base = row_base + ti.c_row0;  // first output row of the tile
    tile_dma<NIA, NIB, NW, BPOL>(sA0, sB0, nkl > 0, kt0, ra_rsrc, rb_rsrc, a_off, b_off, bks, wave);
    if constexpr (NS > 2)
        tile_dma<NIA, NIB, NW, BPOL>(sA1, sB1, nkl > 1, kt0 + 1, ra_rsrc, rb_rsrc, a_off, b_off, bks, wave);
    if constexpr (NS > 3)
        tile_dma<NIA, NIB, NW, BPOL>(sA2, sB2, nkl > 2, kt0 + 2, ra_rsrc, rb_rsrc, a_off, b_off, bks, wave);

// One k-tile step j: wait until tile j is in LDS for every wave (the NS - 2
// tiles issued after it, real or out of range, may stay in flight) and every
// wave is done with the stage about to be refilled; refill it with tile
// j + NS - 1; multiply tile j.
#define LMOE_KSTEP(SA, SB, NA, NB)                                                                            \
    {                                                                                                         \
        wait_vm_lgkm0<(NS - 2) * NI>();                                                                       \
        __builtin_amdgcn_s_barrier();                                                                         \
        __builtin_amdgcn_sched_barrier(0);                                                                    \
        dma_mma<E, TM, TN, WTM, WTN, BQ8, NIA, NIB, NW, XM, BM, BPOL>(                                        \
            NA, NB, SA, SB, j + NS - 1 < nkl, (unsigned)(kt0 + j + NS - 1), ra_rsrc, rb_rsrc, a_off, b_off, bks,  \
            wave, wave_live, acc, wm, wn, lane, XM > 0 ? &accx : nullptr, rows_valid > BM);                  \
        __builtin_amdgcn_sched_barrier(0);                                                                    \
        if (++j >= nkl)                                                                                       \
            break;                                                                                            \
    }

    int j = 0;
    if (nkl <= 0) {
        // an empty K range: the products are zero
    } else if constexpr (NS == 2) {
        for (;;) {
            LMOE_KSTEP(sA0, sB0, sA1, sB1)
            LMOE_KSTEP(sA1, sB1, sA0, sB0)
        }
    } else if constexpr (NS == 3) {
        for (;;) {
            LMOE_KSTEP(sA0, sB0, sA2, sB2)
            LMOE_KSTEP(sA1, sB1, sA0, sB0)
            LMOE_KSTEP(sA2, sB2, sA1, sB1)
        }
    } else {
        for (;;) {
            LMOE_KSTEP(sA0, sB0, sA3, sB3)
            LMOE_KSTEP(sA1, sB1, sA0, sB0)
            LMOE_KSTEP(sA2, sB2, sA1, sB1)
            LMOE_KSTEP(sA3, sB3, sA2, sB2)
        }
    }
#undef LMOE_KSTEP

    if (!GROUPED && p.splitk > 1) {
        // raw fp32 partial sums; the reduce kernel applies the epilogue
        float *P = p.partial + (int64_t)split * p.M * p.N;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int rl = wm * WTM + i * 32 + (lane & 31);
            if (rl >= rows_valid)
                continue;
            const int64_t row = row_base + rl;
#pragma unroll
            for (int jj = 0; jj < TN; ++jj)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + wn * WTN + jj * 32 + 8 * g + 4 * (lane >> 5);
                    if (col < p.N)
                        store4(P + row * p.N + col, acc[i][jj][4 * g], acc[i][jj][4 * g + 1], acc[i][jj][4 * g + 2],
                               acc[i][jj][4 * g + 3]);
                }
        }
        return;
    }

    const float *cs = (BQ8 && p.scaleB) ? p.scaleB + (int64_t)expert * p.N : nullptr;  // column scales
    // an all-fp32 output without bias or scales: staged through LDS when the
    // waves' areas fit in two stage arrays
    constexpr int WAVE_F = 32 * WTN * 4 / 16;  // 16-byte units of a wave's fp32 area
    constexpr bool F32_IN_A = NW <= 2 * ((BM * 8) / WAVE_F);
    constexpr bool F32_FITS = F32_IN_A || NW <= 2 * ((BN * CHB) / WAVE_F);
    static_assert(ACT == ACT_NONE || (F32_FITS && !BQ8), "activation epilogues: fp32 staging");
    if constexpr (F32_FITS) {
        if (ACT != ACT_NONE || (p.c_split >= p.N && p.glu_from >= p.N && !p.bias32 && !cs)) {
            constexpr int PER = (F32_IN_A ? BM * 8 : BN * CHB) / WAVE_F;
            wait_vm_lgkm0<0>();
            __builtin_amdgcn_s_barrier();
            uint4 *stg = (F32_IN_A ? (wave < PER ? sA0 : sA1) : (wave < PER ? sB0 : sB1)) + (wave % PER) * WAVE_F;
            store_tile_staged_f32<E, TM, TN, WTM, WTN, ACT>(p, acc, c_row_base, rows_valid, n0, wm, wn, lane, stg);
            return;
        }
    }
    // fp32 outputs, and tiles that hold router columns or straddle the start
    // of the gated pairs: straight from the registers
    if (sizeof(E) != 2 || n0 < p.c_split || (n0 < p.glu_from && n0 + BN > p.glu_from)) {
        store_tile_direct<E, TM, TN, WTM, WTN>(p, acc, c_row_base, rows_valid, n0, wm, wn, lane, cs);
        if constexpr (XM > 0) {
            if (rows_valid > BM && wave_live)
                store_tile_direct<E, XM, 1, XR, 32>(p, accx, c_row_base + BM, rows_valid - BM,
                                                    n0 + wn * WTN + wm * 32, 0, 0, lane, cs);
        }
        return;
    }
    if constexpr (sizeof(E) == 2) {
        // every wave is done with the k-tiles (no load is in flight after the
        // last k-step): the first two A (else B) stage arrays hold the waves'
        // epilogue areas
        constexpr int WAVE_U = 32 * WTN * 2 / 16;  // 16-byte units per wave area
        constexpr bool IN_A = NW <= 2 * ((BM * 8) / WAVE_U);
        constexpr int PER_ARR = (IN_A ? BM * 8 : BN * CHB) / WAVE_U;  // areas per stage array
        static_assert(PER_ARR >= 1 && NW <= 2 * PER_ARR, "epilogue areas fit in two stage arrays");
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        uint4 *stg = (IN_A ? (wave < PER_ARR ? sA0 : sA1) : (wave < PER_ARR ? sB0 : sB1)) + (wave % PER_ARR) * WAVE_U;
        constexpr int CPR = WAVE_U / 32;  // 16-byte chunks per staged row
        if (n0 >= p.glu_from) {
            if constexpr ((CPR & (CPR - 1)) == 0)
                store_tile_staged_glu<E, TM, TN, WTM, WTN>(p, acc, c_row_base, rows_valid, n0, wm, wn, lane, stg, cs);
            else  // the gated staging needs power-of-two rows
                store_tile_direct<E, TM, TN, WTM, WTN>(p, acc, c_row_base, rows_valid, n0, wm, wn, lane, cs);
        } else
            store_tile_staged<E, TM, TN, WTM, WTN>(p, acc, c_row_base, rows_valid, n0, wm, wn, lane, stg, cs);
        if constexpr (XM > 0) {
            // the extra rows: XR x 32 outputs per wave, straight from the registers
            if (rows_valid > BM && wave_live)
                store_tile_direct<E, XM, 1, XR, 32>(p, accx, c_row_base + BM, rows_valid - BM,
                                                    n0 + wn * WTN + wm * 32, 0, 0, lane, cs);
        }
    }
#endif
}

// Split-K epilogue: out = epilogue(sum_{s < S} partial[s]) in fixed split
// order, four columns per thread; same epilogue as the GEMM kernel.
template <typename E>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmParams p)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one group of 4 columns
    const int groups = p.N / 4;
    if (q >= (int64_t)p.M * groups)
        return;
    const int64_t row = q / groups;
    const int col = (int)(q - row * groups) * 4;
    // gated pairs: the thread of a gate group also sums its value group
    // (8 columns on); the thread of a value group has nothing to do
    const bool glu = col >= p.glu_from;
    if (glu && ((col - p.glu_from) & 15) >= 8)
        return;
    float v[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.splitk; ++s) {
        const float *src = p.partial + ((int64_t)s * p.M + row) * p.N + col;
        const float4 x = *reinterpret_cast<const float4 *>(src);
        v[0] += x.x;
        v[1] += x.y;
        v[2] += x.z;
        v[3] += x.w;
        if (glu) {
            const float4 w = *reinterpret_cast<const float4 *>(src + 8);
            u[0] += w.x;
            u[1] += w.y;
            u[2] += w.z;
            u[3] += w.w;
        }
    }
    if (glu) {
        for (int r = 0; r < 4; ++r)
            v[r] = glu_value(v[r], u[r]);
        store4(static_cast<E *>(p.C) + row * p.ldc + glu_out_col(p, col), v[0], v[1], v[2], v[3]);
        return;
    }
    store_out4<E>(p, row, col, v);
}


template <int BM, int BN, int NS>
constexpr size_t gemm_lds_bytes()
{
    return (size_t)NS * (BM + BN) * 8 * 16;
}

}  // namespace lmoe
