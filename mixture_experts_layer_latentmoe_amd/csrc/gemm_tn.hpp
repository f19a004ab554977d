// C[m][n] = sum_k A[k][m] B[k][n] for bf16 operands stored with the OUTPUT
// dimensions contiguous ("MN-major": A is [K][lda], B is [K][ldb]), fp32
// output.  These are the weight gradients of the layer: a sum over tokens (or
// over one expert's dispatch rows) of outer products of two row-major
// activations, e.g. dW2_e = H_e^T dY_e.  Reading the operands in this layout
// spares the transposes the K-contiguous GEMM (gemm.hpp) would need.
//
// Batched mode (k_offsets != nullptr): batch e sums over rows
// [k_offsets[e], k_offsets[e + 1]) and writes output rows e M .. e M + M - 1;
// an empty range writes zeros.  Dense mode sums over rows [0, K).
//
// k-tiles are 64 rows.  A k-tile of one operand sits in LDS as 64 rows x 128
// elements (256 bytes per row); the 32-byte segment s of row r is stored at
// segment s ^ (2 (r % 4)).  LDS DMA fills it (lane-sequential 16-byte
// writes); the MFMA fragments come out of it with gfx950's transposing read
// ds_read_b64_tr_b16: in a group of 16 lanes, lane j supplies the address of
// 4 consecutive elements of row kb + j / 4, columns c0 + 4 (j % 4), and lane
// i receives column c0 + i of rows kb .. kb + 3 (measured on the device:
// lane i, element q <- lane 4 q + i / 4, element i % 4).  Two such reads
// give the 8 k-values of a 32x32x16 MFMA fragment; the segment swizzle puts
// the 8 (row, segment) pairs of a half-wave's read in 8 different banks.
#pragma once

#include "gemm.hpp"

namespace lmoe {

typedef short v4s16 __attribute__((ext_vector_type(4)));

// One transposing LDS read: 8 bytes at byte offset `off` of the stage.
__device__ __forceinline__ uint2 lds_read_tr16(const uint4 *stage, unsigned off)
{
    const v4s16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s16 *)((__attribute__((address_space(3))) char *)LMOE_LDS(stage) + off));
    return __builtin_bit_cast(uint2, v);
}

// k-step: the DMA of the next k-tile into na, nb (out-of-range offsets read
// nothing), then the k-tile in sa, sb into the accumulators.  restrict: the
// DMA does not write what the reads read.
template <int TM, int TN, int NI>
__device__ __forceinline__ void tn_step(uint4 *__restrict__ na, uint4 *__restrict__ nb, const uint4 *__restrict__ sa,
                                        const uint4 *__restrict__ sb, __amdgpu_buffer_rsrc_t ra,
                                        __amdgpu_buffer_rsrc_t rb, const unsigned (&a_off)[NI],
                                        const unsigned (&b_off)[NI], unsigned da, unsigned db, int wave, bool live,
                                        f32x16 (&acc)[TM][TN], const unsigned (&ra_off)[TM][2],
                                        const unsigned (&rb_off)[TN][2])
{
#pragma unroll
    for (int i = 0; i < NI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LMOE_LDS(na + (i * 4 + wave) * 64), 16,
                                                 a_off[i] < kOOB ? a_off[i] + da : kOOB, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LMOE_LDS(nb + (i * 4 + wave) * 64), 16,
                                                 b_off[i] < kOOB ? b_off[i] + db : kOOB, 0, 0, 0);
    if (!live)
        return;
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // k16 steps: rows 16 s .. 16 s + 15 (4096 bytes)
        uint4 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint2 lo = lds_read_tr16(sa, ra_off[i][0] + 4096u * s);
            const uint2 hi = lds_read_tr16(sa, ra_off[i][1] + 4096u * s);
            af[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint2 lo = lds_read_tr16(sb, rb_off[j][0] + 4096u * s);
            const uint2 hi = lds_read_tr16(sb, rb_off[j][1] + 4096u * s);
            bfr[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = Mfma32<bf16>::run(bfr[j], af[i], acc[i][j]);
    }
}

// 128x128 output tiles, 4 waves of 64x64, two LDS stages.  p.A / p.lda /
// p.a_bytes, p.B / p.ldb / p.b_bytes: the MN-major operands; p.M, p.N:
// output size per batch; p.K: rows (dense mode);
// p.k_offsets / p.n_batches: batched mode; p.C32 / p.ldc32: fp32 output.
// M and N are multiples of 8 (a 16-byte chunk never straddles the edge).
template <int STAGE = 0>
__global__ __launch_bounds__(256) void gemm_tn_kernel(const GemmParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BM = 128, BN = 128, WN = 2, NW = 4, NT = 256;
    constexpr int WTM = 64, WTN = 64, TM = 2, TN = 2;
    constexpr int UNITS = 64 * 16;   // 16-byte units of one operand's k-tile
    constexpr int NI = UNITS / NT;   // DMA instructions per thread and operand
    __shared__ uint4 sA0[UNITS], sA1[UNITS], sB0[UNITS], sB1[UNITS];

    TileInfo ti;
    if (!locate_tile<BM, BN, false>(p, ti))
        return;
    const int m0 = (int)ti.row_base, n0 = ti.n0, rows_valid = ti.rows_valid;
    const int e = ti.expert;
    const int kstart = p.k_offsets ? p.k_offsets[e] : 0;
    const int krows = (p.k_offsets ? p.k_offsets[e + 1] : p.K) - kstart;
    const int nk = (krows + 63) / 64;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave - (wave / WN) * WN;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, p.b_bytes);
    // DMA: LDS unit P = row r = P / 16, unit u = P % 16 -> stored segment u / 2,
    // half u % 2; it holds logical segment (u / 2) ^ (2 (r % 4)) of the row
    unsigned a_off[NI], b_off[NI];
    int a_row[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int P = (i * NW + wave) * 64 + lane, r = P >> 4, u = P & 15;
        const int col = (((u >> 1) ^ (2 * (r & 3))) << 4) + 8 * (u & 1);  // element within the 128-wide tile
        a_row[i] = r;
        a_off[i] = (m0 + col + 8 <= p.M && r < krows)
                       ? (unsigned)(((int64_t)(kstart + r) * p.lda + m0 + col) * 2) : kOOB;
        b_off[i] = (n0 + col + 8 <= p.N && r < krows)
                       ? (unsigned)(((int64_t)(kstart + r) * p.ldb + n0 + col) * 2) : kOOB;
    }
    // transposing reads: lane group g = lane / 16, j = lane % 16; fragment of
    // rows mb .. mb + 31 of the tile, k rows kb = 8 (g / 2) + 4 q + j / 4
    unsigned ra_off[TM][2], rb_off[TN][2];
    {
        const int g = lane >> 4, j = lane & 15;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = 8 * (g >> 1) + 4 * q + (j >> 2);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int seg = (wm * WTM + i * 32 + 16 * (g & 1)) >> 4;
                ra_off[i][q] = (unsigned)(row * 256 + ((seg ^ (2 * (row & 3))) << 5) + 8 * (j & 3));
            }
#pragma unroll
            for (int jn = 0; jn < TN; ++jn) {
                const int seg = (wn * WTN + jn * 32 + 16 * (g & 1)) >> 4;
                rb_off[jn][q] = (unsigned)(row * 256 + ((seg ^ (2 * (row & 3))) << 5) + 8 * (j & 3));
            }
        }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc[i][jn][q] = 0.f;
    const bool live = (wm * WTM < rows_valid) && (n0 + wn * WTN < p.N);
    const unsigned a_step = (unsigned)(64 * p.lda * 2), b_step = (unsigned)(64 * p.ldb * 2);

    // rows past the range read as zeros: per k-tile, a lane's row must stay
    // below krows (offsets set to kOOB here when it does not)
    auto tile_offs = [&](int kt, unsigned (&ao)[NI], unsigned (&bo)[NI]) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool ok = kt < nk && a_row[i] + 64 * kt < krows;
            ao[i] = ok ? a_off[i] : kOOB;
            bo[i] = ok ? b_off[i] : kOOB;
        }
    };
    unsigned ao[NI], bo[NI];
    tile_offs(0, ao, bo);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LMOE_LDS(sA0 + (i * NW + wave) * 64), 16, ao[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LMOE_LDS(sB0 + (i * NW + wave) * 64), 16, bo[i], 0, 0, 0);
    }
    for (int j = 0; j < nk; j += 2) {
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        tile_offs(j + 1, ao, bo);
        tn_step<TM, TN, NI>(sA1, sB1, sA0, sB0, ra, rb, ao, bo, (unsigned)(j + 1) * a_step, (unsigned)(j + 1) * b_step,
                            wave, live, acc, ra_off, rb_off);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 >= nk)
            break;
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        tile_offs(j + 2, ao, bo);
        tn_step<TM, TN, NI>(sA0, sB0, sA1, sB1, ra, rb, ao, bo, (unsigned)(j + 2) * a_step, (unsigned)(j + 2) * b_step,
                            wave, live, acc, ra_off, rb_off);
        __builtin_amdgcn_sched_barrier(0);
    }

    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    uint4 *stg = (wave < 2 ? sA0 : sA1) + (wave & 1) * 512;  // 32 rows x 64 fp32 per wave
    store_tile_staged_f32<bf16, TM, TN, WTM, WTN, ACT_NONE>(p, acc, ti.c_row0 + m0, rows_valid, n0, wm, wn, lane,
                                                            stg);
#endif
}

}  // namespace lmoe
