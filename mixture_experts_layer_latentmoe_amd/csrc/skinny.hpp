// Dense GEMMs with few rows (decode batches): C = epilogue(A B) for
// M <= 32 * MT rows.  Such a product is bound by streaming B (the weights)
// from HBM once; the split of K over workgroups that the tiled kernel needs
// to occupy the chip writes partial sums as large as the weights and needs a
// second pass.  Here one workgroup owns COLS output columns and all of K:
// its NW waves each take a contiguous range of k-tiles, and the NW partial
// tiles are summed in LDS in wave order, which keeps the result independent
// of timing.  The epilogue is the tiled kernel's (store_out4).
//
// Operands of a wave, per k-tile (128 bytes of K: four k-steps of 32 bytes):
//  - A (activations, every row of M): copied by LDS DMA into the wave's own
//    two-stage LDS area, in the tiled kernel's swizzled layout (full 128-byte
//    lines per load), then read as MFMA fragments.  No other wave touches the
//    area, so a wave only waits for its own loads (no barrier in the loop).
//  - B (weights): straight into registers from the fragment-major copy
//    (fragmajor_kernel), where the 32 rows x 32 bytes of one k-step are one
//    1 KiB run; every B byte is used once, so LDS would buy nothing.
// A fragment is 16 bytes of row l % 32 at byte 16 (l / 32) of the k-step, the
// operand layout of the 32x32 MFMA (Mfma32).  B is passed as the MFMA's first
// operand, so lane l accumulates output row l % 32 and output columns
// 8 g + 4 (l / 32) + {0..3} of register group g.  COLS = 16 leaves B rows
// 16..31 out of range (zeros): half the bytes per workgroup, twice the
// workgroups.  STAGE only names the layer stage (one symbol per stage).
#pragma once

#include "gemm.hpp"

namespace lmoe {

// One pipeline step of a wave: k-tile tn of A by LDS DMA into the stage wr
// (lane l of DMA instruction i writes unit 64 i + l) and its four B
// fragments into bn (no valid tile: every load is out of range and reads
// nothing; the loads stay unconditional, so that the compiler's count of
// loads in flight stays exact); then, if MULT, the k-tile held in the stage
// rd times the fragments bc.  wr and rd are different LDS arrays.
template <typename E, int MT, int NIA, bool MULT>
__device__ __forceinline__ void skinny_step(uint4 *__restrict__ wr, const uint4 *__restrict__ rd, bool valid, int tn,
                                            __amdgpu_buffer_rsrc_t ra, const unsigned (&a_off)[NIA],
                                            __amdgpu_buffer_rsrc_t rb, unsigned b_off, uint4 (&bn)[4],
                                            const uint4 (&bc)[4], f32x16 (&acc)[MT], int r, int h)
{
#pragma unroll
    for (int i = 0; i < NIA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LMOE_LDS(wr + i * 64), 16,
                                                 valid ? a_off[i] + (unsigned)tn * 128u : kOOB, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
        bn[u] = buf_load16(rb, valid ? b_off + (unsigned)(4 * tn + u) * 1024u : kOOB);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the multiplies wait
    if constexpr (MULT) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = 2 * u + h;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int rr = i * 32 + r;
                acc[i] = Mfma32<E>::run(bc[u], rd[rr * 8 + (c ^ ((rr >> 1) & 7))], acc[i]);
            }
        }
    }
}

template <typename E, int MT, int NW, int COLS, int STAGE = 0>
__global__ __launch_bounds__(64 * NW) void skinny_gemm_kernel(const GemmParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(MT >= 1 && NW >= 1 && (COLS == 16 || COLS == 32), "skinny shape");
    constexpr int AU = MT * 32 * 8;  // 16-byte units of one A k-tile (MT * 32 rows x 128 bytes)
    constexpr int NIA = AU / 64;     // LDS-DMA instructions per A k-tile
    constexpr int ES = (int)sizeof(E);
    // two stages in two arrays, so that the compiler sees that reads of one
    // stage do not depend on the DMA in flight into the other
    __shared__ uint4 sA0[NW * AU], sA1[NW * AU];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * COLS;

    // this wave's k-tiles [t0, t1)
    const int nkt = p.K * ES / 128, nsteps = nkt * 4;
    const int per = (nkt + NW - 1) / NW;
    const int t0 = min(nkt, wave * per), t1 = min(nkt, t0 + per);

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.Bfrag, (int64_t)((p.N + 31) / 32) * nsteps * 1024);
    unsigned a_off[NIA];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int P = i * 64 + lane, r = P >> 3, c = (P & 7) ^ ((r >> 1) & 7);
        a_off[i] = r < p.M ? (unsigned)((int64_t)r * p.lda * ES) + c * 16 : kOOB;
    }
    const int r = lane & 31, h = lane >> 5, nb = n0 + r;
    const unsigned b_off =
        (r < COLS && nb < p.N) ? (unsigned)(((int64_t)(nb >> 5) * nsteps) * 1024 + (nb & 31) * 32) + 16u * h : kOOB;

    f32x16 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            acc[i][q] = 0.f;

    // two k-tiles in flight: while one stage is multiplied the other loads.
    // The compiler orders each stage's LDS reads after the DMA that filled it
    // (skinny_step's restrict-qualified stages tell it that the DMA in flight
    // into the other stage does not matter); the explicit LDS wait before a
    // step keeps a refill from overtaking the reads of the step before.
    uint4 b0[4], b1[4];
    uint4 *const w0 = sA0 + wave * AU, *const w1 = sA1 + wave * AU;
    skinny_step<E, MT, NIA, false>(w0, w1, t0 < t1, t0, ra, a_off, rb, b_off, b0, b1, acc, r, h);
    int t = t0;
    for (; t + 1 < t1; t += 2) {
        wait_vm_lgkm0<63>();
        skinny_step<E, MT, NIA, true>(w1, w0, true, t + 1, ra, a_off, rb, b_off, b1, b0, acc, r, h);
        wait_vm_lgkm0<63>();
        skinny_step<E, MT, NIA, true>(w0, w1, t + 2 < t1, t + 2, ra, a_off, rb, b_off, b0, b1, acc, r, h);
    }
    if (t < t1) {
        wait_vm_lgkm0<63>();
        skinny_step<E, MT, NIA, true>(w1, w0, false, 0, ra, a_off, rb, b_off, b1, b0, acc, r, h);
    }

    // partial tiles, lane-contiguous, each wave over its own stage-0 area
    // (which only it has used), then fixed-order sums over the waves
    static_assert(sizeof(sA0) >= (size_t)NW * MT * 16 * 64 * 4, "reduction area");
    float *red = reinterpret_cast<float *>(sA0);  // [NW][MT][16][64]
    wait_vm_lgkm0<0>();
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            red[((wave * MT + i) * 16 + q) * 64 + lane] = acc[i][q];
    __syncthreads();

    // output groups of four columns: (m-tile i, register group g, lane ln)
    for (int t = tid; t < MT * 4 * 64; t += 64 * NW) {
        const int i = t >> 8, g = (t >> 6) & 3, ln = t & 63;
        const int row = i * 32 + (ln & 31), col = n0 + 8 * g + 4 * (ln >> 5);
        if (row >= p.M || col >= p.N || col - n0 >= COLS)
            continue;
        // gated pairs: n0 and glu_from are multiples of 16, so gate groups
        // are the even g and their values the next register group
        const bool glu = col >= p.glu_from;
        if (glu && (g & 1))
            continue;
        float v[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < NW; ++w)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                v[c] += red[((w * MT + i) * 16 + 4 * g + c) * 64 + ln];
                if (glu)
                    u[c] += red[((w * MT + i) * 16 + 4 * g + 4 + c) * 64 + ln];
            }
        if (glu) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                v[c] = glu_value(v[c], u[c]);
            store4(static_cast<E *>(p.C) + row * p.ldc + glu_out_col(p, col), v[0], v[1], v[2], v[3]);
            continue;
        }
        store_out4<E>(p, row, col, v);
    }
#endif
}

constexpr int kFewRowMaxSplits = 8;  // p.splitk of fewrow_split_kernel
constexpr int kCoherentLoad = 16;    // cache policy of a buffer load: sc1 (device-coherent)

// Few-row dense GEMMs with K split over workgroups.  The kernel above gives a
// workgroup all of K, so every workgroup copies all of A (the 64 activation
// rows) from L2: with 16 columns per workgroup that is 4x the weight bytes
// it streams, and at N = 2048 only 128 workgroups run.  Here a workgroup owns
// 32 NB columns and one of S contiguous k-tile ranges (p.splitk), so A
// costs 64 / (32 NB) of the weight bytes and ceil(N / 32 NB) * S workgroups
// fill the chip.  Each of its NW waves takes a sub-range of at most 4 / MT
// k-tiles and issues every load of it at once -- A by LDS DMA into its own
// area, B into registers -- so a wave waits for memory once, not once per
// k-tile.  The wave tiles are summed in LDS in wave order; a workgroup then
// stores its fp32 tile (lane-contiguous) to p.partial, and the last of the S
// workgroups of a column group to arrive (a counter per group in p.counters,
// which that workgroup sets back to zero) sums the S tiles in split order
// and applies the epilogue.  The result does not depend on which workgroup
// arrives last.  S = 1: no partials, no counter.  S <= kFewRowMaxSplits.
template <typename E, int MT, int NB, int NW, int STAGE = 0>
__global__ __launch_bounds__(64 * NW) void fewrow_split_kernel(const GemmParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert((MT == 1 || MT == 2) && (NB == 1 || NB == 2) && NW >= 1 && NW <= 16, "few-row shape");
    constexpr int SMAX = kFewRowMaxSplits;
    constexpr int KTM = 4 / MT;                 // k-tiles of a wave per round
    constexpr int AU = MT * 32 * 8;             // 16-byte units of one A k-tile
    constexpr int NIA = AU / 64;                // LDS-DMA instructions per A k-tile
    constexpr int ES = (int)sizeof(E);
    constexpr int TV = MT * NB * 16 * 64;       // floats of a workgroup tile (lane-contiguous)
    constexpr int A_UNITS = NW * KTM * AU;      // wave areas of A
    constexpr int R_UNITS = (NW + 1) * TV / 4;  // wave tiles + the summed tile
    static_assert(TV % (64 * NW) == 0, "tile split over the threads");
    __shared__ uint4 lds[A_UNITS > R_UNITS ? A_UNITS : R_UNITS];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = p.splitk;
    const int cg = blockIdx.x / S, split = blockIdx.x - cg * S;
    const int n0 = cg * 32 * NB;

    // k-tiles of this split [k0, k1), of this wave [t0, t1)
    const int nkt = p.K * ES / 128, nsteps = nkt * 4;
    const int per = (nkt + S - 1) / S;
    const int k0 = min(nkt, split * per), k1 = min(nkt, k0 + per);
    const int wper = (k1 - k0 + NW - 1) / NW;
    const int t0 = min(k1, k0 + wave * wper), t1 = min(k1, t0 + wper);

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
    const int nblk = (p.N + 31) / 32;  // 32-row blocks of the fragment-major copy
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.Bfrag, (int64_t)nblk * nsteps * 1024);
    unsigned a_off[NIA];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int P = i * 64 + lane, r = P >> 3, c = (P & 7) ^ ((r >> 1) & 7);
        a_off[i] = r < p.M ? (unsigned)((int64_t)r * p.lda * ES) + c * 16 : kOOB;
    }
    const int r = lane & 31, h = lane >> 5;
    unsigned b_off[NB];
    bool b_ok[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int blk = cg * NB + nb;
        b_ok[nb] = blk < nblk;
        b_off[nb] = (unsigned)((int64_t)blk * nsteps * 1024) + r * 32 + 16 * h;
    }

    f32x16 acc[MT][NB];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc[i][nb][q] = 0.f;

    uint4 *const wa = lds + wave * KTM * AU;
    for (int base = t0; base < t1; base += KTM) {
        wait_vm_lgkm0<0>();  // the previous round's LDS reads are done before its area is refilled
        uint4 b[KTM][4][NB];
#pragma unroll
        for (int kt = 0; kt < KTM; ++kt) {
            const bool valid = base + kt < t1;
            const unsigned tn = (unsigned)(base + kt);
#pragma unroll
            for (int i = 0; i < NIA; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LMOE_LDS(wa + kt * AU + i * 64), 16,
                                                         valid ? a_off[i] + tn * 128u : kOOB, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    b[kt][u][nb] = buf_load16(rb, (valid && b_ok[nb]) ? b_off[nb] + (4 * tn + u) * 1024u : kOOB);
        }
        wait_vm_lgkm0<0>();
#pragma unroll
        for (int kt = 0; kt < KTM; ++kt) {
            if (base + kt >= t1)
                break;
            const uint4 *rd = wa + kt * AU;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = 2 * u + h;
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int rr = i * 32 + r;
                    const uint4 af = rd[rr * 8 + (c ^ ((rr >> 1) & 7))];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[i][nb] = Mfma32<E>::run(b[kt][u][nb], af, acc[i][nb]);
                }
            }
        }
    }

    // wave tiles -> LDS, summed in wave order
    __syncthreads();  // every wave is done with its A area
    float *red = reinterpret_cast<float *>(lds);  // [NW][MT][NB][16][64]
    float *fin = red + NW * TV;                   // [MT][NB][16][64]
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                red[wave * TV + ((i * NB + nb) * 16 + q) * 64 + lane] = acc[i][nb][q];
    __syncthreads();
    constexpr int PT = TV / (64 * NW);  // values per thread
    float v[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = tid + j * 64 * NW;
        float sum = 0.f;
        for (int w = 0; w < NW; ++w)
            sum += red[w * TV + t];
        v[j] = sum;
    }

    if (S > 1) {
        // The tiles cross workgroups (and XCDs, each with its own L2) through
        // device-coherent accesses -- stores written through to the device
        // level and loads that do not hit a stale cached copy (the sc1 policy
        // of agent-scope atomics) -- ordered by waiting for the stores to
        // complete before the count.  A device-scope fence would do it too,
        // but it writes back the whole L2 of the XCD: measured, every split
        // then added ~35 us.
        float *mine = p.partial + ((int64_t)cg * S + split) * TV;
#pragma unroll
        for (int j = 0; j < PT; ++j)
            __hip_atomic_store(mine + tid + j * 64 * NW, v[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_vm_lgkm0<0>();  // this thread's stores are complete
        __syncthreads();     // ... and every thread's
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(p.counters + cg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = old == S - 1;
            if (old == S - 1)
                __hip_atomic_store(p.counters + cg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!s_last)
            return;
        // every load issued before the first add: splits past S read as zeros
        // (out of the buffer's range), and a sum that starts at +0 is unchanged
        // by adding +0
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.partial + (int64_t)cg * S * TV, (int64_t)S * TV * 4);
        float x[SMAX][PT];
#pragma unroll
        for (int sp = 0; sp < SMAX; ++sp)
#pragma unroll
            for (int j = 0; j < PT; ++j)
                x[sp][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                         rp, (unsigned)((sp * TV + tid + j * 64 * NW) * 4), 0,
                                                         kCoherentLoad));
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            float sum = 0.f;
#pragma unroll
            for (int sp = 0; sp < SMAX; ++sp)
                sum += x[sp][j];
            v[j] = sum;
        }
    }
#pragma unroll
    for (int j = 0; j < PT; ++j)
        fin[tid + j * 64 * NW] = v[j];
    __syncthreads();

    // output groups of four columns: (m-tile i, column block nb, register group g, lane ln)
    for (int t = tid; t < MT * NB * 4 * 64; t += 64 * NW) {
        const int i = t / (NB * 256), nb = (t >> 8) % NB, g = (t >> 6) & 3, ln = t & 63;
        const int row = i * 32 + (ln & 31), col = n0 + 32 * nb + 8 * g + 4 * (ln >> 5);
        if (row >= p.M || col >= p.N)
            continue;
        const float *f = fin + (i * NB + nb) * 16 * 64;
        // gated pairs: n0 and glu_from are multiples of 16, so gate groups
        // are the even g and their values the next register group
        const bool glu = col >= p.glu_from;
        if (glu && (g & 1))
            continue;
        float o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            o[c] = f[(4 * g + c) * 64 + ln];
        if (glu) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o[c] = glu_value(o[c], f[(4 * g + 4 + c) * 64 + ln]);
            store4(static_cast<E *>(p.C) + row * p.ldc + glu_out_col(p, col), o[0], o[1], o[2], o[3]);
            continue;
        }
        store_out4<E>(p, row, col, o);
    }
#endif
}

}  // namespace lmoe
