// Fused routed-expert MLP: Y[rows_e] = act(z[perm[rows_e]] W1_e) W2_e, with the
// hidden activations kept on chip.
//
// Page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through
// Equations, Architecture, Code and ...": Figure 9 and the LatentMoE code
// block -- a latent expert is two matrices around a squared ReLU, run on the
// l-wide latent rows of the tokens routed to it.  The unfused form writes the
// hidden layer H [rows, m] to HBM and reads it back (2 x 277 MB at the
// README layer's widths); here it never leaves the compute unit.
//
// One workgroup (8 waves) owns BM dispatch rows of one expert (one entry of
// the device tile table) and the whole output row block Y [BM, l], held in
// the waves' accumulators.  It walks m in chunks of MC columns:
//   phase 1  H_c [BM, MC] = act(Z [BM, l] W1 [:, chunk])   (K = l, 64-wide
//            k-tiles of Z and W1 by LDS DMA)
//            -> activation in registers, rounded to bf16, into an LDS buffer
//            laid out like an A operand tile
//   phase 2  Y [BM, l] += H_c [BM, MC] W2 [chunk, :]      (K = MC, KS2 rows
//            of W2 per step by LDS DMA, H_c fragments from LDS)
// Every step (a phase-1 k-tile or a phase-2 slice) moves through one ring of
// NS LDS slots: one barrier per step, the DMA of step j + NS - 1 in flight
// while step j multiplies, exactly as in the tiled GEMM (gemm.hpp).  Each
// step issues the same number NI of DMA instructions, which keeps the wait
// counts constant: the shorter kind of step adds out-of-range loads (they
// write zeros) into the part of its slot that it does not use.
// Gated experts (GLU): the W1 bank interleaves gate and value columns by 8
// (repack), a chunk holds 2 MC B columns, and phase 1 forms silu(gate) * value.
//
// Layouts: Z rows are gathered through perm (dispatch row -> token) straight
// into LDS; W1 per expert is k-tile-major [l/64][nb1][64], W2 [m/64][l][64].
// A W2 slice of KS2 k-values is KS2 * 2 bytes of each of the l rows of a
// k-tile: in LDS, CH2 = KS2 / 8 chunks of 16 bytes per row, chunk c of row r
// at c ^ ((r / (16 / CH2)) % CH2), which spreads 16 consecutive rows over the
// 16 bank groups for the fragment reads (the A-tile rule for CH2 = 8).
#pragma once

#include "gemm.hpp"

namespace lmoe {

struct MlpParams {
    const void *Z;     // [T, ldz] E: z in the first l columns
    int64_t ldz;       // elements
    int64_t z_bytes;   // bytes of the Z buffer (range of its loads)
    const int *gather; // dispatch row -> token
    const void *W1;    // per expert [l / 64][nb1][64]
    const void *W2;    // per expert [m / 64][l][64]
    void *Y;           // [P, l] E
    int l, m, nb1;
    const int4 *tile_info;
    const int *n_mtiles, *offsets;
};

template <int CH2> __device__ __forceinline__ int swz2(int r) { return (r / (16 / CH2)) & (CH2 - 1); }

// Phase 1 epilogue: the wave's H_c accumulators -> act -> bf16 -> the H
// buffer ([MC / 64][BM rows][8 chunks], chunk c of row r at c ^ ((r >> 1) & 7)).
// A lane holds row
// wm WTM + 32 i + lane % 32 and B columns base + 8 g + 4 (lane / 32) + {0..3}
// of register group g (base = wn WTN + 32 j); gated, groups 0 and 2 are gates
// whose values sit in groups 1 and 3, output column base / 2 + 4 g + 4 (lane / 32).
template <int BM, int TM, int TN, int WTM, int WTN, bool GLU>
__device__ __forceinline__ void mlp_store_h(f32x16 (&acc)[TM][TN], uint4 *hbuf, int wm, int wn, int lane, bool live)
{
    const int lr = lane & 31, lc = lane >> 5;
    char *hb = reinterpret_cast<char *>(hbuf);
    auto put4 = [&](int R, int C0, float a, float b, float c, float d) {
        const int kt = C0 >> 6, ch = (C0 & 63) >> 3, sub = C0 & 7;
        bf16 v[4] = {from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c), from_f32<bf16>(d)};
        *reinterpret_cast<uint2 *>(hb + ((kt * BM + R) * 8 + (ch ^ ((R >> 1) & 7))) * 16 + sub * 2) =
            *reinterpret_cast<const uint2 *>(v);
    };
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int R = wm * WTM + i * 32 + lr;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int base = wn * WTN + j * 32;
            if constexpr (!GLU) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float t = live ? fmaxf(acc[i][j][4 * g + r], 0.f) : 0.f;
                        v[r] = t * t;
                    }
                    put4(R, base + 8 * g + 4 * lc, v[0], v[1], v[2], v[3]);
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; g += 2) {
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = live ? glu_value(acc[i][j][4 * g + r], acc[i][j][4 * g + 4 + r]) : 0.f;
                    put4(R, base / 2 + 4 * g + 4 * lc, v[0], v[1], v[2], v[3]);
                }
            }
        }
    }
}

// A lane's LDS byte offsets of its MFMA fragments, computed once per kernel.
// Every fragment read of both phases is (row of the lane) x 128 (64 for the
// W2 slices) + (its swizzled 16-byte chunk) + a compile-time part: the row
// swizzle of a wave's rows depends only on lane % 32 (wave tiles start at
// multiples of 16 rows), and a k16-step's chunk pair 2 m + lane / 32 takes
// four values, m = 0..3.  With these offsets the compile-time part (fragment
// row block, H buffer k-tile) folds into the reads' immediate offsets: the
// loop holds 44 address registers instead of the 72 the compiler kept when
// it formed each step's addresses itself (256 VGPRs, one fragment register
// pair in rotation); 245 VGPRs now, the same reads and MFMAs, bit-identical
// sums.  Measured at readme_acc: 421-424 -> 407-417 us.
struct MlpOffs {
    unsigned p1a[4], p1b[4];  // phase 1: Z rows, W1 columns; k16-step m
    unsigned p2a[4];          // phase 2: H rows; chunk pair m
    unsigned p2b[2];          // phase 2: W2 slice rows; k16-step s of the slice
};

template <int WTM1, int WTN1, int WTM2, int WTN2, int CH2>
__device__ __forceinline__ MlpOffs mlp_offsets(int lane, int wm1, int wn1, int wm2, int wn2)
{
    static_assert(WTM1 % 16 == 0 && WTN1 % 16 == 0 && WTM2 % 16 == 0 && WTN2 % 16 == 0 && CH2 == 4,
                  "row swizzles of a wave's rows depend on the lane only");
    const int L = lane & 31, h = lane >> 5, sw = (L >> 1) & 7, swb = (L >> 2) & 3;
    MlpOffs o;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const unsigned x = (unsigned)(((2 * m + h) ^ sw) * 16);
        o.p1a[m] = (unsigned)(wm1 * WTM1 + L) * 128u + x;
        o.p1b[m] = (unsigned)(wn1 * WTN1 + L) * 128u + x;
        o.p2a[m] = (unsigned)(wm2 * WTM2 + L) * 128u + x;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
        o.p2b[q] = (unsigned)(wn2 * WTN2 + L) * 64u + (unsigned)(((2 * q + h) ^ swb) * 16);
    return o;
}

// Phase 1 multiply of one step: one 64-wide k-tile of Z (a) and W1 (b), both
// in the current slot, fragments at the lane's precomputed offsets.  The
// operands are restrict-qualified: the compiler then tells these LDS reads
// apart from the DMA into the next slot that is still in flight, and does not
// wait for it (same rule as gemm.hpp's dma_mma).
template <int TM, int TN>
__device__ __forceinline__ void mlp_mma1_off(f32x16 (&acc)[TM][TN], const uint4 *__restrict__ a,
                                             const uint4 *__restrict__ b, const MlpOffs &o)
{
    const char *ac = reinterpret_cast<const char *>(a), *bc = reinterpret_cast<const char *>(b);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint4 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            af[i] = *reinterpret_cast<const uint4 *>(ac + o.p1a[s] + i * 32 * 128);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bfr[j] = *reinterpret_cast<const uint4 *>(bc + o.p1b[s] + j * 32 * 128);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = Mfma32<bf16>::run(bfr[j], af[i], acc[i][j]);
    }
}

// Phase 2 multiply of one step: k-values K0 .. K0 + 8 CH2 - 1 of the chunk,
// A fragments from the H buffer, B fragments (W2 slice) from the slot.
template <int BM, int TM, int TN, int CH2, int K0>
__device__ __forceinline__ void mlp_mma2_off(f32x16 (&acc)[TM][TN], const uint4 *hbuf, const uint4 *__restrict__ b,
                                             const MlpOffs &o)
{
    const char *hc = reinterpret_cast<const char *>(hbuf), *bc = reinterpret_cast<const char *>(b);
#pragma unroll
    for (int s = 0; s < CH2 / 2; ++s) {
        const int kk = K0 + 16 * s, kt = kk >> 6, m = (kk & 63) >> 4;
        uint4 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            af[i] = *reinterpret_cast<const uint4 *>(hc + o.p2a[m] + (kt * BM + i * 32) * 128);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bfr[j] = *reinterpret_cast<const uint4 *>(bc + o.p2b[s] + j * 32 * 64);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = Mfma32<bf16>::run(bfr[j], af[i], acc[i][j]);
    }
}

template <int BM, int LW, int MC, int KS2, int NS, int WM1, int WN1, int WM2, int WN2, bool GLU>
struct MlpShape {
    static constexpr int NW = 8, NT = 512;
    static constexpr int NB1 = GLU ? 2 * MC : MC;  // W1 B columns per chunk
    static constexpr int WTM1 = BM / WM1, WTN1 = NB1 / WN1, TM1 = WTM1 / 32, TN1 = WTN1 / 32;
    static constexpr int WTM2 = BM / WM2, WTN2 = LW / WN2, TM2 = WTM2 / 32, TN2 = WTN2 / 32;
    static constexpr int CH2 = KS2 / 8;
    static constexpr int NIA1 = BM * 8 / NT, NIB1 = NB1 * 8 / NT, NIB2 = LW * CH2 / NT;
    static constexpr int NI = (NIA1 + NIB1 > NIB2) ? NIA1 + NIB1 : NIB2;
    static constexpr int S1 = LW / 64, S2 = MC / KS2, SPC = S1 + S2;
    static constexpr int SLOT1 = (BM + NB1) * 8, SLOT2 = LW * CH2;
    static constexpr int SLOT = SLOT1 > SLOT2 ? SLOT1 : SLOT2;  // uint4 units per ring slot
    static constexpr int HBUF = BM * MC / 8;                     // uint4 units of the H buffer
    static constexpr size_t lds_bytes() { return (size_t)(NS * SLOT + HBUF) * 16; }
    // the padding loads of the shorter kind of step land past its tiles
    static_assert(SLOT1 + (NI - NIA1 - NIB1) * NT <= SLOT && SLOT2 + (NI - NIB2) * NT <= SLOT, "padding room");
    static_assert(WM1 * WN1 == NW && WM2 * WN2 == NW, "8 waves");
    static_assert(TM1 >= 1 && TN1 >= 1 && TM2 >= 1 && TN2 >= 1, "wave tiles");
    static_assert(NIA1 >= 1 && NIB1 >= 1 && NIB2 >= 1, "DMA per thread");
    static_assert(NIA1 * NT == BM * 8 && NIB1 * NT == NB1 * 8 && NIB2 * NT == LW * CH2, "DMA covers the tiles");
    static_assert(MC % 64 == 0 && MC % KS2 == 0 && (KS2 == 16 || KS2 == 32 || KS2 == 64), "chunk and slice");
    static_assert((NS == 3 || NS == 4) && SPC % NS == 0 && S1 >= NS - 1, "whole turns of the ring per chunk");
    static_assert(!GLU || WTN1 % 32 == 0, "gated pairs inside one MFMA tile");
};

// DMA of the step at position POS of a chunk (phase by POS) for chunk c into
// slot dst; issue false: every load out of range (no next chunk).  The part
// of a load's source offset that is the same for every lane (the step's k
// position, the chunk, the instruction's row block) goes in the scalar offset,
// which is also where a load is sent out of range (a lane's offset register
// then stays the same for the whole kernel, so no LDS read result is ever
// assigned to it, which would make the compiler wait for the DMA);
// a lane's W1 and W2 units differ between instructions by whole row blocks
// (64 rows of W1, 512 / CH2 rows of W2, the swizzle unchanged), so one
// register each holds a lane's part.
template <class SH, int BM, int LW, int MC, int KS2, int POS>
__device__ __forceinline__ void mlp_dma(uint4 *__restrict__ dst, int c, bool issue, int nb1,
                                        __amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rw1,
                                        __amdgpu_buffer_rsrc_t rw2, const unsigned (&a_off)[SH::NIA1],
                                        unsigned b1_off, unsigned b2_off, int wave)
{
    constexpr int NW = SH::NW;
    if constexpr (POS < SH::S1) {
        const unsigned kz = (unsigned)POS * 128u, kw = (unsigned)(POS * nb1 + c * SH::NB1) * 128u;
#pragma unroll
        for (int i = 0; i < SH::NIA1; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, LMOE_LDS(dst + (i * NW + wave) * 64), 16, a_off[i],
                                                     issue ? kz : kOOB, 0, 0);
#pragma unroll
        for (int i = 0; i < SH::NIB1; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw1, LMOE_LDS(dst + BM * 8 + (i * NW + wave) * 64), 16, b1_off,
                                                     issue ? kw + (unsigned)i * (64u * 128u) : kOOB, 0, 0);
#pragma unroll
        for (int i = 0; i < SH::NI - SH::NIA1 - SH::NIB1; ++i)  // padding: zeros past the phase-1 tiles
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw1, LMOE_LDS(dst + SH::SLOT1 + (i * NW + wave) * 64), 16, kOOB, 0,
                                                     0, 0);
    } else {
        const int k0 = c * MC + (POS - SH::S1) * KS2;
        const unsigned koff = (unsigned)((k0 >> 6) * LW) * 128u + (unsigned)(k0 & 63) * 2u;
#pragma unroll
        for (int i = 0; i < SH::NIB2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw2, LMOE_LDS(dst + (i * NW + wave) * 64), 16, b2_off,
                                                     issue ? koff + (unsigned)i * (unsigned)(SH::NT / SH::CH2) * 128u
                                                           : kOOB,
                                                     0, 0);
#pragma unroll
        for (int i = 0; i < SH::NI - SH::NIB2; ++i)  // padding: zeros past the W2 slice
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw2, LMOE_LDS(dst + SH::SLOT2 + (i * NW + wave) * 64), 16, kOOB, 0,
                                                     0, 0);
    }
}

// The unrolled steps of one chunk.  Step POS multiplies from slot POS % NS
// while the DMA of step POS + NS - 1 (this chunk, or the next chunk's first
// NS - 1) fills slot (POS + NS - 1) % NS.  One barrier per step: it waits
// until the slot of step POS has landed for every wave (the loads of the
// NS - 2 steps after it may stay in flight) and until every wave is done with
// the slot about to be refilled.
template <class SH, int BM, int LW, int MC, int KS2, int NS, bool GLU>
struct MlpChunk {
    template <int Q>
    static __device__ __forceinline__ uint4 *slot(uint4 *s0, uint4 *s1, uint4 *s2, uint4 *s3)
    {
        return (Q % NS == 0) ? s0 : (Q % NS == 1) ? s1 : (Q % NS == 2) ? s2 : s3;
    }
    template <int POS>
    static __device__ __forceinline__ void run(uint4 *__restrict__ s0, uint4 *__restrict__ s1, uint4 *__restrict__ s2,
                                               uint4 *__restrict__ s3, uint4 *hbuf, int c, bool more, int nb1,
                                               __amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rw1,
                                               __amdgpu_buffer_rsrc_t rw2, const unsigned (&a_off)[SH::NIA1],
                                               unsigned b1_off, unsigned b2_off, int wave, int lane,
                                               f32x16 (&accH)[SH::TM1][SH::TN1], f32x16 (&accY)[SH::TM2][SH::TN2],
                                               int wm1, int wn1, int wm2, int wn2, bool live2, const MlpOffs &of)
    {
        constexpr int AHEAD = POS + NS - 1;
        constexpr int NXT = AHEAD < SH::SPC ? AHEAD : AHEAD - SH::SPC;
        uint4 *nxt = slot<NXT>(s0, s1, s2, s3);
        const uint4 *cur = slot<POS>(s0, s1, s2, s3);
        wait_vm_lgkm0<(NS - 2) * SH::NI>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (AHEAD < SH::SPC)
            mlp_dma<SH, BM, LW, MC, KS2, NXT>(nxt, c, true, nb1, rz, rw1, rw2, a_off, b1_off, b2_off, wave);
        else
            mlp_dma<SH, BM, LW, MC, KS2, NXT>(nxt, c + 1, more, nb1, rz, rw1, rw2, a_off, b1_off, b2_off, wave);
        if constexpr (POS < SH::S1) {
            if constexpr (POS == 0) {  // a new chunk (zeroed here, the accumulators are dead in phase 2)
#pragma unroll
                for (int i = 0; i < SH::TM1; ++i)
#pragma unroll
                    for (int jj = 0; jj < SH::TN1; ++jj)
#pragma unroll
                        for (int q = 0; q < 16; ++q)
                            accH[i][jj][q] = 0.f;
            }
            // no skip for padding rows here: with one, the compiler also waited
            // for the DMA in flight before this step's LDS reads
            mlp_mma1_off<SH::TM1, SH::TN1>(accH, cur, cur + BM * 8, of);
            if constexpr (POS == SH::S1 - 1)
                mlp_store_h<BM, SH::TM1, SH::TN1, SH::WTM1, SH::WTN1, GLU>(accH, hbuf, wm1, wn1, lane, true);
        } else {
            if (live2)
                mlp_mma2_off<BM, SH::TM2, SH::TN2, SH::CH2, (POS - SH::S1) * KS2>(accY, hbuf, cur, of);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (POS + 1 < SH::SPC)
            run<POS + 1>(s0, s1, s2, s3, hbuf, c, more, nb1, rz, rw1, rw2, a_off, b1_off, b2_off, wave, lane, accH,
                         accY, wm1, wn1, wm2, wn2, live2, of);
    }
};

// STAGE only names the layer stage (one kernel symbol per stage).
template <int BM, int LW, int MC, int KS2, int NS, int WM1, int WN1, int WM2, int WN2, bool GLU, int STAGE>
__global__ __launch_bounds__(512, 1) void expert_mlp_kernel(const MlpParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using SH = MlpShape<BM, LW, MC, KS2, NS, WM1, WN1, WM2, WN2, GLU>;
    constexpr int NW = SH::NW;
    __shared__ uint4 slot0[SH::SLOT], slot1[SH::SLOT], slot2[SH::SLOT], slot3[NS > 3 ? SH::SLOT : 1];
    __shared__ uint4 hbuf[SH::HBUF];

    const int t = xcd_logical_tile(blockIdx.x, *p.n_mtiles);
    if (t < 0)
        return;
    const int4 rec = p.tile_info[t];
    const int expert = rec.x;
    const int rows_valid = min(BM, rec.z);
    const int64_t row_base = rec.y;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm1 = wave / WN1, wn1 = wave - wm1 * WN1;
    const int wm2 = wave / WN2, wn2 = wave - wm2 * WN2;

    const __amdgpu_buffer_rsrc_t rz = make_rsrc(p.Z, p.z_bytes);
    const int64_t w1_bytes = (int64_t)p.l * p.nb1 * 2, w2_bytes = (int64_t)p.m * p.l * 2;
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(static_cast<const char *>(p.W1) + expert * w1_bytes, w1_bytes);
    const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(static_cast<const char *>(p.W2) + expert * w2_bytes, w2_bytes);
    unsigned a_off[SH::NIA1];
#pragma unroll
    for (int i = 0; i < SH::NIA1; ++i) {
        const int P = (i * NW + wave) * 64 + lane, r = P >> 3, c = (P & 7) ^ ((r >> 1) & 7);
        a_off[i] = kOOB;
        if (r < rows_valid)
            a_off[i] = (unsigned)((int64_t)p.gather[row_base + r] * p.ldz * 2) + c * 16;
    }
    // instruction i of a lane loads row r + 64 i of W1 and row r + i NT / CH2 of
    // W2 at the same chunk position (the swizzles repeat every 16 rows)
    static_assert((SH::NT / SH::CH2) % 16 == 0, "W2 row blocks keep the swizzle");
    unsigned b1_off, b2_off;
    {
        const int P = wave * 64 + lane, r = P >> 3, c = (P & 7) ^ ((r >> 1) & 7);
        b1_off = (unsigned)r * 128u + c * 16;
        const int r2 = P / SH::CH2, c2 = (P % SH::CH2) ^ swz2<SH::CH2>(r2);
        b2_off = (unsigned)r2 * 128u + c2 * 16;
    }

    f32x16 accH[SH::TM1][SH::TN1], accY[SH::TM2][SH::TN2];  // accH is zeroed at each chunk's first step
#pragma unroll
    for (int i = 0; i < SH::TM2; ++i)
#pragma unroll
        for (int j = 0; j < SH::TN2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                accY[i][j][q] = 0.f;

    // waves whose rows are all padding skip their phase-2 multiplies
    const bool live2 = wm2 * SH::WTM2 < rows_valid;
    const int nchunks = p.m / MC;
    const MlpOffs of = mlp_offsets<SH::WTM1, SH::WTN1, SH::WTM2, SH::WTN2, SH::CH2>(lane, wm1, wn1, wm2, wn2);
    mlp_dma<SH, BM, LW, MC, KS2, 0>(slot0, 0, true, p.nb1, rz, rw1, rw2, a_off, b1_off, b2_off, wave);
    mlp_dma<SH, BM, LW, MC, KS2, 1>(slot1, 0, true, p.nb1, rz, rw1, rw2, a_off, b1_off, b2_off, wave);
    if constexpr (NS > 3)
        mlp_dma<SH, BM, LW, MC, KS2, 2>(slot2, 0, true, p.nb1, rz, rw1, rw2, a_off, b1_off, b2_off, wave);
    for (int c = 0; c < nchunks; ++c)
        MlpChunk<SH, BM, LW, MC, KS2, NS, GLU>::template run<0>(slot0, slot1, slot2, slot3, hbuf, c, c + 1 < nchunks,
                                                                p.nb1, rz, rw1, rw2, a_off, b1_off, b2_off, wave,
                                                                lane, accH, accY, wm1, wn1, wm2, wn2, live2, of);

    // Y [rows, l] through LDS: every wave is done with the ring (no load in flight)
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    constexpr int WAVE_U = 32 * SH::WTN2 * 2 / 16;  // 16-byte units of a wave's staging area
    constexpr int PER = SH::SLOT / WAVE_U;
    static_assert(PER >= 1 && NW <= 3 * PER, "staging areas fit in three slots");
    uint4 *stg = (wave < PER ? slot0 : wave < 2 * PER ? slot1 : slot2) + (wave % PER) * WAVE_U;
    GemmParams gp{};
    gp.C = p.Y;
    gp.ldc = p.l;
    gp.N = p.l;
    gp.c_split = 0;
    gp.relu2_from = 1 << 30;
    gp.glu_from = 1 << 30;
    if (live2)
        store_tile_staged<bf16, SH::TM2, SH::TN2, SH::WTM2, SH::WTN2>(gp, accY, row_base, rows_valid, 0, wm2, wn2, lane,
                                                                      stg);
#endif
}

}  // namespace lmoe
