// Weighted combine in the latent width l:
//   u[t] = sum_{k < K'} gate[t, k] * Y[pos[t, k]]     (fp32, slot order)
// Page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through
// Equations, Architecture, Code and ...": Figure 8 (the selected experts'
// weighted outputs are summed at the latent width before W_up) and the
// LatentMoE code block.  Gather form: one wave per token reads its K' rows
// of Y (16-byte chunks, coalesced along the row) and writes u once; no
// atomics, so the sum order is fixed.
#pragma once

#include "common.hpp"

namespace lmoe {

// BATCH (decode batches): a lane issues its chunk's loads of 8 slots at a
// time before summing them, one memory round trip for K' <= 8 instead of the
// compiler's batches of 4; same sum order.
template <typename E, bool BATCH = false>
__global__ __launch_bounds__(256) void combine_kernel(const E *__restrict__ Y, const int *__restrict__ pos,
                                                      const float *__restrict__ gate, int T, int K, int l,
                                                      E *__restrict__ out, int64_t ldo)
{
    constexpr int VEC = 16 / (int)sizeof(E);
    __shared__ int s_pos[4][64];
    __shared__ float s_gate[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    const bool live = t < T;
    if (live && lane < K) {
        s_pos[wave][lane] = pos[(int64_t)t * K + lane];
        s_gate[wave][lane] = gate[(int64_t)t * K + lane];
    }
    __syncthreads();
    if (!live)
        return;
    const int nchunk = l / VEC;
    for (int c = lane; c < nchunk; c += 64) {
        float acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            acc[v] = 0.f;
        if constexpr (BATCH) {
            for (int k0 = 0; k0 < K; k0 += 8) {
                uint4 raw[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    raw[j] = (k0 + j < K)
                                 ? *reinterpret_cast<const uint4 *>(Y + (int64_t)s_pos[wave][k0 + j] * l + c * VEC)
                                 : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (k0 + j >= K)
                        break;
                    const float g = s_gate[wave][k0 + j];
                    const E *vals = reinterpret_cast<const E *>(&raw[j]);
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        acc[v] += g * to_f32(vals[v]);
                }
            }
        } else {
#pragma unroll 4
            for (int k = 0; k < K; ++k) {
                const int p = s_pos[wave][k];
                const float g = s_gate[wave][k];
                const uint4 raw = *reinterpret_cast<const uint4 *>(Y + (int64_t)p * l + c * VEC);
                const E *vals = reinterpret_cast<const E *>(&raw);
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    acc[v] += g * to_f32(vals[v]);
            }
        }
        E o[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            o[v] = from_f32<E>(acc[v]);
        *reinterpret_cast<uint4 *>(out + (int64_t)t * ldo + c * VEC) = *reinterpret_cast<const uint4 *>(o);
    }
}

}  // namespace lmoe
