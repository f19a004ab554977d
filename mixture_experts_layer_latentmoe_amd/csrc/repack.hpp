// Weight repacking at create time: [in, out] row-major -> [out, in] (K
// contiguous), written into a destination with its own row stride so that
// several matrices can share one K-contiguous array:
//   dst[row(c) * dst_ld + r] = src[r * C + c]   for every batch b
// with row(c) = c, or for the two halves of a gated expert's first GEMM
// (glu_off 0: the gate matrix, 8: the value matrix) row(c) =
// 16 (c / 8) + c % 8 + glu_off: blocks of 8 gate rows alternate with the 8
// value rows of the same outputs.
#pragma once

#include "common.hpp"

namespace lmoe {

template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *__restrict__ src, int64_t R, int64_t C,
                                                        int64_t src_bstride, E *__restrict__ dst,
                                                        int64_t dst_ld, int64_t dst_bstride, int glu_off)
{
    __shared__ E tile[32][33];
    const int64_t b = blockIdx.z;
    const int64_t c0 = (int64_t)blockIdx.x * 32, r0 = (int64_t)blockIdx.y * 32;
    const E *s = src + b * src_bstride;
    E *d = dst + b * dst_bstride;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int i = ty; i < 32; i += 8) {
        const int64_t r = r0 + i, c = c0 + tx;
        if (r < R && c < C)
            tile[i][tx] = s[r * C + c];
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
        const int64_t c = c0 + i, r = r0 + tx;
        const int64_t row = glu_off < 0 ? c : 16 * (c >> 3) + (c & 7) + glu_off;
        if (r < R && c < C)
            d[row * dst_ld + r] = tile[tx][i];
    }
}

// Fragment-major copy of K-contiguous rows for the few-row GEMM kernel: the
// 32 bytes of k-step j of rows 32 b .. 32 b + 31 form one 1 KiB block,
//   dst[((n / 32) * S + j) * 1024 + (n % 32) * 32 + t] = src[n * row_bytes + 32 j + t],
// S = row_bytes / 32 steps per row; rows n >= N of the last block are zeros.
// One thread per 16-byte unit, in source order.
__global__ __launch_bounds__(256) void fragmajor_kernel(const char *__restrict__ src, int64_t N, int64_t row_bytes,
                                                        char *__restrict__ dst)
{
    const int64_t S = row_bytes / 32;
    const int64_t units = ((N + 31) / 32) * 32 * S * 2;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
        const int64_t n = u / (S * 2), rem = u - n * S * 2, j = rem >> 1, t = (rem & 1) * 16;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < N)
            v = *reinterpret_cast<const uint4 *>(src + n * row_bytes + 32 * j + t);
        *reinterpret_cast<uint4 *>(dst + ((n / 32) * S + j) * 1024 + (n % 32) * 32 + t) = v;
    }
}

}  // namespace lmoe
