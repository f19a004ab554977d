// Weight repacking at create time: [in, out] row-major -> [out, in] (K
// contiguous), written into a destination with its own row stride so that
// several matrices can share one K-contiguous array:
//   dst[c * dst_ld + r] = src[r * C + c]   for every batch b
#pragma once

#include "common.hpp"

namespace lmoe {

template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *__restrict__ src, int64_t R, int64_t C,
                                                        int64_t src_bstride, E *__restrict__ dst,
                                                        int64_t dst_ld, int64_t dst_bstride)
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
        if (r < R && c < C)
            d[c * dst_ld + r] = tile[tx][i];
    }
}

}  // namespace lmoe
