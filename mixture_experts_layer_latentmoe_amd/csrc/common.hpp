// Shared device helpers for the LatentMoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace lmoe {

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename E> __device__ __forceinline__ E from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bf16 conversion rounds to nearest even.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// One 16-byte fragment per lane feeds one "k-step" of a 16x16 output tile.
// bf16: the 8 values are k = 8*(lane/16) .. +7 of a 32-wide step, exactly the
// operand layout of v_mfma_f32_16x16x32_bf16.
// f32: the 4 values are k = 4*(lane/16) + j of a 16-wide step; the four
// v_mfma_f32_16x16x4f32 issues take element j of every lane, so each k of
// the step is summed exactly once (A and B use the same k order).
// Output (either type): lane l holds D[4*(l/16) + r][l % 16], r = 0..3, where
// the row index of D follows the FIRST operand and the column the second.
template <typename E> struct Mfma;

template <> struct Mfma<bf16> {
    static __device__ __forceinline__ f32x4 run(const uint4 &a, const uint4 &b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    static __device__ __forceinline__ f32x4 run(const uint4 &a, const uint4 &b, f32x4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
        return c;
    }
};

// 32x32 output tiles (v_mfma_f32_32x32x16_bf16 runs at the full dense rate on
// gfx950; the 16x16x32 form measured at little more than half of it).
// A lane's 16-byte fragment holds k = 8*(lane/32) .. +7 of a 16-wide bf16
// step, or k = 4*(lane/32) + j of an 8-wide fp32 step (four
// v_mfma_f32_32x32x2f32 issues, element j of every lane each).  Row (first
// operand) / column (second operand) of the tile = lane % 32.
// Output: lane l holds D[8*(q/4) + 4*(l/32) + q%4][l % 32], q = 0..15.
template <typename E> struct Mfma32;

template <> struct Mfma32<bf16> {
    static __device__ __forceinline__ f32x16 run(const uint4 &a, const uint4 &b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <> struct Mfma32<float> {
    static __device__ __forceinline__ f32x16 run(const uint4 &a, const uint4 &b, f32x16 c)
    {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
        return c;
    }
};

// Store 4 consecutive outputs of one row.
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d)
{
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d)
{
    bf16 v[4] = {from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c), from_f32<bf16>(d)};
    *reinterpret_cast<uint2 *>(p) = *reinterpret_cast<const uint2 *>(v);
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup i -> XCD i % 8),
// each XCD with its own L2.  Give XCD x a contiguous range of logical tiles so
// that tiles sharing operands meet in the same L2.  Returns -1 for a workgroup
// with no tile.  `total` may be known only on the device (grouped GEMMs).
__device__ __forceinline__ int xcd_logical_tile(int bid, int total)
{
    const int per = (total + 7) >> 3;
    const int xcd = bid & 7, j = bid >> 3;
    if (j >= per)
        return -1;
    const int t = xcd * per + j;
    return t < total ? t : -1;
}

}  // namespace lmoe
