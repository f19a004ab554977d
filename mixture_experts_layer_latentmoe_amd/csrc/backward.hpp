// Kernels of the layer's backward pass besides the GEMMs (gemm.hpp).
//
// Gated experts keep the forward's B-column order throughout: in every
// block of 16 columns, 8 gate columns then the 8 value columns of the same
// outputs (the interleave of transpose_kernel's row map).  Pre-activations
// of the routed experts are fp32 [P, nb1] (their activation and its
// gradient are formed in the epilogues of the grouped GEMMs that produce
// them and dH); those of the shared experts sit in the x-pass's raw output
// XA [T, l + g S m_s] (z first) in E.
#pragma once

#include "common.hpp"

namespace lmoe {

__device__ __forceinline__ float bwd_silu(float g) { return g / (1.f + expf(-g)); }
__device__ __forceinline__ float bwd_sigmoid(float g) { return 1.f / (1.f + expf(-g)); }

// Column j of a gated block layout: the gate and value column of output j.
__device__ __forceinline__ int glu_gate_col(int j) { return 16 * (j >> 3) + (j & 7); }

// zh[t] = [z | act(shared pre-activations)] from the x-pass's raw output.
template <typename E>
__global__ __launch_bounds__(256) void xpass_act_kernel(const E *__restrict__ XA, int64_t ld_xa, int T, int l, int sms,
                                                        int gated, E *__restrict__ zh, int64_t ld_zh)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int w = l + sms;
    if (q >= (int64_t)T * w)
        return;
    const int64_t t = q / w;
    const int c = (int)(q - t * w);
    const E *row = XA + t * ld_xa;
    float v;
    if (c < l) {
        v = to_f32(row[c]);
    } else if (!gated) {
        const float a = fmaxf(to_f32(row[c]), 0.f);
        v = a * a;
    } else {
        const int gc = l + glu_gate_col(c - l);
        v = bwd_silu(to_f32(row[gc])) * to_f32(row[gc + 8]);
    }
    zh[t * ld_zh + c] = from_f32<E>(v);
}

// Eight consecutive values of E as one 16-byte (bf16) or two (fp32) moves.
template <typename E> __device__ __forceinline__ void load8(const E *p, float (&v)[8])
{
    if constexpr (sizeof(E) == 2) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        const E *e = reinterpret_cast<const E *>(&u);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = to_f32(e[i]);
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
}
template <typename E> __device__ __forceinline__ void store8(E *p, const float (&v)[8])
{
    if constexpr (sizeof(E) == 2) {
        E e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            e[i] = from_f32<E>(v[i]);
        *reinterpret_cast<uint4 *>(p) = *reinterpret_cast<const uint4 *>(e);
    } else {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// dz[t, 8 g ..] = sum_k dz_perm[pos[t, k], 8 g ..] (slot order) -> dX[t, col0 ..].
template <typename E>
__global__ __launch_bounds__(256) void gather_sum8_kernel(const E *__restrict__ dzp, const int *__restrict__ pos, int T,
                                                          int K, int l, E *__restrict__ dX, int64_t ld_dx, int col0)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int gpr = l / 8;
    if (q >= (int64_t)T * gpr)
        return;
    const int64_t t = q / gpr;
    const int g = (int)(q - t * gpr);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, v[8];
    for (int k = 0; k < K; ++k) {
        load8(dzp + (int64_t)pos[t * K + k] * l + 8 * g, v);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] += v[i];
    }
    store8(dX + t * ld_dx + col0 + 8 * g, acc);
}

// Gradient through the activation: from dh (width m or m_s) and the
// pre-activation, the gradient of the pre-activation (width nb = m, or 2m
// gated in the block layout).  d relu(a)^2 = 2 relu(a); d silu(g) v =
// (silu'(g) v, silu(g)), silu'(g) = sigma(g) (1 + g (1 - sigma(g))).
template <typename E, typename PRE>
__device__ __forceinline__ void act_grad(const PRE *pre, const E *dh, int j, bool gated, E *dpre)
{
    const float d = to_f32(dh[j]);
    if (!gated) {
        const float a = to_f32(pre[j]);
        dpre[j] = from_f32<E>(a > 0.f ? 2.f * a * d : 0.f);
        return;
    }
    const int c = glu_gate_col(j);
    const float g = to_f32(pre[c]), v = to_f32(pre[c + 8]), sg = bwd_sigmoid(g);
    dpre[c] = from_f32<E>(d * v * sg * (1.f + g * (1.f - sg)));
    dpre[c + 8] = from_f32<E>(d * g * sg);
}

// Shared experts: the shared part of dX_in [T, n_x] (columns from col0 on)
// from dh_s (dUH columns l .. l + S m_s) and the raw shared pre-activations
// in XA (columns l ..).
template <typename E>
__global__ __launch_bounds__(256) void shared_act_grad_kernel(const E *__restrict__ XA, int64_t ld_xa,
                                                              const E *__restrict__ dUH, int64_t ld_duh, int T,
                                                              int l, int sms, int gated, E *__restrict__ dX,
                                                              int64_t ld_dx, int col0)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)T * sms)
        return;
    const int64_t t = q / sms;
    const int j = (int)(q - t * sms);
    act_grad<E, E>(XA + t * ld_xa + l, dUH + t * ld_duh + l, j, gated != 0, dX + t * ld_dx + col0);
}

// Gates and combine, backward, one workgroup per token t:
//   dY_perm[pos[t,k]] = gate[t,k] du[t]          (du = dUH[t, 0:l])
//   dg_k = <du[t], Y_perm[pos[t,k]]>             (fp32, fixed order)
//   ds[t, e] = g_k (dg_k - sum_j g_j dg_j) for e = idx[t,k], 0 for the rest
// ds is written to dX[t, 0:N'].
template <typename E>
__global__ __launch_bounds__(256) void gate_combine_grad_kernel(const E *__restrict__ dUH, int64_t ld_duh,
                                                                const E *__restrict__ Yp, const int *__restrict__ pos,
                                                                const int *__restrict__ idx,
                                                                const float *__restrict__ gate, int K, int l, int N,
                                                                E *__restrict__ dYp, E *__restrict__ dX,
                                                                int64_t ld_dx)
{
    __shared__ float s_dg[64];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const E *du = dUH + t * ld_duh;
    for (int k = wave; k < K; k += 4) {
        const int64_t p = pos[t * K + k];
        const float g = gate[t * K + k];
        float acc = 0.f;
        for (int j = lane; j < l; j += 64) {
            const float d = to_f32(du[j]);
            dYp[p * l + j] = from_f32<E>(g * d);
            acc += d * to_f32(Yp[p * l + j]);
        }
        // fixed-order reduction over the 64 lanes
        for (int off = 32; off >= 1; off >>= 1)
            acc += __shfl_xor(acc, off, 64);
        if (lane == 0)
            s_dg[k] = acc;
    }
    __syncthreads();
    float gdg = 0.f;
    for (int k = 0; k < K; ++k)
        gdg += gate[t * K + k] * s_dg[k];
    E *ds = dX + t * ld_dx;
    for (int e = tid; e < N; e += 256)
        ds[e] = from_f32<E>(0.f);
    __syncthreads();
    for (int k = tid; k < K; k += 256) {
        const float g = gate[t * K + k];
        ds[idx[t * K + k]] = from_f32<E>(g * (s_dg[k] - gdg));
    }
}

// Padded per-expert offsets: koff[0] = 0, koff[e + 1] = koff[e] +
// roundup(counts[e], pad).  One workgroup of 1024 threads (N' <= 1024).
__global__ __launch_bounds__(1024) void padded_offsets_kernel(const int *__restrict__ counts, int N, int pad,
                                                              int *__restrict__ koff)
{
    __shared__ int s[1024];
    const int tid = threadIdx.x;
    const int v = tid < N ? (counts[tid] + pad - 1) / pad * pad : 0;
    s[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan (Hillis-Steele)
        const int a = tid >= off ? s[tid - off] : 0;
        __syncthreads();
        s[tid] += a;
        __syncthreads();
    }
    if (tid == 0)
        koff[0] = 0;
    if (tid < N)
        koff[tid + 1] = s[tid];
}

// Transpose rows of src into K-contiguous rows of dst with padded segments:
// dst[c][q] (row length ld_dst) for q in [koff[e], koff[e + 1]) holds
// column c of source row offs[e] + (q - koff[e]) while that is below
// offs[e + 1], else 0.  Without segments (koff == nullptr) q < rows maps to
// row q, and q in [rows, ld_dst) is 0.  gather (nullable) maps a row to the
// source row actually read.  32 x 32 tiles through LDS.
template <typename E>
__global__ __launch_bounds__(256) void pad_transpose_kernel(const E *__restrict__ src, int64_t ld_src, int rows,
                                                            int C, const int *__restrict__ gather,
                                                            const int *__restrict__ offs,
                                                            const int *__restrict__ koff, int nseg,
                                                            E *__restrict__ dst, int64_t ld_dst)
{
    __shared__ float tile[32][33];
    const int64_t q0 = (int64_t)blockIdx.y * 32;
    const int c0 = blockIdx.x * 32;
    const int64_t qend = koff ? koff[nseg] : ld_dst;
    if (q0 >= qend)
        return;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int i = ty; i < 32; i += 8) {
        const int64_t q = q0 + i;
        int64_t row = -1;
        if (q < qend) {
            if (koff) {
                int lo = 0, hi = nseg - 1;  // the segment e with koff[e] <= q < koff[e + 1]
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (koff[mid] <= q)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                const int64_t r = q - koff[lo];
                if (r < offs[lo + 1] - offs[lo])
                    row = offs[lo] + r;
            } else if (q < rows) {
                row = q;
            }
        }
        const int c = c0 + tx;
        float v = 0.f;
        if (row >= 0 && c < C) {
            const int64_t sr = gather ? gather[row] : row;
            v = to_f32(src[sr * ld_src + c]);
        }
        tile[i][tx] = v;
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
        const int c = c0 + i;
        const int64_t q = q0 + tx;
        if (c < C && q < qend)
            dst[c * ld_dst + q] = from_f32<E>(tile[tx][i]);
    }
}

// The same map as pad_transpose_kernel in 64 x 64 tiles with 16-byte loads
// and stores.  Padded segments are multiples of 64 long, so a tile of 64
// destination columns q0 .. q0 + 63 (q0 a multiple of 64) lies in one
// segment: one lookup per tile.  Needs C, ld_src and the source base
// 16-byte aligned in elements of E, and ld_dst a multiple of 64.
template <typename E>
__global__ __launch_bounds__(256) void pad_transpose64_kernel(const E *__restrict__ src, int64_t ld_src, int rows,
                                                              int C, const int *__restrict__ gather,
                                                              const int *__restrict__ offs,
                                                              const int *__restrict__ koff, int nseg,
                                                              E *__restrict__ dst, int64_t ld_dst)
{
    constexpr int VEC = 16 / (int)sizeof(E);  // elements per 16-byte access
    constexpr int TPR = 64 / VEC;             // threads per 64-element row
    constexpr int RPP = 256 / TPR;            // rows per pass
    __shared__ E tile[64][64 + 2];            // [c][q]
    __shared__ int64_t s_base;                // source row of q0 (-1: none)
    __shared__ int s_valid;                   // valid rows from q0 on
    const int64_t q0 = (int64_t)blockIdx.y * 64;
    const int c0 = blockIdx.x * 64;
    const int64_t qend = koff ? koff[nseg] : ld_dst;
    if (q0 >= qend)
        return;
    const int tid = threadIdx.x;
    if (tid == 0) {
        if (koff) {
            int lo = 0, hi = nseg - 1;  // the segment e with koff[e] <= q0 < koff[e + 1]
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (koff[mid] <= q0)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int64_t r = q0 - koff[lo];
            s_base = offs[lo] + r;
            s_valid = (int)max((int64_t)0, (int64_t)(offs[lo + 1] - offs[lo]) - r);
        } else {
            s_base = q0;
            s_valid = (int)max((int64_t)0, (int64_t)rows - q0);
        }
    }
    __syncthreads();
    const int64_t base = s_base;
    const int valid = s_valid;
    const int cl = (tid % TPR) * VEC;  // first column of this thread's 16 bytes
    for (int rr = tid / TPR; rr < 64; rr += RPP) {
        E v[VEC];
        if (rr < valid && c0 + cl < C) {
            const int64_t row = gather ? gather[base + rr] : base + rr;
            *reinterpret_cast<uint4 *>(v) = *reinterpret_cast<const uint4 *>(src + row * ld_src + c0 + cl);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                v[i] = from_f32<E>(0.f);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            tile[cl + i][rr] = v[i];
    }
    __syncthreads();
    const int ql = (tid % TPR) * VEC;
    for (int cc = tid / TPR; cc < 64; cc += RPP) {
        if (c0 + cc >= C || q0 + ql >= qend)
            continue;
        E v[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            v[i] = tile[cc][ql + i];
        *reinterpret_cast<uint4 *>(dst + (int64_t)(c0 + cc) * ld_dst + q0 + ql) = *reinterpret_cast<const uint4 *>(v);
    }
}

// A bank of k-tile-major matrices with the roles of rows and K swapped,
// per batch b of size R x C:  src[((r / bk) C + c) bk + r % bk] (K = R) ->
// dst[((c / bk) R + r) bk + c % bk] (K = C).  R and C are multiples of bk;
// 64 x 64 element tiles.
template <typename E, int BK>
__global__ __launch_bounds__(256) void retile_kernel(const E *__restrict__ src, int R, int C, E *__restrict__ dst)
{
    __shared__ E tile[BK][BK + 1];
    const int64_t b = blockIdx.z;
    const int rb = blockIdx.y, cb = blockIdx.x;  // tile (rb, cb): rows rb BK.., cols cb BK..
    const E *s = src + b * (int64_t)R * C;
    E *d = dst + b * (int64_t)R * C;
    for (int i = threadIdx.x; i < BK * BK; i += 256) {
        const int cc = i / BK, rr = i % BK;  // read along r (contiguous in src)
        tile[cc][rr] = s[((int64_t)rb * C + cb * BK + cc) * BK + rr];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < BK * BK; i += 256) {
        const int rr = i / BK, cc = i % BK;  // write along c (contiguous in dst)
        d[((int64_t)cb * R + rb * BK + rr) * BK + cc] = tile[cc][rr];
    }
}

// Column blocks of an fp32 [rows, ld] matrix to separate outputs:
// dst[b][r][j] = src[r][col0 + map(b, j)] for b < nb, j < w, where map is
// b w + j, or for gated pairs (block layout of 2 w columns per b) the gate
// (sel 0) or value (sel 1) column of output j.
__global__ __launch_bounds__(256) void split_cols_kernel(const float *__restrict__ src, int64_t ld, int rows, int col0,
                                                         int nb, int w, int gated_sel, float *__restrict__ dst)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)nb * rows * w)
        return;
    const int j = (int)(q % w);
    const int64_t br = q / w;
    const int r = (int)(br % rows), b = (int)(br / rows);
    int c;
    if (gated_sel < 0)
        c = b * w + j;
    else
        c = b * 2 * w + glu_gate_col(j) + 8 * gated_sel;
    dst[q] = src[(int64_t)r * ld + col0 + c];
}

// Column sums of ds (dX[:, 0:N'], E) over the tokens: the router-bias gradient.
template <typename E>
__global__ __launch_bounds__(256) void col_sum_kernel(const E *__restrict__ dX, int64_t ld, int T, int N,
                                                      float *__restrict__ out)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= N)
        return;
    float acc = 0.f;
    for (int t = 0; t < T; ++t)
        acc += to_f32(dX[(int64_t)t * ld + e]);
    out[e] = acc;
}

}  // namespace lmoe
