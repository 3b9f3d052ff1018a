// Row-wise device helpers shared by the LayerNorm kernels (norm.hip, and the
// stream-K reduce fused with the LayerNorm that follows it in gemm_sk.hip):
// one 256-thread workgroup per row, 8-element fp16 vectors per thread.
#pragma once
#include "fg_internal.h"

namespace fg {
namespace row {

constexpr int NT = 256;

// sum over a workgroup of T threads (sh: T / 64 floats)
template <int T = NT>
__device__ __forceinline__ float block_sum(float v, float* sh) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) sh[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < T / 64; ++i) t += sh[i];
    return t;
}

__device__ __forceinline__ void load8(const __half* p, float v[8]) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xffff)));
        v[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
    }
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)__half_as_ushort(__float2half_rn(a)) |
           ((uint32_t)__half_as_ushort(__float2half_rn(b)) << 16);
}

// LayerNorm (biased variance, eps 1e-5) of a row of width h whose vectors
// vi = threadIdx.x + i NT (vi < h / 8) are in v; s is this thread's sum of
// its elements.  Two passes over the registers: mean, then variance.
template <int MAXV>
__device__ __forceinline__ void layernorm_row(const float (&v)[MAXV][8], float s, int64_t h,
                                              const __half* __restrict__ g,
                                              const __half* __restrict__ b,
                                              __half* __restrict__ y, float* sh) {
    const int nv = (int)(h / 8);
    const float mean = block_sum(s, sh) / (float)h;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int vi = threadIdx.x + i * NT;
        if (vi < nv) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float d = v[i][j] - mean;
                q += d * d;
            }
        }
    }
    const float var = block_sum(q, sh) / (float)h;
    const float rstd = 1.0f / sqrtf(var + 1e-5f);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int vi = threadIdx.x + i * NT;
        if (vi < nv) {
            float gv[8], bv[8];
            load8(g + vi * 8, gv);
            load8(b + vi * 8, bv);
            uint4 o;
            uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ow[j] = pack2((v[i][2 * j] - mean) * rstd * gv[2 * j] + bv[2 * j],
                              (v[i][2 * j + 1] - mean) * rstd * gv[2 * j + 1] + bv[2 * j + 1]);
            *reinterpret_cast<uint4*>(y + vi * 8) = o;
        }
    }
}

}  // namespace row
}  // namespace fg
