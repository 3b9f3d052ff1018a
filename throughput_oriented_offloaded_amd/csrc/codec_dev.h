// Device-side arithmetic of the group-wise 4-bit min-max codec, shared by the
// standalone quantizer and by the kernels that write the KV cache.
//
// Method: "FlexGen 完全拆解" (pinghaoyang.com.cn), section "权重压缩与 KV Cache
// 压缩": q(x) = round((x - x_min) / (x_max - x_min) * (2^b - 1)) with b = 4 and
// x^ = x_min + q * (x_max - x_min) / (2^b - 1); groups of 64, two codes per
// byte, fp16 (min, scale) per group (bjbfmj.com FlexGen walkthrough §6.3).
//
// Every operation below is one IEEE binary32 operation (no contraction into
// FMA, correctly rounded division, rint = nearest-even) so that codes and
// metadata are bit-identical to a plain CPU evaluation of the same formula.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

namespace fg {

struct QParams {
    float mn;     // group minimum, -0 canonicalised to +0
    float range;  // max - min
    float inv;    // 15 / range (0 for a constant group)
};

__device__ __forceinline__ QParams qparams(float mn, float mx) {
#pragma clang fp contract(off)
    QParams p;
    p.mn = mn + 0.0f;
    float m2 = mx + 0.0f;
    p.range = m2 - p.mn;
    p.inv = p.range > 0.0f ? 15.0f / p.range : 0.0f;
    return p;
}

__device__ __forceinline__ uint32_t qcode(float v, const QParams& p) {
#pragma clang fp contract(off)
    if (!(p.range > 0.0f)) return 0u;
    float d = v - p.mn;
    float r = __builtin_rintf(d * p.inv);
    int q = (int)r;
    q = q < 0 ? 0 : (q > 15 ? 15 : q);
    return (uint32_t)q;
}

// fp16 bits of the stored (min, scale) pair.
__device__ __forceinline__ uint32_t qmeta_bits(const QParams& p) {
#pragma clang fp contract(off)
    __half a = __float2half_rn(p.mn);
    __half b = __float2half_rn(p.range / 15.0f);
    return (uint32_t)__half_as_ushort(a) | ((uint32_t)__half_as_ushort(b) << 16);
}

// x^ = fp16(mn + q * scale): a binary32 multiply, then a binary32 add.
__device__ __forceinline__ __half dq_value(uint32_t q, float mn, float sc) {
#pragma clang fp contract(off)
    float t = (float)q * sc;
    float r = mn + t;
    return __float2half_rn(r);
}

__device__ __forceinline__ float h2f_bits(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xffffu)));
}

}  // namespace fg
