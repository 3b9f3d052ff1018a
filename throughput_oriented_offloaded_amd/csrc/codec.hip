// Standalone group-wise 4-bit quantizer / dequantizer (fg_quant_group4,
// fg_dequant_group4).  HBM-bound: per element 2 B read + 0.5 B codes +
// 4/64 B meta written (quantize), the reverse for dequantize.
//
// Two layouts of the group axis:
//  * inner == 1 (groups contiguous, e.g. a K/V row): 8 lanes own one group,
//    each loading 16 B; the group min/max is reduced across those 8 lanes of
//    the wavefront.
//  * inner > 1 (groups strided, e.g. a weight [N, K] grouped along N): one
//    thread owns 4 adjacent columns of one group and walks its 64 rows; the
//    wavefront reads 64 x 4 consecutive columns = 512 B per row, coalesced.
//    Min/max are taken in a first pass, codes in a second pass that hits L2.
#include "codec_dev.h"
#include "fg_internal.h"
#include "fg_trace.h"

namespace fg {
namespace {

constexpr int G = 64;

__device__ __forceinline__ void unpack8(const uint4& r, float v[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = h2f_bits(w[i]);
        v[2 * i + 1] = h2f_bits(w[i] >> 16);
    }
}

// ---------------------------------------------------------------- inner == 1
__global__ __launch_bounds__(256) void quant_contig_kernel(const __half* __restrict__ x,
                                                           int64_t ngroups,
                                                           uint8_t* __restrict__ codes,
                                                           uint32_t* __restrict__ meta) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t g = tid >> 3;
    const int sub = (int)(tid & 7);
    const bool valid = g < ngroups;   // uniform over each 8-lane set
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (valid) raw = *reinterpret_cast<const uint4*>(x + g * G + sub * 8);
    float v[8];
    unpack8(raw, v);
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, v[i]);
        mx = fmaxf(mx, v[i]);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, off));
        mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    const QParams p = qparams(mn, mx);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= qcode(v[i], p) << (4 * i);
    if (valid) {
        *reinterpret_cast<uint32_t*>(codes + g * (G / 2) + sub * 4) = packed;
        if (sub == 0) meta[g] = qmeta_bits(p);
    }
}

__global__ __launch_bounds__(256) void dequant_contig_kernel(const uint8_t* __restrict__ codes,
                                                             const uint32_t* __restrict__ meta,
                                                             int64_t ngroups,
                                                             __half* __restrict__ y) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t g = tid >> 3;
    const int sub = (int)(tid & 7);
    if (g >= ngroups) return;
    const uint32_t packed = *reinterpret_cast<const uint32_t*>(codes + g * (G / 2) + sub * 4);
    const uint32_t m = meta[g];
    const float mn = h2f_bits(m), sc = h2f_bits(m >> 16);
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __half a = dq_value((packed >> (8 * i)) & 15u, mn, sc);
        __half b = dq_value((packed >> (8 * i + 4)) & 15u, mn, sc);
        out[i] = (uint32_t)__half_as_ushort(a) | ((uint32_t)__half_as_ushort(b) << 16);
    }
    *reinterpret_cast<uint4*>(y + g * G + sub * 8) = make_uint4(out[0], out[1], out[2], out[3]);
}

// ----------------------------------------------------------------- inner > 1
template <int C>
struct Cols;
template <>
struct Cols<4> {
    using T = uint2;
    __device__ static void load(const __half* p, float v[4]) {
        uint2 r = *reinterpret_cast<const uint2*>(p);
        v[0] = h2f_bits(r.x); v[1] = h2f_bits(r.x >> 16);
        v[2] = h2f_bits(r.y); v[3] = h2f_bits(r.y >> 16);
    }
};
template <>
struct Cols<1> {
    __device__ static void load(const __half* p, float v[1]) { v[0] = __half2float(*p); }
};

template <int C>
__global__ __launch_bounds__(256) void quant_strided_kernel(const __half* __restrict__ x,
                                                            int64_t outer, int64_t axis,
                                                            int64_t inner,
                                                            uint8_t* __restrict__ codes,
                                                            __half* __restrict__ meta) {
    const int64_t ngroups = axis / G;
    const int64_t ncol = inner / C;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tid >= outer * ngroups * ncol) return;
    const int64_t ci = tid % ncol;
    const int64_t og = tid / ncol;
    const int64_t g = og % ngroups, o = og / ngroups;
    const int64_t i0 = ci * C;
    const __half* base = x + (o * axis + g * G) * inner + i0;

    float mn[C], mx[C];
#pragma unroll
    for (int c = 0; c < C; ++c) { mn[c] = INFINITY; mx[c] = -INFINITY; }
    for (int j = 0; j < G; ++j) {
        float v[C];
        Cols<C>::load(base + (int64_t)j * inner, v);
#pragma unroll
        for (int c = 0; c < C; ++c) { mn[c] = fminf(mn[c], v[c]); mx[c] = fmaxf(mx[c], v[c]); }
    }
    QParams p[C];
#pragma unroll
    for (int c = 0; c < C; ++c) p[c] = qparams(mn[c], mx[c]);

    uint8_t* cbase = codes + (o * (axis / 2) + g * (G / 2)) * inner + i0;
    for (int j = 0; j < G; j += 2) {
        float a[C], b[C];
        Cols<C>::load(base + (int64_t)j * inner, a);
        Cols<C>::load(base + (int64_t)(j + 1) * inner, b);
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < C; ++c) word |= (qcode(a[c], p[c]) | (qcode(b[c], p[c]) << 4)) << (8 * c);
        if constexpr (C == 4)
            *reinterpret_cast<uint32_t*>(cbase + (int64_t)(j / 2) * inner) = word;
        else
            cbase[(int64_t)(j / 2) * inner] = (uint8_t)word;
    }
    __half* mbase = meta + (o * ngroups + g) * 2 * inner + i0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        uint32_t bits = qmeta_bits(p[c]);
        mbase[c] = __ushort_as_half((unsigned short)(bits & 0xffff));
        mbase[inner + c] = __ushort_as_half((unsigned short)(bits >> 16));
    }
}

// Strided groups, 4 columns per thread, the whole 64-row group held in
// registers (64 x 8 B): every row is loaded once, all loads issued before any
// is used; consecutive threads own consecutive columns, so a workgroup reads
// 2 KB contiguous per row.  Min / max on packed fp16 pairs (exact: the inputs
// are fp16); the codes use the codec's fp32 formula.
__global__ __launch_bounds__(256) void quant_strided_reg_kernel(const __half* __restrict__ x,
                                                                int64_t outer, int64_t axis,
                                                                int64_t inner,
                                                                uint8_t* __restrict__ codes,
                                                                __half* __restrict__ meta) {
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    const int64_t ngroups = axis / G;
    const int64_t ncol = inner / 4;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tid >= outer * ngroups * ncol) return;
    const int64_t ci = tid % ncol;
    const int64_t og = tid / ncol;
    const int64_t g = og % ngroups, o = og / ngroups;
    const int64_t i0 = ci * 4;
    const __half* base = x + (o * axis + g * G) * inner + i0;

    uint2 r[G];
#pragma unroll
    for (int j = 0; j < G; ++j) r[j] = *reinterpret_cast<const uint2*>(base + (int64_t)j * inner);
    h2v lo_mn = __builtin_bit_cast(h2v, r[0].x), lo_mx = lo_mn;   // columns 0, 1
    h2v hi_mn = __builtin_bit_cast(h2v, r[0].y), hi_mx = hi_mn;   // columns 2, 3
#pragma unroll
    for (int j = 1; j < G; ++j) {
        const h2v a = __builtin_bit_cast(h2v, r[j].x), b = __builtin_bit_cast(h2v, r[j].y);
        lo_mn = __builtin_elementwise_min(lo_mn, a);
        lo_mx = __builtin_elementwise_max(lo_mx, a);
        hi_mn = __builtin_elementwise_min(hi_mn, b);
        hi_mx = __builtin_elementwise_max(hi_mx, b);
    }
    QParams p[4];
    p[0] = qparams((float)lo_mn[0], (float)lo_mx[0]);
    p[1] = qparams((float)lo_mn[1], (float)lo_mx[1]);
    p[2] = qparams((float)hi_mn[0], (float)hi_mx[0]);
    p[3] = qparams((float)hi_mn[1], (float)hi_mx[1]);

    uint8_t* cbase = codes + (o * (axis / 2) + g * (G / 2)) * inner + i0;
#pragma unroll
    for (int j = 0; j < G; j += 2) {
        const uint32_t A[2] = {r[j].x, r[j].y}, B[2] = {r[j + 1].x, r[j + 1].y};
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float a = h2f_bits(A[c >> 1] >> (16 * (c & 1)));
            const float b = h2f_bits(B[c >> 1] >> (16 * (c & 1)));
            word |= (qcode(a, p[c]) | (qcode(b, p[c]) << 4)) << (8 * c);
        }
        *reinterpret_cast<uint32_t*>(cbase + (int64_t)(j / 2) * inner) = word;
    }
    __half* mbase = meta + (o * ngroups + g) * 2 * inner + i0;
    uint32_t mb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) mb[c] = qmeta_bits(p[c]);
    *reinterpret_cast<uint2*>(mbase) = make_uint2((mb[0] & 0xffffu) | (mb[1] << 16), (mb[2] & 0xffffu) | (mb[3] << 16));
    *reinterpret_cast<uint2*>(mbase + inner) =
        make_uint2((mb[0] >> 16) | (mb[1] & 0xffff0000u), (mb[2] >> 16) | (mb[3] & 0xffff0000u));
}

template <int C>
__global__ __launch_bounds__(256) void dequant_strided_kernel(const uint8_t* __restrict__ codes,
                                                              const __half* __restrict__ meta,
                                                              int64_t outer, int64_t axis,
                                                              int64_t inner,
                                                              __half* __restrict__ y) {
    const int64_t ngroups = axis / G;
    const int64_t ncol = inner / C;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tid >= outer * ngroups * ncol) return;
    const int64_t ci = tid % ncol;
    const int64_t og = tid / ncol;
    const int64_t g = og % ngroups, o = og / ngroups;
    const int64_t i0 = ci * C;
    const __half* mbase = meta + (o * ngroups + g) * 2 * inner + i0;
    float mn[C], sc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        mn[c] = __half2float(mbase[c]);
        sc[c] = __half2float(mbase[inner + c]);
    }
    const uint8_t* cbase = codes + (o * (axis / 2) + g * (G / 2)) * inner + i0;
    __half* ybase = y + (o * axis + g * G) * inner + i0;
    for (int j = 0; j < G; j += 2) {
        uint32_t word;
        if constexpr (C == 4)
            word = *reinterpret_cast<const uint32_t*>(cbase + (int64_t)(j / 2) * inner);
        else
            word = cbase[(int64_t)(j / 2) * inner];
        if constexpr (C == 4) {
            uint32_t e[4], f[4];   // rows j, j + 1 of the 4 columns
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t byte = (word >> (8 * c)) & 0xffu;
                e[c] = __half_as_ushort(dq_value(byte & 15u, mn[c], sc[c]));
                f[c] = __half_as_ushort(dq_value(byte >> 4, mn[c], sc[c]));
            }
            *reinterpret_cast<uint2*>(ybase + (int64_t)j * inner) = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
            *reinterpret_cast<uint2*>(ybase + (int64_t)(j + 1) * inner) = make_uint2(f[0] | (f[1] << 16), f[2] | (f[3] << 16));
        } else {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                uint32_t byte = (word >> (8 * c)) & 0xffu;
                ybase[(int64_t)j * inner + c] = dq_value(byte & 15u, mn[c], sc[c]);
                ybase[(int64_t)(j + 1) * inner + c] = dq_value(byte >> 4, mn[c], sc[c]);
            }
        }
    }
}

int grid_of(int64_t threads) { return (int)cdiv(threads, 256); }

}  // namespace

int launch_quant_g4(const __half* x, int64_t outer, int64_t axis, int64_t inner, uint8_t* codes,
                    __half* meta, hipStream_t st) {
    const int64_t ngroups = axis / G;
    const double ne = (double)outer * axis * inner;
    TraceScope ts(TK_QUANT, st, 0.0, ne * 2 + ne / 2 + ne / 64 * 4);
    if (inner == 1) {
        const int64_t n = outer * ngroups;
        quant_contig_kernel<<<grid_of(n * 8), 256, 0, st>>>(x, n, codes,
                                                           reinterpret_cast<uint32_t*>(meta));
        FG_LAUNCHED("quant_contig_kernel");
    } else if (inner % 4 == 0) {
        quant_strided_reg_kernel<<<grid_of(outer * ngroups * (inner / 4)), 256, 0, st>>>(
            x, outer, axis, inner, codes, meta);
        FG_LAUNCHED("quant_strided_reg_kernel");
    } else {
        quant_strided_kernel<1><<<grid_of(outer * ngroups * inner), 256, 0, st>>>(
            x, outer, axis, inner, codes, meta);
        FG_LAUNCHED("quant_strided_kernel<1>");
    }
    return FG_OK;
}

int launch_dequant_g4(const uint8_t* codes, const __half* meta, int64_t outer, int64_t axis,
                      int64_t inner, __half* y, hipStream_t st) {
    const int64_t ngroups = axis / G;
    const double ne = (double)outer * axis * inner;
    TraceScope ts(TK_DEQUANT, st, 0.0, ne * 2 + ne / 2 + ne / 64 * 4);
    if (inner == 1) {
        const int64_t n = outer * ngroups;
        dequant_contig_kernel<<<grid_of(n * 8), 256, 0, st>>>(
            codes, reinterpret_cast<const uint32_t*>(meta), n, y);
        FG_LAUNCHED("dequant_contig_kernel");
    } else if (inner % 4 == 0) {
        dequant_strided_kernel<4><<<grid_of(outer * ngroups * (inner / 4)), 256, 0, st>>>(
            codes, meta, outer, axis, inner, y);
        FG_LAUNCHED("dequant_strided_kernel<4>");
    } else {
        dequant_strided_kernel<1><<<grid_of(outer * ngroups * inner), 256, 0, st>>>(
            codes, meta, outer, axis, inner, y);
        FG_LAUNCHED("dequant_strided_kernel<1>");
    }
    return FG_OK;
}

}  // namespace fg

// -------------------------------------------------------------------- C ABI
namespace {
int check_codec_args(const void* a, const void* b, const void* c, int64_t outer, int64_t axis,
                     int64_t inner, int32_t group) {
    FG_CHECK_ARG(a && b && c, "null pointer argument");
    FG_CHECK_ARG(outer >= 1 && axis >= 1 && inner >= 1,
                 "sizes must be positive (outer %lld, axis %lld, inner %lld)", (long long)outer,
                 (long long)axis, (long long)inner);
    FG_CHECK_SUP(group == 64, "only group size 64 is supported (got %d)", group);
    FG_CHECK_ARG(axis % group == 0, "axis %lld is not a multiple of the group %d",
                 (long long)axis, group);
    FG_CHECK_ARG(outer <= (int64_t)1 << 40 && axis <= (int64_t)1 << 40 &&
                     inner <= (int64_t)1 << 40 && outer * axis <= ((int64_t)1 << 62) / inner,
                 "tensor too large");
    return FG_OK;
}
}  // namespace

extern "C" int fg_quant_group4(const void* x, int64_t outer, int64_t axis, int64_t inner,
                               int32_t group, void* codes, void* meta, void* stream) {
    fg::clear_error();
    FG_TRY(check_codec_args(x, codes, meta, outer, axis, inner, group));
    FG_CHECK_ARG(((uintptr_t)x % 16) == 0 && ((uintptr_t)codes % 4) == 0 &&
                     ((uintptr_t)meta % 4) == 0,
                 "x must be 16-byte aligned, codes and meta 4-byte aligned");
    return fg::launch_quant_g4(static_cast<const __half*>(x), outer, axis, inner,
                               static_cast<uint8_t*>(codes), static_cast<__half*>(meta),
                               fg::as_stream(stream));
}

extern "C" int fg_dequant_group4(const void* codes, const void* meta, int64_t outer,
                                 int64_t axis, int64_t inner, int32_t group, void* y,
                                 void* stream) {
    fg::clear_error();
    FG_TRY(check_codec_args(codes, meta, y, outer, axis, inner, group));
    FG_CHECK_ARG(((uintptr_t)y % 16) == 0 && ((uintptr_t)codes % 4) == 0 &&
                     ((uintptr_t)meta % 4) == 0,
                 "y must be 16-byte aligned, codes and meta 4-byte aligned");
    return fg::launch_dequant_g4(static_cast<const uint8_t*>(codes),
                                 static_cast<const __half*>(meta), outer, axis, inner,
                                 static_cast<__half*>(y), fg::as_stream(stream));
}
