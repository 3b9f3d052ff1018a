// Causal prompt attention for the prefill ("FlexGen 完全拆解", section
// "从 Transformer 推理的数据流重新定义卸载": K, V, Q of all s prompt tokens
// are computed at once, and token t attends to tokens 0..t).
//
// Workgroup = (sequence, head, tile of query rows).  Lanes: HD/32 lanes per
// query row, each owning 32 dims of q and of the output accumulator.  Key and
// value tiles of 64 positions are staged in LDS and shared by every row of
// the tile; softmax is online (running max and sum per row), applied per
// chunk of 8 keys so the accumulator is rescaled once per chunk.
//
// The attention flops are ~3% of the prefill's projection flops at the OPT
// shapes, so this kernel stays on the vector ALUs.
#include "fg_internal.h"
#include "fg_trace.h"

namespace fg {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int KT = 64;     // keys per LDS tile
constexpr int CH = 8;      // keys per softmax chunk

__device__ __forceinline__ float lo_half(uint32_t w) {
    return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu)));
}
__device__ __forceinline__ float hi_half(uint32_t w) {
    return __half2float(__ushort_as_half((unsigned short)(w >> 16)));
}

template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const __half* __restrict__ qkv,
                                                           int32_t s, int32_t nh,
                                                           __half* __restrict__ out) {
    constexpr int LPP = HD / 32;
    constexpr int ROWS = 256 / LPP;
    constexpr int PADH = HD + 8;     // LDS row stride in halves (breaks bank aliasing)
    __shared__ __align__(16) __half ks[KT * PADH];
    __shared__ __align__(16) __half vs[KT * PADH];

    const int h1 = nh * HD;
    const int64_t ld = 3 * (int64_t)h1;
    const int ntiles = (s + ROWS - 1) / ROWS;
    const int tile = blockIdx.x % ntiles;
    const int64_t bh = blockIdx.x / ntiles;
    const int64_t b = bh / nh;
    const int h = (int)(bh % nh);
    const int lane = threadIdx.x;
    const int qi = lane % LPP;
    const int r = tile * ROWS + lane / LPP;       // query row of this lane
    const bool row_ok = r < s;
    const int rr = row_ok ? r : s - 1;

    const __half* seq = qkv + b * (int64_t)s * ld;
    float qv[32];
    {
        const uint4* p = reinterpret_cast<const uint4*>(seq + rr * ld + h * HD + qi * 32);
        const float qs = LOG2E / sqrtf((float)HD);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint4 w = p[k];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qv[8 * k + 2 * j] = lo_half(ww[j]) * qs;
                qv[8 * k + 2 * j + 1] = hi_half(ww[j]) * qs;
            }
        }
    }
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int last_row = min(s - 1, tile * ROWS + ROWS - 1);
    for (int k0 = 0; k0 <= last_row; k0 += KT) {
        __syncthreads();
        // stage K and V rows k0..k0+KT-1 (16-byte chunks; HD/8 chunks per row)
        for (int c = threadIdx.x; c < KT * (HD / 8); c += 256) {
            const int j = c / (HD / 8), part = c % (HD / 8);
            const int key = min(k0 + j, s - 1);
            const __half* src = seq + key * ld + h * HD + part * 8;
            *reinterpret_cast<uint4*>(&ks[j * PADH + part * 8]) =
                *reinterpret_cast<const uint4*>(src + h1);
            *reinterpret_cast<uint4*>(&vs[j * PADH + part * 8]) =
                *reinterpret_cast<const uint4*>(src + 2 * h1);
        }
        __syncthreads();
        const int jmax = min(KT, last_row - k0 + 1);
        for (int j0 = 0; j0 < jmax; j0 += CH) {
            float sc[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int j = j0 + c;
                float part = 0.f;
                if (j < jmax) {
                    const uint4* kp = reinterpret_cast<const uint4*>(&ks[j * PADH + qi * 32]);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        uint4 w = kp[k];
                        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            part = fmaf(qv[8 * k + 2 * t], lo_half(ww[t]), part);
                            part = fmaf(qv[8 * k + 2 * t + 1], hi_half(ww[t]), part);
                        }
                    }
                }
#pragma unroll
                for (int off = 1; off < LPP; off <<= 1) part += __shfl_xor(part, off);
                sc[c] = (j < jmax && k0 + j <= r) ? part : -INFINITY;
            }
            float mnew = m;
#pragma unroll
            for (int c = 0; c < CH; ++c) mnew = fmaxf(mnew, sc[c]);
            if (mnew == -INFINITY) continue;
            const float alpha = exp2f(m - mnew);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] *= alpha;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const float w = exp2f(sc[c] - mnew);
                if (w == 0.f) continue;
                l += w;
                const uint4* vp = reinterpret_cast<const uint4*>(&vs[(j0 + c) * PADH + qi * 32]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint4 wv = vp[k];
                    const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        acc[8 * k + 2 * t] = fmaf(w, lo_half(ww[t]), acc[8 * k + 2 * t]);
                        acc[8 * k + 2 * t + 1] = fmaf(w, hi_half(ww[t]), acc[8 * k + 2 * t + 1]);
                    }
                }
            }
            m = mnew;
        }
    }
    if (row_ok) {
        const float inv = 1.0f / l;
        uint32_t o[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            o[j] = (uint32_t)__half_as_ushort(__float2half_rn(acc[2 * j] * inv)) |
                   ((uint32_t)__half_as_ushort(__float2half_rn(acc[2 * j + 1] * inv)) << 16);
        uint4* op = reinterpret_cast<uint4*>(out + (b * (int64_t)s + r) * h1 + h * HD + qi * 32);
#pragma unroll
        for (int k = 0; k < 4; ++k) op[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
    }
}

}  // namespace

int launch_attn_prefill(const __half* qkv, int32_t b, int32_t s, const fg_dims* d, __half* out,
                        hipStream_t st) {
    if (b == 0 || s == 0) return FG_OK;
    const int rows = 256 / (d->head_dim / 32);
    const int64_t grid = (int64_t)b * d->n_heads * cdiv(s, rows);
    if (grid > INT32_MAX) return set_error(FG_ERR_UNSUPPORTED, "prefill grid too large");
    TraceScope ts(TK_ATTN_PREFILL, st, 4.0 * b * d->h1 * (double)s * (s + 1) / 2,
                  (double)b * s * d->h1 * 2 * 4);
    if (d->head_dim == 128)
        attn_prefill_kernel<128><<<(unsigned)grid, 256, 0, st>>>(qkv, s, d->n_heads, out);
    else
        attn_prefill_kernel<64><<<(unsigned)grid, 256, 0, st>>>(qkv, s, d->n_heads, out);
    FG_LAUNCHED("attn_prefill_kernel");
    return FG_OK;
}

}  // namespace fg

extern "C" int fg_attn_prefill(const void* qkv, int32_t b, int32_t s, const fg_dims* d, void* out,
                               void* stream) {
    fg::clear_error();
    FG_TRY(fg::check_dims(d));
    FG_CHECK_ARG(qkv && out, "null pointer argument");
    FG_CHECK_ARG(b >= 0 && s >= 0, "negative sizes");
    FG_CHECK_ARG(((uintptr_t)qkv | (uintptr_t)out) % 16 == 0, "pointers must be 16-byte aligned");
    return fg::launch_attn_prefill((const __half*)qkv, b, s, d, (__half*)out, fg::as_stream(stream));
}
