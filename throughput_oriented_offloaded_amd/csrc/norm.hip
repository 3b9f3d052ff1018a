// Row-wise kernels of the decoder: LayerNorm, token + position embedding,
// greedy argmax.  All HBM/latency-bound and tiny next to the projections and
// attention; each row is one 256-thread workgroup reading 16-byte vectors.
#include "fg_trace.h"
#include "rowops.h"

namespace fg {
namespace {

using row::NT;
using row::load8;
using row::pack2;

// LayerNorm of one row per workgroup; up to MAXV 8-element vectors per thread
// stay in registers between the mean, variance and output passes.
template <int MAXV>
__global__ __launch_bounds__(NT) void layernorm_kernel(const __half* __restrict__ x, int64_t h,
                                                       const __half* __restrict__ g,
                                                       const __half* __restrict__ b,
                                                       __half* __restrict__ y) {
    __shared__ float sh[NT / 64];
    const int64_t r = blockIdx.x;
    const __half* xr = x + r * h;
    const int nv = (int)(h / 8);
    float v[MAXV][8];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int vi = threadIdx.x + i * NT;
        if (vi < nv) {
            load8(xr + vi * 8, v[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) s += v[i][j];
        }
    }
    row::layernorm_row<MAXV>(v, s, h, g, b, y + r * h, sh);
}

__global__ __launch_bounds__(NT) void embed_kernel(const int32_t* __restrict__ tok,
                                                   const int32_t* __restrict__ pos,
                                                   int32_t pos_const, int64_t pos_period,
                                                   const __half* __restrict__ E, int64_t vocab,
                                                   const __half* __restrict__ P, int64_t max_pos,
                                                   int64_t h1, __half* __restrict__ x) {
    const int64_t row = blockIdx.x;
    int64_t t = tok[row];
    t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
    int64_t p = pos ? (int64_t)pos[row] : (int64_t)pos_const + (pos_period > 0 ? row % pos_period : 0);
    p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
    const __half* er = E + t * h1;
    const __half* pr = P + p * h1;
    for (int64_t vi = threadIdx.x; vi < h1 / 8; vi += NT) {
        float a[8], c[8];
        load8(er + vi * 8, a);
        load8(pr + vi * 8, c);
        uint4 o;
        uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
        for (int j = 0; j < 4; ++j) ow[j] = pack2(a[2 * j] + c[2 * j], a[2 * j + 1] + c[2 * j + 1]);
        *reinterpret_cast<uint4*>(x + row * h1 + vi * 8) = o;
    }
}

__device__ __forceinline__ void better(float& bv, int64_t& bi, float v, int64_t i) {
    if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__global__ __launch_bounds__(NT) void argmax_kernel(const __half* __restrict__ logits, int64_t n,
                                                    int32_t* __restrict__ out) {
    __shared__ float sv[NT / 64];
    __shared__ int64_t si[NT / 64];
    const int64_t row = blockIdx.x;
    const __half* lr = logits + row * n;
    float bv = -INFINITY;
    int64_t bi = INT64_MAX;
    if (n % 8 == 0) {
        for (int64_t vi = threadIdx.x; vi < n / 8; vi += NT) {
            float v[8];
            load8(lr + vi * 8, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) better(bv, bi, v[j], vi * 8 + j);
        }
    } else {
        for (int64_t i = threadIdx.x; i < n; i += NT) better(bv, bi, __half2float(lr[i]), i);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int64_t oi = __shfl_xor(bi, off);
        better(bv, bi, ov, oi);
    }
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) { sv[w] = bv; si[w] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < NT / 64; ++i) better(bv, bi, sv[i], si[i]);
        out[row] = (int32_t)(bi == INT64_MAX ? 0 : bi);
    }
}

}  // namespace

int launch_layernorm(const __half* x, int64_t rows, int64_t h, const __half* g, const __half* b,
                     __half* y, hipStream_t st) {
    if (rows == 0) return FG_OK;
    TraceScope ts(TK_LAYERNORM, st, 0.0, (double)rows * h * 4 + (double)h * 4);
    const int64_t nv = h / 8;
    if (nv <= NT * 2) {
        layernorm_kernel<2><<<(unsigned)rows, NT, 0, st>>>(x, h, g, b, y);
    } else if (nv <= NT * 8) {
        layernorm_kernel<8><<<(unsigned)rows, NT, 0, st>>>(x, h, g, b, y);
    } else if (nv <= NT * 16) {
        layernorm_kernel<16><<<(unsigned)rows, NT, 0, st>>>(x, h, g, b, y);
    } else {
        return set_error(FG_ERR_UNSUPPORTED, "layernorm width %lld exceeds 32768", (long long)h);
    }
    FG_LAUNCHED("layernorm_kernel");
    return FG_OK;
}

int launch_embed(const int32_t* tok, const int32_t* pos, int32_t pos_const, int64_t pos_period,
                 int64_t rows, const __half* E, int64_t vocab, const __half* P, int64_t max_pos,
                 int64_t h1, __half* x, hipStream_t st) {
    if (rows == 0) return FG_OK;
    TraceScope ts(TK_EMBED, st, 0.0, (double)rows * h1 * 6);
    embed_kernel<<<(unsigned)rows, NT, 0, st>>>(tok, pos, pos_const, pos_period, E, vocab, P,
                                                max_pos, h1, x);
    FG_LAUNCHED("embed_kernel");
    return FG_OK;
}

int launch_argmax(const __half* logits, int64_t rows, int64_t n, int32_t* out, hipStream_t st) {
    if (rows == 0) return FG_OK;
    TraceScope ts(TK_ARGMAX, st, 0.0, (double)rows * n * 2);
    argmax_kernel<<<(unsigned)rows, NT, 0, st>>>(logits, n, out);
    FG_LAUNCHED("argmax_kernel");
    return FG_OK;
}

}  // namespace fg

extern "C" int fg_layernorm(const void* x, int64_t rows, int64_t h, const void* gamma,
                            const void* beta, void* y, void* stream) {
    fg::clear_error();
    FG_CHECK_ARG(x && gamma && beta && y, "null pointer argument");
    FG_CHECK_ARG(rows >= 0 && rows < (1ll << 31) && h > 0, "bad sizes (rows %lld, h %lld)",
                 (long long)rows, (long long)h);
    FG_CHECK_SUP(h % 8 == 0, "h (%lld) must be a multiple of 8", (long long)h);
    FG_CHECK_ARG(((uintptr_t)x | (uintptr_t)y | (uintptr_t)gamma | (uintptr_t)beta) % 16 == 0,
                 "pointers must be 16-byte aligned");
    return fg::launch_layernorm((const __half*)x, rows, h, (const __half*)gamma,
                                (const __half*)beta, (__half*)y, fg::as_stream(stream));
}

extern "C" int fg_embed(const int32_t* tok, const int32_t* pos, int64_t rows, const void* E,
                        int64_t vocab, const void* P, int64_t max_pos, int64_t h1, void* x,
                        void* stream) {
    fg::clear_error();
    FG_CHECK_ARG(tok && pos && E && P && x, "null pointer argument");
    FG_CHECK_ARG(rows >= 0 && rows < (1ll << 31) && vocab > 0 && max_pos > 0 && h1 > 0,
                 "bad sizes");
    FG_CHECK_SUP(h1 % 8 == 0, "h1 must be a multiple of 8");
    FG_CHECK_ARG(((uintptr_t)E | (uintptr_t)P | (uintptr_t)x) % 16 == 0,
                 "tables and output must be 16-byte aligned");
    return fg::launch_embed(tok, pos, 0, 0, rows, (const __half*)E, vocab, (const __half*)P,
                            max_pos, h1, (__half*)x, fg::as_stream(stream));
}

extern "C" int fg_argmax(const void* logits, int64_t rows, int64_t n, int32_t* out,
                         void* stream) {
    fg::clear_error();
    FG_CHECK_ARG(logits && out, "null pointer argument");
    FG_CHECK_ARG(rows >= 0 && rows < (1ll << 31) && n > 0, "bad sizes");
    FG_CHECK_ARG(n % 8 != 0 || (uintptr_t)logits % 16 == 0,
                 "logits must be 16-byte aligned when n %% 8 == 0");
    return fg::launch_argmax((const __half*)logits, rows, n, out, fg::as_stream(stream));
}
