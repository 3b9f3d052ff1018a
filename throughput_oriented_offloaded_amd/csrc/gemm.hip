// Projection GEMM of the decoder: y = act(x W^T + bias) + residual, with W in
// fp16 or in the group-wise 4-bit format, dequantized on the fly.
//
// Why MFMA: in the zig-zag block every GPU batch of the block passes through
// the resident layer before the next layer runs ("FlexGen 完全拆解", section
// "FlexGen 的核心:计算图分块与张量生命周期"), so one weight pass serves
// M = bls rows and the contraction is dense (2*M flops per weight element,
// 512 flop/B for 4-bit weights at M = 144).  Compression targets storage and
// I/O and the data are restored to fp16 before compute (section "权重压缩与
// KV Cache 压缩"): the 4-bit codes are unpacked to fp16 in registers and fed to
// v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//
// Two kernel families:
//  * decode-shaped contractions (M up to a few hundred rows) run the
//    stream-K pipelined kernel of gemm_sk.hip;
//  * large-M contractions (the prefill, M = gbs * s) run the tiled kernel
//    below: 128 x 128 tiles of 2 x 2 waves, k-step 64 double-buffered in LDS
//    through registers.  MFMA A operand = weight rows (16 n x 32 k), B operand
//    = activation rows (32 k x 16 m), so each lane's 4 accumulators are 4
//    consecutive output columns.
// When the tile count alone cannot fill the CUs the contraction is split over
// grid.z; fp32 partials go to the workspace and a reduce kernel applies the
// epilogue in a fixed order (deterministic, independent of the row count).
#include "gemm_common.h"
#include "fg_trace.h"

namespace fg {
namespace gemm {
namespace {

template <int MB_, int NB_, int WM_, int WN_, bool Q4_>
struct Cfg {
    static constexpr int MB = MB_, NB = NB_, WM = WM_, WN = WN_;
    static constexpr bool Q4 = Q4_;
    static constexpr int BM = WM * MB * 16;
    static constexpr int BN = WN * NB * 16;
    static constexpr int BK = 64;
    static constexpr int NT = WM * WN * 64;
    static constexpr int XS = BK + 8;    // activation row stride in LDS (halves)
    static constexpr int WS = BK + 8;    // fp16 weight row stride in LDS (halves)
    static constexpr int CS = BK + 16;   // code row stride in LDS (bytes)
    static constexpr int X_BYTES = BM * XS * 2;
    static constexpr int C_BYTES = Q4 ? (BN / 2) * CS : 0;
    static constexpr int M_BYTES = Q4 ? (BN / 64) * 2 * BK * 2 : 0;
    static constexpr int W_BYTES = Q4 ? C_BYTES + M_BYTES : BN * WS * 2;
    static constexpr int STAGE = X_BYTES + W_BYTES;
    // 16-byte chunks per stage
    static constexpr int X_CH = BM * BK / 8;
    static constexpr int W_CH = Q4 ? (BN / 2) * BK / 16 : BN * BK / 8;
    static constexpr int M_CH = Q4 ? (BN / 64) * 2 * BK / 8 : 0;
    static constexpr int X_IT = (X_CH + NT - 1) / NT;
    static constexpr int W_IT = (W_CH + NT - 1) / NT;
    static constexpr int M_IT = (M_CH + NT - 1) / NT;
    static_assert(!Q4 || NB * 16 == 64, "4-bit tiles give each wave one 64-row group");
};

template <class C>
__global__ __launch_bounds__(C::NT) void gemm_kernel(Params p) {
    __shared__ __align__(16) unsigned char smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % C::WN;
    const int wm = wave / C::WN;
    const int64_t n0 = (int64_t)blockIdx.x * C::BN;
    const int64_t m0 = (int64_t)blockIdx.y * C::BM;
    const int64_t kbeg = (int64_t)blockIdx.z * p.kchunk;
    const int64_t kend = min(p.K, kbeg + p.kchunk);
    const int nk = kbeg < kend ? (int)((kend - kbeg) / C::BK) : 0;

    f4 acc[C::NB][C::MB];
#pragma unroll
    for (int i = 0; i < C::NB; ++i)
#pragma unroll
        for (int j = 0; j < C::MB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    uint4 rx[C::X_IT], rw[C::W_IT], rm[C::M_IT > 0 ? C::M_IT : 1];

    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < C::X_IT; ++i) {
            const int c = tid + i * C::NT;
            const int row = c / (C::BK / 8), col = (c % (C::BK / 8)) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < C::X_CH && m0 + row < p.M)
                v = *reinterpret_cast<const uint4*>(p.x + (m0 + row) * p.ldx + k0 + col);
            rx[i] = v;
        }
        if constexpr (C::Q4) {
            const uint8_t* codes = static_cast<const uint8_t*>(p.w);
#pragma unroll
            for (int i = 0; i < C::W_IT; ++i) {
                const int c = tid + i * C::NT;
                const int row = c / (C::BK / 16), col = (c % (C::BK / 16)) * 16;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c < C::W_CH && n0 + 2 * row < p.N)
                    v = *reinterpret_cast<const uint4*>(codes + (n0 / 2 + row) * p.K + k0 + col);
                rw[i] = v;
            }
#pragma unroll
            for (int i = 0; i < C::M_IT; ++i) {
                const int c = tid + i * C::NT;
                const int row = c / (C::BK / 8), col = (c % (C::BK / 8)) * 8;   // row = g*2 + which
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c < C::M_CH && n0 + (row / 2) * 64 < p.N)
                    v = *reinterpret_cast<const uint4*>(p.meta + ((n0 / 64) * 2 + row) * p.K + k0 + col);
                rm[i] = v;
            }
        } else {
            const __half* w = static_cast<const __half*>(p.w);
#pragma unroll
            for (int i = 0; i < C::W_IT; ++i) {
                const int c = tid + i * C::NT;
                const int row = c / (C::BK / 8), col = (c % (C::BK / 8)) * 8;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c < C::W_CH && n0 + row < p.N)
                    v = *reinterpret_cast<const uint4*>(w + (n0 + row) * p.K + k0 + col);
                rw[i] = v;
            }
        }
    };

    auto sstore = [&](int buf) {
        unsigned char* base = smem + buf * C::STAGE;
        __half* xs = reinterpret_cast<__half*>(base);
#pragma unroll
        for (int i = 0; i < C::X_IT; ++i) {
            const int c = tid + i * C::NT;
            if (c < C::X_CH) {
                const int row = c / (C::BK / 8), col = (c % (C::BK / 8)) * 8;
                *reinterpret_cast<uint4*>(xs + row * C::XS + col) = rx[i];
            }
        }
        if constexpr (C::Q4) {
            unsigned char* cs = base + C::X_BYTES;
            __half* ms = reinterpret_cast<__half*>(base + C::X_BYTES + C::C_BYTES);
#pragma unroll
            for (int i = 0; i < C::W_IT; ++i) {
                const int c = tid + i * C::NT;
                if (c < C::W_CH) {
                    const int row = c / (C::BK / 16), col = (c % (C::BK / 16)) * 16;
                    *reinterpret_cast<uint4*>(cs + row * C::CS + col) = rw[i];
                }
            }
#pragma unroll
            for (int i = 0; i < C::M_IT; ++i) {
                const int c = tid + i * C::NT;
                if (c < C::M_CH) {
                    const int row = c / (C::BK / 8), col = (c % (C::BK / 8)) * 8;
                    *reinterpret_cast<uint4*>(ms + row * C::BK + col) = rm[i];
                }
            }
        } else {
            __half* ws = reinterpret_cast<__half*>(base + C::X_BYTES);
#pragma unroll
            for (int i = 0; i < C::W_IT; ++i) {
                const int c = tid + i * C::NT;
                if (c < C::W_CH) {
                    const int row = c / (C::BK / 8), col = (c % (C::BK / 8)) * 8;
                    *reinterpret_cast<uint4*>(ws + row * C::WS + col) = rw[i];
                }
            }
        }
    };

    auto compute = [&](int buf) {
        const unsigned char* base = smem + buf * C::STAGE;
        const __half* xs = reinterpret_cast<const __half*>(base);
        const int r16 = lane & 15;
        const int kq = (lane >> 4) * 8;
#pragma unroll
        for (int kk = 0; kk < C::BK; kk += 32) {
            h8 a[C::NB];
            if constexpr (C::Q4) {
                const unsigned char* cs = base + C::X_BYTES;
                const __half* ms = reinterpret_cast<const __half*>(base + C::X_BYTES + C::C_BYTES);
                const int nl0 = wn * C::NB * 16;           // first weight row of this wave
                const int g = nl0 / 64;
                const uint4 mn = *reinterpret_cast<const uint4*>(ms + (g * 2 + 0) * C::BK + kk + kq);
                const uint4 sc = *reinterpret_cast<const uint4*>(ms + (g * 2 + 1) * C::BK + kk + kq);
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    const int nl = nl0 + nb * 16 + r16;
                    const uint2 c = *reinterpret_cast<const uint2*>(cs + (nl >> 1) * C::CS + kk + kq);
                    a[nb] = dequant8(c, (uint32_t)(nl & 1) * 4u, mn, sc);
                }
            } else {
                const __half* ws = reinterpret_cast<const __half*>(base + C::X_BYTES);
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    const int nl = (wn * C::NB + nb) * 16 + r16;
                    a[nb] = *reinterpret_cast<const h8*>(ws + nl * C::WS + kk + kq);
                }
            }
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
                const int ml = (wm * C::MB + mb) * 16 + r16;
                const h8 bx = *reinterpret_cast<const h8*>(xs + ml * C::XS + kk + kq);
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[nb], bx, acc[nb][mb], 0, 0, 0);
            }
        }
    };

    if (nk > 0) {
        gload(kbeg);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) gload(kbeg + (int64_t)(kt + 1) * C::BK);
            compute(kt & 1);
            if (more) sstore((kt + 1) & 1);
            __syncthreads();
        }
    }

    // epilogue: lane holds D[n .. n+3][m]
    const int r16 = lane & 15;
    const int nq = (lane >> 4) * 4;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        const int64_t n = n0 + (wn * C::NB + nb) * 16 + nq;
        if (n >= p.N) continue;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
            const int64_t m = m0 + (wm * C::MB + mb) * 16 + r16;
            if (m < p.M) store4(p, m, n, acc[nb][mb], blockIdx.z);
        }
    }
}

// Sum the S split-K partials in split order, then bias / ReLU / residual.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(Params p, int S) {
    const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;   // element (m, n..n+3)
    if (idx >= p.M * p.N) return;
    const int64_t m = idx / p.N, n = idx % p.N;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
        const float4 v = *reinterpret_cast<const float4*>(p.part + ((int64_t)s * p.M + m) * p.N + n);
        o[0] += v.x; o[1] += v.y; o[2] += v.z; o[3] += v.w;
    }
    if (p.bias) {
        const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
        o[0] += h2f(bb.x); o[1] += h2f(bb.x >> 16);
        o[2] += h2f(bb.y); o[3] += h2f(bb.y >> 16);
    }
    if (p.act == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = fmaxf(o[i], 0.f);
    }
    if (p.residual) {
        const uint2 rr = *reinterpret_cast<const uint2*>(p.residual + m * p.ldy + n);
        o[0] += h2f(rr.x); o[1] += h2f(rr.x >> 16);
        o[2] += h2f(rr.y); o[3] += h2f(rr.y >> 16);
    }
    *reinterpret_cast<uint2*>(p.y + m * p.ldy + n) = make_uint2(pack_h2(o[0], o[1]), pack_h2(o[2], o[3]));
}

// ----------------------------------------------------------- configurations
// Prefill-shaped (M = gbs * s): 2 x 2 waves, 128 x 128 tile.
using PreQ = Cfg<4, 4, 2, 2, true>;
using PreF = Cfg<4, 4, 2, 2, false>;

// Rows up to which the pipelined decode kernel is used.
constexpr int64_t PIPE_MAX_M = 4 * 144;

// Tiled (prefill-shaped) launch: 128 x 128 tiles, the k range split until the
// launch has about two workgroups per CU of the 256-CU part (a constant, so
// the plan and its workspace size depend on the shape only), keeping at least
// 4 k-steps of 64 per split.
struct Plan {
    int64_t mt, nt;  // tiles
    int S;           // k splits
    int64_t kchunk;
};

Plan make_plan(int64_t M, int64_t N, int64_t K) {
    Plan pl{};
    pl.mt = cdiv(M, 128);
    pl.nt = cdiv(N, 128);
    const int64_t ksteps = K / 64;
    const int64_t tiles = pl.mt * pl.nt;
    int S = 1;
    if (tiles < 512) {
        S = (int)std::min<int64_t>(cdiv(512, tiles), 16);
        S = (int)std::min<int64_t>(S, std::max<int64_t>(1, ksteps / 4));
    }
    pl.kchunk = cdiv(ksteps, S) * 64;
    pl.S = (int)cdiv(K, pl.kchunk);
    return pl;
}

template <class C>
int run_tiled(const Params& p, const Plan& pl, hipStream_t st) {
    dim3 grid((unsigned)pl.nt, (unsigned)pl.mt, (unsigned)pl.S);
    gemm_kernel<C><<<grid, C::NT, 0, st>>>(p);
    FG_LAUNCHED("gemm_kernel");
    return FG_OK;
}

}  // namespace
}  // namespace gemm

size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t) {
    if (M <= gemm::PIPE_MAX_M) {
        const gemm::SkSched sc = gemm::sk_schedule(M, N, K);
        return sc.slots > 1 ? (size_t)sc.slots * M * N * sizeof(float) : 0;
    }
    const gemm::Plan pl = gemm::make_plan(M, N, K);
    return pl.S > 1 ? (size_t)pl.S * M * N * sizeof(float) : 0;
}

int launch_linear(const LinearArgs& a, hipStream_t st) {
    using namespace gemm;
    if (a.M == 0 || a.N == 0) return FG_OK;
    if (a.ln_y && a.ldy != a.N) return set_error(FG_ERR_INVALID, "layernorm of the output needs ldy == N");
    const bool q4 = a.fmt == FG_FMT_Q4G64;
    Params p{};
    p.x = a.x; p.M = a.M; p.K = a.K; p.ldx = a.ldx;
    p.w = a.w; p.meta = a.meta; p.N = a.N;
    p.bias = a.bias; p.act = a.act; p.residual = a.residual;
    p.y = a.y; p.ldy = a.ldy;
    p.part = nullptr;
    // algorithmic work: 2MNK flops; weights once, activations in, outputs out
    const double Md = (double)p.M, Nd = (double)p.N, Kd = (double)p.K;
    const double wbytes = q4 ? Nd * Kd / 2 + Nd / 64 * Kd * 4 : Nd * Kd * 2;
    const double gbytes = wbytes + 2 * Md * Kd + 2 * Md * Nd * (p.residual ? 2 : 1) + (p.bias ? 2 * Nd : 0);
    auto need_ws = [&](size_t need) -> int {
        if (!a.ws || a.ws_bytes < need)
            return set_error(FG_ERR_CAPACITY, "linear needs %zu workspace bytes, got %zu", need,
                             a.ws ? a.ws_bytes : (size_t)0);
        p.part = static_cast<float*>(a.ws);
        return FG_OK;
    };

    if (a.M <= PIPE_MAX_M) {
        const SkSched sc = sk_schedule(a.M, a.N, a.K);
        if (sc.slots > 1) FG_TRY(need_ws((size_t)sc.slots * a.M * a.N * sizeof(float)));
        {
            TraceScope ts(q4 ? TK_GEMM_Q4 : TK_GEMM_F16, st, 2 * Md * Nd * Kd, gbytes);
            FG_TRY(launch_sk(p, sc, q4, st));
        }
        if (sc.slots > 1 && a.ln_y) {
            TraceScope ts(TK_REDUCE_LN, st, 0.0,
                          Md * Nd * (4.0 * sc.slots + 2.0 * (a.residual ? 3 : 2)) + 4 * Nd);
            return launch_sk_reduce_ln(p, sc, a.ln_g, a.ln_b, a.ln_y, st);
        }
        if (sc.slots > 1) {
            TraceScope ts(TK_SPLITK_REDUCE, st, 0.0,
                          Md * Nd * (4.0 * sc.slots + 2.0 * (a.residual ? 2 : 1)));
            FG_TRY(launch_sk_reduce(p, sc, st));
        }
        return a.ln_y ? launch_layernorm(a.y, a.M, a.N, a.ln_g, a.ln_b, a.ln_y, st) : FG_OK;
    }

    const Plan pl = make_plan(a.M, a.N, a.K);
    p.kchunk = pl.kchunk;
    if (pl.S > 1) FG_TRY(need_ws((size_t)pl.S * a.M * a.N * sizeof(float)));
    {
        TraceScope ts(q4 ? TK_GEMM_Q4 : TK_GEMM_F16, st, 2 * Md * Nd * Kd, gbytes);
        const int rc = q4 ? run_tiled<PreQ>(p, pl, st) : run_tiled<PreF>(p, pl, st);
        if (rc != FG_OK) return rc;
    }
    if (pl.S > 1) {
        const int64_t n4 = a.M * a.N / 4;
        TraceScope ts(TK_SPLITK_REDUCE, st, 0.0,
                      (double)a.M * a.N * (4.0 * pl.S + 2.0 * (a.residual ? 2 : 1)));
        splitk_reduce_kernel<<<(unsigned)cdiv(n4, 256), 256, 0, st>>>(p, pl.S);
        FG_LAUNCHED("splitk_reduce_kernel");
    }
    return a.ln_y ? launch_layernorm(a.y, a.M, a.N, a.ln_g, a.ln_b, a.ln_y, st) : FG_OK;
}

}  // namespace fg

extern "C" size_t fg_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return std::max(fg::linear_ws_bytes(M, N, K, FG_FMT_F16),
                    fg::linear_ws_bytes(M, N, K, FG_FMT_Q4G64));
}

extern "C" int fg_linear(const void* x, int64_t M, int64_t K, int32_t fmt, const void* w,
                         const void* m, int64_t N, const void* bias, int32_t act,
                         const void* residual, void* y, void* ws, size_t ws_bytes, void* stream) {
    fg::clear_error();
    FG_CHECK_ARG(x && w && y, "null pointer argument");
    FG_CHECK_ARG(fmt == FG_FMT_F16 || fmt == FG_FMT_Q4G64, "unknown weight format %d", fmt);
    FG_CHECK_ARG(fmt != FG_FMT_Q4G64 || m, "4-bit weights need their metadata");
    FG_CHECK_ARG(M >= 0 && M < (1ll << 31) && N > 0 && N < (1ll << 31) && K > 0 && K < (1ll << 31),
                 "bad sizes (M %lld, N %lld, K %lld)", (long long)M, (long long)N, (long long)K);
    FG_CHECK_SUP(K % 64 == 0, "K (%lld) must be a multiple of 64", (long long)K);
    FG_CHECK_SUP(fmt == FG_FMT_Q4G64 ? N % 64 == 0 : N % 8 == 0,
                 "N (%lld) must be a multiple of %d", (long long)N, fmt == FG_FMT_Q4G64 ? 64 : 8);
    FG_CHECK_ARG(act == 0 || act == 1, "unknown activation %d", act);
    FG_CHECK_ARG(((uintptr_t)x | (uintptr_t)w | (uintptr_t)y | (uintptr_t)m |
                  (uintptr_t)residual) % 16 == 0 && (uintptr_t)bias % 8 == 0,
                 "x, w, meta, y, residual must be 16-byte aligned, bias 8-byte aligned");
    fg::LinearArgs a{};
    a.x = (const __half*)x; a.M = M; a.K = K; a.ldx = K;
    a.fmt = fmt; a.w = w; a.meta = (const __half*)m; a.N = N;
    a.bias = (const __half*)bias; a.act = act; a.residual = (const __half*)residual;
    a.y = (__half*)y; a.ldy = N; a.ws = ws; a.ws_bytes = ws_bytes;
    return fg::launch_linear(a, fg::as_stream(stream));
}
