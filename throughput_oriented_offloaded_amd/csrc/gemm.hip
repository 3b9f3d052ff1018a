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
// Every shape runs the stream-K kernel family of gemm_sk.hip / gemm_sk32.hip:
//  * decode-shaped contractions (M up to a few hundred rows): exactly 256
//    workgroups share the (tile, k-step) iterations; tiles split between
//    workgroups leave fp32 partials that a reduce kernel sums in a fixed
//    order (deterministic) and finishes with the epilogue;
//  * large-M contractions (the prefill, M = gbs * s): fp16 weights go to the
//    256 x 256-tile kernel of gemm_tile.hip; 4-bit weights (the prefill
//    restores them to fp16 first) take whole stream-K tiles g, g + 256, ...
//    in a banded order.
#include "gemm_common.h"
#include "fg_trace.h"

namespace fg {

bool linear_is_dp(int64_t M) { return M > gemm::kSkDpRows; }

size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t) {
    const gemm::SkSched sc = gemm::sk_schedule(M, N, K);
    return gemm::sk_ws_bytes(sc, M, N);
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
    p.tile_ns = nullptr;
    // algorithmic work: 2MNK flops; weights once, activations in, outputs out
    const double Md = (double)p.M, Nd = (double)p.N, Kd = (double)p.K;
    const double wbytes = q4 ? Nd * Kd / 2 + Nd / 64 * Kd * 4 : Nd * Kd * 2;
    const double gbytes = wbytes + 2 * Md * Kd + 2 * Md * Nd * (p.residual ? 2 : 1) + (p.bias ? 2 * Nd : 0);
    auto need_ws = [&](size_t need) -> int {
        if (!a.ws || a.ws_bytes < need)
            return set_error(FG_ERR_CAPACITY, "linear needs %zu workspace bytes, got %zu", need,
                             a.ws ? a.ws_bytes : (size_t)0);
        return FG_OK;
    };

    if (!q4 && linear_is_dp(a.M) && tile_fits(p)) {
        {
            TraceScope ts(TK_GEMM_F16, st, 2 * Md * Nd * Kd, gbytes);
            FG_TRY(launch_tile(p, st));
        }
        return a.ln_y ? launch_layernorm(a.y, a.M, a.N, a.ln_g, a.ln_b, a.ln_y, st) : FG_OK;
    }
    const SkSched sc = sk_schedule(a.M, a.N, a.K);
    if (!sc.dp && sc.T >= (1ll << 31))
        return set_error(FG_ERR_UNSUPPORTED, "decode GEMM: %lld (tile, k-step) iterations", (long long)sc.T);
    if (sc.slots > 1) {
        FG_TRY(need_ws(sk_ws_bytes(sc, a.M, a.N)));
        p.part = static_cast<float*>(a.ws);
        p.tile_ns = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(a.ws) + sk_part_bytes(sc, a.M, a.N));
    }
    {
        // the stream-K launch records the trace events itself
        TraceScope ts(kExtLaunch, q4 ? TK_GEMM_Q4 : TK_GEMM_F16, st, 2 * Md * Nd * Kd, gbytes,
                      a.proj >= 1 && a.proj <= 4 ? TK_PROJ_QKV + a.proj - 1 : -1);
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
