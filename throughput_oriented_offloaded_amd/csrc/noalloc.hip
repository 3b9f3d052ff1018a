// fg_linear_noalloc: the projection GEMM of fg_linear for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The stream-K partials that fg_linear
// keeps in a caller workspace live here in a file-scope device array instead,
// one copy per GPU, held until the process ends.
//
// The array's host-side name is only a stand-in for the symbol; its device
// address on each GPU comes from hipGetSymbolAddress, taken once per device on
// the first call there (with that device current) and kept in g_scratch.  Only
// that address is passed to the kernels.
#include <mutex>

#include "fg_internal.h"

namespace fg {
namespace {

constexpr size_t kScratchBytes = (size_t)96 << 20;   // 96 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's scratch array (resolved once per device).
int scratch_ptr(void** out) {
    int dev = -1;
    FG_HIP(hipGetDevice(&dev));
    FG_CHECK_SUP(dev >= 0 && dev < kMaxDevices, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(FG_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s",
                             hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FG_OK;
}

}  // namespace
}  // namespace fg

extern "C" size_t fg_linear_noalloc_max_bytes(void) { return fg::kScratchBytes; }

extern "C" int fg_linear_noalloc(const void* x, int64_t M, int64_t K, int32_t fmt, const void* w,
                                 const void* m, int64_t N, const void* bias, int32_t act,
                                 const void* residual, void* y, void* stream) {
    fg::clear_error();
    // the same validation as fg_linear, then the scratch bound
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
    const size_t need = fg_linear_workspace_bytes(M, N, K);
    FG_CHECK_SUP(need <= fg::kScratchBytes,
                 "M %lld x N %lld x K %lld needs %zu bytes of partials, beyond the %zu-byte scratch "
                 "of fg_linear_noalloc (use fg_linear with a workspace)",
                 (long long)M, (long long)N, (long long)K, need, fg::kScratchBytes);
    void* ws = nullptr;
    FG_TRY(fg::scratch_ptr(&ws));
    fg::LinearArgs a{};
    a.x = (const __half*)x; a.M = M; a.K = K; a.ldx = K;
    a.fmt = fmt; a.w = w; a.meta = (const __half*)m; a.N = N;
    a.bias = (const __half*)bias; a.act = act; a.residual = (const __half*)residual;
    a.y = (__half*)y; a.ldy = N; a.ws = ws; a.ws_bytes = fg::kScratchBytes;
    return fg::launch_linear(a, fg::as_stream(stream));
}
