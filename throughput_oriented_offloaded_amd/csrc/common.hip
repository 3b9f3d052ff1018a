// Status strings, per-thread error detail, device queries, closed-form sizes.
#include <atomic>
#include <cstdio>
#include <cstring>

#include "fg_internal.h"

namespace fg {

namespace {
thread_local char g_err[512] = {0};
}

int set_error(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_err[0] = 0; }

int num_cus() {
    static std::atomic<int> cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int check_dims(const fg_dims* d) {
    FG_CHECK_ARG(d != nullptr, "null fg_dims");
    FG_CHECK_ARG(d->h1 > 0 && d->h2 > 0 && d->n_heads > 0 && d->head_dim > 0,
                 "dims must be positive (h1 %d, h2 %d, heads %d, head_dim %d)", d->h1, d->h2,
                 d->n_heads, d->head_dim);
    FG_CHECK_ARG((int64_t)d->n_heads * d->head_dim == d->h1,
                 "h1 (%d) != n_heads (%d) * head_dim (%d)", d->h1, d->n_heads, d->head_dim);
    FG_CHECK_SUP(d->head_dim == 64 || d->head_dim == 128, "head_dim %d unsupported (64 or 128)",
                 d->head_dim);
    FG_CHECK_SUP(d->h1 % 64 == 0 && d->h2 % 64 == 0,
                 "h1 (%d) and h2 (%d) must be multiples of 64", d->h1, d->h2);
    return FG_OK;
}

}  // namespace fg

extern "C" {

int fg_abi_version(void) { return 3; }

const char* fg_status_str(int status) {
    switch (status) {
        case FG_OK: return "ok";
        case FG_ERR_INVALID: return "invalid argument";
        case FG_ERR_UNSUPPORTED: return "unsupported";
        case FG_ERR_CAPACITY: return "capacity exceeded";
        case FG_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* fg_last_error(void) { return fg::g_err; }

// M_W = l (8 h1^2 + 4 h1 h2) bytes in fp16 ("FlexGen 完全拆解", section
// "从 Transformer 推理的数据流重新定义卸载"); 4-bit: half a byte per element
// plus an fp16 (min, scale) pair per 64 elements.
int64_t fg_weight_bytes(const fg_dims* d, int32_t n_layers, int32_t fmt) {
    if (!d || n_layers < 0 || d->h1 <= 0 || d->h2 <= 0) return -1;
    const int64_t h1 = d->h1, h2 = d->h2;
    const int64_t elems = 4 * h1 * h1 + 2 * h1 * h2;
    if (fmt == FG_FMT_F16) return n_layers * 2 * elems;
    if (fmt == FG_FMT_Q4G64) return n_layers * (elems / 2 + elems / 64 * 4);
    return -1;
}

// M_KV = 4 b l h1 (s + n) bytes in fp16 (same section); 4-bit: 9/32 of it.
int64_t fg_kv_bytes(const fg_dims* d, int32_t n_layers, int32_t bls, int32_t s, int32_t n,
                    int32_t fmt) {
    if (!d || n_layers < 0 || bls < 0 || s < 0 || n < 0 || d->h1 <= 0) return -1;
    const int64_t elems = 2 * (int64_t)bls * n_layers * d->h1 * (int64_t)(s + n);
    if (fmt == FG_FMT_F16) return 2 * elems;
    if (fmt == FG_FMT_Q4G64) return elems / 2 + elems / 64 * 4;
    return -1;
}

}  // extern "C"
