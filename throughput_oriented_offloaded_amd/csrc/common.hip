// Status strings, per-thread error detail, device queries, closed-form sizes.
#include <algorithm>
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

namespace {
struct PlanBytes {
    int64_t weights, stage, kv, slots, ws, emb, act, total;
};

int plan_bytes(const fg_dims* d, const fg_plan* p, PlanBytes& b) {
    FG_TRY(fg::check_dims(d));
    FG_CHECK_ARG(p != nullptr, "null fg_plan");
    FG_CHECK_ARG(p->n_layers >= 1 && p->max_len >= 1 && p->bls_dev >= 0 && p->bls_host >= 0 &&
                     p->bls_dev + p->bls_host >= 1 && p->gbs >= 1 && p->s >= 0 && p->vocab >= 0,
                 "bad plan (layers %d, max_len %d, bls %d + %d, gbs %d, s %d)", p->n_layers,
                 p->max_len, p->bls_dev, p->bls_host, p->gbs, p->s);
    FG_CHECK_ARG(p->fmt_w == FG_FMT_F16 || p->fmt_w == FG_FMT_Q4G64, "unknown weight format %d", p->fmt_w);
    FG_CHECK_ARG(p->fmt_kv == FG_FMT_F16 || p->fmt_kv == FG_FMT_Q4G64, "unknown cache format %d", p->fmt_kv);
    FG_CHECK_ARG(p->n_tiered >= 0 && p->n_tiered <= p->n_layers, "n_tiered %d outside [0, %d]",
                 p->n_tiered, p->n_layers);
    FG_CHECK_ARG(p->n_tiered == 0 || p->fmt_w == FG_FMT_F16, "weight tiering keeps fp16 weights");
    FG_CHECK_ARG(p->bls_host % p->gbs == 0, "host-resident sequences (%d) must be whole GPU batches of %d",
                 p->bls_host, p->gbs);
    const int64_t h1 = d->h1, h2 = d->h2, l = p->n_layers, bls = p->bls_dev + p->bls_host;
    // matrices, minus the host halves of tiered layers (2 h1^2 + h1 h2 fp16
    // elements each), plus biases and the two LayerNorms of every layer
    b.weights = fg_weight_bytes(d, p->n_layers, p->fmt_w) - p->n_tiered * 2 * (2 * h1 * h1 + h1 * h2) +
                l * 2 * (5 * h1 + h2 + 4 * h1);
    b.stage = p->n_tiered ? 2 * (int64_t)fg_stage_bytes(d) : 0;
    b.kv = p->bls_dev ? fg_kv_bytes(d, p->n_layers, p->bls_dev, p->max_len, 0, p->fmt_kv) : 0;
    b.slots = p->bls_host ? 2 * (int64_t)fg_kvtier_slot_bytes(d, p->gbs, p->max_len, p->fmt_kv) : 0;
    int64_t ws = (int64_t)fg_workspace_bytes(d, (int64_t)p->gbs * p->s, p->fmt_w);
    ws = std::max<int64_t>(ws, (int64_t)fg_workspace_bytes(d, bls, p->fmt_w));
    if (p->vocab) ws = std::max<int64_t>(ws, (int64_t)fg_linear_workspace_bytes(bls, p->vocab, h1));
    b.ws = ws;
    b.emb = 2 * (p->vocab + p->max_len + 2) * h1;
    b.act = 2 * bls * std::max(p->s, 1) * h1 + 2 * bls * p->vocab;   // prompt activations, logits
    b.total = b.weights + b.stage + b.kv + b.slots + b.ws + b.emb + b.act;
    return FG_OK;
}
}  // namespace

int64_t fg_plan_device_bytes(const fg_dims* d, const fg_plan* p) {
    fg::clear_error();
    PlanBytes b{};
    if (plan_bytes(d, p, b) != FG_OK) return -1;
    return b.total;
}

int fg_check_capacity(const fg_dims* d, const fg_plan* p, int64_t budget_bytes) {
    fg::clear_error();
    FG_CHECK_ARG(budget_bytes >= 0, "negative budget");
    PlanBytes b{};
    FG_TRY(plan_bytes(d, p, b));
    int64_t budget = budget_bytes;
    const char* what = "budget";
    if (budget == 0) {
        size_t free_b = 0, total_b = 0;
        FG_HIP(hipMemGetInfo(&free_b, &total_b));
        budget = (int64_t)free_b;
        what = "free device memory";
    }
    if (b.total > budget)
        return fg::set_error(FG_ERR_CAPACITY,
                             "plan needs %.2f GB of HBM > %s %.2f GB (weights %.2f, stage %.2f, "
                             "KV %.2f, KV slots %.2f, workspace %.2f, embeddings %.2f, activations "
                             "and logits %.2f)",
                             b.total / 1e9, what, budget / 1e9, b.weights / 1e9, b.stage / 1e9,
                             b.kv / 1e9, b.slots / 1e9, b.ws / 1e9, b.emb / 1e9, b.act / 1e9);
    return FG_OK;
}

}  // extern "C"
