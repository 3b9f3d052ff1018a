// Kernel tracing: when enabled, every launch of the library gets two HIP
// events on its stream, tagged with its kind and the algorithmic work of that
// launch (flops, HBM bytes): recorded around the launch, or, for the launches
// that take them (hipExtLaunchKernelGGL), recorded by the launch itself at
// the kernel's start and end.  fg_trace_collect waits for the events and
// returns, per kind, the launch count, the summed durations and the summed
// work, from which a caller derives achieved TFLOP/s or GB/s per kernel.
#include <mutex>
#include <vector>

#include "fg_trace.h"

namespace fg {
namespace {

struct Rec {
    int kind, kind2;   // kinds credited with the bracket (-1: none)
    hipEvent_t a, b;
    double flops, bytes;
    bool dropped;      // launch-recorded scope whose events no launch took
};

thread_local long t_ext_pending = -1;   // record index of this thread's pending ext scope

std::mutex g_mu;
bool g_on = false;
uint64_t g_mask = ~0ull;          // kinds that are recorded while tracing is on
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;   // free events

void give(hipEvent_t e) {
    if (e) g_pool.push_back(e);
}

hipEvent_t take() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    // timing-only events: no system-scope fence on record (the cache
    // write-back and invalidation it implies would be timed with the kernel
    // and slow the work that follows); collection waits on them and reads
    // elapsed times only
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

const char* kNames[TK_COUNT] = {
    "quant_g4", "dequant_g4", "gemm_q4", "gemm_f16", "splitk_reduce", "attn_decode_q4",
    "attn_decode_f16", "kv_store", "attn_prefill", "layernorm", "embed", "argmax",
    "reduce_layernorm", "attn_topk_q4", "attn_topk_f16", "kv_h2d", "kv_d2h", "w_h2d",
    "proj_qkv", "proj_out", "proj_fc1", "proj_fc2"};

}  // namespace

bool trace_on() { return g_on; }

// The record of a new scope (its events taken from the pool), or -1 when
// tracing is off, neither kind is wanted or no event can be had.  Called with
// g_mu held.
static long open_record(int kind, int kind2, double flops, double bytes) {
    auto wanted = [](int k) { return k >= 0 && k < TK_COUNT && ((g_mask >> k) & 1ull) ? k : -1; };
    const int k1 = wanted(kind), k2 = wanted(kind2);
    if (!g_on || (k1 < 0 && k2 < 0)) return -1;
    Rec r{k1, k2, take(), take(), flops, bytes, false};
    if (!r.a || !r.b) {
        give(r.a);
        give(r.b);
        return -1;
    }
    g_recs.push_back(r);
    return (long)g_recs.size() - 1;
}

TraceScope::TraceScope(int kind, hipStream_t st, double flops, double bytes, int kind2) {
    if (!g_on) return;
    std::lock_guard<std::mutex> lk(g_mu);
    const long i = open_record(kind, kind2, flops, bytes);
    if (i < 0) return;
    // a launch that cannot be traced is simply not recorded; its events go
    // back to the pool
    if (hipEventRecord(g_recs[i].a, st) != hipSuccess) {
        give(g_recs[i].a);
        give(g_recs[i].b);
        g_recs.pop_back();
        return;
    }
    st_ = st;
    idx_ = i;
}

TraceScope::TraceScope(ExtLaunch, int kind, hipStream_t st, double flops, double bytes, int kind2) {
    ext_ = true;
    if (!g_on) return;
    std::lock_guard<std::mutex> lk(g_mu);
    const long i = open_record(kind, kind2, flops, bytes);
    if (i < 0) return;
    st_ = st;
    idx_ = i;
    t_ext_pending = i;
}

TraceScope::~TraceScope() {
    if (idx_ < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (idx_ >= (long)g_recs.size()) return;   // tracing was reset meanwhile
    if (!ext_) {
        (void)hipEventRecord(g_recs[idx_].b, st_);
        return;
    }
    if (t_ext_pending == idx_) {               // no launch took the events
        t_ext_pending = -1;
        g_recs[idx_].dropped = true;
    }
}

void trace_take_ext(hipEvent_t* start, hipEvent_t* stop) {
    *start = *stop = nullptr;
    if (t_ext_pending < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (t_ext_pending < (long)g_recs.size()) {
        *start = g_recs[t_ext_pending].a;
        *stop = g_recs[t_ext_pending].b;
    }
    t_ext_pending = -1;
}

}  // namespace fg

extern "C" int fg_trace_enable(int on) {
    std::lock_guard<std::mutex> lk(fg::g_mu);
    for (auto& r : fg::g_recs) {
        fg::g_pool.push_back(r.a);
        fg::g_pool.push_back(r.b);
    }
    fg::g_recs.clear();
    fg::g_on = on != 0;
    return FG_OK;
}

extern "C" int fg_trace_kinds(uint64_t mask) {
    std::lock_guard<std::mutex> lk(fg::g_mu);
    fg::g_mask = mask;
    return FG_OK;
}

extern "C" const char* fg_trace_kind_name(int kind) {
    return (kind >= 0 && kind < fg::TK_COUNT) ? fg::kNames[kind] : "";
}

extern "C" int fg_trace_collect(int32_t n_kinds, int64_t* count, double* ms, double* flops,
                                double* bytes) {
    fg::clear_error();
    FG_CHECK_ARG(count && ms && flops && bytes, "null output array");
    FG_CHECK_ARG(n_kinds >= fg::TK_COUNT, "need room for %d kinds", (int)fg::TK_COUNT);
    for (int k = 0; k < n_kinds; ++k) { count[k] = 0; ms[k] = flops[k] = bytes[k] = 0.0; }
    std::lock_guard<std::mutex> lk(fg::g_mu);
    // every record is visited: one that cannot be timed is left out of the
    // sums and the first such failure is reported after the rest are summed
    hipError_t first = hipSuccess;
    const char* what = "";
    for (auto& r : fg::g_recs) {
        if (r.dropped) continue;
        hipError_t e = hipEventSynchronize(r.b);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
        else what = "hipEventSynchronize";
        if (e != hipSuccess) {
            if (first == hipSuccess) {
                first = e;
                if (!*what) what = "hipEventElapsedTime";
            }
            continue;
        }
        for (const int k : {r.kind, r.kind2}) {
            if (k < 0) continue;
            count[k] += 1;
            ms[k] += t;
            flops[k] += r.flops;
            bytes[k] += r.bytes;
        }
    }
    if (first != hipSuccess)
        return fg::set_error(FG_ERR_HIP, "%s failed: %s (records that could be timed are summed)", what,
                             hipGetErrorString(first));
    return fg::TK_COUNT;
}
