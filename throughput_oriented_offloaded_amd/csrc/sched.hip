// Block schedule over all layers of one pass, with optional weight tiering.
//
// Method ("FlexGen 完全拆解", sections "一个层级流水的伪代码" and "三条关键数据
// 通路如何重叠"; bjbfmj.com walkthrough §6.4): one layer's weights are resident
// while every GPU batch of the block passes through it; the weights of the
// next layer are moved while the current layer computes.  Here the moved part
// is the host-resident half of a layer's fp16 weights (W_Q, W_K rows and W_1
// in pinned host memory), copied by hipMemcpyAsync on a side stream into one
// of two device stage buffers.  Per tiered layer t (in layer order, buffer
// b = t mod 2):
//   copy stream:    wait released[b]; H2D [W_Q; W_K] -> stage[b].qkv rows
//                   0..2h1; D2D W_V -> rows 2h1..3h1; H2D W_1 -> stage[b].w1;
//                   record staged[b]
//   compute stream: wait staged[b]; the layer on stage[b]; record released[b]
// The copy of tiered layer t+2 is issued right after layer t has been
// enqueued, so it runs while layer t+1 computes.  released[] is recorded on
// the compute stream at the start of every call, so the first copies of a
// call never overwrite a buffer that earlier work still reads.
#include <new>
#include <vector>

#include "fg_internal.h"
#include "fg_trace.h"

struct fg_sched {
    unsigned char* stage[2];
    size_t stage_bytes;
    hipEvent_t staged[2];
    hipEvent_t released[2];
    int device;
};

namespace fg {
namespace {

size_t qkv_stage_bytes(const fg_dims* d) {
    return align_up((size_t)3 * d->h1 * d->h1 * 2, 256);
}

int check_tier(const fg_dims* d, int32_t n, const fg_layer_w* w, const fg_tier_w* tier) {
    for (int32_t j = 0; j < n; ++j) {
        const fg_tier_w& t = tier[j];
        if (!t.qk_host) {
            FG_CHECK_ARG(!t.v_dev && !t.w1_host, "layer %d: partial tier entry", j);
            continue;
        }
        FG_CHECK_SUP(w[j].fmt == FG_FMT_F16, "layer %d: weight tiering needs fp16 weights", j);
        FG_CHECK_ARG(t.v_dev && t.w1_host, "layer %d: null tier pointer", j);
        FG_CHECK_ARG(((uintptr_t)t.qk_host | (uintptr_t)t.v_dev | (uintptr_t)t.w1_host) % 16 == 0,
                     "layer %d: tier tensors must be 16-byte aligned", j);
        for (const void* hp : {t.qk_host, t.w1_host}) {
            hipPointerAttribute_t at{};
            if (hipPointerGetAttributes(&at, hp) != hipSuccess || at.type != hipMemoryTypeHost) {
                (void)hipGetLastError();
                return set_error(FG_ERR_INVALID, "layer %d: host weights must be pinned (hipHostMalloc)", j);
            }
        }
    }
    (void)d;
    return FG_OK;
}

// Runs `layer(j, w_j, check_only)` for every layer, staging tiered layers as
// described above.  Every layer is validated before anything is enqueued
// (tiered layers with their stage pointers in place).
template <class F>
int run_layers(fg_sched* sc, const fg_dims* d, int32_t n, const fg_layer_w* w,
               const fg_tier_w* tier, hipStream_t st, hipStream_t cp, int32_t flags, F&& layer) {
    if (!tier) {
        for (int32_t j = 0; j < n; ++j) FG_TRY(layer(j, w[j], true));
        for (int32_t j = 0; j < n; ++j) FG_TRY(layer(j, w[j], false));
        return FG_OK;
    }
    FG_CHECK_ARG(sc, "weight tiering needs a scheduler (fg_sched_create)");
    FG_CHECK_ARG(cp && cp != st, "weight tiering needs a copy stream distinct from the compute stream");
    FG_CHECK_ARG(fg_stage_bytes(d) <= sc->stage_bytes, "stage buffers of %zu bytes < %zu needed",
                 sc->stage_bytes, fg_stage_bytes(d));
    FG_TRY(check_tier(d, n, w, tier));
    int cur_dev = -1;
    FG_HIP(hipGetDevice(&cur_dev));
    FG_CHECK_ARG(cur_dev == sc->device, "scheduler created on device %d, called on %d", sc->device,
                 cur_dev);

    std::vector<int32_t> tl;   // tiered layers in order
    for (int32_t j = 0; j < n; ++j)
        if (tier[j].qk_host) tl.push_back(j);
    const size_t qkv_b = qkv_stage_bytes(d);
    for (int32_t j = 0, t = 0; j < n; ++j) {
        fg_layer_w wj = w[j];
        if (t < (int32_t)tl.size() && tl[t] == j) {
            wj.w_qkv = sc->stage[t & 1];
            wj.w_1 = sc->stage[t & 1] + qkv_b;
            ++t;
        }
        FG_TRY(layer(j, wj, true));
    }
    const size_t qk_bytes = (size_t)2 * d->h1 * d->h1 * 2, v_bytes = (size_t)d->h1 * d->h1 * 2;
    const size_t w1_bytes = (size_t)d->h2 * d->h1 * 2;
    auto stage_copy = [&](int32_t t) -> int {   // t: index into tl
        const int b = t & 1;
        const fg_tier_w& tw = tier[tl[t]];
        unsigned char* base = sc->stage[b];
        FG_HIP(hipStreamWaitEvent(cp, sc->released[b], 0));
        {
            // traced as host -> device bytes (the device-resident W_V rows
            // moved beside them are a few percent of the time)
            TraceScope ts(TK_W_H2D, cp, 0.0, (double)(qk_bytes + w1_bytes));
            FG_HIP(hipMemcpyAsync(base, tw.qk_host, qk_bytes, hipMemcpyHostToDevice, cp));
            FG_HIP(hipMemcpyAsync(base + qk_bytes, tw.v_dev, v_bytes, hipMemcpyDeviceToDevice, cp));
            FG_HIP(hipMemcpyAsync(base + qkv_b, tw.w1_host, w1_bytes, hipMemcpyHostToDevice, cp));
        }
        FG_HIP(hipEventRecord(sc->staged[b], cp));
        return FG_OK;
    };

    // buffers are free once the compute stream's earlier work is done
    if (!(flags & FG_SCHED_FIRST_STAGED)) {
        FG_HIP(hipEventRecord(sc->released[0], st));
    }
    FG_HIP(hipEventRecord(sc->released[1], st));
    const int32_t T = (int32_t)tl.size();
    if (T > 0 && !(flags & FG_SCHED_FIRST_STAGED)) FG_TRY(stage_copy(0));
    if (T > 1) FG_TRY(stage_copy(1));

    int32_t t = 0;
    for (int32_t j = 0; j < n; ++j) {
        if (t < T && tl[t] == j) {
            const int b = t & 1;
            fg_layer_w wj = w[j];
            wj.w_qkv = sc->stage[b];
            wj.w_1 = sc->stage[b] + qkv_b;
            FG_HIP(hipStreamWaitEvent(st, sc->staged[b], 0));
            FG_TRY(layer(j, wj, false));
            FG_HIP(hipEventRecord(sc->released[b], st));
            if (t + 2 < T) FG_TRY(stage_copy(t + 2));
            ++t;
        } else {
            FG_TRY(layer(j, w[j], false));
        }
    }
    // the next call's first tiered layer goes to buffer 0
    if (T > 0 && (flags & FG_SCHED_STAGE_NEXT)) FG_TRY(stage_copy(0));
    return FG_OK;
}

// The host batches of every layer of a KV-tiered call, in execution order:
// layer j's batch k (k >= nb_dev) is unit j * (nb - nb_dev) + k - nb_dev.
int kv_units(const fg_kv_tier* kvt, int32_t n_layers, int32_t gbs, int32_t nb, KvPipe& pipe) {
    if (!kvt) return FG_OK;
    FG_CHECK_ARG(kvt->host, "KV tier: null host cache array");
    FG_CHECK_ARG(kvt->nb_dev >= 0 && kvt->nb_dev <= nb, "KV tier: nb_dev %d outside [0, nb %d]",
                 kvt->nb_dev, nb);
    for (int32_t j = 0; j < n_layers; ++j)
        for (int32_t k = kvt->nb_dev; k < nb; ++k) pipe.add(&kvt->host[j], (k - kvt->nb_dev) * gbs);
    return FG_OK;
}

KvTierCall kv_call(const fg_kv_tier* kvt, KvPipe* pipe, int32_t j, int32_t nb) {
    if (!kvt) return KvTierCall{};
    return KvTierCall{pipe, kvt->pipe, &kvt->host[j], kvt->nb_dev, j * (nb - kvt->nb_dev)};
}

}  // namespace
}  // namespace fg

extern "C" size_t fg_stage_bytes(const fg_dims* d) {
    if (!d || d->h1 <= 0 || d->h2 <= 0) return 0;
    return fg::qkv_stage_bytes(d) + fg::align_up((size_t)d->h2 * d->h1 * 2, 256);
}

extern "C" int fg_sched_create(fg_sched** out, void* stage, size_t stage_bytes) {
    fg::clear_error();
    FG_CHECK_ARG(out && stage && stage_bytes > 0, "null pointer or empty stage");
    FG_CHECK_ARG((uintptr_t)stage % 256 == 0 && stage_bytes % 256 == 0,
                 "stage must be 256-byte aligned and a multiple of 256 bytes");
    *out = nullptr;
    fg_sched* sc = new (std::nothrow) fg_sched();
    FG_CHECK_ARG(sc, "out of host memory");
    sc->stage[0] = static_cast<unsigned char*>(stage);
    sc->stage[1] = static_cast<unsigned char*>(stage) + stage_bytes;
    sc->stage_bytes = stage_bytes;
    int rc = FG_OK;
    int made = 0;
    if (hipGetDevice(&sc->device) != hipSuccess) rc = FG_ERR_HIP;
    for (int i = 0; i < 2 && rc == FG_OK; ++i) {
        if (hipEventCreateWithFlags(&sc->staged[i], hipEventDisableTiming) != hipSuccess) { rc = FG_ERR_HIP; break; }
        ++made;
        if (hipEventCreateWithFlags(&sc->released[i], hipEventDisableTiming) != hipSuccess) { rc = FG_ERR_HIP; break; }
        ++made;
    }
    if (rc != FG_OK) {
        for (int i = 0; i < made; ++i) (void)hipEventDestroy(i % 2 == 0 ? sc->staged[i / 2] : sc->released[i / 2]);
        delete sc;
        return fg::set_error(FG_ERR_HIP, "fg_sched_create: %s", hipGetErrorString(hipGetLastError()));
    }
    *out = sc;
    return FG_OK;
}

extern "C" int fg_sched_destroy(fg_sched* sc) {
    fg::clear_error();
    if (!sc) return FG_OK;
    for (int i = 0; i < 2; ++i) {
        (void)hipEventDestroy(sc->staged[i]);
        (void)hipEventDestroy(sc->released[i]);
    }
    delete sc;
    return FG_OK;
}

extern "C" int fg_model_prefill(fg_sched* sc, const fg_dims* d, int32_t n_layers,
                                const fg_layer_w* w, const fg_tier_w* tier, const fg_kv* kv,
                                void* x, int32_t gbs, int32_t nb, int32_t s, void* ws,
                                size_t ws_bytes, void* stream, void* copy_stream, int32_t flags,
                                const fg_kv_tier* kvt) {
    using namespace fg;
    clear_error();
    FG_TRY(check_dims(d));
    FG_CHECK_ARG(n_layers >= 1 && w && kv, "need n_layers >= 1 and layer arrays");
    hipStream_t st = as_stream(stream);
    KvPipe pipe(kvt ? kvt->pipe : nullptr, d, gbs, 0, st);
    FG_TRY(kv_units(kvt, n_layers, gbs, nb, pipe));
    return run_layers(sc, d, n_layers, w, tier, st, as_stream(copy_stream), flags,
                      [&](int32_t j, const fg_layer_w& wj, bool chk) {
                          const KvTierCall kc = kv_call(kvt, chk ? nullptr : &pipe, j, nb);
                          return layer_prefill(d, &wj, x, gbs, nb, s, &kv[j], ws, ws_bytes, st, chk,
                                               kvt ? &kc : nullptr);
                      });
}

extern "C" int fg_model_decode_step(fg_sched* sc, const fg_dims* d, int32_t n_layers,
                                    const fg_layer_w* w, const fg_tier_w* tier, const fg_kv* kv,
                                    void* x, int32_t gbs, int32_t nb, int32_t pos, void* ws,
                                    size_t ws_bytes, void* stream, void* copy_stream,
                                    int32_t flags, int32_t attn_topk_ppm, const fg_kv_tier* kvt) {
    using namespace fg;
    clear_error();
    FG_TRY(check_dims(d));
    FG_CHECK_ARG(n_layers >= 1 && w && kv, "need n_layers >= 1 and layer arrays");
    hipStream_t st = as_stream(stream);
    // host batches attended by the host CPU, no weight tiering: the CPU's
    // attention overlapped with the GPU's work on the other rows
    if (!tier && kvt && kvt->host && kvt->nb_dev >= 0 && kvt->nb_dev < nb && kvtier_host_attention_on(kvt->pipe) &&
        attn_topk_count(pos, attn_topk_ppm) < 0) {
        bool used = false;
        FG_TRY(model_decode_host_overlap(d, n_layers, w, kv, x, gbs, nb, pos, ws, ws_bytes, st, kvt, &used));
        if (used) return FG_OK;
    }
    KvPipe pipe(kvt ? kvt->pipe : nullptr, d, gbs, pos, st);
    FG_TRY(kv_units(kvt, n_layers, gbs, nb, pipe));
    return run_layers(sc, d, n_layers, w, tier, st, as_stream(copy_stream), flags,
                      [&](int32_t j, const fg_layer_w& wj, bool chk) {
                          // each layer's input LayerNorm runs fused into the
                          // previous layer's last residual sum
                          const KvTierCall kc = kv_call(kvt, chk ? nullptr : &pipe, j, nb);
                          return layer_decode(d, &wj, x, gbs, nb, pos, &kv[j], ws, ws_bytes, st, chk,
                                              j > 0, j + 1 < n_layers ? &w[j + 1] : nullptr,
                                              attn_topk_ppm, kvt ? &kc : nullptr);
                      });
}

extern "C" int fg_prefetch(void* dst_dev, const void* src_pinned, size_t bytes, void* copy_stream,
                           void* done) {
    using namespace fg;
    clear_error();
    FG_CHECK_ARG(bytes == 0 || (dst_dev && src_pinned), "null pointer argument");
    hipStream_t cp = as_stream(copy_stream);
    if (bytes > 0) {
        hipPointerAttribute_t as{}, ad{};
        if (hipPointerGetAttributes(&as, src_pinned) != hipSuccess || as.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return set_error(FG_ERR_INVALID, "fg_prefetch: the source must be pinned host memory (hipHostMalloc)");
        }
        if (hipPointerGetAttributes(&ad, dst_dev) != hipSuccess || ad.type != hipMemoryTypeDevice) {
            (void)hipGetLastError();
            return set_error(FG_ERR_INVALID, "fg_prefetch: the destination must be device memory");
        }
        TraceScope ts(TK_W_H2D, cp, 0.0, (double)bytes);
        FG_HIP(hipMemcpyAsync(dst_dev, src_pinned, bytes, hipMemcpyHostToDevice, cp));
    }
    if (done) FG_HIP(hipEventRecord(static_cast<hipEvent_t>(done), cp));
    return FG_OK;
}
