// KV-cache tiering: the cache of some GPU batches lives in pinned host memory
// and passes through two device slots.
//
// Method ("FlexGen 完全拆解", sections "三条关键数据通路如何重叠" and "一个层级
// 流水的伪代码"; bjbfmj.com walkthrough §6.4, load_cache / store_cache): while
// GPU batch k computes, the cache of batch k+1 is loaded and the new entries
// of the batch before are stored.  Here a "unit" is one host-resident GPU
// batch of one layer; the units of a call are numbered in execution order
// (layer by layer, batch by batch) and unit u uses slot u mod 2:
//   copy stream:    [u >= 2: wait stored[u mod 2]] load(u): rows [0, n) of
//                   every (sequence, head) of the unit's K, V (and metadata),
//                   host -> slot, as 2-D copies; record ready[u mod 2]
//   compute stream: wait ready[u mod 2]; the unit's kernel on the slot;
//                   record done[u mod 2]
//   store stream:   wait done[u mod 2]; store(u): the rows the kernel wrote,
//                   slot -> host; record stored[u mod 2]
// Loads are enqueued one unit ahead (load(u+1) before store(u)), so the copy
// stream moves the next batch's history while the current one computes;
// load(u+2) reuses the slot of u and waits until store(u), which itself
// waited for unit u's kernel, has read it.  Stores run on a stream of their
// own (device -> host traffic does not hold up the loads).  A call's first
// loads wait for every store of the calls before it (the store stream runs
// in order, so its latest two records cover them), which also orders each
// history load after the store of that history's last row.
#include <new>

#include "fg_internal.h"
#include "fg_trace.h"
#include "host_attn.h"

struct fg_kvtier {
    unsigned char* slot[2];
    size_t slot_bytes;
    hipStream_t cp;       // loads (the caller's copy stream)
    hipStream_t sp;       // stores (created here, default priority)
    hipEvent_t ready[2];
    hipEvent_t done[2];
    hipEvent_t stored[2];
    int device;
    // decode attention of the host batches on the host CPU (when hstage):
    // pinned staging, per lane of host batches [rows, 3 h1] (q, k, v in) then
    // [rows, h1] (attention out); the CPU threads; per lane the event that
    // marks the rows' arrival; the lanes' compute streams and the events that
    // order them against the caller's stream (start, lane 0 done, lane 1 done)
    unsigned char* hstage = nullptr;
    size_t hstage_bytes = 0;
    fg::HostPool* pool = nullptr;
    hipEvent_t hready[2] = {nullptr, nullptr};
    hipStream_t hs[2] = {nullptr, nullptr};
    hipEvent_t hev[3] = {nullptr, nullptr, nullptr};
};

namespace fg {
namespace {

// One cache of `nseq` sequences: the four tensors' byte offsets (codes of K,
// codes of V, metadata of K, of V), each 256-byte aligned, and their row sizes.
struct SlotLayout {
    size_t off[4];
    size_t row[4];
    size_t total;
};

SlotLayout slot_layout(const fg_dims* d, int32_t nseq, int32_t max_len, int32_t fmt) {
    SlotLayout L{};
    const size_t rows = (size_t)nseq * d->n_heads * max_len;
    const bool q4 = fmt == FG_FMT_Q4G64;
    const size_t code = q4 ? (size_t)d->head_dim / 2 : (size_t)d->head_dim * 2;
    const size_t meta = q4 ? (size_t)d->head_dim / 64 * 4 : 0;
    const size_t rs[4] = {code, code, meta, meta};
    size_t at = 0;
    for (int t = 0; t < 4; ++t) {
        L.off[t] = at;
        L.row[t] = rs[t];
        at += align_up(rows * rs[t], 256);
    }
    L.total = at;
    return L;
}

void* tensor_of(const fg_kv* kv, int t) {
    return t == 0 ? kv->k : t == 1 ? kv->v : t == 2 ? kv->k_meta : kv->v_meta;
}

}  // namespace

int kvtier_check(const fg_kvtier* kt, const fg_dims* d, const fg_kv* dev, const fg_kv* host,
                 int32_t gbs, int32_t n_host_seq, int32_t end_pos) {
    FG_CHECK_ARG(host, "KV tier: null host cache");
    FG_CHECK_ARG(host->fmt == dev->fmt, "KV tier: host cache format %d differs from the device's %d",
                 host->fmt, dev->fmt);
    FG_CHECK_ARG(host->k && host->v && (host->fmt != FG_FMT_Q4G64 || (host->k_meta && host->v_meta)),
                 "KV tier: null host cache tensors");
    FG_CHECK_ARG(host->n_seq >= n_host_seq, "KV tier: host cache holds %d sequences, %d needed",
                 host->n_seq, n_host_seq);
    FG_CHECK_ARG(end_pos <= host->max_len, "KV tier: position %d beyond the host cache's max_len %d",
                 end_pos - 1, host->max_len);
    FG_CHECK_ARG(kt, "KV tier: null tier object (fg_kvtier_create)");
    const size_t need = slot_layout(d, gbs, host->max_len, host->fmt).total;
    if (need > kt->slot_bytes)
        return set_error(FG_ERR_CAPACITY, "KV tier: slots of %zu bytes < %zu needed", kt->slot_bytes,
                         need);
    int cur = -1;
    FG_HIP(hipGetDevice(&cur));
    FG_CHECK_ARG(cur == kt->device, "KV tier created on device %d, called on %d", kt->device, cur);
    const int nt = host->fmt == FG_FMT_Q4G64 ? 4 : 2;
    for (int t = 0; t < nt; ++t) {
        hipPointerAttribute_t at{};
        if (hipPointerGetAttributes(&at, tensor_of(host, t)) != hipSuccess ||
            at.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return set_error(FG_ERR_INVALID, "KV tier: host cache must be pinned (hipHostMalloc)");
        }
    }
    return FG_OK;
}

KvPipe::KvPipe(fg_kvtier* kt, const fg_dims* d, int32_t gbs, int32_t load_rows, hipStream_t st)
    : kt_(kt), d_(d), gbs_(gbs), load_rows_(load_rows), st_(st) {}

void KvPipe::add(const fg_kv* host, int32_t seq0) { unit_.push_back(Unit{host, seq0}); }

fg_kv KvPipe::slot(int32_t u) const {
    const fg_kv* h = unit_[u].host;
    const SlotLayout L = slot_layout(d_, gbs_, h->max_len, h->fmt);
    unsigned char* b = kt_->slot[u & 1];
    fg_kv s{};
    s.fmt = h->fmt;
    s.k = b + L.off[0];
    s.v = b + L.off[1];
    s.k_meta = h->fmt == FG_FMT_Q4G64 ? b + L.off[2] : nullptr;
    s.v_meta = h->fmt == FG_FMT_Q4G64 ? b + L.off[3] : nullptr;
    s.max_len = h->max_len;
    s.n_seq = gbs_;
    return s;
}

// rows [lo, hi) of every (sequence, head) between unit u's host cache and its
// slot, as one 2-D copy per tensor
int KvPipe::copy(int32_t u, int32_t lo, int32_t hi, bool to_host) {
    if (hi <= lo) return FG_OK;
    const Unit& un = unit_[u];
    const fg_kv* h = un.host;
    const SlotLayout L = slot_layout(d_, gbs_, h->max_len, h->fmt);
    const int nt = h->fmt == FG_FMT_Q4G64 ? 4 : 2;
    const size_t height = (size_t)gbs_ * d_->n_heads;
    double bytes = 0;
    for (int t = 0; t < nt; ++t) bytes += (double)height * (hi - lo) * L.row[t];
    hipStream_t cs = to_host ? kt_->sp : kt_->cp;
    TraceScope ts(to_host ? TK_KV_D2H : TK_KV_H2D, cs, 0.0, bytes);
    for (int t = 0; t < nt; ++t) {
        const size_t r = L.row[t], pitch = (size_t)h->max_len * r;
        unsigned char* hp = static_cast<unsigned char*>(tensor_of(h, t)) +
                            (size_t)un.seq0 * d_->n_heads * pitch + (size_t)lo * r;
        unsigned char* dp = kt_->slot[u & 1] + L.off[t] + (size_t)lo * r;
        const size_t width = (size_t)(hi - lo) * r;
        if (to_host)
            FG_HIP(hipMemcpy2DAsync(hp, pitch, dp, pitch, width, height, hipMemcpyDeviceToHost, cs));
        else
            FG_HIP(hipMemcpy2DAsync(dp, pitch, hp, pitch, width, height, hipMemcpyHostToDevice, cs));
    }
    return FG_OK;
}

int KvPipe::begin(int32_t u, fg_kv* slot_out) {
    const int32_t n = (int32_t)unit_.size();
    FG_CHECK_ARG(u >= 0 && u < n && u == begun_, "KV tier: unit %d out of order", u);
    // loads through u + 1 (the next one runs while unit u computes); load(v)
    // for v >= 2 follows store(v - 2), enqueued by end(v - 2)
    if (loaded_ == 0) {   // every store of earlier calls before this call's loads
        FG_HIP(hipStreamWaitEvent(kt_->cp, kt_->stored[0], 0));
        FG_HIP(hipStreamWaitEvent(kt_->cp, kt_->stored[1], 0));
    }
    while (loaded_ <= u + 1 && loaded_ < n) {
        FG_CHECK_ARG(loaded_ < 2 || stored_ >= loaded_ - 1, "KV tier: slot of unit %d still in use",
                     loaded_);
        if (loaded_ >= 2) FG_HIP(hipStreamWaitEvent(kt_->cp, kt_->stored[loaded_ & 1], 0));
        FG_TRY(copy(loaded_, 0, load_rows_, false));
        FG_HIP(hipEventRecord(kt_->ready[loaded_ & 1], kt_->cp));
        ++loaded_;
    }
    FG_HIP(hipStreamWaitEvent(st_, kt_->ready[u & 1], 0));
    *slot_out = slot(u);
    begun_ = u + 1;
    return FG_OK;
}

int KvPipe::end(int32_t u, int32_t lo, int32_t hi) {
    FG_CHECK_ARG(u == stored_ && u < begun_, "KV tier: unit %d ended out of order", u);
    FG_HIP(hipEventRecord(kt_->done[u & 1], st_));
    FG_HIP(hipStreamWaitEvent(kt_->sp, kt_->done[u & 1], 0));
    FG_TRY(copy(u, lo, hi, true));
    FG_HIP(hipEventRecord(kt_->stored[u & 1], kt_->sp));
    ++stored_;
    return FG_OK;
}

// ------------------------------------------------ host-CPU attention path
bool kvtier_host_attention_on(const fg_kvtier* kt) { return kt && kt->hstage; }

size_t host_stage_bytes(const fg_dims* d, int64_t rows) {
    return align_up((size_t)rows * 4 * (size_t)d->h1 * 2, 256);
}

int kvtier_host_check(const fg_kvtier* kt, const fg_kv* host, const fg_dims* d, int64_t rows,
                      int32_t topk) {
    FG_CHECK_SUP(topk < 0, "host attention computes dense attention only (no Top-K sparse V)");
    const size_t need = host_stage_bytes(d, rows);
    if (kt->hstage_bytes < need)
        return set_error(FG_ERR_CAPACITY, "host attention: stage of %zu bytes < %zu needed", kt->hstage_bytes,
                         need);
    return FG_OK;
}

int kvtier_host_send(const fg_kvtier* kt, int lane, size_t off, const __half* qkv, int64_t rows, int64_t h1,
                     hipStream_t st) {
    FG_HIP(hipMemcpyAsync(kt->hstage + off, qkv, (size_t)rows * 3 * h1 * 2, hipMemcpyDeviceToHost, st));
    FG_HIP(hipEventRecord(kt->hready[lane], st));
    return FG_OK;
}

int kvtier_host_attend(const fg_kvtier* kt, int lane, size_t off, const fg_kv* host, int32_t seq0,
                       const fg_dims* d, int64_t rows, int32_t pos, __half* out, hipStream_t st) {
    // the host cache's rows stored by earlier calls (the prefill's) and this
    // layer's q, k, v rows must have landed before the CPU reads them
    FG_HIP(hipEventSynchronize(kt->stored[0]));
    FG_HIP(hipEventSynchronize(kt->stored[1]));
    FG_HIP(hipEventSynchronize(kt->hready[lane]));
    const int64_t h1 = d->h1;
    const uint16_t* qkv = reinterpret_cast<const uint16_t*>(kt->hstage + off);
    uint16_t* o = reinterpret_cast<uint16_t*>(kt->hstage + off) + rows * 3 * h1;
    FG_TRY(host_attn_decode(qkv, 3 * h1, host, seq0, (int32_t)rows, d, pos, true, o, *kt->pool));
    FG_HIP(hipMemcpyAsync(out, o, (size_t)rows * h1 * 2, hipMemcpyHostToDevice, st));
    return FG_OK;
}

size_t kvtier_host_stage_capacity(const fg_kvtier* kt) { return kt->hstage_bytes; }

void kvtier_host_lanes(const fg_kvtier* kt, hipStream_t* lane_streams, hipEvent_t* events) {
    lane_streams[0] = kt->hs[0];
    lane_streams[1] = kt->hs[1];
    for (int i = 0; i < 3; ++i) events[i] = kt->hev[i];
}

}  // namespace fg

// -------------------------------------------------------------------- C ABI
extern "C" size_t fg_kvtier_slot_bytes(const fg_dims* d, int32_t gbs, int32_t max_len, int32_t fmt) {
    if (fg::check_dims(d) != FG_OK || gbs < 1 || max_len < 1 ||
        (fmt != FG_FMT_F16 && fmt != FG_FMT_Q4G64)) {
        fg::clear_error();
        return 0;
    }
    return fg::slot_layout(d, gbs, max_len, fmt).total;
}

extern "C" int fg_kvtier_create(fg_kvtier** out, void* slots, size_t slot_bytes, void* copy_stream) {
    fg::clear_error();
    FG_CHECK_ARG(out && slots && slot_bytes > 0, "null pointer or empty slots");
    FG_CHECK_ARG((uintptr_t)slots % 256 == 0 && slot_bytes % 256 == 0,
                 "slots must be 256-byte aligned and a multiple of 256 bytes");
    FG_CHECK_ARG(copy_stream, "KV tier needs a copy stream (not the null stream)");
    *out = nullptr;
    fg_kvtier* kt = new (std::nothrow) fg_kvtier();
    FG_CHECK_ARG(kt, "out of host memory");
    kt->slot[0] = static_cast<unsigned char*>(slots);
    kt->slot[1] = static_cast<unsigned char*>(slots) + slot_bytes;
    kt->slot_bytes = slot_bytes;
    kt->cp = fg::as_stream(copy_stream);
    hipEvent_t* ev[6] = {&kt->ready[0], &kt->ready[1], &kt->done[0],
                         &kt->done[1], &kt->stored[0], &kt->stored[1]};
    int made = 0;
    bool ok = hipGetDevice(&kt->device) == hipSuccess;
    while (ok && made < 6) {
        if (hipEventCreateWithFlags(ev[made], hipEventDisableTiming) != hipSuccess) ok = false;
        else ++made;
    }
    bool have_sp = ok && hipStreamCreateWithFlags(&kt->sp, hipStreamNonBlocking) == hipSuccess;
    // the first call's loads wait for these (complete at once)
    if (have_sp && (hipEventRecord(kt->stored[0], kt->sp) != hipSuccess ||
                    hipEventRecord(kt->stored[1], kt->sp) != hipSuccess)) {
        (void)hipStreamDestroy(kt->sp);
        have_sp = false;
    }
    if (!have_sp) {
        for (int i = 0; i < made; ++i) (void)hipEventDestroy(*ev[i]);
        delete kt;
        return fg::set_error(FG_ERR_HIP, "fg_kvtier_create: %s", hipGetErrorString(hipGetLastError()));
    }
    *out = kt;
    return FG_OK;
}

extern "C" size_t fg_kvtier_host_stage_bytes(const fg_dims* d, int32_t n_host_seq) {
    if (fg::check_dims(d) != FG_OK || n_host_seq < 1) {
        fg::clear_error();
        return 0;
    }
    return fg::host_stage_bytes(d, n_host_seq);
}

extern "C" int fg_kvtier_host_attention(fg_kvtier* kt, void* stage, size_t stage_bytes, int32_t n_threads) {
    fg::clear_error();
    FG_CHECK_ARG(kt, "null tier object");
    if (!stage) {
        delete kt->pool;
        kt->pool = nullptr;
        kt->hstage = nullptr;
        kt->hstage_bytes = 0;
        return FG_OK;
    }
    FG_CHECK_ARG(stage_bytes > 0, "empty stage");
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, stage) != hipSuccess || at.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fg::set_error(FG_ERR_INVALID, "host attention: the stage must be pinned host memory");
    }
    for (int i = 0; i < 2; ++i) {
        if (!kt->hready[i]) FG_HIP(hipEventCreateWithFlags(&kt->hready[i], hipEventDisableTiming));
        if (!kt->hs[i]) FG_HIP(hipStreamCreateWithFlags(&kt->hs[i], hipStreamNonBlocking));
    }
    for (int i = 0; i < 3; ++i)
        if (!kt->hev[i]) FG_HIP(hipEventCreateWithFlags(&kt->hev[i], hipEventDisableTiming));
    fg::HostPool* pool = nullptr;
    try {
        pool = new fg::HostPool(n_threads);
    } catch (const std::bad_alloc&) {
        return fg::set_error(FG_ERR_CAPACITY, "host attention: out of host memory");
    }
    delete kt->pool;
    kt->pool = pool;
    kt->hstage = static_cast<unsigned char*>(stage);
    kt->hstage_bytes = stage_bytes;
    return FG_OK;
}

extern "C" int fg_kvtier_destroy(fg_kvtier* kt) {
    fg::clear_error();
    if (!kt) return FG_OK;
    delete kt->pool;
    for (int i = 0; i < 2; ++i) {
        if (kt->hready[i]) (void)hipEventDestroy(kt->hready[i]);
        if (kt->hs[i]) {
            (void)hipStreamSynchronize(kt->hs[i]);
            (void)hipStreamDestroy(kt->hs[i]);
        }
    }
    for (int i = 0; i < 3; ++i)
        if (kt->hev[i]) (void)hipEventDestroy(kt->hev[i]);
    (void)hipStreamSynchronize(kt->sp);
    (void)hipStreamDestroy(kt->sp);
    for (int i = 0; i < 2; ++i) {
        (void)hipEventDestroy(kt->ready[i]);
        (void)hipEventDestroy(kt->done[i]);
        (void)hipEventDestroy(kt->stored[i]);
    }
    delete kt;
    return FG_OK;
}
