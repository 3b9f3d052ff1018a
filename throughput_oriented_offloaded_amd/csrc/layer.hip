// One decoder layer, prefill and decode-block forms.
//
// Pre-LN OPT-style layer: x += Attn(LN1(x)) W_O^T + b_O; x += ReLU(LN2(x)
// W_1^T + b_1) W_2^T + b_2, with K, V kept in the per-layer cache ("FlexGen
// 完全拆解", section "从 Transformer 推理的数据流重新定义卸载").
//
// Block schedule (section "FlexGen 的核心:计算图分块与张量生命周期" and the
// pipeline pseudocode of section "一个层级流水的伪代码"): while one layer's
// weights are resident, every GPU batch of the block passes through it.  Here
// the weights live in HBM; the decode block issues each projection once over
// all bls = gbs * nb rows, so every weight byte is read once per layer per
// step for the whole block.  The prefill walks the block's GPU batches one at
// a time (workspace bounded by one GPU batch of gbs * s rows).
#include <string>
#include <system_error>
#include <thread>

#include "fg_internal.h"

namespace fg {
namespace {

struct WsLayout {
    size_t a, qkv, o, f, part, wdq, total;
};

// fp16 copies of a 4-bit layer's four weight matrices for the prefill-shaped
// GEMMs (the large-M fp16 kernel).
bool prefill_dequant(int64_t rows, int32_t fmt) { return fmt == FG_FMT_Q4G64 && linear_is_dp(rows); }
size_t wdq_elems(const fg_dims* d) {
    const size_t h1 = d->h1, h2 = d->h2;
    return 3 * h1 * h1 + h1 * h1 + 2 * h2 * h1;
}

size_t part_bytes(const fg_dims* d, int64_t rows, int32_t fmt) {
    const int64_t h1 = d->h1, h2 = d->h2;
    size_t m = 0;
    m = std::max(m, linear_ws_bytes(rows, 3 * h1, h1, fmt));
    m = std::max(m, linear_ws_bytes(rows, h1, h1, fmt));
    m = std::max(m, linear_ws_bytes(rows, h2, h1, fmt));
    m = std::max(m, linear_ws_bytes(rows, h1, h2, fmt));
    return m;
}

WsLayout layout(const fg_dims* d, int64_t rows, int32_t fmt) {
    WsLayout L{};
    const size_t A = 256;
    size_t off = 0;
    L.a = off;   off = align_up(off + (size_t)rows * d->h1 * 2, A);
    L.qkv = off; off = align_up(off + (size_t)rows * 3 * d->h1 * 2, A);
    L.o = off;   off = align_up(off + (size_t)rows * d->h1 * 2, A);
    L.f = off;   off = align_up(off + (size_t)rows * d->h2 * 2, A);
    L.part = off;
    off = align_up(off + part_bytes(d, rows, fmt), A);
    L.wdq = off;
    if (prefill_dequant(rows, fmt)) off = align_up(off + wdq_elems(d) * 2, A);
    L.total = off;
    return L;
}

int check_layer(const fg_dims* d, const fg_layer_w* w, const void* x, const fg_kv* kv,
                const void* ws) {
    FG_TRY(check_dims(d));
    FG_CHECK_ARG(w && x && kv && ws, "null pointer argument");
    FG_CHECK_ARG(w->fmt == FG_FMT_F16 || w->fmt == FG_FMT_Q4G64, "unknown weight format %d",
                 w->fmt);
    FG_CHECK_ARG(w->w_qkv && w->b_qkv && w->w_o && w->b_o && w->w_1 && w->b_1 && w->w_2 &&
                     w->b_2 && w->ln1_g && w->ln1_b && w->ln2_g && w->ln2_b,
                 "null weight pointer");
    FG_CHECK_ARG(w->fmt != FG_FMT_Q4G64 || (w->m_qkv && w->m_o && w->m_1 && w->m_2),
                 "null 4-bit weight metadata");
    FG_CHECK_ARG(kv->fmt == FG_FMT_F16 || kv->fmt == FG_FMT_Q4G64, "unknown cache format %d",
                 kv->fmt);
    FG_CHECK_ARG(kv->k && kv->v && (kv->fmt != FG_FMT_Q4G64 || (kv->k_meta && kv->v_meta)),
                 "null cache tensors");
    const uintptr_t al = (uintptr_t)x | (uintptr_t)ws | (uintptr_t)w->w_qkv | (uintptr_t)w->w_o |
                         (uintptr_t)w->w_1 | (uintptr_t)w->w_2 | (uintptr_t)w->ln1_g |
                         (uintptr_t)w->ln1_b | (uintptr_t)w->ln2_g | (uintptr_t)w->ln2_b |
                         (uintptr_t)kv->k | (uintptr_t)kv->v | (uintptr_t)w->m_qkv |
                         (uintptr_t)w->m_o | (uintptr_t)w->m_1 | (uintptr_t)w->m_2;
    FG_CHECK_ARG(al % 16 == 0, "tensors must be 16-byte aligned");
    FG_CHECK_ARG(((uintptr_t)w->b_qkv | (uintptr_t)w->b_o | (uintptr_t)w->b_1 |
                  (uintptr_t)w->b_2) % 8 == 0, "biases must be 8-byte aligned");
    FG_CHECK_ARG(((uintptr_t)kv->k_meta | (uintptr_t)kv->v_meta) % 4 == 0,
                 "cache metadata must be 4-byte aligned");
    return FG_OK;
}

// ln_g / ln_b / ln_y: optional LayerNorm of the output rows (fused with the
// split-k sum when the GEMM has one); dq: bit `which` set when that matrix's
// pointer holds an fp16 copy of 4-bit weights
int lin(const fg_layer_w* w, int which, const __half* x, int64_t M, int64_t K, int64_t N,
        int32_t act, const __half* res, __half* y, void* part, size_t part_bytes, hipStream_t st,
        const void* ln_g = nullptr, const void* ln_b = nullptr, __half* ln_y = nullptr,
        unsigned dq = 0) {
    LinearArgs a{};
    a.x = x; a.M = M; a.K = K; a.ldx = K; a.fmt = w->fmt; a.N = N; a.act = act;
    if (dq & (1 << which)) a.fmt = FG_FMT_F16;   // restored to fp16 for this call
    a.residual = res; a.y = y; a.ldy = N; a.ws = part; a.ws_bytes = part_bytes;
    a.ln_g = (const __half*)ln_g; a.ln_b = (const __half*)ln_b; a.ln_y = ln_y;
    a.proj = which + 1;
    switch (which) {
        case 0: a.w = w->w_qkv; a.meta = (const __half*)w->m_qkv; a.bias = (const __half*)w->b_qkv; break;
        case 1: a.w = w->w_o; a.meta = (const __half*)w->m_o; a.bias = (const __half*)w->b_o; break;
        case 2: a.w = w->w_1; a.meta = (const __half*)w->m_1; a.bias = (const __half*)w->b_1; break;
        default: a.w = w->w_2; a.meta = (const __half*)w->m_2; a.bias = (const __half*)w->b_2; break;
    }
    return launch_linear(a, st);
}

// The block's sequences against the device cache and, with a KV tier, the
// host cache; positions below end_pos must fit.
int check_block(const fg_dims* d, const fg_kv* kv, int32_t gbs, int32_t nb, int32_t end_pos,
                const KvTierCall* kvt) {
    FG_CHECK_ARG(gbs >= 1 && nb >= 1, "block %d x %d is empty", gbs, nb);
    const int32_t nd = kvt ? kvt->nb_dev : nb;
    if (kvt) FG_CHECK_ARG(nd >= 0 && nd <= nb, "KV tier: nb_dev %d outside [0, nb %d]", nd, nb);
    FG_CHECK_ARG(end_pos >= 1, "position %d is negative", end_pos - 1);
    if (nd > 0) {   // the device cache is not read when every batch is on the host
        FG_CHECK_ARG((int64_t)gbs * nd <= kv->n_seq,
                     "block %d x %d exceeds the cache's %d sequences", gbs, nd, kv->n_seq);
        FG_CHECK_ARG(end_pos <= kv->max_len, "position %d outside [0, max_len %d)", end_pos - 1,
                     kv->max_len);
    }
    if (kvt && nd < nb)
        FG_TRY(kvtier_check(kvt->kt, d, kv, kvt->host, gbs, (nb - nd) * gbs, end_pos));
    return FG_OK;
}

// The buffers of one decode call's workspace.
struct DecWs {
    __half *a, *qkv, *o, *f;
    void* part;
    size_t pb;
};
DecWs dec_ws(void* ws, const WsLayout& L) {
    unsigned char* base = static_cast<unsigned char*>(ws);
    return DecWs{(__half*)(base + L.a), (__half*)(base + L.qkv), (__half*)(base + L.o), (__half*)(base + L.f),
                 base + L.part, L.wdq - L.part};
}

// A decode layer up to its attention: LN1 (unless the previous layer fused
// it into the workspace) and the QKV projection of `rows` rows of x.
int dec_pre(const fg_dims* d, const fg_layer_w* w, __half* xh, int64_t rows, const DecWs& b, hipStream_t st,
            bool ln1_done) {
    const int64_t h1 = d->h1;
    if (!ln1_done)
        FG_TRY(launch_layernorm(xh, rows, h1, (const __half*)w->ln1_g, (const __half*)w->ln1_b, b.a, st));
    return lin(w, 0, b.a, rows, h1, 3 * h1, 0, nullptr, b.qkv, b.part, b.pb, st);
}

// A decode layer after its attention (rows in b.o): out-projection + residual
// with LN2 fused, FC1 + ReLU, FC2 + residual (with the next layer's LN1
// fused when `next`).
int dec_post(const fg_dims* d, const fg_layer_w* w, __half* xh, int64_t rows, const DecWs& b, hipStream_t st,
             const fg_layer_w* next) {
    const int64_t h1 = d->h1, h2 = d->h2;
    FG_TRY(lin(w, 1, b.o, rows, h1, h1, 0, xh, xh, b.part, b.pb, st, w->ln2_g, w->ln2_b, b.a));
    FG_TRY(lin(w, 2, b.a, rows, h1, h2, 1, nullptr, b.f, b.part, b.pb, st));
    if (next) return lin(w, 3, b.f, rows, h2, h1, 0, xh, xh, b.part, b.pb, st, next->ln1_g, next->ln1_b, b.a);
    return lin(w, 3, b.f, rows, h2, h1, 0, xh, xh, b.part, b.pb, st);
}

}  // namespace

// Positions whose V a sparse step reads: the fraction ppm / 1e6 of the
// history, rounded up; dense (-1) when that is the whole history.
int32_t attn_topk_count(int32_t pos, int32_t ppm) {
    if (ppm <= 0 || ppm >= 1000000) return -1;
    const int64_t k = ((int64_t)pos * ppm + 999999) / 1000000;
    return k < pos ? (int32_t)k : -1;
}

int layer_decode(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs, int32_t nb,
                 int32_t pos, const fg_kv* kv, void* ws, size_t ws_bytes, hipStream_t st,
                 bool check_only, bool ln1_done, const fg_layer_w* next, int32_t attn_topk_ppm,
                 const KvTierCall* kvt) {
    FG_TRY(check_layer(d, w, x, kv, ws));
    FG_TRY(check_block(d, kv, gbs, nb, pos + 1, kvt));
    FG_CHECK_ARG(attn_topk_ppm >= 0, "attn_topk_ppm %d is negative", attn_topk_ppm);
    const int32_t topk = attn_topk_count(pos, attn_topk_ppm);
    FG_CHECK_SUP(topk < 0 || pos <= kAttnTopkMaxPos, "Top-K attention: history %d longer than %d",
                 pos, kAttnTopkMaxPos);
    const int64_t bls = (int64_t)gbs * nb;
    // host batches' attention on the host CPU (the tier's choice)
    const bool host_attn = kvt && kvt->nb_dev < nb && kvtier_host_attention_on(kvt->kt);
    if (host_attn) FG_TRY(kvtier_host_check(kvt->kt, kvt->host, d, (int64_t)(nb - kvt->nb_dev) * gbs, topk));
    const WsLayout L = layout(d, bls, w->fmt);
    if (ws_bytes < L.total)
        return set_error(FG_ERR_CAPACITY, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
    if (check_only) return FG_OK;
    const DecWs b = dec_ws(ws, L);
    __half* qkv = b.qkv;
    __half* o = b.o;
    __half* xh = (__half*)x;
    const int64_t h1 = d->h1;

    FG_TRY(dec_pre(d, w, xh, bls, b, st, ln1_done));
    // GPU batches with a device-resident cache in one launch; the others one
    // by one on their slot of the KV tier (history loaded, row pos appended
    // there and stored back).  Attention reads rows < pos and takes the
    // current token from the fresh k, v; row pos is stored by a kernel of its
    // own right after it.  Stored from inside the attention kernel, the
    // append's few scattered writes land among the cache stream's reads and
    // cost about 14 us per OPT-175B layer on gfx950 (the attention alone: 189
    // against 172 us); after it, they drain during the next GEMM.
    const int32_t nd = kvt ? kvt->nb_dev : nb;
    // With host attention, the host batches' q, k, v rows go to the host
    // first, the device batches' attention runs while the CPU computes theirs,
    // and their attention rows come back before the out-projection.
    if (host_attn)
        FG_TRY(kvtier_host_send(kvt->kt, 0, 0, qkv + (int64_t)nd * gbs * 3 * h1, (int64_t)(nb - nd) * gbs, h1, st));
    FG_TRY(launch_attn_decode(qkv, qkv + h1, qkv + 2 * h1, 3 * h1, kv, nd * gbs, d, pos, 0, o, st,
                              topk));
    FG_TRY(launch_kv_store(qkv + h1, qkv + 2 * h1, 3 * h1, kv, 0, nd * gbs, pos, 1, d, st));
    if (host_attn)
        FG_TRY(kvtier_host_attend(kvt->kt, 0, 0, kvt->host, 0, d, (int64_t)(nb - nd) * gbs, pos,
                                  o + (int64_t)nd * gbs * h1, st));
    for (int32_t k = host_attn ? nb : nd; k < nb; ++k) {
        const int32_t u = kvt->u0 + (k - nd);
        const __half* q = qkv + (int64_t)k * gbs * 3 * h1;
        fg_kv slot;
        FG_TRY(kvt->pipe->begin(u, &slot));
        FG_TRY(launch_attn_decode(q, q + h1, q + 2 * h1, 3 * h1, &slot, gbs, d, pos, 0,
                                  o + (int64_t)k * gbs * h1, st, topk));
        FG_TRY(launch_kv_store(q + h1, q + 2 * h1, 3 * h1, &slot, 0, gbs, pos, 1, d, st));
        FG_TRY(kvt->pipe->end(u, pos, pos + 1));
    }
    return dec_post(d, w, xh, bls, b, st, next);
}

// A decode step of the whole model whose host batches' attention runs on the
// host CPU, overlapped with GPU work ("FlexGen 完全拆解": the CPU delegation of
// section "为什么有时应该在 CPU 上算注意力", overlapped with compute as the
// data paths of section "三条关键数据通路如何重叠" are).  With one fused block
// GEMM per projection, a layer's out-projection needs every row's attention,
// so the GPU would wait while the CPU attends.  Here the block's rows split
// into lanes that share only the weights:
//  * the device batches (cache in HBM): every layer enqueued at once on the
//    caller's stream;
//  * the host batches, in one lane or two of whole GPU batches, each on a
//    stream of the tier's, driven layer by layer by the calling thread.
//    While the CPU attends one lane's layer, the GPU runs the other lane's
//    out-projection, MLP and next QKV projection, and the device lane.
// Each lane multiplies its own rows, so each weight byte is read once per
// lane per layer (the cost of the overlap).  *used: false, with nothing
// enqueued, when the workspace cannot hold the lanes' buffers or the layers'
// weight formats differ; the caller then takes the serialized path.
int model_decode_host_overlap(const fg_dims* d, int32_t n_layers, const fg_layer_w* w, const fg_kv* kv,
                              void* x, int32_t gbs, int32_t nb, int32_t pos, void* ws, size_t ws_bytes,
                              hipStream_t st, const fg_kv_tier* kvt, bool* used) {
    *used = false;
    const int32_t nd = kvt->nb_dev, nh = nb - kvt->nb_dev;
    const fg_kvtier* kt = kvt->pipe;
    // every layer validated as the serialized path does (weights, block,
    // caches, host stage for all host rows)
    for (int32_t j = 0; j < n_layers; ++j) {
        const KvTierCall kc{nullptr, kt, &kvt->host[j], nd, 0};
        FG_TRY(layer_decode(d, &w[j], x, gbs, nb, pos, &kv[j], ws, ws_bytes, st, true, j > 0,
                            j + 1 < n_layers ? &w[j + 1] : nullptr, 0, &kc));
        if (w[j].fmt != w[0].fmt) return FG_OK;
    }
    const int nl = nh >= 2 ? 2 : 1;
    const int64_t h1 = d->h1;
    int64_t rows[2] = {(int64_t)((nh + 1) / 2) * gbs, (int64_t)(nh / 2) * gbs};
    const int64_t seq0[2] = {0, rows[0]};
    const size_t off[2] = {0, host_stage_bytes(d, rows[0])};
    if (off[1] + host_stage_bytes(d, rows[1]) > kvtier_host_stage_capacity(kt)) return FG_OK;
    // workspaces: the device lane's, then each host lane's
    const size_t A = 256;
    const WsLayout Ld = layout(d, (int64_t)nd * gbs, w[0].fmt);
    WsLayout Ll[2];
    size_t at = nd > 0 ? align_up(Ld.total, A) : 0, lane_at[2];
    for (int l = 0; l < nl; ++l) {
        Ll[l] = layout(d, rows[l], w[0].fmt);
        lane_at[l] = at;
        at += align_up(Ll[l].total, A);
    }
    if (at > ws_bytes) return FG_OK;
    hipStream_t ls[2];
    hipEvent_t ev[3];
    kvtier_host_lanes(kt, ls, ev);
    *used = true;

    unsigned char* base = static_cast<unsigned char*>(ws);
    __half* xh = (__half*)x;
    FG_HIP(hipEventRecord(ev[0], st));   // the lanes start after the caller's work so far
    for (int l = 0; l < nl; ++l) FG_HIP(hipStreamWaitEvent(ls[l], ev[0], 0));
    // the device lane is enqueued by a thread of its own, so that its
    // launches do not delay the host lanes' first attention
    int dev_rc = FG_OK;
    std::string dev_err;
    auto device_lane = [&]() {
        for (int32_t j = 0; nd > 0 && j < n_layers; ++j) {
            dev_rc = layer_decode(d, &w[j], x, gbs, nd, pos, &kv[j], ws, Ld.total, st, false, j > 0,
                                  j + 1 < n_layers ? &w[j + 1] : nullptr, 0, nullptr);
            if (dev_rc != FG_OK) {
                dev_err = fg_last_error();
                return;
            }
        }
    };
    std::thread dev_thread;
    try {
        dev_thread = std::thread(device_lane);
    } catch (const std::system_error&) {
        device_lane();   // no thread to spare: enqueued here first
    }
    DecWs b[2];
    __half* xl[2];
    for (int l = 0; l < nl; ++l) {
        b[l] = dec_ws(base + lane_at[l], Ll[l]);
        xl[l] = xh + ((int64_t)nd * gbs + seq0[l]) * h1;
    }
    auto lanes = [&]() -> int {
        for (int l = 0; l < nl; ++l) {
            FG_TRY(dec_pre(d, &w[0], xl[l], rows[l], b[l], ls[l], false));
            FG_TRY(kvtier_host_send(kt, l, off[l], b[l].qkv, rows[l], h1, ls[l]));
        }
        for (int32_t j = 0; j < n_layers; ++j) {
            const fg_layer_w* next = j + 1 < n_layers ? &w[j + 1] : nullptr;
            for (int l = 0; l < nl; ++l) {
                FG_TRY(kvtier_host_attend(kt, l, off[l], &kvt->host[j], (int32_t)seq0[l], d, rows[l], pos, b[l].o,
                                          ls[l]));
                FG_TRY(dec_post(d, &w[j], xl[l], rows[l], b[l], ls[l], next));
                if (next) {
                    FG_TRY(dec_pre(d, next, xl[l], rows[l], b[l], ls[l], true));
                    FG_TRY(kvtier_host_send(kt, l, off[l], b[l].qkv, rows[l], h1, ls[l]));
                }
            }
        }
        return FG_OK;
    };
    const int rc = lanes();
    if (dev_thread.joinable()) dev_thread.join();
    // the caller's stream continues after both lanes, also after an error
    // (nothing enqueued on a lane is left unordered against later work)
    for (int l = 0; l < nl; ++l) {
        FG_HIP(hipEventRecord(ev[1 + l], ls[l]));
        FG_HIP(hipStreamWaitEvent(st, ev[1 + l], 0));
    }
    if (dev_rc != FG_OK) return set_error(dev_rc, "%s", dev_err.c_str());
    return rc;
}

int layer_prefill(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs, int32_t nb,
                  int32_t s, const fg_kv* kv, void* ws, size_t ws_bytes, hipStream_t st,
                  bool check_only, const KvTierCall* kvt) {
    FG_TRY(check_layer(d, w, x, kv, ws));
    FG_CHECK_ARG(s >= 1, "prompt length %d < 1", s);
    FG_TRY(check_block(d, kv, gbs, nb, s, kvt));
    const int64_t rows = (int64_t)gbs * s;
    const WsLayout L = layout(d, rows, w->fmt);
    if (ws_bytes < L.total)
        return set_error(FG_ERR_CAPACITY, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
    if (check_only) return FG_OK;
    unsigned char* base = static_cast<unsigned char*>(ws);
    __half* a = (__half*)(base + L.a);
    __half* qkv = (__half*)(base + L.qkv);
    __half* o = (__half*)(base + L.o);
    __half* f = (__half*)(base + L.f);
    void* part = base + L.part;
    const size_t pb = L.wdq - L.part;
    const int64_t h1 = d->h1, h2 = d->h2;

    // Prefill-shaped GEMMs with 4-bit weights: each matrix is restored to fp16
    // once per layer (the compression is for storage and transfer; compute is
    // fp16) and every GPU batch of the block multiplies on the fp16 path.
    // Re-dequantizing a weight tile for every tile of rows, as the fused kernel
    // would, costs more than this one pass at these row counts.
    fg_layer_w wl = *w;
    unsigned dq = 0;   // matrices multiplied from an fp16 copy (bit = which)
    if (prefill_dequant(rows, w->fmt)) {
        dq = 0xFu;
        __half* p_qkv = (__half*)(base + L.wdq);
        __half* p_o = p_qkv + 3 * h1 * h1;
        __half* p_1 = p_o + h1 * h1;
        __half* p_2 = p_1 + h2 * h1;
        FG_TRY(launch_dequant_g4((const uint8_t*)w->w_qkv, (const __half*)w->m_qkv, 1, 3 * h1, h1, p_qkv, st));
        FG_TRY(launch_dequant_g4((const uint8_t*)w->w_o, (const __half*)w->m_o, 1, h1, h1, p_o, st));
        FG_TRY(launch_dequant_g4((const uint8_t*)w->w_1, (const __half*)w->m_1, 1, h2, h1, p_1, st));
        FG_TRY(launch_dequant_g4((const uint8_t*)w->w_2, (const __half*)w->m_2, 1, h1, h2, p_2, st));
        wl.w_qkv = p_qkv; wl.w_o = p_o; wl.w_1 = p_1; wl.w_2 = p_2;
        wl.m_qkv = wl.m_o = wl.m_1 = wl.m_2 = nullptr;
    }
    for (int32_t k = 0; k < nb; ++k) {     // GPU batches of the block, one layer resident
        __half* xh = (__half*)x + (int64_t)k * rows * h1;
        FG_TRY(launch_layernorm(xh, rows, h1, (const __half*)wl.ln1_g, (const __half*)wl.ln1_b, a, st));
        FG_TRY(lin(&wl, 0, a, rows, h1, 3 * h1, 0, nullptr, qkv, part, pb, st, nullptr, nullptr, nullptr, dq));
        FG_TRY(launch_attn_prefill(qkv, gbs, s, d, o, st));
        if (!kvt || k < kvt->nb_dev) {
            FG_TRY(launch_kv_store(qkv + h1, qkv + 2 * h1, 3 * h1, kv, k * gbs, gbs, 0, s, d, st));
        } else {   // written to the batch's slot, then stored to the host cache
            const int32_t u = kvt->u0 + (k - kvt->nb_dev);
            fg_kv slot;
            FG_TRY(kvt->pipe->begin(u, &slot));
            FG_TRY(launch_kv_store(qkv + h1, qkv + 2 * h1, 3 * h1, &slot, 0, gbs, 0, s, d, st));
            FG_TRY(kvt->pipe->end(u, 0, s));
        }
        FG_TRY(lin(&wl, 1, o, rows, h1, h1, 0, xh, xh, part, pb, st, wl.ln2_g, wl.ln2_b, a, dq));
        FG_TRY(lin(&wl, 2, a, rows, h1, h2, 1, nullptr, f, part, pb, st, nullptr, nullptr, nullptr, dq));
        FG_TRY(lin(&wl, 3, f, rows, h2, h1, 0, xh, xh, part, pb, st, nullptr, nullptr, nullptr, dq));
    }
    return FG_OK;
}

size_t layer_ws_bytes(const fg_dims* d, int64_t rows, int32_t fmt) { return layout(d, rows, fmt).total; }

}  // namespace fg

extern "C" size_t fg_workspace_bytes(const fg_dims* d, int64_t rows, int32_t fmt_w) {
    if (!d || rows < 0 || d->h1 <= 0 || d->h2 <= 0) return 0;
    return fg::layer_ws_bytes(d, rows, fmt_w);
}

extern "C" int fg_layer_decode_block(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs,
                                     int32_t nb, int32_t pos, const fg_kv* kv, void* ws,
                                     size_t ws_bytes, void* stream, int32_t attn_topk_ppm,
                                     const fg_kv_tier* kvt) {
    fg::clear_error();
    fg::KvTierCall kc{};
    if (kvt) {
        kc = fg::KvTierCall{nullptr, kvt->pipe, kvt->host, kvt->nb_dev, 0};
        FG_TRY(fg::layer_decode(d, w, x, gbs, nb, pos, kv, ws, ws_bytes, fg::as_stream(stream), true,
                                false, nullptr, attn_topk_ppm, &kc));
    }
    fg::KvPipe pipe(kvt ? kvt->pipe : nullptr, d, gbs, pos, fg::as_stream(stream));
    if (kvt) {
        for (int32_t k = kvt->nb_dev; k < nb; ++k) pipe.add(kvt->host, (k - kvt->nb_dev) * gbs);
        kc.pipe = &pipe;
    }
    return fg::layer_decode(d, w, x, gbs, nb, pos, kv, ws, ws_bytes, fg::as_stream(stream), false,
                            false, nullptr, attn_topk_ppm, kvt ? &kc : nullptr);
}

extern "C" int fg_layer_prefill(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs,
                                int32_t nb, int32_t s, const fg_kv* kv, void* ws, size_t ws_bytes,
                                void* stream, const fg_kv_tier* kvt) {
    fg::clear_error();
    fg::KvTierCall kc{};
    if (kvt) {
        kc = fg::KvTierCall{nullptr, kvt->pipe, kvt->host, kvt->nb_dev, 0};
        FG_TRY(fg::layer_prefill(d, w, x, gbs, nb, s, kv, ws, ws_bytes, fg::as_stream(stream), true,
                                 &kc));
    }
    fg::KvPipe pipe(kvt ? kvt->pipe : nullptr, d, gbs, 0, fg::as_stream(stream));
    if (kvt) {
        for (int32_t k = kvt->nb_dev; k < nb; ++k) pipe.add(kvt->host, (k - kvt->nb_dev) * gbs);
        kc.pipe = &pipe;
    }
    return fg::layer_prefill(d, w, x, gbs, nb, s, kv, ws, ws_bytes, fg::as_stream(stream), false,
                             kvt ? &kc : nullptr);
}
