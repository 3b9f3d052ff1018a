/*
 * fg — 4-bit zig-zag block decode of an OPT-style decoder on MI355X (gfx950).
 *
 * C ABI of libfg.so.  Every entry point takes plain device pointers and sizes;
 * fp16 tensors are raw binary16 arrays, row-major unless stated.  `stream` is
 * a hipStream_t passed as void* (NULL = the null stream).
 *
 * Pages the operations come from (cited by title and section):
 *   [P2] "FlexGen 完全拆解:用线性规划编排 GPU、CPU 与 SSD 上的大模型推理"
 *        (pinghaoyang.com.cn)
 *   [P1] bjbfmj.com FlexGen walkthrough (sections 一…八 cited as §1…§8)
 *
 * Conventions shared by every call:
 *   - Ownership: the caller allocates and owns every buffer.  Calls keep no
 *     pointer after they return.  Buffers must stay valid until the work
 *     enqueued on `stream` has finished.
 *   - Asynchrony: calls only validate on the host and enqueue kernels; the
 *     results are ready once the stream is synchronised.
 *   - Errors: arguments are checked on the host before anything is launched;
 *     a failed check returns a negative status, launches nothing and leaves
 *     every buffer untouched.  A failing HIP runtime call returns
 *     FG_ERR_HIP.  fg_last_error() gives the detail of the calling thread's
 *     last failure.  No C++ exception crosses this interface.
 *   - Threading: calls are stateless and may be issued from several threads.
 */
#ifndef FG_H
#define FG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
enum {
    FG_OK = 0,
    FG_ERR_INVALID = -1,      /* null pointer, bad size, inconsistent shapes */
    FG_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim 96) */
    FG_ERR_CAPACITY = -3,     /* workspace or cache too small for the request */
    FG_ERR_HIP = -4           /* a HIP runtime call failed */
};

const char* fg_status_str(int status);
/* Detail of the calling thread's last failing call ("" if none). */
const char* fg_last_error(void);
/* ABI version, bumped on any incompatible change of this header (2: the
 * block-decode entry points take attn_topk_ppm; 3: the layer and model
 * passes take a KV tier, fg_kv_tier). */
int fg_abi_version(void);

/* ----------------------------------------------------------------- formats */
enum {
    FG_FMT_F16 = 0,     /* fp16 tensor */
    FG_FMT_Q4G64 = 1    /* 4-bit codes + fp16 (min, scale) per group of 64 */
};

/* Decoder dimensions: hidden h1, MLP h2, heads n_heads of head_dim each.
 * Requires h1 = n_heads * head_dim, h1 % 64 == 0, h2 % 64 == 0,
 * head_dim in {64, 128}. */
typedef struct {
    int32_t h1, h2, n_heads, head_dim;
} fg_dims;

/* ------------------------------------------------------------------- codec */
/*
 * Group-wise asymmetric 4-bit min-max quantization ([P2] "权重压缩与 KV Cache
 * 压缩", quantize equation; [P1] §6.3 CompressionConfig num_bits 4,
 * group_size 64, asymmetric, two 4-bit values per uint8, fp16 scale tensor).
 *
 * x: fp16 viewed as [outer, axis, inner]; each run of `group` consecutive
 * elements along `axis` (fixed outer, inner) is one group.  Per group, in
 * binary32 with one rounding per operation:
 *   mn, mx = min, max (-0 canonicalised to +0); range = mx - mn;
 *   q = range > 0 ? clamp(rint((x - mn) * (15 / range)), 0, 15) : 0
 *   (rint: nearest, ties to even; 15/range computed once per group).
 * codes: uint8 [outer, axis/2, inner]; byte j of a group holds element 2j in
 *   its low nibble and element 2j+1 in its high nibble.
 * meta:  fp16  [outer, axis/group, 2, inner] = (fp16(mn), fp16(range / 15)).
 * Weights [N, K] are quantized with outer = 1, axis = N, inner = K (groups
 * along output channels); the KV cache with inner = 1 along head_dim.
 * Requirements: group == 64, axis % 64 == 0, outer, inner >= 1.
 * Results are bit-identical to the CPU definition for identical inputs.
 */
int fg_quant_group4(const void* x, int64_t outer, int64_t axis, int64_t inner,
                    int32_t group, void* codes, void* meta, void* stream);

/* Inverse ([P2] dequantize equation): y = fp16(mn + q * scale), a binary32
 * multiply then add.  Same layouts and requirements as fg_quant_group4. */
int fg_dequant_group4(const void* codes, const void* meta, int64_t outer, int64_t axis,
                      int64_t inner, int32_t group, void* y, void* stream);

/* ------------------------------------------------------------ layer weights */
/*
 * One decoder layer ([P2] "从 Transformer 推理的数据流重新定义卸载": four
 * h1 x h1 attention matrices and two MLP matrices; pre-LN, ReLU MLP).
 * Matrices are [N = out, K = in]: w_qkv [3*h1, h1] stacks W_Q, W_K, W_V rows;
 * w_o [h1, h1]; w_1 [h2, h1]; w_2 [h1, h2].
 *   fmt FG_FMT_F16:   w_* fp16; m_* unused (NULL).
 *   fmt FG_FMT_Q4G64: w_* = codes [N/2, K], m_* = meta [N/64, 2, K]
 *                     (fg_quant_group4 with outer 1, axis N, inner K).
 * Biases b_* [N] and LayerNorm gamma/beta [h1] are fp16 in both formats.
 */
typedef struct {
    int32_t fmt;
    const void *w_qkv, *m_qkv, *b_qkv;
    const void *w_o, *m_o, *b_o;
    const void *w_1, *m_1, *b_1;
    const void *w_2, *m_2, *b_2;
    const void *ln1_g, *ln1_b, *ln2_g, *ln2_b;
} fg_layer_w;

/*
 * One layer's KV cache for n_seq sequences and max_len positions
 * ([P2] KV append: K_{1:s+t} = Concat(K_{1:s+t-1}, X_t W_K), same for V).
 *   fmt FG_FMT_Q4G64: k, v = codes [n_seq, n_heads, max_len, head_dim/2];
 *                     k_meta, v_meta = fp16 [n_seq, n_heads, max_len, head_dim/64, 2]
 *                     (groups of 64 along head_dim, [P1] §6.3 group_dim 2).
 *   fmt FG_FMT_F16:   k, v = fp16 [n_seq, n_heads, max_len, head_dim]; metas NULL.
 */
typedef struct {
    int32_t fmt;
    void *k, *k_meta, *v, *v_meta;
    int32_t max_len;
    int32_t n_seq;
} fg_kv;

/* ---------------------------------------------------------- KV append / attn */
/*
 * Append one position: quantize (or copy, for fp16 caches) k_new, v_new of
 * each of the first bls sequences into position `pos` of the cache.
 * k_new, v_new: fp16 rows of stride ld elements (ld >= h1), head h at
 * columns [h*head_dim, (h+1)*head_dim).  Requires 0 <= pos < max_len,
 * 1 <= bls <= n_seq, kv->fmt matching the function.
 */
int fg_kv_append_q4(const void* k_new, const void* v_new, int64_t ld, const fg_kv* kv,
                    int32_t bls, const fg_dims* d, int32_t pos, void* stream);
int fg_kv_append_f16(const void* k_new, const void* v_new, int64_t ld, const fg_kv* kv,
                     int32_t bls, const fg_dims* d, int32_t pos, void* stream);

/*
 * Decode attention for one new token per sequence at position `pos`
 * ([P2] decode: the single query attends to all s+t cached keys).
 * out[b, h*hd + c] = sum_p softmax_p(q.k_p / sqrt(hd)) v_p[c] over p = 0..pos:
 * positions < pos come from the cache (dequantized in registers for 4-bit
 * caches); position pos uses the fresh fp16 k_new, v_new.  With fuse_append
 * != 0 the same launch also appends k_new, v_new at pos (as fg_kv_append_*).
 * q, k_new, v_new: fp16 rows of stride ld; out: fp16 [bls, h1] (stride h1).
 */
int fg_attn_decode_q4(const void* q, const void* k_new, const void* v_new, int64_t ld,
                      const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos,
                      int32_t fuse_append, void* out, void* stream);
int fg_attn_decode_f16(const void* q, const void* k_new, const void* v_new, int64_t ld,
                       const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos,
                       int32_t fuse_append, void* out, void* stream);

/*
 * Decode attention with Top-K sparse V ([P2] "权重压缩与 KV Cache 压缩": the
 * scores use every Key, and only the Values of the highest-scoring positions
 * are read).  As fg_attn_decode_*, except that the V sum covers the `topk`
 * cached positions of highest score (ties: lower position first) plus the
 * current token (its fresh v_new), while the softmax normalizer keeps every
 * score (no renormalization over the selected set).  The pages' setting is
 * topk = ceil(0.1 * pos).  Requires 0 <= topk <= pos and pos <= 8192 (the
 * whole history's scores are held on chip); FG_ERR_UNSUPPORTED above that.
 * topk = pos equals the dense result.
 */
int fg_attn_decode_topk_q4(const void* q, const void* k_new, const void* v_new, int64_t ld,
                           const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos,
                           int32_t topk, int32_t fuse_append, void* out, void* stream);
int fg_attn_decode_topk_f16(const void* q, const void* k_new, const void* v_new, int64_t ld,
                            const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos,
                            int32_t topk, int32_t fuse_append, void* out, void* stream);

/*
 * Causal prompt attention ([P2] prefill over all s prompt tokens):
 * qkv fp16 [b*s, 3*h1] rows (q | k | v); out fp16 [b*s, h1];
 * row t of a sequence attends to its rows 0..t.
 */
int fg_attn_prefill(const void* qkv, int32_t b, int32_t s, const fg_dims* d, void* out,
                    void* stream);

/* --------------------------------------------------------- decoder pieces */
/*
 * y = act(x W^T + bias) + residual, fp32 accumulation on fp16 MFMA, one
 * rounding to fp16.  x fp16 [M, K]; W [N, K] in `fmt` (q4: codes w, meta m,
 * dequantized on the fly); bias fp16 [N] or NULL; act: 0 none, 1 ReLU
 * (applied before the residual); residual fp16 [M, N] or NULL and may equal y.
 * ws: device scratch of ws_bytes >= fg_linear_workspace_bytes(M, N, K) (may
 * be NULL when that is 0).  Requires K % 64 == 0, N % 64 == 0 for q4 and
 * N % 8 == 0 for fp16.
 */
int fg_linear(const void* x, int64_t M, int64_t K, int32_t fmt, const void* w, const void* m,
              int64_t N, const void* bias, int32_t act, const void* residual, void* y,
              void* ws, size_t ws_bytes, void* stream);
size_t fg_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * fg_linear without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, layout, results and errors as
 * fg_linear minus ws / ws_bytes.  The split-k partials live in a device
 * array of fg_linear_noalloc_max_bytes() (96 MiB) that the library holds on
 * each GPU it runs on until the process ends; shapes whose partials
 * (fg_linear_workspace_bytes) exceed it are refused with
 * FG_ERR_UNSUPPORTED.  No part of the array needs to start at zero: every
 * partial a call reads was written earlier in the same call.  All calls on
 * one GPU share its array, so calls that overlap on that GPU (concurrent
 * streams, threads) race; calls ordered on one stream do not.  Allocates
 * nothing on the host or the device.
 */
size_t fg_linear_noalloc_max_bytes(void);
int fg_linear_noalloc(const void* x, int64_t M, int64_t K, int32_t fmt, const void* w, const void* m,
                      int64_t N, const void* bias, int32_t act, const void* residual, void* y,
                      void* stream);

/* Row LayerNorm over the last dim h (biased variance, eps 1e-5):
 * y = (x - mean) / sqrt(var + eps) * gamma + beta.  x, y fp16 [rows, h]. */
int fg_layernorm(const void* x, int64_t rows, int64_t h, const void* gamma, const void* beta,
                 void* y, void* stream);

/* x[r] = fp16(E[tok[r]] + P[pos[r]]): tok, pos int32 [rows] (device),
 * E fp16 [vocab, h1], P fp16 [max_pos, h1].  Ids are clamped to the tables'
 * ranges on the device (the host cannot see device-resident ids). */
int fg_embed(const int32_t* tok, const int32_t* pos, int64_t rows, const void* E, int64_t vocab,
             const void* P, int64_t max_pos, int64_t h1, void* x, void* stream);

/* out[r] = index of the largest fp16 value of row r of logits [rows, n]
 * (lowest index on ties). */
int fg_argmax(const void* logits, int64_t rows, int64_t n, int32_t* out, void* stream);

/* --------------------------------------------------------------- KV tier */
/*
 * KV-cache tiering to pinned host memory ([P2] "三条关键数据通路如何重叠" and
 * "一个层级流水的伪代码": the cache of GPU batch k+1 is loaded while batch k
 * computes, and the new entries of a batch are stored back afterwards;
 * [P1] §6.4 load_cache / store_cache).
 *
 * The block's GPU batches 0..nb_dev-1 keep their cache in the device cache
 * `kv` of the layer calls; batches nb_dev..nb-1 keep theirs in `host[j]`, a
 * cache of the same format in pinned host memory (hipHostMalloc) whose
 * sequence i is block sequence nb_dev*gbs + i.  For every host batch of every
 * layer the library copies its history (positions 0..pos-1; K, V and their
 * metadata, as 2-D copies of the cache's rows) into one of two device slots,
 * runs that batch's attention on the slot (appending position pos there), and
 * copies the appended row back to `host[j]`; prefill writes positions
 * 0..s-1 of the slot and copies them back.  Loads run on the copy stream
 * given at creation and stores on a stream the tier object creates, ordered
 * by events: over the call's host batches u (layer by layer), load(u+1) is
 * issued before store(u), so the load of the next batch, also across a layer
 * boundary, runs while the current one computes, and load(u+2) waits for
 * store(u) to have read the slot.  A call's loads wait for all stores of
 * earlier calls; a caller reading the host caches synchronizes the device.
 *
 * slots: caller-owned device memory of 2 * slot_bytes (256-byte aligned);
 * slot_bytes >= fg_kvtier_slot_bytes(d, gbs, max_len, fmt) of every call
 * (max_len: the host caches').  copy_stream: a caller-owned stream other
 * than the compute streams of the calls (default priority); it must stay
 * valid until fg_kvtier_destroy.  One fg_kvtier serves one call at a time;
 * its slots must not be touched while a call's work is in flight.
 */
typedef struct fg_kvtier fg_kvtier;   /* opaque: two slots, copy stream, events */

size_t fg_kvtier_slot_bytes(const fg_dims* d, int32_t gbs, int32_t max_len, int32_t fmt);
int fg_kvtier_create(fg_kvtier** out, void* slots, size_t slot_bytes, void* copy_stream);
int fg_kvtier_destroy(fg_kvtier* kt);

/*
 * Decode attention on the host CPU for host-resident GPU batches ([P2]
 * "为什么有时应该在 CPU 上算注意力": when a batch's cache is on the CPU side and
 * the link is the bottleneck, the CPU computes that batch's attention, and
 * only the current token's q, k, v (3·h1 values per sequence) go down the
 * link and its attention row (h1 values) comes back, instead of the whole
 * history).  The pages turn this off with 4-bit compression, since on their
 * host the CPU's dequantization costs what the smaller transfer saves; here
 * both formats are delegated: a 4-bit history is read compressed and
 * dequantized in registers, and the new row is quantized on the CPU with the
 * codec's exact arithmetic (the same bytes as the device quantizer).
 *
 * After fg_kvtier_host_attention(kt, stage, stage_bytes, n_threads) with a
 * non-NULL stage, the decode calls of that tier (fg_layer_decode_block,
 * fg_model_decode_step) no longer move host batches' histories through the
 * slots.  Per layer they copy the host batches' q, k, v rows into `stage`,
 * wait on the host until they have arrived, compute the host batches'
 * attention with n_threads CPU threads, append their k, v at row pos of the
 * host cache directly, and copy the attention rows back; the calls
 * therefore return only after the GPU has reached the last layer's
 * attention.  fg_layer_decode_block does this on the call's stream (the
 * device batches' attention is enqueued first and runs meanwhile).
 * fg_model_decode_step without weight tiering overlaps the CPU's attention
 * with GPU work: the device batches run every layer on the call's stream
 * (enqueued from a second host thread) and the host batches run as one or
 * two lanes of whole GPU batches on two streams the tier object creates, so
 * that the GPU computes one lane while the CPU attends the other; each lane
 * multiplies its own rows (each weight read once per lane per layer), and
 * the call's stream waits for the lanes before the call returns.  It needs
 * workspace for the lanes' buffers side by side (a little more than the
 * whole block's: each lane has its own split-k partials); with less, or with
 * weight tiering, it takes the serialized form above.  Results of the
 * two forms agree within rounding (their GEMMs sum partials in different
 * orders).  Prefill calls keep using the slots.  stage:
 * caller-owned pinned host memory of stage_bytes >=
 * fg_kvtier_host_stage_bytes(d, n_host_seq), n_host_seq the host-resident
 * sequences of a call ((nb - nb_dev) * gbs); it must not be touched while a
 * call's work is in flight.  n_threads <= 0: all hardware threads.  stage
 * NULL: back to the slots.
 */
size_t fg_kvtier_host_stage_bytes(const fg_dims* d, int32_t n_host_seq);
int fg_kvtier_host_attention(fg_kvtier* kt, void* stage, size_t stage_bytes, int32_t n_threads);

/*
 * The host-CPU attention itself, on host memory only (no GPU involved): for
 * sequences seq0 .. seq0+nseq-1 of the cache `kv` (host pointers; fp16 for
 * the _f16 entry point, 4-bit for _q4, whose cached values are min + code *
 * scale in fp32 and whose append quantizes k, v as fg_kv_append_q4 does) at
 * position pos, the history rows < pos from the cache and the current token
 * from its fresh k, v.  qkv: fp16 [nseq, ld] rows, q at column 0, k at h1, v
 * at 2*h1 (ld >= 3*h1).  out: fp16 [nseq, h1].  append != 0: also store k, v
 * at row pos of the cache.  Scores, softmax and the V sum in fp32, one fp16
 * rounding per output.  Runs on n_threads threads (<= 0: all hardware
 * threads) and returns when done.  FG_ERR_UNSUPPORTED for a cache of the
 * other format;
 * FG_ERR_INVALID for sequences or pos outside the cache, ld < 3*h1, null
 * pointers or bad dims; FG_ERR_CAPACITY when host memory for the threads'
 * score buffers runs out (out is then incomplete).
 */
int fg_attn_decode_host_f16(const void* qkv, int64_t ld, const fg_kv* kv, int32_t seq0, int32_t nseq,
                            const fg_dims* d, int32_t pos, int32_t append, void* out,
                            int32_t n_threads);
int fg_attn_decode_host_q4(const void* qkv, int64_t ld, const fg_kv* kv, int32_t seq0, int32_t nseq,
                           const fg_dims* d, int32_t pos, int32_t append, void* out,
                           int32_t n_threads);

/* KV tier of one layer or model call.  host: one pinned host cache (layer
 * calls) or n_layers of them (model calls), each with n_seq >=
 * (nb - nb_dev) * gbs and max_len > the call's last position.  With a tier,
 * the device cache `kv` needs n_seq >= nb_dev * gbs only.  NULL tier: every
 * sequence in `kv`. */
typedef struct {
    fg_kvtier* pipe;
    const fg_kv* host;
    int32_t nb_dev;
} fg_kv_tier;

/* ---------------------------------------------------------------- layers */
/*
 * Prefill one layer for a block of nb GPU batches of gbs sequences each
 * (bls = gbs * nb), prompt length s ([P2] "FlexGen 的核心:计算图分块…":
 * inside one layer every GPU batch of the block runs before the next layer).
 * x: fp16 [bls*s, h1], in/out (row b*s + t = token t of sequence b).
 * Per GPU batch: LN1 -> QKV -> causal attention -> append K, V of positions
 * 0..s-1 to kv -> out-proj + residual -> LN2 -> FC1 + ReLU -> FC2 + residual.
 * ws: ws_bytes >= fg_workspace_bytes(d, gbs * s, w->fmt).
 */
int fg_layer_prefill(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs, int32_t nb,
                     int32_t s, const fg_kv* kv, void* ws, size_t ws_bytes, void* stream,
                     const fg_kv_tier* kvt);

/*
 * One decode step of one layer for the whole block (bls = gbs * nb new
 * tokens, one per sequence, all at position pos) — the zig-zag block's inner
 * loop ([P2] block schedule; pipeline pseudocode in "一个层级流水的伪代码").
 * The layer's weights are read once for all bls rows: every projection is one
 * contraction over bls rows; attention runs per (sequence, head) with the
 * fused K, V append at pos.
 * x: fp16 [bls, h1], in/out.  ws: ws_bytes >= fg_workspace_bytes(d, bls, w->fmt).
 *
 * attn_topk_ppm selects Top-K sparse V attention ([P2] "权重压缩与 KV Cache
 * 压缩"; the semantics of fg_attn_decode_topk_*) with
 * topk = ceil(pos * attn_topk_ppm / 1e6) cached positions; the pages' 10% is
 * 100000.  0, any value >= 1000000, and any step where that topk reaches pos
 * (e.g. pos = 0) run dense attention.  Negative: FG_ERR_INVALID.  A sparse
 * step with pos > 8192 returns FG_ERR_UNSUPPORTED before anything is enqueued.
 * kvt: KV tier (see fg_kv_tier; kvt->host is this layer's host cache) or NULL.
 */
int fg_layer_decode_block(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs,
                          int32_t nb, int32_t pos, const fg_kv* kv, void* ws, size_t ws_bytes,
                          void* stream, int32_t attn_topk_ppm, const fg_kv_tier* kvt);

/* Device scratch needed by one layer pass over `rows` token rows
 * (decode: rows = bls; prefill: rows = gbs * s). */
size_t fg_workspace_bytes(const fg_dims* d, int64_t rows, int32_t fmt_w);

/* ------------------------------------------------------ block schedule */
/*
 * Every layer of one pass, in block order ([P2] "一个层级流水的伪代码":
 * token step outermost, then layers, then the block's GPU batches):
 * fg_model_prefill runs fg_layer_prefill for layers 0..n_layers-1,
 * fg_model_decode_step runs fg_layer_decode_block for them.  w and kv are
 * arrays of n_layers; the other arguments are those of the per-layer calls.
 *
 * Weight tiering ([P2] "三条关键数据通路如何重叠": the next layer's
 * weights are prefetched while the current layer computes; [P1] §6.4 CPU
 * weights in pinned memory moved by load_weight).  With tier != NULL, layer j
 * with tier[j].qk_host != NULL keeps half of its fp16 weights in pinned host
 * memory (fmt must be FG_FMT_F16):
 *   qk_host: pinned host fp16 [2*h1, h1]  = the W_Q, W_K rows of W_qkv;
 *   v_dev:   device fp16 [h1, h1]         = the W_V rows of W_qkv;
 *   w1_host: pinned host fp16 [h2, h1]    = W_1;
 * that layer's w->w_qkv and w->w_1 are then not read.  Before the layer runs,
 * [W_Q; W_K] and W_1 are copied host -> device and W_V device -> device into
 * one of the two stage buffers of `sc`, on copy_stream, ordered by events:
 * the copy of a tiered layer is issued while the tiered layer before it
 * computes, and waits until the layer two tiered layers back has released
 * its buffer.  copy_stream must differ from stream (both default priority).
 * flags (decode and prefill):
 *   FG_SCHED_FIRST_STAGED  the first tiered layer was already staged by the
 *                          previous call (issued with FG_SCHED_STAGE_NEXT);
 *   FG_SCHED_STAGE_NEXT    after the last layer, stage the first tiered layer
 *                          for the next call.
 * Without tiering (tier == NULL) sc, copy_stream and flags are ignored and
 * may be NULL / 0.  The stage buffers are owned by the caller and must not be
 * touched while a call's work is in flight.
 * attn_topk_ppm (decode): as in fg_layer_decode_block, for every layer; every
 * layer is checked before the first is enqueued.
 * kvt: KV tier with kvt->host[j] the host cache of layer j, or NULL.
 */
enum { FG_SCHED_FIRST_STAGED = 1, FG_SCHED_STAGE_NEXT = 2 };

typedef struct {
    const void* qk_host;
    const void* v_dev;
    const void* w1_host;
} fg_tier_w;

typedef struct fg_sched fg_sched;   /* opaque: stage buffers + copy events */

/* Bytes of ONE stage buffer for tiered layers of shape d: fp16 W_qkv
 * [3*h1, h1] followed (256-byte aligned) by fp16 W_1 [h2, h1]. */
size_t fg_stage_bytes(const fg_dims* d);
/* stage: caller-owned device memory of 2 * stage_bytes (two buffers), with
 * stage_bytes >= fg_stage_bytes of every shape it will serve.  Creates the
 * copy / release events on the current device (host-side allocation, once). */
int fg_sched_create(fg_sched** out, void* stage, size_t stage_bytes);
int fg_sched_destroy(fg_sched* sc);

int fg_model_prefill(fg_sched* sc, const fg_dims* d, int32_t n_layers, const fg_layer_w* w,
                     const fg_tier_w* tier, const fg_kv* kv, void* x, int32_t gbs, int32_t nb,
                     int32_t s, void* ws, size_t ws_bytes, void* stream, void* copy_stream,
                     int32_t flags, const fg_kv_tier* kvt);
int fg_model_decode_step(fg_sched* sc, const fg_dims* d, int32_t n_layers, const fg_layer_w* w,
                         const fg_tier_w* tier, const fg_kv* kv, void* x, int32_t gbs,
                         int32_t nb, int32_t pos, void* ws, size_t ws_bytes, void* stream,
                         void* copy_stream, int32_t flags, int32_t attn_topk_ppm,
                         const fg_kv_tier* kvt);

/* One host -> device copy of the tiering path, for callers that run their
 * own layer-ahead schedule ([P2] "三条关键数据通路如何重叠": the next layer's
 * weights move over PCIe while the current layer computes; fg_model_* issue
 * the same copies themselves).  Enqueues `bytes` from src_pinned (pinned
 * host memory: hipHostMalloc, torch pin_memory) to dst_dev (device memory)
 * on copy_stream, then records `done` (a hipEvent_t, or NULL) on that stream
 * so that the compute stream can wait for it.  bytes == 0 records only the
 * event.  Errors: null pointers with bytes > 0, pageable or device source, or
 * a destination that is not device memory: FG_ERR_INVALID, nothing enqueued.
 * Allocates nothing; the caller owns both buffers and keeps them alive until
 * the copy is done.  Traced as kind "w_h2d". */
int fg_prefetch(void* dst_dev, const void* src_pinned, size_t bytes, void* copy_stream,
                void* done);

/* --------------------------------------------------------------- sizes */
/* Bytes of the six layer matrices of n_layers layers ([P2]: M_W =
 * l (8 h1^2 + 4 h1 h2) in fp16; 4-bit: codes + 4 bytes of meta per 64). */
int64_t fg_weight_bytes(const fg_dims* d, int32_t n_layers, int32_t fmt);
/* Bytes of the KV cache ([P2]: M_KV = 4 b l h1 (s + n) in fp16; 4-bit:
 * 9/32 of that). */
int64_t fg_kv_bytes(const fg_dims* d, int32_t n_layers, int32_t bls, int32_t s, int32_t n,
                    int32_t fmt);

/* ------------------------------------------------------------ capacity */
/*
 * Placement of a whole model on one GPU, for the capacity pre-check.  The
 * block schedule keeps every layer's weights and the whole block's KV cache
 * alive for the run, so the block is bounded by memory ([P2] "FlexGen 的核心:
 * 计算图分块与张量生命周期": the peak holds the weights in use, the block's
 * activations and the block's cache at s + n positions, which bounds bls).
 *   n_layers, fmt_w:  the decoder's layers and their weight format;
 *   n_tiered:         fp16 layers whose W_Q, W_K rows and W_1 live in pinned
 *                     host memory (staged through two device stage buffers);
 *   fmt_kv, max_len:  cache format and positions allocated per sequence;
 *   bls_dev:          sequences whose cache is in HBM;
 *   bls_host, gbs:    sequences whose cache is in pinned host memory (whole
 *                     GPU batches of gbs, moved through two device slots);
 *                     gbs also sizes the prefill's workspace;
 *   s:                prompt length (the block's prompt activations);
 *   vocab:            rows of the tied embedding (and the LM head's logits).
 */
typedef struct {
    int32_t n_layers, fmt_w, n_tiered, fmt_kv, max_len, bls_dev, bls_host, gbs, s;
    int64_t vocab;
} fg_plan;
/* Device bytes the plan keeps in HBM: device-resident weights, biases and
 * LayerNorms, stage buffers, the device cache, KV tier slots, the larger of
 * the prefill and decode workspaces (with the LM head's), the embeddings, the
 * block's prompt activations and the logits.  -1 on an invalid plan (detail
 * in fg_last_error). */
int64_t fg_plan_device_bytes(const fg_dims* d, const fg_plan* p);
/* FG_OK if fg_plan_device_bytes fits budget_bytes, or the device's free
 * memory (hipMemGetInfo on the current device) when budget_bytes is 0;
 * FG_ERR_CAPACITY otherwise, with the byte breakdown in fg_last_error.  Meant
 * to run before anything of the model is allocated; it allocates nothing. */
int fg_check_capacity(const fg_dims* d, const fg_plan* p, int64_t budget_bytes);

/* --------------------------------------------------------------- tracing */
/*
 * Per-kernel timing for roofline reports.  While enabled, each kernel launch
 * of this library is bracketed by two HIP events recorded on its own launch
 * stream and tagged with its kind and algorithmic work (flops; HBM bytes:
 * weights once, activations in and out, KV history at 9/16 byte per element
 * for 4-bit caches).  fg_trace_enable(on) discards earlier records and starts
 * (on != 0) or stops recording.  fg_trace_collect waits for the recorded
 * events and fills, per kind k < n_kinds, the launch count, summed duration
 * (ms), summed flops and summed bytes; it returns the number of kinds (or a
 * negative status).  A record whose events cannot be waited on or timed is
 * left out of the sums; the others are still summed, and the first such
 * failure is then returned as FG_ERR_HIP.  A launch whose events cannot be
 * created or recorded is not recorded.  fg_trace_kind_name names a kind.
 * Recording adds two event records per launch; it is off by default.
 */
int fg_trace_enable(int on);
/* Bit k of mask selects kind k for recording while tracing is on (default:
 * all kinds).  Launches of unselected kinds carry no events at all, so a
 * caller can time the kernels it reports without slowing the others. */
int fg_trace_kinds(uint64_t mask);
int fg_trace_collect(int32_t n_kinds, int64_t* count, double* ms, double* flops, double* bytes);
const char* fg_trace_kind_name(int kind);

#ifdef __cplusplus
}
#endif
#endif /* FG_H */
