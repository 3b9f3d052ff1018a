// Internal declarations shared by the translation units of libfg.so.
// Not part of the C ABI (see include/fg.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/fg.h"

namespace fg {

// ------------------------------------------------------------------ errors
// Records a formatted detail for fg_last_error() and returns `status`.
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define FG_CHECK_ARG(cond, ...)                                      \
    do {                                                             \
        if (!(cond)) return ::fg::set_error(FG_ERR_INVALID, __VA_ARGS__); \
    } while (0)

#define FG_CHECK_SUP(cond, ...)                                          \
    do {                                                                 \
        if (!(cond)) return ::fg::set_error(FG_ERR_UNSUPPORTED, __VA_ARGS__); \
    } while (0)

#define FG_HIP(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess)                                                     \
            return ::fg::set_error(FG_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// After a kernel launch: reports a launch failure as FG_ERR_HIP.
#define FG_LAUNCHED(name)                                                         \
    do {                                                                          \
        hipError_t e_ = hipGetLastError();                                        \
        if (e_ != hipSuccess)                                                     \
            return ::fg::set_error(FG_ERR_HIP, "launch of %s failed: %s", name,   \
                                   hipGetErrorString(e_));                        \
    } while (0)

#define FG_TRY(expr)                  \
    do {                              \
        int st_ = (expr);             \
        if (st_ != FG_OK) return st_; \
    } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Compute units of the current device (cached per device).
int num_cus();

// Validates an fg_dims (h1 = heads * head_dim, multiples of 64, head_dim 64/128).
int check_dims(const fg_dims* d);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------ launch helpers
// All take device pointers that the public entry points validated.

// Codec over [outer, axis, inner], group 64.
int launch_quant_g4(const __half* x, int64_t outer, int64_t axis, int64_t inner, uint8_t* codes,
                    __half* meta, hipStream_t st);
int launch_dequant_g4(const uint8_t* codes, const __half* meta, int64_t outer, int64_t axis,
                      int64_t inner, __half* y, hipStream_t st);

// GEMM y = act(x W^T + bias) + residual.  ldx / ldy are row strides (elements).
struct LinearArgs {
    const __half* x;
    int64_t M, K, ldx;
    int32_t fmt;
    const void* w;       // fp16 [N, K] or q4 codes [N/2, K]
    const __half* meta;  // q4 meta [N/64, 2, K]
    int64_t N;
    const __half* bias;
    int32_t act;         // 0 none, 1 relu
    const __half* residual;
    __half* y;
    int64_t ldy;
    void* ws;
    size_t ws_bytes;
    // optional: LayerNorm (gamma ln_g, beta ln_b) of every finished output
    // row (width N, requires ldy == N) into ln_y [M, N], fused with the
    // split-k sum where there is one
    const __half* ln_g;
    const __half* ln_b;
    __half* ln_y;
    // optional: which projection of a decoder layer this is (1 QKV, 2 out,
    // 3 FC1, 4 FC2; 0 none), traced as a kind of its own beside the GEMM's
    int32_t proj;
};
int launch_linear(const LinearArgs& a, hipStream_t st);
size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t fmt);
// M rows take the data-parallel (prefill-shaped) GEMM schedule
bool linear_is_dp(int64_t M);
// KV tiering (kvtier.hip): validation of a tier against the device cache
// `dev`, for n_host_seq host sequences of GPU batches of gbs and positions
// below end_pos.
int kvtier_check(const fg_kvtier* kt, const fg_dims* d, const fg_kv* dev, const fg_kv* host,
                 int32_t gbs, int32_t n_host_seq, int32_t end_pos);
// Decode attention of the host-resident GPU batches on the host CPU
// (kvtier.hip, attn_host.cpp), when the tier has a host stage: checks (fp16
// host cache, dense attention, stage size for `rows` host sequences); send:
// the rows' q, k, v to the stage at byte offset `off` and the lane's event
// (lane 0 or 1), on st; attend: wait for that event on the host, compute the
// attention of host sequences seq0 .. seq0 + rows - 1 and append their k, v
// at pos in the host cache on the CPU, copy the attention rows to `out` on
// st.  A lane's stage region is host_stage_bytes(d, its rows).  lanes: the
// tier's two lane compute streams and its start / lane-done events.
bool kvtier_host_attention_on(const fg_kvtier* kt);
size_t host_stage_bytes(const fg_dims* d, int64_t rows);
int kvtier_host_check(const fg_kvtier* kt, const fg_kv* host, const fg_dims* d, int64_t rows, int32_t topk);
int kvtier_host_send(const fg_kvtier* kt, int lane, size_t off, const __half* qkv, int64_t rows, int64_t h1,
                     hipStream_t st);
int kvtier_host_attend(const fg_kvtier* kt, int lane, size_t off, const fg_kv* host, int32_t seq0,
                       const fg_dims* d, int64_t rows, int32_t pos, __half* out, hipStream_t st);
size_t kvtier_host_stage_capacity(const fg_kvtier* kt);
void kvtier_host_lanes(const fg_kvtier* kt, hipStream_t* lane_streams, hipEvent_t* events);
// The host-resident GPU batches ("units") of one call, in execution order,
// moved through the tier object's two slots.  begin(u): loads enqueued
// through unit u + 1 (rows [0, load_rows) each), the compute stream made to
// wait for unit u's, and u's slot returned as a cache of gbs sequences;
// end(u, lo, hi): rows [lo, hi) of the slot copied back to the host after the
// compute stream's work so far.  Units are begun and ended strictly in order,
// each ended before the next is begun.
class KvPipe {
  public:
    KvPipe(fg_kvtier* kt, const fg_dims* d, int32_t gbs, int32_t load_rows, hipStream_t st);
    void add(const fg_kv* host, int32_t seq0);
    int begin(int32_t u, fg_kv* slot);
    int end(int32_t u, int32_t lo, int32_t hi);

  private:
    struct Unit {
        const fg_kv* host;
        int32_t seq0;
    };
    fg_kv slot(int32_t u) const;
    int copy(int32_t u, int32_t lo, int32_t hi, bool to_host);
    fg_kvtier* kt_;
    const fg_dims* d_;
    int32_t gbs_, load_rows_;
    hipStream_t st_;
    std::vector<Unit> unit_;
    int32_t loaded_ = 0, begun_ = 0, stored_ = 0;
};
// KV tier of one layer pass: GPU batches nb_dev.. use host (their first is
// unit u0 of pipe); pipe is null in check-only passes.
struct KvTierCall {
    KvPipe* pipe;
    const fg_kvtier* kt;
    const fg_kv* host;
    int32_t nb_dev;
    int32_t u0;
};
// One decoder layer (layer.hip): arguments validated, then (unless
// check_only) enqueued on st.
// ln1_done: the layer's input LayerNorm is already in the workspace (the
// previous layer fused it); next: if not null, that layer's input LayerNorm is
// fused into this layer's last residual sum.  attn_topk_ppm: Top-K sparse V
// over ceil(pos * ppm / 1e6) cached positions (0 or >= 1e6: dense).
int layer_decode(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs, int32_t nb,
                 int32_t pos, const fg_kv* kv, void* ws, size_t ws_bytes, hipStream_t st,
                 bool check_only, bool ln1_done, const fg_layer_w* next, int32_t attn_topk_ppm,
                 const KvTierCall* kvt);
// Top-K count of a decode step at position pos: -1 (dense) unless
// 0 < ppm < 1e6 selects fewer than pos positions.
int32_t attn_topk_count(int32_t pos, int32_t ppm);
int layer_prefill(const fg_dims* d, const fg_layer_w* w, void* x, int32_t gbs, int32_t nb,
                  int32_t s, const fg_kv* kv, void* ws, size_t ws_bytes, hipStream_t st,
                  bool check_only, const KvTierCall* kvt);
size_t layer_ws_bytes(const fg_dims* d, int64_t rows, int32_t fmt);
// A whole decode step with the host batches' attention on the host CPU,
// overlapped with the GPU's work on the other rows (layer.hip); *used false
// (nothing enqueued) when it does not apply, see the definition.
int model_decode_host_overlap(const fg_dims* d, int32_t n_layers, const fg_layer_w* w, const fg_kv* kv,
                              void* x, int32_t gbs, int32_t nb, int32_t pos, void* ws, size_t ws_bytes,
                              hipStream_t st, const fg_kv_tier* kvt, bool* used);

int launch_layernorm(const __half* x, int64_t rows, int64_t h, const __half* g, const __half* b,
                     __half* y, hipStream_t st);
int launch_embed(const int32_t* tok, const int32_t* pos, int32_t pos_const, int64_t pos_period,
                 int64_t rows, const __half* E, int64_t vocab, const __half* P, int64_t max_pos,
                 int64_t h1, __half* x, hipStream_t st);
int launch_argmax(const __half* logits, int64_t rows, int64_t n, int32_t* out, hipStream_t st);

// KV cache: store nt consecutive positions t0.. of nseq sequences starting at
// sequence seq0.  Row (b, t) of k/v is at k + ((b * nt) + t) * ld.
int launch_kv_store(const __half* k, const __half* v, int64_t ld, const fg_kv* kv, int32_t seq0,
                    int32_t nseq, int32_t t0, int32_t nt, const fg_dims* d, hipStream_t st);
// topk < 0: dense decode attention; topk >= 0: Top-K sparse V (V read for
// the topk cached positions of highest score only)
int launch_attn_decode(const __half* q, const __half* k_new, const __half* v_new, int64_t ld,
                       const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos, int fuse,
                       __half* out, hipStream_t st, int32_t topk = -1);
constexpr int32_t kAttnTopkMaxPos = 8192;   // Top-K: the whole history's scores in LDS
int launch_attn_prefill(const __half* qkv, int32_t b, int32_t s, const fg_dims* d, __half* out,
                        hipStream_t st);

}  // namespace fg
