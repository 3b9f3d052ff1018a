/*
 * CPU oracle for the 4-bit zig-zag block decode of an OPT-style decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library and never calls it.
 *
 * Sources (cited by page title and section):
 *   [P2] "FlexGen 完全拆解:用线性规划编排 GPU、CPU 与 SSD 上的大模型推理"
 *        (pinghaoyang.com.cn), sections "从 Transformer 推理的数据流重新定义卸载"
 *        (prefill/decode projections and the KV append equations),
 *        "权重压缩与 KV Cache 压缩" (the quantize and dequantize equations,
 *        4-bit, group 64, weights grouped along output channels, KV along the
 *        hidden dimension).
 *   [P1] bjbfmj.com FlexGen walkthrough, §6.3 (CompressionConfig: num_bits 4,
 *        group_size 64, group_dim 0 for weights / 2 for the cache, asymmetric;
 *        two 4-bit values packed per uint8; an fp16 scale tensor per group).
 *
 * fp16 values travel as their IEEE binary16 bit patterns (uint16_t).
 * All floating-point reductions run in double; results are rounded to fp16
 * (round-to-nearest-even, one rounding) at every tensor boundary.
 */
#ifndef FG_ORACLE_H
#define FG_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OpenMP threads used by the parallel loops (timing only; results do not
 * depend on it). */
void or_set_threads(int32_t n);
int32_t or_get_threads(void);


/* binary16 <-> double.  or_d2h rounds once, to nearest, ties to even. */
double   or_h2d(uint16_t h);
uint16_t or_d2h(double x);
/* binary16 -> binary32 and binary32 -> binary16 (exact / one RNE rounding) */
float    or_h2f(uint16_t h);
uint16_t or_f2h(float x);

/* Group-wise asymmetric 4-bit min-max codec ([P2] "权重压缩与 KV Cache 压缩";
 * [P1] §6.3).  The tensor is viewed as [outer, axis, inner]; every run of
 * `group` consecutive elements along `axis` (at fixed outer, inner) is one
 * group.  codes: [outer, axis/2, inner] bytes, element 2j of a group pair in
 * the low nibble of byte j, element 2j+1 in the high nibble.
 * meta: [outer, axis/group, 2, inner] fp16 = (min, scale) per group. */
void or_quant_g4(const uint16_t* x, int64_t outer, int64_t axis, int64_t inner,
                 int32_t group, uint8_t* codes, uint16_t* meta);
void or_dequant_g4(const uint8_t* codes, const uint16_t* meta, int64_t outer,
                   int64_t axis, int64_t inner, int32_t group, uint16_t* y);

/* y = LayerNorm(x) * gamma + beta over the last dim h (biased variance). */
void or_layernorm(const uint16_t* x, int64_t rows, int64_t h, const uint16_t* gamma,
                  const uint16_t* beta, double eps, uint16_t* y);

/* y[m,n] = fp16( act( sum_k x[m,k] w[n,k] + bias[n] ) + residual[m,n] ).
 * act = ReLU when relu != 0.  bias / residual may be NULL.  y may alias
 * residual.  Row strides: ldx for x, ldy for y and residual. */
void or_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* w,
               int64_t N, const uint16_t* bias, int32_t relu, const uint16_t* residual,
               uint16_t* y, int64_t ldy);

/* Causal self-attention over a prompt of s tokens per sequence.
 * qkv: [b*s, 3*h1] rows (q | k | v, head h at columns h*hd..h*hd+hd-1 within
 * each third); out: [b*s, h1].  Scores are q.k / sqrt(hd). */
void or_attn_prefill(const uint16_t* qkv, int64_t b, int64_t s, int64_t nh, int64_t hd,
                     uint16_t* out);

/* Single-query attention of decode position `pos`.  Positions 0..pos-1 are
 * read from the history khist / vhist ([b, nh, lmax, hd] fp16, already
 * dequantized when the cache is 4-bit); position pos uses the fresh k, v.
 * q, k_new, v_new: rows of stride ld (elements), head h at h*hd.
 * out: [b, nh*hd]. */
void or_attn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                    int64_t ld, int64_t b, int64_t nh, int64_t hd, const uint16_t* khist,
                    const uint16_t* vhist, int64_t lmax, int64_t pos, uint16_t* out);

/* Decode attention with Top-K sparse V: softmax over every score, V summed
 * over the topk cached positions of highest score (ties: lower position) and
 * the current token, no renormalization. */
void or_attn_decode_topk(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         int64_t ld, int64_t b, int64_t nh, int64_t hd, const uint16_t* khist,
                         const uint16_t* vhist, int64_t lmax, int64_t pos, int64_t topk,
                         uint16_t* out);

/* Embedding: x[r] = fp16(E[tok[r]] + P[pos[r]]). */
void or_embed(const int32_t* tok, const int32_t* pos, int64_t rows, const uint16_t* E,
              const uint16_t* P, int64_t h1, uint16_t* x);

/* Greedy pick: index of the largest fp16 value of each row (lowest on ties). */
void or_argmax(const uint16_t* logits, int64_t rows, int64_t n, int32_t* out);

#ifdef __cplusplus
}
#endif
#endif
