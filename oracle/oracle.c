/*
 * CPU oracle for the 4-bit zig-zag block decode of an OPT-style decoder.
 *
 * TEST INFRASTRUCTURE ONLY: the definition the GPU library is checked
 * against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no -ffast-math:
 * the codec depends on IEEE binary32 semantics, one operation at a time).
 * OpenMP only splits independent output rows, groups or (sequence, head)
 * pairs; every reduction runs serially in double, in index order.
 *
 * Page citations are given per function; see oracle.h for the page titles.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdlib.h>

/* ------------------------------------------------------------- threading */
/* Number of OpenMP threads the parallel loops below use (timing of the CPU
 * baseline at one thread and at all cores); no effect on any result. */
void or_set_threads(int32_t n) { omp_set_num_threads(n > 0 ? n : 1); }
int32_t or_get_threads(void) { return (int32_t)omp_get_max_threads(); }

/* ---------------------------------------------------------------- binary16 */
/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 holds zero and subnormals (value = frac * 2^-24). */

double or_h2d(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

uint16_t or_d2h(double x) {
    if (isnan(x)) return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: integer multiple of 2^-24, nearest-even.  A result
         * of 1024 is the bit pattern of the smallest normal, as it should be. */
        double q = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)q;
    }
    int E;
    frexp(a, &E);                 /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                /* a in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(a, 10 - e));   /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e > 15) return sign | 0x7C00;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024);
}

float or_h2f(uint16_t h) { return (float)or_h2d(h); }
uint16_t or_f2h(float x) { return or_d2h((double)x); }

/* The 65536 binary16 values as doubles, filled from or_h2d when the library
 * loads; it only saves repeating the same decode in the inner loops. */
static double h2d_tab[65536];
__attribute__((constructor)) static void fill_h2d_tab(void) {
    for (int i = 0; i < 65536; ++i) h2d_tab[i] = or_h2d((uint16_t)i);
}
#define H2D(h) (h2d_tab[(uint16_t)(h)])

/* ------------------------------------------------------------------- codec */
/* [P2] "权重压缩与 KV Cache 压缩": q(x) = round((x - x_min) / (x_max - x_min)
 * * (2^b - 1)), b = 4; dequantization x^ = x_min + q / (2^b - 1) *
 * (x_max - x_min), i.e. x_min plus q times the scale (x_max - x_min)/15.
 * [P1] §6.3: groups of 64, two 4-bit values per byte, fp16 scale tensor.
 *
 * Arithmetic, in binary32, one rounding per operation:
 *   mn, mx = min, max of the group; -0 is canonicalised to +0 (mn + 0.0f);
 *   range = mx - mn;
 *   range > 0: inv = 15 / range (one division per group), q = rint((x - mn) * inv)
 *              (nearest, ties to even), clamped to [0, 15];
 *   range == 0: q = 0 (constant group, reconstructed as mn exactly);
 *   meta = (fp16(mn), fp16(range / 15)).
 * Dequantization: x^ = fp16(mn + q * scale), multiply then add. */

static inline int64_t code_index(int64_t o, int64_t a, int64_t i, int64_t axis, int64_t inner) {
    return (o * (axis / 2) + a / 2) * inner + i;
}

static inline int64_t meta_index(int64_t o, int64_t g, int64_t which, int64_t ngroups,
                                 int64_t inner, int64_t i) {
    return ((o * ngroups + g) * 2 + which) * inner + i;
}

void or_quant_g4(const uint16_t* x, int64_t outer, int64_t axis, int64_t inner,
                 int32_t group, uint8_t* codes, uint16_t* meta) {
    const int64_t ngroups = axis / group;
    const int64_t units = outer * ngroups;
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t o = u / ngroups, g = u % ngroups;
        for (int64_t i = 0; i < inner; ++i) {
            float mn = INFINITY, mx = -INFINITY;
            for (int64_t j = 0; j < group; ++j) {
                float v = or_h2f(x[(o * axis + g * group + j) * inner + i]);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            mn = mn + 0.0f;
            mx = mx + 0.0f;
            const float range = mx - mn;
            const float inv = range > 0.0f ? 15.0f / range : 0.0f;
            for (int64_t j = 0; j < group; j += 2) {
                int qq[2];
                for (int t = 0; t < 2; ++t) {
                    int q = 0;
                    if (range > 0.0f) {
                        float v = or_h2f(x[(o * axis + g * group + j + t) * inner + i]);
                        float d = v - mn;
                        float r = rintf(d * inv);
                        q = (int)r;
                        if (q < 0) q = 0;
                        if (q > 15) q = 15;
                    }
                    qq[t] = q;
                }
                codes[code_index(o, g * group + j, i, axis, inner)] =
                    (uint8_t)(qq[0] | (qq[1] << 4));
            }
            meta[meta_index(o, g, 0, ngroups, inner, i)] = or_f2h(mn);
            meta[meta_index(o, g, 1, ngroups, inner, i)] = or_f2h(range / 15.0f);
        }
    }
}

void or_dequant_g4(const uint8_t* codes, const uint16_t* meta, int64_t outer,
                   int64_t axis, int64_t inner, int32_t group, uint16_t* y) {
    const int64_t ngroups = axis / group;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t a = 0; a < axis; ++a) {
            const int64_t g = a / group;
            for (int64_t i = 0; i < inner; ++i) {
                uint8_t byte = codes[code_index(o, a, i, axis, inner)];
                int q = (a % 2 == 0) ? (byte & 15) : (byte >> 4);
                float mn = or_h2f(meta[meta_index(o, g, 0, ngroups, inner, i)]);
                float sc = or_h2f(meta[meta_index(o, g, 1, ngroups, inner, i)]);
                float t = (float)q * sc;
                float r = mn + t;
                y[(o * axis + a) * inner + i] = or_f2h(r);
            }
        }
    }
}

/* -------------------------------------------------------------- LayerNorm */
/* Pre-LN decoder: normalise each row to zero mean and unit (biased)
 * variance, then scale by gamma and shift by beta. */
void or_layernorm(const uint16_t* x, int64_t rows, int64_t h, const uint16_t* gamma,
                  const uint16_t* beta, double eps, uint16_t* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * h;
        double mean = 0.0;
        for (int64_t j = 0; j < h; ++j) mean += H2D(xr[j]);
        mean /= (double)h;
        double var = 0.0;
        for (int64_t j = 0; j < h; ++j) {
            double d = H2D(xr[j]) - mean;
            var += d * d;
        }
        var /= (double)h;
        const double rstd = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < h; ++j) {
            double v = (H2D(xr[j]) - mean) * rstd * H2D(gamma[j]) + H2D(beta[j]);
            y[r * h + j] = or_d2h(v);
        }
    }
}

/* ------------------------------------------------------------------ linear */
/* [P2] "从 Transformer 推理的数据流重新定义卸载": K = X W_K, V = X W_V,
 * Q = X W_Q and the MLP matrices.  Weights are stored [N = out, K = in], so
 * each output is the dot product of an input row with a weight row. */
void or_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* w,
               int64_t N, const uint16_t* bias, int32_t relu, const uint16_t* residual,
               uint16_t* y, int64_t ldy) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t* wr = w + n * K;
        for (int64_t m = 0; m < M; ++m) {
            const uint16_t* xr = x + m * ldx;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += H2D(xr[k]) * H2D(wr[k]);
            if (bias) acc += H2D(bias[n]);
            if (relu && acc < 0.0) acc = 0.0;
            if (residual) acc += H2D(residual[m * ldy + n]);
            y[m * ldy + n] = or_d2h(acc);
        }
    }
}

/* --------------------------------------------------------------- attention */
/* Scaled dot-product attention, softmax(q k^T / sqrt(hd)) v, computed with
 * the row maximum subtracted before exponentiation (an identity of softmax). */

void or_attn_prefill(const uint16_t* qkv, int64_t b, int64_t s, int64_t nh, int64_t hd,
                     uint16_t* out) {
    const int64_t h1 = nh * hd, ld = 3 * h1;
    const double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t bi = 0; bi < b; ++bi) {
        for (int64_t h = 0; h < nh; ++h) {
            double sc[s > 0 ? s : 1];
            for (int64_t t = 0; t < s; ++t) {
                const uint16_t* q = qkv + (bi * s + t) * ld + h * hd;
                double mx = -INFINITY;
                for (int64_t j = 0; j <= t; ++j) {   /* causal: keys 0..t */
                    const uint16_t* k = qkv + (bi * s + j) * ld + h1 + h * hd;
                    double d = 0.0;
                    for (int64_t c = 0; c < hd; ++c) d += H2D(q[c]) * H2D(k[c]);
                    sc[j] = d * scale;
                    if (sc[j] > mx) mx = sc[j];
                }
                double sum = 0.0;
                for (int64_t j = 0; j <= t; ++j) {
                    sc[j] = exp(sc[j] - mx);
                    sum += sc[j];
                }
                for (int64_t c = 0; c < hd; ++c) {
                    double o = 0.0;
                    for (int64_t j = 0; j <= t; ++j)
                        o += sc[j] * H2D(qkv[(bi * s + j) * ld + 2 * h1 + h * hd + c]);
                    out[(bi * s + t) * h1 + h * hd + c] = or_d2h(o / sum);
                }
            }
        }
    }
}

void or_attn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                    int64_t ld, int64_t b, int64_t nh, int64_t hd, const uint16_t* khist,
                    const uint16_t* vhist, int64_t lmax, int64_t pos, uint16_t* out) {
    const int64_t h1 = nh * hd;
    const double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t bi = 0; bi < b; ++bi) {
        for (int64_t h = 0; h < nh; ++h) {
            double sc[pos + 1];
            const uint16_t* qr = q + bi * ld + h * hd;
            const uint16_t* kh = khist + (bi * nh + h) * lmax * hd;
            const uint16_t* vh = vhist + (bi * nh + h) * lmax * hd;
            double mx = -INFINITY;
            for (int64_t p = 0; p <= pos; ++p) {
                const uint16_t* kr = (p < pos) ? kh + p * hd : k_new + bi * ld + h * hd;
                double d = 0.0;
                for (int64_t c = 0; c < hd; ++c) d += H2D(qr[c]) * H2D(kr[c]);
                sc[p] = d * scale;
                if (sc[p] > mx) mx = sc[p];
            }
            double sum = 0.0;
            for (int64_t p = 0; p <= pos; ++p) {
                sc[p] = exp(sc[p] - mx);
                sum += sc[p];
            }
            for (int64_t c = 0; c < hd; ++c) {
                double o = 0.0;
                for (int64_t p = 0; p <= pos; ++p) {
                    const uint16_t* vr = (p < pos) ? vh + p * hd : v_new + bi * ld + h * hd;
                    o += sc[p] * H2D(vr[c]);
                }
                out[bi * h1 + h * hd + c] = or_d2h(o / sum);
            }
        }
    }
}

/* Top-K sparse-V decode attention ([P2] "权重压缩与 KV Cache 压缩": scores
 * from all Keys, then only the Values of the highest-scoring 10% are loaded).
 * Readings where the page is silent: the softmax is over every score (all
 * are computed); the V sum covers the topk cached positions of highest score
 * (ties: lower position first) plus the current token, whose fresh v needs no
 * cache read; the weights are not renormalized over the selected set. */
typedef struct {
    double s;
    int64_t p;
} or_scored;

static int or_scored_desc(const void* a, const void* b) {
    const or_scored* x = (const or_scored*)a;
    const or_scored* y = (const or_scored*)b;
    if (x->s != y->s) return x->s > y->s ? -1 : 1;
    return x->p < y->p ? -1 : (x->p > y->p ? 1 : 0);
}

void or_attn_decode_topk(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         int64_t ld, int64_t b, int64_t nh, int64_t hd, const uint16_t* khist,
                         const uint16_t* vhist, int64_t lmax, int64_t pos, int64_t topk,
                         uint16_t* out) {
    const int64_t h1 = nh * hd;
    const double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t bi = 0; bi < b; ++bi) {
        for (int64_t h = 0; h < nh; ++h) {
            double sc[pos + 1];
            or_scored order[pos > 0 ? pos : 1];
            unsigned char sel[pos > 0 ? pos : 1];
            const uint16_t* qr = q + bi * ld + h * hd;
            const uint16_t* kh = khist + (bi * nh + h) * lmax * hd;
            const uint16_t* vh = vhist + (bi * nh + h) * lmax * hd;
            double mx = -INFINITY;
            for (int64_t p = 0; p <= pos; ++p) {
                const uint16_t* kr = (p < pos) ? kh + p * hd : k_new + bi * ld + h * hd;
                double d = 0.0;
                for (int64_t c = 0; c < hd; ++c) d += H2D(qr[c]) * H2D(kr[c]);
                sc[p] = d * scale;
                if (sc[p] > mx) mx = sc[p];
            }
            /* the topk cached positions of highest score */
            for (int64_t p = 0; p < pos; ++p) {
                order[p].s = sc[p];
                order[p].p = p;
                sel[p] = 0;
            }
            qsort(order, (size_t)pos, sizeof(or_scored), or_scored_desc);
            for (int64_t i = 0; i < topk && i < pos; ++i) sel[order[i].p] = 1;
            /* softmax weights over every position */
            double sum = 0.0;
            for (int64_t p = 0; p <= pos; ++p) {
                sc[p] = exp(sc[p] - mx);
                sum += sc[p];
            }
            for (int64_t c = 0; c < hd; ++c) {
                double o = 0.0;
                for (int64_t p = 0; p <= pos; ++p) {
                    if (p < pos && !sel[p]) continue;
                    const uint16_t* vr = (p < pos) ? vh + p * hd : v_new + bi * ld + h * hd;
                    o += sc[p] * H2D(vr[c]);
                }
                out[bi * h1 + h * hd + c] = or_d2h(o / sum);
            }
        }
    }
}

/* ------------------------------------------------------- embedding, argmax */
void or_embed(const int32_t* tok, const int32_t* pos, int64_t rows, const uint16_t* E,
              const uint16_t* P, int64_t h1, uint16_t* x) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < h1; ++j)
            x[r * h1 + j] = or_d2h(H2D(E[(int64_t)tok[r] * h1 + j]) +
                                   H2D(P[(int64_t)pos[r] * h1 + j]));
}

void or_argmax(const uint16_t* logits, int64_t rows, int64_t n, int32_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t best = 0;
        double bv = H2D(logits[r * n]);
        for (int64_t j = 1; j < n; ++j) {
            double v = H2D(logits[r * n + j]);
            if (v > bv) { bv = v; best = j; }
        }
        out[r] = (int32_t)best;
    }
}
