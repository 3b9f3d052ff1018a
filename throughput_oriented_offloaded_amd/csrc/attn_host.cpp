// Decode attention on the host CPU for sequences whose fp16 KV cache lives in
// host memory.
//
// Method ("FlexGen 完全拆解", section "为什么有时应该在 CPU 上算注意力"): when a
// GPU batch's cache already sits on the CPU side and the link is the
// bottleneck, computing that batch's single-query attention on the CPU moves
// only the current token's activations across the link (about 4·b·h1 bytes)
// instead of the cache (about 4·b·s·h1 bytes).  With 4-bit compression the
// pages switch this delegation off (on their host the CPU's dequantization
// costs what the smaller transfer saves); here both fp16 and 4-bit caches are
// delegated, and the 4-bit history is read compressed, dequantized in
// registers (fp32 min + code * scale), its new row quantized on the CPU with
// the codec's exact arithmetic.
//
// Arithmetic (the attention the GPU kernels compute, with roundings of its
// own): scores q·k / sqrt(head_dim) in fp32 from fp16 q and cache rows,
// softmax over the history and the current token, weighted V sum in fp32,
// one rounding to fp16 per output element.  Work items are (sequence, head) pairs; each item's
// arithmetic does not depend on which thread runs it, so results do not
// depend on the thread count.
//
// Host code only: built with the host compiler; AVX2 + FMA + F16C where the
// CPU has them (checked at run time), plain C++ otherwise.
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <condition_variable>
#include <cstring>
#include <limits>
#include <memory>
#include <mutex>
#include <new>
#include <system_error>
#include <thread>
#include <vector>

#include "host_attn.h"

namespace fg {

// ------------------------------------------------------------ thread pool
struct HostPool::State {
    std::vector<std::thread> th;
    std::mutex mu;
    std::condition_variable cv_work, cv_done;
    const std::function<void(int64_t, int64_t)>* f = nullptr;
    int64_t items = 0, chunk = 1;
    std::atomic<int64_t> next{0};
    int pending = 0;      // workers not yet done with the current loop
    uint64_t gen = 0;     // loop number
    bool stop = false;

    void work(const std::function<void(int64_t, int64_t)>* fn, int64_t n, int64_t c) {
        for (;;) {
            const int64_t b = next.fetch_add(c);
            if (b >= n) return;
            (*fn)(b, std::min(b + c, n));
        }
    }
    void worker() {
        uint64_t seen = 0;
        for (;;) {
            std::unique_lock<std::mutex> lk(mu);
            cv_work.wait(lk, [&] { return stop || gen != seen; });
            if (stop) return;
            seen = gen;
            const auto* fn = f;
            const int64_t n = items, c = chunk;
            lk.unlock();
            work(fn, n, c);
            lk.lock();
            if (--pending == 0) cv_done.notify_one();
        }
    }
};

HostPool::HostPool(int n) : s_(new State), nthreads_(1) {
    if (n <= 0) n = (int)std::max(1u, std::thread::hardware_concurrency());
    for (int i = 1; i < n; ++i) {
        try {
            s_->th.emplace_back([this] { s_->worker(); });
        } catch (const std::system_error&) {
            break;   // fewer workers: the loops still run, on fewer threads
        }
    }
    nthreads_ = 1 + (int)s_->th.size();
}

HostPool::~HostPool() {
    {
        std::lock_guard<std::mutex> lk(s_->mu);
        s_->stop = true;
    }
    s_->cv_work.notify_all();
    for (auto& t : s_->th) t.join();
    delete s_;
}

void HostPool::run(int64_t items, const std::function<void(int64_t, int64_t)>& f) {
    if (items <= 0) return;
    const int64_t chunk = std::max<int64_t>(1, items / ((int64_t)nthreads_ * 8));
    if (s_->th.empty()) {
        f(0, items);
        return;
    }
    {
        std::lock_guard<std::mutex> lk(s_->mu);
        s_->f = &f;
        s_->items = items;
        s_->chunk = chunk;
        s_->next.store(0);
        s_->pending = (int)s_->th.size();
        ++s_->gen;
    }
    s_->cv_work.notify_all();
    s_->work(&f, items, chunk);
    std::unique_lock<std::mutex> lk(s_->mu);
    s_->cv_done.wait(lk, [&] { return s_->pending == 0; });
}

namespace {

// ------------------------------------------------------- one (seq, head)
// Inputs of one work item: the fresh q, k, v of the head, its cache rows
// (row p at K + p * hd), the output slot, and the cache row to append at.
struct Item {
    const uint16_t* q;
    const uint16_t* kn;
    const uint16_t* vn;
    uint16_t* K;
    uint16_t* V;
    uint16_t* out;
};

inline float h2f(uint16_t h) {
    _Float16 v;
    std::memcpy(&v, &h, 2);
    return (float)v;
}
inline uint16_t f2h(float f) {
    const _Float16 v = (_Float16)f;   // round to nearest even
    uint16_t h;
    std::memcpy(&h, &v, 2);
    return h;
}

void item_scalar(const Item& it, int hd, int pos, float* s) {
    float qf[256];
    const float scale = 1.0f / std::sqrt((float)hd);
    for (int d = 0; d < hd; ++d) qf[d] = h2f(it.q[d]) * scale;
    auto dot = [&](const uint16_t* r) {
        float a = 0.f;
        for (int d = 0; d < hd; ++d) a += qf[d] * h2f(r[d]);
        return a;
    };
    const float snew = dot(it.kn);
    float m = snew;
    for (int p = 0; p < pos; ++p) {
        s[p] = dot(it.K + (int64_t)p * hd);
        m = std::max(m, s[p]);
    }
    float l = 0.f;
    for (int p = 0; p < pos; ++p) {
        s[p] = std::exp(s[p] - m);
        l += s[p];
    }
    const float en = std::exp(snew - m);
    float acc[256];
    for (int d = 0; d < hd; ++d) acc[d] = 0.f;
    for (int p = 0; p < pos; ++p) {
        const uint16_t* r = it.V + (int64_t)p * hd;
        for (int d = 0; d < hd; ++d) acc[d] += s[p] * h2f(r[d]);
    }
    const float inv = 1.0f / (l + en);
    for (int d = 0; d < hd; ++d) it.out[d] = f2h((acc[d] + en * h2f(it.vn[d])) * inv);
}

#define FG_AVX2 __attribute__((target("avx2,fma,f16c")))

FG_AVX2 inline __m256 ld8(const uint16_t* p) {
    return _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(p)));
}
FG_AVX2 inline float hsum(__m256 v) {
    __m128 a = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
    a = _mm_hadd_ps(a, a);
    a = _mm_hadd_ps(a, a);
    return _mm_cvtss_f32(a);
}
// e^x for x <= 0: x log2(e) = n + f with n = floor, f in [0, 1); 2^f =
// e^(f ln 2) from its Taylor series to degree 7 (relative error below
// 1.4e-6 on [0, ln 2)); 2^n added to the exponent field.  Inputs below -87
// are clamped there (e^-87 is about 1.6e-38, just above the smallest normal
// float), which keeps 2^n normal.
FG_AVX2 inline __m256 exp8(__m256 x) {
    x = _mm256_max_ps(x, _mm256_set1_ps(-87.0f));
    const __m256 t = _mm256_mul_ps(x, _mm256_set1_ps(1.44269504089f));
    const __m256 n = _mm256_floor_ps(t);
    const __m256 g = _mm256_mul_ps(_mm256_sub_ps(t, n), _mm256_set1_ps(0.69314718056f));
    __m256 p = _mm256_set1_ps(1.0f / 5040.0f);
    p = _mm256_fmadd_ps(p, g, _mm256_set1_ps(1.0f / 720.0f));
    p = _mm256_fmadd_ps(p, g, _mm256_set1_ps(1.0f / 120.0f));
    p = _mm256_fmadd_ps(p, g, _mm256_set1_ps(1.0f / 24.0f));
    p = _mm256_fmadd_ps(p, g, _mm256_set1_ps(1.0f / 6.0f));
    p = _mm256_fmadd_ps(p, g, _mm256_set1_ps(0.5f));
    p = _mm256_fmadd_ps(p, g, _mm256_set1_ps(1.0f));
    p = _mm256_fmadd_ps(p, g, _mm256_set1_ps(1.0f));
    const __m256i e = _mm256_slli_epi32(_mm256_cvtps_epi32(n), 23);
    return _mm256_castsi256_ps(_mm256_add_epi32(_mm256_castps_si256(p), e));
}

// q (scaled, NV x 8 floats) . one row of fp16
template <int NV>
FG_AVX2 inline float dotq(const __m256* qv, const uint16_t* r) {
    __m256 a0 = _mm256_setzero_ps(), a1 = _mm256_setzero_ps();
#pragma unroll
    for (int i = 0; i < NV; i += 2) {
        a0 = _mm256_fmadd_ps(ld8(r + 8 * i), qv[i], a0);
        a1 = _mm256_fmadd_ps(ld8(r + 8 * i + 8), qv[i + 1], a1);
    }
    return hsum(_mm256_add_ps(a0, a1));
}

// s: room for pos rounded up to 8 scores
template <int HD>
FG_AVX2 void item_avx2(const Item& it, int pos, float* s) {
    constexpr int NV = HD / 8;
    const __m256 scale = _mm256_set1_ps(1.0f / std::sqrt((float)HD));
    __m256 qv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) qv[i] = _mm256_mul_ps(ld8(it.q + 8 * i), scale);
    auto dot = [&](const uint16_t* r) { return dotq<NV>(qv, r); };
    const float snew = dot(it.kn);
    float m = snew;
    for (int p = 0; p < pos; ++p) {
        s[p] = dot(it.K + (int64_t)p * HD);
        m = std::max(m, s[p]);
    }
    const int pos8 = (pos + 7) & ~7;
    for (int p = pos; p < pos8; ++p) s[p] = -std::numeric_limits<float>::infinity();
    const __m256 mv = _mm256_set1_ps(m);
    __m256 lv = _mm256_setzero_ps();
    for (int p = 0; p < pos8; p += 8) {
        const __m256 e = exp8(_mm256_sub_ps(_mm256_loadu_ps(s + p), mv));
        _mm256_storeu_ps(s + p, e);
        lv = _mm256_add_ps(lv, e);
    }
    const float en = _mm256_cvtss_f32(exp8(_mm256_set1_ps(snew - m)));
    __m256 acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = _mm256_setzero_ps();
    for (int p = 0; p < pos; ++p) {
        const __m256 w = _mm256_set1_ps(s[p]);
        const uint16_t* r = it.V + (int64_t)p * HD;
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = _mm256_fmadd_ps(ld8(r + 8 * i), w, acc[i]);
    }
    const __m256 env = _mm256_set1_ps(en);
    const __m256 inv = _mm256_set1_ps(1.0f / (hsum(lv) + en));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const __m256 o = _mm256_mul_ps(_mm256_fmadd_ps(ld8(it.vn + 8 * i), env, acc[i]), inv);
        _mm_storeu_si128(reinterpret_cast<__m128i*>(it.out + 8 * i),
                         _mm256_cvtps_ph(o, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC));
    }
}

// ------------------------------------------------------ 4-bit cache rows
// One (sequence, head) of a 4-bit cache: per position hd/2 bytes of codes
// (byte i holds dims 2i, low nibble, and 2i + 1) and an fp16 (min, scale)
// pair per 64-dim group.  A cached value is min + code * scale, evaluated in
// fp32 (no fp16 rounding of the dequantized value), so per group
//   q . x = min * sum(q) + scale * sum(q_d code_d)
//   sum_p w_p x_pd = sum_p (w_p scale_p) code_pd + sum_p w_p min_p.
struct ItemQ4 {
    const uint16_t* q;
    const uint16_t* kn;
    const uint16_t* vn;
    uint8_t* K;
    uint8_t* V;
    uint16_t* Km;
    uint16_t* Vm;
    uint16_t* out;
};

// The codec's quantization of one row of hd fp16 values (groups of 64): min
// and max in binary32 with -0 made +0, inv = 15 / range by division, code =
// rint((x - min) * inv) clamped to [0, 15], meta = (fp16(min), fp16(range /
// 15)); one binary32 operation per step and no contraction, so the bytes are
// those of the device quantizer.
void quant_row(const uint16_t* x, int hd, uint8_t* codes, uint16_t* meta) {
#pragma clang fp contract(off)
    for (int g = 0; g < hd / 64; ++g) {
        const uint16_t* xs = x + 64 * g;
        float mn = h2f(xs[0]), mx = mn;
        for (int i = 1; i < 64; ++i) {
            const float v = h2f(xs[i]);
            mn = v < mn ? v : mn;
            mx = v > mx ? v : mx;
        }
        mn = mn + 0.0f;
        mx = mx + 0.0f;
        const float range = mx - mn;
        const float inv = range > 0.0f ? 15.0f / range : 0.0f;
        auto code = [&](uint16_t h) -> unsigned {
            if (!(range > 0.0f)) return 0u;
            const float d = h2f(h) - mn;
            const float r = std::nearbyint(d * inv);
            int q = (int)r;
            q = q < 0 ? 0 : (q > 15 ? 15 : q);
            return (unsigned)q;
        };
        for (int i = 0; i < 32; ++i) codes[32 * g + i] = (uint8_t)(code(xs[2 * i]) | (code(xs[2 * i + 1]) << 4));
        meta[2 * g] = f2h(mn);
        meta[2 * g + 1] = f2h(range / 15.0f);
    }
}

void item_q4_scalar(const ItemQ4& it, int hd, int pos, float* s) {
    const int G = hd / 64, hb = hd / 2;
    float qf[256], sq[4] = {0.f, 0.f, 0.f, 0.f};
    const float scale = 1.0f / std::sqrt((float)hd);
    for (int d = 0; d < hd; ++d) {
        qf[d] = h2f(it.q[d]) * scale;
        sq[d / 64] += qf[d];
    }
    float snew = 0.f;
    for (int d = 0; d < hd; ++d) snew += qf[d] * h2f(it.kn[d]);
    float m = snew;
    for (int p = 0; p < pos; ++p) {
        const uint8_t* c = it.K + (int64_t)p * hb;
        const uint16_t* mm = it.Km + (int64_t)p * 2 * G;
        float a = 0.f;
        for (int g = 0; g < G; ++g) {
            float dg = 0.f;
            for (int i = 0; i < 32; ++i) {
                const unsigned b = c[32 * g + i];
                dg += qf[64 * g + 2 * i] * (float)(b & 15u) + qf[64 * g + 2 * i + 1] * (float)(b >> 4);
            }
            a += h2f(mm[2 * g]) * sq[g] + h2f(mm[2 * g + 1]) * dg;
        }
        s[p] = a;
        m = std::max(m, a);
    }
    float l = 0.f;
    for (int p = 0; p < pos; ++p) {
        s[p] = std::exp(s[p] - m);
        l += s[p];
    }
    const float en = std::exp(snew - m);
    float acc[256], bs[4] = {0.f, 0.f, 0.f, 0.f};
    for (int d = 0; d < hd; ++d) acc[d] = 0.f;
    for (int p = 0; p < pos; ++p) {
        const uint8_t* c = it.V + (int64_t)p * hb;
        const uint16_t* mm = it.Vm + (int64_t)p * 2 * G;
        for (int g = 0; g < G; ++g) {
            const float a = s[p] * h2f(mm[2 * g + 1]);
            bs[g] += s[p] * h2f(mm[2 * g]);
            for (int i = 0; i < 32; ++i) {
                const unsigned b = c[32 * g + i];
                acc[64 * g + 2 * i] += a * (float)(b & 15u);
                acc[64 * g + 2 * i + 1] += a * (float)(b >> 4);
            }
        }
    }
    const float inv = 1.0f / (l + en);
    for (int d = 0; d < hd; ++d) it.out[d] = f2h((acc[d] + bs[d / 64] + en * h2f(it.vn[d])) * inv);
}

// 8 code bytes as 8 int lanes: low nibbles (even dims), high nibbles (odd)
FG_AVX2 inline void nib8(const uint8_t* p, __m256& lo, __m256& hi) {
    const __m256i b = _mm256_cvtepu8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(p)));
    lo = _mm256_cvtepi32_ps(_mm256_and_si256(b, _mm256_set1_epi32(15)));
    hi = _mm256_cvtepi32_ps(_mm256_srli_epi32(b, 4));
}

template <int HD>
FG_AVX2 void item_q4_avx2(const ItemQ4& it, int pos, float* s) {
    constexpr int G = HD / 64, HB = HD / 2, NV = HD / 16;   // NV: 8-byte code chunks per row
    const float scale = 1.0f / std::sqrt((float)HD);
    // q in code order: chunk k lane j is byte 8k + j, i.e. dims 16k + 2j (even) and 16k + 2j + 1 (odd)
    __m256 qe[NV], qo[NV];
    float sq[G];
    {
        alignas(32) float e[HD / 2], o[HD / 2];
        for (int i = 0; i < HD / 2; ++i) {
            e[i] = h2f(it.q[2 * i]) * scale;
            o[i] = h2f(it.q[2 * i + 1]) * scale;
        }
        for (int g = 0; g < G; ++g) {
            float t = 0.f;
            for (int i = 32 * g; i < 32 * g + 32; ++i) t += e[i] + o[i];
            sq[g] = t;
        }
        for (int k = 0; k < NV; ++k) {
            qe[k] = _mm256_load_ps(e + 8 * k);
            qo[k] = _mm256_load_ps(o + 8 * k);
        }
    }
    float snew = 0.f;
    for (int d = 0; d < HD; ++d) snew += h2f(it.q[d]) * scale * h2f(it.kn[d]);
    float m = snew;
    for (int p = 0; p < pos; ++p) {
        const uint8_t* c = it.K + (int64_t)p * HB;
        const uint16_t* mm = it.Km + (int64_t)p * 2 * G;
        __m256 tot = _mm256_setzero_ps();
        float base = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            __m256 a0 = _mm256_setzero_ps(), a1 = _mm256_setzero_ps();
#pragma unroll
            for (int k = 4 * g; k < 4 * g + 4; ++k) {
                __m256 lo, hi;
                nib8(c + 8 * k, lo, hi);
                a0 = _mm256_fmadd_ps(lo, qe[k], a0);
                a1 = _mm256_fmadd_ps(hi, qo[k], a1);
            }
            tot = _mm256_fmadd_ps(_mm256_add_ps(a0, a1), _mm256_set1_ps(h2f(mm[2 * g + 1])), tot);
            base += h2f(mm[2 * g]) * sq[g];
        }
        s[p] = base + hsum(tot);
        m = std::max(m, s[p]);
    }
    const int pos8 = (pos + 7) & ~7;
    for (int p = pos; p < pos8; ++p) s[p] = -std::numeric_limits<float>::infinity();
    const __m256 mv = _mm256_set1_ps(m);
    __m256 lv = _mm256_setzero_ps();
    for (int p = 0; p < pos8; p += 8) {
        const __m256 e = exp8(_mm256_sub_ps(_mm256_loadu_ps(s + p), mv));
        _mm256_storeu_ps(s + p, e);
        lv = _mm256_add_ps(lv, e);
    }
    const float en = _mm256_cvtss_f32(exp8(_mm256_set1_ps(snew - m)));
    __m256 ae[NV], ao[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) ae[k] = ao[k] = _mm256_setzero_ps();
    float bs[G];
    for (int g = 0; g < G; ++g) bs[g] = 0.f;
    for (int p = 0; p < pos; ++p) {
        const uint8_t* c = it.V + (int64_t)p * HB;
        const uint16_t* mm = it.Vm + (int64_t)p * 2 * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const __m256 a = _mm256_set1_ps(s[p] * h2f(mm[2 * g + 1]));
            bs[g] += s[p] * h2f(mm[2 * g]);
#pragma unroll
            for (int k = 4 * g; k < 4 * g + 4; ++k) {
                __m256 lo, hi;
                nib8(c + 8 * k, lo, hi);
                ae[k] = _mm256_fmadd_ps(lo, a, ae[k]);
                ao[k] = _mm256_fmadd_ps(hi, a, ao[k]);
            }
        }
    }
    alignas(32) float e[HD / 2], o[HD / 2];
    for (int k = 0; k < NV; ++k) {
        _mm256_store_ps(e + 8 * k, ae[k]);
        _mm256_store_ps(o + 8 * k, ao[k]);
    }
    const float inv = 1.0f / (hsum(lv) + en);
    for (int i = 0; i < HD / 2; ++i) {
        const float b = bs[i / 32];
        it.out[2 * i] = f2h((e[i] + b + en * h2f(it.vn[2 * i])) * inv);
        it.out[2 * i + 1] = f2h((o[i] + b + en * h2f(it.vn[2 * i + 1])) * inv);
    }
}

#define FG_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx2,fma,f16c")))

// 16 code bytes as 16 int lanes: low nibbles (even dims), high nibbles (odd)
FG_AVX512 inline void nib16(const uint8_t* p, __m512& lo, __m512& hi) {
    const __m512i b = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(p)));
    lo = _mm512_cvtepi32_ps(_mm512_and_si512(b, _mm512_set1_epi32(15)));
    hi = _mm512_cvtepi32_ps(_mm512_srli_epi32(b, 4));
}

// The 4-bit item on 16-lane vectors (the same arithmetic as item_q4_avx2,
// twice the values per instruction; the dequantization is what bounds the
// 4-bit item, where the fp16 one is bound by memory).
template <int HD>
FG_AVX512 void item_q4_avx512(const ItemQ4& it, int pos, float* s) {
    constexpr int G = HD / 64, HB = HD / 2, NV = HD / 32;   // NV: 16-byte code chunks per row
    const float scale = 1.0f / std::sqrt((float)HD);
    // chunk k lane j is byte 16k + j: dims 32k + 2j (even) and 32k + 2j + 1 (odd)
    __m512 qe[NV], qo[NV];
    float sq[G];
    {
        alignas(64) float e[HD / 2], o[HD / 2];
        for (int i = 0; i < HD / 2; ++i) {
            e[i] = h2f(it.q[2 * i]) * scale;
            o[i] = h2f(it.q[2 * i + 1]) * scale;
        }
        for (int g = 0; g < G; ++g) {
            float t = 0.f;
            for (int i = 32 * g; i < 32 * g + 32; ++i) t += e[i] + o[i];
            sq[g] = t;
        }
        for (int k = 0; k < NV; ++k) {
            qe[k] = _mm512_load_ps(e + 16 * k);
            qo[k] = _mm512_load_ps(o + 16 * k);
        }
    }
    float snew = 0.f;
    for (int d = 0; d < HD; ++d) snew += h2f(it.q[d]) * scale * h2f(it.kn[d]);
    float m = snew;
    for (int p = 0; p < pos; ++p) {
        const uint8_t* c = it.K + (int64_t)p * HB;
        const uint16_t* mm = it.Km + (int64_t)p * 2 * G;
        __m512 tot = _mm512_setzero_ps();
        float base = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
#pragma unroll
            for (int k = 2 * g; k < 2 * g + 2; ++k) {
                __m512 lo, hi;
                nib16(c + 16 * k, lo, hi);
                a0 = _mm512_fmadd_ps(lo, qe[k], a0);
                a1 = _mm512_fmadd_ps(hi, qo[k], a1);
            }
            tot = _mm512_fmadd_ps(_mm512_add_ps(a0, a1), _mm512_set1_ps(h2f(mm[2 * g + 1])), tot);
            base += h2f(mm[2 * g]) * sq[g];
        }
        s[p] = base + _mm512_reduce_add_ps(tot);
        m = std::max(m, s[p]);
    }
    const int pos8 = (pos + 7) & ~7;
    for (int p = pos; p < pos8; ++p) s[p] = -std::numeric_limits<float>::infinity();
    const __m256 mv = _mm256_set1_ps(m);
    __m256 lv = _mm256_setzero_ps();
    for (int p = 0; p < pos8; p += 8) {
        const __m256 e = exp8(_mm256_sub_ps(_mm256_loadu_ps(s + p), mv));
        _mm256_storeu_ps(s + p, e);
        lv = _mm256_add_ps(lv, e);
    }
    const float en = _mm256_cvtss_f32(exp8(_mm256_set1_ps(snew - m)));
    __m512 ae[NV], ao[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) ae[k] = ao[k] = _mm512_setzero_ps();
    float bs[G];
    for (int g = 0; g < G; ++g) bs[g] = 0.f;
    for (int p = 0; p < pos; ++p) {
        const uint8_t* c = it.V + (int64_t)p * HB;
        const uint16_t* mm = it.Vm + (int64_t)p * 2 * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const __m512 a = _mm512_set1_ps(s[p] * h2f(mm[2 * g + 1]));
            bs[g] += s[p] * h2f(mm[2 * g]);
#pragma unroll
            for (int k = 2 * g; k < 2 * g + 2; ++k) {
                __m512 lo, hi;
                nib16(c + 16 * k, lo, hi);
                ae[k] = _mm512_fmadd_ps(lo, a, ae[k]);
                ao[k] = _mm512_fmadd_ps(hi, a, ao[k]);
            }
        }
    }
    alignas(64) float e[HD / 2], o[HD / 2];
    for (int k = 0; k < NV; ++k) {
        _mm512_store_ps(e + 16 * k, ae[k]);
        _mm512_store_ps(o + 16 * k, ao[k]);
    }
    const float inv = 1.0f / (hsum(lv) + en);
    for (int i = 0; i < HD / 2; ++i) {
        const float b = bs[i / 32];
        it.out[2 * i] = f2h((e[i] + b + en * h2f(it.vn[2 * i])) * inv);
        it.out[2 * i + 1] = f2h((o[i] + b + en * h2f(it.vn[2 * i + 1])) * inv);
    }
}

// FG_HOST_ATTN_SCALAR=1 runs the plain C++ items and FG_HOST_ATTN_AVX2=1 the
// AVX2 ones, e.g. to test them on a host that has wider extensions.
bool env_on(const char* name) {
    const char* v = getenv(name);
    return v && strcmp(v, "1") == 0;
}

// AVX2 + FMA + F16C present and not switched off
bool have_avx2() {
    static const bool ok = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
                           __builtin_cpu_supports("f16c") && !env_on("FG_HOST_ATTN_SCALAR");
    return ok;
}

// AVX-512 F + BW + VL as well, and not switched off
bool have_avx512() {
    static const bool ok = have_avx2() && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                           __builtin_cpu_supports("avx512vl") && !env_on("FG_HOST_ATTN_AVX2");
    return ok;
}

}  // namespace

int check_host_attn(const void* qkv, int64_t ld, const fg_kv* kv, int32_t seq0, int32_t nseq,
                    const fg_dims* d, int32_t pos, const void* out) {
    int st = check_dims(d);
    if (st != FG_OK) return st;
    if (!qkv || !kv || !out) return set_error(FG_ERR_INVALID, "null pointer argument");
    if (kv->fmt != FG_FMT_F16 && kv->fmt != FG_FMT_Q4G64)
        return set_error(FG_ERR_UNSUPPORTED, "host attention: unknown cache format %d", kv->fmt);
    if (!kv->k || !kv->v || (kv->fmt == FG_FMT_Q4G64 && (!kv->k_meta || !kv->v_meta)))
        return set_error(FG_ERR_INVALID, "null cache tensors");
    if (seq0 < 0 || nseq < 0 || (int64_t)seq0 + nseq > kv->n_seq)
        return set_error(FG_ERR_INVALID, "sequences [%d, %d) outside the cache's %d", seq0, seq0 + nseq,
                         kv->n_seq);
    if (pos < 0 || pos >= kv->max_len)
        return set_error(FG_ERR_INVALID, "pos %d outside [0, max_len %d)", pos, kv->max_len);
    if (ld < 3ll * d->h1) return set_error(FG_ERR_INVALID, "row stride %lld < 3 h1", (long long)ld);
    return FG_OK;
}

int host_attn_decode(const uint16_t* qkv, int64_t ld, const fg_kv* kv, int32_t seq0, int32_t nseq,
                     const fg_dims* d, int32_t pos, bool append, uint16_t* out, HostPool& pool) {
    const int nh = d->n_heads, hd = d->head_dim;
    const int64_t h1 = d->h1, ml = kv->max_len;
    uint16_t* kc = static_cast<uint16_t*>(kv->k);
    uint16_t* vc = static_cast<uint16_t*>(kv->v);
    const bool q4 = kv->fmt == FG_FMT_Q4G64;
    uint8_t* kq = static_cast<uint8_t*>(kv->k);
    uint8_t* vq = static_cast<uint8_t*>(kv->v);
    uint16_t* kmq = static_cast<uint16_t*>(kv->k_meta);
    uint16_t* vmq = static_cast<uint16_t*>(kv->v_meta);
    const int hb = hd / 2, mg = hd / 64 * 2;   // code bytes and meta values per cache row
    const bool avx = have_avx2(), avx512 = have_avx512();
    // nothing may leave a worker by exception (it would end the process, or
    // end run() while other threads still use f): a chunk whose score buffer
    // cannot be allocated is skipped and reported after the loop
    std::atomic<bool> no_mem{false};
    std::function<void(int64_t, int64_t)> f = [&](int64_t b, int64_t e) {
        std::unique_ptr<float[]> buf(new (std::nothrow) float[(size_t)((pos + 7) & ~7) + 8]);
        if (!buf) {
            no_mem.store(true);
            return;
        }
        float* s = buf.get();
        for (int64_t u = b; u < e; ++u) {
            const int64_t sq = u / nh;
            const int h = (int)(u - sq * nh);
            const uint16_t* r = qkv + sq * ld + (int64_t)h * hd;
            uint16_t* o = out + sq * h1 + (int64_t)h * hd;
            const int64_t rows0 = ((seq0 + sq) * nh + h) * ml;   // first cache row of this (sequence, head)
            if (q4) {
                ItemQ4 it{r, r + h1, r + 2 * h1, kq + rows0 * hb, vq + rows0 * hb, kmq + rows0 * mg, vmq + rows0 * mg, o};
                if (avx512 && hd == 64) item_q4_avx512<64>(it, pos, s);
                else if (avx512 && hd == 128) item_q4_avx512<128>(it, pos, s);
                else if (avx && hd == 64) item_q4_avx2<64>(it, pos, s);
                else if (avx && hd == 128) item_q4_avx2<128>(it, pos, s);
                else item_q4_scalar(it, hd, pos, s);
                if (append) {
                    quant_row(it.kn, hd, it.K + (int64_t)pos * hb, it.Km + (int64_t)pos * mg);
                    quant_row(it.vn, hd, it.V + (int64_t)pos * hb, it.Vm + (int64_t)pos * mg);
                }
                continue;
            }
            const int64_t row0 = rows0 * hd;
            Item it{r, r + h1, r + 2 * h1, kc + row0, vc + row0, o};
            if (avx && hd == 64) item_avx2<64>(it, pos, s);
            else if (avx && hd == 128) item_avx2<128>(it, pos, s);
            else item_scalar(it, hd, pos, s);
            if (append) {
                std::memcpy(it.K + (int64_t)pos * hd, it.kn, (size_t)hd * 2);
                std::memcpy(it.V + (int64_t)pos * hd, it.vn, (size_t)hd * 2);
            }
        }
    };
    pool.run((int64_t)nseq * nh, f);
    if (no_mem.load()) return set_error(FG_ERR_CAPACITY, "host attention: out of host memory");
    return FG_OK;
}

}  // namespace fg

namespace {
int host_attn_entry(int32_t fmt, const void* qkv, int64_t ld, const fg_kv* kv, int32_t seq0, int32_t nseq,
                    const fg_dims* d, int32_t pos, int32_t append, void* out, int32_t n_threads) {
    fg::clear_error();
    if (kv && kv->fmt != fmt)
        return fg::set_error(FG_ERR_UNSUPPORTED, "host attention: a cache of format %d given to the %s entry point",
                             kv->fmt, fmt == FG_FMT_Q4G64 ? "4-bit" : "fp16");
    int st = fg::check_host_attn(qkv, ld, kv, seq0, nseq, d, pos, out);
    if (st != FG_OK) return st;
    try {
        fg::HostPool pool(n_threads);
        return fg::host_attn_decode(static_cast<const uint16_t*>(qkv), ld, kv, seq0, nseq, d, pos, append != 0,
                                    static_cast<uint16_t*>(out), pool);
    } catch (const std::bad_alloc&) {
        return fg::set_error(FG_ERR_CAPACITY, "host attention: out of host memory");
    }
}
}  // namespace

extern "C" int fg_attn_decode_host_f16(const void* qkv, int64_t ld, const fg_kv* kv, int32_t seq0,
                                       int32_t nseq, const fg_dims* d, int32_t pos, int32_t append,
                                       void* out, int32_t n_threads) {
    return host_attn_entry(FG_FMT_F16, qkv, ld, kv, seq0, nseq, d, pos, append, out, n_threads);
}

extern "C" int fg_attn_decode_host_q4(const void* qkv, int64_t ld, const fg_kv* kv, int32_t seq0,
                                      int32_t nseq, const fg_dims* d, int32_t pos, int32_t append,
                                      void* out, int32_t n_threads) {
    return host_attn_entry(FG_FMT_Q4G64, qkv, ld, kv, seq0, nseq, d, pos, append, out, n_threads);
}
