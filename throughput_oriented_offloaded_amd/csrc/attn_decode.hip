// Decode attention over a 4-bit (or fp16) KV cache, with the new token's K, V
// appended in the same launch, and the kernel that stores K, V rows into the
// cache (prompt positions after the prefill, or one appended position).
//
// Method ("FlexGen 完全拆解", section "从 Transformer 推理的数据流重新定义卸载"):
// at decode step t the single query of each sequence attends to all s+t cached
// keys; the cache grows by Concat(K_{1:s+t-1}, X_t W_K) (same for V).  The
// cache is stored group-wise 4-bit with groups of 64 along one head's hidden
// dim (section "权重压缩与 KV Cache 压缩"; bjbfmj.com walkthrough §6.3
// group_dim 2) and dequantized in registers while it streams.
//
// Mapping (MI355X, wave64): one wavefront per (sequence, head).  A lane owns
// 32 consecutive dims of the head (16 B of codes, inside one 64-group) and one
// "slot" of positions: hd=128 -> 4 lanes per position, 16 positions per
// wavefront step; hd=64 -> 2 lanes per position, 32 per step.  Each lane keeps
// its own online-softmax state (running max, sum, 32 accumulators) over the
// positions of its slot; the slots are merged once at the end with wavefront
// shuffles.  No LDS and no barriers: the kernel is a pure HBM stream of
// codes + metadata (9/16 byte per cached element).
//
// Reading of the current token (stated in fg.h): positions < pos come from the
// cache; position pos uses the fresh fp16 k, v.
//
// Score with 4-bit keys, per lane (its dims D inside group g):
//   sum_{d in D} q_d (mn_g + sc_g c_d) = mn_g * sum_D q_d + sc_g * sum_D q_d c_d,
// so each element costs one byte->float conversion and one FMA.  V is
// accumulated the same way: acc_d += (w sc) c_d, plus one scalar w mn per lane.
#include "codec_dev.h"
#include "fg_internal.h"
#include "fg_trace.h"

namespace fg {
namespace {

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float lo_half(uint32_t w) {
    return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu)));
}
__device__ __forceinline__ float hi_half(uint32_t w) {
    return __half2float(__ushort_as_half((unsigned short)(w >> 16)));
}

// Byte j of a dword as float (compiles to v_cvt_f32_ubyte{j}).
template <int J>
__device__ __forceinline__ float ub(uint32_t w) {
    return (float)((w >> (8 * J)) & 0xffu);
}

// sum_{i<32} q[i] * code_i over 16 bytes of packed nibbles (element 2j of a
// byte pair in the low nibble).
__device__ __forceinline__ float dot_codes(const uint4& c, const float q[32]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x0f0f0f0fu;
        const uint32_t hi = (w[k] >> 4) & 0x0f0f0f0fu;
        s0 = fmaf(q[8 * k + 0], ub<0>(lo), s0);
        s1 = fmaf(q[8 * k + 1], ub<0>(hi), s1);
        s0 = fmaf(q[8 * k + 2], ub<1>(lo), s0);
        s1 = fmaf(q[8 * k + 3], ub<1>(hi), s1);
        s0 = fmaf(q[8 * k + 4], ub<2>(lo), s0);
        s1 = fmaf(q[8 * k + 5], ub<2>(hi), s1);
        s0 = fmaf(q[8 * k + 6], ub<3>(lo), s0);
        s1 = fmaf(q[8 * k + 7], ub<3>(hi), s1);
    }
    return s0 + s1;
}

__device__ __forceinline__ void acc_codes(const uint4& c, float ws, float acc[32]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x0f0f0f0fu;
        const uint32_t hi = (w[k] >> 4) & 0x0f0f0f0fu;
        acc[8 * k + 0] = fmaf(ws, ub<0>(lo), acc[8 * k + 0]);
        acc[8 * k + 1] = fmaf(ws, ub<0>(hi), acc[8 * k + 1]);
        acc[8 * k + 2] = fmaf(ws, ub<1>(lo), acc[8 * k + 2]);
        acc[8 * k + 3] = fmaf(ws, ub<1>(hi), acc[8 * k + 3]);
        acc[8 * k + 4] = fmaf(ws, ub<2>(lo), acc[8 * k + 4]);
        acc[8 * k + 5] = fmaf(ws, ub<2>(hi), acc[8 * k + 5]);
        acc[8 * k + 6] = fmaf(ws, ub<3>(lo), acc[8 * k + 6]);
        acc[8 * k + 7] = fmaf(ws, ub<3>(hi), acc[8 * k + 7]);
    }
}

__device__ __forceinline__ void load32h(const __half* p, float v[32]) {
    const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint4 r = p4[k];
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * k + 2 * j] = lo_half(w[j]);
            v[8 * k + 2 * j + 1] = hi_half(w[j]);
        }
    }
}

// Quantize 32 fp16 values that form half of a 64-group whose other half sits
// in the neighbouring lane (lane ^ 1); returns the 16 code bytes and the
// (min, scale) fp16 bits of the group.
__device__ __forceinline__ uint4 quant_half_group(const float v[32], uint32_t& meta_bits) {
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
        mn = fminf(mn, v[i]);
        mx = fmaxf(mx, v[i]);
    }
    mn = fminf(mn, __shfl_xor(mn, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    const QParams p = qparams(mn, mx);
    meta_bits = qmeta_bits(p);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) x |= qcode(v[8 * k + j], p) << (4 * j);
        w[k] = x;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int HD, bool Q4, int U>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const __half* __restrict__ q, const __half* __restrict__ k_new,
    const __half* __restrict__ v_new, int64_t ld, void* __restrict__ kc,
    __half* __restrict__ km, void* __restrict__ vc, __half* __restrict__ vm, int32_t lmax,
    int32_t nh, int32_t bls, int32_t pos, int fuse, __half* __restrict__ out) {
    constexpr int LPP = HD / 32;       // lanes per position
    constexpr int SLOTS = 64 / LPP;    // positions per wavefront step
    constexpr int GPH = HD / 64;       // 64-groups per head
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, h)
    if (unit >= (int64_t)bls * nh) return;
    const int64_t b = unit / nh;
    const int h = (int)(unit % nh);
    const int qi = lane % LPP;          // which 32 dims
    const int slot = lane / LPP;
    const int g = (qi * 32) / 64;       // group of those dims

    // q pre-scaled so that scores come out in log2 units
    const float qs = LOG2E / sqrtf((float)HD);
    float qv[32];
    load32h(q + b * ld + h * HD + qi * 32, qv);
    float qsum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        qv[i] *= qs;
        qsum += qv[i];
    }

    const int64_t head_row0 = unit * (int64_t)lmax;   // cache row of (b, h, position 0)
    float m = -INFINITY, l = 0.f, accm = 0.f;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;

    for (int base = 0; base < pos; base += SLOTS * U) {
        float sc[U];
        if constexpr (Q4) {
            uint4 kcode[U], vcode[U];
            uint32_t kmeta[U], vmeta[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = base + u * SLOTS + slot;
                if (p < pos) {
                    const int64_t row = head_row0 + p;
                    kcode[u] = *reinterpret_cast<const uint4*>((const uint8_t*)kc + row * (HD / 2) + qi * 16);
                    vcode[u] = *reinterpret_cast<const uint4*>((const uint8_t*)vc + row * (HD / 2) + qi * 16);
                    kmeta[u] = *reinterpret_cast<const uint32_t*>(km + (row * GPH + g) * 2);
                    vmeta[u] = *reinterpret_cast<const uint32_t*>(vm + (row * GPH + g) * 2);
                } else {
                    kcode[u] = vcode[u] = make_uint4(0, 0, 0, 0);
                    kmeta[u] = vmeta[u] = 0;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float part = lo_half(kmeta[u]) * qsum + hi_half(kmeta[u]) * dot_codes(kcode[u], qv);
#pragma unroll
                for (int off = 1; off < LPP; off <<= 1) part += __shfl_xor(part, off);
                sc[u] = (base + u * SLOTS + slot < pos) ? part : -INFINITY;
            }
            float mnew = m;
#pragma unroll
            for (int u = 0; u < U; ++u) mnew = fmaxf(mnew, sc[u]);
            if (mnew != -INFINITY) {
                const float alpha = exp2f(m - mnew);
                l *= alpha;
                accm *= alpha;
#pragma unroll
                for (int i = 0; i < 32; ++i) acc[i] *= alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float w = exp2f(sc[u] - mnew);
                    l += w;
                    accm = fmaf(w, lo_half(vmeta[u]), accm);
                    acc_codes(vcode[u], w * hi_half(vmeta[u]), acc);
                }
                m = mnew;
            }
        } else {
            float kv[U][32];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = base + u * SLOTS + slot;
                if (p < pos) {
                    load32h((const __half*)kc + (head_row0 + p) * HD + qi * 32, kv[u]);
                } else {
#pragma unroll
                    for (int i = 0; i < 32; ++i) kv[u][i] = 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) part = fmaf(qv[i], kv[u][i], part);
#pragma unroll
                for (int off = 1; off < LPP; off <<= 1) part += __shfl_xor(part, off);
                sc[u] = (base + u * SLOTS + slot < pos) ? part : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = base + u * SLOTS + slot;
                if (p < pos) {
                    load32h((const __half*)vc + (head_row0 + p) * HD + qi * 32, kv[u]);
                } else {
#pragma unroll
                    for (int i = 0; i < 32; ++i) kv[u][i] = 0.f;
                }
            }
            float mnew = m;
#pragma unroll
            for (int u = 0; u < U; ++u) mnew = fmaxf(mnew, sc[u]);
            if (mnew != -INFINITY) {
                const float alpha = exp2f(m - mnew);
                l *= alpha;
#pragma unroll
                for (int i = 0; i < 32; ++i) acc[i] *= alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float w = exp2f(sc[u] - mnew);
                    l += w;
#pragma unroll
                    for (int i = 0; i < 32; ++i) acc[i] = fmaf(w, kv[u][i], acc[i]);
                }
                m = mnew;
            }
        }
    }

    // the current token: fresh fp16 k, v
    float kn[32], vn[32];
    load32h(k_new + b * ld + h * HD + qi * 32, kn);
    load32h(v_new + b * ld + h * HD + qi * 32, vn);
    float snew = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) snew = fmaf(qv[i], kn[i], snew);
#pragma unroll
    for (int off = 1; off < LPP; off <<= 1) snew += __shfl_xor(snew, off);

    // merge the slots of the wavefront
    float M = fmaxf(m, snew);
#pragma unroll
    for (int off = LPP; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = (m == -INFINITY) ? 0.f : exp2f(m - M);
    l *= f;
    accm *= f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= f;
#pragma unroll
    for (int off = LPP; off < 64; off <<= 1) {
        l += __shfl_xor(l, off);
        accm += __shfl_xor(accm, off);
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] += __shfl_xor(acc[i], off);
    }
    const float wn = exp2f(snew - M);
    const float inv = 1.0f / (l + wn);

    if (slot == 0) {
        uint32_t o[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float a0 = (acc[2 * j] + accm + wn * vn[2 * j]) * inv;
            const float a1 = (acc[2 * j + 1] + accm + wn * vn[2 * j + 1]) * inv;
            o[j] = (uint32_t)__half_as_ushort(__float2half_rn(a0)) |
                   ((uint32_t)__half_as_ushort(__float2half_rn(a1)) << 16);
        }
        uint4* op = reinterpret_cast<uint4*>(out + b * (int64_t)nh * HD + h * HD + qi * 32);
#pragma unroll
        for (int k = 0; k < 4; ++k) op[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
    }

    if (fuse) {
        const int64_t row = head_row0 + pos;
        if constexpr (Q4) {
            uint32_t kmb, vmb;
            const uint4 kq = quant_half_group(kn, kmb);   // all lanes: shuffles need the full wave
            const uint4 vq = quant_half_group(vn, vmb);
            if (slot == 0) {
                *reinterpret_cast<uint4*>((uint8_t*)kc + row * (HD / 2) + qi * 16) = kq;
                *reinterpret_cast<uint4*>((uint8_t*)vc + row * (HD / 2) + qi * 16) = vq;
                if ((qi & 1) == 0) {
                    *reinterpret_cast<uint32_t*>(km + (row * GPH + g) * 2) = kmb;
                    *reinterpret_cast<uint32_t*>(vm + (row * GPH + g) * 2) = vmb;
                }
            }
        } else if (slot == 0) {
            const uint4* ks = reinterpret_cast<const uint4*>(k_new + b * ld + h * HD + qi * 32);
            const uint4* vs = reinterpret_cast<const uint4*>(v_new + b * ld + h * HD + qi * 32);
            uint4* kd = reinterpret_cast<uint4*>((__half*)kc + row * HD + qi * 32);
            uint4* vd = reinterpret_cast<uint4*>((__half*)vc + row * HD + qi * 32);
#pragma unroll
            for (int k = 0; k < 4; ++k) { kd[k] = ks[k]; vd[k] = vs[k]; }
        }
    }
}

// Store nt positions (t0..t0+nt-1) of nseq sequences (seq0..) into the cache.
// One wavefront per (sequence, head); lanes as in the attention kernel.
template <int HD, bool Q4>
__global__ __launch_bounds__(256) void kv_store_kernel(const __half* __restrict__ k,
                                                       const __half* __restrict__ v, int64_t ld,
                                                       void* __restrict__ kc, __half* __restrict__ km,
                                                       void* __restrict__ vc, __half* __restrict__ vm,
                                                       int32_t lmax, int32_t nh, int32_t seq0,
                                                       int32_t nseq, int32_t t0, int32_t nt) {
    constexpr int LPP = HD / 32;
    constexpr int SLOTS = 64 / LPP;
    constexpr int GPH = HD / 64;
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= (int64_t)nseq * nh) return;
    const int64_t bl = unit / nh;   // sequence within this call
    const int h = (int)(unit % nh);
    const int qi = lane % LPP, slot = lane / LPP, g = (qi * 32) / 64;
    const int64_t head_row0 = ((seq0 + bl) * (int64_t)nh + h) * lmax;
    for (int base = 0; base < nt; base += SLOTS) {
        const int t = base + slot;
        const bool ok = t < nt;    // whole 4- or 2-lane groups agree
        const int tt = ok ? t : nt - 1;
        const __half* ks = k + (bl * nt + tt) * ld + h * HD + qi * 32;
        const __half* vs = v + (bl * nt + tt) * ld + h * HD + qi * 32;
        const int64_t row = head_row0 + t0 + tt;
        if constexpr (Q4) {
            float kv[32], vv[32];
            load32h(ks, kv);
            load32h(vs, vv);
            uint32_t kmb, vmb;
            const uint4 kq = quant_half_group(kv, kmb);
            const uint4 vq = quant_half_group(vv, vmb);
            if (ok) {
                *reinterpret_cast<uint4*>((uint8_t*)kc + row * (HD / 2) + qi * 16) = kq;
                *reinterpret_cast<uint4*>((uint8_t*)vc + row * (HD / 2) + qi * 16) = vq;
                if ((qi & 1) == 0) {
                    *reinterpret_cast<uint32_t*>(km + (row * GPH + g) * 2) = kmb;
                    *reinterpret_cast<uint32_t*>(vm + (row * GPH + g) * 2) = vmb;
                }
            }
        } else if (ok) {
            const uint4* k4 = reinterpret_cast<const uint4*>(ks);
            const uint4* v4 = reinterpret_cast<const uint4*>(vs);
            uint4* kd = reinterpret_cast<uint4*>((__half*)kc + row * HD + qi * 32);
            uint4* vd = reinterpret_cast<uint4*>((__half*)vc + row * HD + qi * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) { kd[j] = k4[j]; vd[j] = v4[j]; }
        }
    }
}

}  // namespace

int launch_kv_store(const __half* k, const __half* v, int64_t ld, const fg_kv* kv, int32_t seq0,
                    int32_t nseq, int32_t t0, int32_t nt, const fg_dims* d, hipStream_t st) {
    if (nseq == 0 || nt == 0) return FG_OK;
    const int64_t units = (int64_t)nseq * d->n_heads;
    const unsigned grid = (unsigned)cdiv(units, 4);
    const bool q4 = kv->fmt == FG_FMT_Q4G64;
    const double ne = (double)nseq * nt * d->h1 * 2;       // K and V elements
    TraceScope ts(TK_KV_STORE, st, 0.0, ne * 2 + (q4 ? ne / 2 + ne / 64 * 4 : ne * 2));
#define FG_KV_STORE(HD_, Q_)                                                                 \
    kv_store_kernel<HD_, Q_><<<grid, 256, 0, st>>>(k, v, ld, kv->k, (__half*)kv->k_meta, kv->v, \
                                                   (__half*)kv->v_meta, kv->max_len, d->n_heads, \
                                                   seq0, nseq, t0, nt)
    if (d->head_dim == 128) {
        if (q4) FG_KV_STORE(128, true); else FG_KV_STORE(128, false);
    } else {
        if (q4) FG_KV_STORE(64, true); else FG_KV_STORE(64, false);
    }
#undef FG_KV_STORE
    FG_LAUNCHED("kv_store_kernel");
    return FG_OK;
}

int launch_attn_decode(const __half* q, const __half* k_new, const __half* v_new, int64_t ld,
                       const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos, int fuse,
                       __half* out, hipStream_t st) {
    if (bls == 0) return FG_OK;
    const int64_t units = (int64_t)bls * d->n_heads;
    const unsigned grid = (unsigned)cdiv(units, 4);
    const bool q4 = kv->fmt == FG_FMT_Q4G64;
    // algorithmic HBM bytes: K and V history (4-bit: codes + meta = 9/16 B per
    // element), the q / k_new / v_new rows, the output, the appended position
    const double hist = 2.0 * bls * pos * d->h1;
    const double per_elem = q4 ? 9.0 / 16.0 : 2.0;
    const double bytes = hist * per_elem + (double)bls * d->h1 * 2 * 4 +
                         (fuse ? 2.0 * bls * d->h1 * per_elem : 0.0);
    TraceScope ts(q4 ? TK_ATTN_DECODE_Q4 : TK_ATTN_DECODE_F16, st,
                  4.0 * bls * (pos + 1) * (double)d->h1, bytes);
#define FG_ATTN(HD_, Q_, U_)                                                                  \
    attn_decode_kernel<HD_, Q_, U_><<<grid, 256, 0, st>>>(                                    \
        q, k_new, v_new, ld, kv->k, (__half*)kv->k_meta, kv->v, (__half*)kv->v_meta,          \
        kv->max_len, d->n_heads, bls, pos, fuse, out)
    if (d->head_dim == 128) {
        if (q4) FG_ATTN(128, true, 4); else FG_ATTN(128, false, 2);
    } else {
        if (q4) FG_ATTN(64, true, 4); else FG_ATTN(64, false, 2);
    }
#undef FG_ATTN
    FG_LAUNCHED("attn_decode_kernel");
    return FG_OK;
}

}  // namespace fg

// -------------------------------------------------------------------- C ABI
namespace {
int check_kv_call(const void* a, const void* b, const void* c, int64_t ld, const fg_kv* kv,
                  int32_t bls, const fg_dims* d, int32_t pos, int32_t fmt) {
    FG_TRY(fg::check_dims(d));
    FG_CHECK_ARG(a && b && c && kv, "null pointer argument");
    FG_CHECK_ARG(kv->fmt == fmt, "cache format %d does not match this entry point (%d)", kv->fmt,
                 fmt);
    FG_CHECK_ARG(kv->k && kv->v, "null cache tensors");
    FG_CHECK_ARG(fmt != FG_FMT_Q4G64 || (kv->k_meta && kv->v_meta), "null cache metadata");
    FG_CHECK_ARG(bls >= 1 && bls <= kv->n_seq, "bls %d outside [1, n_seq %d]", bls, kv->n_seq);
    FG_CHECK_ARG(pos >= 0 && pos < kv->max_len, "pos %d outside [0, max_len %d)", pos,
                 kv->max_len);
    FG_CHECK_ARG(ld >= d->h1 && ld % 8 == 0, "row stride %lld must be >= h1 and a multiple of 8",
                 (long long)ld);
    FG_CHECK_ARG(((uintptr_t)a | (uintptr_t)b | (uintptr_t)c | (uintptr_t)kv->k |
                  (uintptr_t)kv->v) % 16 == 0,
                 "rows and cache must be 16-byte aligned");
    FG_CHECK_ARG(((uintptr_t)kv->k_meta | (uintptr_t)kv->v_meta) % 4 == 0,
                 "cache metadata must be 4-byte aligned");
    return FG_OK;
}
}  // namespace

extern "C" int fg_kv_append_q4(const void* k_new, const void* v_new, int64_t ld, const fg_kv* kv,
                               int32_t bls, const fg_dims* d, int32_t pos, void* stream) {
    fg::clear_error();
    FG_TRY(check_kv_call(k_new, v_new, k_new, ld, kv, bls, d, pos, FG_FMT_Q4G64));
    return fg::launch_kv_store((const __half*)k_new, (const __half*)v_new, ld, kv, 0, bls, pos,
                               1, d, fg::as_stream(stream));
}

extern "C" int fg_kv_append_f16(const void* k_new, const void* v_new, int64_t ld, const fg_kv* kv,
                                int32_t bls, const fg_dims* d, int32_t pos, void* stream) {
    fg::clear_error();
    FG_TRY(check_kv_call(k_new, v_new, k_new, ld, kv, bls, d, pos, FG_FMT_F16));
    return fg::launch_kv_store((const __half*)k_new, (const __half*)v_new, ld, kv, 0, bls, pos,
                               1, d, fg::as_stream(stream));
}

extern "C" int fg_attn_decode_q4(const void* q, const void* k_new, const void* v_new, int64_t ld,
                                 const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos,
                                 int32_t fuse_append, void* out, void* stream) {
    fg::clear_error();
    FG_TRY(check_kv_call(q, k_new, v_new, ld, kv, bls, d, pos, FG_FMT_Q4G64));
    FG_CHECK_ARG(out && (uintptr_t)out % 16 == 0, "out must be non-null and 16-byte aligned");
    return fg::launch_attn_decode((const __half*)q, (const __half*)k_new, (const __half*)v_new, ld,
                                  kv, bls, d, pos, fuse_append != 0, (__half*)out,
                                  fg::as_stream(stream));
}

extern "C" int fg_attn_decode_f16(const void* q, const void* k_new, const void* v_new, int64_t ld,
                                  const fg_kv* kv, int32_t bls, const fg_dims* d, int32_t pos,
                                  int32_t fuse_append, void* out, void* stream) {
    fg::clear_error();
    FG_TRY(check_kv_call(q, k_new, v_new, ld, kv, bls, d, pos, FG_FMT_F16));
    FG_CHECK_ARG(out && (uintptr_t)out % 16 == 0, "out must be non-null and 16-byte aligned");
    return fg::launch_attn_decode((const __half*)q, (const __half*)k_new, (const __half*)v_new, ld,
                                  kv, bls, d, pos, fuse_append != 0, (__half*)out,
                                  fg::as_stream(stream));
}
