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
// Mapping (MI355X, wave64): one workgroup of NW wavefronts per (sequence,
// head).  A lane owns 32 consecutive dims of the head (16 B of 4-bit codes,
// inside one 64-group, or 64 B of fp16) and one position per step: hd=128 ->
// 4 lanes per position, 16 positions per wavefront step.  The history is
// processed in two passes per chunk of positions:
//   1. scores of all positions into LDS (K stream), chunk maximum;
//   2. softmax weights from LDS, weighted V sum (V stream).
// so the running maximum changes once per chunk, not once per position.  The
// per-lane partial sums are merged at the end with DPP row reductions and LDS.
// 4-bit rows are streamed with non-temporal loads (each byte is read once per
// step; one load instruction covers whole consecutive rows); fp16 rows use
// cached loads, since a lane's 64 B take 4 instructions that share lines.
// Every load is unconditional (positions past the end are clamped to the last
// valid row and masked afterwards) so the compiler keeps several loads in
// flight per lane.
//
// Arithmetic of the 4-bit path.  A nibble c becomes the fp16 value 1024 + c
// with one byte permute (0x64 as the high byte), and v_dot2_f32_f16 multiplies
// two fp16 pairs exactly and accumulates in fp32:
//   score:  sum_{d in D} q_d (mn_g + sc_g c_d)
//             = mn_g * S_q + sc_g * (sum_d q_d (1024 + c_d) - 1024 S_q),
//   output: sum_p w_p (mn_p + sc_p c_pd)
//             = sum_p w_p mn_p + sum_p w^_p (1024 + c_pd) - 1024 sum_p w^_p,
// with S_q the sum of the lane's q values and w^_p = fp16(w_p sc_p); the V sum
// pairs two positions per dot2 (the same dim of positions p, p').
//
// Reading of the current token (stated in fg.h): positions < pos come from the
// cache; position pos uses the fresh fp16 k, v.
#include <hip/hip_ext.h>

#include <algorithm>

#include "codec_dev.h"
#include "fg_internal.h"
#include "fg_trace.h"

namespace fg {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
// positions per chunk of scores in LDS (32 KB); longer histories take several
// chunks with a running maximum
constexpr int kAttnChunk = 8192;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo_half(uint32_t w) {
    return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu)));
}
__device__ __forceinline__ float hi_half(uint32_t w) {
    return __half2float(__ushort_as_half((unsigned short)(w >> 16)));
}
__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ __forceinline__ float dot2(uint32_t a, h2 b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), b, c, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
// sum over the LPP lanes of one position (lane ^ 1, lane ^ 2 inside a quad)
template <int LPP>
__device__ __forceinline__ float pos_sum(float v) {
    v += dpp<0xB1>(v);
    if constexpr (LPP == 4) v += dpp<0x4E>(v);
    return v;
}
// sum over the lanes of one row of 16 that own the same dims (lane % LPP)
template <int LPP>
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<0x128>(v);   // row_ror:8
    v += dpp<0x124>(v);   // row_ror:4
    if constexpr (LPP == 2) v += dpp<0x122>(v);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ int wave_isum(int v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ float wave_fsum(float v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
    return v;
}
// order-preserving unsigned key of a float (larger score, larger key)
__device__ __forceinline__ uint32_t score_key(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint4 ld_stream(const uint8_t* p) {
    const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

constexpr uint32_t MAGIC = 0x64646464u;   // fp16 0x64XX = 1024 + XX for XX < 16
constexpr uint32_t SEL_B01 = 0x04010400u; // (1024 + byte 0, 1024 + byte 1)
constexpr uint32_t SEL_B23 = 0x04030402u; // (1024 + byte 2, 1024 + byte 3)
constexpr uint32_t SEL_LO = 0x05040100u;  // (low half of a, low half of b)
constexpr uint32_t SEL_HI = 0x07060302u;  // (high half of a, high half of b)

// One lane's share of a cache row: 32 dims.
template <bool Q4> struct Row;
template <> struct Row<true> { uint4 c; };                      // 16 B of nibbles
template <> struct Row<false> { uint4 c[4]; };                  // 64 B of fp16

template <bool Q4>
__device__ __forceinline__ Row<Q4> load_row(const uint8_t* p) {
    Row<Q4> r;
    if constexpr (Q4) {
        r.c = ld_stream(p);
    } else {
#pragma unroll
        // cached loads: the 4 loads of a lane's 64 B each touch every line of
        // the step's rows (other lanes take the rest of each line), so the
        // lines must stay in L1 between them (non-temporal: 3740 -> cached
        // 5940 GB/s for 64-dim heads)
        for (int k = 0; k < 4; ++k) r.c[k] = *reinterpret_cast<const uint4*>(p + 16 * k);
    }
    return r;
}

// q of the lane's 32 dims as fp16 pairs.  4-bit path: in nibble-unpack order
// (q0,q2),(q4,q6),(q1,q3),(q5,q7) per 8 dims; fp16 path: natural pairs.
template <bool Q4>
__device__ __forceinline__ void load_q(const __half* src, h2 qp[16]) {
    const uint4* q4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint4 r = q4[k];
        if constexpr (Q4) {
            qp[4 * k + 0] = as_h2(__builtin_amdgcn_perm(r.y, r.x, SEL_LO));
            qp[4 * k + 1] = as_h2(__builtin_amdgcn_perm(r.w, r.z, SEL_LO));
            qp[4 * k + 2] = as_h2(__builtin_amdgcn_perm(r.y, r.x, SEL_HI));
            qp[4 * k + 3] = as_h2(__builtin_amdgcn_perm(r.w, r.z, SEL_HI));
        } else {
            qp[4 * k + 0] = as_h2(r.x);
            qp[4 * k + 1] = as_h2(r.y);
            qp[4 * k + 2] = as_h2(r.z);
            qp[4 * k + 3] = as_h2(r.w);
        }
    }
}

// 4-bit: sum_d q_d (1024 + c_d) over the lane's 32 dims, starting from acc.
__device__ __forceinline__ float kdot_q4(const uint4& c, const h2 qp[16], float acc) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x0f0f0f0fu, hi = (w[k] >> 4) & 0x0f0f0f0fu;
        acc = dot2(__builtin_amdgcn_perm(MAGIC, lo, SEL_B01), qp[4 * k + 0], acc);
        acc = dot2(__builtin_amdgcn_perm(MAGIC, lo, SEL_B23), qp[4 * k + 1], acc);
        acc = dot2(__builtin_amdgcn_perm(MAGIC, hi, SEL_B01), qp[4 * k + 2], acc);
        acc = dot2(__builtin_amdgcn_perm(MAGIC, hi, SEL_B23), qp[4 * k + 3], acc);
    }
    return acc;
}

// 4-bit: acc_d += wA (1024 + cA_d) + wB (1024 + cB_d) over 32 dims of two
// positions A, B (bytes of A and B interleaved first, so one permute builds
// the fp16 pair of one dim).
__device__ __forceinline__ void vacc_q4(const uint4& a, const uint4& b, h2 w, float acc[32]) {
    const uint32_t A[4] = {a.x, a.y, a.z, a.w}, B[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t X = __builtin_amdgcn_perm(B[k], A[k], 0x05010400u);   // A0 B0 A1 B1
        const uint32_t Y = __builtin_amdgcn_perm(B[k], A[k], 0x07030602u);   // A2 B2 A3 B3
        const uint32_t xl = X & 0x0f0f0f0fu, xh = (X >> 4) & 0x0f0f0f0fu;
        const uint32_t yl = Y & 0x0f0f0f0fu, yh = (Y >> 4) & 0x0f0f0f0fu;
        acc[8 * k + 0] = dot2(__builtin_amdgcn_perm(MAGIC, xl, SEL_B01), w, acc[8 * k + 0]);
        acc[8 * k + 2] = dot2(__builtin_amdgcn_perm(MAGIC, xl, SEL_B23), w, acc[8 * k + 2]);
        acc[8 * k + 1] = dot2(__builtin_amdgcn_perm(MAGIC, xh, SEL_B01), w, acc[8 * k + 1]);
        acc[8 * k + 3] = dot2(__builtin_amdgcn_perm(MAGIC, xh, SEL_B23), w, acc[8 * k + 3]);
        acc[8 * k + 4] = dot2(__builtin_amdgcn_perm(MAGIC, yl, SEL_B01), w, acc[8 * k + 4]);
        acc[8 * k + 6] = dot2(__builtin_amdgcn_perm(MAGIC, yl, SEL_B23), w, acc[8 * k + 6]);
        acc[8 * k + 5] = dot2(__builtin_amdgcn_perm(MAGIC, yh, SEL_B01), w, acc[8 * k + 5]);
        acc[8 * k + 7] = dot2(__builtin_amdgcn_perm(MAGIC, yh, SEL_B23), w, acc[8 * k + 7]);
    }
}

// fp16: acc_d += wA vA_d + wB vB_d over 32 dims of two positions.
__device__ __forceinline__ void vacc_f16(const Row<false>& a, const Row<false>& b, h2 w,
                                         float acc[32]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t A[4] = {a.c[k].x, a.c[k].y, a.c[k].z, a.c[k].w};
        const uint32_t B[4] = {b.c[k].x, b.c[k].y, b.c[k].z, b.c[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[8 * k + 2 * i] = dot2(__builtin_amdgcn_perm(B[i], A[i], SEL_LO), w, acc[8 * k + 2 * i]);
            acc[8 * k + 2 * i + 1] =
                dot2(__builtin_amdgcn_perm(B[i], A[i], SEL_HI), w, acc[8 * k + 2 * i + 1]);
        }
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
__device__ __forceinline__ uint4 quant_half_group(const uint4 r[4], uint32_t& meta_bits) {
    // 32 fp16 values kept packed (16 registers); each is widened where used
    const uint32_t w[16] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w,
                            r[2].x, r[2].y, r[2].z, r[2].w, r[3].x, r[3].y, r[3].z, r[3].w};
    float mn = lo_half(w[0]), mx = mn;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a = lo_half(w[i]), c = hi_half(w[i]);
        mn = fminf(mn, fminf(a, c));
        mx = fmaxf(mx, fmaxf(a, c));
    }
    mn = fminf(mn, __shfl_xor(mn, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    const QParams p = qparams(mn, mx);
    meta_bits = qmeta_bits(p);
    uint32_t out[4];
#pragma unroll 1
    for (int k = 0; k < 4; ++k) {
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x |= qcode(lo_half(w[4 * k + j]), p) << (8 * j);
            x |= qcode(hi_half(w[4 * k + j]), p) << (8 * j + 4);
        }
        out[k] = x;
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// the lane's 32 fp16 values of a row (16 B aligned)
__device__ __forceinline__ void load32p(const __half* p, uint4 r[4]) {
    const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = p4[k];
}

// NW wavefronts per (sequence, head); MULTI: the history may exceed one chunk
// of `chunk` positions (scores in dynamic LDS), merged with a running maximum.
template <int HD, bool Q4, int NW, bool MULTI, bool SPARSE = false>
__device__ __forceinline__ void attn_decode_body(
    const __half* __restrict__ q, const __half* __restrict__ k_new,
    const __half* __restrict__ v_new, int64_t ld, void* __restrict__ kc,
    __half* __restrict__ km, void* __restrict__ vc, __half* __restrict__ vm, int32_t lmax,
    int32_t nh, int32_t pos, int32_t chunk, int fuse, int32_t topk, __half* __restrict__ out) {
    static_assert(!(MULTI && SPARSE), "Top-K selection needs every score of the history in LDS");
    constexpr int LPP = HD / 32;           // lanes per position
    constexpr int SLOTS = 64 / LPP;        // positions per wavefront step
    constexpr int GPH = HD / 64;           // 64-groups per head
    constexpr int WGP = NW * SLOTS;        // positions per workgroup step
    constexpr int ROWS = 4;                // rows of 16 lanes
    constexpr int RB = Q4 ? HD / 2 : HD * 2;   // bytes of one cache row
    constexpr int U1 = Q4 ? 4 : 2;         // steps per batch of loads, pass 1
    constexpr int U2 = Q4 ? 2 : 1;         // pairs of steps per batch, pass 2
    extern __shared__ float smem[];
    float* sVn = smem;                                  // Top-K: [HD] the current token's v (fp32)
    float* sS = smem + (SPARSE ? HD : 0);               // [chunk] scores (log2 units)
    float* sRed = sS + chunk;                           // [NW*ROWS*LPP][32]
    float* sFix = sRed + NW * ROWS * LPP * 32;          // [NW*ROWS*LPP]
    float* sL = sFix + NW * ROWS * LPP;                 // [NW*ROWS]
    float* sMax = sL + NW * ROWS;                       // [NW]
    // Top-K: per-wave counts (two alternating sets), the selected count, the
    // per-wave parts of the normalizer over all scores, the selected
    // positions in index order (16 bits each: a Top-K history is one chunk of
    // at most 8192 positions, which keeps the launch under 64 KB of LDS with
    // four wavefronts)
    int* sCnt = reinterpret_cast<int*>(sMax + NW);      // [2][NW]
    int* sSel = sCnt + 2 * NW;                          // [1]
    float* sLw = reinterpret_cast<float*>(sSel + 1);    // [NW] per-wave normalizer parts
    unsigned short* sIdx = reinterpret_cast<unsigned short*>(sSel + 1 + NW);   // [chunk]

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t unit = blockIdx.x;                    // (b, h)
    const int64_t b = unit / nh;
    const int h = (int)(unit - b * nh);
    const int qi = lane % LPP;                          // which 32 dims
    const int slot = lane / LPP;
    const int g = qi >> 1;                              // 64-group of those dims
    const int lp = wv * SLOTS + slot;                   // position offset in a step
    const int64_t row0 = unit * (int64_t)lmax;          // cache row of (b, h, 0)
    const uint8_t* kcp = (const uint8_t*)kc + row0 * RB + qi * (RB / LPP);
    const uint8_t* vcp = (const uint8_t*)vc + row0 * RB + qi * (RB / LPP);
    const uint32_t* kmp = reinterpret_cast<const uint32_t*>(km) + row0 * GPH + g;
    const uint32_t* vmp = reinterpret_cast<const uint32_t*>(vm) + row0 * GPH + g;
    const float qscale = LOG2E / sqrtf((float)HD);      // scores in log2 units
    const h2 one2 = {(_Float16)1.0f, (_Float16)1.0f};

    // Top-K: the current token's v for the output, requested first and
    // parked in LDS once q has arrived, so that its load latency is not
    // exposed after the selection and the gathered pass (measured: the
    // output phase of a workgroup 2.1 -> 1.0 us at the OPT-175B shape; the
    // dense kernel gains nothing from it)
    constexpr int OD = (HD + NW * 64 - 1) / (NW * 64);
    float vnd[OD];
    if constexpr (SPARSE) {
#pragma unroll
        for (int i = 0; i < OD; ++i) {
            const int d = threadIdx.x + i * NW * 64;
            vnd[i] = d < HD ? __half2float(v_new[b * ld + h * HD + d]) : 0.f;
        }
    }

    h2 qp[16];
    load_q<Q4>(q + b * ld + h * HD + qi * 32, qp);
    float qsum = 0.f;
    if constexpr (Q4) {
#pragma unroll
        for (int i = 0; i < 16; ++i) qsum = __builtin_amdgcn_fdot2(qp[i], one2, qsum, false);
    }
    const float qoff = -1024.0f * qsum;
    if constexpr (SPARSE) {
#pragma unroll
        for (int i = 0; i < OD; ++i) {
            const int d = threadIdx.x + i * NW * 64;
            if (d < HD) sVn[d] = vnd[i];
        }
    }

    // score of the current token (fresh fp16 k, same pair order as qp)
    float snew;
    {
        h2 kp[16];
        load_q<Q4>(k_new + b * ld + h * HD + qi * 32, kp);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s = __builtin_amdgcn_fdot2(kp[i], qp[i], s, false);
        snew = pos_sum<LPP>(s) * qscale;
    }

    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    float l = 0.f, fix = 0.f;      // fix: sum w mn - 1024 sum w^ (4-bit only)
    float M = snew;                // running maximum (log2 units)

    auto run_chunk = [&](int c0, int n) {
        const int last = c0 + n - 1;                    // last valid position
        const int nst = (n + WGP - 1) / WGP;
        // pass 1: scores
        float mloc = -INFINITY;
        auto kscore = [&](int j, const Row<Q4>& r, uint32_t meta) {
            float s;
            if constexpr (Q4) {
                s = lo_half(meta) * qsum + hi_half(meta) * kdot_q4(r.c, qp, qoff);
            } else {
                s = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    s = dot2(r.c[k].x, qp[4 * k + 0], s);
                    s = dot2(r.c[k].y, qp[4 * k + 1], s);
                    s = dot2(r.c[k].z, qp[4 * k + 2], s);
                    s = dot2(r.c[k].w, qp[4 * k + 3], s);
                }
            }
            s = pos_sum<LPP>(s) * qscale;
            const int pl = j * WGP + lp;
            if (pl < n) {
                mloc = fmaxf(mloc, s);
                if (qi == 0) sS[pl] = s;
            }
        };
        int j = 0;
        for (; j + U1 <= nst; j += U1) {
            Row<Q4> r[U1];
            uint32_t meta[U1];
#pragma unroll
            for (int u = 0; u < U1; ++u) {
                const int64_t p = min(c0 + (j + u) * WGP + lp, last);
                r[u] = load_row<Q4>(kcp + p * RB);
                if constexpr (Q4) meta[u] = kmp[p * GPH];
            }
#pragma unroll
            for (int u = 0; u < U1; ++u) kscore(j + u, r[u], Q4 ? meta[u] : 0u);
        }
        for (; j < nst; ++j) {
            const int64_t p = min(c0 + j * WGP + lp, last);
            const Row<Q4> r = load_row<Q4>(kcp + p * RB);
            const uint32_t meta = Q4 ? kmp[p * GPH] : 0u;
            kscore(j, r, meta);
        }
        mloc = wave_max(mloc);
        if (lane == 0) sMax[wv] = mloc;
        __syncthreads();
        float mc = sMax[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) mc = fmaxf(mc, sMax[w]);
        if constexpr (MULTI) {
            if (mc > M) {               // uniform over the workgroup
                const float alpha = exp2f(M - mc);
                l *= alpha;
                fix *= alpha;
#pragma unroll
                for (int i = 0; i < 32; ++i) acc[i] *= alpha;
                M = mc;
            }
        } else {
            M = fmaxf(M, mc);
        }
        // pass 2: weighted V of positions pa, pb (dense: pairs of steps j, j+1;
        // Top-K: pairs of entries of the selected list, the normalizer having
        // been taken over every score)
        auto vacc2 = [&](int pa, int pb, bool oka, bool okb, const Row<Q4>& ra, const Row<Q4>& rb,
                         uint32_t ma, uint32_t mb) {
            const float wa = oka ? exp2f(sS[oka ? pa : 0] - M) : 0.f;
            const float wb = okb ? exp2f(sS[okb ? pb : 0] - M) : 0.f;
            if constexpr (Q4) {
                const uint32_t mA = oka ? ma : 0u, mB = okb ? mb : 0u;
                if constexpr (!SPARSE) l += wa + wb;
                h2 wh;
                wh[0] = (_Float16)(wa * hi_half(mA));
                wh[1] = (_Float16)(wb * hi_half(mB));
                fix = fmaf(wa, lo_half(mA), fmaf(wb, lo_half(mB), fix));
                fix = __builtin_amdgcn_fdot2(wh, -1024.0f * one2, fix, false);
                vacc_q4(ra.c, rb.c, wh, acc);
            } else {
                h2 wh;
                wh[0] = (_Float16)wa;
                wh[1] = (_Float16)wb;
                if constexpr (!SPARSE) l = __builtin_amdgcn_fdot2(wh, one2, l, false);
                vacc_f16(ra, rb, wh, acc);
            }
        };
        auto vpair = [&](int ja, const Row<Q4>& ra, const Row<Q4>& rb, uint32_t ma, uint32_t mb) {
            const int pa = ja * WGP + lp, pb = pa + WGP;
            vacc2(pa, pb, pa < n, pb < n, ra, rb, ma, mb);
        };
        if constexpr (SPARSE) {
            // the topk positions of highest score, ties to the lower position:
            // tau = the topk-th largest key (bitwise search: count(key >= tau)
            // >= topk), then wave 0 lists the positions in index order with
            // key > tau, and the first topk - count(key > tau) with key == tau.
            // Counts are wave ballots (a scalar popcount per key slot), summed
            // over the wavefronts through LDS.  The search stops as soon as
            // exactly topk keys are >= the candidate: those are then the topk
            // highest, with no tie at the threshold (the next key is lower).
            //
            // One barrier per count: the two sets of sCnt alternate, so a wave
            // that runs ahead writes the set that every wave had finished
            // reading before the barrier it has just passed.
            int cset = 0;
            auto block_count = [&](int c) -> int {
                if constexpr (NW == 1) {
                    return c;
                } else {
                    int* cnt = sCnt + cset * NW;
                    cset ^= 1;
                    if (lane == 0) cnt[wv] = c;
                    __syncthreads();
                    int t = 0;
#pragma unroll
                    for (int w = 0; w < NW; ++w) t += cnt[w];
                    return t;
                }
            };
            constexpr int KR = 10;                      // keys held per lane
            const int kk = topk < n ? topk : n;
            const bool search_needed = kk > 0 && kk < n;
            // a history of up to KR * NW * 64 positions is held as keys in
            // registers (0: below every real key) while every thread adds up
            // its positions' softmax weights; a longer one is read from LDS
            const bool in_regs = n <= KR * NW * 64;
            uint32_t kr[KR];
            float lpart = 0.f;
            if (in_regs) {
#pragma unroll
                for (int i = 0; i < KR; ++i) {
                    const int p = threadIdx.x + i * NW * 64;
                    const float sp = p < n ? sS[p] : 0.f;
                    kr[i] = p < n ? score_key(sp) : 0u;
                    if (p < n) lpart += exp2f(sp - M);
                }
            } else {
                for (int p = threadIdx.x; p < n; p += NW * 64) lpart += exp2f(sS[p] - M);
            }
            lpart = wave_fsum(lpart);
            if (lane == 0) sLw[wv] = lpart;            // summed after the barrier below
            uint32_t tau = 0;
            int n_gt = 0;
            auto search = [&](auto count_ge) {
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t cand = tau | (1u << bit);
                    const int c = block_count(count_ge(cand));
                    if (c >= kk) {
                        tau = cand;
                        if (c == kk) {          // key > cand - 1 selects exactly kk
                            tau = cand - 1u;
                            n_gt = kk;
                            return;
                        }
                    }
                }
                n_gt = block_count(count_ge(tau + 1u));
            };
            if (search_needed) {
                if (in_regs) {
                    search([&](uint32_t c) -> int {
                        int t = 0;
#pragma unroll
                        for (int i = 0; i < KR; ++i) t += (int)__builtin_popcountll(__ballot(kr[i] >= c));
                        return t;
                    });
                } else {
                    search([&](uint32_t c) -> int {
                        int t = 0;
                        for (int p0 = 0; p0 < n; p0 += NW * 64) {
                            const int p = p0 + threadIdx.x;
                            t += (int)__builtin_popcountll(__ballot(p < n && score_key(sS[p < n ? p : 0]) >= c));
                        }
                        return t;
                    });
                }
            }
            if (wv == 0) {
                const int need_eq = kk - n_gt;
                int cnt = 0, eq_seen = 0;
                // one 64-position block of the listing; key: the score key of
                // position p (only read when a search ran)
                auto list64 = [&](int p, uint32_t key) {
                    const bool valid = p < n;
                    bool sel;
                    if (kk >= n) {
                        sel = valid;
                    } else if (kk == 0) {
                        sel = false;
                    } else if (need_eq > 0) {
                        const bool eq = valid && key == tau;
                        const uint64_t eqm = __ballot(eq);
                        const int rank = eq_seen + (int)__builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(eqm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
                        eq_seen += (int)__builtin_popcountll(eqm);
                        sel = (valid && key > tau) || (eq && rank < need_eq);
                    } else {
                        sel = valid && key > tau;
                    }
                    const uint64_t sm = __ballot(sel);
                    const int off = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
                    if (sel) sIdx[cnt + off] = (unsigned short)p;
                    cnt += (int)__builtin_popcountll(sm);
                };
                if (NW == 1 && in_regs && search_needed) {
                    // one wavefront: key slot i of lane l is position 64 i + l
#pragma unroll
                    for (int i = 0; i < KR; ++i) {
                        if (i * 64 >= n) break;
                        list64(i * 64 + lane, kr[i]);
                    }
                } else {
                    for (int base = 0; base < n; base += 64) {
                        const int p = base + lane;
                        list64(p, search_needed && p < n ? score_key(sS[p]) : 0u);
                    }
                }
                if (lane == 0) sSel[0] = cnt;
            }
            __syncthreads();
            const int nsel = sSel[0];
            const int npr = (nsel + 2 * WGP - 1) / (2 * WGP);
            auto epos = [&](int e) -> int { return sIdx[e < nsel ? e : nsel - 1]; };
            int pr = 0;
            for (; pr + U2 <= npr; pr += U2) {
                Row<Q4> ra[U2], rb[U2];
                uint32_t ma[U2], mb[U2];
                int pa[U2], pb[U2];
#pragma unroll
                for (int u = 0; u < U2; ++u) {
                    const int ea = 2 * (pr + u) * WGP + lp;
                    pa[u] = epos(ea);
                    pb[u] = epos(ea + WGP);
                    ra[u] = load_row<Q4>(vcp + (int64_t)pa[u] * RB);
                    rb[u] = load_row<Q4>(vcp + (int64_t)pb[u] * RB);
                    if constexpr (Q4) {
                        ma[u] = vmp[(int64_t)pa[u] * GPH];
                        mb[u] = vmp[(int64_t)pb[u] * GPH];
                    }
                }
#pragma unroll
                for (int u = 0; u < U2; ++u) {
                    const int ea = 2 * (pr + u) * WGP + lp;
                    vacc2(pa[u], pb[u], ea < nsel, ea + WGP < nsel, ra[u], rb[u],
                          Q4 ? ma[u] : 0u, Q4 ? mb[u] : 0u);
                }
            }
            for (; pr < npr; ++pr) {
                const int ea = 2 * pr * WGP + lp;
                const int pa = epos(ea), pb = epos(ea + WGP);
                const Row<Q4> ra = load_row<Q4>(vcp + (int64_t)pa * RB);
                const Row<Q4> rb = load_row<Q4>(vcp + (int64_t)pb * RB);
                const uint32_t ma = Q4 ? vmp[(int64_t)pa * GPH] : 0u, mb = Q4 ? vmp[(int64_t)pb * GPH] : 0u;
                vacc2(pa, pb, ea < nsel, ea + WGP < nsel, ra, rb, ma, mb);
            }
            return;
        }
        const int npr = (nst + 1) / 2;
        int pr = 0;
        for (; pr + U2 <= npr; pr += U2) {
            Row<Q4> ra[U2], rb[U2];
            uint32_t ma[U2], mb[U2];
#pragma unroll
            for (int u = 0; u < U2; ++u) {
                const int pa = c0 + 2 * (pr + u) * WGP + lp;
                const int64_t qa = min(pa, last), qb = min(pa + WGP, last);
                ra[u] = load_row<Q4>(vcp + qa * RB);
                rb[u] = load_row<Q4>(vcp + qb * RB);
                if constexpr (Q4) {
                    ma[u] = vmp[qa * GPH];
                    mb[u] = vmp[qb * GPH];
                }
            }
#pragma unroll
            for (int u = 0; u < U2; ++u)
                vpair(2 * (pr + u), ra[u], rb[u], Q4 ? ma[u] : 0u, Q4 ? mb[u] : 0u);
        }
        for (; pr < npr; ++pr) {
            const int pa = c0 + 2 * pr * WGP + lp;
            const int64_t qa = min(pa, last), qb = min(pa + WGP, last);
            const Row<Q4> ra = load_row<Q4>(vcp + qa * RB);
            const Row<Q4> rb = load_row<Q4>(vcp + qb * RB);
            const uint32_t ma = Q4 ? vmp[qa * GPH] : 0u, mb = Q4 ? vmp[qb * GPH] : 0u;
            vpair(2 * pr, ra, rb, ma, mb);
        }
    };
    if constexpr (MULTI) {
        for (int c0 = 0; c0 < pos; c0 += chunk) {
            run_chunk(c0, min(chunk, pos - c0));
            __syncthreads();            // sS and sMax are rewritten by the next chunk
        }
    } else if (pos > 0) {
        run_chunk(0, pos);
    }

    // merge the lanes: row sums (DPP) -> LDS -> one thread per output dim
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = row_sum<LPP>(acc[i]);
    fix = row_sum<LPP>(fix);
    l = row_sum<LPP>(l);
    if ((lane & 15) < LPP) {
        const int r = (wv * ROWS + (lane >> 4)) * LPP + qi;
        float4* dst = reinterpret_cast<float4*>(sRed + r * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dst[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
        sFix[r] = fix;
        if (qi == 0) sL[wv * ROWS + (lane >> 4)] = l;
    }
    __syncthreads();
    const float wn = exp2f(snew - M);
    // Top-K: the thread index afresh (an opaque copy); otherwise the compiler
    // keeps the prologue's LDS address of sVn alive through the passes, and
    // may spill it
    int tx = (int)threadIdx.x;
    if constexpr (SPARSE) asm("" : "+v"(tx));
#pragma unroll
    for (int i = 0; i < OD; ++i) {
        const int d = tx + i * NW * 64;
        if (d >= HD) break;
        const int dq = d >> 5, e = d & 31;
        float s = 0.f, L = 0.f;
#pragma unroll
        for (int r = 0; r < NW * ROWS; ++r) {
            s += sRed[(r * LPP + dq) * 32 + e] + sFix[r * LPP + dq];
            L += sL[r];
        }
        if constexpr (SPARSE) {                         // every score's weight
            L = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) L += sLw[w];
            if (pos == 0) L = 0.f;
        }
        const float vnd_d = SPARSE ? sVn[d] : __half2float(v_new[b * ld + h * HD + d]);
        out[b * (int64_t)nh * HD + h * HD + d] = __float2half_rn((s + wn * vnd_d) / (L + wn));
    }

    // append the current token at row pos (the passes above read rows < pos
    // only), K then V
    if (fuse && wv == 0) {
        const int64_t row = row0 + pos;
        if constexpr (Q4) {
#pragma unroll 1
            for (int t = 0; t < 2; ++t) {
                const __half* src = (t == 0 ? k_new : v_new) + b * ld + h * HD + qi * 32;
                uint4 x[4];
                load32p(src, x);
                uint32_t mbits;
                const uint4 code = quant_half_group(x, mbits);   // all lanes: shuffles need the full wave
                if (slot == 0) {
                    *reinterpret_cast<uint4*>((uint8_t*)(t == 0 ? kc : vc) + row * (HD / 2) + qi * 16) = code;
                    if ((qi & 1) == 0)
                        *reinterpret_cast<uint32_t*>((t == 0 ? km : vm) + (row * GPH + g) * 2) = mbits;
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

#define FG_ATTN_PARAMS                                                                      \
    const __half *__restrict__ q, const __half *__restrict__ k_new,                          \
        const __half *__restrict__ v_new, int64_t ld, void *__restrict__ kc,                 \
        __half *__restrict__ km, void *__restrict__ vc, __half *__restrict__ vm,             \
        int32_t lmax, int32_t nh, int32_t pos, int32_t chunk, int fuse, int32_t topk,              \
        __half *__restrict__ out
#define FG_ATTN_ARGS q, k_new, v_new, ld, kc, km, vc, vm, lmax, nh, pos, chunk, fuse, topk, out

// history in one chunk: register budget of 6 (4-bit) or 5 (fp16) wavefronts per SIMD
template <int HD, bool Q4, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(Q4 ? 6 : 5)))
void attn_decode_kernel(FG_ATTN_PARAMS) {
    attn_decode_body<HD, Q4, NW, false>(FG_ATTN_ARGS);
}

// histories longer than one chunk
template <int HD, bool Q4, int NW>
__global__ __launch_bounds__(NW * 64) void attn_decode_multi_kernel(FG_ATTN_PARAMS) {
    attn_decode_body<HD, Q4, NW, true>(FG_ATTN_ARGS);
}

// Top-K sparse V (history in one chunk): register budget of 5 wavefronts per
// SIMD (the selection and the gathered pass need a few more registers)
template <int HD, bool Q4, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(5)))
void attn_decode_topk_kernel(FG_ATTN_PARAMS) {
    attn_decode_body<HD, Q4, NW, false, true>(FG_ATTN_ARGS);
}
#undef FG_ATTN_ARGS
#undef FG_ATTN_PARAMS

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
            uint4 kv[4], vv[4];
            load32p(ks, kv);
            load32p(vs, vv);
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

// One position (the decode step's append): the slots of a wavefront take
// SLOTS different (sequence, head) units, one position each.  With the
// many-position kernel above a wavefront would quantize the same row in
// every slot, and the exact codec's divisions make that kernel VALU-bound
// (24 us for the OPT-175B block against about 3 here).
template <int HD, bool Q4>
__global__ __launch_bounds__(256) void kv_append_kernel(const __half* __restrict__ k,
                                                        const __half* __restrict__ v, int64_t ld,
                                                        void* __restrict__ kc, __half* __restrict__ km,
                                                        void* __restrict__ vc, __half* __restrict__ vm,
                                                        int32_t lmax, int32_t nh, int32_t seq0,
                                                        int32_t nseq, int32_t t0) {
    constexpr int LPP = HD / 32;
    constexpr int SLOTS = 64 / LPP;
    constexpr int GPH = HD / 64;
    const int lane = threadIdx.x & 63;
    const int64_t units = (int64_t)nseq * nh;
    const int64_t u0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * SLOTS;
    if (u0 >= units) return;                     // whole wavefront
    const int qi = lane % LPP, slot = lane / LPP, g = (qi * 32) / 64;
    const int64_t unit = u0 + slot;
    const bool ok = unit < units;                // whole 4- or 2-lane groups agree
    const int64_t uu = ok ? unit : units - 1;
    const int64_t bl = uu / nh;                  // sequence within this call
    const int h = (int)(uu - bl * nh);
    const __half* ks = k + bl * ld + h * HD + qi * 32;
    const __half* vs = v + bl * ld + h * HD + qi * 32;
    const int64_t row = ((seq0 + bl) * (int64_t)nh + h) * lmax + t0;
    if constexpr (Q4) {
        uint4 kv[4], vv[4];
        load32p(ks, kv);
        load32p(vs, vv);
        uint32_t kmb, vmb;
        const uint4 kq = quant_half_group(kv, kmb);   // every lane: the group's halves meet by shuffle
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

int launch_kv_store(const __half* k, const __half* v, int64_t ld, const fg_kv* kv, int32_t seq0,
                    int32_t nseq, int32_t t0, int32_t nt, const fg_dims* d, hipStream_t st) {
    if (nseq == 0 || nt == 0) return FG_OK;
    const int64_t units = (int64_t)nseq * d->n_heads;
    const unsigned grid = (unsigned)cdiv(units, 4);
    const bool q4 = kv->fmt == FG_FMT_Q4G64;
    const double ne = (double)nseq * nt * d->h1 * 2;       // K and V elements
    TraceScope ts(TK_KV_STORE, st, 0.0, ne * 2 + (q4 ? ne / 2 + ne / 64 * 4 : ne * 2));
    if (nt == 1) {
        const int slots = 64 / (d->head_dim / 32);
        const unsigned g1 = (unsigned)cdiv(units, 4 * (int64_t)slots);
#define FG_KV_APPEND(HD_, Q_)                                                                  \
    kv_append_kernel<HD_, Q_><<<g1, 256, 0, st>>>(k, v, ld, kv->k, (__half*)kv->k_meta, kv->v,   \
                                                  (__half*)kv->v_meta, kv->max_len, d->n_heads,  \
                                                  seq0, nseq, t0)
        if (d->head_dim == 128) {
            if (q4) FG_KV_APPEND(128, true); else FG_KV_APPEND(128, false);
        } else {
            if (q4) FG_KV_APPEND(64, true); else FG_KV_APPEND(64, false);
        }
#undef FG_KV_APPEND
        FG_LAUNCHED("kv_append_kernel");
        return FG_OK;
    }
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
                       __half* out, hipStream_t st, int32_t topk) {
    if (bls == 0) return FG_OK;
    const bool sparse = topk >= 0;
    if (sparse && pos > kAttnTopkMaxPos)
        return set_error(FG_ERR_UNSUPPORTED, "Top-K attention: history %d longer than %d", pos,
                         kAttnTopkMaxPos);
    const int64_t units = (int64_t)bls * d->n_heads;
    const bool q4 = kv->fmt == FG_FMT_Q4G64;
    // algorithmic HBM bytes: K history and the V rows read (all, or the topk
    // selected; 4-bit: codes + meta = 9/16 B per element), the q / k_new /
    // v_new rows, the output, the appended position
    const int32_t vrows = sparse ? std::min(topk, pos) : pos;
    const double per_elem = q4 ? 9.0 / 16.0 : 2.0;
    const double bytes = (double)bls * (pos + vrows) * d->h1 * per_elem +
                         (double)bls * d->h1 * 2 * 4 + (fuse ? 2.0 * bls * d->h1 * per_elem : 0.0);
    const double flops = 2.0 * bls * (pos + 1) * (double)d->h1 + 2.0 * bls * (vrows + 1) * (double)d->h1;
    // the launch below records the trace events itself
    TraceScope ts(kExtLaunch, sparse ? (q4 ? TK_ATTN_TOPK_Q4 : TK_ATTN_TOPK_F16)
                                     : (q4 ? TK_ATTN_DECODE_Q4 : TK_ATTN_DECODE_F16),
                  st, flops, bytes);
    // with enough (sequence, head) pairs to fill the chip: two wavefronts per
    // pair for the 4-bit cache (a launch at the OPT-175B block shape, 13824
    // pairs, otherwise runs 2.25 rounds of resident wavefronts; measured
    // 177 -> 165 us with three 1 GB caches rotated), one for fp16 (two measured
    // 2% slower) and for Top-K; otherwise four, splitting the positions
    const int nw = units >= 2048 ? (q4 && !sparse ? 2 : 1) : 4;
    const bool multi = pos > kAttnChunk;
    const int chunk = multi ? kAttnChunk : (int)std::max<int64_t>(cdiv(pos, 64) * 64, 64);
    const int lpp = d->head_dim / 32;
    const size_t lds = sizeof(float) * ((size_t)chunk + nw * 4 * lpp * 33 + nw * 4 + nw) +
                       (sparse ? sizeof(float) * d->head_dim + sizeof(int) * (3 * (size_t)nw + 1) +
                                     sizeof(uint16_t) * chunk
                               : 0);
    static_assert(kAttnTopkMaxPos <= 65536, "Top-K positions are listed in 16 bits");
    // every launch stays within 64 KB of dynamic LDS (the largest: Top-K over
    // 8192 positions with four wavefronts of head_dim 128, 58.2 KB)
    if (lds > 65536)
        return set_error(FG_ERR_UNSUPPORTED, "decode attention needs %zu bytes of LDS", lds);
    hipEvent_t ea, eb;
    trace_take_ext(&ea, &eb);
#define FG_ATTN(HD_, Q_, NW_, MU_)                                                           \
    hipExtLaunchKernelGGL(                                                                   \
        (sparse ? attn_decode_topk_kernel<HD_, Q_, NW_>                                      \
                : (MU_ ? attn_decode_multi_kernel<HD_, Q_, NW_> : attn_decode_kernel<HD_, Q_, NW_>)), \
        dim3((unsigned)units), dim3(NW_ * 64), (uint32_t)lds, st, ea, eb, 0u,                \
        q, k_new, v_new, ld, kv->k, (__half*)kv->k_meta, kv->v, (__half*)kv->v_meta,         \
        kv->max_len, d->n_heads, pos, chunk, fuse, topk, out)
#define FG_ATTN_NW(HD_, Q_, MU_)                        \
    do {                                                \
        if (nw == 1) FG_ATTN(HD_, Q_, 1, MU_);          \
        else if (nw == 2) FG_ATTN(HD_, Q_, 2, MU_);     \
        else FG_ATTN(HD_, Q_, 4, MU_);                  \
    } while (0)
#define FG_ATTN_MU(HD_, Q_)                             \
    do {                                                \
        if (multi) FG_ATTN_NW(HD_, Q_, true);           \
        else FG_ATTN_NW(HD_, Q_, false);                \
    } while (0)
    if (d->head_dim == 128) {
        if (q4) FG_ATTN_MU(128, true); else FG_ATTN_MU(128, false);
    } else {
        if (q4) FG_ATTN_MU(64, true); else FG_ATTN_MU(64, false);
    }
#undef FG_ATTN_MU
#undef FG_ATTN_NW
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

extern "C" int fg_attn_decode_topk_q4(const void* q, const void* k_new, const void* v_new,
                                      int64_t ld, const fg_kv* kv, int32_t bls, const fg_dims* d,
                                      int32_t pos, int32_t topk, int32_t fuse_append, void* out,
                                      void* stream) {
    fg::clear_error();
    FG_TRY(check_kv_call(q, k_new, v_new, ld, kv, bls, d, pos, FG_FMT_Q4G64));
    FG_CHECK_ARG(out && (uintptr_t)out % 16 == 0, "out must be non-null and 16-byte aligned");
    FG_CHECK_ARG(topk >= 0 && topk <= pos, "topk %d outside [0, pos %d]", topk, pos);
    FG_CHECK_SUP(pos <= fg::kAttnTopkMaxPos, "Top-K attention: history %d longer than %d", pos,
                 fg::kAttnTopkMaxPos);
    return fg::launch_attn_decode((const __half*)q, (const __half*)k_new, (const __half*)v_new, ld,
                                  kv, bls, d, pos, fuse_append != 0, (__half*)out,
                                  fg::as_stream(stream), topk);
}

extern "C" int fg_attn_decode_topk_f16(const void* q, const void* k_new, const void* v_new,
                                       int64_t ld, const fg_kv* kv, int32_t bls, const fg_dims* d,
                                       int32_t pos, int32_t topk, int32_t fuse_append, void* out,
                                       void* stream) {
    fg::clear_error();
    FG_TRY(check_kv_call(q, k_new, v_new, ld, kv, bls, d, pos, FG_FMT_F16));
    FG_CHECK_ARG(out && (uintptr_t)out % 16 == 0, "out must be non-null and 16-byte aligned");
    FG_CHECK_ARG(topk >= 0 && topk <= pos, "topk %d outside [0, pos %d]", topk, pos);
    FG_CHECK_SUP(pos <= fg::kAttnTopkMaxPos, "Top-K attention: history %d longer than %d", pos,
                 fg::kAttnTopkMaxPos);
    return fg::launch_attn_decode((const __half*)q, (const __half*)k_new, (const __half*)v_new, ld,
                                  kv, bls, d, pos, fuse_append != 0, (__half*)out,
                                  fg::as_stream(stream), topk);
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
