// Causal prompt attention for the prefill ("FlexGen 完全拆解", section
// "从 Transformer 推理的数据流重新定义卸载": K, V, Q of all s prompt tokens
// are computed at once, and token t attends to tokens 0..t).
//
// Flash-style on 16x16x32 f16 MFMA, fp32 accumulation and online softmax in
// log2 units.  Workgroup = (sequence, head, block of 64 query rows), 4
// wavefronts of 16 rows each.  Keys and values come in tiles of 64 positions
// staged in LDS (the next tile is loaded into registers while the current one
// is used): K row-major, V transposed (dims x positions) so both MFMA operands
// are read as contiguous 8-element fragments.
//
//  * scores are computed transposed, S^T = K Q^T (A = 16 key rows x 32 dims,
//    B = Q^T held in registers): lane l then holds 16 scores of query row
//    l mod 16, at positions 16 t + 4 (l / 16) + i (t < 4, i < 4);
//  * those are exactly the positions that lane supplies as the B operand of
//    O^T = V^T P^T for a 32-position k-step, in the order {4 (l / 16) + i} then
//    {16 + 4 (l / 16) + i}; the A operand (V^T rows) is read in the same order,
//    so P never leaves its lane;
//  * the output accumulators of a lane all belong to its query row, so the
//    rescale by exp2(m_old - m_new) and the final 1 / l are per-lane scalars.
#include "fg_internal.h"
#include "fg_trace.h"

namespace fg {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int KT = 64;     // positions per key / value tile
constexpr int QB = 64;     // query rows per workgroup

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr uint32_t SEL_LO = 0x05040100u;  // (low half of a, low half of b)
constexpr uint32_t SEL_HI = 0x07060302u;  // (high half of a, high half of b)

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return (uint32_t)__half_as_ushort(__float2half_rn(a)) |
           ((uint32_t)__half_as_ushort(__float2half_rn(b)) << 16);
}

template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const __half* __restrict__ qkv,
                                                           int32_t s, int32_t nh, int32_t nqb,
                                                           __half* __restrict__ out) {
    constexpr int KS = HD / 32;          // 32-dim k-steps of a score
    constexpr int DT = HD / 16;          // 16-dim output tiles
    constexpr int KPAD = HD + 8;         // K tile row stride (halves)
    constexpr int VPAD = KT + 8;         // V^T tile row stride (halves)
    constexpr int OCT = HD / 8;          // 8-dim octets of a row
    constexpr int KCH = KT * OCT / 256;  // K 16-byte chunks per thread
    constexpr int VTASK = (KT / 4) * OCT;   // V tasks: 4 positions x 8 dims
    __shared__ __align__(16) __half ks[KT * KPAD];
    __shared__ __align__(16) __half vt[HD * VPAD];

    const int h1 = nh * HD;
    const int64_t ld = 3 * (int64_t)h1;
    // larger query blocks (more tiles) first
    const int qblk = nqb - 1 - (int)(blockIdx.x % nqb);
    const int64_t bh = blockIdx.x / nqb;
    const int64_t b = bh / nh;
    const int h = (int)(bh - b * nh);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int q0w = qblk * QB + wave * 16;          // first query row of this wave
    const int q = q0w + r16;                        // this lane's query row
    const int qe = min(q, s - 1);                   // rows past s behave as row s-1
    const __half* seq = qkv + b * (int64_t)s * ld + h * HD;

    // Q^T fragments: row qe, dims 32 ks + 8 g4 .. + 8
    h8 qf[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k)
        qf[k] = *reinterpret_cast<const h8*>(seq + (int64_t)qe * ld + 32 * k + 8 * g4);
    const float qscale = LOG2E / sqrtf((float)HD);

    f4 oacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = f4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    // tiles needed by the workgroup: positions 0 .. min(last row, s - 1)
    const int last = min(qblk * QB + QB - 1, s - 1);
    const int ntile = last / KT + 1;
    const int wlast = min(q0w + 15, s - 1);         // last row of this wave

    // staging: the next tile's K rows (KCH 16-byte chunks per thread) and,
    // for the first VTASK threads, 4 positions x 8 dims of V
    uint4 kr0, kr1, kr2, kr3, vr0, vr1, vr2, vr3;
    const int kc_j = tid / OCT, kc_o = tid % OCT;          // chunk i: position kc_j + i * (256 / OCT)
    const int v_pq = tid / OCT, v_o = tid % OCT;
    const bool v_own = tid < VTASK;
#define FG_KROW(I, P0) (seq + (int64_t)min((P0) + kc_j + (I) * (256 / OCT), s - 1) * ld + h1 + kc_o * 8)
#define FG_VROW(J, P0) (seq + (int64_t)min((P0) + 4 * v_pq + (J), s - 1) * ld + 2 * h1 + v_o * 8)
#define FG_GLOAD(P0)                                                                  \
    do {                                                                              \
        kr0 = *reinterpret_cast<const uint4*>(FG_KROW(0, P0));                        \
        kr1 = *reinterpret_cast<const uint4*>(FG_KROW(1, P0));                        \
        if (KCH > 2) {                                                                \
            kr2 = *reinterpret_cast<const uint4*>(FG_KROW(2, P0));                    \
            kr3 = *reinterpret_cast<const uint4*>(FG_KROW(3, P0));                    \
        }                                                                             \
        if (v_own) {                                                                  \
            vr0 = *reinterpret_cast<const uint4*>(FG_VROW(0, P0));                    \
            vr1 = *reinterpret_cast<const uint4*>(FG_VROW(1, P0));                    \
            vr2 = *reinterpret_cast<const uint4*>(FG_VROW(2, P0));                    \
            vr3 = *reinterpret_cast<const uint4*>(FG_VROW(3, P0));                    \
        }                                                                             \
    } while (0)
    static_assert(KCH == 2 || KCH == 4, "K staging: 2 or 4 chunks per thread");

    FG_GLOAD(0);
    for (int t = 0; t < ntile; ++t) {
        __syncthreads();                 // the previous tile is no longer read
        {
            *reinterpret_cast<uint4*>(&ks[(kc_j + 0 * (256 / OCT)) * KPAD + kc_o * 8]) = kr0;
            *reinterpret_cast<uint4*>(&ks[(kc_j + 1 * (256 / OCT)) * KPAD + kc_o * 8]) = kr1;
            if (KCH > 2) {
                *reinterpret_cast<uint4*>(&ks[(kc_j + 2 * (256 / OCT)) * KPAD + kc_o * 8]) = kr2;
                *reinterpret_cast<uint4*>(&ks[(kc_j + 3 * (256 / OCT)) * KPAD + kc_o * 8]) = kr3;
            }
            if (v_own) {
                // 4 positions x 8 dims -> V^T rows 8 o + e, columns 4 pq .. 4 pq + 3
                const uint32_t w0[4] = {vr0.x, vr0.y, vr0.z, vr0.w}, w1[4] = {vr1.x, vr1.y, vr1.z, vr1.w};
                const uint32_t w2[4] = {vr2.x, vr2.y, vr2.z, vr2.w}, w3[4] = {vr3.x, vr3.y, vr3.z, vr3.w};
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const uint2 lo = make_uint2(__builtin_amdgcn_perm(w1[e2], w0[e2], SEL_LO),
                                                __builtin_amdgcn_perm(w3[e2], w2[e2], SEL_LO));
                    const uint2 hi = make_uint2(__builtin_amdgcn_perm(w1[e2], w0[e2], SEL_HI),
                                                __builtin_amdgcn_perm(w3[e2], w2[e2], SEL_HI));
                    *reinterpret_cast<uint2*>(&vt[(8 * v_o + 2 * e2) * VPAD + 4 * v_pq]) = lo;
                    *reinterpret_cast<uint2*>(&vt[(8 * v_o + 2 * e2 + 1) * VPAD + 4 * v_pq]) = hi;
                }
            }
        }
        __syncthreads();
        if (t + 1 < ntile) FG_GLOAD((t + 1) * KT);   // in flight while this tile is used
#undef FG_GLOAD
#undef FG_VROW
#undef FG_KROW
        const int p0 = t * KT;
        if (p0 > wlast) continue;        // every position of the tile is masked for this wave

        // S^T tiles: 16 positions x 16 query rows each
        f4 sacc[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            sacc[pt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const h8 kf = *reinterpret_cast<const h8*>(&ks[(16 * pt + r16) * KPAD + 32 * k + 8 * g4]);
                sacc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[k], sacc[pt], 0, 0, 0);
            }
        }
        // scale, causal mask (position > row, or past s), tile maximum of the row
        float mt = -INFINITY;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = p0 + 16 * pt + 4 * g4 + i;
                const float v = (p <= qe) ? sacc[pt][i] * qscale : -INFINITY;
                sacc[pt][i] = v;
                mt = fmaxf(mt, v);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);   // finite: position 0 <= qe is in tile 0
        const float alpha = exp2f(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
        // P as the B operand of two 32-position k-steps
        h8 pb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pa = exp2f(sacc[2 * j][i] - mn), pc = exp2f(sacc[2 * j + 1][i] - mn);
                l += pa + pc;
                pb[j][i] = (_Float16)pa;
                pb[j][4 + i] = (_Float16)pc;
            }
        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const __half* row = &vt[(16 * dt + r16) * VPAD + 32 * j + 4 * g4];
                const uint2 a0 = *reinterpret_cast<const uint2*>(row);
                const uint2 a1 = *reinterpret_cast<const uint2*>(row + 16);
                const h8 vf = __builtin_bit_cast(h8, make_uint4(a0.x, a0.y, a1.x, a1.y));
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[j], oacc[dt], 0, 0, 0);
            }
    }
    // the row's sum is spread over the 4 lanes with the same query row
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (q < s) {
        const float inv = 1.0f / l;
        __half* orow = out + (b * (int64_t)s + q) * h1 + h * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g4) =
                make_uint2(pack_h2(oacc[dt][0] * inv, oacc[dt][1] * inv),
                           pack_h2(oacc[dt][2] * inv, oacc[dt][3] * inv));
    }
}

}  // namespace

int launch_attn_prefill(const __half* qkv, int32_t b, int32_t s, const fg_dims* d, __half* out,
                        hipStream_t st) {
    if (b == 0 || s == 0) return FG_OK;
    if (d->head_dim != 64 && d->head_dim != 128)
        return set_error(FG_ERR_UNSUPPORTED, "prefill attention: head_dim %d", d->head_dim);
    const int nqb = (int)cdiv(s, QB);
    const int64_t grid = (int64_t)b * d->n_heads * nqb;
    if (grid > INT32_MAX) return set_error(FG_ERR_UNSUPPORTED, "prefill grid too large");
    TraceScope ts(TK_ATTN_PREFILL, st, 4.0 * b * d->h1 * (double)s * (s + 1) / 2,
                  (double)b * s * d->h1 * 2 * 4);
    if (d->head_dim == 128)
        attn_prefill_kernel<128><<<(unsigned)grid, 256, 0, st>>>(qkv, s, d->n_heads, nqb, out);
    else
        attn_prefill_kernel<64><<<(unsigned)grid, 256, 0, st>>>(qkv, s, d->n_heads, nqb, out);
    FG_LAUNCHED("attn_prefill_kernel");
    return FG_OK;
}

}  // namespace fg

extern "C" int fg_attn_prefill(const void* qkv, int32_t b, int32_t s, const fg_dims* d, void* out,
                               void* stream) {
    fg::clear_error();
    FG_TRY(fg::check_dims(d));
    FG_CHECK_ARG(qkv && out, "null pointer argument");
    FG_CHECK_ARG(b >= 0 && s >= 0, "negative sizes");
    FG_CHECK_ARG(((uintptr_t)qkv | (uintptr_t)out) % 16 == 0, "pointers must be 16-byte aligned");
    return fg::launch_attn_prefill((const __half*)qkv, b, s, d, (__half*)out, fg::as_stream(stream));
}
