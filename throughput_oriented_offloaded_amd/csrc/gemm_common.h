// Pieces shared by the projection GEMM kernels (gemm.hip, gemm_sk.hip, gemm_sk32.hip).
#pragma once

#include "fg_internal.h"

namespace fg {
namespace gemm {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// y = act(x W^T + bias) + residual; tiles shared between workgroups leave
// fp32 partials in `part`.
struct Params {
    const __half* x;
    int64_t M, K, ldx;
    const void* w;       // fp16 [N, K] or 4-bit codes [N/2, K]
    const __half* meta;  // 4-bit (min, scale) rows [N/64, 2, K]
    int64_t N;
    const __half* bias;
    int32_t act;
    const __half* residual;
    __half* y;
    int64_t ldy;
    float* part;         // stream-K partials [slots][M][N] or null
    int32_t* tile_ns;    // stream-K with partials: segments of each tile [tiles],
                         // written by the workgroup that ends the tile
};

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return (uint32_t)__half_as_ushort(__float2half_rn(a)) |
           ((uint32_t)__half_as_ushort(__float2half_rn(b)) << 16);
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xffffu)));
}

// 8 consecutive k codes of one weight row (nibble `sh` of 8 bytes) -> fp16
// w = q * scale + min with the (min, scale) pairs of those k: nibble ->
// (0x6400 | q) = 1024 + q via v_perm_b32, minus 1024 (exact), then one fused
// fp16 multiply-add, so q * scale + min is rounded once, to fp16 (the fp32
// definition rounds to fp32 first; the two differ only where that first
// rounding lands on an fp16 tie).
__device__ __forceinline__ h8 dequant8(uint2 c, uint32_t sh, const uint4& mn, const uint4& sc) {
    const uint32_t d0 = (c.x >> sh) & 0x0f0f0f0fu;
    const uint32_t d1 = (c.y >> sh) & 0x0f0f0f0fu;
    const uint32_t magic = 0x64646464u;
    uint32_t p[4];
    p[0] = __builtin_amdgcn_perm(magic, d0, 0x04010400u);
    p[1] = __builtin_amdgcn_perm(magic, d0, 0x04030402u);
    p[2] = __builtin_amdgcn_perm(magic, d1, 0x04010400u);
    p[3] = __builtin_amdgcn_perm(magic, d1, 0x04030402u);
    const uint32_t mw[4] = {mn.x, mn.y, mn.z, mn.w};
    const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
    const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    h8 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h2 q = __builtin_bit_cast(h2, p[i]) - k1024;
        h2 w = __builtin_elementwise_fma(q, __builtin_bit_cast(h2, sw[i]),
                                         __builtin_bit_cast(h2, mw[i]));
        out[2 * i] = w[0];
        out[2 * i + 1] = w[1];
    }
    return out;
}

// Epilogue of one lane: 4 consecutive output columns n..n+3 of row m, with
// bias, ReLU and residual, written as fp16.
__device__ __forceinline__ void store4_final(const Params& p, int64_t m, int64_t n, const f4& v) {
    float o[4] = {v[0], v[1], v[2], v[3]};
    if (p.bias) {
        const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
        o[0] += h2f(bb.x); o[1] += h2f(bb.x >> 16);
        o[2] += h2f(bb.y); o[3] += h2f(bb.y >> 16);
    }
    if (p.act == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = fmaxf(o[i], 0.f);
    }
    if (p.residual) {
        const uint2 rr = *reinterpret_cast<const uint2*>(p.residual + m * p.ldy + n);
        o[0] += h2f(rr.x); o[1] += h2f(rr.x >> 16);
        o[2] += h2f(rr.y); o[3] += h2f(rr.y >> 16);
    }
    *reinterpret_cast<uint2*>(p.y + m * p.ldy + n) =
        make_uint2(pack_h2(o[0], o[1]), pack_h2(o[2], o[3]));
}

// Epilogue of one lane: 8 consecutive output columns n..n+7 of row m (two
// 8-byte halves: bias, residual and y need only 8-byte alignment).
__device__ __forceinline__ void store8_final(const Params& p, int64_t m, int64_t n, const float (&v)[8]) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = v[i];
    if (p.bias) {
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n + 4 * hlf);
            o[4 * hlf + 0] += h2f(bb.x); o[4 * hlf + 1] += h2f(bb.x >> 16);
            o[4 * hlf + 2] += h2f(bb.y); o[4 * hlf + 3] += h2f(bb.y >> 16);
        }
    }
    if (p.act == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaxf(o[i], 0.f);
    }
    if (p.residual) {
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const uint2 rr = *reinterpret_cast<const uint2*>(p.residual + m * p.ldy + n + 4 * hlf);
            o[4 * hlf + 0] += h2f(rr.x); o[4 * hlf + 1] += h2f(rr.x >> 16);
            o[4 * hlf + 2] += h2f(rr.y); o[4 * hlf + 3] += h2f(rr.y >> 16);
        }
    }
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf)
        *reinterpret_cast<uint2*>(p.y + m * p.ldy + n + 4 * hlf) =
            make_uint2(pack_h2(o[4 * hlf], o[4 * hlf + 1]), pack_h2(o[4 * hlf + 2], o[4 * hlf + 3]));
}

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory
// operations are outstanding / until every LDS operation has completed
constexpr int vmcnt_wait(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int LGKM_ZERO = 15 | (3 << 14) | (7 << 4);

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane.
// The LDS base travels in M0 (wave-uniform).
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)lds);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(g)
                 : "memory", "m0");
}
// Same, addressed as a wave-uniform 64-bit base (SGPRs) plus a 32-bit
// per-lane byte offset.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, const void* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)lds);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(voff), "s"(base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Stream-K schedule of the decode-shaped kernel (gemm_sk.hip): T = tiles x nk
// iterations (tile, 64-wide k-step) split over G workgroups, workgroup g
// taking the contiguous range [bnd[g], bnd[g+1]).
constexpr int kSkGroups = 256;   // one workgroup per CU of the 256-CU part
constexpr int64_t kSkDpRows = 576;   // above: data-parallel whole tiles (prefill shapes)
struct SkSched {
    int64_t T, G, nk;     // iterations, workgroups, k-steps per tile
    int64_t ntn, bm, bn;  // N tiles, tile rows, tile columns
    int64_t slots;        // partial slots per output element (1: none needed)
    int32_t wide;         // 1: 32-row blocks on 32x32x16 MFMA (gemm_sk32.hip)
    int32_t dp;           // 1: data-parallel, whole tiles g, g + G, ... (large M)
    int64_t tiles, mt;    // output tiles; M tiles
    int64_t band;         // dp: M tiles per band of the tile order
    // stream-K: iteration ranges balanced by time rather than by count: a
    // workgroup pays a fixed cost per segment (tile) it touches (pipeline
    // fill, the merge of the k-halves, the tile's stores) on top of its
    // k-steps, so ranges that cross a tile boundary are made shorter; empty
    // ranges are allowed
    int32_t bnd[kSkGroups + 1];
    // partial slot of workgroup g's first segment (g minus the owner of that
    // tile's first iteration); every later segment starts at its tile's
    // first k-step and takes slot 0
    int16_t slot0[kSkGroups];
};

// Output tile of linear index `tile`.  Stream-K: row-major (tm, tn).  Data-
// parallel: bands of `band` M tiles, M tile fastest inside a band, so the G
// tiles in flight at once cover about band x G/band tiles and share their
// activation and weight slices through L2 and the infinity cache.
__device__ __host__ __forceinline__ void sk_tile_coords(const SkSched& sc, int64_t tile, int64_t& tm,
                                                        int64_t& tn) {
    if (!sc.dp) {
        tm = tile / sc.ntn;
        tn = tile - tm * sc.ntn;
        return;
    }
    const int64_t per_band = sc.band * sc.ntn;
    const int64_t b = tile / per_band, r = tile - b * per_band;
    const int64_t left = sc.mt - b * sc.band;
    const int64_t gm = left < sc.band ? left : sc.band;      // the last band may be narrower
    tm = b * sc.band + r % gm;
    tn = r / gm;
}

// workgroup holding iteration x < T: the g with bnd[g] <= x < bnd[g + 1]
// (the last g with bnd[g] <= x, which skips empty ranges)
inline int32_t sk_owner_in(const int32_t* bnd, int32_t G, int64_t x) {
    int32_t lo = 0, hi = G;   // bnd[lo] <= x < bnd[hi]
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (bnd[mid] <= x) lo = mid;
        else hi = mid;
    }
    return lo;
}
inline int32_t sk_owner(const SkSched& sc, int64_t x) { return sk_owner_in(sc.bnd, (int32_t)sc.G, x); }
// Bytes of a stream-K launch's workspace: the partials, then (256-byte
// aligned) the segment count of every tile.
inline size_t sk_part_bytes(const SkSched& sc, int64_t M, int64_t N) {
    return (sc.slots * M * N * sizeof(float) + 255) / 256 * 256;
}
inline size_t sk_ws_bytes(const SkSched& sc, int64_t M, int64_t N) {
    return sc.slots > 1 ? sk_part_bytes(sc, M, N) + (size_t)sc.tiles * sizeof(int32_t) : 0;
}
SkSched sk_schedule(int64_t M, int64_t N, int64_t K);
int launch_sk(const Params& p, const SkSched& sc, bool q4, hipStream_t st);
int launch_sk32(const Params& p, const SkSched& sc, bool q4, hipStream_t st);
int launch_sk_reduce(const Params& p, const SkSched& sc, hipStream_t st);
// large-M fp16 GEMM (gemm_tile.hip): 256 x 256 tiles, whole K per workgroup
bool tile_fits(const Params& p);
int launch_tile(const Params& p, hipStream_t st);
// sk_reduce fused with the LayerNorm of each finished row (width N, ldy == N,
// N <= 32768) into ln_y [M, N]
int launch_sk_reduce_ln(const Params& p, const SkSched& sc, const __half* g, const __half* b,
                        __half* ln_y, hipStream_t st);


}  // namespace gemm
}  // namespace fg
