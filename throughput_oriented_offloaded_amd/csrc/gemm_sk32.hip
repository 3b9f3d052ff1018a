// Decode-shaped projection GEMM on 32x32x16 MFMA: y = act(x W^T + bias) +
// residual for a block of up to a few hundred rows, W in fp16 or in the
// group-wise 4-bit format, on the stream-K schedule of gemm_sk.hip.
//
// Why a second decode kernel (gfx950 measurements): a 32x32x16 f16 MFMA does
// twice the work of a 16x16x32 one per issue, and VALU work issued between
// them costs it far less matrix-core throughput (about 80% of peak with 2-4
// packed-fp16 VALU per MFMA at two wavefronts per SIMD, where 16x16x32 drops
// below 50% with one).  So here:
//  * rows come in blocks of 32 (a tile of 96 or 160 rows, where those fit the
//    block better than the other kernel's 128 or 144; rows past M repeat the
//    last row and are never stored);
//  * the weights are the A operand: lane l holds 8 consecutive k of weight row
//    (l mod 32) of a 32-row block, the activations the B operand (8 k of row
//    l mod 32), and the 16 accumulators of a lane are 4 groups of 4
//    consecutive output columns of one row: vector stores in the epilogue;
//  * 4-bit weights are dequantized in packed fp16: the nibble becomes the
//    fp16 value 1024 + q by a byte permute, 1024 is subtracted exactly, and
//    one fused multiply-add q * scale + min rounds once to fp16, with the
//    (min, scale) pairs taken from LDS as they are stored (no conversion);
//  * the workgroup is 8 wavefronts as in the 16x16x32 kernel: 4 columns of 64
//    weight rows (one 4-bit group each, two 32-row MFMA blocks) times 2
//    k-halves, added through LDS at the end; direct-to-LDS loads into an
//    NS-deep ring of stage buffers [meta | X tile | weight tile] with XOR
//    swizzles; each k-half of a stage is two MFMA k-steps of 16, and the next
//    step's weight fragments are dequantized while the current step's MFMAs
//    issue.
#include <hip/hip_ext.h>

#include "fg_trace.h"
#include "gemm_common.h"

namespace fg {
namespace gemm {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

template <int MB_, bool Q4_, int NS_>
struct SK32 {
    static constexpr int MB = MB_, NS = NS_, NW = 8;
    static constexpr bool Q4 = Q4_;
    static constexpr int BM = MB * 32, BN = 256, BK = 64, NT = NW * 64;
    static constexpr int M_INS = Q4 ? 1 : 0;            // (min, scale) rows of 4 groups: 1 KB
    static constexpr int X_INS = BM / 8;                 // activation tile: BM rows x 128 B
    static constexpr int C_INS = Q4 ? BN / 32 : BN / 8;  // 4-bit codes or fp16 weight rows
    static constexpr int INS = M_INS + X_INS + C_INS;    // 1 KB load instructions per stage
    static constexpr int LWL = INS / NW;                 // loads per wavefront ...
    static constexpr int XW = INS % NW;                  // ... plus one for the first XW
    static constexpr int LWH = LWL + (XW ? 1 : 0);
    static constexpr int M_BYTES = M_INS * 1024;
    static constexpr int X_BYTES = BM * 128;
    static constexpr int STAGE = INS * 1024;
    // k-half merge: one region per weight column (MB blocks x 16 floats x 64 lanes)
    static constexpr int MERGE = MB * 4096;
    static constexpr int PER_BUF = STAGE / MERGE;
    static_assert(PER_BUF >= 1 && (4 + PER_BUF - 1) / PER_BUF <= NS, "merge space");
    static_assert(LWH * (NS - 1) <= 63, "vmcnt range");
};

template <class C>
__global__ __launch_bounds__(C::NT) void sk32_kernel(Params p, SkSched sc) {
    __shared__ __align__(16) unsigned char sb0[C::STAGE];
    __shared__ __align__(16) unsigned char sb1[C::STAGE];
    __shared__ __align__(16) unsigned char sb2[C::NS > 2 ? C::STAGE : 16];
    __shared__ __align__(16) unsigned char sb3[C::NS > 3 ? C::STAGE : 16];
    __shared__ __align__(16) unsigned char sb4[C::NS > 4 ? C::STAGE : 16];
    auto buf = [&](int s) -> unsigned char* {
        return s == 0 ? sb0 : (s == 1 ? sb1 : (s == 2 ? sb2 : (s == 3 ? sb3 : sb4)));
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave >> 2, wc = wave & 3;      // k-half, weight column
    const bool hiw = wave < C::XW;                // issues LWH loads per stage
    const int r32 = lane & 31, hl = lane >> 5;    // operand row, 8-k half of a k-step
    const uint32_t shn = (uint32_t)(r32 & 1) * 4u;   // nibble of this lane's weight row
    const int64_t g = blockIdx.x;
    const int64_t it_beg = sc.bnd[g], it_end = sc.bnd[g + 1];

    for (int64_t it = it_beg; it < it_end;) {
        const int64_t tile = it / sc.nk;
        const int kb = (int)(it - tile * sc.nk);
        const int ke = (int)(min(it_end, (tile + 1) * sc.nk) - tile * sc.nk);
        it = tile * sc.nk + ke;
        const int64_t tm = tile / sc.ntn, tn = tile - tm * sc.ntn;
        const int64_t n0 = tn * C::BN, m0 = tm * C::BM;
        const int nk = ke - kb;
        const int64_t kbeg = (int64_t)kb * C::BK;

        f16v acc[2][C::MB];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < C::MB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        // load slots of this wave: a wave-uniform base (tile origin at kbeg)
        // and a per-lane byte offset inside the tile; rows past M or N are
        // clamped (their results are never stored)
        const char* sbase[C::LWH];
        uint32_t voff[C::LWH];
        int ksh[C::LWH];
#pragma unroll
        for (int i = 0; i < C::LWH; ++i) {
            const int j = min(wave + i * C::NW, C::INS - 1);
            if (j < C::M_INS) {
                const int c = j * 64 + lane;
                const int row = c >> 3, col = c & 7;            // row = group * 2 + (min | scale)
                const int64_t gg = min(n0 / 64 + (row >> 1), p.N / 64 - 1) - n0 / 64;
                sbase[i] = (const char*)(p.meta + (n0 / 64) * 2 * p.K + kbeg);
                voff[i] = (uint32_t)(((gg * 2 + (row & 1)) * p.K + col * 8) * 2);
                ksh[i] = 1;
            } else if (j < C::M_INS + C::X_INS) {
                const int c = (j - C::M_INS) * 64 + lane;
                const int row = c >> 3, kc = (c & 7) ^ (row & 7);
                const int64_t gr = min(m0 + row, p.M - 1) - m0;
                sbase[i] = (const char*)(p.x + m0 * p.ldx + kbeg);
                voff[i] = (uint32_t)((gr * p.ldx + kc * 8) * 2);
                ksh[i] = 1;
            } else {
                const int c = (j - C::M_INS - C::X_INS) * 64 + lane;
                if constexpr (C::Q4) {
                    const int row = c >> 2, ch = (c & 3) ^ ((row >> 1) & 3);
                    const int64_t gr = min(n0 / 2 + row, p.N / 2 - 1) - n0 / 2;
                    sbase[i] = (const char*)p.w + (n0 / 2) * p.K + kbeg;
                    voff[i] = (uint32_t)(gr * p.K + ch * 16);
                    ksh[i] = 0;
                } else {
                    const int row = c >> 3, kc = (c & 7) ^ (row & 7);
                    const int64_t gr = min(n0 + row, p.N - 1) - n0;
                    sbase[i] = (const char*)((const __half*)p.w + n0 * p.K + kbeg);
                    voff[i] = (uint32_t)((gr * p.K + kc * 8) * 2);
                    ksh[i] = 1;
                }
            }
            // wave-uniform: keep base and shift in scalar registers
            // (readfirstlane returns a signed int: widen through uint32_t)
            const uint64_t bb = (uint64_t)(uintptr_t)sbase[i];
            const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bb >> 32));
            const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bb);
            sbase[i] = (const char*)(uintptr_t)(((uint64_t)bhi << 32) | (uint64_t)blo);
            ksh[i] = __builtin_amdgcn_readfirstlane(ksh[i]);
        }
        // stages past the end reload the last one, so every stage issues the
        // same number of loads per wave (the vmcnt arithmetic holds)
        auto issue = [&](unsigned char* base, int ks) {
            const int64_t koff = (int64_t)min(ks, nk - 1) * C::BK;
#pragma unroll
            for (int i = 0; i < C::LWH; ++i) {
                if (i < C::LWL || hiw) {
                    const int j = wave + i * C::NW;
                    dma16s(sbase[i] + (koff << ksh[i]), voff[i], base + j * 1024);
                }
            }
        };

        // fragments of k-step ks (0, 1) of this wave's k-half: k = 32 kh + 16 ks + 8 hl + 0..7
        auto read_x = [&](const unsigned char* base, int mb, int ks) -> h8 {
            const int row = mb * 32 + r32;
            const int kc = (kh * 4 + ks * 2 + hl) ^ (row & 7);
            return *reinterpret_cast<const h8*>(base + C::M_BYTES + (row * 8 + kc) * 16);
        };
        auto read_c = [&](const unsigned char* base, int nb, int ks) -> uint2 {
            const int nl = wc * 64 + nb * 32 + r32;
            const int row = nl >> 1, ch = (kh * 2 + ks) ^ ((row >> 1) & 3);
            return *reinterpret_cast<const uint2*>(base + C::M_BYTES + C::X_BYTES + (row * 4 + ch) * 16 + hl * 8);
        };
        auto read_w16 = [&](const unsigned char* base, int nb, int ks) -> h8 {
            const int nl = wc * 64 + nb * 32 + r32;
            const int kc = (kh * 4 + ks * 2 + hl) ^ (nl & 7);
            return *reinterpret_cast<const h8*>(base + C::X_BYTES + (nl * 8 + kc) * 16);
        };
        auto read_meta = [&](const unsigned char* base, int ks, uint4& mn, uint4& s4) {
            const int off = (kh * 32 + ks * 16 + hl * 8) * 2;
            mn = *reinterpret_cast<const uint4*>(base + (wc * 2 + 0) * 128 + off);
            s4 = *reinterpret_cast<const uint4*>(base + (wc * 2 + 1) * 128 + off);
        };
        // MFMAs of one k-step, each activation fragment replaced by `nxt`'s
        // fragment of k-step nks right after its last use
        auto step = [&](h8 w0, h8 w1, h8 (&xf)[C::MB], const unsigned char* nxt, int nks) {
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
                acc[0][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(w0, xf[mb], acc[0][mb], 0, 0, 0);
                acc[1][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(w1, xf[mb], acc[1][mb], 0, 0, 0);
                xf[mb] = read_x(nxt, mb, nks);
            }
        };
        // interleave: per activation block 2 MFMAs with VALU between them and
        // 1 LDS read; the VALU starts at the third block (the first ones give
        // the code / metadata reads of the step time to land)
        auto pattern_b = [&]() {
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                if (mb >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                if (mb >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
            }
        };

        h8 xf[C::MB];
        h8 w0, w1;               // weight fragments of the current k-step
        // the next step's fragments are complete here: the compiler may not
        // sink their dequantization past the barrier, next to the first use
        // (it would then run as one VALU block beside no MFMA)
        auto pin = [](h8& a, h8& b) { asm volatile("" : "+v"(a), "+v"(b)); };
        // codes and (min, scale) pairs of one k-step -> its two weight fragments
        auto load_step = [&](const unsigned char* base, int ks, uint2& c0, uint2& c1, uint4& mn, uint4& s4) {
            c0 = read_c(base, 0, ks);
            c1 = read_c(base, 1, ks);
            read_meta(base, ks, mn, s4);
        };
        // prologue: NS stages in flight; publish stage 0 and read its fragments
#pragma unroll
        for (int s = 0; s < C::NS; ++s) issue(buf(s), s);
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::LWL * (C::NS - 1)));
        __builtin_amdgcn_s_barrier();
        {
            const unsigned char* b0 = buf(0);
            if constexpr (C::Q4) {
                uint2 c0, c1;
                uint4 mn, s4;
                load_step(b0, 0, c0, c1, mn, s4);
                w0 = dequant8(c0, shn, mn, s4);
                w1 = dequant8(c1, shn, mn, s4);
            } else {
                w0 = read_w16(b0, 0, 0);
                w1 = read_w16(b0, 1, 0);
            }
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) xf[mb] = read_x(b0, mb, 0);
        }

        // each stage enters with its k-step 0 activation and weight fragments
        // in registers
        for (int kt = 0; kt < nk; kt += C::NS) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const int i = kt + s;
                if (i < nk) {
                    const unsigned char* cur = buf(s);
                    const unsigned char* nxt = buf((s + 1) % C::NS);
                    // k-step 0; k-step 1's weights read and prepared meanwhile
                    h8 v0, v1;
                    if constexpr (C::Q4) {
                        uint2 c0, c1;
                        uint4 mn, s4;
                        load_step(cur, 1, c0, c1, mn, s4);
                        v0 = dequant8(c0, shn, mn, s4);
                        v1 = dequant8(c1, shn, mn, s4);
                    } else {
                        v0 = read_w16(cur, 0, 1);
                        v1 = read_w16(cur, 1, 1);
                    }
                    step(w0, w1, xf, cur, 1);
                    if constexpr (C::Q4) pattern_b();
                    pin(v0, v1);
                    w0 = v0;
                    w1 = v1;
                    // stage i+1 has landed for every wave (the wait is the one
                    // of the waves with fewer loads: stronger for the others),
                    // and no wave still reads stage i: refill its buffer with
                    // stage i+NS
                    __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::LWL * (C::NS - 2)));
                    __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
                    __builtin_amdgcn_s_barrier();
                    issue(buf(s), i + C::NS);
                    // k-step 1; the next stage's k-step 0 fragments meanwhile
                    if constexpr (C::Q4) {
                        uint2 c0, c1;
                        uint4 mn, s4;
                        load_step(nxt, 0, c0, c1, mn, s4);
                        v0 = dequant8(c0, shn, mn, s4);
                        v1 = dequant8(c1, shn, mn, s4);
                    } else {
                        v0 = read_w16(nxt, 0, 0);
                        v1 = read_w16(nxt, 1, 0);
                    }
                    step(w0, w1, xf, nxt, 0);
                    if constexpr (C::Q4) pattern_b();
                    pin(v0, v1);
                    w0 = v0;
                    w1 = v1;
                }
            }
        }
        // no load may still be writing LDS when the buffers are reused
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
        __builtin_amdgcn_s_barrier();

        // add the two k-halves (kh = 1 -> LDS -> kh = 0), one column block per round
        // the whole tile in this segment: final outputs; else its partial slot
        const bool full = kb == 0 && ke == (int)sc.nk;
        const int slot = kb == 0 ? 0 : (int)sc.slot0[g];
        // the workgroup that ends a tile records how many segments it has
        if (p.tile_ns && ke == (int)sc.nk && tid == 0) p.tile_ns[tile] = slot + 1;
        float4* reg = reinterpret_cast<float4*>(buf(wc / C::PER_BUF) + (wc % C::PER_BUF) * C::MERGE);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            if (kh == 1) {
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        reg[(mb * 4 + q4) * 64 + lane] =
                            make_float4(acc[nb][mb][4 * q4], acc[nb][mb][4 * q4 + 1],
                                        acc[nb][mb][4 * q4 + 2], acc[nb][mb][4 * q4 + 3]);
            }
            __syncthreads();
            if (kh == 0) {
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb) {
                    const int64_t m = m0 + mb * 32 + r32;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const float4 o = reg[(mb * 4 + q4) * 64 + lane];
                        f4 v = {acc[nb][mb][4 * q4] + o.x, acc[nb][mb][4 * q4 + 1] + o.y,
                                acc[nb][mb][4 * q4 + 2] + o.z, acc[nb][mb][4 * q4 + 3] + o.w};
                        const int64_t n = n0 + wc * 64 + nb * 32 + q4 * 8 + hl * 4;
                        if (m < p.M && n < p.N) {
                            if (full) {
                                store4_final(p, m, n, v);
                            } else {
                                float* dst = p.part + ((int64_t)slot * p.M + m) * p.N + n;
                                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                            }
                        }
                    }
                }
            }
            __syncthreads();
        }
    }
}

template <class C>
int run32(const Params& p, const SkSched& sc, hipStream_t st) {
    hipEvent_t ea, eb;   // the enclosing trace scope's events, if any
    trace_take_ext(&ea, &eb);
    hipExtLaunchKernelGGL(sk32_kernel<C>, dim3((unsigned)sc.G), dim3(C::NT), 0, st, ea, eb, 0u, p, sc);
    FG_LAUNCHED("sk32_kernel");
    return FG_OK;
}

}  // namespace

int launch_sk32(const Params& p, const SkSched& sc, bool q4, hipStream_t st) {
    const int MB = (int)(sc.bm / 32);
    if (q4) {
        switch (MB) {
            case 3: return run32<SK32<3, true, 5>>(p, sc, st);
            case 5: return run32<SK32<5, true, 5>>(p, sc, st);
            default: break;
        }
    } else {
        switch (MB) {
            case 3: return run32<SK32<3, false, 3>>(p, sc, st);
            case 5: return run32<SK32<5, false, 3>>(p, sc, st);
            default: break;
        }
    }
    return set_error(FG_ERR_UNSUPPORTED, "no 32-row decode kernel for %lld-row tiles", (long long)sc.bm);
}

}  // namespace gemm
}  // namespace fg
