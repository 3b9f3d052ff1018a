// Pipelined projection GEMM for decode-shaped contractions (M = bls rows, a
// few hundred at most): y = act(x W^T + bias) + residual with W in fp16 or in
// the group-wise 4-bit format.
//
// Why this shape of kernel (gfx950 measurements):
//  * The weights stream from HBM once per layer and step; what limits the
//    kernel is keeping the MFMA pipe fed, so the tile keeps every m row of the
//    block (M = 144 -> 9 blocks of 16) and 4 waves x 64 weight rows (one
//    4-bit group per wave) along N.
//  * Global -> LDS traffic uses direct-to-LDS loads (global_load_lds_dwordx4,
//    16 B per lane) into an NS-deep ring of stage buffers, so several k-steps
//    are in flight without staging registers; each stage is published with an
//    explicit s_waitcnt vmcnt + s_barrier.  The loads are issued as inline asm
//    so that the compiler adds no waits of its own on the LDS ring.
//  * LDS layout per stage: [meta | X tile | weight tile], 1 KB per load
//    instruction, with XOR swizzles chosen so that fragment reads are free of
//    bank conflicts (measured: zero SQ_LDS_BANK_CONFLICT).
//  * Each k-step is processed in two 32-wide halves, software-pipelined: the
//    MFMAs of one half run while the LDS reads and the dequantization of the
//    next half proceed, so MFMA issue is rarely starved.
//  * Weight fragments are the MFMA A operand (16 n x 32 k), activation rows the
//    B operand (32 k x 16 m): each lane's 4 accumulators are 4 consecutive
//    output columns, stored as one 8-byte (fp16) or 16-byte (partial) write.
#include "gemm_common.h"

namespace fg {
namespace gemm {
namespace {

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
#pragma clang diagnostic pop

template <int MB_, bool Q4_, int NS_>
struct PC {
    static constexpr int MB = MB_, NS = NS_, WN = 4;
    static constexpr bool Q4 = Q4_;
    static constexpr int BM = MB * 16, BN = WN * 64, BK = 64, NT = WN * 64;
    static constexpr int M_INS = Q4 ? 1 : 0;           // (min, scale) rows of 4 groups: 1 KB
    static constexpr int X_INS = BM / 8;                // activation tile: BM rows x 128 B
    static constexpr int C_INS = Q4 ? BN / 32 : BN / 8; // 4-bit codes or fp16 weight rows
    static constexpr int INS = M_INS + X_INS + C_INS;   // 1 KB load instructions per stage
    static constexpr int LW = (INS + WN - 1) / WN;      // per wave
    static constexpr int M_BYTES = M_INS * 1024;
    static constexpr int X_BYTES = BM * 128;
    static constexpr int STAGE = INS * 1024;
    static_assert(X_INS * 1024 == X_BYTES, "tile rows");
    static_assert(LW * (NS - 1) <= 63, "vmcnt range");
};

template <class C>
__global__ __launch_bounds__(C::NT) void pipe_kernel(Params p) {
    __shared__ __align__(16) unsigned char sb0[C::STAGE];
    __shared__ __align__(16) unsigned char sb1[C::STAGE];
    __shared__ __align__(16) unsigned char sb2[C::STAGE];
    __shared__ __align__(16) unsigned char sb3[C::NS > 3 ? C::STAGE : 16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * C::BN;
    const int64_t m0 = (int64_t)blockIdx.y * C::BM;
    const int64_t kbeg = (int64_t)blockIdx.z * p.kchunk;
    const int64_t kend = min(p.K, kbeg + p.kchunk);
    const int nk = kbeg < kend ? (int)((kend - kbeg) / C::BK) : 0;

    f4 acc[4][C::MB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < C::MB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) {
        // per-lane global address of each of this wave's load slots at k = kbeg;
        // rows past M or N are clamped (their results are never stored)
        const char* gp[C::LW];
        int ksh[C::LW];
#pragma unroll
        for (int i = 0; i < C::LW; ++i) {
            const int j = min(wave + i * C::WN, C::INS - 1);  // spare slots repeat the last load
            if (j < C::M_INS) {
                const int c = j * 64 + lane;
                const int row = c >> 3, col = c & 7;            // row = group * 2 + (min | scale)
                const int64_t gg = min(n0 / 64 + (row >> 1), p.N / 64 - 1);
                gp[i] = (const char*)(p.meta + (gg * 2 + (row & 1)) * p.K + kbeg + col * 8);
                ksh[i] = 1;
            } else if (j < C::M_INS + C::X_INS) {
                const int c = (j - C::M_INS) * 64 + lane;
                const int row = c >> 3, kc = (c & 7) ^ (row & 7);
                const int64_t gr = min(m0 + row, p.M - 1);
                gp[i] = (const char*)(p.x + gr * p.ldx + kbeg + kc * 8);
                ksh[i] = 1;
            } else {
                const int c = (j - C::M_INS - C::X_INS) * 64 + lane;
                if constexpr (C::Q4) {
                    const int row = c >> 2, ch = (c & 3) ^ ((row >> 1) & 3);
                    const int64_t gr = min(n0 / 2 + row, p.N / 2 - 1);
                    gp[i] = (const char*)p.w + gr * p.K + kbeg + ch * 16;
                    ksh[i] = 0;
                } else {
                    const int row = c >> 3, kc = (c & 7) ^ (row & 7);
                    const int64_t gr = min(n0 + row, p.N - 1);
                    gp[i] = (const char*)((const __half*)p.w + gr * p.K + kbeg + kc * 8);
                    ksh[i] = 1;
                }
            }
        }
        auto buf = [&](int s) -> unsigned char* {
            return s == 0 ? sb0 : (s == 1 ? sb1 : (s == 2 ? sb2 : sb3));
        };
        // stages past the end reload the last one into a free buffer, so every
        // stage issues the same number of loads (the vmcnt arithmetic holds)
        auto issue = [&](unsigned char* base, int ks) {
            const int64_t koff = (int64_t)min(ks, nk - 1) * C::BK;
#pragma unroll
            for (int i = 0; i < C::LW; ++i) {
                const int j = min(wave + i * C::WN, C::INS - 1);
                dma16(gp[i] + (koff << ksh[i]), base + j * 1024);
            }
        };

        h8 xa[C::MB], xb[C::MB], wa[4], wb[4];
        uint2 cr[4];
        uint4 mnr, scr;
        const uint32_t shn = (uint32_t)(r16 & 1) * 4u;   // nibble of this lane's weight row
        auto read_half = [&](const unsigned char* base, int kk, h8* xf, h8* wf16) {
            if constexpr (C::Q4) {
                mnr = *reinterpret_cast<const uint4*>(base + (wave * 2 + 0) * 128 + (kk * 32 + q * 8) * 2);
                scr = *reinterpret_cast<const uint4*>(base + (wave * 2 + 1) * 128 + (kk * 32 + q * 8) * 2);
                const unsigned char* cs = base + C::M_BYTES + C::X_BYTES;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int nl = wave * 64 + nb * 16 + r16;
                    const int row = nl >> 1, ch = (kk * 2 + (q >> 1)) ^ ((row >> 1) & 3);
                    cr[nb] = *reinterpret_cast<const uint2*>(cs + (row * 4 + ch) * 16 + (q & 1) * 8);
                }
            } else {
                const unsigned char* ws = base + C::M_BYTES + C::X_BYTES;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int nl = wave * 64 + nb * 16 + r16;
                    const int kc = (kk * 4 + q) ^ (nl & 7);
                    wf16[nb] = *reinterpret_cast<const h8*>(ws + (nl * 8 + kc) * 16);
                }
            }
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
                const int row = mb * 16 + r16;
                const int kc = (kk * 4 + q) ^ (row & 7);
                xf[mb] = *reinterpret_cast<const h8*>(base + C::M_BYTES + (row * 8 + kc) * 16);
            }
        };
        // MFMAs of one half with the current fragments; the next half's weight
        // fragments are dequantized in between
        auto mfma_half = [&](const h8* wcur, const h8* xcur, h8* wnext) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                if constexpr (C::Q4) wnext[nb] = dequant8(cr[nb], shn, mnr, scr);
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wcur[nb], xcur[mb],
                                                                         acc[nb][mb], 0, 0, 0);
            }
        };

        // prologue: all NS stages in flight; publish stage 0
#pragma unroll
        for (int s = 0; s < C::NS; ++s) issue(buf(s), s);
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::LW * (C::NS - 1)));
        __builtin_amdgcn_s_barrier();
        read_half(buf(0), 0, xa, wa);
        if constexpr (C::Q4) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) wa[nb] = dequant8(cr[nb], shn, mnr, scr);
        }

        for (int kt = 0; kt < nk; kt += C::NS) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const int i = kt + s;
                if (i < nk) {
                    // half 0 of stage i is in (wa, xa); fetch half 1
                    read_half(buf(s), 1, xb, wb);
                    mfma_half(wa, xa, wb);
                    // stage i+1 has landed for this wave; after the barrier it has
                    // for every wave, and no wave still reads stage i's buffer
                    __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::LW * (C::NS - 2)));
                    __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
                    __builtin_amdgcn_s_barrier();
                    issue(buf(s), i + C::NS);
                    // half 1 of stage i is in (wb, xb); fetch half 0 of stage i+1
                    read_half(buf((s + 1) % C::NS), 0, xa, wa);
                    mfma_half(wb, xb, wa);
                }
            }
        }
        // no load may still be writing LDS when the workgroup retires
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    }

    const int nq = q * 4;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int64_t n = n0 + wave * 64 + nb * 16 + nq;
        if (n >= p.N) continue;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
            const int64_t m = m0 + mb * 16 + r16;
            if (m < p.M) store4(p, m, n, acc[nb][mb], blockIdx.z);
        }
    }
}

template <class C>
int run(const Params& p, int S, hipStream_t st) {
    const dim3 grid((unsigned)cdiv(p.N, C::BN), (unsigned)cdiv(p.M, C::BM), (unsigned)S);
    pipe_kernel<C><<<grid, C::NT, 0, st>>>(p);
    FG_LAUNCHED("pipe_kernel");
    return FG_OK;
}

}  // namespace

int pipe_mb_for(int64_t M) {
    if (M <= 16) return 1;
    if (M <= 32) return 2;
    if (M <= 64) return 4;
    if (M <= 128) return 8;
    // 144-row tiles unless 128-row tiles pad less (e.g. M = 256)
    return cdiv(M, 128) * 128 < cdiv(M, 144) * 144 ? 8 : 9;
}

int launch_pipe(const Params& p, int MB, bool q4, int S, hipStream_t st) {
    if (q4) {
        switch (MB) {
            case 1: return run<PC<1, true, 4>>(p, S, st);
            case 2: return run<PC<2, true, 4>>(p, S, st);
            case 4: return run<PC<4, true, 4>>(p, S, st);
            case 8: return run<PC<8, true, 4>>(p, S, st);
            default: return run<PC<9, true, 4>>(p, S, st);
        }
    }
    switch (MB) {
        case 1: return run<PC<1, false, 3>>(p, S, st);
        case 2: return run<PC<2, false, 3>>(p, S, st);
        case 4: return run<PC<4, false, 3>>(p, S, st);
        case 8: return run<PC<8, false, 3>>(p, S, st);
        default: return run<PC<9, false, 3>>(p, S, st);
    }
}

}  // namespace gemm
}  // namespace fg
