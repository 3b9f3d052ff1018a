// Decode-shaped projection GEMM (M = bls rows, a few hundred at most):
// y = act(x W^T + bias) + residual with W in fp16 or in the group-wise 4-bit
// format, on a stream-K schedule.
//
// Why this shape of kernel (gfx950 measurements):
//  * MFMA issue from a single wavefront per SIMD reaches about half of the
//    matrix-core peak; two wavefronts per SIMD reach about 80%.  A workgroup
//    is 8 wavefronts: 4 columns of 64 weight rows (one 4-bit group each) times
//    2 k-halves.  The two wavefronts of a SIMD own the same outputs and the two
//    32-wide halves of every 64-wide k-step; their fp32 accumulators are added
//    through LDS at the end.  Every m row of the tile (up to 144) stays in the
//    tile, so each dequantized weight fragment feeds MB MFMAs.
//  * Dequantization runs on the fp32 VALU path: nibble -> v_cvt_f32_ubyte,
//    w = fma(q, scale, min) (the codec's multiply-then-add: q * scale is exact
//    in binary32, so the one rounding of the FMA equals the rounding of the
//    add), v_cvt_pk_f16_f32 into the MFMA operand.  Packed fp16 arithmetic
//    next to MFMA issue costs far more matrix-core throughput than these.
//  * Global -> LDS traffic uses direct-to-LDS loads (global_load_lds_dwordx4)
//    into an NS-deep ring of stage buffers [meta | X tile | weight tile], with
//    explicit s_waitcnt vmcnt + s_barrier publication and XOR swizzles.
//  * 4-bit k-steps: stages are published two ahead, so step i reads step
//    i+1's codes and (min, scale) row at its start and dequantizes step i+1's
//    four weight fragments in the MFMA shadows of its own rows; activation
//    fragments stream two rows ahead.  The step is a fixed sequence of
//    single-instruction volatile asm statements (each MFMA followed by 3-4
//    VALU instructions): the compiler's scheduler otherwise packed the MFMAs
//    together and ran the dequantization as one long VALU burst.
//  * Column pairs: lane-row i of column blocks 2p and 2p + 1 holds weight
//    columns 32p + 2i and 32p + 2i + 1, the two nibbles of one code byte, so
//    one 8-byte LDS read feeds two fragments; the (min, scale) values reach
//    every lane through row_newbcast DPP sources of the fp16 -> fp32
//    conversions, from one 2-byte read per lane.
//  * fp16 k-steps: stage i+1 is published at the end of step i and the next
//    step's fragments are read while the last MFMAs of step i issue.
//  * Stream-K: exactly G workgroups, each taking an equal contiguous share of
//    the (tile, k-step) iterations, so no tail of partly filled rounds.  A tile
//    covered by one workgroup is written with its epilogue; a tile shared by
//    several leaves fp32 partials in per-segment slots, summed in segment order
//    (deterministic) by sk_reduce_kernel.
#include <mutex>
#include <unordered_map>

#include <hip/hip_ext.h>

#include "fg_trace.h"
#include "gemm_common.h"
#include "rowops.h"

namespace fg {
namespace gemm {
namespace {

template <int MB_, bool Q4_, int NS_>
struct SK {
    static constexpr int MB = MB_, NS = NS_, WN = 4, NW = 8;
    static constexpr bool Q4 = Q4_;
    static constexpr int BM = MB * 16, BN = WN * 64, BK = 64, NT = NW * 64;
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
    // k-half merge: 8 regions (column x 2 fragments) of MB KB in the stage buffers
    static constexpr int PER_BUF = STAGE / (MB * 1024);
    static_assert(PER_BUF >= 1 && (8 + PER_BUF - 1) / PER_BUF <= NS, "merge space");
    static_assert(LWH * (NS - 1) <= 63, "vmcnt range");
};

// byte J of a dword as float (v_cvt_f32_ubyteJ)
template <int J>
__device__ __forceinline__ float ubf(uint32_t w) {
    return (float)((w >> (8 * J)) & 0xffu);
}

// Single instructions as volatile asm statements.  Volatile asm keeps its
// order relative to other volatile asm and to memory operations, so a k-step
// written as a sequence of them issues exactly in that order: each MFMA
// followed by the VALU work that fills its shadow.  The compiler's hazard
// tracking does not see inside asm, so callers keep the required distances:
// an s_nop before a DPP read or an MFMA operand read of a VGPR that a VALU
// instruction may have just written, and before any non-MFMA read of an MFMA
// result.
// An empty register constraint: the value is materialised in a VGPR as is
// and the compiler cannot derive anything from it.
template <class T>
__device__ __forceinline__ void pin(T& v) {
    asm("" : "+v"(v));
}

namespace op {
__device__ __forceinline__ void mfma(f4& c, const h8& a, const h8& b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void nop1() { asm volatile("s_nop 1"); }
__device__ __forceinline__ void nop_mfma_result() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }
// fp16 in the low half of lane J of each 16-lane row -> fp32 in every lane
template <int J>
__device__ __forceinline__ void bcast_f16(float& d, uint32_t v) {
    asm volatile("v_cvt_f32_f16_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf" : "=v"(d) : "v"(v), "i"(J));
}
__device__ __forceinline__ void lo_nibbles(uint32_t& d, uint32_t v) {
    asm volatile("v_and_b32 %0, 0xf0f0f0f, %1" : "=v"(d) : "v"(v));
}
__device__ __forceinline__ void shr4(uint32_t& d, uint32_t v) {
    asm volatile("v_lshrrev_b32 %0, 4, %1" : "=v"(d) : "v"(v));
}
template <int J>
__device__ __forceinline__ void ubyte(float& d, uint32_t v) {
    if constexpr (J == 0) asm volatile("v_cvt_f32_ubyte0 %0, %1" : "=v"(d) : "v"(v));
    if constexpr (J == 1) asm volatile("v_cvt_f32_ubyte1 %0, %1" : "=v"(d) : "v"(v));
    if constexpr (J == 2) asm volatile("v_cvt_f32_ubyte2 %0, %1" : "=v"(d) : "v"(v));
    if constexpr (J == 3) asm volatile("v_cvt_f32_ubyte3 %0, %1" : "=v"(d) : "v"(v));
}
__device__ __forceinline__ void fma(float& d, float a, float b, float c) {
    asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
}
// two fp32 -> packed fp16 pair, round to nearest even
__device__ __forceinline__ void pk(uint32_t& d, float a, float b) {
    asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
}
}  // namespace op

// VALU work of one 4-bit k-step, as a list of NOPS single instructions:
//  0..15: the (min, scale) row broadcasts, fp16 -> fp32 (min of k 0..7, then
//         scale of k 0..7);
//  then per column pair p and code dword hh (k 4hh..4hh+3), 23 instructions:
//         low / high nibbles of the dword (even / odd column of each byte),
//         4 + 4 conversions, 4 + 4 FMAs q * scale + min, 4 packs into the
//         fp16 fragments of column blocks 2p (even) and 2p + 1 (odd).
struct Dq {
    static constexpr int NOPS = 16 + 4 * 23;
    float mn[8], sc[8];
    uint32_t de, dd;
    float fe[4], fo[4];
};
template <int K>
__device__ __forceinline__ void dq_op(Dq& S, uint32_t mv, const uint2 (&cn)[2], uint32_t (&wn)[4][4]) {
    if constexpr (K < 8) {
        if constexpr (K == 0) op::nop1();   // DPP source: no VALU write just before
        op::bcast_f16<K>(S.mn[K], mv);
    } else if constexpr (K < 16) {
        op::bcast_f16<K>(S.sc[K - 8], mv);
    } else {
        constexpr int c = (K - 16) / 23, o = (K - 16) % 23, pp = c >> 1, hh = c & 1;
        const uint32_t cw = hh ? cn[pp].y : cn[pp].x;
        if constexpr (o == 0) op::lo_nibbles(S.de, cw);
        else if constexpr (o == 1) op::shr4(S.dd, cw);
        else if constexpr (o == 2) op::lo_nibbles(S.dd, S.dd);
        else if constexpr (o < 7) op::ubyte<o - 3>(S.fe[o - 3], S.de);
        else if constexpr (o < 11) op::fma(S.fe[o - 7], S.fe[o - 7], S.sc[4 * hh + o - 7], S.mn[4 * hh + o - 7]);
        else if constexpr (o < 15) op::ubyte<o - 11>(S.fo[o - 11], S.dd);
        else if constexpr (o < 19) op::fma(S.fo[o - 15], S.fo[o - 15], S.sc[4 * hh + o - 15], S.mn[4 * hh + o - 15]);
        else if constexpr (o == 19) op::pk(wn[2 * pp][2 * hh], S.fe[0], S.fe[1]);
        else if constexpr (o == 20) op::pk(wn[2 * pp][2 * hh + 1], S.fe[2], S.fe[3]);
        else if constexpr (o == 21) op::pk(wn[2 * pp + 1][2 * hh], S.fo[0], S.fo[1]);
        else op::pk(wn[2 * pp + 1][2 * hh + 1], S.fo[2], S.fo[3]);
    }
}
template <int K, int E>
__device__ __forceinline__ void dq_ops(Dq& S, uint32_t mv, const uint2 (&cn)[2], uint32_t (&wn)[4][4]) {
    if constexpr (K < E) {
        dq_op<K>(S, mv, cn, wn);
        dq_ops<K + 1, E>(S, mv, cn, wn);
    }
}

// One 4-bit k-step: MB rows of 4 MFMAs (one activation fragment, the 4
// weight fragments of this step).  The VALU list of the next step's
// fragments fills the MFMA shadows of rows 1..MB-1 evenly (row 0 waits for
// the codes just requested); activation fragments are read PD rows ahead.
template <int MB, int PD, int ROW, class RX, class RXN>
__device__ __forceinline__ void q4_rows(f4 (&acc)[4][MB], const uint32_t (&w)[4][4], h8 (&xq)[MB], h8 (&xn)[PD],
                                        Dq& S, uint32_t mv, const uint2 (&cn)[2], uint32_t (&wn)[4][4],
                                        const RX& read_cur, const RXN& read_nxt) {
    if constexpr (ROW < MB) {
        constexpr int NSLOT = MB > 1 ? 4 * (MB - 1) : 4;
        if constexpr (ROW + PD < MB) xq[ROW + PD] = read_cur(ROW + PD);
        else xn[ROW + PD - MB] = read_nxt(ROW + PD - MB);
        auto slot = [&](auto nbc) {
            constexpr int nb = decltype(nbc)::value;
            op::mfma(acc[nb][ROW], __builtin_bit_cast(h8, make_uint4(w[nb][0], w[nb][1], w[nb][2], w[nb][3])), xq[ROW]);
            if constexpr (MB == 1 || ROW > 0) {
                constexpr int sidx = (MB > 1 ? (ROW - 1) * 4 : 0) + nb;
                dq_ops<sidx * Dq::NOPS / NSLOT, (sidx + 1) * Dq::NOPS / NSLOT>(S, mv, cn, wn);
            }
        };
        slot(std::integral_constant<int, 0>{});
        slot(std::integral_constant<int, 1>{});
        slot(std::integral_constant<int, 2>{});
        slot(std::integral_constant<int, 3>{});
        q4_rows<MB, PD, ROW + 1>(acc, w, xq, xn, S, mv, cn, wn, read_cur, read_nxt);
    }
}

template <class C>
__global__ __launch_bounds__(C::NT) void sk_kernel(Params p, SkSched sc) {
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
    const int r16 = lane & 15, q = lane >> 4;
    const uint32_t shn = (uint32_t)(r16 & 1) * 4u;   // nibble of this lane's weight row
    const int64_t g = blockIdx.x;
    const int64_t it_beg = sc.dp ? 0 : sc.bnd[g], it_end = sc.dp ? 0 : sc.bnd[g + 1];

    int64_t it = it_beg, next_tile = g;
    for (;;) {
        int64_t tile;
        int kb, ke;
        if (sc.dp) {   // whole tiles g, g + G, ...
            tile = next_tile;
            if (tile >= sc.tiles) break;
            next_tile += sc.G;
            kb = 0;
            ke = (int)sc.nk;
        } else {       // stream-K: this workgroup's share of the iterations
            if (it >= it_end) break;
            tile = it / sc.nk;
            kb = (int)(it - tile * sc.nk);
            ke = (int)(min(it_end, (tile + 1) * sc.nk) - tile * sc.nk);
            it = tile * sc.nk + ke;
        }
        int64_t tm, tn;
        sk_tile_coords(sc, tile, tm, tn);
        const int64_t n0 = tn * C::BN, m0 = tm * C::BM;
        const int nk = ke - kb;
        const int64_t kbeg = (int64_t)kb * C::BK;

        f4 acc[4][C::MB];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < C::MB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

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

        auto read_x = [&](const unsigned char* base, int mb) -> h8 {
            const int row = mb * 16 + r16;
            const int kc = (kh * 4 + q) ^ (row & 7);
            return *reinterpret_cast<const h8*>(base + C::M_BYTES + (row * 8 + kc) * 16);
        };
        // fp16 weight fragment of column block nb: lane-row i holds column
        // wc*64 + 16nb + i
        auto read_w16 = [&](const unsigned char* base, int nb) -> h8 {
            const int nl = wc * 64 + nb * 16 + r16;
            const int kc = (kh * 4 + q) ^ (nl & 7);
            return *reinterpret_cast<const h8*>(base + C::X_BYTES + (nl * 8 + kc) * 16);
        };
        // activation fragment rows: row mb*16 + r16 (chunk swizzle by r16 & 7)
        const uint32_t xoff = (uint32_t)(C::M_BYTES + (r16 * 8 + ((kh * 4 + q) ^ (r16 & 7))) * 16);
        // (min, scale) of this lane's 8 k: lane t of each 16-lane row reads one
        // fp16 value (t < 8: min of k0 + t, else scale of k0 + t - 8); the row
        // broadcasts of the dequantization list spread them to every lane
        const uint32_t moff = (uint32_t)((wc * 2 + (r16 >> 3)) * 128 + (kh * 32 + q * 8 + (r16 & 7)) * 2);
        auto load_meta = [&](const unsigned char* base) -> uint32_t {
            return *reinterpret_cast<const unsigned short*>(base + moff);
        };
        // 4-bit codes of column pair pp: lane-row i of column blocks 2pp / 2pp+1
        // holds weight columns wc*64 + 32pp + 2i / 2i+1, the two nibbles of
        // one code byte, so one 8-byte read (8 k) feeds both fragments
        const int cch = (kh * 2 + (q >> 1)) ^ ((r16 >> 1) & 3);
        const uint32_t coff = (uint32_t)(C::M_BYTES + C::X_BYTES + (wc * 32 + r16) * 64 + cch * 16 + (q & 1) * 8);
        auto read_cp = [&](const unsigned char* base, int pp) -> uint2 {
            return *reinterpret_cast<const uint2*>(base + coff + pp * 1024);
        };

        if constexpr (C::Q4) {
            // 4-bit weights.  Stages are published two ahead: at the barrier
            // that ends step i every stage up to i + 2 has landed.  Step i
            // reads step i+1's codes and metadata first and dequantizes its
            // four weight fragments in the MFMA shadows of its own rows; the
            // two fragment sets alternate between wa and wb (the loop runs two
            // turns of the stage ring per iteration), so nothing is copied.
            constexpr int PD = C::MB < 2 ? C::MB : 2;
            static_assert(C::NS >= 3, "stages published two ahead");
            Dq S;
            uint32_t wa[4][4], wb[4][4];
            h8 xc[PD];
            // stages 0 and 1 first (step 0 computes on 0 and dequantizes 1):
            // every workgroup of a launch fills its pipeline at once, and
            // requesting the later stages only after these have landed lets
            // the first MFMAs start sooner; the loop's waits are unchanged
            // (the stages are still issued in order)
            issue(buf(0), 0);
            issue(buf(1), 1);
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int st = 2; st < C::NS; ++st) issue(buf(st), st);
            {
                const unsigned char* b0 = buf(0);
                const uint2 c0[2] = {read_cp(b0, 0), read_cp(b0, 1)};
                dq_ops<0, Dq::NOPS>(S, load_meta(b0), c0, wa);
#pragma unroll
                for (int j = 0; j < PD; ++j) xc[j] = read_x(b0, j);
            }
            auto q4_step = [&](int st, int i, uint32_t(&w)[4][4], uint32_t(&wn)[4][4]) {
                const unsigned char* cur = buf(st);
                const unsigned char* nxt = buf((st + 1) % C::NS);
                const uint2 cn[2] = {read_cp(nxt, 0), read_cp(nxt, 1)};
                const uint32_t mv = load_meta(nxt);
                h8 xq[C::MB], xn[PD];
#pragma unroll
                for (int j = 0; j < PD; ++j) xq[j] = xc[j];
                // activation fragment of row mb at xo + 2 KB * mb (the lane
                // offset is pinned per step so that the row offsets stay
                // immediates instead of nine hoisted registers)
                uint32_t xo = xoff;
                pin(xo);
                op::nop1();   // MFMA operands: no VALU write just before
                q4_rows<C::MB, PD, 0>(acc, w, xq, xn, S, mv, cn, wn,
                                      [&](int mb) { return *reinterpret_cast<const h8*>(cur + xo + mb * 2048); },
                                      [&](int j) { return *reinterpret_cast<const h8*>(nxt + xo + j * 2048); });
#pragma unroll
                for (int j = 0; j < PD; ++j) xc[j] = xn[j];
                // stages up to i+2 have landed for every wave (the wait is the
                // one of the waves with fewer loads: stronger for the others)
                // and no wave still reads stage i: refill its buffer with
                // stage i+NS
                __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::LWL * (C::NS - 3)));
                __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
                __builtin_amdgcn_s_barrier();
                issue(buf(st), i + C::NS);
            };
            for (int kt = 0; kt < nk; kt += 2 * C::NS) {
#pragma unroll
                for (int u = 0; u < 2 * C::NS; ++u) {
                    const int i = kt + u;
                    if (i < nk) {
                        if (u & 1) q4_step(u % C::NS, i, wb, wa);
                        else q4_step(u % C::NS, i, wa, wb);
                    }
                }
            }
            op::nop_mfma_result();
        } else {
            // fp16 weights: stage i+1 is published at the end of step i; the
            // next step's fragments are read during its last column block
            h8 xf[C::MB];
            h8 wf16[4];
            h8 wcur;
#pragma unroll
            for (int st = 0; st < C::NS; ++st) issue(buf(st), st);
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::LWL * (C::NS - 1)));
            __builtin_amdgcn_s_barrier();
            {
                const unsigned char* b0 = buf(0);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) wf16[nb] = read_w16(b0, nb);
                wcur = wf16[0];
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb) xf[mb] = read_x(b0, mb);
            }
            for (int kt = 0; kt < nk; kt += C::NS) {
#pragma unroll
                for (int st = 0; st < C::NS; ++st) {
                    const int i = kt + st;
                    if (i < nk) {
                        const unsigned char* nxt = buf((st + 1) % C::NS);
#pragma unroll
                        for (int nb = 0; nb < 3; ++nb) {
                            const h8 wnext = wf16[nb + 1];
#pragma unroll
                            for (int mb = 0; mb < C::MB; ++mb)
                                acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wcur, xf[mb], acc[nb][mb], 0, 0, 0);
                            wcur = wnext;
                        }
                        // stage i+1 has landed for every wave and no wave still
                        // reads stage i: refill its buffer with stage i+NS
                        __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::LWL * (C::NS - 2)));
                        __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
                        __builtin_amdgcn_s_barrier();
                        issue(buf(st), i + C::NS);
#pragma unroll
                        for (int nb = 0; nb < 3; ++nb) wf16[nb] = read_w16(nxt, nb);
                        const h8 w0n = wf16[0];
                        // each activation fragment is replaced by the next
                        // step's right after its last use
#pragma unroll
                        for (int mb = 0; mb < C::MB; ++mb) {
                            acc[3][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wcur, xf[mb], acc[3][mb], 0, 0, 0);
                            xf[mb] = read_x(nxt, mb);
                        }
                        wf16[3] = read_w16(nxt, 3);
                        wcur = w0n;
                    }
                }
            }
        }
        // no load may still be writing LDS when the buffers are reused
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
        __builtin_amdgcn_s_barrier();

        // add the two k-halves (kh = 1 -> LDS -> kh = 0), two fragments per round
        // the whole tile in this segment: final outputs; else its partial slot
        const bool full = sc.dp || (kb == 0 && ke == (int)sc.nk);
        const int slot = (sc.dp || kb == 0) ? 0 : (int)sc.slot0[g];
        // the workgroup that ends a tile records how many segments it has
        if (p.tile_ns && ke == (int)sc.nk && tid == 0) p.tile_ns[tile] = slot + 1;
        const int nq = q * 4;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wc * 2 + j;
                float4* reg = reinterpret_cast<float4*>(buf(r / C::PER_BUF) + (r % C::PER_BUF) * C::MB * 1024);
                const int nb = rd * 2 + j;
                if (kh == 1) {
#pragma unroll
                    for (int mb = 0; mb < C::MB; ++mb)
                        reg[mb * 64 + lane] = make_float4(acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]);
                }
            }
            __syncthreads();
            if (C::Q4 && kh == 0) {
                // column pair rd: acc[2rd + h][mb][t] is column 8q + 2t + h of
                // the pair's 32, so a lane holds 8 consecutive columns
                const float4* reg0 = reinterpret_cast<const float4*>(buf((wc * 2) / C::PER_BUF) + ((wc * 2) % C::PER_BUF) * C::MB * 1024);
                const float4* reg1 = reinterpret_cast<const float4*>(buf((wc * 2 + 1) / C::PER_BUF) + ((wc * 2 + 1) % C::PER_BUF) * C::MB * 1024);
                const int64_t n = n0 + wc * 64 + rd * 32 + q * 8;
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb) {
                    const float4 o0 = reg0[mb * 64 + lane], o1 = reg1[mb * 64 + lane];
                    const f4 a0 = acc[rd * 2][mb], a1 = acc[rd * 2 + 1][mb];
                    float v[8] = {a0[0] + o0.x, a1[0] + o1.x, a0[1] + o0.y, a1[1] + o1.y,
                                  a0[2] + o0.z, a1[2] + o1.z, a0[3] + o0.w, a1[3] + o1.w};
                    const int64_t m = m0 + mb * 16 + r16;
                    if (m < p.M && n < p.N) {
                        if (full) {
                            store8_final(p, m, n, v);
                        } else {
                            float* dst = p.part + ((int64_t)slot * p.M + m) * p.N + n;
                            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                            *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
                        }
                    }
                }
            }
            if (!C::Q4 && kh == 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int r = wc * 2 + j;
                    const float4* reg = reinterpret_cast<const float4*>(buf(r / C::PER_BUF) + (r % C::PER_BUF) * C::MB * 1024);
                    const int nb = rd * 2 + j;
                    const int64_t n = n0 + wc * 64 + nb * 16 + nq;
#pragma unroll
                    for (int mb = 0; mb < C::MB; ++mb) {
                        const float4 o = reg[mb * 64 + lane];
                        f4 v = acc[nb][mb];
                        v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
                        const int64_t m = m0 + mb * 16 + r16;
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

// Sum the per-segment partials of shared tiles in segment order, then bias /
// ReLU / residual.  Tiles written whole by one workgroup are skipped.
// Generic form (64-bit indices): any shape.
__global__ __launch_bounds__(256) void sk_reduce64_kernel(Params p, SkSched sc) {
    const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;   // element (m, n..n+3)
    if (idx >= p.M * p.N) return;
    const int64_t m = idx / p.N, n = idx % p.N;
    const int64_t tile = (m / sc.bm) * sc.ntn + n / sc.bn;
    const int ns = p.tile_ns[tile];
    if (ns == 1) return;                 // whole tile written by one workgroup
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t s = 0; s < ns; ++s) {
        const float4 v = *reinterpret_cast<const float4*>(p.part + (s * p.M + m) * p.N + n);
        o[0] += v.x; o[1] += v.y; o[2] += v.z; o[3] += v.w;
    }
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
    *reinterpret_cast<uint2*>(p.y + m * p.ldy + n) = make_uint2(pack_h2(o[0], o[1]), pack_h2(o[2], o[3]));
}

// acc += the ns >= 1 slots at pr, pr + MN, ... in slot order, in two steps:
// slot_load issues the first SMAX loads together (clamped addresses, so they
// are always valid), slot_add adds them, slots past the first through a
// select.  A load whose use sits under `if (q < ns)` is sunk into that branch
// by the compiler, which then waits for each slot's round trip to memory
// before requesting the next.
template <int SMAX>
__device__ __forceinline__ void slot_load(f4 (&o)[SMAX], const float* pr, int64_t MN, int ns) {
#pragma unroll
    for (int q = 0; q < SMAX; ++q) o[q] = *reinterpret_cast<const f4*>(pr + min(q, ns - 1) * MN);
}
template <int SMAX>
__device__ __forceinline__ void slot_add(f4& acc, const f4 (&o)[SMAX], const float* pr, int64_t MN, int ns) {
    acc += o[0];
#pragma unroll
    for (int q = 1; q < SMAX; ++q) {
        const f4 t = acc + o[q];
        acc = q < ns ? t : acc;
    }
    // only the widest instantiation serves schedules with more slots (a loop
    // here splits the caller into blocks the scheduler does not cross)
    if constexpr (SMAX >= 8)
        for (int q = SMAX; q < ns; ++q) acc += *reinterpret_cast<const f4*>(pr + q * MN);
}
template <int SMAX>
__device__ __forceinline__ void slot_sum(f4& acc, const float* pr, int64_t MN, int ns) {
    f4 o[SMAX];
    slot_load<SMAX>(o, pr, MN, ns);
    slot_add<SMAX>(acc, o, pr, MN, ns);
}

// Epilogue of 4 summed columns without branches: + bias, ReLU, + residual
// (each applied through a select when present; the same operations in the
// same order as the GEMM's own epilogue).
__device__ __forceinline__ void epi4(f4& acc, uint2 bb, uint2 rr, bool has_b, bool relu, bool has_r) {
    const float b4[4] = {h2f(bb.x), h2f(bb.x >> 16), h2f(bb.y), h2f(bb.y >> 16)};
    const float r4[4] = {h2f(rr.x), h2f(rr.x >> 16), h2f(rr.y), h2f(rr.y >> 16)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float v = acc[j];
        v = has_b ? v + b4[j] : v;
        v = relu ? fmaxf(v, 0.f) : v;
        v = has_r ? v + r4[j] : v;
        acc[j] = v;
    }
}

// Decode shapes (the host checks that the schedule fits 32-bit arithmetic):
// one workgroup per (row, 1024 columns), so no index division per element;
// a wavefront's 256 columns are one tile, whose segment count is a scalar
// load (the scalar cache serves it, instead of a vector round trip before
// the slot loads can be addressed); the slot loads unrolled up to SMAX with
// clamped addresses, all in flight at once.
template <int SMAX>
__global__ __launch_bounds__(256) void sk_reduce_kernel(Params p, SkSched sc) {
    const int m = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const uint32_t tile = (uint32_t)(m / (int)sc.bm) * (uint32_t)sc.ntn + (uint32_t)(blockIdx.x * 4 + wave);
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= p.N) return;
    const int ns = p.tile_ns[tile];
    if (ns == 1) return;                 // whole tile written by one workgroup
    const int64_t MN = p.M * p.N;
    const float* pr = p.part + (int64_t)m * p.N + n;
    // bias and residual requested with the slots (from a valid stand-in
    // address when absent, the value then unused), so that no branch sinks
    // their loads behind the sum
    const uint2 bb = *reinterpret_cast<const uint2*>(p.bias ? p.bias + n : p.y + (int64_t)m * p.ldy + n);
    const uint2 rr = *reinterpret_cast<const uint2*>(p.residual ? p.residual + (int64_t)m * p.ldy + n
                                                                : p.y + (int64_t)m * p.ldy + n);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    slot_sum<SMAX>(acc, pr, MN, ns);
    epi4(acc, bb, rr, p.bias != nullptr, p.act == 1, p.residual != nullptr);
    *reinterpret_cast<uint2*>(p.y + (int64_t)m * p.ldy + n) =
        make_uint2(pack_h2(acc[0], acc[1]), pack_h2(acc[2], acc[3]));
}

// The same sum for whole rows, fused with the LayerNorm of the finished
// fp16 row (the next sublayer's input).  One 1024-thread workgroup per row,
// 4 columns per thread and unit; every partial of a row is requested before
// any is used (the slot loads are unrolled up to SMAX with clamped addresses),
// and tiles written whole by one workgroup are read back from y.
constexpr int kLnTiles = 128;   // column tiles of a row: h <= 32768
constexpr int kLnThreads = 1024;

template <int MAXU, int SMAX>
__global__ __launch_bounds__(kLnThreads) void sk_reduce_ln_kernel(Params p, SkSched sc,
                                                                 const __half* __restrict__ g,
                                                                 const __half* __restrict__ b,
                                                                 __half* __restrict__ ln_y) {
    constexpr int NT = kLnThreads;
    __shared__ float sh[NT / 64];
    const int64_t m = blockIdx.x;
    const int64_t tm = m / sc.bm;
    const int nu = (int)(p.N / 4);
    // unit i of a wavefront is the 256-column tile wave + 16 i (or, past the
    // row's end, the last one, which the clamped units read): its segment
    // count is one scalar load
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int* nsp = p.tile_ns + tm * sc.ntn;
    int nsw[MAXU];
#pragma unroll
    for (int i = 0; i < MAXU; ++i) nsw[i] = nsp[min(wave + (NT / 64) * i, (nu - 1) >> 6)];
    const int64_t MN = p.M * p.N;
    __half* yr = p.y + m * p.ldy;
    const __half* rr = p.residual ? p.residual + m * p.ldy : nullptr;
    const float* pr = p.part + m * p.N;
    float v[MAXU][4];
    uint2 wr[MAXU];   // summed fp16 outputs, stored after the loads of every
                      // unit (no store between two units' loads)
    // LayerNorm gamma and beta, requested with the first loads where the
    // registers allow (up to 4 units per thread), else at the end
    constexpr bool early_gb = MAXU <= 4;
    uint2 gg[MAXU], be[MAXU];
    float s = 0.f;
    // units in groups of UG: every load of a group (its slots, the residual
    // or the finished y, the bias) is requested before any of them is used,
    // without branches (stand-in addresses in the row when one is absent)
    constexpr int UG = (24 / (SMAX + 2)) < 1 ? 1 : ((24 / (SMAX + 2)) > MAXU ? MAXU : 24 / (SMAX + 2));
#pragma unroll
    for (int i0 = 0; i0 < MAXU; i0 += UG) {
        f4 o[UG][SMAX];
        uint2 h16[UG], bb[UG];
        int nsu[UG];
#pragma unroll
        for (int j = 0; j < UG; ++j) {
            const int i = i0 + j;
            if (i < MAXU) {
                const int u = min((int)threadIdx.x + i * NT, nu - 1);   // clamped: loads stay in the row
                const int64_t n = (int64_t)u * 4;
                const int ns = nsw[i];
                nsu[j] = ns;
                slot_load<SMAX>(o[j], pr + n, MN, ns);
                // whole tile: y is final; shared tile: partials + bias /
                // ReLU / residual
                h16[j] = *reinterpret_cast<const uint2*>(ns == 1 || !rr ? yr + n : rr + n);
                bb[j] = *reinterpret_cast<const uint2*>(p.bias ? p.bias + n : yr + n);
                if constexpr (early_gb) {
                    gg[i] = *reinterpret_cast<const uint2*>(g + n);
                    be[i] = *reinterpret_cast<const uint2*>(b + n);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < UG; ++j) {
            const int i = i0 + j;
            if (i < MAXU) {
                const int u = min((int)threadIdx.x + i * NT, nu - 1);
                const int ns = nsu[j];
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                slot_add<SMAX>(acc, o[j], pr + (int64_t)u * 4, MN, ns);
                epi4(acc, bb[j], h16[j], p.bias != nullptr, p.act == 1, rr != nullptr);
                const uint2 w = ns == 1 ? h16[j] : make_uint2(pack_h2(acc[0], acc[1]), pack_h2(acc[2], acc[3]));
                const bool mine = (int)threadIdx.x + i * NT < nu;
                wr[i] = w;
                // the LayerNorm sees the row as stored (fp16)
                v[i][0] = h2f(w.x); v[i][1] = h2f(w.x >> 16); v[i][2] = h2f(w.y); v[i][3] = h2f(w.y >> 16);
                if (mine) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = (int)threadIdx.x + i * NT;
        if (u < nu && nsw[i] > 1) *reinterpret_cast<uint2*>(yr + (int64_t)u * 4) = wr[i];
    }
    const float mean = row::block_sum<NT>(s, sh) / (float)p.N;
    float qs = 0.f;
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        if ((int)threadIdx.x + i * NT < nu) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float d = v[i][j] - mean;
                qs += d * d;
            }
        }
    }
    const float var = row::block_sum<NT>(qs, sh) / (float)p.N;
    const float rstd = 1.0f / sqrtf(var + 1e-5f);
    __half* out = ln_y + m * p.N;
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = (int)threadIdx.x + i * NT;
        if (u < nu) {
            if constexpr (!early_gb) {
                gg[i] = *reinterpret_cast<const uint2*>(g + u * 4);
                be[i] = *reinterpret_cast<const uint2*>(b + u * 4);
            }
            const float gv[4] = {h2f(gg[i].x), h2f(gg[i].x >> 16), h2f(gg[i].y), h2f(gg[i].y >> 16)};
            const float bv[4] = {h2f(be[i].x), h2f(be[i].x >> 16), h2f(be[i].y), h2f(be[i].y >> 16)};
            *reinterpret_cast<uint2*>(out + u * 4) =
                make_uint2(pack_h2((v[i][0] - mean) * rstd * gv[0] + bv[0], (v[i][1] - mean) * rstd * gv[1] + bv[1]),
                           pack_h2((v[i][2] - mean) * rstd * gv[2] + bv[2], (v[i][3] - mean) * rstd * gv[3] + bv[3]));
        }
    }
}

template <class C>
int run(const Params& p, const SkSched& sc, hipStream_t st) {
    hipEvent_t ea, eb;   // the enclosing trace scope's events, if any
    trace_take_ext(&ea, &eb);
    hipExtLaunchKernelGGL(sk_kernel<C>, dim3((unsigned)sc.G), dim3(C::NT), 0, st, ea, eb, 0u, p, sc);
    FG_LAUNCHED("sk_kernel");
    return FG_OK;
}

}  // namespace

// Tile rows.  Up to 64 rows: one tile of 16-row blocks (16x16x32 kernel
// here).  Beyond, the candidates are 128- or 144-row tiles of this kernel and
// 96-, 128- or 160-row tiles of the 32x32x16 kernel (gemm_sk32.hip): the
// fewest tiles along M (each one streams the weights once), then the least
// padding, then this kernel.  Measured on gfx950 at equal padding the two
// kernels run within 1-2% of each other (the 32x32x16 one issues far less
// VALU per flop but the clock drops accordingly), so the fit decides.
int64_t sk_rows_for(int64_t M, int32_t& wide) {
    wide = 0;
    if (M <= 64) return M <= 16 ? 16 : (M <= 32 ? 32 : 64);
    struct Cand { int64_t bm; int32_t wide; };
    const Cand cands[] = {{128, 0}, {144, 0}, {96, 1}, {128, 1}, {160, 1}};
    Cand best = cands[0];
    for (const Cand& c : cands) {
        const int64_t t = cdiv(M, c.bm), tb = cdiv(M, best.bm);
        if (t < tb || (t == tb && t * c.bm < tb * best.bm)) best = c;
    }
    wide = best.wide;
    return best.bm;
}

namespace {

// Fills bnd[0..G] so that every workgroup's estimated time, its k-steps plus
// R k-steps per segment (tile) it touches, is at most tau; false if the T
// iterations do not fit in G workgroups that way.
bool sk_fill(SkSched& sc, double tau, double R) {
    int64_t x = 0;
    sc.bnd[0] = 0;
    for (int64_t g = 0; g < sc.G; ++g) {
        double budget = tau;
        const int64_t start = x;
        while (x < sc.T) {
            const int64_t tile_end = (x / sc.nk + 1) * sc.nk;
            const double avail = budget - R;   // entering a segment
            if (avail < 1.0) break;
            const int64_t take = std::min<int64_t>(tile_end - x, (int64_t)avail);
            x += take;
            budget = avail - (double)take;
            if (x < tile_end) break;           // budget spent inside the tile
        }
        if (x == start && x < sc.T && budget == tau) return false;   // not even one k-step fits
        sc.bnd[g + 1] = (int32_t)x;
    }
    return x >= sc.T;
}

// Time-balanced stream-K ranges: the least tau (bisection) for which the
// greedy fill covers every iteration.  R, the fixed cost of a segment in
// k-steps, was measured on gfx950 for 144-row tiles of 4-bit weights (about
// 13 us of pipeline fill, k-half merge and stores against about 1 us per
// k-step); tiles of fewer rows have cheaper k-steps, so R grows as 144 / bm.
void sk_balance(SkSched& sc) {
    const double R = std::min(48.0, 12.0 * 144.0 / (double)sc.bm);
    double lo = (double)sc.T / (double)sc.G, hi = (double)sc.T / (double)sc.G + 4.0 * R + (double)sc.nk;
    while (!sk_fill(sc, hi, R)) hi *= 2.0;
    for (int i = 0; i < 40 && hi - lo > 0.25; ++i) {
        const double mid = 0.5 * (lo + hi);
        if (sk_fill(sc, mid, R)) hi = mid;
        else lo = mid;
    }
    sk_fill(sc, hi, R);
    // most segments any tile is cut into (1: every workgroup covers whole tiles)
    sc.slots = 1;
    for (int64_t t = 0; t < sc.tiles; ++t)
        sc.slots = std::max<int64_t>(sc.slots, sk_owner(sc, (t + 1) * sc.nk - 1) - sk_owner(sc, t * sc.nk) + 1);
    for (int64_t g = 0; g < sc.G; ++g) {
        const int64_t b = sc.bnd[g];
        sc.slot0[g] = (b >= sc.T || b % sc.nk == 0) ? 0 : (int16_t)(g - sk_owner(sc, b - b % sc.nk));
    }
}

struct SkKey {
    int64_t M, N, K;
    bool operator==(const SkKey& o) const { return M == o.M && N == o.N && K == o.K; }
};
struct SkKeyHash {
    size_t operator()(const SkKey& k) const {
        return std::hash<int64_t>()(k.M * 1000003 + k.N * 10007 + k.K);
    }
};

}  // namespace

SkSched sk_schedule(int64_t M, int64_t N, int64_t K) {
    SkSched sc{};
    sc.bn = 256;
    sc.ntn = cdiv(N, sc.bn);
    sc.nk = K / 64;
    if (M > kSkDpRows) {
        // many tiles per workgroup: data-parallel whole tiles, no partials;
        // 128- or 144-row tiles, whichever pads M less
        sc.dp = 1;
        sc.bm = cdiv(M, 144) * 144 <= cdiv(M, 128) * 128 ? 144 : 128;
        sc.mt = cdiv(M, sc.bm);
        sc.tiles = sc.mt * sc.ntn;
        sc.T = sc.tiles * sc.nk;
        sc.G = std::min<int64_t>(kSkGroups, sc.tiles);
        sc.band = 16;
        sc.slots = 1;
        return sc;
    }
    // the balanced ranges are a pure function of the shape: computed once
    static std::mutex mu;
    static std::unordered_map<SkKey, SkSched, SkKeyHash> cache;
    const SkKey key{M, N, K};
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    sc.bm = sk_rows_for(M, sc.wide);
    sc.mt = cdiv(M, sc.bm);
    sc.tiles = sc.mt * sc.ntn;
    sc.T = sc.tiles * sc.nk;
    // one workgroup per CU of the 256-CU part (a constant, so the schedule and
    // its workspace depend on the shape only), at least 4 k-steps each
    sc.G = std::max<int64_t>(1, std::min<int64_t>(kSkGroups, sc.T / 4));
    if (sc.T >= (1ll << 31)) return sc;   // refused by the caller (ranges are 32-bit)
    sk_balance(sc);
    std::lock_guard<std::mutex> lk(mu);
    cache.emplace(key, sc);
    return sc;
}

int launch_sk(const Params& p, const SkSched& sc, bool q4, hipStream_t st) {
    if (sc.wide) return launch_sk32(p, sc, q4, st);
    const int MB = (int)(sc.bm / 16);
    if (q4) {
        switch (MB) {
            case 1: return run<SK<1, true, 5>>(p, sc, st);
            case 2: return run<SK<2, true, 5>>(p, sc, st);
            case 4: return run<SK<4, true, 5>>(p, sc, st);
            case 8: return run<SK<8, true, 5>>(p, sc, st);
            default: return run<SK<9, true, 5>>(p, sc, st);
        }
    }
    switch (MB) {
        case 1: return run<SK<1, false, 3>>(p, sc, st);
        case 2: return run<SK<2, false, 3>>(p, sc, st);
        case 4: return run<SK<4, false, 3>>(p, sc, st);
        case 8: return run<SK<8, false, 3>>(p, sc, st);
        default: return run<SK<9, false, 3>>(p, sc, st);
    }
}

int launch_sk_reduce(const Params& p, const SkSched& sc, hipStream_t st) {
    const bool fits32 = sc.bn == 256 && p.M <= 65535 && p.N % 4 == 0 && sc.T < (1ll << 31);
    if (!fits32) {
        const int64_t n4 = p.M * p.N / 4;
        sk_reduce64_kernel<<<(unsigned)cdiv(n4, 256), 256, 0, st>>>(p, sc);
        FG_LAUNCHED("sk_reduce64_kernel");
        return FG_OK;
    }
    const dim3 grid((unsigned)cdiv(p.N, 1024), (unsigned)p.M);
    if (sc.slots <= 2) sk_reduce_kernel<2><<<grid, 256, 0, st>>>(p, sc);
    else if (sc.slots <= 3) sk_reduce_kernel<3><<<grid, 256, 0, st>>>(p, sc);
    else if (sc.slots <= 4) sk_reduce_kernel<4><<<grid, 256, 0, st>>>(p, sc);
    else if (sc.slots <= 6) sk_reduce_kernel<6><<<grid, 256, 0, st>>>(p, sc);
    else sk_reduce_kernel<8><<<grid, 256, 0, st>>>(p, sc);
    FG_LAUNCHED("sk_reduce_kernel");
    return FG_OK;
}

int launch_sk_reduce_ln(const Params& p, const SkSched& sc, const __half* g, const __half* b,
                        __half* ln_y, hipStream_t st) {
    const int64_t nu = p.N / 4;
    if (p.N % 8 != 0 || p.ldy != p.N || sc.bn != 256 || sc.ntn > kLnTiles || nu > kLnThreads * 8)
        return set_error(FG_ERR_UNSUPPORTED, "fused reduce + layernorm: width %lld", (long long)p.N);
    const unsigned rows = (unsigned)p.M;
    const int64_t need = cdiv(nu, (int64_t)kLnThreads);   // units per thread
    const int mu = need <= 4 ? (int)need : (need <= 6 ? 6 : 8);
    const int sm = sc.slots <= 2 ? 2 : (sc.slots <= 4 ? 4 : (sc.slots <= 6 ? 6 : 8));
#define FG_RLN(U, S) sk_reduce_ln_kernel<U, S><<<rows, kLnThreads, 0, st>>>(p, sc, g, b, ln_y)
#define FG_RLN_S(U) (sm == 2 ? FG_RLN(U, 2) : (sm == 4 ? FG_RLN(U, 4) : (sm == 6 ? FG_RLN(U, 6) : FG_RLN(U, 8))))
    switch (mu) {
        case 1: FG_RLN_S(1); break;
        case 2: FG_RLN_S(2); break;
        case 3: FG_RLN_S(3); break;
        case 4: FG_RLN_S(4); break;
        case 6: FG_RLN_S(6); break;
        default: FG_RLN_S(8); break;
    }
#undef FG_RLN_S
#undef FG_RLN
    FG_LAUNCHED("sk_reduce_ln_kernel");
    return FG_OK;
}

}  // namespace gemm
}  // namespace fg
