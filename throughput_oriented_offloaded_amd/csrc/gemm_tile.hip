// Large-M projection GEMM (the prefill, M = gbs * s rows): y = act(x W^T +
// bias) + residual with fp16 activations and fp16 weights (4-bit matrices are
// restored to fp16 once per layer before the prefill's contractions).
//
// The prefill runs every decoder layer over all s positions of each GPU batch
// ("FlexGen 完全拆解", section "FlexGen 的核心:计算图分块与张量生命周期"), so
// these contractions are dense and compute-bound; the pages restore
// compressed weights to fp16 before compute (section "权重压缩与 KV Cache
// 压缩").
//
// Shape of the kernel (gfx950):
//  * 256 x 256 output tiles, 8 wavefronts (two per SIMD), each owning 128
//    rows x 64 columns as 4 x 8 blocks of v_mfma_f32_16x16x32_f16 (the
//    weights are the A operand, so a lane's 4 accumulators of a block are 4
//    consecutive output columns of one row); the 128 accumulators per lane
//    live in AGPRs.  A second wavefront per SIMD keeps MFMAs issuing while
//    the other waits on LDS reads or the stage barrier (measured 10-14%
//    faster than one wavefront owning 128 x 128, at 1.5x the fragment reads);
//  * k-steps of 64, two stages of 64 KB [x rows | weight rows] filled by
//    direct-to-LDS loads (one stage in flight while the other is used), rows
//    XOR-swizzled in 16-byte chunks so that fragment reads are conflict-free;
//  * each stage is two k32 sub-steps of 32 MFMAs per wavefront: the
//    fragments of the next sub-step are read while the current one's MFMAs
//    issue, and the one barrier per stage sits after the first four MFMAs of
//    the last sub-step; the stage is a fixed sequence (MFMAs as volatile asm)
//    with the LDS reads and the direct-to-LDS requests placed between MFMAs;
//  * the 32 workgroups an XCD runs at once cover an aligned 8 x 4 block of
//    tiles and share its activation and weight panels in that XCD's L2; the
//    blocks are dealt to the 8 XCDs round-robin along the tile-rows (K up to
//    16384: the XCDs share activation panels through the infinity cache) or
//    along the tile-columns (longer K: they share weight panels), measured
//    2-4% faster than giving each XCD a contiguous range of its own.
#include "gemm_common.h"
#include "fg_trace.h"

namespace fg {
namespace gemm {
namespace {

constexpr int TB = 256;                 // tile rows and columns
constexpr int TBK = 64;                 // k per stage
constexpr int TSUB = TBK / 32;          // MFMA k-steps per stage
constexpr int TNS = 2;                  // stages in the ring
constexpr int TNT = 512;                // threads (8 wavefronts)
constexpr int T_ROWB = TBK * 2;         // bytes of one row in a stage (8 chunks of 16 B)
constexpr int T_XB = TB * T_ROWB;       // x rows of a stage: 32 KB
constexpr int T_STAGE = 2 * T_XB;       // [x | w]: 64 KB
constexpr int T_INS = T_STAGE / 1024;   // 1 KB load instructions per stage
constexpr int T_LW = T_INS / 8;         // per wavefront
constexpr int T_GM = 8;                 // tile-rows per group
static_assert(T_LW * (TNS - 1) <= 63, "vmcnt range");

// One MFMA as a volatile asm statement, accumulator in AGPRs: volatile asm
// keeps its order relative to the other volatile statements (the
// direct-to-LDS loads, barriers, waits) and to LDS reads, so a stage issues
// exactly as written.  The compiler's waits for LDS reads still precede the
// first MFMA that uses a fragment.
__device__ __forceinline__ void mfma16(f4& c, const h8& a, const h8& b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

__global__ __launch_bounds__(TNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void tile_kernel(Params p, int64_t tiles_m, int64_t tiles_n, int64_t grid) {
    __shared__ __align__(16) unsigned char sb0[T_STAGE];
    __shared__ __align__(16) unsigned char sb1[T_STAGE];
    auto buf = [&](int s) -> unsigned char* { return s == 0 ? sb0 : sb1; };

    // block id -> tile (ids are dealt to the 8 XCDs round-robin, so id b
    // runs on XCD b mod 8 as slot b / 8 of that XCD's sequence)
    const int64_t b = blockIdx.x;
    int64_t m0, n0;
    if (tiles_m % T_GM == 0 && tiles_n % 4 == 0 && (tiles_m * tiles_n) % 256 == 0) {
        // 8 x 4 blocks of tiles: slot s of XCD x is tile s mod 32 of block
        // 8 (s / 32) + x, taken down the block's 8 tile-rows, then across its
        // 4 tile-columns; blocks in order along the tile-rows (K <= 16384) or
        // along the tile-columns
        const int64_t x = b % 8, sl = b / 8;
        const int64_t gb = (sl / 32) * 8 + x, inner = sl % 32;
        int64_t rb, cb;
        if (p.K <= 16384) {
            rb = gb / (tiles_n / 4);
            cb = gb % (tiles_n / 4);
        } else {
            rb = gb % (tiles_m / T_GM);
            cb = gb / (tiles_m / T_GM);
        }
        m0 = (rb * T_GM + inner % T_GM) * TB;
        n0 = (cb * 4 + inner / T_GM) * TB;
    } else {
        // consecutive ids of one XCD, then groups of 8 tile-rows
        // (column-major inside a group)
        const int64_t t = (b % 8) * (grid / 8) + b / 8;
        if (t >= tiles_m * tiles_n) return;   // whole workgroup: before any barrier
        const int64_t per_group = T_GM * tiles_n;
        const int64_t first_m = (t / per_group) * T_GM;
        const int64_t gm = min((int64_t)T_GM, tiles_m - first_m);
        const int64_t wi = t % per_group;
        m0 = (first_m + wi % gm) * TB;
        n0 = (wi / gm) * TB;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;   // 128 rows x 64 columns per wavefront
    const int r32 = lane & 31, hl = lane >> 5;
    const int nk = (int)(p.K / TBK);

    // load slots: instruction j = wave + 8 i covers 8 rows of the stage (x
    // rows for j < 32, weight rows after); lane -> row 8 (j mod 32) + lane / 8,
    // LDS chunk lane % 8 holding global chunk (lane % 8) ^ (row & 7).
    // Rows past M or N repeat the last row (never stored).
    const char* sbase[T_LW];
    uint32_t voff[T_LW];
#pragma unroll
    for (int i = 0; i < T_LW; ++i) {
        const int j = wave + 8 * i;
        const int row = 8 * (j % 32) + (lane >> 3);
        const int gch = (lane & 7) ^ (row & 7);
        if (j < 32) {
            const int64_t gr = min(m0 + row, p.M - 1) - m0;
            sbase[i] = (const char*)(p.x + m0 * p.ldx);
            voff[i] = (uint32_t)((gr * p.ldx) * 2 + gch * 16);
        } else {
            const int64_t gr = min(n0 + row, p.N - 1) - n0;
            sbase[i] = (const char*)((const __half*)p.w + n0 * p.K);
            voff[i] = (uint32_t)((gr * p.K) * 2 + gch * 16);
        }
        const uint64_t bb = (uint64_t)(uintptr_t)sbase[i];
        const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bb >> 32));
        const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bb);
        sbase[i] = (const char*)(uintptr_t)(((uint64_t)bhi << 32) | (uint64_t)blo);
    }
    // stages past the end reload the last one (same load count per stage)
    auto issue1 = [&](unsigned char* base, int ks, int i) {
        const int64_t koff = (int64_t)min(ks, nk - 1) * (TBK * 2);
        dma16s(sbase[i] + koff, voff[i], base + (wave + 8 * i) * 1024);
    };
    auto issue = [&](unsigned char* base, int ks) {
#pragma unroll
        for (int i = 0; i < T_LW; ++i) issue1(base, ks, i);
    };

    // fragments: lane l holds 8 consecutive k (chunk 4s + q of sub-step s)
    // of row r16 of a 16-row block; 4 weight blocks (A) and 8 activation
    // blocks (B) per sub-step
    const int r16 = lane & 15, q = lane >> 4;
    uint32_t xo[TSUB], wo[TSUB];
#pragma unroll
    for (int s = 0; s < TSUB; ++s) {
        xo[s] = (uint32_t)((wm * 128 + r16) * T_ROWB + (((4 * s + q) ^ (r16 & 7)) * 16));
        wo[s] = (uint32_t)(T_XB + (wn * 64 + r16) * T_ROWB + (((4 * s + q) ^ (r16 & 7)) * 16));
    }
    auto read_x = [&](const unsigned char* base, int s, int j) -> h8 {
        return *reinterpret_cast<const h8*>(base + xo[s] + j * 16 * T_ROWB);
    };
    auto read_w = [&](const unsigned char* base, int s, int i) -> h8 {
        return *reinterpret_cast<const h8*>(base + wo[s] + i * 16 * T_ROWB);
    };

    f4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    // activation fragments double-buffered (x0 / x1); weight fragments in one
    // set: w[i] of the next sub-step is read once row i of the current one is
    // done, w[3] at the start of the sub-step that uses it
    h8 x0[8], x1[8], w[4];
#pragma unroll
    for (int st = 0; st < TNS; ++st) issue(buf(st), st);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(T_LW * (TNS - 1)));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) x0[j] = read_x(buf(0), 0, j);
#pragma unroll
    for (int i = 0; i < 3; ++i) w[i] = read_w(buf(0), 0, i);

    // One stage: TSUB sub-steps of 32 MFMAs (acc[i][j], row i outer).  Between
    // the MFMAs: the sub-step's own w[3], then the next sub-step's activation
    // fragments and, row by row, its weight fragments.  In the last sub-step
    // the stage's buffer is released after four MFMAs (every wave's reads of
    // it done, stage ks+1 landed) by the stage's one barrier; the next stage's
    // fragments and the request of stage ks+2 into the released buffer follow.
    auto substep = [&](const unsigned char* cur, const unsigned char* nxt, int s, int ks, unsigned char* rel,
                       h8 (&xa)[8], h8 (&xb)[8]) {
        const bool last = s + 1 == TSUB;
        const unsigned char* src = last ? nxt : cur;
        const int sn = last ? 0 : s + 1;
#pragma unroll
        for (int idx = 0; idx < 32; ++idx) {
            const int i = idx >> 3, j = idx & 7;
            mfma16(acc[i][j], w[i], xa[j]);
            if (idx == 0) w[3] = read_w(cur, s, 3);
            if (last && idx == 3) {
                __builtin_amdgcn_s_waitcnt(vmcnt_wait(T_LW * (TNS - 2)));
                __builtin_amdgcn_s_waitcnt(LGKM_ZERO);
                __builtin_amdgcn_s_barrier();
            }
            if (idx >= 4 && idx < 28 && (idx - 4) % 3 == 0) xb[(idx - 4) / 3] = read_x(src, sn, (idx - 4) / 3);
            if (j == 7 && i < 3) w[i] = read_w(src, sn, i);
            if (last && idx >= 4 && idx < 4 + T_LW) issue1(rel, ks + TNS, idx - 4);
        }
    };
    for (int kt = 0; kt < nk; kt += TNS) {
#pragma unroll
        for (int st = 0; st < TNS; ++st) {
            const int ks = kt + st;
            if (ks < nk) {
                unsigned char* cur = buf(st);
                const unsigned char* nxt = buf((st + 1) % TNS);
#pragma unroll
                for (int s = 0; s < TSUB; ++s) {
                    if (s & 1) substep(cur, nxt, s, ks, cur, x1, x0);
                    else substep(cur, nxt, s, ks, cur, x0, x1);
                }
            }
        }
    }
    // drain the reloads past the end before the workgroup exits; the MFMA
    // results are read by VALU below (an XDL write needs up to 11 wait states)
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    asm volatile("s_nop 7\n\ts_nop 7");

    // epilogue: acc[i][j][e] is column n0 + wn*128 + 16 i + 4 q + e of row
    // m0 + wm*128 + 16 j + r16
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t m = m0 + wm * 128 + 16 * j + r16;
        if (m >= p.M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + wn * 64 + 16 * i + 4 * q;
            if (n < p.N) store4_final(p, m, n, acc[i][j]);
        }
    }
}

}  // namespace

// 32-bit per-lane offsets inside a tile: 255 rows of the longer operand
bool tile_fits(const Params& p) {
    const int64_t ld = p.ldx > p.K ? p.ldx : p.K;
    return p.K % TBK == 0 && p.N % 4 == 0 && 255 * ld * 2 + 64 < (1ll << 32);
}

int launch_tile(const Params& p, hipStream_t st) {
    if (!tile_fits(p)) return set_error(FG_ERR_UNSUPPORTED, "large-M GEMM: K %% 32, N %% 4, offsets in 32 bits");
    const int64_t tm = (p.M + TB - 1) / TB, tn = (p.N + TB - 1) / TB;
    const int64_t grid = (tm * tn + 7) / 8 * 8;
    if (grid >= (1ll << 31)) return set_error(FG_ERR_UNSUPPORTED, "large-M GEMM: too many tiles");
    tile_kernel<<<(unsigned)grid, TNT, 0, st>>>(p, tm, tn, grid);
    FG_LAUNCHED("tile_kernel");
    return FG_OK;
}

}  // namespace gemm
}  // namespace fg
