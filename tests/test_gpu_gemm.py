"""GPU parity of fg_linear (fp16 and dequant-fused 4-bit MFMA GEMM) against the
oracle's fp64 linear on the oracle's own dequantized weights."""
import numpy as np
import pytest

import oracle
from helpers import assert_close, dev16, np16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def _run(L, fmt, M, N, K, bias=True, act=0, residual=False, inplace=False, seed=0):
    import torch
    rng = np.random.default_rng(seed + M * 7 + N * 3 + K)
    x = (rng.standard_normal((M, K))).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    b = (rng.standard_normal(N) * 0.02).astype(np.float16) if bias else None
    r = (rng.standard_normal((M, N))).astype(np.float16) if residual else None
    xd, wd = dev16(x), dev16(w)
    if fmt == "q4":
        codes = torch.empty((N // 2, K), dtype=torch.uint8, device="cuda")
        meta = torch.empty((N // 64, 2, K), dtype=torch.float16, device="cuda")
        L.fg_quant_group4(wd, 1, N, K, codes, meta)
        wc, wm, f = codes, meta, L.FG_FMT_Q4G64
        rc, rm = oracle.quant_weight(w)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(np16(meta), rm)
        w_ref = oracle.dequant_weight(rc, rm, N, K)
    else:
        wc, wm, f = wd, None, L.FG_FMT_F16
        w_ref = w
    bd = dev16(b) if bias else None
    rd = dev16(r) if residual else None
    y = rd if inplace else torch.empty((M, N), dtype=torch.float16, device="cuda")
    wsb = L.fg_linear_workspace_bytes(M, N, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    L.fg_linear(xd, M, K, f, wc, wm, N, bd, act, rd, y, ws, wsb)
    torch.cuda.synchronize()
    ref = oracle.linear(x, w_ref, b, relu=bool(act), residual=r)
    return np16(y), ref


SHAPES = [  # M, N, K
    (1, 64, 64), (4, 2304, 768), (4, 768, 3072), (16, 256, 128), (17, 320, 192),
    (100, 192, 256), (128, 512, 256), (144, 768, 768), (144, 3072, 768), (144, 768, 3072),
    (145, 256, 128), (300, 512, 192), (700, 384, 128), (1000, 128, 64), (2048, 256, 256),
    # 32-row-block decode tiles: 96 rows (ragged N), 128 x 2, exactly 160
    (72, 320, 192), (96, 768, 1024), (256, 1024, 512), (160, 512, 2048),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_linear_q4(L, M, N, K):
    got, ref = _run(L, "q4", M, N, K)
    assert_close(got, ref, f"q4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", SHAPES + [(5, 200, 64), (144, 1000, 128), (3, 50272, 64)])
def test_linear_f16(L, M, N, K):
    got, ref = _run(L, "f16", M, N, K)
    assert_close(got, ref, f"f16 {M}x{N}x{K}")


# more than 576 rows with fp16 weights: the 256 x 256-tile kernel (ragged M
# and N, a partial last group of tile-rows, K of one and of many stages)
TILE_SHAPES = [(577, 256, 64), (1300, 1000, 320), (4100, 2304, 256), (2600, 768, 1024), (1024, 8, 64)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_linear_f16_large_m(L, M, N, K):
    got, ref = _run(L, "f16", M, N, K)
    assert_close(got, ref, f"f16 {M}x{N}x{K}")


# whole 8 x 4 blocks of 256 x 256 tiles (M = 2048, N = 8192: 256 tiles), the
# order the XCDs take the blocks in: along the tile-rows for K <= 16384,
# along the tile-columns beyond
@pytest.mark.parametrize("K", [320, 16448])
def test_linear_f16_large_m_block_orders(L, K):
    """Every output tile is computed once, wherever the block order sends it:
    three rows of every tile-row against the oracle over all columns."""
    import torch
    M, N = 2048, 8192
    rng = np.random.default_rng(K)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    b = (rng.standard_normal(N) * 0.02).astype(np.float16)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    wsb = L.fg_linear_workspace_bytes(M, N, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    L.fg_linear(dev16(x), M, K, L.FG_FMT_F16, dev16(w), None, N, dev16(b), 0, None, y, ws, wsb)
    torch.cuda.synchronize()
    rows = np.array([t * 256 + o for t in range(M // 256) for o in (0, 137, 255)])
    ref = oracle.linear(np.ascontiguousarray(x[rows]), w, b)
    assert_close(np16(y)[rows], ref, f"f16 {M}x{N}x{K} sampled rows")


def test_linear_large_m_epilogues(L):
    got, ref = _run(L, "f16", 1000, 512, 1024, act=1)
    assert_close(got, ref, "relu")
    assert np.all(got.view(np.float16) >= 0)
    got, ref = _run(L, "f16", 1000, 512, 512, residual=True)
    assert_close(got, ref, "residual")
    got, ref = _run(L, "f16", 1000, 512, 512, residual=True, inplace=True)
    assert_close(got, ref, "residual in place")
    got, ref = _run(L, "f16", 700, 264, 192, bias=False)
    assert_close(got, ref, "no bias")


@pytest.mark.parametrize("fmt", ["q4", "f16"])
def test_linear_epilogues(L, fmt):
    got, ref = _run(L, fmt, 144, 512, 1024, act=1)
    assert_close(got, ref, "relu")
    assert np.all(got.view(np.float16) >= 0)
    got, ref = _run(L, fmt, 144, 512, 2048, residual=True)
    assert_close(got, ref, "residual")
    got, ref = _run(L, fmt, 144, 512, 2048, residual=True, inplace=True)
    assert_close(got, ref, "residual in place")
    got, ref = _run(L, fmt, 37, 256, 192, bias=False)
    assert_close(got, ref, "no bias")


def test_linear_rows_independent_of_batch_split(L):
    """Same M, any split of the rows into GPU batches: a row's result depends
    only on that row (bitwise), which is what lets the block be one GEMM."""
    import torch
    rng = np.random.default_rng(9)
    M, N, K = 144, 512, 1024
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    wd = dev16(w)
    codes = torch.empty((N // 2, K), dtype=torch.uint8, device="cuda")
    meta = torch.empty((N // 64, 2, K), dtype=torch.float16, device="cuda")
    L.fg_quant_group4(wd, 1, N, K, codes, meta)
    wsb = L.fg_linear_workspace_bytes(M, N, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    y1 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    L.fg_linear(dev16(x), M, K, L.FG_FMT_Q4G64, codes, meta, N, None, 0, None, y1, ws, wsb)
    perm = rng.permutation(M)
    y2 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    L.fg_linear(dev16(x[perm]), M, K, L.FG_FMT_Q4G64, codes, meta, N, None, 0, None, y2, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(y1[torch.from_numpy(perm).cuda()], y2)


@pytest.mark.parametrize("M,N,K", [(144, 768, 3072), (144, 4096, 4096), (40, 1024, 8192)])
def test_linear_shared_tiles_any_workspace(L, M, N, K):
    """Tiles split over many workgroups (fp32 partials in the workspace, summed
    in segment order): correct from a workspace full of garbage, bit-identical
    over repeated calls on the same workspace and after another shape used it."""
    import torch
    rng = np.random.default_rng(M + N + K)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    b = (rng.standard_normal(N) * 0.02).astype(np.float16)
    codes = torch.empty((N // 2, K), dtype=torch.uint8, device="cuda")
    meta = torch.empty((N // 64, 2, K), dtype=torch.float16, device="cuda")
    L.fg_quant_group4(dev16(w), 1, N, K, codes, meta)
    rc, rm = oracle.quant_weight(w)
    wsb = L.fg_linear_workspace_bytes(M, N, K)
    assert wsb > 0, "shape must share tiles"
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device="cuda")
    xd, bd = dev16(x), dev16(b)
    ys = []
    for _ in range(4):
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        L.fg_linear(xd, M, K, L.FG_FMT_Q4G64, codes, meta, N, bd, 0, None, y, ws, wsb)
        ys.append(y)
    # another shape through the same workspace, then this one again
    y_o = torch.empty((M, 256), dtype=torch.float16, device="cuda")
    L.fg_linear(xd, M, K, L.FG_FMT_Q4G64, codes, meta, 256, None, 0, None, y_o, ws, wsb)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    L.fg_linear(xd, M, K, L.FG_FMT_Q4G64, codes, meta, N, bd, 0, None, y, ws, wsb)
    ys.append(y)
    torch.cuda.synchronize()
    ref = oracle.linear(x, oracle.dequant_weight(rc, rm, N, K), b)
    assert_close(np16(ys[0]), ref, f"q4 shared tiles {M}x{N}x{K}")
    for i, yi in enumerate(ys[1:], 1):
        assert torch.equal(yi, ys[0]), f"call {i} differs bitwise"
    ref_o = oracle.linear(x, oracle.dequant_weight(rc[:128], rm[:4], 256, K), None)
    assert_close(np16(y_o), ref_o, "q4 first 256 columns")


OPT175_PROJ = [  # N, K, act, residual: QKV, out-projection, FC1 (ReLU), FC2
    (3 * 12288, 12288, 0, False), (12288, 12288, 0, True), (49152, 12288, 1, False),
    (12288, 49152, 0, True)]


@pytest.mark.parametrize("N,K,act,res", OPT175_PROJ)
def test_linear_q4_opt175b_shapes_sampled(L, N, K, act, res):
    """The decode GEMM at the OPT-175B block (M = 144) on full weights,
    quantized on the device in one call, through the stream-K path the
    benchmark times.  The oracle quantizes the sampled 64-row groups itself
    from the same fp16 weights (the device's codes must equal them) and
    computes the sampled outputs from its own dequantized rows."""
    import torch
    import synth
    M = 144
    lay = N // 1024 + K // 1024          # distinct seeds per shape
    w = synth.normal_f16((N, K), synth.tensor_seed(7, lay, "w_1"), "cuda", std=0.02)
    x = synth.normal_f16((M, K), synth.tensor_seed(7, lay, "x"), "cuda")
    b = synth.normal_f16((N,), synth.tensor_seed(7, lay, "b_1"), "cuda", std=0.02)
    r = synth.normal_f16((M, N), synth.tensor_seed(7, lay, "vhist"), "cuda") if res else None
    codes = torch.empty((N // 2, K), dtype=torch.uint8, device="cuda")
    meta = torch.empty((N // 64, 2, K), dtype=torch.float16, device="cuda")
    L.fg_quant_group4(w, 1, N, K, codes, meta)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    wsb = L.fg_linear_workspace_bytes(M, N, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    L.fg_linear(x, M, K, L.FG_FMT_Q4G64, codes, meta, N, b, act, r, y, ws, wsb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N + K)
    groups = sorted(set(rng.integers(0, N // 64, size=3).tolist()) | {0, N // 64 - 1})
    rows = np.sort(rng.choice(M, size=6, replace=False))
    xs = np16(x)[rows]
    ys = np16(y)[rows]
    rs = np16(r)[rows] if res else None
    bh = np16(b)
    for g in groups:
        wg = np16(w[g * 64:(g + 1) * 64])
        rc, rm = oracle.quant_weight(wg)
        assert np.array_equal(codes[g * 32:(g + 1) * 32].cpu().numpy(), rc), f"codes of group {g}"
        assert np.array_equal(np16(meta[g:g + 1]), rm), f"meta of group {g}"
        w_ref = oracle.dequant_weight(rc, rm, 64, K)
        resid = np.ascontiguousarray(rs[:, g * 64:(g + 1) * 64]) if res else None
        ref = oracle.linear(xs, w_ref, bh[g * 64:(g + 1) * 64], relu=bool(act), residual=resid)
        got = ys[:, g * 64:(g + 1) * 64]
        assert_close(got, ref, f"M=144 N={N} K={K} group {g}")
    # every tile here is shared (up to 6 segments): the fixed summation order
    # gives the same bits on every call, whatever order the segments finish in
    y2 = torch.empty_like(y)
    for i in range(12):
        L.fg_linear(x, M, K, L.FG_FMT_Q4G64, codes, meta, N, b, act, r, y2, ws, wsb)
        torch.cuda.synchronize()
        assert torch.equal(y2, y), f"repeat {i} differs bitwise"

