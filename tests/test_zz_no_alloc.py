"""fg_linear_noalloc (the projection GEMM with its split-k partials in the
library's own device array, for callers that cannot allocate) against
fg_linear with a caller workspace: identical outputs, bit for bit, over calls
in a row on one stream, the second with a smaller input, a later call again
at full size, and 4-bit as well as fp16 weights."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, np16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def _case(L, M, N, K, fmt, seed, residual=True):
    import torch
    from throughput_oriented_offloaded_amd.model import quantize_weight
    x = synth.activations(M, K, seed=seed, device="cuda")
    w = synth.normal_f16((N, K), seed + 1, device="cuda")
    b = synth.normal_f16((N,), seed + 2, device="cuda")
    r = synth.activations(M, N, seed=seed + 3, device="cuda") if residual else None
    if fmt == L.FG_FMT_Q4G64:
        wc, m = quantize_weight(w)
    else:
        wc, m = w, None
    return x, wc, m, b, r, w


def _pair(L, M, N, K, fmt, seed, act=0):
    import torch
    x, wc, m, b, r, w = _case(L, M, N, K, fmt, seed)
    need = L.fg_linear_workspace_bytes(M, N, K)
    assert 0 < need <= L._L.fg_linear_noalloc_max_bytes()     # split-k partials are in play
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    y_ws = torch.empty((M, N), dtype=torch.float16, device="cuda")
    y_na = torch.empty_like(y_ws)
    L.fg_linear(x, M, K, fmt, wc, m, N, b, act, r, y_ws, ws, ws.numel())
    L.fg_linear_noalloc(x, M, K, fmt, wc, m, N, b, act, r, y_na)
    torch.cuda.synchronize()
    return x, wc, m, b, r, w, y_ws, y_na


def test_noalloc_matches_workspace_calls_in_a_row(L):
    import torch
    # the OPT-175B out-projection at bls 144 (partials of 7 slots, 49.5 MB),
    # then a smaller 4-bit shape, then FC1-like fp16, then full size again
    shapes = [(144, 12288, 12288, L.FG_FMT_Q4G64, 0), (20, 1024, 768, L.FG_FMT_Q4G64, 1),
              (40, 3072, 768, L.FG_FMT_F16, 1), (144, 12288, 12288, L.FG_FMT_Q4G64, 0)]
    for i, (M, N, K, fmt, act) in enumerate(shapes):
        x, wc, m, b, r, w, y_ws, y_na = _pair(L, M, N, K, fmt, seed=100 + 10 * i, act=act)
        assert torch.equal(y_ws, y_na), f"call {i}: {M}x{N}x{K} differs from fg_linear"
        if M * N <= 40 * 3072:     # small shapes: also held to the oracle
            Wn = np16(w)
            if fmt == L.FG_FMT_Q4G64:
                Wn = oracle.dequant_weight(*oracle.quant_weight(Wn), N, K)
            ref = oracle.linear(np16(x), Wn, np16(b), relu=bool(act), residual=np16(r))
            assert_close(np16(y_na), ref, f"call {i} vs oracle")
