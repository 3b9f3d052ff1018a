"""GPU checks of the per-kernel timing that the benchmark's rooflines rest on:
launch-recorded kinds (the decode GEMM, whose projection kinds share its
record, and decode attention), a kind bracketed by events around its launch
(the LayerNorm and the K/V append), and the kind mask."""
import pytest

import synth

pytestmark = pytest.mark.gpu

SHP = dict(h1=512, h2=2048, nh=4, hd=128)


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


@pytest.fixture(scope="module")
def block(L):
    """One 4-bit decode layer at bls 4 x 3 with a 4-bit cache of 20 positions,
    and a function running one decode step of it."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV, DeviceLayer
    h1, h2, nh, hd = SHP["h1"], SHP["h2"], SHP["nh"], SHP["hd"]
    gbs, nb, P = 4, 3, 20
    bls = gbs * nb
    W = synth.layer_weights(h1, h2, 0, seed=5, random_ln=True)
    lay = DeviceLayer.from_fp16({k: v.cuda() for k, v in W.items()}, L.FG_FMT_Q4G64)
    d = L.dims(h1, h2, nh, hd)
    kv = DeviceKV(L.FG_FMT_Q4G64, bls, nh, hd, P + 4, "cuda")
    kh, vh = synth.kv_history(bls, nh, P, hd, seed=6, device="cuda")
    for p in range(P):
        L.fg_kv_append_q4(kh[:, p].contiguous(), vh[:, p].contiguous(), h1, kv.struct, bls, d, p)
    x0 = synth.activations(bls, h1, seed=7, device="cuda")
    x = x0.clone()
    ws = torch.empty(L.fg_workspace_bytes(d, bls, L.FG_FMT_Q4G64), dtype=torch.uint8, device="cuda")

    def step():
        x.copy_(x0)
        L.fg_layer_decode_block(d, lay.struct, x, gbs, nb, P, kv.struct, ws, ws.numel())
    torch.cuda.synchronize()
    return step


def _traced(L, step, kinds, n):
    import torch
    L.fg_trace_kinds(kinds)
    L.fg_trace_enable(True)
    try:
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        return L.fg_trace_collect()
    finally:
        L.fg_trace_enable(False)
        L.fg_trace_kinds(None)


def test_every_kind_of_a_decode_layer_is_timed(L, block):
    n = 3
    tr = _traced(L, block, None, n)
    assert tr["gemm_q4"]["count"] == 4 * n
    for k in ("proj_qkv", "proj_out", "proj_fc1", "proj_fc2"):
        assert tr[k]["count"] == n, k
        assert tr[k]["ms"] > 0
    # the projection kinds are credited with the GEMM's own records
    proj_ms = sum(tr[k]["ms"] for k in ("proj_qkv", "proj_out", "proj_fc1", "proj_fc2"))
    assert proj_ms == pytest.approx(tr["gemm_q4"]["ms"], rel=1e-9)
    proj_fl = sum(tr[k]["flops"] for k in ("proj_qkv", "proj_out", "proj_fc1", "proj_fc2"))
    assert proj_fl == pytest.approx(tr["gemm_q4"]["flops"], rel=1e-12)
    h1, h2 = SHP["h1"], SHP["h2"]
    assert tr["gemm_q4"]["flops"] == pytest.approx(n * 2 * 12 * (3 * h1 * h1 + h1 * h1 + 2 * h1 * h2))
    assert tr["attn_decode_q4"]["count"] == n and tr["attn_decode_q4"]["ms"] > 0
    assert tr["kv_store"]["count"] == n and tr["kv_store"]["ms"] > 0   # the append, bracketed
    assert tr["layernorm"]["count"] == n                                # LN1, bracketed


def test_kind_mask_records_only_the_named_kinds(L, block):
    tr = _traced(L, block, ["attn_decode_q4"], 2)
    assert set(tr) == {"attn_decode_q4"} and tr["attn_decode_q4"]["count"] == 2
    tr = _traced(L, block, ["proj_out"], 2)              # a projection without its GEMM kind
    assert set(tr) == {"proj_out"} and tr["proj_out"]["count"] == 2
    tr = _traced(L, block, [], 2)
    assert tr == {}
