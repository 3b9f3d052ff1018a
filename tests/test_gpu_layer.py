"""GPU parity of fg_layer_decode_block / fg_layer_prefill and of the whole
model against the oracle (max|err| <= 1e-2 max|ref| + 1e-3), plus the
block-partition invariance of the zig-zag decode."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, dev16, np16, ranked_kv

pytestmark = pytest.mark.gpu

OPT125 = dict(h1=768, h2=3072, nh=12, hd=64)


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def _layer(L, shp, fmt, seed, random_ln=True):
    """Device layer (quantized on the device for q4) + the oracle's fp16 view of it."""
    from throughput_oriented_offloaded_amd.model import DeviceLayer
    W = synth.layer_weights(shp["h1"], shp["h2"], 0, seed=seed, random_ln=random_ln)
    dl = DeviceLayer.from_fp16({k: v.cuda() for k, v in W.items()},
                               L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16)
    d = oracle.Dims(shp["h1"], shp["h2"], shp["nh"], shp["hd"])
    Wn = {k: v.numpy().view(np.uint16) for k, v in W.items()}
    if fmt == "q4":
        Wq = oracle.quant_layer(d, Wn)
        for name in ("qkv", "o", "1", "2"):
            assert np.array_equal(dl.t["w_" + name].cpu().numpy(), Wq["c_" + name])
            assert np.array_equal(np16(dl.t["m_" + name]), Wq["m_" + name])
        Wn = oracle.dequant_layer(d, Wq)
    return dl, Wn, d


def _history(L, shp, fmt, bls, P, lmax, seed):
    from throughput_oriented_offloaded_amd.model import DeviceKV
    h1, nh, hd = shp["h1"], shp["nh"], shp["hd"]
    kv = DeviceKV(L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16, bls, nh, hd, lmax, "cuda")
    kh, vh = synth.kv_history(bls, nh, P, hd, seed=seed)
    d = L.dims(h1, shp["h2"], nh, hd)
    app = L.fg_kv_append_q4 if fmt == "q4" else L.fg_kv_append_f16
    khd, vhd = kh.cuda(), vh.cuda()
    for p in range(P):
        app(khd[:, p].contiguous(), vhd[:, p].contiguous(), h1, kv.struct, bls, d, p)
    oc = oracle.KVCache(fmt, bls, nh, hd, lmax)
    if P:
        oc.store(kh.numpy().view(np.uint16), vh.numpy().view(np.uint16), 0)
    return kv, oc, d


@pytest.mark.parametrize("fmt,kvfmt", [("q4", "q4"), ("f16", "f16"), ("q4", "f16")])
@pytest.mark.parametrize("P", [0, 7, 40])
def test_decode_block_matches_oracle(L, fmt, kvfmt, P):
    import torch
    bls, lmax = 6, 48
    dl, Wn, od = _layer(L, OPT125, fmt, seed=3)
    kv, oc, d = _history(L, OPT125, kvfmt, bls, P, lmax, seed=4)
    x = synth.activations(bls, OPT125["h1"], seed=5)
    xd = x.cuda()
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    L.fg_layer_decode_block(d, dl.struct, xd, 3, 2, P, kv.struct, ws, ws.numel())
    torch.cuda.synchronize()
    ref, _, _ = oracle.layer_decode(od, Wn, x.numpy().view(np.uint16), P, oc)
    assert_close(np16(xd), ref, f"decode block {fmt}/{kvfmt} pos {P}")
    # cache history below P untouched and equal to the oracle's codes
    if kvfmt == "q4":
        assert np.array_equal(kv.k[:, :, :P].cpu().numpy(), oc.k[:, :, :P])
    # the appended row at P dequantizes to the oracle's within the tolerance
    if kvfmt == "q4":
        from throughput_oriented_offloaded_amd import _lib as LL  # noqa: F401
        got_c = kv.k[:, :, P].cpu().numpy()
        same = np.mean(got_c == oc.k[:, :, P])
        assert same > 0.9, f"appended codes agree on only {same:.3f}"


def _ranked_history(L, kvfmt, q, bls, P, lmax, seed):
    """Device cache and oracle cache of P positions with evenly spread scores
    against q (helpers.ranked_kv).  q: float [bls, nh, hd]."""
    from throughput_oriented_offloaded_amd.model import DeviceKV
    bls_, nh, hd = q.shape
    h1 = nh * hd
    kx, vx = ranked_kv(q, P, seed)
    kv = DeviceKV(L.FG_FMT_Q4G64 if kvfmt == "q4" else L.FG_FMT_F16, bls, nh, hd, lmax, "cuda")
    d = L.dims(h1, OPT125["h2"], nh, hd)
    app = L.fg_kv_append_q4 if kvfmt == "q4" else L.fg_kv_append_f16
    kd, vd = dev16(kx), dev16(vx)
    for p in range(P):
        app(kd[:, p].contiguous(), vd[:, p].contiguous(), h1, kv.struct, bls, d, p)
    oc = oracle.KVCache(kvfmt, bls, nh, hd, lmax)
    oc.store(kx, vx, 0)
    return kv, oc, d


@pytest.mark.parametrize("wfmt,kvfmt,P", [("q4", "q4", 40), ("f16", "f16", 40), ("q4", "f16", 300),
                                          ("q4", "q4", 300)])
def test_decode_block_topk_matches_oracle(L, wfmt, kvfmt, P):
    """Top-K sparse V inside the block decode (attn_topk_ppm 100000: the pages'
    10%, topk = ceil(P / 10)) against the oracle's layer at attn_topk 0.1; the
    dense oracle is far outside the tolerance, so the sparse path was taken."""
    import copy
    import torch
    bls, lmax = 6, P + 4
    h1, nh, hd = OPT125["h1"], OPT125["nh"], OPT125["hd"]
    dl, Wn, od = _layer(L, OPT125, wfmt, seed=31)
    x = synth.activations(bls, h1, seed=32)
    xn = x.numpy().view(np.uint16)
    qkv = oracle.linear(oracle.layernorm(xn, Wn["ln1_g"], Wn["ln1_b"]), Wn["w_qkv"], Wn["b_qkv"])
    q = oracle.to_f16(qkv[:, :h1]).astype(np.float64).reshape(bls, nh, hd)
    kv, oc, d = _ranked_history(L, kvfmt, q, bls, P, lmax, seed=33)
    topk = oracle.topk_count(P, 0.1)
    k64 = oracle.to_f16(oc.history()[0]).astype(np.float64)
    for b in range(bls):
        for h in range(nh):
            sc = np.sort(k64[b, h, :P] @ q[b, h])[::-1] / np.sqrt(hd)
            assert sc[topk - 1] - sc[topk] > 0.5 * 3.0 / P, "scores not spread as built"
    oc_dense = copy.deepcopy(oc)
    xd = x.cuda()
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    L.fg_layer_decode_block(d, dl.struct, xd, 3, 2, P, kv.struct, ws, ws.numel(),
                            attn_topk_ppm=100000)
    torch.cuda.synchronize()
    ref, _, _ = oracle.layer_decode(od, Wn, xn, P, oc, attn_topk=0.1)
    err, tol = assert_close(np16(xd), ref, f"top-k decode block {wfmt}/{kvfmt} pos {P}")
    dense, _, _ = oracle.layer_decode(od, Wn, xn, P, oc_dense)
    from helpers import f32
    assert np.abs(f32(dense) - f32(ref)).max() > 4 * tol


def test_decode_block_topk_dense_limits(L):
    """attn_topk_ppm 0, 1000000 and any fraction whose count reaches pos all
    give the dense block decode, bit for bit."""
    import torch
    bls, P, lmax = 6, 7, 12
    dl, _, _ = _layer(L, OPT125, "q4", seed=41)
    outs = []
    for ppm in (0, 1000000, 900000):          # ceil(7 * 0.9) = 7 = pos
        kv, _, d = _history(L, OPT125, "q4", bls, P, lmax, seed=42)
        xd = synth.activations(bls, OPT125["h1"], seed=43).cuda()
        ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
        L.fg_layer_decode_block(d, dl.struct, xd, 3, 2, P, kv.struct, ws, ws.numel(),
                                attn_topk_ppm=ppm)
        torch.cuda.synchronize()
        outs.append(xd.clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# FFN wide enough (h2 > 32768) that FC2 keeps its 4-bit weights in the
# prefill-shaped GEMMs while the other three run from fp16 copies
WIDE_FF = dict(h1=128, h2=33024, nh=2, hd=64)


@pytest.mark.parametrize("shp,fmt,s", [
    (OPT125, "q4", 37), (OPT125, "f16", 37),
    # 600 rows per GPU batch: the prefill-shaped (data-parallel) GEMMs
    (OPT125, "q4", 300), (OPT125, "f16", 300), (WIDE_FF, "q4", 300)])
def test_prefill_matches_oracle(L, shp, fmt, s):
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV
    gbs, nb = 2, 2
    bls = gbs * nb
    dl, Wn, od = _layer(L, shp, fmt, seed=7)
    d = L.dims(shp["h1"], shp["h2"], shp["nh"], shp["hd"])
    kv = DeviceKV(dl.fmt, bls, shp["nh"], shp["hd"], s + 2, "cuda")
    x = synth.activations(bls * s, shp["h1"], seed=8)
    xd = x.cuda()
    ws = torch.empty(L.fg_workspace_bytes(d, gbs * s, dl.fmt), dtype=torch.uint8, device="cuda")
    L.fg_layer_prefill(d, dl.struct, xd, gbs, nb, s, kv.struct, ws, ws.numel())
    torch.cuda.synchronize()
    oc = oracle.KVCache("q4" if fmt == "q4" else "f16", bls, shp["nh"], shp["hd"], s + 2)
    ref = oracle.layer_prefill(od, Wn, x.numpy().view(np.uint16), bls, s, oc)
    assert_close(np16(xd), ref, f"prefill {fmt}")
    # cached history: dequantized K, V within tolerance of the oracle's
    from helpers import f32
    if fmt == "q4":
        h1 = shp["h1"]
        kd = torch.empty((bls * shp["nh"] * (s + 2), shp["hd"]), dtype=torch.float16, device="cuda")
        L.fg_dequant_group4(kv.k, kv.km, bls * shp["nh"] * (s + 2), shp["hd"], 1, kd)
        torch.cuda.synchronize()
        got = np16(kd).reshape(bls, shp["nh"], s + 2, shp["hd"])[:, :, :s]
        want = oc.history()[0][:, :, :s]
        assert np.abs(f32(got) - f32(want)).max() <= 0.15 * np.abs(f32(want)).max()
        assert np.mean(kv.k[:, :, :s].cpu().numpy() == oc.k[:, :, :s]) > 0.9


def test_decode_partition_invariance(L):
    """bls = 12 as 12 x 1, 4 x 3, 1 x 12: identical outputs bit for bit."""
    import torch
    bls, P, lmax = 12, 20, 24
    dl, _, _ = _layer(L, OPT125, "q4", seed=11)
    outs = []
    for gbs, nb in ((12, 1), (4, 3), (1, 12)):
        kv, _, d = _history(L, OPT125, "q4", bls, P, lmax, seed=12)
        xd = synth.activations(bls, OPT125["h1"], seed=13).cuda()
        ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
        L.fg_layer_decode_block(d, dl.struct, xd, gbs, nb, P, kv.struct, ws, ws.numel())
        torch.cuda.synchronize()
        outs.append((xd.clone(), kv.k.clone(), kv.vm.clone()))
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])
        assert torch.equal(o[2], outs[0][2])


def test_decode_sequence_independence(L):
    """A sequence's output does not depend on the other sequences in the block."""
    import torch
    bls, P, lmax = 8, 10, 12
    dl, _, _ = _layer(L, OPT125, "q4", seed=21)
    kv, _, d = _history(L, OPT125, "q4", bls, P, lmax, seed=22)
    x = synth.activations(bls, OPT125["h1"], seed=23).cuda()
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    x1 = x.clone()
    L.fg_layer_decode_block(d, dl.struct, x1, bls, 1, P, kv.struct, ws, ws.numel())
    kv2, _, _ = _history(L, OPT125, "q4", bls, P, lmax, seed=22)
    x2 = x.clone()
    x2[1::2] = 0.5 * x2[1::2] + 0.25      # perturb the odd sequences only
    L.fg_layer_decode_block(d, dl.struct, x2, bls, 1, P, kv2.struct, ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.equal(x1[0::2], x2[0::2])


@pytest.mark.parametrize("wfmt,kvfmt", [("q4", "q4"), ("f16", "f16")])
def test_model_end_to_end_opt125m_shape(L, wfmt, kvfmt):
    """2-layer OPT-125m-shape decoder, gbs 4 x 1, s = 32, n = 8 greedy steps.
    The oracle is teacher-forced with the device's tokens; every step's logits
    must meet the tolerance and the device's pick must be (near-)best for the oracle."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape
    sh = Shape(n_layers=2, h1=768, h2=3072, n_heads=12, head_dim=64)
    bls, s, n = 4, 32, 8
    f = L.FG_FMT_Q4G64 if wfmt == "q4" else L.FG_FMT_F16
    Ws = [synth.layer_weights(sh.h1, sh.h2, j, seed=0) for j in range(sh.n_layers)]
    emb = synth.embeddings(sh.h1, s + n, seed=0)
    toks = synth.tokens(bls, s, seed=0)
    layers = [DeviceLayer.from_fp16({k: v.cuda() for k, v in W.items()}, f) for W in Ws]
    m = Model(sh, layers, {k: v.cuda() for k, v in emb.items()},
              L.FG_FMT_Q4G64 if kvfmt == "q4" else L.FG_FMT_F16, bls, s + n)
    out, lgs = m.generate(toks.cuda(), n, gbs=bls, nb=1)
    torch.cuda.synchronize()
    gtok = out.cpu().numpy()
    d = oracle.Dims(sh.h1, sh.h2, sh.n_heads, sh.head_dim)
    ol = []
    for W in Ws:
        Wn = {k: v.numpy().view(np.uint16) for k, v in W.items()}
        ol.append(oracle.dequant_layer(d, oracle.quant_layer(d, Wn)) if wfmt == "q4" else Wn)
    e = {k: v.numpy().view(np.uint16) for k, v in emb.items()}
    om = oracle.Model(d, ol, e["embed"], e["pos"], e["lnf_g"], e["lnf_b"], kvfmt, s + n, bls)
    refs = [om.prefill(toks.numpy())[0]]
    for t in range(1, n):
        refs.append(om.decode(gtok[:, t - 1], s + t - 1)[0])
    agree = 0
    for t in range(n):
        got = np16(lgs[t])
        err, tol = assert_close(got, refs[t], f"logits step {t}")
        r = oracle.to_f16(refs[t]).astype(np.float32)
        best = r.max(1)
        picked = r[np.arange(bls), gtok[:, t]]
        assert np.all(picked >= best - 2 * tol), "device pick far from the oracle's best"
        agree += int(np.sum(gtok[:, t] == r.argmax(1)))
    assert agree >= 0.9 * bls * n


def test_model_attn_topk_option(L):
    """Model(attn_topk=): 1.0 is the dense model bit for bit; 0.1 reaches the
    sparse kernel through fg_model_decode_step (logits move; the prefill,
    which has no Top-K, does not)."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape
    sh = Shape(n_layers=2, h1=768, h2=3072, n_heads=12, head_dim=64)
    bls, s, n = 4, 40, 3
    Ws = [synth.layer_weights(sh.h1, sh.h2, j, seed=0) for j in range(sh.n_layers)]
    emb = {k: v.cuda() for k, v in synth.embeddings(sh.h1, s + n, seed=0).items()}
    toks = synth.tokens(bls, s, seed=5).cuda()
    layers = [DeviceLayer.from_fp16({k: v.cuda() for k, v in W.items()}, L.FG_FMT_Q4G64) for W in Ws]
    runs = {}
    for frac in (0.0, 1.0, 0.1):
        m = Model(sh, layers, emb, L.FG_FMT_Q4G64, bls, s + n, attn_topk=frac)
        forced = torch.zeros((bls, n), dtype=torch.int32, device="cuda")
        runs[frac] = m.generate(toks, n, gbs=2, nb=2, forced=forced)[1]
    torch.cuda.synchronize()
    for a, b in zip(runs[0.0], runs[1.0]):
        assert torch.equal(a, b)
    assert torch.equal(runs[0.0][0], runs[0.1][0])
    assert not torch.equal(runs[0.0][1], runs[0.1][1])


def test_decode_block_opt175b_shape_sampled(L):
    """One OPT-175B-shape layer (4-bit weights and cache, random LayerNorms)
    decoding the benchmark's block: gbs 48 x 3, history of 528 positions,
    the same launches as a benchmark step (stream-K GEMMs, split-k sums fused
    with LayerNorm, one-wavefront attention per (sequence, head)).  The
    library's weight codes equal the oracle's; three sampled sequences (first,
    middle and last GPU batch) are checked against the oracle's layer."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV, DeviceLayer
    h1, h2, nh, hd = 12288, 49152, 96, 128
    gbs, nb, P = 48, 3, 528
    bls, lmax = gbs * nb, P + 16
    W = synth.layer_weights(h1, h2, 0, seed=3, device="cuda", random_ln=True)
    dl = DeviceLayer.from_fp16(W, L.FG_FMT_Q4G64)
    od = oracle.Dims(h1, h2, nh, hd)
    Wq = oracle.quant_layer(od, {k: np16(v) for k, v in W.items()})
    del W
    for name in ("qkv", "o", "1", "2"):
        assert np.array_equal(dl.t["w_" + name].cpu().numpy(), Wq["c_" + name]), name
        assert np.array_equal(np16(dl.t["m_" + name]), Wq["m_" + name]), name
    Wd = oracle.dequant_layer(od, Wq)
    del Wq
    d = L.dims(h1, h2, nh, hd)
    kv = DeviceKV(L.FG_FMT_Q4G64, bls, nh, hd, lmax, "cuda")
    kh, vh = synth.kv_history(bls, nh, P, hd, seed=4, device="cuda")
    for p in range(P):
        L.fg_kv_append_q4(kh[:, p].contiguous(), vh[:, p].contiguous(), h1, kv.struct, bls, d, p)
    sample = np.array([0, 70, bls - 1])
    oc = oracle.KVCache("q4", len(sample), nh, hd, lmax)
    oc.store(np16(kh[sample]), np16(vh[sample]), 0)
    del kh, vh
    x = synth.activations(bls, h1, seed=5, device="cuda")
    x0 = np16(x)[sample]
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    L.fg_layer_decode_block(d, dl.struct, x, gbs, nb, P, kv.struct, ws, ws.numel())
    torch.cuda.synchronize()
    ref, _, _ = oracle.layer_decode(od, Wd, x0, P, oc)
    assert_close(np16(x)[sample], ref, "OPT-175B-shape decode block, sampled sequences")
