"""KV-cache tiering on the GPU: the caches of some GPU batches live in pinned
host memory and pass through two device slots ("FlexGen 完全拆解", sections
"三条关键数据通路如何重叠" and "一个层级流水的伪代码": load_cache /
store_cache around each GPU batch).  The tiered path runs the same kernels as
the all-device one on the same data, so its results must agree bit for bit:
the layer output, the host cache rows (history and appended position), and
whole generations; one case is also held against the oracle.

Shapes keep every attention launch below 2048 (sequence, head) pairs, where
the kernel's work split does not depend on the number of sequences, so a
batch run alone sums in the same order as the whole block."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, np16

pytestmark = pytest.mark.gpu

OPT125 = dict(h1=768, h2=3072, nh=12, hd=64)


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def _fmt(L, f):
    return L.FG_FMT_Q4G64 if f == "q4" else L.FG_FMT_F16


def _tensors(kv):
    return [t for t in (kv.k, kv.v, kv.km, kv.vm) if t is not None]


def _filled_cache(L, kvfmt, bls, P, lmax, seed):
    """Device cache of bls sequences with P appended positions."""
    from throughput_oriented_offloaded_amd.model import DeviceKV
    h1, nh, hd = OPT125["h1"], OPT125["nh"], OPT125["hd"]
    kv = DeviceKV(_fmt(L, kvfmt), bls, nh, hd, lmax, "cuda")
    d = L.dims(h1, OPT125["h2"], nh, hd)
    kh, vh = synth.kv_history(bls, nh, P, hd, seed=seed)
    app = L.fg_kv_append_q4 if kvfmt == "q4" else L.fg_kv_append_f16
    khd, vhd = kh.cuda(), vh.cuda()
    for p in range(P):
        app(khd[:, p].contiguous(), vhd[:, p].contiguous(), h1, kv.struct, bls, d, p)
    return kv, d, kh, vh


def _split(L, kv, kvfmt, n_dev, bls, lmax):
    """The same cache split: sequences [0, n_dev) on a device cache, the rest
    in a pinned host cache."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV
    nh, hd = OPT125["nh"], OPT125["hd"]
    dev = DeviceKV(_fmt(L, kvfmt), max(n_dev, 1), nh, hd, lmax, "cuda")
    host = DeviceKV(_fmt(L, kvfmt), bls - n_dev, nh, hd, lmax, "pinned")
    for a, dd, hh in zip(_tensors(kv), _tensors(dev), _tensors(host)):
        if n_dev:
            dd.copy_(a[:n_dev])
        hh.copy_(a[n_dev:])
    torch.cuda.synchronize()
    return dev, host


def _tier(L, d, gbs, lmax, kvfmt):
    import torch
    sb = L.fg_kvtier_slot_bytes(d, gbs, lmax, _fmt(L, kvfmt))
    slots = torch.empty(2 * sb, dtype=torch.uint8, device="cuda")
    cp = torch.cuda.Stream()
    return L.fg_kvtier_create(slots, sb, cp), slots, cp


@pytest.mark.parametrize("kvfmt", ["q4", "f16"])
@pytest.mark.parametrize("nb_dev", [0, 1, 2])
@pytest.mark.parametrize("P,ppm", [(0, 0), (7, 0), (40, 0), (40, 100000)])
def test_layer_decode_kv_tier_bit_exact(L, kvfmt, nb_dev, P, ppm):
    """fg_layer_decode_block with batches nb_dev.. on the host against the
    all-device call: same output, and the host cache equals the device cache's
    rows 0..P (history untouched, position P appended) bit for bit."""
    import torch
    from test_gpu_layer import _layer
    gbs, nb, lmax = 3, 3, 48
    bls = gbs * nb
    dl, _, _ = _layer(L, OPT125, "q4", seed=51)
    kv, d, _, _ = _filled_cache(L, kvfmt, bls, P, lmax, seed=52)
    dev, host = _split(L, kv, kvfmt, nb_dev * gbs, bls, lmax)
    x = synth.activations(bls, OPT125["h1"], seed=53).cuda()
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    x_ref = x.clone()
    L.fg_layer_decode_block(d, dl.struct, x_ref, gbs, nb, P, kv.struct, ws, ws.numel(),
                            attn_topk_ppm=ppm)
    torch.cuda.synchronize()
    kt, slots, cp = _tier(L, d, gbs, lmax, kvfmt)
    try:
        t = L.KvTier(kt, _ptr_kv(L, host), nb_dev)
        x_t = x.clone()
        L.fg_layer_decode_block(d, dl.struct, x_t, gbs, nb, P, dev.struct, ws, ws.numel(),
                                attn_topk_ppm=ppm, kvt=t)
        torch.cuda.synchronize()
        cp.synchronize()
    finally:
        L.fg_kvtier_destroy(kt)
    assert torch.equal(x_t, x_ref)
    n_dev = nb_dev * gbs
    for a, dd, hh in zip(_tensors(kv), _tensors(dev), _tensors(host)):
        assert torch.equal(hh[:, :, :P + 1], a[n_dev:, :, :P + 1].cpu())
        if n_dev:
            assert torch.equal(dd[:n_dev, :, :P + 1], a[:n_dev, :, :P + 1])


def _ptr_kv(L, host):
    import ctypes
    return ctypes.pointer(host.struct)


def test_layer_decode_kv_tier_matches_oracle(L):
    """Two of three GPU batches on the host, 4-bit weights and cache, against
    the oracle's layer (max|err| <= 1e-2 max|ref| + 1e-3)."""
    import torch
    from test_gpu_layer import _layer
    gbs, nb, lmax, P = 2, 3, 24, 17
    bls = gbs * nb
    dl, Wn, od = _layer(L, OPT125, "q4", seed=61)
    kv, d, kh, vh = _filled_cache(L, "q4", bls, P, lmax, seed=62)
    dev, host = _split(L, kv, "q4", gbs, bls, lmax)
    x = synth.activations(bls, OPT125["h1"], seed=63)
    xd = x.cuda()
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    kt, slots, cp = _tier(L, d, gbs, lmax, "q4")
    try:
        L.fg_layer_decode_block(d, dl.struct, xd, gbs, nb, P, dev.struct, ws, ws.numel(),
                                kvt=L.KvTier(kt, _ptr_kv(L, host), 1))
        torch.cuda.synchronize()
        cp.synchronize()
    finally:
        L.fg_kvtier_destroy(kt)
    oc = oracle.KVCache("q4", bls, OPT125["nh"], OPT125["hd"], lmax)
    oc.store(kh.numpy().view(np.uint16), vh.numpy().view(np.uint16), 0)
    ref, _, _ = oracle.layer_decode(od, Wn, x.numpy().view(np.uint16), P, oc)
    assert_close(np16(xd), ref, "KV-tiered decode block")
    assert np.array_equal(host.k[:, :, :P].numpy(), oc.k[gbs:, :, :P])


@pytest.mark.parametrize("kv_host_seqs,gbs,nb,topk", [(4, 2, 3, 0.0), (6, 2, 3, 0.0), (3, 3, 2, 0.0),
                                                       (4, 2, 3, 0.1)])
def test_model_generation_kv_tier_bit_exact(L, kv_host_seqs, gbs, nb, topk):
    """2-layer OPT-125m-shape model, prefill s = 20 and 5 decode steps, with
    the last kv_host_seqs sequences' caches in pinned host memory: tokens,
    every step's logits and the caches equal the all-device model's.  The
    loads cross layer boundaries (one host batch of layer 0 is followed by
    layer 1's) and the slots are reused across calls.  topk: the same with
    Top-K sparse V at that fraction on both models."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape
    sh = Shape(n_layers=2, h1=768, h2=3072, n_heads=12, head_dim=64)
    bls, s, n = gbs * nb, 20, 6
    Ws = [synth.layer_weights(sh.h1, sh.h2, j, seed=0) for j in range(sh.n_layers)]
    emb = synth.embeddings(sh.h1, s + n, seed=0)
    toks = synth.tokens(bls, s, seed=3).cuda()
    layers = [DeviceLayer.from_fp16({k: v.cuda() for k, v in W.items()}, L.FG_FMT_Q4G64) for W in Ws]
    embd = {k: v.cuda() for k, v in emb.items()}
    ref = Model(sh, layers, embd, L.FG_FMT_Q4G64, bls, s + n, attn_topk=topk)
    tr = Model(sh, layers, embd, L.FG_FMT_Q4G64, bls, s + n, kv_host_seqs=kv_host_seqs,
               attn_topk=topk)
    out_r, lg_r = ref.generate(toks, n, gbs=gbs, nb=nb)
    out_t, lg_t = tr.generate(toks, n, gbs=gbs, nb=nb)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_t)
    for a, b in zip(lg_r, lg_t):
        assert torch.equal(a, b)
    n_dev = bls - kv_host_seqs
    for j in range(sh.n_layers):
        for a, dd, hh in zip(_tensors(ref.kv[j]), _tensors(tr.kv[j]), _tensors(tr.kv_host[j])):
            assert torch.equal(hh[:, :, :s + n - 1], a[n_dev:, :, :s + n - 1].cpu())
            if n_dev:
                assert torch.equal(dd[:, :, :s + n - 1], a[:n_dev, :, :s + n - 1])


# ------------------------------------------------ attention on the host CPU
def _host_attn_tier(L, d, gbs, lmax, n_host_seq, threads=4):
    """A tier whose decode calls compute the host batches' attention on the
    CPU (fp16 cache), with its pinned stage."""
    import torch
    kt, slots, cp = _tier(L, d, gbs, lmax, "f16")
    hb = L.fg_kvtier_host_stage_bytes(d, n_host_seq)
    stage = torch.empty(hb, dtype=torch.uint8, pin_memory=True)
    L.fg_kvtier_host_attention(kt, stage, hb, threads)
    return kt, slots, cp, stage


@pytest.mark.parametrize("fmt", ["f16", "q4"])
@pytest.mark.parametrize("nb_dev,P", [(0, 17), (1, 17), (2, 40), (1, 0)])
def test_layer_decode_host_attention(L, nb_dev, P, fmt):
    """fg_layer_decode_block with the host batches' attention on the CPU
    ([P2] "为什么有时应该在 CPU 上算注意力"; fp16 and 4-bit caches): the layer
    output against the oracle and against the all-device call (the CPU's
    roundings differ, so within the tolerance), the device batches' rows bit
    for bit, and the host cache: history untouched, row P the fresh k, v, bit
    for bit equal to what the all-device call appended (for the 4-bit cache:
    the CPU's quantizer gives the device quantizer's bytes)."""
    import torch
    from test_gpu_layer import _layer
    gbs, nb, lmax = 2, 3, 48
    bls = gbs * nb
    dl, Wn, od = _layer(L, OPT125, "q4", seed=71)
    kv, d, kh, vh = _filled_cache(L, fmt, bls, P, lmax, seed=72)
    dev, host = _split(L, kv, fmt, nb_dev * gbs, bls, lmax)
    x = synth.activations(bls, OPT125["h1"], seed=73)
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    x_ref = x.cuda()
    L.fg_layer_decode_block(d, dl.struct, x_ref, gbs, nb, P, kv.struct, ws, ws.numel())
    torch.cuda.synchronize()
    kt, slots, cp, stage = _host_attn_tier(L, d, gbs, lmax, (nb - nb_dev) * gbs)
    try:
        x_h = x.cuda()
        L.fg_layer_decode_block(d, dl.struct, x_h, gbs, nb, P, dev.struct, ws, ws.numel(),
                                kvt=L.KvTier(kt, _ptr_kv(L, host), nb_dev))
        torch.cuda.synchronize()
    finally:
        L.fg_kvtier_destroy(kt)
    oc = oracle.KVCache(fmt, bls, OPT125["nh"], OPT125["hd"], lmax)
    if P:
        oc.store(kh.numpy().view(np.uint16), vh.numpy().view(np.uint16), 0)
    ref, _, _ = oracle.layer_decode(od, Wn, x.numpy().view(np.uint16), P, oc)
    assert_close(np16(x_h), ref, "host-attention decode block vs oracle")
    assert_close(np16(x_h), np16(x_ref), "host-attention decode block vs all-device")
    n_dev = nb_dev * gbs
    if n_dev:
        assert torch.equal(x_h[:n_dev], x_ref[:n_dev])
    for a, hh in zip(_tensors(kv), _tensors(host)):
        assert torch.equal(hh[:, :, :P + 1], a[n_dev:, :, :P + 1].cpu())


@pytest.mark.parametrize("host_batches,kv_fmt", [(1, "f16"), (2, "f16"), (3, "f16"), (2, "q4"), (3, "q4")])
def test_model_decode_host_attention(L, host_batches, kv_fmt):
    """2-layer OPT-125m-shape model, fp16 weights, an fp16 or 4-bit cache, one,
    two or all three GPU batches' caches on the host: the prefill goes through the slots,
    the decode steps' host attention runs on the CPU, overlapped with the GPU's
    work on the other rows (a device lane of the remaining batches, one or
    two host lanes).  Teacher-forced on the all-device model's tokens, every
    decode step's logits agree within the tolerance and the host caches hold
    the same rows."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape
    sh = Shape(n_layers=2, h1=768, h2=3072, n_heads=12, head_dim=64)
    gbs, nb, s, n = 2, 3, 20, 5
    bls = gbs * nb
    Ws = [synth.layer_weights(sh.h1, sh.h2, j, seed=0) for j in range(sh.n_layers)]
    emb = synth.embeddings(sh.h1, s + n, seed=0)
    toks = synth.tokens(bls, s, seed=5).cuda()
    layers = [DeviceLayer.from_fp16({k: v.cuda() for k, v in W.items()}, L.FG_FMT_F16) for W in Ws]
    embd = {k: v.cuda() for k, v in emb.items()}
    kf = L.FG_FMT_F16 if kv_fmt == "f16" else L.FG_FMT_Q4G64
    ref = Model(sh, layers, embd, kf, bls, s + n)
    ha = Model(sh, layers, embd, kf, bls, s + n, kv_host_seqs=host_batches * gbs,
               kv_host_attention=True, host_threads=4)
    lg_r, tok_r = ref.prefill(toks, gbs, nb)
    lg_h, tok_h = ha.prefill(toks, gbs, nb)
    assert torch.equal(lg_r, lg_h)
    tok = tok_r
    for i in range(n - 1):
        lg_r, nxt = ref.decode_step(tok, s + i, gbs, nb)
        lg_h, _ = ha.decode_step(tok, s + i, gbs, nb)
        torch.cuda.synchronize()
        assert_close(np16(lg_h), np16(lg_r), f"decode step {i} logits")
        tok = nxt
    n_dev = bls - host_batches * gbs
    for j in range(sh.n_layers):
        for a, hh in zip(_tensors(ref.kv[j]), _tensors(ha.kv_host[j])):
            assert torch.equal(hh[:, :, :s], a[n_dev:, :, :s].cpu())
            if kv_fmt == "q4":   # decode rows: codes of nearly equal k, v (rounding differs)
                continue
            got = hh[:, :, s:s + n - 1].float()
            want = a[n_dev:, :, s:s + n - 1].float().cpu()
            assert (got - want).abs().max() <= 1e-2 * want.abs().max() + 1e-3


def test_host_attention_refusals(L):
    """Top-K sparse V (over either cache format), a small stage, an unpinned
    stage: refused on the host before anything is enqueued."""
    import torch
    from test_gpu_layer import _layer
    gbs, nb, lmax, P = 2, 2, 24, 9
    bls = gbs * nb
    dl, _, _ = _layer(L, OPT125, "q4", seed=81)
    d = L.dims(OPT125["h1"], OPT125["h2"], OPT125["nh"], OPT125["hd"])
    x = synth.activations(bls, OPT125["h1"], seed=82).cuda()
    ws = torch.empty(L.fg_workspace_bytes(d, bls, dl.fmt), dtype=torch.uint8, device="cuda")
    kv16, _, _, _ = _filled_cache(L, "f16", bls, P, lmax, seed=83)
    dev16_, host16 = _split(L, kv16, "f16", gbs, bls, lmax)
    kvq, _, _, _ = _filled_cache(L, "q4", bls, P, lmax, seed=84)
    devq, hostq = _split(L, kvq, "q4", gbs, bls, lmax)
    x0 = x.clone()
    kt, slots, cp, stage = _host_attn_tier(L, d, gbs, lmax, gbs)
    try:
        with pytest.raises(L.FgError) as e:
            L.fg_layer_decode_block(d, dl.struct, x, gbs, nb, P, devq.struct, ws, ws.numel(),
                                    attn_topk_ppm=100000, kvt=L.KvTier(kt, _ptr_kv(L, hostq), 1))
        assert e.value.status == L.FG_ERR_UNSUPPORTED
        with pytest.raises(L.FgError) as e:
            L.fg_layer_decode_block(d, dl.struct, x, gbs, nb, P, dev16_.struct, ws, ws.numel(),
                                    attn_topk_ppm=100000, kvt=L.KvTier(kt, _ptr_kv(L, host16), 1))
        assert e.value.status == L.FG_ERR_UNSUPPORTED
        small = torch.empty(256, dtype=torch.uint8, pin_memory=True)
        L.fg_kvtier_host_attention(kt, small, 256, 2)
        with pytest.raises(L.FgError) as e:
            L.fg_layer_decode_block(d, dl.struct, x, gbs, nb, P, dev16_.struct, ws, ws.numel(),
                                    kvt=L.KvTier(kt, _ptr_kv(L, host16), 1))
        assert e.value.status == L.FG_ERR_CAPACITY
        plain = torch.empty(1 << 20, dtype=torch.uint8)
        with pytest.raises(L.FgError) as e:
            L.fg_kvtier_host_attention(kt, plain, plain.numel(), 2)
        assert e.value.status == L.FG_ERR_INVALID
        torch.cuda.synchronize()
    finally:
        L.fg_kvtier_destroy(kt)
    assert torch.equal(x, x0), "refused calls must not touch x"
