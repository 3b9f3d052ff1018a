"""Weight tiering (half of each fp16 layer in pinned host memory, staged on a
side stream by the library's block schedule): the tiered model must produce
exactly the tokens and logits of the fully resident one (same kernels on the
same weight bytes), over prefill and several decode steps, for every pattern
of tiered layers; and the resident fp16 model itself is checked against the
oracle in test_gpu_layer.py."""
import numpy as np
import pytest

import synth
from helpers import assert_close, np16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def _models(L, pattern, n_layers=3):
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape, TierLayer
    sh = Shape(n_layers=n_layers, h1=768, h2=3072, n_heads=12, head_dim=64)
    bls, s, n = 4, 32, 5
    Ws = [{k: v.cuda() for k, v in synth.layer_weights(sh.h1, sh.h2, j, seed=3).items()}
          for j in range(sh.n_layers)]
    emb = {k: v.cuda() for k, v in synth.embeddings(sh.h1, s + n, seed=3).items()}
    f16 = L.FG_FMT_F16
    res = Model(sh, [DeviceLayer.from_fp16(W, f16) for W in Ws], emb, L.FG_FMT_Q4G64, bls, s + n)
    layers, tier = [], []
    for j, W in enumerate(Ws):
        if pattern[j]:
            dl, tl = TierLayer.split(W, f16)
            layers.append(dl)
            tier.append(tl)
        else:
            layers.append(DeviceLayer.from_fp16(W, f16))
            tier.append(None)
    tiered = Model(sh, layers, emb, L.FG_FMT_Q4G64, bls, s + n, tier=tier)
    toks = synth.tokens(bls, s, seed=3).cuda()
    return res, tiered, toks, n, bls


@pytest.mark.parametrize("pattern", [(1, 1, 1), (1, 0, 1), (0, 1, 0), (1, 1, 0)])
def test_tiered_model_matches_resident(L, pattern):
    import torch
    res, tiered, toks, n, bls = _models(L, pattern)
    out_r, lg_r = res.generate(toks, n, gbs=2, nb=2)
    out_t, lg_t = tiered.generate(toks, n, gbs=2, nb=2)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_t)
    for a, b in zip(lg_r, lg_t):
        assert torch.equal(a, b)
    # the staged buffers really carry the host halves: after the run, the
    # first tiered layer's stage (buffer 0, staged for a next pass) holds them
    first = next(j for j, p in enumerate(pattern) if p)
    t = tiered.tier[first]
    h1 = t.v_dev.shape[0]
    stage = tiered._stage[: L.fg_stage_bytes(tiered.d)].view(torch.float16)
    qkv = stage[: 3 * h1 * h1].view(3 * h1, h1)
    assert torch.equal(qkv[: 2 * h1].cpu(), t.qk_host)
    assert torch.equal(qkv[2 * h1:], t.v_dev)


def test_tiering_rejects_pageable_host_memory(L):
    import torch
    from throughput_oriented_offloaded_amd.model import Model
    res, tiered, toks, n, bls = _models(L, (1, 0, 0))
    t = tiered.tier[0]
    t.qk_host = t.qk_host.clone()            # pageable copy: must be refused
    t.struct.qk_host = L.ptr(t.qk_host)
    tiered._tier_arr[0] = t.struct
    with pytest.raises(L.FgError) as e:
        tiered.generate(toks, 2, gbs=4, nb=1)
    assert e.value.status == L.FG_ERR_INVALID and "pinned" in str(e.value)


def test_weight_and_kv_tiering_together(L):
    """Weight tiering (host halves of layers 0 and 2) and KV tiering (the last
    GPU batch's cache in pinned host memory) in one model, each on its own
    copy stream: tokens and logits equal the fully resident model's."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape, TierLayer
    res, _, toks, n, bls = _models(L, (1, 0, 1))
    sh = res.shape
    s = toks.shape[1]
    Ws = [{k: v.cuda() for k, v in synth.layer_weights(sh.h1, sh.h2, j, seed=3).items()}
          for j in range(sh.n_layers)]
    layers, tier = [], []
    for j, W in enumerate(Ws):
        if j != 1:
            dl, tl = TierLayer.split(W, L.FG_FMT_F16)
            layers.append(dl)
            tier.append(tl)
        else:
            layers.append(DeviceLayer.from_fp16(W, L.FG_FMT_F16))
            tier.append(None)
    both = Model(sh, layers, res.emb, L.FG_FMT_Q4G64, bls, s + n, tier=tier, kv_host_seqs=2)
    out_r, lg_r = res.generate(toks, n, gbs=2, nb=2)
    out_b, lg_b = both.generate(toks, n, gbs=2, nb=2)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_b)
    for a, b in zip(lg_r, lg_b):
        assert torch.equal(a, b)
