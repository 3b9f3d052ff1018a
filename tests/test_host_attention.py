"""Decode attention on the host CPU over an fp16 host cache
(fg_attn_decode_host_f16; [P2] "为什么有时应该在 CPU 上算注意力"): runs here,
with no GPU, against the oracle's attention; the appended row; thread-count
invariance; a slice of the cache's sequences; argument errors."""
import numpy as np
import pytest

import oracle
from helpers import assert_close

CASES = [  # bls, nh, hd, pos
    (1, 1, 64, 0), (2, 3, 64, 1), (2, 3, 64, 17), (3, 2, 128, 130), (4, 8, 64, 527), (2, 2, 128, 1000),
    (1, 2, 128, 8191),   # the longest history a cache of 8192 rows holds
]


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def _cache(L, kc, vc):
    """fg_kv over host tensors (kept alive by the caller)."""
    import torch
    kt, vt = torch.from_numpy(kc), torch.from_numpy(vc)
    kv = L.KV()
    kv.fmt, kv.k, kv.v = L.FG_FMT_F16, kt.data_ptr(), vt.data_ptr()
    kv.k_meta = kv.v_meta = None
    kv.n_seq, _, kv.max_len, _ = kc.shape
    return kv, kt, vt


def _inputs(bls, nh, hd, pos, seed):
    rng = np.random.default_rng(seed)
    h1 = nh * hd
    lmax = pos + 2
    qkv = (rng.standard_normal((bls, 3 * h1)) * 2).astype(np.float16)
    kc = rng.standard_normal((bls, nh, lmax, hd)).astype(np.float16)
    vc = (rng.standard_normal((bls, nh, lmax, hd)) * 2).astype(np.float16)
    return qkv, kc, vc, lmax


@pytest.mark.parametrize("bls,nh,hd,pos", CASES)
def test_host_attention_matches_oracle(L, bls, nh, hd, pos):
    import torch
    h1 = nh * hd
    qkv, kc, vc, lmax = _inputs(bls, nh, hd, pos, seed=pos * 7 + nh)
    ref = oracle.attn_decode(qkv, bls, nh, hd, kc, vc, lmax, pos)
    kv, kt, vt = _cache(L, kc.copy(), vc.copy())
    out = torch.empty((bls, h1), dtype=torch.float16)
    L.fg_attn_decode_host_f16(torch.from_numpy(qkv), 3 * h1, kv, 0, bls, L.dims(h1, 4 * h1, nh, hd), pos, 1,
                              out, n_threads=4)
    assert_close(out.numpy().view(np.uint16), ref.view(np.uint16), f"host attention pos {pos}")
    # the current token's k, v appended at row pos; every other row untouched
    q3 = qkv.reshape(bls, 3, nh, hd)
    got_k, got_v = kt.numpy(), vt.numpy()
    assert np.array_equal(got_k[:, :, pos].view(np.uint16), q3[:, 1].view(np.uint16))
    assert np.array_equal(got_v[:, :, pos].view(np.uint16), q3[:, 2].view(np.uint16))
    rest = [p for p in range(lmax) if p != pos]
    assert np.array_equal(got_k[:, :, rest].view(np.uint16), kc[:, :, rest].view(np.uint16))
    assert np.array_equal(got_v[:, :, rest].view(np.uint16), vc[:, :, rest].view(np.uint16))


def test_host_attention_thread_count_invariant(L):
    """Each (sequence, head) is computed whole by one thread: the bits do not
    depend on how many threads share the work."""
    import torch
    bls, nh, hd, pos = 4, 6, 64, 300
    h1 = nh * hd
    qkv, kc, vc, _ = _inputs(bls, nh, hd, pos, seed=3)
    d = L.dims(h1, 4 * h1, nh, hd)
    outs = []
    for n in (1, 3, 8):
        kv, _kt, _vt = _cache(L, kc.copy(), vc.copy())
        out = torch.empty((bls, h1), dtype=torch.float16)
        L.fg_attn_decode_host_f16(torch.from_numpy(qkv), 3 * h1, kv, 0, bls, d, pos, 0, out, n_threads=n)
        outs.append(out.numpy().view(np.uint16).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_host_attention_sequence_slice_and_row_stride(L):
    """Sequences 1..2 of a 4-sequence cache, q/k/v rows inside wider rows."""
    import torch
    nseq, nh, hd, pos = 4, 2, 128, 40
    h1 = nh * hd
    qkv, kc, vc, lmax = _inputs(nseq, nh, hd, pos, seed=11)
    ld = 3 * h1 + 64
    wide = np.zeros((2, ld), np.float16)
    wide[:, :3 * h1] = qkv[1:3]
    ref = oracle.attn_decode(qkv[1:3], 2, nh, hd, kc[1:3], vc[1:3], lmax, pos)
    kv, kt, _vt = _cache(L, kc.copy(), vc.copy())
    out = torch.empty((2, h1), dtype=torch.float16)
    L.fg_attn_decode_host_f16(torch.from_numpy(wide), ld, kv, 1, 2, L.dims(h1, 4 * h1, nh, hd), pos, 1, out)
    assert_close(out.numpy().view(np.uint16), ref.view(np.uint16), "sequences 1..2")
    got_k = kt.numpy()
    assert np.array_equal(got_k[[0, 3]].view(np.uint16), kc[[0, 3]].view(np.uint16)), "other sequences untouched"


def test_host_attention_argument_errors(L):
    import torch
    nh, hd, pos = 2, 64, 5
    h1 = nh * hd
    qkv, kc, vc, lmax = _inputs(2, nh, hd, pos, seed=1)
    d = L.dims(h1, 4 * h1, nh, hd)
    out = torch.empty((2, h1), dtype=torch.float16)
    q = torch.from_numpy(qkv)
    kv, _kt, _vt = _cache(L, kc.copy(), vc.copy())
    with pytest.raises(L.FgError) as e:
        L.fg_attn_decode_host_f16(q, 3 * h1, kv, 0, 2, d, lmax, 0, out)
    assert e.value.status == L.FG_ERR_INVALID
    with pytest.raises(L.FgError) as e:
        L.fg_attn_decode_host_f16(q, 3 * h1 - 8, kv, 0, 2, d, pos, 0, out)
    assert e.value.status == L.FG_ERR_INVALID
    with pytest.raises(L.FgError) as e:
        L.fg_attn_decode_host_f16(q, 3 * h1, kv, 1, 2, d, pos, 0, out)
    assert e.value.status == L.FG_ERR_INVALID
    kv.fmt = L.FG_FMT_Q4G64
    with pytest.raises(L.FgError) as e:
        L.fg_attn_decode_host_f16(q, 3 * h1, kv, 0, 2, d, pos, 0, out)
    assert e.value.status == L.FG_ERR_UNSUPPORTED
