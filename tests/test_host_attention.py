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


# ------------------------------------------------------------ 4-bit caches
Q4_CASES = [  # bls, nh, hd, pos
    (1, 1, 64, 0), (2, 3, 64, 17), (3, 2, 128, 130), (4, 8, 64, 527), (2, 2, 128, 1000), (1, 2, 128, 4000),
]


def _q4_cache(L, kc16, vc16):
    """The oracle's codec over fp16 histories [b, nh, lmax, hd] (groups of 64
    along hd), as an fg_kv of host tensors, and the dequantized fp16
    histories the oracle attends over."""
    import torch
    b, nh, lmax, hd = kc16.shape
    out = []
    for h in (kc16, vc16):
        codes, meta = oracle.quant_g4(h.reshape(-1), b * nh * lmax, hd, 1)
        deq = oracle.dequant_g4(codes, meta, b * nh * lmax, hd, 1).reshape(b, nh, lmax, hd)
        out.append((torch.from_numpy(codes.reshape(b, nh, lmax, hd // 2).copy()),
                    torch.from_numpy(meta.reshape(b, nh, lmax, hd // 64, 2).view(np.int16).copy()), deq))
    (kt, kmt, kdq), (vt, vmt, vdq) = out
    kv = L.KV()
    kv.fmt, kv.k, kv.v, kv.k_meta, kv.v_meta = L.FG_FMT_Q4G64, kt.data_ptr(), vt.data_ptr(), kmt.data_ptr(), vmt.data_ptr()
    kv.n_seq, kv.max_len = b, lmax
    return kv, (kt, kmt, vt, vmt), kdq, vdq


@pytest.mark.parametrize("bls,nh,hd,pos,mode", [c + ("native",) for c in Q4_CASES] +
                         [c + (m,) for c in Q4_CASES[:4] for m in ("avx2", "scalar")])
def test_host_attention_q4_matches_oracle(L, bls, nh, hd, pos, mode):
    """A 4-bit cache (the oracle's codec) attended on the host against the
    oracle's attention over the dequantized fp16 history, in the widest items
    the host has (AVX-512 or AVX2), in the AVX2 ones and in the plain C++ ones
    (child processes with FG_HOST_ATTN_AVX2=1 or FG_HOST_ATTN_SCALAR=1), and
    the appended row: the codec's bytes for the fresh k, v."""
    if mode != "native":
        import subprocess
        import sys
        env = dict(__import__("os").environ, **{"FG_HOST_ATTN_" + mode.upper(): "1"})
        node = f"{__file__}::test_host_attention_q4_matches_oracle[{bls}-{nh}-{hd}-{pos}-native]"
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", node],
                           env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
        assert "1 passed" in r.stdout
        return
    import torch
    h1 = nh * hd
    qkv, kc, vc, lmax = _inputs(bls, nh, hd, pos, seed=pos * 5 + hd)
    kv, keep, kdq, vdq = _q4_cache(L, kc.view(np.uint16), vc.view(np.uint16))
    ref = oracle.attn_decode(qkv, bls, nh, hd, kdq, vdq, lmax, pos)
    out = torch.empty((bls, h1), dtype=torch.float16)
    L.fg_attn_decode_host_q4(torch.from_numpy(qkv), 3 * h1, kv, 0, bls, L.dims(h1, 4 * h1, nh, hd), pos, 1,
                             out, n_threads=4)
    assert_close(out.numpy().view(np.uint16), ref.view(np.uint16), f"4-bit host attention pos {pos}")
    # row pos holds the codec's bytes of the fresh k and v; the other rows are untouched
    q3 = qkv.reshape(bls, 3, nh, hd).view(np.uint16)
    kt, kmt, vt, vmt = keep
    for t, (codes_t, meta_t) in enumerate(((kt, kmt), (vt, vmt))):
        c_ref, m_ref = oracle.quant_g4(np.ascontiguousarray(q3[:, 1 + t]).reshape(-1), bls * nh, hd, 1)
        assert np.array_equal(codes_t.numpy()[:, :, pos].reshape(-1), c_ref.reshape(-1)), "appended codes"
        assert np.array_equal(meta_t.numpy()[:, :, pos].view(np.uint16).reshape(-1), m_ref.reshape(-1)), "appended meta"


def test_host_q4_append_special_groups(L):
    """The CPU quantizer of the append on the codec's special cases: a
    constant group (codes 0, scale 0), a group of -0 and +0, a group whose
    values sit halfway between codes (ties to even), and extreme fp16 values:
    bytes equal the oracle codec's."""
    import torch
    nh, hd, pos, lmax = 4, 64, 3, 8
    h1 = nh * hd
    qkv = np.zeros((1, 3 * h1), np.float16)
    k = qkv[0, h1:2 * h1].reshape(nh, hd)
    k[0] = 1.5                                              # constant
    k[1] = np.where(np.arange(hd) % 2 == 0, -0.0, 0.0)     # signed zeros
    k[2] = (np.arange(hd) % 31) * 0.5                       # range 15: codes at halves -> ties
    k[3] = np.where(np.arange(hd) % 3 == 0, 65504.0, -65504.0)
    qkv[0, 2 * h1:] = qkv[0, h1:2 * h1]
    kc = np.zeros((1, nh, lmax, hd), np.uint16)
    kv, keep, _, _ = _q4_cache(L, kc, kc.copy())
    out = torch.empty((1, h1), dtype=torch.float16)
    L.fg_attn_decode_host_q4(torch.from_numpy(qkv), 3 * h1, kv, 0, 1, L.dims(h1, 4 * h1, nh, hd), pos, 1, out)
    c_ref, m_ref = oracle.quant_g4(np.ascontiguousarray(k).view(np.uint16).reshape(-1), nh, hd, 1)
    kt, kmt, _, _ = keep
    assert np.array_equal(kt.numpy()[0, :, pos].reshape(-1), c_ref.reshape(-1))
    assert np.array_equal(kmt.numpy()[0, :, pos].view(np.uint16).reshape(-1), m_ref.reshape(-1))


def test_host_attention_q4_thread_count_invariant(L):
    import torch
    bls, nh, hd, pos = 3, 4, 128, 200
    h1 = nh * hd
    qkv, kc, vc, _ = _inputs(bls, nh, hd, pos, seed=21)
    d = L.dims(h1, 4 * h1, nh, hd)
    outs = []
    for n in (1, 5):
        kv, _keep, _, _ = _q4_cache(L, kc.view(np.uint16), vc.view(np.uint16))
        out = torch.empty((bls, h1), dtype=torch.float16)
        L.fg_attn_decode_host_q4(torch.from_numpy(qkv), 3 * h1, kv, 0, bls, d, pos, 0, out, n_threads=n)
        outs.append(out.numpy().view(np.uint16).copy())
    assert np.array_equal(outs[0], outs[1])


def test_host_attention_format_mismatch(L):
    """Each entry point takes its own cache format only."""
    import torch
    nh, hd, pos = 2, 64, 5
    h1 = nh * hd
    qkv, kc, vc, _ = _inputs(2, nh, hd, pos, seed=2)
    d = L.dims(h1, 4 * h1, nh, hd)
    out = torch.empty((2, h1), dtype=torch.float16)
    kv, _keep, _, _ = _q4_cache(L, kc.view(np.uint16), vc.view(np.uint16))
    with pytest.raises(L.FgError) as e:
        L.fg_attn_decode_host_f16(torch.from_numpy(qkv), 3 * h1, kv, 0, 2, d, pos, 0, out)
    assert e.value.status == L.FG_ERR_UNSUPPORTED
    kv16, _kt, _vt = _cache(L, kc.copy(), vc.copy())
    with pytest.raises(L.FgError) as e:
        L.fg_attn_decode_host_q4(torch.from_numpy(qkv), 3 * h1, kv16, 0, 2, d, pos, 0, out)
    assert e.value.status == L.FG_ERR_UNSUPPORTED
    kv.k_meta = None
    with pytest.raises(L.FgError) as e:
        L.fg_attn_decode_host_q4(torch.from_numpy(qkv), 3 * h1, kv, 0, 2, d, pos, 0, out)
    assert e.value.status == L.FG_ERR_INVALID


@pytest.mark.parametrize("bls,nh,hd,pos", [(2, 3, 64, 17), (3, 2, 128, 130)])
def test_host_attention_scalar_items(bls, nh, hd, pos):
    """The plain C++ fp16 items (FG_HOST_ATTN_SCALAR=1, in a child process)
    against the oracle, as the AVX2 ones are."""
    import os
    import subprocess
    import sys
    env = dict(os.environ, FG_HOST_ATTN_SCALAR="1")
    node = f"{__file__}::test_host_attention_matches_oracle[{bls}-{nh}-{hd}-{pos}]"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", node],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "1 passed" in r.stdout
