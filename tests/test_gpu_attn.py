"""GPU parity of the KV append and decode / prefill attention against the oracle.

Cache contents are bit-exact (same fp16 rows quantized by both sides); the
attention outputs meet max|err| <= 1e-2 max|ref| + 1e-3."""
import numpy as np
import pytest

import oracle
from helpers import assert_close, dev16, np16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def _setup(L, fmt, bls, nh, hd, P, lmax, seed):
    """Fill positions 0..P-1 of a device cache and of an oracle cache from the
    same seeded fp16 rows; return both and a fresh (q | k_new | v_new) block."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV
    rng = np.random.default_rng(seed)
    h1 = nh * hd
    d = L.dims(h1, 4 * h1, nh, hd)
    fmt_id = L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16
    kv = DeviceKV(fmt_id, bls, nh, hd, lmax, "cuda")
    kx = (rng.standard_normal((bls, P, h1)) * 2).astype(np.float16)
    vx = (rng.standard_normal((bls, P, h1)) * 2).astype(np.float16)
    append = L.fg_kv_append_q4 if fmt == "q4" else L.fg_kv_append_f16
    kd, vd = dev16(kx), dev16(vx)
    for p in range(P):
        append(kd[:, p].contiguous(), vd[:, p].contiguous(), h1, kv.struct, bls, d, p)
    oc = oracle.KVCache(fmt, bls, nh, hd, lmax)
    if P:
        oc.store(kx, vx, 0)
    qkv = (rng.standard_normal((bls, 3 * h1)) * 2).astype(np.float16)
    return d, kv, oc, qkv


def _cache_equal(kv, oc, upto):
    assert np.array_equal(kv.k.cpu().numpy().view(oc.k.dtype)[:, :, :upto], oc.k[:, :, :upto])
    assert np.array_equal(kv.v.cpu().numpy().view(oc.v.dtype)[:, :, :upto], oc.v[:, :, :upto])
    if oc.km is not None:
        assert np.array_equal(np16(kv.km)[:, :, :upto], oc.km[:, :, :upto])
        assert np.array_equal(np16(kv.vm)[:, :, :upto], oc.vm[:, :, :upto])


CASES = [  # fmt, bls, nh, hd, pos
    ("q4", 1, 1, 128, 0), ("q4", 3, 5, 128, 1), ("q4", 2, 3, 128, 15), ("q4", 2, 2, 128, 16),
    ("q4", 2, 2, 128, 17), ("q4", 1, 3, 128, 64), ("q4", 2, 2, 128, 65), ("q4", 1, 2, 128, 200),
    ("q4", 2, 1, 128, 527), ("q4", 3, 5, 64, 33), ("q4", 2, 12, 64, 39), ("q4", 1, 1, 64, 0),
    ("f16", 2, 3, 128, 0), ("f16", 3, 5, 128, 40), ("f16", 2, 2, 64, 77), ("f16", 1, 32, 64, 130),
    # histories longer than one LDS chunk of scores (8192 positions): running maximum
    ("q4", 1, 2, 64, 8192), ("q4", 1, 2, 128, 8193), ("q4", 2, 1, 64, 17000),
    ("f16", 1, 2, 64, 9000),
]


@pytest.mark.parametrize("fmt,bls,nh,hd,pos", [("q4", 7, 11, 128, 5), ("q4", 9, 15, 64, 2),
                                                 ("f16", 7, 11, 128, 3), ("f16", 5, 13, 64, 0)])
def test_append_one_position_over_many_workgroups(L, fmt, bls, nh, hd, pos):
    """The one-position append takes 16 (head_dim 128) or 32 (64) (sequence,
    head) units per wavefront: with 77 / 135 / 65 units the last workgroup is
    partly empty and its last wavefront ragged.  Row pos of every unit equals
    the oracle's codec bit for bit, and the rows around it keep their
    contents."""
    from throughput_oriented_offloaded_amd.model import DeviceKV
    rng = np.random.default_rng(bls * 100 + nh)
    h1 = nh * hd
    d = L.dims(h1, 4 * h1, nh, hd)
    fmt_id = L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16
    lmax = pos + 2
    kv = DeviceKV(fmt_id, bls, nh, hd, lmax, "cuda")
    oc = oracle.KVCache(fmt, bls, nh, hd, lmax)
    kx = (rng.standard_normal((bls, 1, h1)) * 3).astype(np.float16)
    vx = (rng.standard_normal((bls, 1, h1)) * 3).astype(np.float16)
    append = L.fg_kv_append_q4 if fmt == "q4" else L.fg_kv_append_f16
    # k and v rows inside one wider buffer (row stride 3 h1), as the layer passes them
    qkv = np.zeros((bls, 3 * h1), np.float16)
    qkv[:, h1:2 * h1], qkv[:, 2 * h1:] = kx[:, 0], vx[:, 0]
    buf = dev16(qkv)
    append(buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos)
    oc.store(kx, vx, pos)
    _cache_equal(kv, oc, lmax)          # row pos as the oracle; every other row still zero


@pytest.mark.parametrize("fmt,bls,nh,hd,pos", CASES)
def test_decode_attention_and_append(L, fmt, bls, nh, hd, pos):
    import torch
    lmax = pos + 3
    d, kv, oc, qkv = _setup(L, fmt, bls, nh, hd, pos, lmax, seed=pos * 31 + nh)
    _cache_equal(kv, oc, pos)
    h1 = nh * hd
    buf = dev16(qkv)
    out = torch.empty((bls, h1), dtype=torch.float16, device="cuda")
    fn = L.fg_attn_decode_q4 if fmt == "q4" else L.fg_attn_decode_f16
    fn(buf, buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos, 1, out)
    torch.cuda.synchronize()
    kh, vh = oc.history()
    ref = oracle.attn_decode(qkv, bls, nh, hd, kh, vh, lmax, pos)
    assert_close(np16(out), ref, f"{fmt} attention pos {pos}")
    # the fused append wrote position pos exactly as the codec would
    q3 = qkv.reshape(bls, 1, 3, h1)
    oc.store(q3[:, :, 1], q3[:, :, 2], pos)
    _cache_equal(kv, oc, pos + 1)
    # unfused launch: identical output, cache row pos + 1 left untouched
    out2 = torch.empty_like(out)
    if pos + 1 < lmax:
        before = kv.k[:, :, pos + 1].clone()
        fn(buf, buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos + 1, 0, out2)
        torch.cuda.synchronize()
        assert torch.equal(before, kv.k[:, :, pos + 1])
        kh, vh = oc.history()
        ref2 = oracle.attn_decode(qkv, bls, nh, hd, kh, vh, lmax, pos + 1)
        assert_close(np16(out2), ref2, f"{fmt} attention pos {pos + 1} (unfused)")


def _sampled_check(L, fmt, bls, nh, hd, pos, lmax, seed):
    """Device cache filled by one append per position from synthetic rows on
    the device; the decode launch checked on sampled (sequence, head) pairs."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV
    import synth
    h1 = nh * hd
    d = L.dims(h1, 4 * h1, nh, hd)
    fmt_id = L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16
    append = L.fg_kv_append_q4 if fmt == "q4" else L.fg_kv_append_f16
    attn = L.fg_attn_decode_q4 if fmt == "q4" else L.fg_attn_decode_f16
    kv = DeviceKV(fmt_id, bls, nh, hd, lmax, "cuda")
    kh, vh = synth.kv_history(bls, nh, pos, hd, seed=seed, device="cuda")
    for p in range(pos):   # append every history position (one launch each)
        append(kh[:, p].contiguous(), vh[:, p].contiguous(), h1, kv.struct, bls, d, p)
    qkv = synth.activations(bls, 3 * h1, seed=seed + 1, device="cuda", std=2.0)
    out = torch.empty((bls, h1), dtype=torch.float16, device="cuda")
    attn(qkv, qkv[:, h1:], qkv[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos, 1, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    seqs = sorted(set([0, bls - 1] + list(rng.integers(0, bls, 3))))
    for b in seqs:
        heads = sorted(set([0, nh - 1] + list(rng.integers(0, nh, 3))))
        khb = np16(kh[b]).reshape(pos, nh, hd)[:, heads]          # [pos, H, hd]
        vhb = np16(vh[b]).reshape(pos, nh, hd)[:, heads]
        oc = oracle.KVCache(fmt, 1, len(heads), hd, lmax)
        if pos:
            oc.store(khb.reshape(1, pos, -1), vhb.reshape(1, pos, -1), 0)
        # device cache rows of these heads equal the oracle's
        assert np.array_equal(kv.k[b, heads, :pos].cpu().numpy().view(oc.k.dtype), oc.k[0, :, :pos])
        if fmt == "q4":
            assert np.array_equal(np16(kv.vm[b, heads, :pos]), oc.vm[0, :, :pos])
        q3 = np16(qkv[b]).reshape(3, nh, hd)[:, heads].reshape(1, -1)
        hist = oc.history()
        ref = oracle.attn_decode(q3, 1, len(heads), hd, hist[0], hist[1], lmax, pos)
        got = np16(out[b]).reshape(nh, hd)[heads].reshape(1, -1)
        assert_close(got, ref, f"{fmt} pos {pos} seq {b} heads {heads}")


def test_decode_attention_full_shape_sampled(L):
    """OPT-175B shape (96 heads x 128) at bls = 144, context 528 (s + n/2): the
    launch the benchmark times; sampled (sequence, head) pairs against the oracle."""
    _sampled_check(L, "q4", 144, 96, 128, 528, 544, seed=5)


@pytest.mark.parametrize("fmt,pos", [("q4", 0), ("q4", 37), ("f16", 61), ("q4", 8300), ("f16", 8300),
                                     ("q4", 1)])
def test_decode_attention_one_wave_per_head(L, fmt, pos):
    """2048 (sequence, head) pairs: the launch with two wavefronts per pair for
    the 4-bit cache and one for fp16; short, ragged and multi-chunk histories."""
    _sampled_check(L, fmt, 32, 64, 64, pos, pos + 2, seed=11 + pos)


@pytest.mark.parametrize("b,s,nh,hd", [(1, 1, 1, 128), (2, 5, 3, 128), (1, 64, 2, 128),
                                       (2, 65, 2, 128), (1, 130, 1, 64), (3, 32, 12, 64),
                                       (1, 300, 2, 128)])
def test_prefill_attention(L, b, s, nh, hd):
    import torch
    rng = np.random.default_rng(b * 100 + s)
    h1 = nh * hd
    qkv = (rng.standard_normal((b * s, 3 * h1)) * 2).astype(np.float16)
    out = torch.empty((b * s, h1), dtype=torch.float16, device="cuda")
    L.fg_attn_prefill(dev16(qkv), b, s, L.dims(h1, 4 * h1, nh, hd), out)
    torch.cuda.synchronize()
    assert_close(np16(out), oracle.attn_prefill(qkv, b, s, nh, hd), f"prefill b{b} s{s}")


# ------------------------------------------------------------ Top-K sparse V
SPARSE_CASES = [  # fmt, bls, nh, hd, pos, topk
    ("q4", 1, 1, 128, 0, 0), ("q4", 3, 5, 128, 1, 1), ("q4", 2, 3, 128, 17, 2),
    ("q4", 2, 2, 128, 64, 0), ("q4", 2, 2, 128, 64, 64), ("q4", 2, 2, 128, 200, 20),
    ("q4", 1, 2, 64, 527, 53), ("q4", 2, 3, 64, 130, 13),
    ("f16", 2, 3, 128, 40, 4), ("f16", 1, 4, 64, 130, 13), ("f16", 2, 2, 128, 33, 33),
    # one wavefront per (sequence, head)
    ("q4", 16, 128, 64, 100, 10), ("f16", 16, 128, 64, 70, 7),
]


def _score_gaps(qkv, kh, bls, nh, hd, pos, topk):
    """Smallest gap, over all (sequence, head), between the topk-th and the
    next score (fp64, natural units)."""
    gap = np.inf
    k64 = oracle.to_f16(kh).astype(np.float64)
    for b in range(bls):
        for h in range(nh):
            q = qkv[b, h * hd:(h + 1) * hd].astype(np.float64)
            s = np.sort(k64[b, h, :pos] @ q)[::-1] / np.sqrt(hd)
            gap = min(gap, s[topk - 1] - s[topk])
    return gap


def _setup_ranked(L, fmt, bls, nh, hd, P, lmax, seed):
    """As _setup, with keys c_p u + noise and queries along u (u a random +-1
    vector per head, c_p a random permutation of evenly spaced values): every
    head's scores are spread evenly, so the selection does not depend on the
    score rounding of either side (the 4-bit score path carries absolute
    errors around 1e-4)."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV
    rng = np.random.default_rng(seed)
    h1 = nh * hd
    d = L.dims(h1, 4 * h1, nh, hd)
    fmt_id = L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16
    kv = DeviceKV(fmt_id, bls, nh, hd, lmax, "cuda")
    u = rng.choice([-1.0, 1.0], size=(bls, nh, hd))
    c = np.stack([rng.permutation(P) for _ in range(bls * nh)]).reshape(bls, nh, P) * (3.0 / max(P, 1))
    k = c[..., None] * u[:, :, None, :] + rng.standard_normal((bls, nh, P, hd)) * 1e-3
    kx = k.transpose(0, 2, 1, 3).reshape(bls, P, h1).astype(np.float16)
    vx = (rng.standard_normal((bls, P, h1)) * 2).astype(np.float16)
    append = L.fg_kv_append_q4 if fmt == "q4" else L.fg_kv_append_f16
    kd, vd = dev16(kx), dev16(vx)
    for p in range(P):
        append(kd[:, p].contiguous(), vd[:, p].contiguous(), h1, kv.struct, bls, d, p)
    oc = oracle.KVCache(fmt, bls, nh, hd, lmax)
    if P:
        oc.store(kx, vx, 0)
    qkv = (rng.standard_normal((bls, 3 * h1)) * 2).astype(np.float16)
    qkv[:, :h1] = (u.reshape(bls, h1) * 0.5 + rng.standard_normal((bls, h1)) * 0.01).astype(np.float16)
    return d, kv, oc, qkv


@pytest.mark.parametrize("fmt,bls,nh,hd,pos,topk", SPARSE_CASES)
def test_decode_attention_topk(L, fmt, bls, nh, hd, pos, topk):
    import torch
    lmax = pos + 3
    d, kv, oc, qkv = _setup_ranked(L, fmt, bls, nh, hd, pos, lmax, seed=pos * 17 + nh + topk)
    h1 = nh * hd
    kh, vh = oc.history()
    if 0 < topk < pos:
        assert _score_gaps(qkv, kh, bls, nh, hd, pos, topk) > 2e-3
    buf = dev16(qkv)
    out = torch.empty((bls, h1), dtype=torch.float16, device="cuda")
    fn = L.fg_attn_decode_topk_q4 if fmt == "q4" else L.fg_attn_decode_topk_f16
    fn(buf, buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos, topk, 1, out)
    torch.cuda.synchronize()
    ref = oracle.attn_decode_topk(qkv, bls, nh, hd, kh, vh, lmax, pos, topk)
    assert_close(np16(out), ref, f"{fmt} top-{topk} attention pos {pos}")
    q3 = qkv.reshape(bls, 1, 3, h1)
    oc.store(q3[:, :, 1], q3[:, :, 2], pos)
    _cache_equal(kv, oc, pos + 1)


LONG_SPARSE_CASES = [  # fmt, bls, nh, hd, pos, topk
    # one wavefront per (sequence, head): keys held in registers up to 640
    # positions, counted from LDS beyond
    ("q4", 16, 128, 64, 640, 64), ("q4", 16, 128, 64, 1000, 100),
    # four wavefronts: registers up to 2560 positions, LDS beyond
    ("q4", 1, 2, 128, 2560, 256), ("q4", 1, 2, 128, 3000, 300), ("f16", 2, 3, 64, 2561, 257),
    # the longest history a Top-K launch takes (one chunk of 8192 scores)
    ("q4", 1, 2, 128, 8192, 820), ("f16", 1, 2, 64, 8192, 820), ("f16", 1, 2, 128, 8192, 8191),
]


@pytest.mark.parametrize("fmt,bls,nh,hd,pos,topk", LONG_SPARSE_CASES)
def test_decode_attention_topk_long_history(L, fmt, bls, nh, hd, pos, topk):
    """Histories past the register-held selection (640 positions with one
    wavefront per (sequence, head), 2560 with four) up to the 8192-position
    limit.  Keys c_p u (u a +-1 vector per head, no noise) take 256 evenly
    spaced values c, each on a run of positions: positions of one value have
    identical rows, so their scores tie exactly on both sides and the
    selection inside a run goes to the lower positions; distinct values are
    far apart in score.  The topk counts cut through runs."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV
    rng = np.random.default_rng(pos + topk + nh)
    h1 = nh * hd
    lmax = pos + 3
    d = L.dims(h1, 4 * h1, nh, hd)
    fmt_id = L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16
    kv = DeviceKV(fmt_id, bls, nh, hd, lmax, "cuda")
    u = rng.choice([-1.0, 1.0], size=(bls, nh, hd))
    grid = np.arange(256) * (3.0 / 256) - 1.5          # multiples of 2^-8: exact in fp16
    rep = -(-pos // 256)
    c = np.stack([grid[rng.permutation(pos) // rep] for _ in range(bls * nh)]).reshape(bls, nh, pos)
    k = c[..., None] * u[:, :, None, :]
    kx = k.transpose(0, 2, 1, 3).reshape(bls, pos, h1).astype(np.float16)
    vx = (rng.standard_normal((bls, pos, h1)) * 2).astype(np.float16)
    append = L.fg_kv_append_q4 if fmt == "q4" else L.fg_kv_append_f16
    kd, vd = dev16(kx), dev16(vx)
    for p in range(pos):
        append(kd[:, p].contiguous(), vd[:, p].contiguous(), h1, kv.struct, bls, d, p)
    oc = oracle.KVCache(fmt, bls, nh, hd, lmax)
    oc.store(kx, vx, 0)
    qkv = (rng.standard_normal((bls, 3 * h1)) * 2).astype(np.float16)
    qkv[:, :h1] = (u.reshape(bls, h1) * 0.5).astype(np.float16)
    buf = dev16(qkv)
    out = torch.empty((bls, h1), dtype=torch.float16, device="cuda")
    fn = L.fg_attn_decode_topk_q4 if fmt == "q4" else L.fg_attn_decode_topk_f16
    fn(buf, buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos, topk, 1, out)
    torch.cuda.synchronize()
    kh, vh = oc.history()
    ref = oracle.attn_decode_topk(qkv, bls, nh, hd, kh, vh, lmax, pos, topk)
    assert_close(np16(out), ref, f"{fmt} top-{topk} attention pos {pos}")
    dense = oracle.attn_decode(qkv, bls, nh, hd, kh, vh, lmax, pos)
    if topk < pos - rep:
        err = np.abs(oracle.to_f16(np16(out)).astype(np.float32) - oracle.to_f16(dense).astype(np.float32)).max()
        assert err > 1e-2 * np.abs(oracle.to_f16(dense).astype(np.float32)).max() + 1e-3
    q3 = qkv.reshape(bls, 1, 3, h1)
    oc.store(q3[:, :, 1], q3[:, :, 2], pos)
    _cache_equal(kv, oc, pos + 1)


@pytest.mark.parametrize("fmt", ["q4", "f16"])
def test_decode_attention_topk_ties_take_lowest_positions(L, fmt):
    """Zero keys: every score is equal, and the selection must be the lowest
    positions on both sides."""
    import torch
    from throughput_oriented_offloaded_amd.model import DeviceKV
    bls, nh, hd, pos, topk = 2, 3, 128, 50, 7
    h1 = nh * hd
    lmax = pos + 1
    rng = np.random.default_rng(5)
    d = L.dims(h1, 4 * h1, nh, hd)
    fmt_id = L.FG_FMT_Q4G64 if fmt == "q4" else L.FG_FMT_F16
    kv = DeviceKV(fmt_id, bls, nh, hd, lmax, "cuda")
    oc = oracle.KVCache(fmt, bls, nh, hd, lmax)
    kx = np.zeros((bls, pos, h1), np.float16)
    vx = (rng.standard_normal((bls, pos, h1)) * 2).astype(np.float16)
    append = L.fg_kv_append_q4 if fmt == "q4" else L.fg_kv_append_f16
    kd, vd = dev16(kx), dev16(vx)
    for p in range(pos):
        append(kd[:, p].contiguous(), vd[:, p].contiguous(), h1, kv.struct, bls, d, p)
    oc.store(kx, vx, 0)
    qkv = (rng.standard_normal((bls, 3 * h1)) * 2).astype(np.float16)
    qkv[:, h1:2 * h1] = 0
    buf = dev16(qkv)
    out = torch.empty((bls, h1), dtype=torch.float16, device="cuda")
    fn = L.fg_attn_decode_topk_q4 if fmt == "q4" else L.fg_attn_decode_topk_f16
    fn(buf, buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos, topk, 0, out)
    torch.cuda.synchronize()
    kh, vh = oc.history()
    ref = oracle.attn_decode_topk(qkv, bls, nh, hd, kh, vh, lmax, pos, topk)
    assert_close(np16(out), ref, f"{fmt} top-{topk} ties")


def test_decode_attention_topk_all_equals_dense(L):
    """topk = pos takes the sparse kernel through every V row: same result as
    the dense kernel within rounding."""
    import torch
    fmt, bls, nh, hd, pos = "q4", 4, 8, 128, 300
    d, kv, oc, qkv = _setup(L, fmt, bls, nh, hd, pos, pos + 1, seed=77)
    h1 = nh * hd
    buf = dev16(qkv)
    a = torch.empty((bls, h1), dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    L.fg_attn_decode_q4(buf, buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos, 0, a)
    L.fg_attn_decode_topk_q4(buf, buf[:, h1:], buf[:, 2 * h1:], 3 * h1, kv.struct, bls, d, pos, pos, 0, b)
    torch.cuda.synchronize()
    assert_close(np16(b), np16(a), "top-pos vs dense")
