"""Host-side checks of the C ABI (no GPU work): the library loads and exports
every function include/fg.h declares; the closed-form sizes equal the pages'
formulas; bad arguments are rejected on the host before any launch."""
import ctypes

import pytest

import oracle


@pytest.fixture(scope="module")
def L():
    from throughput_oriented_offloaded_amd import _lib
    return _lib


def test_exports_every_declared_symbol(L):
    declared = L.header_symbols()
    assert len(declared) >= 20
    missing = [n for n in declared if n not in L.exported_symbols()]
    assert not missing, missing
    for name in ("fg_quant_group4", "fg_dequant_group4", "fg_layer_prefill",
                 "fg_layer_decode_block", "fg_kv_append_q4", "fg_attn_decode_q4"):
        assert name in declared
    assert L.raw("fg_abi_version")() == 3


def test_status_strings(L):
    assert L.status_str(0) == "ok"
    assert L.status_str(-1) == "invalid argument"
    assert L.status_str(-3) == "capacity exceeded"
    assert L.status_str(99) == "unknown status"


@pytest.mark.parametrize("h1,h2,nh,hd,l", [(768, 3072, 12, 64, 2), (2048, 8192, 32, 64, 24),
                                           (7168, 28672, 56, 128, 48), (9216, 36864, 72, 128, 64),
                                           (12288, 49152, 96, 128, 96)])
def test_size_closed_forms(L, h1, h2, nh, hd, l):
    d = L.dims(h1, h2, nh, hd)
    f16 = L.fg_weight_bytes(d, l, L.FG_FMT_F16)
    assert f16 == oracle.weight_bytes_f16(h1, h2, l)
    assert L.fg_weight_bytes(d, l, L.FG_FMT_Q4G64) * 32 == f16 * 9
    for bls, s, n in ((144, 512, 32), (512, 512, 32), (4, 32, 8)):
        kv = L.fg_kv_bytes(d, l, bls, s, n, L.FG_FMT_F16)
        assert kv == oracle.kv_bytes_f16(h1, l, bls, s, n)
        assert L.fg_kv_bytes(d, l, bls, s, n, L.FG_FMT_Q4G64) * 32 == kv * 9


def test_175b_q4_weights_fit_in_hbm(L):
    """The 4-bit OPT-175B weights (~98 GB) and the 4-bit KV of bls = 144 at
    s + n = 544 (~104 GB) fit together in 288 GB of HBM."""
    d = L.dims(12288, 49152, 96, 128)
    w = L.fg_weight_bytes(d, 96, L.FG_FMT_Q4G64)
    kv = L.fg_kv_bytes(d, 96, 144, 512, 32, L.FG_FMT_Q4G64)
    codes_only = 96 * (4 * 12288 ** 2 + 2 * 12288 * 49152) // 2
    assert abs(codes_only / 1e9 - 88) < 1.5          # "~88 GB" of codes (86.97)
    assert w + kv < 288e9 * 0.75


def _bad(L, name, *args):
    st = L.raw(name)(*args)
    return st, L.last_error()


def test_codec_rejects_bad_arguments(L):
    st, msg = _bad(L, "fg_quant_group4", None, 1, 64, 1, 64, None, None, None)
    assert st == L.FG_ERR_INVALID and "null" in msg
    p = ctypes.c_void_p(1 << 20)    # never dereferenced: validation fails first
    st, msg = _bad(L, "fg_quant_group4", p, 1, 96, 1, 64, p, p, None)
    assert st == L.FG_ERR_INVALID and "multiple" in msg
    st, msg = _bad(L, "fg_quant_group4", p, 1, 128, 1, 32, p, p, None)
    assert st == L.FG_ERR_UNSUPPORTED
    st, msg = _bad(L, "fg_dequant_group4", p, p, 0, 64, 1, 64, p, None)
    assert st == L.FG_ERR_INVALID


def test_linear_rejects_bad_arguments(L):
    p = ctypes.c_void_p(1 << 20)
    st, _ = _bad(L, "fg_linear", p, 4, 100, 0, p, None, 64, None, 0, None, p, None, 0, None)
    assert st == L.FG_ERR_UNSUPPORTED                  # K % 64
    st, _ = _bad(L, "fg_linear", p, 4, 64, 1, p, None, 64, None, 0, None, p, None, 0, None)
    assert st == L.FG_ERR_INVALID                      # q4 without meta
    st, _ = _bad(L, "fg_linear", p, 4, 64, 1, p, p, 100, None, 0, None, p, None, 0, None)
    assert st == L.FG_ERR_UNSUPPORTED                  # q4 N % 64
    st, _ = _bad(L, "fg_linear", p, 4, 64, 0, p, None, 64, None, 7, None, p, None, 0, None)
    assert st == L.FG_ERR_INVALID                      # unknown activation


def _kv(L, fmt=1, max_len=16, n_seq=4):
    p = 1 << 20
    return L.KV(fmt, p, p, p, p, max_len, n_seq)


def test_attention_rejects_bad_arguments(L):
    p = ctypes.c_void_p(1 << 20)
    d = L.dims(256, 1024, 2, 128)
    kv = _kv(L)
    f = L.raw("fg_attn_decode_q4")
    assert f(p, p, p, 768, ctypes.byref(kv), 4, ctypes.byref(d), 16, 1, p, None) == L.FG_ERR_INVALID
    assert "pos" in L.last_error()
    assert f(p, p, p, 768, ctypes.byref(kv), 5, ctypes.byref(d), 3, 1, p, None) == L.FG_ERR_INVALID
    assert f(p, p, p, 100, ctypes.byref(kv), 4, ctypes.byref(d), 3, 1, p, None) == L.FG_ERR_INVALID
    kv16 = _kv(L, fmt=0)
    assert f(p, p, p, 768, ctypes.byref(kv16), 4, ctypes.byref(d), 3, 1, p, None) == L.FG_ERR_INVALID
    bad = L.dims(256, 1024, 4, 64 + 32)
    assert f(p, p, p, 768, ctypes.byref(kv), 4, ctypes.byref(bad), 3, 1, p, None) == L.FG_ERR_INVALID
    d96 = L.dims(192, 768, 2, 96)
    assert f(p, p, p, 768, ctypes.byref(kv), 4, ctypes.byref(d96), 3, 1, p, None) == L.FG_ERR_UNSUPPORTED
    # Top-K: 0 <= topk <= pos, and the history's scores must fit on chip
    t = L.raw("fg_attn_decode_topk_q4")
    assert t(p, p, p, 768, ctypes.byref(kv), 4, ctypes.byref(d), 3, 4, 1, p, None) == L.FG_ERR_INVALID
    assert "topk" in L.last_error()
    assert t(p, p, p, 768, ctypes.byref(kv), 4, ctypes.byref(d), 3, -1, 1, p, None) == L.FG_ERR_INVALID
    assert t(p, p, p, 768, ctypes.byref(kv16), 4, ctypes.byref(d), 3, 1, 1, p, None) == L.FG_ERR_INVALID


def test_layer_rejects_bad_arguments(L):
    p = 1 << 20
    d = L.dims(256, 1024, 2, 128)
    w = L.LayerW(1, *([p] * 16))
    kv = _kv(L, max_len=16, n_seq=4)
    f = L.raw("fg_layer_decode_block")
    need = L.fg_workspace_bytes(d, 4, 1)
    assert need > 0
    st = f(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(p), 2, 2, 3, ctypes.byref(kv),
           ctypes.c_void_p(p), need - 1, None, 0, None)
    assert st == L.FG_ERR_CAPACITY
    st = f(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(p), 3, 2, 3, ctypes.byref(kv),
           ctypes.c_void_p(p), need, None, 0, None)
    assert st == L.FG_ERR_INVALID                     # 6 sequences > n_seq
    st = f(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(p), 2, 2, 3, ctypes.byref(kv),
           ctypes.c_void_p(p), need, None, -1, None)
    assert st == L.FG_ERR_INVALID                     # negative Top-K fraction
    long_kv = _kv(L, max_len=9000, n_seq=4)
    st = f(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(p), 2, 2, 8193, ctypes.byref(long_kv),
           ctypes.c_void_p(p), need, None, 100000, None)
    assert st == L.FG_ERR_UNSUPPORTED                 # sparse history beyond the on-chip scores
    assert "Top-K" in L.last_error()
    w.m_o = None
    st = f(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(p), 2, 2, 3, ctypes.byref(kv),
           ctypes.c_void_p(p), need, None, 0, None)
    assert st == L.FG_ERR_INVALID
    g = L.raw("fg_layer_prefill")
    w.m_o = p
    st = g(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(p), 2, 2, 17, ctypes.byref(kv),
           ctypes.c_void_p(p), 1 << 40, None, None)
    assert st == L.FG_ERR_INVALID                     # s > max_len


def test_workspace_grows_with_rows(L):
    d = L.dims(12288, 49152, 96, 128)
    a = L.fg_workspace_bytes(d, 144, 1)
    b = L.fg_workspace_bytes(d, 48 * 512, 1)
    assert 0 < a < b
    assert L.fg_linear_workspace_bytes(144, 12288, 49152) % 4 == 0


def test_stage_bytes_closed_form(L):
    for h1, h2 in ((768, 3072), (9216, 36864), (2048, 8192)):
        d = L.dims(h1, h2, h1 // 64, 64)
        q = -(-3 * h1 * h1 * 2 // 256) * 256
        w1 = -(-h2 * h1 * 2 // 256) * 256
        assert L.fg_stage_bytes(d) == q + w1
    # OPT-66B shape: the staged half of one layer is 6 h1^2 fp16 of its 12 h1^2
    d = L.dims(9216, 36864, 72, 128)
    assert 2 * 9216 * 9216 * 2 + 36864 * 9216 * 2 == 6 * 9216 * 9216 * 2


def test_model_pass_rejects_bad_arguments(L):
    """The block-schedule entry points validate every layer before enqueueing
    anything (no GPU needed: these all fail on the host)."""
    p = 1 << 20
    d = L.dims(256, 1024, 2, 128)
    ws_need = L.fg_workspace_bytes(d, 4, 1)
    w = (L.LayerW * 2)(L.LayerW(1, *([p] * 16)), L.LayerW(1, *([p] * 16)))
    kvs = (L.KV * 2)(_kv(L, max_len=16, n_seq=4), _kv(L, max_len=16, n_seq=4))
    f = L.raw("fg_model_decode_step")
    V = ctypes.c_void_p
    assert f(None, ctypes.byref(d), 0, w, None, kvs, V(p), 2, 2, 3, V(p), ws_need, None, None, 0, 0, None) \
        == L.FG_ERR_INVALID                            # no layers
    w[1].m_o = None                                    # second layer broken: nothing may run
    assert f(None, ctypes.byref(d), 2, w, None, kvs, V(p), 2, 2, 3, V(p), ws_need, None, None, 0, 0, None) \
        == L.FG_ERR_INVALID
    assert "metadata" in L.last_error()
    w[1].m_o = p
    tier = (L.TierW * 2)(L.TierW(p, p, p), L.TierW())
    assert f(None, ctypes.byref(d), 2, w, tier, kvs, V(p), 2, 2, 3, V(p), ws_need, None, None, 0, 0, None) \
        == L.FG_ERR_INVALID                            # tiering without a scheduler
    assert "scheduler" in L.last_error()
    long_kvs = (L.KV * 2)(_kv(L, max_len=9000, n_seq=4), _kv(L, max_len=9000, n_seq=4))
    assert f(None, ctypes.byref(d), 2, w, None, long_kvs, V(p), 2, 2, 8193, V(p), ws_need, None,
             None, 0, 100000, None) == L.FG_ERR_UNSUPPORTED   # sparse step past the on-chip scores
    g = L.raw("fg_model_prefill")
    assert g(None, ctypes.byref(d), 2, w, None, kvs, V(p), 2, 2, 17, V(p), 1 << 40, None, None, 0, None) \
        == L.FG_ERR_INVALID                            # s > max_len
    assert L.raw("fg_sched_create")(None, V(p), 256) == L.FG_ERR_INVALID
    assert L.raw("fg_sched_destroy")(None) == L.FG_OK


def test_prefetch_rejects_null_pointers(L):
    """fg_prefetch checks its pointers before any HIP call; with nothing to
    copy and no event it enqueues nothing."""
    f = L.raw("fg_prefetch")
    assert f(None, None, 64, None, None) == L.FG_ERR_INVALID
    assert "null" in L.last_error()
    assert f(ctypes.c_void_p(1 << 20), None, 64, None, None) == L.FG_ERR_INVALID
    assert f(None, None, 0, None, None) == L.FG_OK


def test_kv_tier_slot_bytes_closed_form(L):
    """Two K/V code tensors and (4-bit) two metadata tensors of gbs sequences,
    each rounded up to 256 bytes."""
    up = lambda n: -(-n // 256) * 256  # noqa: E731
    for h1, nh, hd, gbs, ml in ((768, 12, 64, 4, 40), (7168, 56, 128, 48, 544), (256, 2, 128, 3, 17)):
        d = L.dims(h1, 4 * h1, nh, hd)
        rows = gbs * nh * ml
        assert L.fg_kvtier_slot_bytes(d, gbs, ml, L.FG_FMT_Q4G64) == \
            2 * up(rows * hd // 2) + 2 * up(rows * hd // 64 * 4)
        assert L.fg_kvtier_slot_bytes(d, gbs, ml, L.FG_FMT_F16) == 2 * up(rows * hd * 2)
    assert L.fg_kvtier_slot_bytes(L.dims(256, 1024, 2, 128), 0, 16, 1) == 0
    assert L.raw("fg_kvtier_create")(None, ctypes.c_void_p(1 << 20), 256, ctypes.c_void_p(1)) \
        == L.FG_ERR_INVALID
    h = ctypes.c_void_p()
    assert L.raw("fg_kvtier_create")(ctypes.byref(h), ctypes.c_void_p((1 << 20) + 8), 256,
                                     ctypes.c_void_p(1)) == L.FG_ERR_INVALID   # misaligned
    assert L.raw("fg_kvtier_destroy")(None) == L.FG_OK


def test_kv_tier_rejects_bad_geometry(L):
    """The host cache and nb_dev are checked before the tier object or any
    device (fails on the host; no GPU needed)."""
    p = 1 << 20
    d = L.dims(256, 1024, 2, 128)
    w = L.LayerW(1, *([p] * 16))
    kv = _kv(L, max_len=16, n_seq=4)
    f = L.raw("fg_layer_decode_block")
    need = L.fg_workspace_bytes(d, 6, 1)
    V = ctypes.c_void_p

    def call(host, nb_dev, pos=3, pipe=None):
        t = L.KvTier(pipe, ctypes.pointer(host), nb_dev)
        return f(ctypes.byref(d), ctypes.byref(w), V(p), 2, 3, pos, ctypes.byref(kv), V(p), need,
                 None, 0, ctypes.byref(t))

    assert call(_kv(L, max_len=16, n_seq=4), 4) == L.FG_ERR_INVALID          # nb_dev > nb
    assert "nb_dev" in L.last_error()
    assert call(_kv(L, max_len=16, n_seq=3), 1) == L.FG_ERR_INVALID          # 4 host sequences needed
    assert "sequences" in L.last_error()
    assert call(_kv(L, fmt=0, max_len=16, n_seq=4), 1) == L.FG_ERR_INVALID   # format differs
    assert call(_kv(L, max_len=3, n_seq=4), 1) == L.FG_ERR_INVALID           # pos 3 beyond host max_len
    assert call(_kv(L, max_len=16, n_seq=4), 1) == L.FG_ERR_INVALID          # no tier object
    assert "tier object" in L.last_error()
    # every batch on the device: the host cache is not consulted
    t = L.KvTier(None, None, 3)
    kv6 = _kv(L, max_len=16, n_seq=6)
    assert f(ctypes.byref(d), ctypes.byref(w), V(p), 2, 3, 3, ctypes.byref(kv6), V(p), need - 1,
             None, 0, ctypes.byref(t)) == L.FG_ERR_CAPACITY
    g = L.raw("fg_model_decode_step")
    ws = (L.LayerW * 1)(w)
    kvs = (L.KV * 1)(kv)
    t = L.KvTier(None, None, 1)
    assert g(None, ctypes.byref(d), 1, ws, None, kvs, V(p), 2, 3, 3, V(p), need, None, None, 0, 0,
             ctypes.byref(t)) == L.FG_ERR_INVALID                        # no host cache array


# ------------------------------------------------------------ capacity
def _plan175(L, bls_dev=144, **kw):
    args = dict(n_layers=96, fmt_w=L.FG_FMT_Q4G64, fmt_kv=L.FG_FMT_Q4G64, max_len=544,
                bls_dev=bls_dev, gbs=48, s=512, vocab=50272)
    args.update(kw)
    return L.dims(12288, 49152, 96, 128), L.plan(**args)


def test_plan_bytes_add_up(L):
    """The plan's device bytes are the closed-form weights and cache plus the
    stated extras: weight tiering moves 2 h1^2 + h1 h2 fp16 elements per
    tiered layer to the host and adds two stage buffers; host-resident GPU
    batches leave the device cache and add two slots."""
    d, p = _plan175(L)
    total = L.fg_plan_device_bytes(d, p)
    w = L.fg_weight_bytes(d, 96, L.FG_FMT_Q4G64)
    kv = L.fg_kv_bytes(d, 96, 144, 544, 0, L.FG_FMT_Q4G64)
    assert w + kv < total < w + kv + 16e9             # workspaces, embeddings, activations
    # more sequences cost at least their cache
    d, p2 = _plan175(L, bls_dev=145)
    assert L.fg_plan_device_bytes(d, p2) - total >= kv // 144
    # fp16, tiering of 40 of 96 layers
    f16 = dict(fmt_w=L.FG_FMT_F16)
    d, pa = _plan175(L, **f16)
    d, pb = _plan175(L, n_tiered=40, **f16)
    h1, h2 = 12288, 49152
    assert L.fg_plan_device_bytes(d, pa) - L.fg_plan_device_bytes(d, pb) == \
        40 * 2 * (2 * h1 * h1 + h1 * h2) - 2 * L.fg_stage_bytes(d)
    # one of three GPU batches' cache on the host
    d, pc = _plan175(L, bls_dev=96, bls_host=48)
    assert L.fg_plan_device_bytes(d, p) - L.fg_plan_device_bytes(d, pc) == \
        kv // 3 - 2 * L.fg_kvtier_slot_bytes(d, 48, 544, L.FG_FMT_Q4G64)


def test_capacity_check_rejects_before_allocating(L):
    """The OPT-175B-shape 4-bit block (bls 48 x 3) fits 288 GB of HBM; with
    fp16 weights (348 GB) it does not, and neither does a 4-bit block of
    bls 512 (its 370 GB of cache); the refusal names the breakdown."""
    d, p = _plan175(L)
    L.fg_check_capacity(d, p, int(288e9))
    d, pf = _plan175(L, fmt_w=L.FG_FMT_F16)
    with pytest.raises(L.FgError) as e:
        L.fg_check_capacity(d, pf, int(288e9))
    assert e.value.status == L.FG_ERR_CAPACITY and "weights" in str(e.value)
    d, pb = _plan175(L, bls_dev=512)
    with pytest.raises(L.FgError) as e:
        L.fg_check_capacity(d, pb, int(288e9))
    assert e.value.status == L.FG_ERR_CAPACITY and "KV" in str(e.value)
    # fp16 with every layer's host half in pinned memory still misses by a few
    # GB; one of the three GPU batches' cache on the host as well fits
    d, pt = _plan175(L, fmt_w=L.FG_FMT_F16, n_tiered=96)
    with pytest.raises(L.FgError):
        L.fg_check_capacity(d, pt, int(288e9))
    d, pt = _plan175(L, fmt_w=L.FG_FMT_F16, n_tiered=96, bls_dev=96, bls_host=48)
    L.fg_check_capacity(d, pt, int(288e9))


def test_capacity_check_rejects_bad_plans(L):
    d, p = _plan175(L, fmt_w=L.FG_FMT_Q4G64, n_tiered=2)
    with pytest.raises(L.FgError) as e:
        L.fg_check_capacity(d, p, int(288e9))
    assert e.value.status == L.FG_ERR_INVALID and "fp16" in str(e.value)
    d, p = _plan175(L, bls_dev=100, bls_host=20)
    with pytest.raises(L.FgError) as e:
        L.fg_check_capacity(d, p, int(288e9))
    assert e.value.status == L.FG_ERR_INVALID and "whole GPU batches" in str(e.value)


def test_linear_noalloc_refuses_shapes_beyond_its_array(L):
    """fg_linear_noalloc keeps its split-k partials in a device array of
    fg_linear_noalloc_max_bytes(); a shape needing more is refused on the
    host, before any launch (the pointers are never dereferenced)."""
    M, N, K = 144, 98304, 12288
    cap = L._L.fg_linear_noalloc_max_bytes()
    assert cap == 96 << 20
    assert L.fg_linear_workspace_bytes(M, N, K) > cap
    p = ctypes.c_void_p(1 << 20)
    st, msg = _bad(L, "fg_linear_noalloc", p, M, K, L.FG_FMT_Q4G64, p, p, N, None, 0, None, p, None)
    assert st == L.FG_ERR_UNSUPPORTED and "scratch" in msg
    st, msg = _bad(L, "fg_linear_noalloc", None, M, K, L.FG_FMT_Q4G64, p, p, N, None, 0, None, p, None)
    assert st == L.FG_ERR_INVALID
