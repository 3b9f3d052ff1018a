"""Pins of the oracle's binary16 conversions and 4-bit codec against facts
fixed outside the oracle: hand-derived worked examples, numpy's IEEE binary16
conversion, exact round-trips of on-grid values, the rounding error bound of
the quantization equation, and layout invariants.

Codec source: "FlexGen 完全拆解" (pinghaoyang.com.cn), section
"权重压缩与 KV Cache 压缩" (quantize / dequantize equations, 4-bit, group 64);
bjbfmj.com FlexGen walkthrough §6.3 (byte packing, fp16 scale tensor).
"""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


# ------------------------------------------------------------------ binary16
def test_h2d_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    L = oracle.lib()
    got = np.array([L.or_h2d(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def test_d2h_matches_numpy_rounding():
    rng = np.random.default_rng(1)
    # normals, subnormals, exact midpoints (ties), overflow boundary
    xs = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
        (np.arange(2048) + 0.5) * 2.0 ** -24,                      # subnormal ties
        (np.arange(1024, 2048) + 0.5) * 2.0 ** -10,                # ties in [1, 2)
        np.array([65504.0, 65519.99, 65520.0, 65536.0, -65520.0, 2.0 ** -25, 2.0 ** -26,
                  3 * 2.0 ** -26, 0.0, -0.0, 1e-30, -1e-30]),
    ])
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.d2h(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------- codec
@pytest.mark.parametrize("name", ["codec_g64_worked.txt", "codec_g64_ties.txt"])
def test_codec_golden(name):
    g = _read_golden(name)
    x = np.array([float(v) for v in g["values"]], np.float16)
    codes, meta = oracle.quant_g4(x, 1, 64, 1)
    assert [int(c, 16) for c in g["codes"]] == codes.ravel().tolist()
    assert [int(m, 16) for m in g["meta"]] == meta.ravel().tolist()
    y = oracle.to_f16(oracle.dequant_g4(codes, meta, 1, 64, 1)).ravel().astype(np.float64)
    want = [float(v) for v in g.get("dequant", g["values"])]
    assert y.tolist() == want


def _ongrid_groups(rng, ngroups):
    """Groups x = mn + q * 2^e with q in 0..15 (both 0 and 15 present) and mn a
    multiple of 2^e: every value and the scale 2^e are exact in fp16."""
    xs, qs = [], []
    for _ in range(ngroups):
        e = int(rng.integers(-10, 3))
        mn = int(rng.integers(-300, 300)) * 2.0 ** e
        q = rng.integers(0, 16, 64)
        q[rng.integers(0, 64)] = 0
        q[rng.integers(0, 64)] = 15
        q[rng.permutation(64)[:2]] = [0, 15]
        xs.append(mn + q * 2.0 ** e)
        qs.append(q)
    x = np.array(xs, np.float64)
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)
    return x.astype(np.float16), np.array(qs)


def test_ongrid_roundtrip_exact():
    rng = np.random.default_rng(7)
    x, q = _ongrid_groups(rng, 500)
    codes, meta = oracle.quant_g4(x, 500, 64, 1)
    lo, hi = codes[..., 0] & 15, codes[..., 0] >> 4
    got_q = np.stack([lo, hi], axis=-1).reshape(500, 64)
    assert np.array_equal(got_q, q)
    y = oracle.dequant_g4(codes, meta, 500, 64, 1).reshape(500, 64)
    assert np.array_equal(y, x.view(np.uint16))


def test_constant_group_exact():
    x = np.full((3, 64), -1.375, np.float16)
    x[1] = 0.0
    x[2] = 6e-5  # fp16 subnormal-adjacent value
    codes, meta = oracle.quant_g4(x, 3, 64, 1)
    assert np.all(codes == 0)
    assert np.all(meta[:, 0, 1, 0] == 0)            # scale 0
    y = oracle.dequant_g4(codes, meta, 3, 64, 1).reshape(3, 64)
    assert np.array_equal(y, x.view(np.uint16))


def test_negative_zero_min_is_canonical():
    x = np.ones(64, np.float16)
    x[5] = -0.0
    x[9] = 0.0
    _, meta = oracle.quant_g4(x, 1, 64, 1)
    assert meta.ravel()[0] == 0x0000          # +0, not 0x8000


def test_error_bound_and_nearest_code():
    """|x - x^| <= range/30 up to fp16 rounding of the scale and the result, and
    each code is the nearest grid index of (x - min) * 15 / range."""
    rng = np.random.default_rng(3)
    G = 2000
    x = (rng.standard_normal((G, 64)) * 10.0 ** rng.uniform(-3, 2, (G, 1))).astype(np.float16)
    codes, meta = oracle.quant_g4(x, G, 64, 1)
    y = oracle.to_f16(oracle.dequant_g4(codes, meta, G, 64, 1)).reshape(G, 64).astype(np.float64)
    xd = x.astype(np.float64)
    mn, mx = xd.min(1, keepdims=True), xd.max(1, keepdims=True)
    rng_ = mx - mn
    ulp = np.abs(np.spacing(x)).astype(np.float64)
    err = np.abs(y - xd)
    assert np.all(err <= rng_ / 30 + rng_ * 2.0 ** -10 + ulp)
    assert np.mean(err > rng_ / 30 + ulp) < 1e-3
    q = np.stack([codes[..., 0] & 15, codes[..., 0] >> 4], -1).reshape(G, 64).astype(np.float64)
    t = (xd - mn) * 15.0 / rng_
    assert np.all(np.abs(q - t) <= 0.5 + 1e-5)
    clear = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-4
    assert np.array_equal(q[clear], np.round(t[clear]))
    # meta holds the exact min and the fp16 rounding of range/15
    assert np.array_equal(oracle.to_f16(meta[:, 0, 0, 0]).astype(np.float64), mn[:, 0])
    sc = oracle.to_f16(meta[:, 0, 1, 0]).astype(np.float64)
    assert np.all(np.abs(sc - rng_[:, 0] / 15) <= np.abs(np.spacing((rng_[:, 0] / 15).astype(np.float16))))


def test_codes_monotone_in_value():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 64)).astype(np.float16)
    codes, _ = oracle.quant_g4(x, 200, 64, 1)
    q = np.stack([codes[..., 0] & 15, codes[..., 0] >> 4], -1).reshape(200, 64)
    order = np.argsort(x.astype(np.float64), axis=1, kind="stable")
    qs = np.take_along_axis(q, order, 1)
    assert np.all(np.diff(qs.astype(int), axis=1) >= 0)
    assert np.all((q >= 0) & (q <= 15))


def test_strided_layout_matches_contiguous():
    """Weights group along N of [N, K] (inner = K > 1).  The same data laid out
    [K, N] with inner = 1 must give the transposed codes and meta."""
    rng = np.random.default_rng(11)
    N, K = 192, 40
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    c, m = oracle.quant_g4(w, 1, N, K)                       # [1, N/2, K], [1, N/64, 2, K]
    ct, mt = oracle.quant_g4(np.ascontiguousarray(w.T), K, N, 1)   # [K, N/2, 1], [K, N/64, 2, 1]
    assert np.array_equal(c[0], ct[:, :, 0].T)
    assert np.array_equal(m[0], mt[..., 0].transpose(1, 2, 0))
    y = oracle.dequant_weight(c.reshape(N // 2, K), m.reshape(N // 64, 2, K), N, K)
    yt = oracle.dequant_g4(ct, mt, K, N, 1)[..., 0].T
    assert np.array_equal(y, yt)


def test_weight_codes_pack_output_channel_pairs():
    """[P1] §6.3: data shape = shape[:group_dim] + (num_groups * group_size/2,) + ...;
    for group_dim 0 of [N, K], byte (j, k) holds rows 2j (low) and 2j+1 (high)."""
    N, K = 64, 3
    w = np.zeros((N, K), np.float16)
    w[:, 0] = np.arange(64) % 16          # range 15, scale 1, codes = value
    w[:, 1] = (np.arange(64) * 7) % 16
    w[:, 2] = 15 - np.arange(64) % 16
    c, m = oracle.quant_weight(w)
    for k in range(K):
        col = w[:, k].astype(int)
        want = col[0::2] | (col[1::2] << 4)
        assert c[:, k].tolist() == want.tolist()
    assert oracle.to_f16(m[0, 1]).tolist() == [1.0, 1.0, 1.0]
