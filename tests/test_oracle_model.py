"""Pins of the oracle's decoder pieces against facts fixed outside the oracle:
library routines on special cases (numpy matmul / softmax), brute force on
tiny shapes written independently of the C code, exact special cases
(identity layers, single-position attention), consistency between the
prefill and decode paths, and the pages' closed-form byte counts with their
printed worked numbers.

Pages: "FlexGen 完全拆解" (pinghaoyang.com.cn) — sections
"问题:显存放不下时…" (worked capacity numbers), "从 Transformer 推理的数据流
重新定义卸载" (M_W, M_KV, KV append), "SSD 不是更慢的显存" (162.5 s);
bjbfmj.com FlexGen walkthrough §6.3 (compression saves about 70%).
"""
import math

import numpy as np
import pytest

import oracle

F16 = np.float16


def f16(a):
    return np.asarray(a, np.float64).astype(F16)


def as64(u):
    return oracle.to_f16(u).astype(np.float64)


def rnd(rng, shape, std=1.0):
    return f16(rng.standard_normal(shape) * std)


# ----------------------------------------------------------------- LayerNorm
def test_layernorm_constant_row_gives_beta():
    rng = np.random.default_rng(0)
    x = np.tile(f16(rng.standard_normal((5, 1))), (1, 96))
    g, b = rnd(rng, 96), rnd(rng, 96)
    y = oracle.layernorm(x, g, b)
    assert np.array_equal(y, b.view(np.uint16)[None].repeat(5, 0))


def test_layernorm_moments_and_affine():
    rng = np.random.default_rng(1)
    x = rnd(rng, (7, 256), 3.0) + F16(5.0)
    one, zero = np.ones(256, F16), np.zeros(256, F16)
    z = as64(oracle.layernorm(x, one, zero))
    assert np.allclose(z.mean(1), 0, atol=2e-3) and np.allclose(z.var(1), 1, atol=5e-3)
    g, b = rnd(rng, 256), rnd(rng, 256)
    y = as64(oracle.layernorm(x, g, b))
    assert np.allclose(y, z * g.astype(np.float64) + b.astype(np.float64), atol=2e-2, rtol=2e-3)
    # invariant to an exact rescaling of the row (x -> 2x is exact in fp16)
    z2 = as64(oracle.layernorm(f16(x.astype(np.float64) * 2), one, zero))
    assert np.allclose(z2, z, atol=2e-3)


def _pin_layernorm(ln):
    """Rows alternating +a, -a over h = 64 have mean 0 and (biased) variance
    a^2 exactly, so LayerNorm with unit gain and zero shift gives
    +-a / sqrt(a^2 + eps), eps = 1e-5 inside the square root.  Small a makes
    eps matter (a = 2^-8: a^2 = 1.5e-5); a = 1 separates the biased variance
    (divide by h) from the unbiased one (h - 1), about 16 fp16 steps apart."""
    h = 64
    one, zero = np.ones(h, F16), np.zeros(h, F16)
    for a in (2.0 ** -8, 2.0 ** -6, 2.0 ** -3, 1.0, 3.0):
        x = f16(np.tile([a, -a], h // 2))[None].repeat(3, 0)
        y = ln(x, one, zero)
        v = a / math.sqrt(a * a + 1e-5)
        want = f16(np.tile([v, -v], h // 2))[None].repeat(3, 0)
        assert np.array_equal(oracle.to_f16(y).view(np.uint16), want.view(np.uint16)), a


def test_layernorm_alternating_rows_closed_form():
    _pin_layernorm(oracle.layernorm)


def _ln_unbiased(x, g, b):
    x = oracle.to_f16(x).astype(np.float64)
    z = (x - x.mean(1, keepdims=True)) / np.sqrt(x.var(1, ddof=1, keepdims=True) + 1e-5)
    return f16(z * g.astype(np.float64) + b.astype(np.float64))


def _ln_eps_outside(x, g, b):
    x = oracle.to_f16(x).astype(np.float64)
    z = (x - x.mean(1, keepdims=True)) / (np.sqrt(x.var(1, keepdims=True)) + 1e-5)
    return f16(z * g.astype(np.float64) + b.astype(np.float64))


def _ln_no_eps(x, g, b):
    x = oracle.to_f16(x).astype(np.float64)
    z = (x - x.mean(1, keepdims=True)) / np.sqrt(x.var(1, keepdims=True))
    return f16(z * g.astype(np.float64) + b.astype(np.float64))


@pytest.mark.parametrize("planted", [_ln_unbiased, _ln_eps_outside, _ln_no_eps])
def test_layernorm_pin_catches_planted_conventions(planted):
    with pytest.raises(AssertionError):
        _pin_layernorm(planted)


def test_layernorm_matches_torch_float64():
    """A library routine: torch's layer_norm (biased variance, eps inside the
    square root, elementwise affine) in float64, rounded once to fp16."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    for h, scale in ((64, 0.01), (768, 1.0), (1000, 30.0)):
        x = rnd(rng, (6, h), scale)
        g, b = rnd(rng, h), rnd(rng, h)
        ref = torch.nn.functional.layer_norm(
            torch.from_numpy(x.astype(np.float64)), (h,), torch.from_numpy(g.astype(np.float64)),
            torch.from_numpy(b.astype(np.float64)), eps=1e-5).numpy()
        got = as64(oracle.layernorm(x, g, b))
        ulp = np.abs(np.spacing(f16(ref))).astype(np.float64)
        assert np.max(np.abs(got - f16(ref).astype(np.float64)) / ulp) <= 1.0


# -------------------------------------------------------------------- linear
def test_linear_matches_numpy_matmul():
    rng = np.random.default_rng(2)
    M, K, N = 9, 192, 70
    x, w, b, r = rnd(rng, (M, K)), rnd(rng, (N, K), 0.05), rnd(rng, N), rnd(rng, (M, N))
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b.astype(np.float64)
    y = as64(oracle.linear(x, w, b))
    assert np.max(np.abs(y - f16(ref).astype(np.float64)) / np.abs(np.spacing(f16(ref)))) <= 1.0
    yr = as64(oracle.linear(x, w, b, relu=True))
    assert np.array_equal(yr, f16(np.maximum(ref, 0)).astype(np.float64)) or \
        np.max(np.abs(yr - np.maximum(ref, 0))) < 1e-2
    yres = as64(oracle.linear(x, w, b, residual=r))
    assert np.allclose(yres, ref + r.astype(np.float64), atol=1e-2, rtol=2e-3)


def test_linear_one_hot_row_selects_column():
    rng = np.random.default_rng(3)
    K, N = 64, 48
    w, b = rnd(rng, (N, K)), rnd(rng, N)
    x = np.zeros((K, K), F16)
    np.fill_diagonal(x, 1.0)
    y = as64(oracle.linear(x, w, b))
    want = f16(w.astype(np.float64).T + b.astype(np.float64)).astype(np.float64)
    assert np.array_equal(y, want)                  # row k = column k of W^T, plus bias
    assert np.array_equal(as64(oracle.linear(x, np.zeros((N, K), F16), b)),
                          np.tile(b.astype(np.float64), (K, 1)))


# ----------------------------------------------------------------- attention
def brute_attention(q, k, v):
    """Independent tiny-shape attention: explicit Python loops."""
    n, d = k.shape
    scores = [sum(float(q[c]) * float(k[j, c]) for c in range(d)) / math.sqrt(d) for j in range(n)]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    tot = sum(w)
    return [sum(w[j] * float(v[j, c]) for j in range(n)) / tot for c in range(d)]


def test_attn_prefill_brute_force_and_first_position():
    rng = np.random.default_rng(4)
    b, s, nh, hd = 2, 6, 2, 64
    h1 = nh * hd
    qkv = rnd(rng, (b * s, 3 * h1))
    out = as64(oracle.attn_prefill(qkv, b, s, nh, hd))
    q3 = qkv.astype(np.float64).reshape(b, s, 3, nh, hd)
    for bi in range(b):
        for h in range(nh):
            for t in range(s):
                want = brute_attention(q3[bi, t, 0, h], q3[bi, :t + 1, 1, h], q3[bi, :t + 1, 2, h])
                got = out[bi * s + t, h * hd:(h + 1) * hd]
                assert np.allclose(got, want, atol=2e-3, rtol=2e-3)
            # position 0 attends only to itself: out = v_0 exactly
            assert np.array_equal(out[bi * s, h * hd:(h + 1) * hd], q3[bi, 0, 2, h])


def test_attn_prefill_equal_keys_average_values():
    rng = np.random.default_rng(5)
    b, s, nh, hd = 1, 5, 1, 64
    qkv = rnd(rng, (s, 3 * hd))
    qkv[:, hd:2 * hd] = qkv[0, hd:2 * hd]          # identical keys -> uniform weights
    out = as64(oracle.attn_prefill(qkv, b, s, nh, hd))
    v = qkv[:, 2 * hd:].astype(np.float64)
    for t in range(s):
        assert np.allclose(out[t], v[:t + 1].mean(0), atol=2e-3)


def test_attn_decode_special_cases_and_brute_force():
    rng = np.random.default_rng(6)
    b, nh, hd, L = 2, 2, 128, 9
    h1 = nh * hd
    qkv = rnd(rng, (b, 3 * h1))
    kh, vh = rnd(rng, (b, nh, L, hd)), rnd(rng, (b, nh, L, hd))
    # pos 0: only the fresh token -> out = v_new exactly
    o0 = oracle.attn_decode(qkv, b, nh, hd, kh, vh, L, 0)
    assert np.array_equal(o0, qkv[:, 2 * h1:].view(np.uint16))
    pos = 6
    o = as64(oracle.attn_decode(qkv, b, nh, hd, kh, vh, L, pos))
    for bi in range(b):
        for h in range(nh):
            sl = slice(h * hd, (h + 1) * hd)
            K = np.concatenate([kh[bi, h, :pos], qkv[bi:bi + 1, h1:2 * h1][:, sl]]).astype(np.float64)
            V = np.concatenate([vh[bi, h, :pos], qkv[bi:bi + 1, 2 * h1:][:, sl]]).astype(np.float64)
            want = brute_attention(qkv[bi, sl].astype(np.float64), K, V)
            assert np.allclose(o[bi, sl], want, atol=2e-3, rtol=2e-3)
    # a dominant key pulls the output onto its value
    qkv2 = qkv.copy()
    kh2 = kh.copy()
    kh2[0, 0, 3] = f16(qkv2[0, :hd].astype(np.float64) * 8)
    o2 = as64(oracle.attn_decode(qkv2, b, nh, hd, kh2, vh, L, pos))
    assert np.allclose(o2[0, :hd], vh[0, 0, 3].astype(np.float64), atol=2e-2)


def test_decode_attention_equals_prefill_row():
    """With an fp16 cache holding the prompt's own K, V, decode attention at
    position t must reproduce prefill row t bit for bit (same sums, two code paths)."""
    rng = np.random.default_rng(8)
    b, s, nh, hd = 2, 7, 2, 64
    h1 = nh * hd
    qkv = rnd(rng, (b * s, 3 * h1))
    pre = oracle.attn_prefill(qkv, b, s, nh, hd)
    q3 = qkv.reshape(b, s, 3, nh, hd)
    kh = np.ascontiguousarray(q3[:, :, 1].transpose(0, 2, 1, 3))
    vh = np.ascontiguousarray(q3[:, :, 2].transpose(0, 2, 1, 3))
    for t in range(s):
        rows = np.ascontiguousarray(qkv.reshape(b, s, 3 * h1)[:, t])
        dec = oracle.attn_decode(rows, b, nh, hd, kh, vh, s, t)
        assert np.array_equal(dec, pre.reshape(b, s, h1)[:, t])


# ------------------------------------------------------------------ KV cache
def test_kv_cache_q4_layout_and_history():
    """Cache groups of 64 along one head's hidden dim ([P1] §6.3 group_dim 2)."""
    rng = np.random.default_rng(9)
    b, nh, hd, L = 2, 3, 128, 5
    c = oracle.KVCache("q4", b, nh, hd, L)
    kx, vx = rnd(rng, (b, 2, nh * hd)), rnd(rng, (b, 2, nh * hd))
    c.store(kx, vx, 1)
    kh, vh = c.history()
    for bi in range(b):
        for h in range(nh):
            for t in range(2):
                for src, dst, codes, meta in ((kx, kh, c.k, c.km), (vx, vh, c.v, c.vm)):
                    vec = src[bi, t, h * hd:(h + 1) * hd]
                    cc, mm = oracle.quant_g4(vec, 1, hd, 1)
                    assert np.array_equal(codes[bi, h, 1 + t], cc.ravel())
                    assert np.array_equal(meta[bi, h, 1 + t], mm.reshape(hd // 64, 2))
                    rt = oracle.dequant_g4(cc, mm, 1, hd, 1).ravel()
                    assert np.array_equal(dst[bi, h, 1 + t], rt)
    assert np.all(c.k[:, :, 0] == 0) and np.all(c.k[:, :, 3:] == 0)


# --------------------------------------------------------------------- layer
def _layer(rng, d, zero=False, zero_bias=False):
    W = {}
    shapes = {"w_qkv": (3 * d.h1, d.h1), "b_qkv": (3 * d.h1,), "w_o": (d.h1, d.h1), "b_o": (d.h1,),
              "w_1": (d.h2, d.h1), "b_1": (d.h2,), "w_2": (d.h1, d.h2), "b_2": (d.h1,)}
    for k, shp in shapes.items():
        is_bias = k.startswith("b_")
        if (zero and not is_bias) or (zero_bias and is_bias):
            W[k] = np.zeros(shp, F16)
        else:
            W[k] = rnd(rng, shp, 0.05)
    for k in ("ln1", "ln2"):
        W[k + "_g"] = f16(1 + 0.1 * rng.standard_normal(d.h1))
        W[k + "_b"] = rnd(rng, d.h1, 0.1)
    return W


D_SMALL = oracle.Dims(h1=128, h2=512, nh=2, hd=64)


@pytest.mark.parametrize("fmt", ["f16", "q4"])
def test_layer_zero_weights_is_identity(fmt):
    rng = np.random.default_rng(10)
    d = D_SMALL
    W = _layer(rng, d, zero=True, zero_bias=True)
    b, s = 2, 4
    x = rnd(rng, (b * s, d.h1))
    c = oracle.KVCache(fmt, b, d.nh, d.hd, s + 2)
    y = oracle.layer_prefill(d, W, x, b, s, c)
    assert np.array_equal(y, x.view(np.uint16))
    x1 = rnd(rng, (b, d.h1))
    y1, _, _ = oracle.layer_decode(d, W, x1, s, c)
    assert np.array_equal(y1, x1.view(np.uint16))


def test_layer_zero_matrices_adds_biases():
    """With every matrix zero, attention sees v = b_v, the MLP sees relu(b_1):
    the layer returns (x + b_o) + b_2, each sum rounded to fp16 once."""
    rng = np.random.default_rng(11)
    d = D_SMALL
    W = _layer(rng, d, zero=True)
    x = rnd(rng, (3, d.h1))
    c = oracle.KVCache("f16", 3, d.nh, d.hd, 2)
    y = as64(oracle.layer_prefill(d, W, x, 3, 1, c))
    step = f16(x.astype(np.float64) + W["b_o"].astype(np.float64))
    want = f16(step.astype(np.float64) + W["b_2"].astype(np.float64)).astype(np.float64)
    assert np.array_equal(y, want)


def test_layer_rows_are_independent():
    rng = np.random.default_rng(12)
    d = D_SMALL
    W = _layer(rng, d)
    b, s = 3, 5
    x = rnd(rng, (b * s, d.h1))
    full = oracle.layer_prefill(d, W, x, b, s, oracle.KVCache("q4", b, d.nh, d.hd, s))
    one = oracle.layer_prefill(d, W, x[s:2 * s], 1, s, oracle.KVCache("q4", 1, d.nh, d.hd, s))
    assert np.array_equal(full[s:2 * s], one)


def test_layer_decode_continues_prefill():
    """Prefill over s-1 tokens then one decode step on token s-1 reproduces the
    last row of a prefill over all s tokens (fp16 cache: identical arithmetic)."""
    rng = np.random.default_rng(13)
    d = D_SMALL
    W = _layer(rng, d)
    b, s = 2, 6
    x = rnd(rng, (b, s, d.h1))
    full = oracle.layer_prefill(d, W, x.reshape(b * s, -1), b, s,
                                oracle.KVCache("f16", b, d.nh, d.hd, s)).reshape(b, s, -1)
    c = oracle.KVCache("f16", b, d.nh, d.hd, s)
    oracle.layer_prefill(d, W, np.ascontiguousarray(x[:, :s - 1]).reshape(b * (s - 1), -1),
                         b, s - 1, c)
    y, _, _ = oracle.layer_decode(d, W, np.ascontiguousarray(x[:, s - 1]), s - 1, c)
    assert np.array_equal(y, full[:, s - 1])


def test_layer_decode_q4_fresh_vs_quantized_current():
    """Reading of the current token: fresh fp16 k, v; the quantized alternative
    must stay within the codec's error (both attend over the same history)."""
    rng = np.random.default_rng(14)
    d = D_SMALL
    W = _layer(rng, d)
    b, s = 2, 5
    x = rnd(rng, (b * s, d.h1))
    ca = oracle.KVCache("q4", b, d.nh, d.hd, s + 1)
    oracle.layer_prefill(d, W, x, b, s, ca)
    cb = oracle.KVCache("q4", b, d.nh, d.hd, s + 1)
    oracle.layer_prefill(d, W, x, b, s, cb)
    x1 = rnd(rng, (b, d.h1))
    ya, oa, _ = oracle.layer_decode(d, W, x1, s, ca, fresh_current=True)
    yb, ob, _ = oracle.layer_decode(d, W, x1, s, cb, fresh_current=False)
    assert np.array_equal(ca.k, cb.k) and np.array_equal(ca.vm, cb.vm)
    assert not np.array_equal(oa, ob)
    assert np.allclose(as64(oa), as64(ob), atol=0.1 * np.abs(as64(oa)).max())


# --------------------------------------------------------------------- model
def test_embed_and_argmax():
    rng = np.random.default_rng(15)
    E, P = rnd(rng, (50, 64)), rnd(rng, (8, 64))
    tok, pos = np.array([3, 49, 0]), np.array([0, 7, 2])
    x = oracle.embed(tok, pos, E, P)
    want = f16(E[tok].astype(np.float64) + P[pos].astype(np.float64))
    assert np.array_equal(x, want.view(np.uint16))
    lg = np.array([[1, 3, 3, 2], [-1, -1, -2, -1], [0, 0, 0, 0]], F16)
    assert oracle.argmax(lg).tolist() == [1, 0, 0]       # ties -> lowest index


def test_model_greedy_is_consistent():
    """Generation bookkeeping: n tokens = 1 from the prefill + n-1 decode steps;
    a decode at position p uses position p's embedding."""
    rng = np.random.default_rng(16)
    d = oracle.Dims(h1=64, h2=256, nh=1, hd=64)
    layers = [_layer(rng, d) for _ in range(2)]
    V, b, s, n = 40, 2, 4, 3
    E, P = rnd(rng, (V, d.h1)), rnd(rng, (s + n, d.h1))
    g, be = np.ones(d.h1, F16), np.zeros(d.h1, F16)
    toks = rng.integers(0, V, (b, s))
    m = oracle.Model(d, layers, E, P, g, be, "f16", s + n, b)
    lg, t1 = m.prefill(toks)
    assert np.array_equal(t1, oracle.argmax(lg))
    # decoding at p = s with token t1 equals prefilling s+1 tokens (fp16 cache)
    lg2, _ = m.decode(t1, s)
    m2 = oracle.Model(d, layers, E, P, g, be, "f16", s + n, b)
    lg_ref, _ = m2.prefill(np.concatenate([toks, t1[:, None]], 1))
    assert np.array_equal(lg2, lg_ref)


def _pin_lm_head(head):
    """The head is the final LayerNorm followed by the tied embedding
    (logits = LN_f(x) E^T).  With zero gain the LayerNorm returns its shift
    beta for every row, so the logits are beta E^T whatever x is; a one-hot
    beta = c e_j picks c times column j of E."""
    rng = np.random.default_rng(22)
    V, h = 50, 64
    E = rnd(rng, (V, h), 0.5)
    x = rnd(rng, (4, h), 2.0)
    zero = np.zeros(h, F16)
    beta = rnd(rng, h)
    lg = as64(head(x, zero, beta, E))
    want = f16(np.tile(E.astype(np.float64) @ beta.astype(np.float64), (4, 1))).astype(np.float64)
    assert lg.shape == (4, V) and np.array_equal(lg, want)
    onehot = np.zeros(h, F16)
    onehot[7] = F16(0.75)
    lg = as64(head(x, zero, onehot, E))
    assert np.array_equal(lg, np.tile(f16(0.75 * E[:, 7].astype(np.float64)).astype(np.float64), (4, 1)))


def test_lm_head_is_final_layernorm_then_tied_embedding():
    _pin_lm_head(oracle.lm_head)


@pytest.mark.parametrize("planted", [
    lambda x, g, b, E: oracle.linear(x, E),                                   # final LN skipped
    lambda x, g, b, E: oracle.linear(oracle.layernorm(x, np.ones_like(g), b), E),   # gain ignored
    lambda x, g, b, E: oracle.linear(oracle.layernorm(x, g, b), E, bias=E[:, 0].copy()),  # stray bias
])
def test_lm_head_pin_catches_planted_mistakes(planted):
    with pytest.raises(AssertionError):
        _pin_lm_head(planted)


def test_model_logits_come_from_the_head():
    """Whole-model bookkeeping: with a zero-gain final LayerNorm every
    sequence's logits are beta E^T after the prefill and after a decode step,
    whatever the layers computed."""
    rng = np.random.default_rng(23)
    d = oracle.Dims(h1=64, h2=256, nh=1, hd=64)
    layers = [_layer(rng, d) for _ in range(2)]
    V, b, s, n = 40, 2, 4, 2
    E, P = rnd(rng, (V, d.h1)), rnd(rng, (s + n, d.h1))
    beta = rnd(rng, d.h1)
    m = oracle.Model(d, layers, E, P, np.zeros(d.h1, F16), beta, "q4", s + n, b)
    want = f16(np.tile(E.astype(np.float64) @ beta.astype(np.float64), (b, 1))).view(np.uint16)
    lg, tok = m.prefill(rng.integers(0, V, (b, s)))
    assert np.array_equal(lg, want)
    lg2, _ = m.decode(tok, s)
    assert np.array_equal(lg2, want)


# --------------------------------------------------------------- closed forms
def test_weight_bytes_175b_worked_number():
    """[P2] "问题…" section: OPT-175B fp16 weights about 325 GB."""
    mw = oracle.weight_bytes_f16(12288, 49152, 96)
    assert mw == 347_892_350_976
    assert round(mw / 2 ** 30, 1) == 324.0          # ~325 "GB" as printed
    assert abs(mw / 1e9 - 325) / 325 < 0.08


def test_kv_bytes_175b_worked_number():
    """[P2]: b = 512, s = 512, n = 32: KV peak about 1.2 TB, 3.8x the weights."""
    mkv = oracle.kv_bytes_f16(12288, 96, 512, 512, 32)
    assert mkv == 4 * 512 * 96 * 12288 * 544
    assert round(mkv / 2 ** 40, 1) == 1.2
    assert round(mkv / oracle.weight_bytes_f16(12288, 49152, 96), 1) == 3.8


def test_ssd_pass_and_compression_saving():
    """[P2] "SSD 不是更慢的显存": 325 GB at 2 GB/s = 162.5 s; [P1] §6.3: 4-bit
    weights save about 70% (codes + fp16 (min, scale) per 64 = 9/32 of fp16)."""
    assert 325 / 2 == 162.5
    n = 12288 * 49152
    assert oracle.q4_bytes(n) * 32 == 2 * n * 9
    saving = 1 - oracle.q4_bytes(n) / (2 * n)
    assert saving == 0.71875 and abs(saving - 0.70) < 0.03


# ------------------------------------------------------- Top-K sparse V
def test_attn_topk_all_positions_is_dense_attention():
    """topk = pos reads every V row: bit-identical to the dense definition."""
    rng = np.random.default_rng(21)
    b, nh, hd, L = 2, 3, 64, 40
    h1 = nh * hd
    qkv = rnd(rng, (b, 3 * h1))
    kh, vh = rnd(rng, (b, nh, L, hd)), rnd(rng, (b, nh, L, hd))
    for pos in (0, 1, 17, 39):
        dense = oracle.attn_decode(qkv, b, nh, hd, kh, vh, L, pos)
        assert np.array_equal(oracle.attn_decode_topk(qkv, b, nh, hd, kh, vh, L, pos, pos), dense)


def test_attn_topk_equal_scores_take_lowest_positions():
    """Equal scores everywhere (zero keys): every weight is 1 / (pos + 1) and the
    tie rule keeps the lowest positions, so out = (v_0 + ... + v_{k-1} + v_new) / (pos + 1)."""
    rng = np.random.default_rng(22)
    b, nh, hd, L, pos = 2, 2, 64, 20, 13
    h1 = nh * hd
    qkv = rnd(rng, (b, 3 * h1))
    qkv[:, h1:2 * h1] = 0
    kh = np.zeros((b, nh, L, hd), np.float16)
    vh = rnd(rng, (b, nh, L, hd))
    for k in (0, 1, 5, 13):
        got = as64(oracle.attn_decode_topk(qkv, b, nh, hd, kh, vh, L, pos, k))
        for bi in range(b):
            for h in range(nh):
                sl = slice(h * hd, (h + 1) * hd)
                want = (vh[bi, h, :k].astype(np.float64).sum(0) + qkv[bi, 2 * h1:][sl].astype(np.float64)) / (pos + 1)
                assert np.allclose(got[bi, sl], want, atol=1e-3, rtol=1e-3)


def test_attn_topk_keeps_weights_of_the_selected_rows():
    """Keys built so that the score grows with the position: the top k are the
    last k rows, and the result equals dense attention over a V whose other
    rows are zero (the weights of the selected rows are the full softmax's:
    no renormalization)."""
    rng = np.random.default_rng(23)
    b, nh, hd, L, pos = 2, 2, 64, 32, 25
    h1 = nh * hd
    qkv = rnd(rng, (b, 3 * h1))
    kh = np.empty((b, nh, L, hd), np.float16)
    for bi in range(b):
        for h in range(nh):
            qv = qkv[bi, h * hd:(h + 1) * hd].astype(np.float64)
            for p in range(L):
                kh[bi, h, p] = f16(qv * (0.02 * p) / np.sqrt(hd))
    vh = rnd(rng, (b, nh, L, hd))
    for k in (1, 3, 10):
        vz = vh.copy()
        vz[:, :, :pos - k] = 0
        dense = oracle.attn_decode(qkv, b, nh, hd, kh, vz, L, pos)
        assert np.array_equal(oracle.attn_decode_topk(qkv, b, nh, hd, kh, vh, L, pos, k), dense)


def test_topk_count_rounds_up():
    assert [oracle.topk_count(p) for p in (0, 1, 9, 10, 11, 528)] == [0, 1, 1, 1, 2, 53]
    assert oracle.topk_count(100, 1.0) == 100 and oracle.topk_count(100, 0.0) == 0
