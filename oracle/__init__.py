"""CPU oracle for the 4-bit zig-zag block decode of an OPT-style decoder.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
definition of what the GPU path computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product package
never does, and this package never imports the product package.  The two share
no code: the arithmetic lives in ``oracle.c`` (plain C, fp64 reductions,
binary32 for the codec), and this module only marshals numpy arrays and
composes those primitives in the order the pages describe.

Pages (cited by title and section):
  [P2] "FlexGen 完全拆解:用线性规划编排 GPU、CPU 与 SSD 上的大模型推理"
       (pinghaoyang.com.cn).
  [P1] bjbfmj.com FlexGen walkthrough (sections numbered 一…八 → §1…§8).

fp16 tensors are numpy ``uint16`` arrays holding binary16 bit patterns (a
``float16`` array may be passed and is reinterpreted, not converted).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = [os.path.join(_HERE, "oracle.c")]
_lock = threading.Lock()
_lib = None

LN_EPS = 1e-5


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (IEEE semantics: no contraction, no fast-math)."""
    if not force and os.path.exists(_SO):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-o", tmp] + _SRC + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                build()
            L = ctypes.CDLL(_SO)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            I32 = ctypes.c_int32
            L.or_h2d.argtypes, L.or_h2d.restype = [ctypes.c_uint16], ctypes.c_double
            L.or_d2h.argtypes, L.or_d2h.restype = [ctypes.c_double], ctypes.c_uint16
            L.or_f2h.argtypes, L.or_f2h.restype = [ctypes.c_float], ctypes.c_uint16
            L.or_h2f.argtypes, L.or_h2f.restype = [ctypes.c_uint16], ctypes.c_float
            L.or_quant_g4.argtypes = [P, I64, I64, I64, I32, P, P]
            L.or_dequant_g4.argtypes = [P, P, I64, I64, I64, I32, P]
            L.or_layernorm.argtypes = [P, I64, I64, P, P, ctypes.c_double, P]
            L.or_linear.argtypes = [P, I64, I64, I64, P, I64, P, I32, P, P, I64]
            L.or_attn_prefill.argtypes = [P, I64, I64, I64, I64, P]
            L.or_attn_decode.argtypes = [P, P, P, I64, I64, I64, I64, P, P, I64, I64, P]
            L.or_attn_decode_topk.argtypes = [P, P, P, I64, I64, I64, I64, P, P, I64, I64, I64, P]
            L.or_embed.argtypes = [P, P, I64, P, P, I64, P]
            L.or_argmax.argtypes = [P, I64, I64, P]
            L.or_set_threads.argtypes, L.or_set_threads.restype = [I32], None
            L.or_get_threads.argtypes, L.or_get_threads.restype = [], I32
            for f in ("or_quant_g4", "or_dequant_g4", "or_layernorm", "or_linear",
                      "or_attn_prefill", "or_attn_decode", "or_attn_decode_topk", "or_embed",
                      "or_argmax"):
                getattr(L, f).restype = None
            _lib = L
    return _lib


def set_threads(n: int) -> None:
    """OpenMP threads of the C primitives (timing only; results do not depend on it)."""
    lib().or_set_threads(int(n))


def get_threads() -> int:
    return int(lib().or_get_threads())


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def to_f16(a) -> np.ndarray:
    """View a uint16 bit-pattern array as float16 (no conversion)."""
    return _u16(a).view(np.float16)


# ------------------------------------------------------------------ binary16
def h2d(h: int) -> float:
    return lib().or_h2d(h)


def d2h(x: float) -> int:
    return lib().or_d2h(x)


# --------------------------------------------------------------------- codec
def quant_g4(x, outer: int, axis: int, inner: int, group: int = 64):
    """[P2] "权重压缩与 KV Cache 压缩", quantization equation; [P1] §6.3.

    Returns (codes uint8 [outer, axis/2, inner], meta uint16 [outer, axis/group, 2, inner])."""
    x = _u16(x)
    assert x.size == outer * axis * inner and axis % group == 0 and group % 2 == 0
    codes = np.empty((outer, axis // 2, inner), np.uint8)
    meta = np.empty((outer, axis // group, 2, inner), np.uint16)
    lib().or_quant_g4(_ptr(x), outer, axis, inner, group, _ptr(codes), _ptr(meta))
    return codes, meta


def dequant_g4(codes, meta, outer: int, axis: int, inner: int, group: int = 64) -> np.ndarray:
    """[P2] "权重压缩与 KV Cache 压缩", dequantization equation."""
    codes = np.ascontiguousarray(codes, np.uint8)
    meta = _u16(meta)
    y = np.empty((outer, axis, inner), np.uint16)
    lib().or_dequant_g4(_ptr(codes), _ptr(meta), outer, axis, inner, group, _ptr(y))
    return y


def quant_weight(w):
    """Weight [N, K]: groups of 64 along the output-channel dim N ([P1] §6.3 group_dim 0;
    [P2] weights grouped along the output channel).  Returns codes [N/2, K], meta [N/64, 2, K]."""
    w = _u16(w)
    N, K = w.shape
    c, m = quant_g4(w, 1, N, K)
    return c.reshape(N // 2, K), m.reshape(N // 64, 2, K)


def dequant_weight(codes, meta, N: int, K: int) -> np.ndarray:
    return dequant_g4(codes, meta, 1, N, K).reshape(N, K)


# -------------------------------------------------------------- model pieces
def layernorm(x, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    x = _u16(x)
    rows, h = x.shape
    y = np.empty_like(x)
    lib().or_layernorm(_ptr(x), rows, h, _ptr(_u16(gamma)), _ptr(_u16(beta)), eps, _ptr(y))
    return y


def linear(x, w, bias=None, relu: bool = False, residual=None) -> np.ndarray:
    """y = act(x w^T + bias) + residual, fp64 accumulation, one fp16 rounding."""
    x = _u16(x)
    w = _u16(w)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape == (N, K)
    y = np.empty((M, N), np.uint16)
    r = None if residual is None else _u16(residual)
    b = None if bias is None else _u16(bias)
    lib().or_linear(_ptr(x), M, K, K, _ptr(w), N, _ptr(b), int(relu), _ptr(r), _ptr(y), N)
    return y


def attn_prefill(qkv, b: int, s: int, nh: int, hd: int) -> np.ndarray:
    qkv = _u16(qkv)
    assert qkv.shape == (b * s, 3 * nh * hd)
    out = np.empty((b * s, nh * hd), np.uint16)
    lib().or_attn_prefill(_ptr(qkv), b, s, nh, hd, _ptr(out))
    return out


def attn_decode(qkv, b: int, nh: int, hd: int, khist, vhist, lmax: int, pos: int) -> np.ndarray:
    """Single query at position pos; rows of qkv are (q | k_new | v_new)."""
    qkv = _u16(qkv)
    h1 = nh * hd
    assert qkv.shape == (b, 3 * h1)
    kh, vh = _u16(khist), _u16(vhist)
    assert kh.shape == (b, nh, lmax, hd) and vh.shape == kh.shape and 0 <= pos < lmax
    out = np.empty((b, h1), np.uint16)
    base = qkv.ctypes.data
    L = lib()
    L.or_attn_decode(ctypes.c_void_p(base), ctypes.c_void_p(base + 2 * h1),
                     ctypes.c_void_p(base + 4 * h1), 3 * h1, b, nh, hd, _ptr(kh), _ptr(vh),
                     lmax, pos, _ptr(out))
    return out


def attn_decode_topk(qkv, b: int, nh: int, hd: int, khist, vhist, lmax: int, pos: int,
                     topk: int) -> np.ndarray:
    """[P2] "权重压缩与 KV Cache 压缩", Top-K sparse attention: as attn_decode,
    but V is summed only over the topk cached positions of highest score (ties:
    lower position first) plus the current token; the softmax normalizer keeps
    every score (no renormalization)."""
    qkv = _u16(qkv)
    h1 = nh * hd
    assert qkv.shape == (b, 3 * h1)
    kh, vh = _u16(khist), _u16(vhist)
    assert kh.shape == (b, nh, lmax, hd) and vh.shape == kh.shape and 0 <= pos < lmax
    assert 0 <= topk <= pos
    out = np.empty((b, h1), np.uint16)
    base = qkv.ctypes.data
    lib().or_attn_decode_topk(ctypes.c_void_p(base), ctypes.c_void_p(base + 2 * h1),
                              ctypes.c_void_p(base + 4 * h1), 3 * h1, b, nh, hd, _ptr(kh), _ptr(vh),
                              lmax, pos, topk, _ptr(out))
    return out


def topk_count(pos: int, frac: float = 0.1) -> int:
    """Number of cached positions whose V is read at sparsity frac: the pages'
    10%, rounded up (at least one position whenever there is history)."""
    return min(pos, -(-int(round(frac * 1_000_000)) * pos // 1_000_000))


def embed(tok, pos, E, P) -> np.ndarray:
    tok = np.ascontiguousarray(tok, np.int32).reshape(-1)
    pos = np.ascontiguousarray(pos, np.int32).reshape(-1)
    E, P = _u16(E), _u16(P)
    h1 = E.shape[1]
    x = np.empty((tok.size, h1), np.uint16)
    lib().or_embed(_ptr(tok), _ptr(pos), tok.size, _ptr(E), _ptr(P), h1, _ptr(x))
    return x


def argmax(logits) -> np.ndarray:
    lg = _u16(logits)
    out = np.empty(lg.shape[0], np.int32)
    lib().or_argmax(_ptr(lg), lg.shape[0], lg.shape[1], _ptr(out))
    return out


# ------------------------------------------------------------------ KV cache
@dataclass
class KVCache:
    """One layer's KV cache for b sequences, nh heads, lmax positions.

    fmt "q4": codes [b, nh, lmax, hd/2] uint8 and meta [b, nh, lmax, hd/64, 2]
    fp16 per tensor — groups of 64 along the hidden dim of one head ([P1] §6.3
    group_dim 2; [P2] KV grouped along the hidden dimension).
    fmt "f16": [b, nh, lmax, hd] fp16."""
    fmt: str
    b: int
    nh: int
    hd: int
    lmax: int
    k: np.ndarray = field(init=False)
    v: np.ndarray = field(init=False)
    km: np.ndarray | None = field(init=False, default=None)
    vm: np.ndarray | None = field(init=False, default=None)

    def __post_init__(self):
        b, nh, L, hd = self.b, self.nh, self.lmax, self.hd
        if self.fmt == "q4":
            self.k = np.zeros((b, nh, L, hd // 2), np.uint8)
            self.v = np.zeros((b, nh, L, hd // 2), np.uint8)
            self.km = np.zeros((b, nh, L, hd // 64, 2), np.uint16)
            self.vm = np.zeros((b, nh, L, hd // 64, 2), np.uint16)
        elif self.fmt == "f16":
            self.k = np.zeros((b, nh, L, hd), np.uint16)
            self.v = np.zeros((b, nh, L, hd), np.uint16)
        else:
            raise ValueError(self.fmt)

    def store(self, kx, vx, t0: int):
        """[P2] KV append: K_{1:s+t} = Concat(K_{1:s+t-1}, new k); same for V.
        kx, vx: [b, nt, nh*hd] fp16 for positions t0..t0+nt-1."""
        kx, vx = _u16(kx), _u16(vx)
        b, nt, h1 = kx.shape
        nh, hd = self.nh, self.hd
        for src, dst, dm in ((kx, self.k, self.km), (vx, self.v, self.vm)):
            per_head = np.ascontiguousarray(src.reshape(b, nt, nh, hd).transpose(0, 2, 1, 3))
            if self.fmt == "f16":
                dst[:, :, t0:t0 + nt, :] = per_head
            else:
                c, m = quant_g4(per_head, b * nh * nt, hd, 1)
                dst[:, :, t0:t0 + nt, :] = c.reshape(b, nh, nt, hd // 2)
                dm[:, :, t0:t0 + nt, :, :] = m.reshape(b, nh, nt, hd // 64, 2)

    def history(self):
        """Stored K, V as fp16 [b, nh, lmax, hd] (dequantized for q4)."""
        if self.fmt == "f16":
            return self.k, self.v
        b, nh, L, hd = self.b, self.nh, self.lmax, self.hd
        out = []
        for c, m in ((self.k, self.km), (self.v, self.vm)):
            y = dequant_g4(c.reshape(b * nh * L, hd // 2, 1), m.reshape(b * nh * L, hd // 64, 2, 1),
                           b * nh * L, hd, 1)
            out.append(y.reshape(b, nh, L, hd))
        return out[0], out[1]


# --------------------------------------------------------------------- layer
@dataclass
class Dims:
    h1: int
    h2: int
    nh: int
    hd: int

    def __post_init__(self):
        assert self.nh * self.hd == self.h1


LAYER_KEYS = ("w_qkv", "b_qkv", "w_o", "b_o", "w_1", "b_1", "w_2", "b_2",
              "ln1_g", "ln1_b", "ln2_g", "ln2_b")


def layer_prefill(d: Dims, W: dict, x, b: int, s: int, cache: KVCache) -> np.ndarray:
    """One pre-LN decoder layer over b prompts of s tokens (rows b*s).

    [P2] "从 Transformer 推理的数据流重新定义卸载": the prompt's K, V, Q come from
    X W_K, X W_V, X W_Q over all s tokens and the K, V stay in the cache for
    the decode steps.  W holds fp16 matrices (for 4-bit weights, the
    dequantized ones)."""
    x = _u16(x)
    a = layernorm(x, W["ln1_g"], W["ln1_b"])
    qkv = linear(a, W["w_qkv"], W["b_qkv"])
    o = attn_prefill(qkv, b, s, d.nh, d.hd)
    q3 = qkv.reshape(b, s, 3, d.h1)
    cache.store(q3[:, :, 1, :], q3[:, :, 2, :], 0)
    x = linear(o, W["w_o"], W["b_o"], residual=x)
    a = layernorm(x, W["ln2_g"], W["ln2_b"])
    f = linear(a, W["w_1"], W["b_1"], relu=True)
    return linear(f, W["w_2"], W["b_2"], residual=x)


def layer_decode(d: Dims, W: dict, x, pos: int, cache: KVCache, fresh_current: bool = True,
                 attn_topk: float = 0.0):
    """One pre-LN decoder layer for one new token per sequence at position pos.

    The new k, v are appended to the cache at pos.  Attention covers 0..pos:
    positions < pos from the (dequantized) cache; position pos from the fresh
    fp16 k, v when fresh_current, else from its own quantized copy.  With
    attn_topk > 0 (fresh_current only) the V sum is the Top-K sparse one over
    topk_count(pos, attn_topk) cached positions.
    Returns (x_out, attn_out, qkv)."""
    x = _u16(x)
    b = x.shape[0]
    a = layernorm(x, W["ln1_g"], W["ln1_b"])
    qkv = linear(a, W["w_qkv"], W["b_qkv"])
    q3 = qkv.reshape(b, 1, 3, d.h1)
    if fresh_current:
        kh, vh = cache.history()
        if attn_topk > 0:
            o = attn_decode_topk(qkv, b, d.nh, d.hd, kh, vh, cache.lmax, pos,
                                 topk_count(pos, attn_topk))
        else:
            o = attn_decode(qkv, b, d.nh, d.hd, kh, vh, cache.lmax, pos)
        cache.store(q3[:, :, 1, :], q3[:, :, 2, :], pos)
    else:
        assert attn_topk == 0
        cache.store(q3[:, :, 1, :], q3[:, :, 2, :], pos)
        kh, vh = cache.history()
        kq = np.ascontiguousarray(kh[:, :, pos, :]).reshape(b, d.h1)
        vq = np.ascontiguousarray(vh[:, :, pos, :]).reshape(b, d.h1)
        qkv2 = np.concatenate([qkv[:, :d.h1], kq, vq], axis=1)
        o = attn_decode(qkv2, b, d.nh, d.hd, kh, vh, cache.lmax, pos)
    x = linear(o, W["w_o"], W["b_o"], residual=x)
    a = layernorm(x, W["ln2_g"], W["ln2_b"])
    f = linear(a, W["w_1"], W["b_1"], relu=True)
    return linear(f, W["w_2"], W["b_2"], residual=x), o, qkv


# --------------------------------------------------------------------- model
def dequant_layer(d: Dims, Wq: dict) -> dict:
    """fp16 view of a 4-bit layer: each matrix replaced by dequant(codes, meta)."""
    W = {k: v for k, v in Wq.items() if not k.startswith(("c_", "m_"))}
    shapes = {"qkv": (3 * d.h1, d.h1), "o": (d.h1, d.h1), "1": (d.h2, d.h1), "2": (d.h1, d.h2)}
    for name, (N, K) in shapes.items():
        if "w_" + name not in W:
            W["w_" + name] = dequant_weight(Wq["c_" + name], Wq["m_" + name], N, K)
    return W


def quant_layer(d: Dims, W: dict) -> dict:
    """4-bit copy of a layer's four matrices (codes c_*, meta m_*); the rest kept fp16."""
    Wq = {k: v for k, v in W.items() if not k.startswith("w_")}
    for name in ("qkv", "o", "1", "2"):
        Wq["c_" + name], Wq["m_" + name] = quant_weight(W["w_" + name])
    return Wq


def lm_head(x_last, lnf_g, lnf_b, E):
    """Final LayerNorm then the tied output projection (logits = LN(x) E^T)."""
    a = layernorm(x_last, lnf_g, lnf_b)
    return linear(a, E)


class Model:
    """Whole-model oracle.  layers: list of fp16 layer dicts (dequantized Ŵ for
    4-bit weights).  Generation order follows [P2] "从硬件画像得到每层时间" (T = l T_pre + l(n-1) T_gen):
    the prefill yields the first generated token and each of the n-1 decode
    steps one more."""

    def __init__(self, d: Dims, layers, E, P, lnf_g, lnf_b, kv_fmt: str, lmax: int, b: int):
        self.d, self.layers, self.E, self.P = d, layers, _u16(E), _u16(P)
        self.lnf_g, self.lnf_b = _u16(lnf_g), _u16(lnf_b)
        self.caches = [KVCache(kv_fmt, b, d.nh, d.hd, lmax) for _ in layers]
        self.b, self.lmax = b, lmax

    def prefill(self, tokens):
        tokens = np.asarray(tokens, np.int32)
        b, s = tokens.shape
        assert b == self.b
        pos = np.tile(np.arange(s, dtype=np.int32), b)
        x = embed(tokens.reshape(-1), pos, self.E, self.P)
        for W, c in zip(self.layers, self.caches):
            x = layer_prefill(self.d, W, x, b, s, c)
        last = x.reshape(b, s, -1)[:, s - 1, :]
        logits = lm_head(last, self.lnf_g, self.lnf_b, self.E)
        return logits, argmax(logits)

    def decode(self, tok, pos: int, attn_topk: float = 0.0):
        tok = np.asarray(tok, np.int32).reshape(-1)
        x = embed(tok, np.full(tok.size, pos, np.int32), self.E, self.P)
        for W, c in zip(self.layers, self.caches):
            x, _, _ = layer_decode(self.d, W, x, pos, c, attn_topk=attn_topk)
        logits = lm_head(x, self.lnf_g, self.lnf_b, self.E)
        return logits, argmax(logits)


# ---------------------------------------------------------- closed-form sizes
def weight_bytes_f16(h1: int, h2: int, l: int) -> int:
    """[P2] "从 Transformer 推理的数据流重新定义卸载": M_W = l (8 h1^2 + 4 h1 h2)
    bytes in fp16 (four h1 x h1 attention matrices, two MLP matrices)."""
    return l * (8 * h1 * h1 + 4 * h1 * h2)


def kv_bytes_f16(h1: int, l: int, b: int, s: int, n: int) -> int:
    """[P2] same section: M_KV = 4 b l h1 (s + n) bytes (K and V, 2 bytes each)."""
    return 4 * b * l * h1 * (s + n)


def q4_bytes(n_elems: int, group: int = 64) -> int:
    """4-bit codes plus an fp16 (min, scale) pair per group ([P1] §6.3)."""
    return n_elems // 2 + (n_elems // group) * 4
