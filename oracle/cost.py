"""Oracle of the offloading cost model and policy search.

TEST INFRASTRUCTURE ONLY (see the package docstring): the plain definition
of the per-layer times and the policy objective, evaluated term by term, and
an exhaustive search over a grid of placements.  The product's linear-program
search is checked against it.

Source: [P2] "FlexGen 完全拆解", sections "用线性规划搜索卸载策略" (the 11
policy variables and the three conservation equations), "从硬件画像得到每层
时间" (T_pre, T_gen as the max of five paths, T = l T_pre + l (n-1) T_gen,
and the disk -> CPU decode term), "为什么固定批量后能变成线性规划" (minimize
T / bls subject to peak memory within each tier's capacity), "FlexGen 的核心:
计算图分块与张量生命周期" (bls = gbs x GPU batches; peak memory terms) and
"从 Transformer 推理的数据流重新定义卸载" (M_W, M_KV).

Where the pages print only one path (disk -> CPU in decode) the others follow
the same pattern (the readings are listed with the design notes):
  * bytes are per layer and per pass of the whole block (bls sequences);
    weights W = 8 h1^2 + 4 h1 h2 in fp16, times the weight compression ratio;
    cache 4 bls L h1 (K and V, fp16) times the cache compression ratio;
    activations 2 bls h1 per token;
  * whatever is not on the GPU crosses CPU -> GPU (disk-resident data passes
    through the CPU); what the layer produces (new cache entries, output
    activations) goes back GPU -> CPU, and on to disk for the disk share;
  * decode uses the average cache length s + n/2; prefill moves no cache in
    and writes s positions out;
  * compute: a decode layer's projections take the longer of their flops
    (2 per weight element per token) at the GPU's GEMM rate and their
    weight bytes at HBM bandwidth; decode attention is the cache bytes read
    at the GPU's attention bandwidth; prefill runs its projections and
    2 bls s^2 h1 causal attention flops at the prompt GEMM rate.

CPU delegation of decode attention ([P2] "为什么有时应该在 CPU 上算注意力": for
a cache already on the CPU side, computing its attention there moves the
current token's activations instead of the cache), as a policy switch: in
decode, the CPU share of the cache (cc) no longer crosses
CPU -> GPU nor comes back; instead each of its sequences sends its q, k, v
rows down (3 h1 fp16) and its attention row up (h1 fp16), the CPU reads that
share of the cache at its attention bandwidth (a sixth path, "cpu", which
overlaps the others like them), and the GPU's attention reads only the
other shares.  The pages' authors switch the delegation off with a
compressed cache, because on their host the CPU's dequantization costs what
the smaller transfer saves; here that is left to the rates: a compressed
cache is read at a rate of its own (stored bytes per second), and without
one the switch is refused.  Parity unpinned for the CPU rates (measured
constants, as the GPU's rates are).
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass

import numpy as np

PATHS = ("c2g", "g2c", "d2c", "c2d", "comp", "cpu")


@dataclass(frozen=True)
class Model:
    l: int
    h1: int
    h2: int
    s: int
    n: int
    w_ratio: float = 1.0      # stored weight bytes / fp16 bytes (4-bit g64: 9/32)
    c_ratio: float = 1.0      # stored cache bytes / fp16 bytes


@dataclass(frozen=True)
class Hardware:
    bw_c2g: float             # bytes/s
    bw_g2c: float
    bw_d2c: float
    bw_c2d: float
    gemm_flops: float         # flop/s (decode-shaped products)
    prefill_flops: float      # flop/s (prompt-shaped products and attention)
    attn_bw: float            # bytes/s of cache read by decode attention
    hbm_bw: float             # bytes/s of weights read by decode projections
    cap_g: float              # bytes
    cap_c: float
    cap_d: float
    alpha_g: float = 1.0      # peak memory is multiplied by these before the
    alpha_c: float = 1.0      # capacity test
    alpha_d: float = 1.0
    cpu_attn_bw: float = 0.0  # bytes/s of fp16 cache read by decode attention on the CPU (0: none)
    cpu_attn_bw_q4: float = 0.0  # the same for a compressed cache, stored bytes/s (0: none)


def layer_weight_bytes(m: Model) -> float:
    """[P2] M_W / l: four h1 x h1 attention matrices and two MLP matrices, fp16."""
    return (8 * m.h1 * m.h1 + 4 * m.h1 * m.h2) * m.w_ratio


def cache_bytes(m: Model, bls: int, length: float) -> float:
    """K and V of bls sequences over `length` positions for one layer."""
    return 4 * bls * length * m.h1 * m.c_ratio


def act_bytes(m: Model, bls: int, tokens: float) -> float:
    return 2 * bls * tokens * m.h1


def path_times(m: Model, hw: Hardware, bls: int, p: dict, phase: str, cpu_attn: bool = False) -> dict:
    """Seconds per layer on each of the six paths for placement p (keys
    wg wc wd hg hc hd cg cc cd) in phase "pre" or "gen"; cpu_attn: decode
    attention of the CPU-resident cache share on the CPU."""
    W = layer_weight_bytes(m)
    off_w = p["wc"] + p["wd"]
    off_c = p["cc"] + p["cd"]
    off_h = p["hc"] + p["hd"]
    mats = 8 * m.h1 * m.h1 + 4 * m.h1 * m.h2          # 2 x weight elements
    if phase == "gen":
        L = m.s + m.n / 2
        cache_in = cache_bytes(m, bls, L)
        cache_out = cache_bytes(m, bls, 1)
        act = act_bytes(m, bls, 1)
        comp = max(bls * mats / hw.gemm_flops, W / hw.hbm_bw) + cache_bytes(m, bls, L) / hw.attn_bw
    else:
        cache_in = 0.0
        cache_out = cache_bytes(m, bls, m.s)
        act = act_bytes(m, bls, m.s)
        comp = (bls * m.s * mats + 2 * bls * m.s * m.s * m.h1) / hw.prefill_flops
    if cpu_attn and phase == "gen":
        rate = hw.cpu_attn_bw if m.c_ratio == 1.0 else hw.cpu_attn_bw_q4
        assert rate > 0, "CPU attention needs the host's rate for this cache format"
        qkv_down, attn_up = 3 * act, act             # fp16 rows of the CPU share's sequences
        gpu_attn = cache_in * (1 - p["cc"]) / hw.attn_bw
        return {
            "c2g": (off_w * W + p["cd"] * cache_in + off_h * act + p["cc"] * attn_up) / hw.bw_c2g,
            "g2c": (p["cd"] * cache_out + off_h * act + p["cc"] * qkv_down) / hw.bw_g2c,
            "d2c": (p["wd"] * W + p["cd"] * cache_in + p["hd"] * act) / hw.bw_d2c,
            "c2d": (p["cd"] * cache_out + p["hd"] * act) / hw.bw_c2d,
            "comp": comp - cache_in / hw.attn_bw + gpu_attn,
            "cpu": p["cc"] * cache_in / rate,
        }
    return {
        "c2g": (off_w * W + off_c * cache_in + off_h * act) / hw.bw_c2g,
        "g2c": (off_c * cache_out + off_h * act) / hw.bw_g2c,
        "d2c": (p["wd"] * W + p["cd"] * cache_in + p["hd"] * act) / hw.bw_d2c,
        "c2d": (p["cd"] * cache_out + p["hd"] * act) / hw.bw_c2d,
        "comp": comp,
        "cpu": 0.0,
    }


def phase_memory(m: Model, bls: int, gbs: int, p: dict, phase: str) -> dict:
    """Bytes held per tier during phase "pre" (the prompt: cache at s
    positions, activations of s tokens per sequence) or "gen" (a decode step:
    cache at its full length s + n, activations of one token per sequence).

    Each tier holds its share of all layers' weights, of the block's cache and
    of the block's activations.  The GPU also holds two layers' worth of the
    off-GPU weight share and two GPU batches' worth of the off-GPU cache share
    (the double buffers the transfers fill) and one GPU batch's working set
    (QKV, attention output, MLP hidden) for the phase's tokens.

    [P2] "FlexGen 的核心:计算图分块与张量生命周期" gives the decode-phase peak
    of a tier that holds one layer's weights, the activations and the whole
    block's cache as w + 2 h1 bls + 4 h1 bls l (s + n): with a weight share
    of 1/l and the whole cache and activation shares on that tier, the "gen"
    figure here is exactly that sum."""
    W = layer_weight_bytes(m)
    length, tokens = (m.s + m.n, 1) if phase == "gen" else (m.s, m.s)
    kv_all = m.l * cache_bytes(m, bls, length)
    act = act_bytes(m, bls, tokens)
    work = 2 * gbs * tokens * (5 * m.h1 + m.h2)
    stage_w = 2 * W * (1 - p["wg"])
    stage_c = 2 * cache_bytes(m, gbs, length) * (1 - p["cg"])
    return {
        "g": p["wg"] * m.l * W + p["cg"] * kv_all + p["hg"] * act + work + stage_w + stage_c,
        "c": p["wc"] * m.l * W + p["cc"] * kv_all + p["hc"] * act,
        "d": p["wd"] * m.l * W + p["cd"] * kv_all + p["hd"] * act,
    }


def peak_memory(m: Model, bls: int, gbs: int, p: dict) -> dict:
    """Bytes held per tier at the peak of the run: the larger of the prompt
    phase and a decode step at full cache length."""
    pre = phase_memory(m, bls, gbs, p, "pre")
    gen = phase_memory(m, bls, gbs, p, "gen")
    return {t: max(pre[t], gen[t]) for t in "gcd"}


def total_time(m: Model, hw: Hardware, bls: int, p: dict, cpu_attn: bool = False) -> float:
    """[P2]: T = l T_pre + l (n - 1) T_gen, each T the max over the paths."""
    t_pre = max(path_times(m, hw, bls, p, "pre").values())
    t_gen = max(path_times(m, hw, bls, p, "gen", cpu_attn).values())
    return m.l * t_pre + m.l * (m.n - 1) * t_gen


def feasible(m: Model, hw: Hardware, bls: int, gbs: int, p: dict, tol: float = 1e-9) -> bool:
    for k in ("w", "h", "c"):
        if abs(p[k + "g"] + p[k + "c"] + p[k + "d"] - 1) > tol:
            return False
        if min(p[k + "g"], p[k + "c"], p[k + "d"]) < -tol:
            return False
    pk = peak_memory(m, bls, gbs, p)
    return hw.alpha_g * pk["g"] <= hw.cap_g * (1 + tol) and \
        hw.alpha_c * pk["c"] <= hw.cap_c * (1 + tol) and \
        hw.alpha_d * pk["d"] <= hw.cap_d * (1 + tol) + tol


def objective(m: Model, hw: Hardware, bls: int, p: dict, cpu_attn: bool = False) -> float:
    """Seconds per sequence, T / bls (the quantity the search minimizes)."""
    return total_time(m, hw, bls, p, cpu_attn) / bls


def grid_search(m: Model, hw: Hardware, bls: int, gbs: int, step: float, cpu_attn: bool = False):
    """Every placement whose fractions are multiples of `step`; returns the
    feasible one of least T / bls and its value (None, inf if none).  With no
    disk capacity only placements without a disk share are visited (any
    other needs disk room for a positive number of bytes)."""
    k = int(round(1 / step))
    if hw.cap_d > 0:
        pairs = [(a * step, b * step) for a in range(k + 1) for b in range(k + 1 - a)]
    else:
        pairs = [(a * step, 1.0 - a * step) for a in range(k + 1)]
    best, best_v = None, np.inf
    for (wg, wc), (hg, hc), (cg, cc) in itertools.product(pairs, pairs, pairs):
        p = {"wg": wg, "wc": wc, "wd": max(0.0, 1 - wg - wc),
             "hg": hg, "hc": hc, "hd": max(0.0, 1 - hg - hc),
             "cg": cg, "cc": cc, "cd": max(0.0, 1 - cg - cc)}
        if not feasible(m, hw, bls, gbs, p):
            continue
        v = objective(m, hw, bls, p, cpu_attn)
        if v < best_v:
            best, best_v = p, v
    return best, best_v
