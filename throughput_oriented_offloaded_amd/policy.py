"""Offloading policy search: the pages' cost model and linear program, with
hardware constants fitted to one MI355X.

"FlexGen 完全拆解" (pinghaoyang.com.cn), sections "用线性规划搜索卸载策略",
"从硬件画像得到每层时间" and "为什么固定批量后能变成线性规划"; bjbfmj.com
walkthrough §6.2 (cost_model.py: search a policy under GPU / CPU / disk
capacities, or estimate a given one, with hardware constants re-fitted per
machine).

A policy is (bls, gbs) and the shares of weights (w), activations (h) and KV
cache (c) on GPU, CPU and disk.  For fixed (bls, gbs) every transfer time,
the compute time and every tier's peak memory are affine in the nine shares,
so the best shares solve a linear program: minimize
(l z_pre + l (n - 1) z_gen) / bls with z_pre, z_gen at least each path's time
in their phase, peak memory x alpha within each capacity, and each tensor
class's shares summing to one.  The search solves it for every (gbs, number
of GPU batches) on a grid and keeps the best.

Per-layer bytes: weights (8 h1^2 + 4 h1 h2) x compression, cache
4 bls L h1 x compression, activations 2 bls h1 per token.  Off-GPU data crosses
CPU -> GPU (disk data through the CPU); new cache entries and outputs go back.
Decode uses the mean cache length s + n/2.  Compute on MI355X: a projection
costs the larger of its flops at the GEMM rate and its weight bytes at HBM
bandwidth (small batches read weights faster than they multiply them);
decode attention reads the cache at the attention kernel's bandwidth;
prefill runs its flops (projections and causal attention) at the prompt
GEMM rate.

CPU attention ("为什么有时应该在 CPU 上算注意力"): the decode attention of the
CPU-resident cache share can run on the host, which then
reads that share at its own bandwidth (a sixth path, "cpu") while only the
q, k, v rows of its sequences go down to the host (3 h1 fp16 each) and their
attention rows come back (h1 fp16), instead of the cache crossing to the
GPU; the GPU's attention reads the other shares only.  A compressed cache is
read at a rate of its own (the pages' authors switch the delegation off with
compression, their CPU's dequantization being too slow; here the measured
rates decide).  The search tries the policy both ways where the machine has
a CPU rate for the workload's cache format.
"""
from __future__ import annotations

import argparse
import json
from dataclasses import asdict, dataclass

import numpy as np

SHARES = ("wg", "wc", "wd", "hg", "hc", "hd", "cg", "cc", "cd")
PATHS = ("c2g", "g2c", "d2c", "c2d", "comp", "cpu")
Q4G64 = 9.0 / 32.0          # 4-bit codes + fp16 (min, scale) per 64, over fp16


@dataclass(frozen=True)
class Workload:
    l: int
    h1: int
    h2: int
    s: int
    n: int
    w_ratio: float = 1.0
    c_ratio: float = 1.0


@dataclass(frozen=True)
class Machine:
    bw_c2g: float            # bytes/s, pinned host -> device
    bw_g2c: float
    bw_d2c: float
    bw_c2d: float
    gemm_flops: float        # decode-shaped projections, flop/s
    prefill_flops: float     # prompt-shaped projections and attention, flop/s
    hbm_bw: float            # weight reads of small-batch projections, bytes/s
    attn_bw: float           # cache reads of decode attention, bytes/s
    cap_g: float             # bytes
    cap_c: float
    cap_d: float
    alpha_g: float = 1.0     # peak-memory multipliers (fragmentation, runtime)
    alpha_c: float = 1.0
    alpha_d: float = 1.0
    cpu_attn_bw: float = 0.0  # fp16 cache read by decode attention on the host, bytes/s (0: none)
    cpu_attn_bw_q4: float = 0.0  # 4-bit cache, stored bytes/s (0: none)


def mi355x(host_bytes: float = 1.0e12, disk_bytes: float = 0.0, disk_bw: float = 2.0e9) -> Machine:
    """One MI355X, constants measured by this package's benchmark:
    pinned host -> device 55.9 GB/s (KV history loads while copying; the
    reverse direction assumed equal), 4-bit decode GEMM 961 TFLOP/s at
    M = 144, prompt-shaped GEMMs and attention 1.09 PFLOP/s effective (OPT-175B
    prefill), decode attention 5.63 TB/s, weight streaming at 5.6 TB/s of the
    8 TB/s HBM.  288 GB of HBM with 10% held back (alpha_g 1.1).  Decode
    attention on 16 host threads, overlapped with the GPU's work, reads an
    fp16 cache at 300 GB/s and a 4-bit one at 165 GB/s of stored bytes
    (history bytes over the whole step).  Host memory and disk are
    machine-specific arguments (no disk tier by default)."""
    return Machine(bw_c2g=55.9e9, bw_g2c=55.9e9, bw_d2c=disk_bw, bw_c2d=disk_bw / 2,
                   gemm_flops=961e12, prefill_flops=1.09e15, hbm_bw=5.6e12, attn_bw=5.63e12,
                   cap_g=288e9, cap_c=host_bytes, cap_d=disk_bytes, alpha_g=1.1, cpu_attn_bw=300e9,
                   cpu_attn_bw_q4=165e9)


MODELS = {   # OPT shapes: layers, h1, h2
    "opt-1.3b": (24, 2048, 8192), "opt-6.7b": (32, 4096, 16384), "opt-13b": (40, 5120, 20480),
    "opt-30b": (48, 7168, 28672), "opt-66b": (64, 9216, 36864), "opt-175b": (96, 12288, 49152),
}


def cpu_rate(wl: Workload, mc: Machine) -> float:
    """Host attention rate for the workload's cache format (0: none)."""
    return mc.cpu_attn_bw if wl.c_ratio == 1.0 else mc.cpu_attn_bw_q4


def _affine(wl: Workload, mc: Machine, bls: int, gbs: int, cpu_attn: bool = False):
    """Coefficients of the nine shares: path times T[phase] = A f + b (6 x 9,
    6) for phase "pre" and "gen", and memory held M = P f + q (3 x 9, 3) for
    tiers g, c, d in each phase ("mem_pre", "mem_gen").  cpu_attn: decode
    attention of the host cache share on the host."""
    if cpu_attn and not cpu_rate(wl, mc) > 0:
        raise ValueError("CPU attention needs the host's attention rate for this cache format")
    h1, h2 = wl.h1, wl.h2
    W = (8 * h1 * h1 + 4 * h1 * h2) * wl.w_ratio
    mats = 8 * h1 * h1 + 4 * h1 * h2
    i = {k: j for j, k in enumerate(SHARES)}
    out = {}
    for ph in ("pre", "gen"):
        if ph == "gen":
            L = wl.s + wl.n / 2
            c_in, c_out, act = 4 * bls * L * h1 * wl.c_ratio, 4 * bls * h1 * wl.c_ratio, 2 * bls * h1
            comp = max(bls * mats / mc.gemm_flops, W / mc.hbm_bw) + c_in / mc.attn_bw
        else:
            c_in, c_out, act = 0.0, 4 * bls * wl.s * h1 * wl.c_ratio, 2 * bls * wl.s * h1
            comp = (bls * wl.s * mats + 2 * bls * wl.s * wl.s * h1) / mc.prefill_flops
        host_attn = cpu_attn and ph == "gen"
        A = np.zeros((6, 9))
        b = np.zeros(6)
        # CPU -> GPU: every off-GPU share of the layer's inputs (host
        # attention: the host share's attention rows instead of its cache)
        for k, v in (("wc", W), ("wd", W), ("cc", act if host_attn else c_in), ("cd", c_in),
                     ("hc", act), ("hd", act)):
            A[0, i[k]] += v / mc.bw_c2g
        # GPU -> CPU: new cache entries and outputs of the off-GPU shares
        # (host attention: the host share's q, k, v rows)
        for k, v in (("cc", 3 * act if host_attn else c_out), ("cd", c_out), ("hc", act), ("hd", act)):
            A[1, i[k]] += v / mc.bw_g2c
        for k, v in (("wd", W), ("cd", c_in), ("hd", act)):
            A[2, i[k]] += v / mc.bw_d2c
        for k, v in (("cd", c_out), ("hd", act)):
            A[3, i[k]] += v / mc.bw_c2d
        b[4] = comp
        if host_attn:                         # the host share leaves the GPU's attention
            A[4, i["cc"]] -= c_in / mc.attn_bw
            A[5, i["cc"]] += c_in / cpu_rate(wl, mc)
        out[ph] = (A, b)
    # peak memory per phase: the prompt (cache at s, activations of s tokens
    # per sequence) and a decode step (cache at s + n, one token); each
    # tier's peak is the larger of the two, so the LP bounds both
    for ph, length, tokens in (("pre", wl.s, wl.s), ("gen", wl.s + wl.n, 1)):
        kv_all = wl.l * 4 * bls * length * h1 * wl.c_ratio
        act_all = 2 * bls * tokens * h1
        P = np.zeros((3, 9))
        q = np.zeros(3)
        for t, tier in enumerate("gcd"):
            P[t, i["w" + tier]] += wl.l * W
            P[t, i["c" + tier]] += kv_all
            P[t, i["h" + tier]] += act_all
        # GPU extras: a batch's working set, double buffers of the off-GPU
        # weight share (2 layers) and cache share (2 GPU batches)
        stage_c = 2 * 4 * gbs * length * h1 * wl.c_ratio
        q[0] = 2 * gbs * tokens * (5 * h1 + h2) + 2 * W + stage_c
        P[0, i["wg"]] -= 2 * W
        P[0, i["cg"]] -= stage_c
        out["mem_" + ph] = (P, q)
    return out


def estimate(wl: Workload, mc: Machine, bls: int, gbs: int, shares: dict, cpu_attn: bool = False) -> dict:
    """Times, throughput and peak memory of one policy."""
    f = np.array([shares[k] for k in SHARES], dtype=np.float64)
    co = _affine(wl, mc, bls, gbs, cpu_attn)
    res = {}
    for ph in ("pre", "gen"):
        A, b = co[ph]
        res["paths_" + ph] = dict(zip(PATHS, (A @ f + b).tolist()))
        res["T_" + ph] = float(np.max(A @ f + b))
    held = [co["mem_" + ph][0] @ f + co["mem_" + ph][1] for ph in ("pre", "gen")]
    res["peak"] = dict(zip("gcd", np.maximum(held[0], held[1]).tolist()))
    res["T"] = wl.l * res["T_pre"] + wl.l * (wl.n - 1) * res["T_gen"]
    res["tokens_per_s"] = bls * wl.n / res["T"]
    res["decode_tokens_per_s"] = bls / (wl.l * res["T_gen"])
    return res


def solve(wl: Workload, mc: Machine, bls: int, gbs: int, limits: dict | None = None,
          cpu_attn: bool = False):
    """Best shares for fixed (bls, gbs): (shares, T / bls) or (None, inf).
    limits: optional {share: (low, high)} bounds, e.g. what an executor can
    realize (activations kept on the GPU, at most half of a layer's weights
    off it).  cpu_attn: decode attention of the host cache share on the host."""
    from scipy.optimize import linprog
    co = _affine(wl, mc, bls, gbs, cpu_attn)
    nv = 11                                   # nine shares, z_pre, z_gen
    rows, rhs = [], []
    for zi, ph in ((9, "pre"), (10, "gen")):
        A, b = co[ph]
        for r in range(len(PATHS)):           # A f + b <= z
            row = np.zeros(nv)
            row[:9] = A[r]
            row[zi] = -1.0
            rows.append(row)
            rhs.append(-b[r])
    for ph in ("pre", "gen"):
        P, q = co["mem_" + ph]
        for t, (cap, alpha) in enumerate(((mc.cap_g, mc.alpha_g), (mc.cap_c, mc.alpha_c),
                                          (mc.cap_d, mc.alpha_d))):
            row = np.zeros(nv)                # alpha (P f + q) <= cap in both phases
            row[:9] = alpha * P[t]
            rows.append(row)
            rhs.append(cap - alpha * q[t])
    A_eq = np.zeros((3, nv))
    for c in range(3):
        A_eq[c, 3 * c:3 * c + 3] = 1.0
    cost = np.zeros(nv)
    cost[9] = wl.l / bls
    cost[10] = wl.l * (wl.n - 1) / bls
    bounds = [(0.0, 1.0)] * 9 + [(0, None)] * 2
    for k, (lo, hi) in (limits or {}).items():
        bounds[SHARES.index(k)] = (lo, hi)
    r = linprog(cost, A_ub=np.array(rows), b_ub=np.array(rhs), A_eq=A_eq, b_eq=np.ones(3),
                bounds=bounds, method="highs")
    if r.status != 0:
        return None, float("inf")
    f = np.clip(r.x[:9], 0.0, 1.0) + 0.0      # (+ 0.0: no negative zeros)
    for c in range(3):                        # renormalize solver round-off
        f[3 * c:3 * c + 3] /= f[3 * c:3 * c + 3].sum()
    return dict(zip(SHARES, f.tolist())), float(r.fun)


def search(wl: Workload, mc: Machine, gbs_list=(8, 16, 24, 32, 48, 64, 96, 128, 192, 256),
           nb_max: int = 64, limits: dict | None = None, cpu_attn: bool | None = None):
    """The (gbs, nb, shares, cpu attention) of least T / bls over gbs_list x
    1..nb_max.  cpu_attn None: both ways where the machine has a host
    attention rate for the cache format, else without."""
    if cpu_attn is None:
        modes = (False, True) if cpu_rate(wl, mc) > 0 else (False,)
    else:
        modes = (cpu_attn,)
    best = None
    for ca in modes:
        for gbs in gbs_list:
            for nb in range(1, nb_max + 1):
                shares, v = solve(wl, mc, gbs * nb, gbs, limits, ca)
                if shares is not None and (best is None or v < best[3]):
                    best = (gbs, nb, shares, v, ca)
    if best is None:
        return None
    gbs, nb, shares, v, ca = best
    return {"gbs": gbs, "num_gpu_batches": nb, "bls": gbs * nb, "shares": shares, "cpu_attention": ca,
            "seconds_per_sequence": v, **estimate(wl, mc, gbs * nb, gbs, shares, ca)}


def executor_limits(fp16_weights: bool) -> dict:
    """Shares this package's executor can realize on one GPU: activations stay
    in HBM; weights go to pinned host memory only for fp16 layers and only
    their W_Q, W_K rows and W_1 (half of a layer); no disk tier."""
    lim = {"hg": (1.0, 1.0), "hc": (0.0, 0.0), "hd": (0.0, 0.0), "wd": (0.0, 0.0), "cd": (0.0, 0.0)}
    lim["wc"] = (0.0, 0.5) if fp16_weights else (0.0, 0.0)
    return lim


def realize(wl: Workload, shares: dict, nb: int) -> dict:
    """The executor's placement nearest above an LP solution: the weight share
    off the GPU rounded up to whole tiered layers (each moves half a layer),
    the cache share rounded up to whole GPU batches.  Returns the number of
    tiered layers, the layers themselves (evenly spaced), the host-resident
    GPU batches and the realized shares."""
    n_tiered = min(wl.l, int(np.ceil(shares["wc"] * 2 * wl.l - 1e-9)))
    nb_host = min(nb, int(np.ceil(shares["cc"] * nb - 1e-9)))
    layers = [j for j in range(wl.l) if (j + 1) * n_tiered // wl.l > j * n_tiered // wl.l]
    sh = {"wg": 1 - n_tiered / (2 * wl.l), "wc": n_tiered / (2 * wl.l), "wd": 0.0,
          "hg": 1.0, "hc": 0.0, "hd": 0.0,
          "cg": 1 - nb_host / nb, "cc": nb_host / nb, "cd": 0.0}
    return {"n_tiered": n_tiered, "tiered_layers": layers, "kv_host_batches": nb_host, "shares": sh}


def search_realized(wl: Workload, mc: Machine, gbs_list=(16, 32, 48, 64), nb_max: int = 8,
                    limits: dict | None = None):
    """The executor's best placement: every (gbs, nb, CPU attention) point's
    LP optimum under `limits`, rounded by realize() and costed as realized
    (CPU attention only where a whole GPU batch's cache ends up on the host);
    the realized placement of least T / bls among those that fit the
    capacities.  Rounding can reverse the LP's ranking: a small host cache
    share with CPU attention wins the continuous program, and the whole GPU
    batch it becomes may leave the host attending far more than it should."""
    modes = (False, True) if cpu_rate(wl, mc) > 0 else (False,)
    best = None
    for ca in modes:
        for gbs in gbs_list:
            for nb in range(1, nb_max + 1):
                bls = gbs * nb
                shares, v_lp = solve(wl, mc, bls, gbs, limits, ca)
                if shares is None:
                    continue
                r = realize(wl, shares, nb)
                ca_r = ca and r["kv_host_batches"] > 0
                est = estimate(wl, mc, bls, gbs, r["shares"], ca_r)
                pk = est["peak"]
                if pk["g"] * mc.alpha_g > mc.cap_g or pk["c"] * mc.alpha_c > mc.cap_c or \
                        pk["d"] * mc.alpha_d > mc.cap_d + 1e-9:
                    continue
                v = est["T"] / bls
                if best is None or v < best["seconds_per_sequence"]:
                    best = {"gbs": gbs, "num_gpu_batches": nb, "bls": bls, "lp_shares": shares,
                            "lp_seconds_per_sequence": v_lp, "cpu_attention": ca_r, **r,
                            "seconds_per_sequence": v, "estimate": est}
    return best


def main(argv=None):
    ap = argparse.ArgumentParser(description="offloading policy search / estimate on one MI355X")
    ap.add_argument("--model", default="opt-175b", choices=sorted(MODELS))
    ap.add_argument("--prompt-len", type=int, default=512)
    ap.add_argument("--gen-len", type=int, default=32)
    ap.add_argument("--cpu-mem", type=float, default=1000.0, help="GB of host memory")
    ap.add_argument("--disk-mem", type=float, default=0.0, help="GB of disk")
    ap.add_argument("--compress", choices=("none", "w", "wc"), default="wc",
                    help="4-bit group-64 compression of weights (w) and cache (c)")
    ap.add_argument("--gpu-batch-size", type=int)
    ap.add_argument("--num-gpu-batches", type=int)
    ap.add_argument("--percent", type=float, nargs=6,
                    help="wg wc cg cc hg hc in percent (disk = the rest): estimate this policy")
    ap.add_argument("--cpu-attention", choices=("auto", "on", "off"), default="auto",
                    help="decode attention of the host cache share on the host")
    a = ap.parse_args(argv)
    l, h1, h2 = MODELS[a.model]
    wl = Workload(l, h1, h2, a.prompt_len, a.gen_len,
                  w_ratio=Q4G64 if a.compress in ("w", "wc") else 1.0,
                  c_ratio=Q4G64 if a.compress == "wc" else 1.0)
    mc = mi355x(a.cpu_mem * 1e9, a.disk_mem * 1e9)
    if a.percent:
        wg, wc, cg, cc, hg, hc = (x / 100 for x in a.percent)
        sh = {"wg": wg, "wc": wc, "wd": 1 - wg - wc, "cg": cg, "cc": cc, "cd": 1 - cg - cc,
              "hg": hg, "hc": hc, "hd": 1 - hg - hc}
        gbs, nb = a.gpu_batch_size or 48, a.num_gpu_batches or 3
        ca = a.cpu_attention == "on"
        out = {"gbs": gbs, "num_gpu_batches": nb, "shares": sh, "cpu_attention": ca,
               **estimate(wl, mc, gbs * nb, gbs, sh, ca)}
    else:
        out = search(wl, mc, cpu_attn=None if a.cpu_attention == "auto" else a.cpu_attention == "on")
    print(json.dumps({"workload": asdict(wl), "policy": out}, indent=1))


if __name__ == "__main__":
    main()
