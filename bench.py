"""Benchmark: zig-zag block decode of an OPT-shape decoder with 4-bit weights and
4-bit KV cache on one MI355X.

A step is one decode step of the whole model for the whole block: embed, every
layer (LN1, QKV dequant-GEMM, decode attention over the 4-bit cache, the new
token's K/V append, out-proj, LN2, FC1, FC2), final LN, LM head and greedy pick, for
bls = gbs x nb sequences at once.  Before the timed region the prompt (s
tokens per sequence) is prefilled and W warm-up steps run; the K timed steps
then generate positions s .. s+K-1 again from the prefill's first token, so
the timed steps are exactly the decode phase of an n = K+1 token generation.

Printed: one JSON line (stdout) with decode tokens/s, the per-kernel roofline
of the dominant kernel (measured live with HIP events on the launch stream
during the timed region), the decode-attention roofline, the pages' generation
throughput, and the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 31] [--warmup 2] [--config 5]
"""
from __future__ import annotations

import argparse
import faulthandler
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s (s=512,n=32) + attn HBM GB/s, dequant-GEMM MFMA % of peak"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

CONFIGS = {
    1: dict(workload="opt-125m-shape 4-bit block decode", l=2, h1=768, h2=3072, nh=12, hd=64,
            w="q4", kv="q4", gbs=4, nb=1, s=32, n=8),
    2: dict(workload="opt-1.3b-shape fp16 block decode", l=24, h1=2048, h2=8192, nh=32, hd=64,
            w="f16", kv="f16", gbs=32, nb=4, s=512, n=32),
    3: dict(workload="opt-30b-shape 4-bit block decode", l=48, h1=7168, h2=28672, nh=56, hd=128,
            w="q4", kv="q4", gbs=48, nb=3, s=512, n=32),
    4: dict(workload="opt-66b-shape fp16 block decode, 50% of weights in pinned host memory",
            l=64, h1=9216, h2=36864, nh=72, hd=128, w="f16", kv="q4", gbs=32, nb=8, s=512, n=32,
            tier=True),
    5: dict(workload="opt-175b-shape 4-bit block decode", l=96, h1=12288, h2=49152, nh=96,
            hd=128, w="q4", kv="q4", gbs=48, nb=3, s=512, n=32),
    6: dict(workload="opt-30b-shape 4-bit block decode, KV cache of every GPU batch in pinned "
                     "host memory", l=48, h1=7168, h2=28672, nh=56, hd=128, w="q4", kv="q4",
            gbs=48, nb=3, s=512, n=32, kv_host_seqs=144),
    7: dict(workload="opt-30b-shape fp16 block decode, 50% of weights in pinned host memory",
            l=48, h1=7168, h2=28672, nh=56, hd=128, w="f16", kv="q4", gbs=32, nb=8, s=512, n=32,
            tier=True),
    # the pages' CPU delegation of attention: the same fp16 cache placement,
    # with the host batches' history moved to the device (8) or their
    # attention computed on the host CPU (9)
    8: dict(workload="opt-1.3b-shape fp16 block decode, fp16 KV cache of two of four GPU batches in "
                     "pinned host memory, moved through the device slots",
            l=24, h1=2048, h2=8192, nh=32, hd=64, w="f16", kv="f16", gbs=32, nb=4, s=512, n=32,
            kv_host_seqs=64),
    9: dict(workload="opt-1.3b-shape fp16 block decode, fp16 KV cache of two of four GPU batches in "
                     "pinned host memory, their attention on the host CPU",
            l=24, h1=2048, h2=8192, nh=32, hd=64, w="f16", kv="f16", gbs=32, nb=4, s=512, n=32,
            kv_host_seqs=64, kv_host_attention=True),
    # config 6 with the host batches' attention on the host CPU over the
    # 4-bit cache (read compressed), instead of moving the history over PCIe
    10: dict(workload="opt-30b-shape 4-bit block decode, KV cache of every GPU batch in pinned "
                      "host memory, attention on the host CPU", l=48, h1=7168, h2=28672, nh=56, hd=128,
             w="q4", kv="q4", gbs=48, nb=3, s=512, n=32, kv_host_seqs=144, kv_host_attention=True),
}
# Workloads that are not run: an earlier version of the OPT-66B-shape tiered run
# ended in a host segmentation fault after its timed decode, and the cause has
# not been found.
REFUSED = {4: "the OPT-66B-shape weight-tiering run is not taken: an earlier version of it ended in "
              "a host segmentation fault after its timed decode, with no cause found; config 7 "
              "measures the same weight tiering at the OPT-30B shape"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu_threads() -> int:
    """CPU threads for host-side attention: the process's CPU share
    (OMP_NUM_THREADS when set, else its affinity), at most 16."""
    n = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    return max(1, min(16, n))


def build_model(cfg, keep_layer0_host: bool):
    import torch
    import synth
    from throughput_oriented_offloaded_amd import _lib as L
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape, TierLayer

    fmt = lambda f: L.FG_FMT_Q4G64 if f == "q4" else L.FG_FMT_F16  # noqa: E731
    sh = Shape(n_layers=cfg["l"], h1=cfg["h1"], h2=cfg["h2"], n_heads=cfg["nh"], head_dim=cfg["hd"])
    tiered = cfg.get("tier_layers")
    if tiered is None and cfg.get("tier"):
        tiered = range(cfg["l"])
    tiered = set(tiered or ())
    layers, tier, host0 = [], ([] if tiered else None), None
    L.fg_trace_enable(True)            # time the weight quantizer (init, not in the step)
    for j in range(sh.n_layers):
        W = synth.layer_weights(sh.h1, sh.h2, j, seed=0, device="cuda")
        if j == 0 and keep_layer0_host:
            host0 = {k: v.cpu() for k, v in W.items()}
        if j in tiered:                # half of the layer's fp16 weights to pinned host memory
            dl, tl = TierLayer.split(W, fmt(cfg["w"]))
            layers.append(dl)
            tier.append(tl)
        elif tier is not None:
            layers.append(DeviceLayer.from_fp16(W, fmt(cfg["w"])))
            tier.append(None)
        else:
            layers.append(DeviceLayer.from_fp16(W, fmt(cfg["w"])))
        del W
        if j % 16 == 0:
            log(f"  layer {j}/{sh.n_layers} ready")
    torch.cuda.synchronize()
    quant = L.fg_trace_collect().get("quant_g4")
    L.fg_trace_enable(False)
    torch.cuda.empty_cache()
    emb = synth.embeddings(sh.h1, cfg["s"] + cfg["n"], seed=0, device="cuda")
    return sh, layers, tier, emb, host0, quant, fmt


def profile_layer(cfg, reps: int):
    """One decoder layer at the config's shape for hardware-counter runs: the
    prefill fills its cache to s, then `reps` decode steps of the whole block
    (the launches the step times), the same `reps` steps again with Top-K
    sparse V at 10% (rewriting those cache rows), then a plain 1 GiB
    device-to-device copy (reads and writes 1 GiB: the calibration of the
    byte counters)."""
    import torch
    import synth
    from throughput_oriented_offloaded_amd import _lib as L
    from throughput_oriented_offloaded_amd.model import DeviceKV, DeviceLayer, Shape
    fmt = lambda f: L.FG_FMT_Q4G64 if f == "q4" else L.FG_FMT_F16  # noqa: E731
    sh = Shape(n_layers=1, h1=cfg["h1"], h2=cfg["h2"], n_heads=cfg["nh"], head_dim=cfg["hd"])
    gbs, nb, s = cfg["gbs"], cfg["nb"], cfg["s"]
    bls, d = gbs * nb, sh.dims
    lay = DeviceLayer.from_fp16(synth.layer_weights(sh.h1, sh.h2, 0, seed=0, device="cuda"),
                                fmt(cfg["w"]))
    kv = DeviceKV(fmt(cfg["kv"]), bls, sh.n_heads, sh.head_dim, s + reps, "cuda")
    ws_b = max(L.fg_workspace_bytes(d, gbs * s, lay.fmt), L.fg_workspace_bytes(d, bls, lay.fmt))
    ws = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    x = synth.activations(bls * s, sh.h1, seed=1, device="cuda")
    L.fg_layer_prefill(d, lay.struct, x, gbs, nb, s, kv.struct, ws, ws_b)
    del x
    xd = synth.activations(bls, sh.h1, seed=2, device="cuda")
    torch.cuda.synchronize()
    log(f"profile-layer: {cfg['workload']}, {reps} decode steps from position {s}")
    for r in range(reps):
        L.fg_layer_decode_block(d, lay.struct, xd, gbs, nb, s + r, kv.struct, ws, ws_b)
    for r in range(reps):
        L.fg_layer_decode_block(d, lay.struct, xd, gbs, nb, s + r, kv.struct, ws, ws_b,
                                attn_topk_ppm=100000)
    torch.cuda.synchronize()
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("profile-layer: done")


# HBM bytes per launch from hardware counters (rocprofv3 FETCH_SIZE / WRITE_SIZE,
# calibrated on a copy of known size), committed per workload with the sha256
# of the measured kernel's sources; reported only while those are unchanged.
TRAFFIC_FILES = {5: "opt175b_q4_decode_hbm_traffic.md"}
TRACE_EVERY = 16    # timed steps between the ones whose roofline kernels carry events
TRACE_FIRST = 8     # the first of them (away from the start of the timed region)
KERNEL_SOURCES = {"gemm_q4": ["gemm_sk.hip", "gemm_sk32.hip", "gemm_common.h"],
                  "attn_decode_q4": ["attn_decode.hip", "codec_dev.h"],
                  "attn_topk_q4": ["attn_decode.hip", "codec_dev.h"]}


def traced_steps(K: int) -> int:
    """Timed steps that carry events: every TRACE_EVERY-th from TRACE_FIRST,
    or the first one when the run is shorter than that."""
    n = len(range(TRACE_FIRST, K, TRACE_EVERY))
    return n if n else 1


def measured_traffic(config: int, kind: str):
    import hashlib
    import re
    name = TRAFFIC_FILES.get(config)
    if not name or kind not in KERNEL_SOURCES:
        return None
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "throughput_oriented_offloaded_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    for line in open(path):
        m = re.match(r"traffic (\S+) (\d+) ([0-9a-f]{64})\s*$", line)
        if m and m.group(1) == kind:
            return int(m.group(2)) if m.group(3) == h.hexdigest() else None
    return None


def roofline(tr, kind, bound, config=None):
    r = tr.get(kind)
    if not r or r["ms"] <= 0:
        return None
    sec = r["ms"] / 1e3
    if bound == "mfma":
        ach = r["flops"] / sec / 1e12
        peak, unit = PEAK_F16_TFLOPS, "TFLOP/s"
    else:
        ach = r["bytes"] / sec / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": measured_traffic(config, kind), "kernel": kind,
            "launches": r["count"], "avg_launch_us": round(r["ms"] * 1e3 / r["count"], 2),
            "algorithmic_per_launch": (r["flops"] if bound == "mfma" else r["bytes"]) / r["count"]}


def topk_attention(model, cfg, L, pos: int, frac: float = 0.1, reps: int = 10):
    """Top-K sparse-V decode attention ([P2] "权重压缩与 KV Cache 压缩": V read
    for the highest-scoring 10% only) on layer 0's cache at history length pos,
    timed with the same HIP-event tracing, beside the dense kernel on the same
    cache.  Returns the sparse kernel's roofline plus both average durations."""
    import torch
    sh, bls = model.shape, model.kv[0].struct.n_seq   # device-resident sequences
    h1 = sh.h1
    topk = min(pos, -(-int(round(frac * 1_000_000)) * pos // 1_000_000))
    g = torch.Generator(device="cuda").manual_seed(11)
    qkv = (torch.randn((bls, 3 * h1), generator=g, device="cuda") * 2).half()
    out = torch.empty((bls, h1), dtype=torch.float16, device="cuda")
    kv = model.kv[0].struct
    q4 = cfg["kv"] == "q4"
    sparse = L.fg_attn_decode_topk_q4 if q4 else L.fg_attn_decode_topk_f16
    dense = L.fg_attn_decode_q4 if q4 else L.fg_attn_decode_f16
    ks, kd = ("attn_topk_q4", "attn_decode_q4") if q4 else ("attn_topk_f16", "attn_decode_f16")
    args = (qkv, qkv[:, h1:], qkv[:, 2 * h1:], 3 * h1, kv, bls, model.d, pos)
    for _ in range(3):
        sparse(*args, topk, 0, out)
        dense(*args, 0, out)
    torch.cuda.synchronize()
    L.fg_trace_kinds([ks, kd])
    L.fg_trace_enable(True)
    for _ in range(reps):
        sparse(*args, topk, 0, out)
        dense(*args, 0, out)
    torch.cuda.synchronize()
    tr = L.fg_trace_collect()
    L.fg_trace_enable(False)
    L.fg_trace_kinds(None)
    r = roofline(tr, ks, "hbm", cfg.get("id"))
    if r:
        r.update({"pos": pos, "topk": topk, "dense_avg_launch_us": round(tr[kd]["ms"] * 1e3 / tr[kd]["count"], 2),
                  "definition": "softmax over every score; V of the topk highest-scoring cached "
                                "positions plus the current token; bytes count the K history, the "
                                "topk V rows read, q/k/v and the output"})
    return r


def sparse_decode(model, cfg, L, tok1, steps: int, no_trace: bool, frac: float = 0.1):
    """Whole decode steps with Top-K sparse V attention at the pages' 10%
    (positions s .. s+steps-1, rewriting the cache rows the dense steps wrote):
    throughput of the same block, and the attention time per step."""
    import torch
    s, bls = cfg["s"], cfg["gbs"] * cfg["nb"]
    kind = "attn_topk_q4" if cfg["kv"] == "q4" else "attn_topk_f16"
    model.attn_topk_ppm = int(round(frac * 1_000_000))
    L.fg_trace_kinds([kind])
    L.fg_trace_enable(not no_trace)
    tok = tok1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        _, tok = model.decode_step(tok, s + i, cfg["gbs"], cfg["nb"])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    tr = L.fg_trace_collect() if not no_trace else {}
    L.fg_trace_enable(False)
    L.fg_trace_kinds(None)
    model.attn_topk_ppm = 0
    r = {"value": round(bls * steps / dt, 2), "unit": "tokens/s", "steps": steps,
         "ms_per_step": round(dt / steps * 1e3, 3), "frac": frac,
         "definition": "block decode steps (every layer) with attention reading the V rows of "
                       "ceil(frac * pos) top-scoring cached positions"}
    if kind in tr:
        r["attn_ms_per_step"] = round(tr[kind]["ms"] / steps, 3)
        r["roofline_attn"] = roofline(tr, kind, "hbm", cfg.get("id"))
    log(f"sparse-V decode: {r['ms_per_step']} ms/step")
    return r


def host_cpu():
    """The host's CPU model, logical CPUs, the CPUs this process may run on and
    the physical cores among them (sysfs topology), and the thread count of
    the all-cores runs: those physical cores, capped by OMP_NUM_THREADS."""
    import subprocess
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        model = next((ln.split(":", 1)[1].strip() for ln in out.splitlines()
                      if ln.startswith("Model name")), None)
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None and os.path.exists("/proc/cpuinfo"):
        model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                      if ln.startswith("model name")), None)
    aff = sorted(os.sched_getaffinity(0))
    cores = set()
    for c in aff:
        try:
            base = f"/sys/devices/system/cpu/cpu{c}/topology/"
            cores.add((open(base + "physical_package_id").read().strip(),
                       open(base + "core_id").read().strip()))
        except OSError:
            cores.add(("cpu", str(c)))
    cap = int(os.environ.get("OMP_NUM_THREADS", len(cores)) or len(cores))
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": len(aff),
            "usable_physical_cores": len(cores), "threads_all_cores": max(1, min(len(cores), cap))}


def gpu_config1():
    """Seconds of the config-1 generation on the GPU (prefill s = 32 and 7
    decode steps of a 2-layer OPT-125m-shape decoder, 4-bit weights and KV,
    bls 4): the second of two runs."""
    import torch
    import synth
    from throughput_oriented_offloaded_amd import _lib as L
    from throughput_oriented_offloaded_amd.model import DeviceLayer, Model, Shape
    c = CONFIGS[1]
    sh = Shape(n_layers=c["l"], h1=c["h1"], h2=c["h2"], n_heads=c["nh"], head_dim=c["hd"])
    layers = [DeviceLayer.from_fp16(synth.layer_weights(sh.h1, sh.h2, j, seed=0, device="cuda"),
                                    L.FG_FMT_Q4G64) for j in range(sh.n_layers)]
    emb = synth.embeddings(sh.h1, c["s"] + c["n"], seed=0, device="cuda")
    toks = synth.tokens(c["gbs"], c["s"], seed=0, device="cuda")
    m = Model(sh, layers, emb, L.FG_FMT_Q4G64, c["gbs"], c["s"] + c["n"])
    dt = 0.0
    for _ in range(2):
        torch.cuda.synchronize()
        t = time.perf_counter()
        m.generate(toks, c["n"], gbs=c["gbs"], nb=c["nb"])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
    return dt


def cpu_baseline(cfg, host0, emb, gpu: dict):
    """The oracle (as it is) on the host's cores, on the five units of the
    measurement plan, each at 1 thread and at all usable physical cores and
    each beside the GPU's time for the same unit.  Units at the benchmark's
    shape run on a bounded sample (a few rows, a slice of one matrix, two
    prompt tokens) and are scaled to the whole unit; the scale is stated per
    unit.  The oracle's cost does not depend on the weight values, so the
    layer's fp16 weights stand in for their dequantized copies.
    value: the oracle's decode tokens/s for the whole block at all cores,
    bls / (l * t_layer + t_head)."""
    import numpy as np
    import oracle
    import synth
    hc = host_cpu()
    n_all = hc["threads_all_cores"]
    d = oracle.Dims(cfg["h1"], cfg["h2"], cfg["nh"], cfg["hd"])
    h1, l, bls, s = cfg["h1"], cfg["l"], cfg["gbs"] * cfg["nb"], cfg["s"]
    ctx = s + cfg["n"] // 2
    Wn = {k: v.numpy().view(np.uint16) for k, v in host0.items()}
    kh, vh = synth.kv_history(4, cfg["nh"], ctx, cfg["hd"], seed=7)
    kh, vh = kh.numpy().view(np.uint16), vh.numpy().view(np.uint16)
    x = synth.activations(4, h1, seed=8).numpy().view(np.uint16)
    qkv = synth.activations(4, 3 * h1, seed=9).numpy().view(np.uint16)
    xp = synth.activations(2 * 2, h1, seed=10).numpy().view(np.uint16)
    E = emb["embed"].cpu().numpy().view(np.uint16)
    g, b = emb["lnf_g"].cpu().numpy().view(np.uint16), emb["lnf_b"].cpu().numpy().view(np.uint16)

    def cache(rows):
        c = oracle.KVCache(cfg["kv"], rows, cfg["nh"], cfg["hd"], ctx + 1)
        c.store(kh[:rows], vh[:rows], 0)
        return c

    def clock(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    # config 1 end to end (the whole unit, no scaling)
    c1 = CONFIGS[1]
    d1 = oracle.Dims(c1["h1"], c1["h2"], c1["nh"], c1["hd"])
    W1 = [oracle.dequant_layer(d1, oracle.quant_layer(d1, {k: v.numpy().view(np.uint16) for k, v in
                               synth.layer_weights(c1["h1"], c1["h2"], j, seed=0).items()}))
          for j in range(c1["l"])]
    e1 = {k: v.numpy().view(np.uint16) for k, v in synth.embeddings(c1["h1"], c1["s"] + c1["n"], seed=0).items()}
    t1 = synth.tokens(c1["gbs"], c1["s"], seed=0).numpy()

    def config1():
        om = oracle.Model(d1, W1, e1["embed"], e1["pos"], e1["lnf_g"], e1["lnf_b"], "q4",
                          c1["s"] + c1["n"], c1["gbs"])
        _, tok = om.prefill(t1)
        for i in range(1, c1["n"]):
            _, tok = om.decode(tok, c1["s"] + i - 1)

    quant_rows = 1024
    elems_layer = 8 * h1 * h1 + 4 * h1 * cfg["h2"]
    units = {
        "config1_end_to_end": dict(
            sample="the whole unit: prefill s=32 and 7 decode steps of the 2-layer OPT-125m-shape "
                   "4-bit decoder, bls 4", scale=1.0, gpu_s=gpu.get("config1_s"),
            run={1: config1, n_all: config1}),
        "quantize_one_layer": dict(
            sample=f"{quant_rows} rows ({quant_rows // 64} groups) of W_1, scaled to the layer's "
                   f"{elems_layer / 2:.4g} elements",
            scale=elems_layer / 2 / (quant_rows * h1), gpu_s=gpu.get("quant_layer_s"),
            run={th: (lambda: oracle.quant_weight(Wn["w_1"][:quant_rows])) for th in (1, n_all)}),
        "decode_attention_one_layer": dict(
            sample=f"1 sequence (1 thread) / 4 sequences (all cores) at context {ctx}: the "
                   f"oracle's cache dequantization and attention, scaled to bls {bls}",
            scale={1: bls / 1, n_all: bls / 4}, gpu_s=gpu.get("attn_layer_s"),
            run={1: None, n_all: None}),
        "decode_layer_block": dict(
            sample=f"1 sequence (1 thread) / 4 sequences (all cores) through one decoder layer "
                   f"at context {ctx}, scaled to bls {bls}",
            scale={1: bls / 1, n_all: bls / 4}, gpu_s=gpu.get("layer_decode_s"),
            run={1: None, n_all: None}),
        "prefill_one_layer_2_sequences": dict(
            sample=f"2 sequences x 2 prompt tokens through one decoder layer, scaled linearly to "
                   f"s = {s} (the projections are over 99% of the work)",
            scale=s / 2, gpu_s=gpu.get("prefill_layer_2seq_s"),
            run={th: (lambda: oracle.layer_prefill(d, Wn, xp, 2, 2, oracle.KVCache(cfg["kv"], 2, cfg["nh"],
                                                                                      cfg["hd"], 2)))
                 for th in (1, n_all)}),
    }
    out_units = {}
    t_head = None
    for name, u in units.items():
        res = {"sample": u["sample"]}
        for th in sorted({1, n_all}):
            oracle.set_threads(th)
            if name == "decode_attention_one_layer":
                rows = 1 if th == 1 else 4
                c = cache(rows)
                meas = clock(lambda: oracle.attn_decode(qkv[:rows], rows, cfg["nh"], cfg["hd"],
                                                        *c.history(), ctx + 1, ctx))
            elif name == "decode_layer_block":
                rows = 1 if th == 1 else 4
                c = cache(rows)
                meas = clock(lambda: oracle.layer_decode(d, Wn, x[:rows], ctx, c))
            else:
                meas = clock(u["run"][th])
            sc = u["scale"][th] if isinstance(u["scale"], dict) else u["scale"]
            key = "1_thread" if th == 1 else "all_cores"
            res["cpu_s_" + key] = round(meas * sc, 4)
            res["measured_s_" + key] = round(meas, 4)
            res["scale_" + key] = round(sc, 3)
        if u["gpu_s"]:
            res["gpu_s"] = round(u["gpu_s"], 6)
            res["gpu_speedup_vs_all_cores"] = round(res["cpu_s_all_cores"] / u["gpu_s"], 1)
        out_units[name] = res
    oracle.set_threads(n_all)
    t_head = clock(lambda: oracle.lm_head(x, g, b, E)) * bls / 4
    t_layer = out_units["decode_layer_block"]["cpu_s_all_cores"]
    tps = bls / (l * t_layer + t_head)
    return {"value": round(tps, 5), "unit": "tokens/s", "cores": n_all, "kind": "oracle",
            "sample": f"decode tokens/s of the whole block (bls {bls}) from the decode_layer_block "
                      f"unit at all cores ({t_layer:.1f} s per layer) times {l} layers plus the LM "
                      f"head ({t_head:.1f} s, 4 rows scaled to {bls}); every unit below at 1 thread "
                      f"and at all cores",
            "host": hc, "threads": {"one": 1, "all_cores": n_all}, "units": out_units}


def plan_policy(cfg, gpu_gb: float, host_gb: float):
    """The pages' cost model and LP search ("FlexGen 完全拆解", sections
    "用线性规划搜索卸载策略" and "为什么固定批量后能变成线性规划") choose gbs,
    the number of GPU batches and the shares of weights and cache off the GPU
    for the config's model under the given HBM and host-memory budgets, over
    gbs in {16, 32, 48, 64} x 1..8 GPU batches, within what this executor
    realizes (activations on the GPU, at most half of an fp16 layer's weights
    off it), with and without decode attention of an fp16 host cache share on
    the host CPU; each point's shares are rounded up to whole tiered layers
    and whole host-resident GPU batches, and the cost model's best realized
    placement is the one run."""
    from throughput_oriented_offloaded_amd import policy as P
    q4 = P.Q4G64
    wl = P.Workload(cfg["l"], cfg["h1"], cfg["h2"], cfg["s"], cfg["n"],
                    w_ratio=q4 if cfg["w"] == "q4" else 1.0, c_ratio=q4 if cfg["kv"] == "q4" else 1.0)
    base = P.mi355x(host_gb * 1e9)
    mc = P.Machine(**{**base.__dict__, "cap_g": gpu_gb * 1e9})
    best = P.search_realized(wl, mc, gbs_list=(16, 32, 48, 64), nb_max=8,
                             limits=P.executor_limits(cfg["w"] == "f16"))
    if best is None:
        raise SystemExit(f"policy: no placement of {cfg['workload']} fits {gpu_gb} GB of HBM and "
                         f"{host_gb} GB of host memory")
    gbs, nb, est = best["gbs"], best["num_gpu_batches"], best["estimate"]
    block = {"gpu_mem_gb": gpu_gb, "host_mem_gb": host_gb, "search": "gbs {16,32,48,64} x nb 1..8",
             "gbs": gbs, "num_gpu_batches": nb, "bls": gbs * nb,
             "lp_shares": {k: round(v, 4) for k, v in best["lp_shares"].items()},
             "realized_shares": {k: round(v, 4) for k, v in best["shares"].items()},
             "tiered_layers": best["n_tiered"], "kv_host_gpu_batches": best["kv_host_batches"],
             "cpu_attention": best["cpu_attention"],
             "predicted_ms_per_step": round(est["T_gen"] * wl.l * 1e3, 2),
             "predicted_prefill_s": round(est["T_pre"] * wl.l, 3),
             "predicted_peak_gb": {k: round(v / 1e9, 2) for k, v in est["peak"].items()}}
    over = dict(gbs=gbs, nb=nb, tier_layers=best["tiered_layers"], tier=False,
                kv_host_seqs=best["kv_host_batches"] * gbs, kv_host_attention=best["cpu_attention"])
    return over, block


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=31)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5, choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true", help="time without per-kernel events")
    ap.add_argument("--policy", choices=("auto",), default=None,
                    help="choose gbs, GPU batches and host shares with the cost model's LP search")
    ap.add_argument("--gpu-mem-gb", type=float, default=288.0, help="HBM budget of --policy auto")
    ap.add_argument("--host-mem-gb", type=float, default=64.0,
                    help="pinned host memory budget of --policy auto")
    ap.add_argument("--profile-layer", type=int, default=0, metavar="R",
                    help="counter-collection driver: one layer of the config (prefilled to s), "
                         "R decode steps, then a 1 GiB device copy that calibrates byte counters")
    args = ap.parse_args()
    faulthandler.enable()
    if args.config in REFUSED:
        print(f"bench.py --config {args.config}: {REFUSED[args.config]}", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the block decode is measured on a single "
              "MI355X (sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    from throughput_oriented_offloaded_amd import _lib as L
    from throughput_oriented_offloaded_amd.model import Model
    import synth

    cfg = dict(CONFIGS[args.config], id=args.config)
    if args.profile_layer:
        profile_layer(cfg, args.profile_layer)
        return
    K, Wm = args.steps, args.warmup
    policy_block = None
    if args.policy:
        over, policy_block = plan_policy(cfg, args.gpu_mem_gb, args.host_mem_gb)
        cfg.update(over)
        cfg["workload"] += (f", placement chosen by the policy search for {args.gpu_mem_gb:g} GB of "
                            f"HBM and {args.host_mem_gb:g} GB of host memory")
        log(f"policy: {json.dumps(policy_block)}")
    bls, s, n = cfg["gbs"] * cfg["nb"], cfg["s"], cfg["n"]
    torch.cuda.set_device(0)
    # capacity pre-check before anything of the model is allocated: the
    # policy's HBM budget, else the device's free memory
    n_tiered = len(set(cfg.get("tier_layers") or ())) if cfg.get("tier_layers") is not None else \
        (cfg["l"] if cfg.get("tier") else 0)
    fmt_of = lambda f: L.FG_FMT_Q4G64 if f == "q4" else L.FG_FMT_F16  # noqa: E731
    max_len = s + max(n, K + 1, Wm + 1)
    kv_host = cfg.get("kv_host_seqs", 0)
    L.fg_check_capacity(L.dims(cfg["h1"], cfg["h2"], cfg["nh"], cfg["hd"]),
                        L.plan(cfg["l"], fmt_of(cfg["w"]), fmt_of(cfg["kv"]), max_len, bls - kv_host,
                               cfg["gbs"], s, synth.VOCAB, n_tiered=n_tiered, bls_host=kv_host),
                        int(args.gpu_mem_gb * 1e9) if args.policy else 0)
    want_cpu = not args.no_cpu_baseline
    t_build = time.time()
    log(f"building {cfg['workload']} ({cfg['l']} layers, bls {bls})")
    sh, layers, tier, emb, host0, quant, fmt = build_model(cfg, want_cpu)
    host_threads = host_cpu_threads()
    model = Model(sh, layers, emb, fmt(cfg["kv"]), bls, max_len, tier=tier,
                  kv_host_seqs=cfg.get("kv_host_seqs", 0),
                  kv_host_attention=cfg.get("kv_host_attention", False), host_threads=host_threads)
    tokens = synth.tokens(bls, s, seed=0, device="cuda")
    torch.cuda.synchronize()
    log(f"built in {time.time() - t_build:.1f} s; prefill s={s} ...")

    t = time.perf_counter()
    _, tok1 = model.prefill(tokens, cfg["gbs"], cfg["nb"])
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t
    log(f"prefill {t_prefill:.2f} s; warmup {Wm} steps")

    gemm_kind = "gemm_q4" if cfg["w"] == "q4" else "gemm_f16"
    attn_kind = "attn_decode_q4" if cfg["kv"] == "q4" else "attn_decode_f16"
    # warm-up steps: every kernel kind traced (the per-kernel breakdown)
    L.fg_trace_kinds(None)
    L.fg_trace_enable(not args.no_trace)
    tok = tok1
    for i in range(Wm):
        _, tok = model.decode_step(tok, s + i, cfg["gbs"], cfg["nb"])
    torch.cuda.synchronize()
    tr_warm = L.fg_trace_collect() if not args.no_trace else {}

    # timed steps: events only for the two roofline kernels (and, with KV
    # tiering, the host <-> slot copies on the copy stream), and only on every
    # TRACE_EVERY-th step from TRACE_FIRST.  The roofline kernels' events are
    # recorded by their own launches (hipExtLaunchKernelGGL: the kernel's start
    # and end, no event packets between kernels); a traced step still takes
    # about 2.7 ms longer than an untraced one at config 5, the sampled steps
    # of the default run hold 768 decode GEMM launches, and the kind mask
    # pauses recording without discarding what was recorded
    kvt_kinds = ["kv_h2d", "kv_d2h"] if cfg.get("kv_host_seqs") else []
    if tier is not None:
        kvt_kinds.append("w_h2d")
    L.fg_trace_kinds([])
    L.fg_trace_enable(not args.no_trace)
    tok = tok1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        traced = i % TRACE_EVERY == TRACE_FIRST % TRACE_EVERY or K <= TRACE_FIRST and i == 0
        L.fg_trace_kinds([gemm_kind, attn_kind] + kvt_kinds if traced else [])
        _, tok = model.decode_step(tok, s + i, cfg["gbs"], cfg["nb"])
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t0
    tr = L.fg_trace_collect() if not args.no_trace else {}
    L.fg_trace_enable(False)
    L.fg_trace_kinds(None)
    ok = bool(((tok >= 0) & (tok < sh.vocab)).all().item())
    log(f"decode {K} steps in {t_dec:.3f} s ({t_dec / K * 1e3:.2f} ms/step); tokens valid: {ok}")

    value = bls * K / t_dec
    t_gen = t_prefill + t_dec / K * (n - 1)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": Wm, "ms_per_step": round(t_dec / K * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "layers": cfg["l"], "h1": cfg["h1"],
                   "h2": cfg["h2"], "heads": cfg["nh"], "head_dim": cfg["hd"], "bls": bls,
                   "gbs": cfg["gbs"], "num_gpu_batches": cfg["nb"], "s": s, "n": n,
                   "weights": "q4g64" if cfg["w"] == "q4" else "f16",
                   "kv_cache": "q4g64" if cfg["kv"] == "q4" else "f16",
                   "parallelism": "single GPU"},
        "roofline": roofline(tr, gemm_kind, "mfma", args.config),
        "roofline_attn": roofline(tr, attn_kind, "hbm", args.config),
        "generation_throughput": {"value": round(bls * n / t_gen, 2), "unit": "tokens/s",
                                  "prefill_s": round(t_prefill, 3),
                                  "definition": "bls*n/(t_prefill + (n-1) decode steps)"},
        # per-kernel breakdown from the warm-up steps (all kinds traced there)
        "kernels": {k: {"launches": v["count"], "ms_per_step": round(v["ms"] / max(Wm, 1), 3),
                        "avg_us": round(v["ms"] * 1e3 / v["count"], 2),
                        "TFLOP/s": round(v["flops"] / (v["ms"] / 1e3) / 1e12, 2) if v["flops"] else None,
                        "GB/s": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1)}
                    for k, v in tr_warm.items()},
        "tokens_valid": ok,
    }
    if not args.no_trace and s + K // 2 <= 8192 and not cfg.get("kv_host_seqs"):
        out["roofline_attn_topk"] = topk_attention(model, cfg, L, s + K // 2)
    if s + K <= 8192 and not cfg.get("kv_host_attention"):   # the host path is dense only
        out["decode_attn_topk"] = sparse_decode(model, cfg, L, tok1, min(K, 8), args.no_trace)
    if tier is not None and "w_h2d" in tr:
        # weight tiering: host bytes staged per step and the copy stream's busy
        # time (HIP events around the scheduler's own copies, traced steps)
        wc = tr["w_h2d"]
        step = t_dec / K
        ns = traced_steps(K)
        kern_s = (tr[gemm_kind]["ms"] + tr[attn_kind]["ms"]) / 1e3 / ns
        busy = wc["ms"] / 1e3 / ns
        out["tiering"] = {
            "host_bytes_per_step": round(wc["bytes"] / ns),
            "h2d_GBs_while_copying": round(wc["bytes"] / (wc["ms"] / 1e3) / 1e9, 2),
            "h2d_GBs_over_step": round(wc["bytes"] / ns / step / 1e9, 2),
            "copy_s_per_step": round(busy, 4), "gemm_attn_s_per_step": round(kern_s, 4),
            "step_s": round(step, 4), "overlap_efficiency": round(max(busy, kern_s) / step, 4),
            "definition": "host halves of the tiered layers (W_Q, W_K rows and W_1) staged by "
                          "hipMemcpyAsync on the scheduler's copy stream, timed by events around "
                          "each layer's copies; overlap = max(copy busy time, GEMM + attention "
                          "time) / step time"}
    if cfg.get("kv_host_seqs") and "kv_h2d" in tr:
        # KV tiering: history bytes loaded per step and the copy stream's busy time
        ld, st_ = tr["kv_h2d"], tr.get("kv_d2h", {"bytes": 0.0, "ms": 0.0})
        step = t_dec / K
        ns = traced_steps(K)
        kern_s = (tr[gemm_kind]["ms"] + tr[attn_kind]["ms"]) / 1e3 / ns
        out["kv_tiering"] = {
            "host_sequences": cfg["kv_host_seqs"], "load_bytes_per_step": round(ld["bytes"] / ns),
            "store_bytes_per_step": round(st_["bytes"] / ns),
            "h2d_GBs_while_copying": round(ld["bytes"] / (ld["ms"] / 1e3) / 1e9, 2),
            "h2d_GBs_over_step": round(ld["bytes"] / ns / step / 1e9, 2),
            "load_s_per_step": round(ld["ms"] / 1e3 / ns, 4),
            "store_s_per_step": round(st_["ms"] / 1e3 / ns, 4),
            "gemm_attn_s_per_step": round(kern_s, 4), "step_s": round(step, 4),
            "overlap_efficiency": round(max(ld["ms"] / 1e3 / ns, kern_s) / step, 4),
            "definition": "loads: 2-D copies of positions 0..pos-1 of every host batch's K, V and "
                          "metadata into a device slot (copy stream); stores: the appended rows "
                          "back (their own stream); overlap = max(load busy time, GEMM + "
                          "attention time) / step time"}
    if cfg.get("kv_host_attention"):
        # per step: the host batches' history the CPU reads (K and V rows of
        # every layer, at the timed steps' mean position) against the rows
        # that cross the link (q, k, v down, the attention row back)
        step = t_dec / K
        p_mean = s + Wm + (K - 1) / 2
        per_elem = 9 / 16 if cfg["kv"] == "q4" else 2     # stored bytes per cached value
        hist = cfg["kv_host_seqs"] * cfg["l"] * p_mean * cfg["h1"] * 2 * per_elem
        link = cfg["kv_host_seqs"] * cfg["l"] * 4 * cfg["h1"] * 2
        out["host_attention"] = {
            "host_sequences": cfg["kv_host_seqs"], "cpu_threads": host_threads, "cache": cfg["kv"],
            "history_bytes_per_step": round(hist), "link_bytes_per_step": round(link),
            "step_s": round(step, 4), "history_GBs_over_step": round(hist / step / 1e9, 2),
            "definition": "the host batches' attention computed by the CPU over the host cache as "
                          "stored (fp16, or 4-bit codes and metadata), only their q, k, v rows and "
                          "attention rows crossing the link; history_GBs_over_step = stored history "
                          "bytes read by the CPU per step / step time (a lower bound on the CPU's rate)"}
    if policy_block is not None:
        policy_block["measured_ms_per_step"] = out["ms_per_step"]
        policy_block["measured_prefill_s"] = round(t_prefill, 3)
        policy_block["measured_over_predicted"] = round(out["ms_per_step"] / policy_block["predicted_ms_per_step"], 3)
        out["policy"] = policy_block
    if quant:
        out["weight_quant"] = {"GB/s": round(quant["bytes"] / (quant["ms"] / 1e3) / 1e9, 1),
                               "frac": round(quant["bytes"] / (quant["ms"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                               "launches": quant["count"]}
    if want_cpu:
        del model, layers, tier
        torch.cuda.empty_cache()
        gpu_units = {
            "config1_s": gpu_config1(),
            "quant_layer_s": quant["ms"] / 1e3 / cfg["l"] if quant else None,
            "attn_layer_s": (tr[attn_kind]["ms"] / tr[attn_kind]["count"] / 1e3) if attn_kind in tr else None,
            "layer_decode_s": t_dec / K / cfg["l"],
            "prefill_layer_2seq_s": t_prefill / cfg["l"] * 2 / bls,
        }
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(cfg, host0, emb, gpu_units)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
