"""OPT-style decoder driven through the C ABI: weights in HBM (fp16 or
group-wise 4-bit) or, for fp16, half of each layer in pinned host memory;
per-layer KV caches; prefill and zig-zag block decode.

Every step runs in libfg.so: this module owns the buffers (allocated with
torch) and hands whole passes to the library's block schedule
(fg_model_prefill / fg_model_decode_step: layers in order, the block's GPU
batches innermost, host-resident weights staged on a side stream; "FlexGen
完全拆解" (pinghaoyang.com.cn), sections "一个层级流水的伪代码" and "三条关键
数据通路如何重叠").
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib as L

MATS = ("qkv", "o", "1", "2")


@dataclass(frozen=True)
class Shape:
    n_layers: int
    h1: int
    h2: int
    n_heads: int
    head_dim: int
    vocab: int = 50272

    @property
    def dims(self) -> L.Dims:
        return L.dims(self.h1, self.h2, self.n_heads, self.head_dim)

    def mat_shape(self, name):
        return {"qkv": (3 * self.h1, self.h1), "o": (self.h1, self.h1),
                "1": (self.h2, self.h1), "2": (self.h1, self.h2)}[name]


def quantize_weight(w: torch.Tensor, stream=None):
    """[N, K] fp16 -> (codes [N/2, K] uint8, meta [N/64, 2, K] fp16), groups along N."""
    N, K = w.shape
    codes = torch.empty((N // 2, K), dtype=torch.uint8, device=w.device)
    meta = torch.empty((N // 64, 2, K), dtype=torch.float16, device=w.device)
    L.fg_quant_group4(w, 1, N, K, codes, meta, stream=stream)
    return codes, meta


class DeviceLayer:
    """One layer's weights on the device plus the fg_layer_w that points at them."""

    def __init__(self, fmt: int, t: dict):
        self.fmt, self.t = fmt, t
        s = L.LayerW()
        s.fmt = fmt
        for name in MATS:
            setattr(s, "w_" + name, L.ptr(t.get("w_" + name)))
            setattr(s, "m_" + name, L.ptr(t.get("m_" + name)))
            setattr(s, "b_" + name, L.ptr(t["b_" + name]))
        for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
            setattr(s, k, L.ptr(t[k]))
        self.struct = s

    @classmethod
    def from_fp16(cls, W: dict, fmt: int, stream=None) -> "DeviceLayer":
        """W: fp16 device tensors (w_*, b_*, ln*).  For 4-bit, the matrices are
        quantized on the device and the fp16 copies are not kept."""
        t = {k: v for k, v in W.items() if not k.startswith("w_")}
        for name in MATS:
            w = W["w_" + name]
            if fmt == L.FG_FMT_Q4G64:
                t["w_" + name], t["m_" + name] = quantize_weight(w, stream)
            else:
                t["w_" + name] = w
        return cls(fmt, t)


class TierLayer:
    """The host-resident half of one fp16 layer: W_Q, W_K rows of W_qkv and W_1
    in pinned host memory, W_V rows on the device (staged next to them)."""

    def __init__(self, W: dict):
        h1 = W["w_qkv"].shape[1]
        h2 = W["w_1"].shape[0]
        qkv = W["w_qkv"]
        # one pinned block per layer ([W_Q; W_K] then W_1): the host allocator
        # rounds blocks up, so two separate tensors would waste more memory
        nq, n1 = 2 * h1 * h1, h2 * h1
        self._host = torch.empty(nq + n1, dtype=torch.float16, pin_memory=True)
        self.qk_host = self._host[:nq].view(2 * h1, h1)
        self.w1_host = self._host[nq:].view(h2, h1)
        self.qk_host.copy_(qkv[:2 * h1])
        self.w1_host.copy_(W["w_1"])
        self.v_dev = qkv[2 * h1:].clone()
        self.struct = L.TierW(L.ptr(self.qk_host), L.ptr(self.v_dev), L.ptr(self.w1_host))

    @property
    def host_bytes(self) -> int:
        return self._host.numel() * 2

    @staticmethod
    def split(W: dict, fmt: int):
        """(DeviceLayer without W_qkv / W_1, TierLayer) from fp16 device weights."""
        assert fmt == L.FG_FMT_F16, "tiering keeps fp16 weights"
        tl = TierLayer(W)
        t = {k: v for k, v in W.items() if k not in ("w_qkv", "w_1")}
        t["w_qkv"] = None
        t["w_1"] = None
        return DeviceLayer(fmt, t), tl


class DeviceKV:
    """One layer's cache: q4 codes [n_seq, nh, max_len, hd/2] + meta
    [n_seq, nh, max_len, hd/64, 2], or fp16 [n_seq, nh, max_len, hd].
    device "pinned": in pinned host memory (a KV tier's host cache)."""

    def __init__(self, fmt: int, n_seq: int, n_heads: int, head_dim: int, max_len: int, device):
        self.fmt = fmt
        shp = (n_seq, n_heads, max_len)
        pin = device == "pinned"
        kw = dict(device="cpu", pin_memory=True) if pin else dict(device=device)
        if fmt == L.FG_FMT_Q4G64:
            self.k = torch.zeros(shp + (head_dim // 2,), dtype=torch.uint8, **kw)
            self.v = torch.zeros(shp + (head_dim // 2,), dtype=torch.uint8, **kw)
            self.km = torch.zeros(shp + (head_dim // 64, 2), dtype=torch.float16, **kw)
            self.vm = torch.zeros(shp + (head_dim // 64, 2), dtype=torch.float16, **kw)
        else:
            self.k = torch.zeros(shp + (head_dim,), dtype=torch.float16, **kw)
            self.v = torch.zeros(shp + (head_dim,), dtype=torch.float16, **kw)
            self.km = self.vm = None
        s = L.KV()
        s.fmt, s.k, s.v = fmt, L.ptr(self.k), L.ptr(self.v)
        s.k_meta, s.v_meta = L.ptr(self.km), L.ptr(self.vm)
        s.max_len, s.n_seq = max_len, n_seq
        self.struct = s


class Model:
    """A decoder of `shape` on one GPU.  layers: list of DeviceLayer; emb: dict
    with embed [vocab, h1], pos [max_pos, h1], lnf_g, lnf_b (fp16, device)."""

    def __init__(self, shape: Shape, layers, emb: dict, kv_fmt: int, n_seq: int, max_len: int,
                 device="cuda", tier=None, attn_topk: float = 0.0, kv_host_seqs: int = 0,
                 kv_host_attention: bool = False, host_threads: int = 0):
        """tier: None, or one TierLayer (or None) per layer for weight tiering.
        attn_topk: 0 for dense decode attention, else the fraction of cached
        positions whose V each decode step reads (Top-K sparse V; the pages
        use 0.1), rounded up per step.
        kv_host_seqs: the last kv_host_seqs sequences keep their KV cache in
        pinned host memory (KV tiering; a whole number of GPU batches at every
        call), moved through two device slots by the library.
        kv_host_attention: the decode steps compute the host-resident
        batches' attention on the host CPU (host_threads threads, 0: all)
        instead of moving their history to the device."""
        assert 0.0 <= attn_topk <= 1.0
        self.attn_topk_ppm = int(round(attn_topk * 1_000_000))
        self.shape, self.layers, self.emb = shape, layers, emb
        self.d = shape.dims
        self.n_seq, self.max_len = n_seq, max_len
        assert 0 <= kv_host_seqs <= n_seq
        self.kv_host_seqs = kv_host_seqs
        assert not kv_host_attention or kv_host_seqs, "host attention needs host-resident sequences"
        self.kv_host_attention, self.host_threads = kv_host_attention, host_threads
        n_dev = max(n_seq - kv_host_seqs, 1)   # the device cache is unused when every batch is on the host
        self.kv = [DeviceKV(kv_fmt, n_dev, shape.n_heads, shape.head_dim, max_len, device)
                   for _ in layers]
        self.kv_host = [DeviceKV(kv_fmt, kv_host_seqs, shape.n_heads, shape.head_dim, max_len, "pinned")
                        for _ in layers] if kv_host_seqs else []
        self._kvt = {}     # gbs -> (tier object, its slots, copy stream, host array)
        self.device = device
        self._ws = None
        n = len(layers)
        self._w_arr = (L.LayerW * n)(*[lay.struct for lay in layers])
        self._kv_arr = (L.KV * n)(*[kv.struct for kv in self.kv])
        self.tier = tier
        self._sched = None
        self._tier_arr = None
        if tier is not None:
            assert len(tier) == n
            self._tier_arr = (L.TierW * n)(*[t.struct if t is not None else L.TierW()
                                            for t in tier])
            sb = L.fg_stage_bytes(self.d)
            self._stage = torch.empty(2 * sb, dtype=torch.uint8, device=device)
            self._sched = L.fg_sched_create(self._stage, sb)
            self._copy_stream = torch.cuda.Stream(device=device)
            self._staged = False

    def __del__(self):
        if getattr(self, "_sched", None):
            torch.cuda.synchronize(self.device)
            L.fg_sched_destroy(self._sched)
            self._sched = None
        if getattr(self, "_kvt", None):
            torch.cuda.synchronize(self.device)
            for kt in self._kvt.values():
                L.fg_kvtier_destroy(kt[0])
            self._kvt = {}

    def kv_tier(self, gbs: int, nb: int):
        """fg_kv_tier of a call with GPU batches of gbs sequences (None
        without KV tiering): two slots of one GPU batch, a copy stream."""
        if not self.kv_host_seqs:
            return None
        assert self.kv_host_seqs % gbs == 0 and gbs * nb == self.n_seq, \
            "host-resident sequences must be whole GPU batches of the block"
        if gbs not in self._kvt:
            sb = L.fg_kvtier_slot_bytes(self.d, gbs, self.max_len, self.kv_host[0].fmt)
            slots = torch.empty(2 * sb, dtype=torch.uint8, device=self.device)
            cp = torch.cuda.Stream(device=self.device)
            host = (L.KV * len(self.kv_host))(*[h.struct for h in self.kv_host])
            kt = L.fg_kvtier_create(slots, sb, cp)
            stage = None
            if self.kv_host_attention:
                hb = L.fg_kvtier_host_stage_bytes(self.d, self.kv_host_seqs)
                stage = torch.empty(hb, dtype=torch.uint8, pin_memory=True)
                L.fg_kvtier_host_attention(kt, stage, hb, self.host_threads)
            self._kvt[gbs] = (kt, slots, cp, host, stage)
        kt, _, _, host, _ = self._kvt[gbs]
        return L.KvTier(kt, host, nb - self.kv_host_seqs // gbs)

    def _sched_args(self):
        """(sched, tier array, copy stream, flags) of the next pass; with tiering
        every pass also stages the first tiered layer for the following one."""
        if self._sched is None:
            return None, None, None, 0
        flags = L.FG_SCHED_STAGE_NEXT | (L.FG_SCHED_FIRST_STAGED if self._staged else 0)
        self._staged = True
        return self._sched, self._tier_arr, self._copy_stream, flags

    def workspace(self, rows: int) -> torch.Tensor:
        fmt = self.layers[0].fmt
        need = max(L.fg_workspace_bytes(self.d, rows, fmt),
                   L.fg_linear_workspace_bytes(self.n_seq, self.shape.vocab, self.shape.h1), 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def _head(self, x_last: torch.Tensor, stream=None):
        """Final LayerNorm, tied LM head (fp16 GEMM on MFMA), greedy pick."""
        sh = self.shape
        rows = x_last.shape[0]
        a = torch.empty_like(x_last)
        L.fg_layernorm(x_last, rows, sh.h1, self.emb["lnf_g"], self.emb["lnf_b"], a, stream=stream)
        logits = torch.empty((rows, sh.vocab), dtype=torch.float16, device=self.device)
        ws = self.workspace(rows)
        L.fg_linear(a, rows, sh.h1, L.FG_FMT_F16, self.emb["embed"], None, sh.vocab, None, 0, None,
                    logits, ws, ws.numel(), stream=stream)
        tok = torch.empty(rows, dtype=torch.int32, device=self.device)
        L.fg_argmax(logits, rows, sh.vocab, tok, stream=stream)
        return logits, tok

    def prefill(self, tokens: torch.Tensor, gbs: int, nb: int, stream=None):
        """tokens int32 [bls, s] (device).  Returns (logits [bls, vocab], next token [bls])."""
        sh = self.shape
        bls, s = tokens.shape
        assert bls == gbs * nb <= self.n_seq and s <= self.max_len
        pos = torch.arange(s, dtype=torch.int32, device=self.device).repeat(bls)
        x = torch.empty((bls * s, sh.h1), dtype=torch.float16, device=self.device)
        L.fg_embed(tokens.reshape(-1), pos, bls * s, self.emb["embed"], sh.vocab, self.emb["pos"],
                   self.emb["pos"].shape[0], sh.h1, x, stream=stream)
        ws = self.workspace(gbs * s)
        sc, tier, cp, flags = self._sched_args()
        L.fg_model_prefill(sc, self.d, self._w_arr, tier, self._kv_arr, x, gbs, nb, s, ws,
                           ws.numel(), stream=stream, copy_stream=cp, flags=flags,
                           kvt=self.kv_tier(gbs, nb))
        last = x.view(bls, s, sh.h1)[:, s - 1, :].contiguous()
        return self._head(last, stream)

    def decode_step(self, tok: torch.Tensor, pos: int, gbs: int, nb: int, stream=None):
        """One new token per sequence at position pos.  Returns (logits, next token)."""
        sh = self.shape
        bls = gbs * nb
        x = self.embed_step(tok, pos, stream)
        ws = self.workspace(bls)
        sc, tier, cp, flags = self._sched_args()
        L.fg_model_decode_step(sc, self.d, self._w_arr, tier, self._kv_arr, x, gbs, nb, pos, ws,
                               ws.numel(), stream=stream, copy_stream=cp, flags=flags,
                               attn_topk_ppm=self.attn_topk_ppm, kvt=self.kv_tier(gbs, nb))
        return self._head(x, stream)

    def embed_step(self, tok: torch.Tensor, pos: int, stream=None) -> torch.Tensor:
        sh = self.shape
        bls = tok.numel()
        posv = torch.full((bls,), pos, dtype=torch.int32, device=self.device)
        x = torch.empty((bls, sh.h1), dtype=torch.float16, device=self.device)
        L.fg_embed(tok, posv, bls, self.emb["embed"], sh.vocab, self.emb["pos"],
                   self.emb["pos"].shape[0], sh.h1, x, stream=stream)
        return x

    def generate(self, tokens: torch.Tensor, n: int, gbs: int, nb: int, stream=None,
                 forced=None):
        """Greedy generation of n tokens: one from the prefill, n-1 decode steps
        ("FlexGen 完全拆解", section "从硬件画像得到每层时间": T = l T_pre +
        l (n-1) T_gen).  forced: optional [bls, n] tokens fed instead of the
        model's own picks (teacher forcing).  Returns (tokens [bls, n], logits list)."""
        bls, s = tokens.shape
        assert s + n - 1 <= self.max_len
        logits, tok = self.prefill(tokens, gbs, nb, stream)
        out, lg = [tok], [logits]
        for t in range(1, n):
            feed = forced[:, t - 1].contiguous() if forced is not None else out[-1]
            logits, tok = self.decode_step(feed, s + t - 1, gbs, nb, stream)
            out.append(tok)
            lg.append(logits)
        return torch.stack(out, 1), lg
