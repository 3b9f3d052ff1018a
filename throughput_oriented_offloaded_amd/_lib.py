"""ctypes binding of libfg.so (include/fg.h).  Argument marshalling only.

Every function takes torch tensors that already live on the GPU (or plain
ints for sizes), passes their data pointers and the current HIP stream to the
C ABI, and raises FgError on a non-zero status.  Nothing here computes: when
the library is missing, importing this module raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfg.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "fg.h")

FG_OK, FG_ERR_INVALID, FG_ERR_UNSUPPORTED, FG_ERR_CAPACITY, FG_ERR_HIP = 0, -1, -2, -3, -4
FG_FMT_F16, FG_FMT_Q4G64 = 0, 1


class FgError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {status_str(status)} ({status}): {detail}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python -m throughput_oriented_offloaded_amd._build)")
_L = ctypes.CDLL(LIB_PATH)

P = ctypes.c_void_p
I32, I64, SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class Dims(ctypes.Structure):
    _fields_ = [("h1", I32), ("h2", I32), ("n_heads", I32), ("head_dim", I32)]


class LayerW(ctypes.Structure):
    _fields_ = [("fmt", I32)] + [(n, P) for n in (
        "w_qkv", "m_qkv", "b_qkv", "w_o", "m_o", "b_o", "w_1", "m_1", "b_1",
        "w_2", "m_2", "b_2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")]


class KV(ctypes.Structure):
    _fields_ = [("fmt", I32), ("k", P), ("k_meta", P), ("v", P), ("v_meta", P),
                ("max_len", I32), ("n_seq", I32)]


class KvTier(ctypes.Structure):
    """fg_kv_tier: tier object, host cache(s), GPU batches kept on the device."""
    _fields_ = [("pipe", P), ("host", ctypes.POINTER(KV)), ("nb_dev", I32)]


class TierW(ctypes.Structure):
    _fields_ = [("qk_host", P), ("v_dev", P), ("w1_host", P)]


class Plan(ctypes.Structure):
    """fg_plan: a model's placement on one GPU (capacity pre-check)."""
    _fields_ = [(n, I32) for n in ("n_layers", "fmt_w", "n_tiered", "fmt_kv", "max_len", "bls_dev",
                                   "bls_host", "gbs", "s")] + [("vocab", I64)]


FG_SCHED_FIRST_STAGED, FG_SCHED_STAGE_NEXT = 1, 2


_PROTOS = {
    "fg_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "fg_last_error": (ctypes.c_char_p, []),
    "fg_abi_version": (ctypes.c_int, []),
    "fg_quant_group4": (ctypes.c_int, [P, I64, I64, I64, I32, P, P, P]),
    "fg_dequant_group4": (ctypes.c_int, [P, P, I64, I64, I64, I32, P, P]),
    "fg_kv_append_q4": (ctypes.c_int, [P, P, I64, ctypes.POINTER(KV), I32, ctypes.POINTER(Dims), I32, P]),
    "fg_kv_append_f16": (ctypes.c_int, [P, P, I64, ctypes.POINTER(KV), I32, ctypes.POINTER(Dims), I32, P]),
    "fg_attn_decode_q4": (ctypes.c_int, [P, P, P, I64, ctypes.POINTER(KV), I32, ctypes.POINTER(Dims),
                                         I32, I32, P, P]),
    "fg_attn_decode_f16": (ctypes.c_int, [P, P, P, I64, ctypes.POINTER(KV), I32, ctypes.POINTER(Dims),
                                          I32, I32, P, P]),
    "fg_attn_decode_topk_q4": (ctypes.c_int, [P, P, P, I64, ctypes.POINTER(KV), I32, ctypes.POINTER(Dims),
                                              I32, I32, I32, P, P]),
    "fg_attn_decode_topk_f16": (ctypes.c_int, [P, P, P, I64, ctypes.POINTER(KV), I32, ctypes.POINTER(Dims),
                                               I32, I32, I32, P, P]),
    "fg_attn_prefill": (ctypes.c_int, [P, I32, I32, ctypes.POINTER(Dims), P, P]),
    "fg_linear": (ctypes.c_int, [P, I64, I64, I32, P, P, I64, P, I32, P, P, P, SZ, P]),
    "fg_linear_workspace_bytes": (SZ, [I64, I64, I64]),
    "fg_linear_noalloc": (ctypes.c_int, [P, I64, I64, I32, P, P, I64, P, I32, P, P, P]),
    "fg_linear_noalloc_max_bytes": (SZ, []),
    "fg_layernorm": (ctypes.c_int, [P, I64, I64, P, P, P, P]),
    "fg_embed": (ctypes.c_int, [P, P, I64, P, I64, P, I64, I64, P, P]),
    "fg_argmax": (ctypes.c_int, [P, I64, I64, P, P]),
    "fg_layer_prefill": (ctypes.c_int, [ctypes.POINTER(Dims), ctypes.POINTER(LayerW), P, I32, I32, I32,
                                        ctypes.POINTER(KV), P, SZ, P, ctypes.POINTER(KvTier)]),
    "fg_layer_decode_block": (ctypes.c_int, [ctypes.POINTER(Dims), ctypes.POINTER(LayerW), P, I32, I32,
                                             I32, ctypes.POINTER(KV), P, SZ, P, I32,
                                             ctypes.POINTER(KvTier)]),
    "fg_workspace_bytes": (SZ, [ctypes.POINTER(Dims), I64, I32]),
    "fg_stage_bytes": (SZ, [ctypes.POINTER(Dims)]),
    "fg_sched_create": (ctypes.c_int, [ctypes.POINTER(P), P, SZ]),
    "fg_sched_destroy": (ctypes.c_int, [P]),
    "fg_prefetch": (ctypes.c_int, [P, P, SZ, P, P]),
    "fg_model_prefill": (ctypes.c_int, [P, ctypes.POINTER(Dims), I32, ctypes.POINTER(LayerW),
                                        ctypes.POINTER(TierW), ctypes.POINTER(KV), P, I32, I32, I32,
                                        P, SZ, P, P, I32, ctypes.POINTER(KvTier)]),
    "fg_model_decode_step": (ctypes.c_int, [P, ctypes.POINTER(Dims), I32, ctypes.POINTER(LayerW),
                                            ctypes.POINTER(TierW), ctypes.POINTER(KV), P, I32, I32,
                                            I32, P, SZ, P, P, I32, I32, ctypes.POINTER(KvTier)]),
    "fg_kvtier_slot_bytes": (SZ, [ctypes.POINTER(Dims), I32, I32, I32]),
    "fg_kvtier_create": (ctypes.c_int, [ctypes.POINTER(P), P, SZ, P]),
    "fg_kvtier_destroy": (ctypes.c_int, [P]),
    "fg_kvtier_host_stage_bytes": (SZ, [ctypes.POINTER(Dims), I32]),
    "fg_kvtier_host_attention": (ctypes.c_int, [P, P, SZ, I32]),
    "fg_attn_decode_host_f16": (ctypes.c_int, [P, I64, ctypes.POINTER(KV), I32, I32, ctypes.POINTER(Dims),
                                               I32, I32, P, I32]),
    "fg_attn_decode_host_q4": (ctypes.c_int, [P, I64, ctypes.POINTER(KV), I32, I32, ctypes.POINTER(Dims),
                                              I32, I32, P, I32]),
    "fg_weight_bytes": (I64, [ctypes.POINTER(Dims), I32, I32]),
    "fg_kv_bytes": (I64, [ctypes.POINTER(Dims), I32, I32, I32, I32, I32]),
    "fg_plan_device_bytes": (I64, [ctypes.POINTER(Dims), ctypes.POINTER(Plan)]),
    "fg_check_capacity": (ctypes.c_int, [ctypes.POINTER(Dims), ctypes.POINTER(Plan), I64]),
    "fg_trace_enable": (ctypes.c_int, [ctypes.c_int]),
    "fg_trace_kinds": (ctypes.c_int, [ctypes.c_uint64]),
    "fg_trace_collect": (ctypes.c_int, [I32, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double)]),
    "fg_trace_kind_name": (ctypes.c_char_p, [ctypes.c_int]),
}
for _name, (_res, _args) in _PROTOS.items():
    _f = getattr(_L, _name)
    _f.restype, _f.argtypes = _res, _args


def header_symbols() -> list[str]:
    """Names of the functions include/fg.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fg_[a-z0-9_]+)\s*\(", txt)))


def exported_symbols() -> list[str]:
    return [n for n in header_symbols() if hasattr(_L, n)]


def status_str(st: int) -> str:
    return _L.fg_status_str(st).decode()


def last_error() -> str:
    return _L.fg_last_error().decode()


def _check(fn: str, st: int):
    if st != FG_OK:
        raise FgError(fn, st, last_error())


def ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_ptr(stream=None) -> int | None:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def dims(h1: int, h2: int, n_heads: int, head_dim: int) -> Dims:
    return Dims(h1, h2, n_heads, head_dim)


# --------------------------------------------------------------- entry points
def fg_quant_group4(x, outer, axis, inner, codes, meta, group=64, stream=None):
    _check("fg_quant_group4", _L.fg_quant_group4(ptr(x), outer, axis, inner, group, ptr(codes),
                                                 ptr(meta), stream_ptr(stream)))


def fg_dequant_group4(codes, meta, outer, axis, inner, y, group=64, stream=None):
    _check("fg_dequant_group4", _L.fg_dequant_group4(ptr(codes), ptr(meta), outer, axis, inner,
                                                     group, ptr(y), stream_ptr(stream)))


def fg_kv_append_q4(k_new, v_new, ld, kv: KV, bls, d: Dims, pos, stream=None):
    _check("fg_kv_append_q4", _L.fg_kv_append_q4(ptr(k_new), ptr(v_new), ld, ctypes.byref(kv), bls,
                                                 ctypes.byref(d), pos, stream_ptr(stream)))


def fg_kv_append_f16(k_new, v_new, ld, kv: KV, bls, d: Dims, pos, stream=None):
    _check("fg_kv_append_f16", _L.fg_kv_append_f16(ptr(k_new), ptr(v_new), ld, ctypes.byref(kv), bls,
                                                   ctypes.byref(d), pos, stream_ptr(stream)))


def fg_attn_decode_q4(q, k_new, v_new, ld, kv: KV, bls, d: Dims, pos, fuse_append, out, stream=None):
    _check("fg_attn_decode_q4", _L.fg_attn_decode_q4(ptr(q), ptr(k_new), ptr(v_new), ld, ctypes.byref(kv),
                                                     bls, ctypes.byref(d), pos, int(fuse_append),
                                                     ptr(out), stream_ptr(stream)))


def fg_attn_decode_f16(q, k_new, v_new, ld, kv: KV, bls, d: Dims, pos, fuse_append, out, stream=None):
    _check("fg_attn_decode_f16", _L.fg_attn_decode_f16(ptr(q), ptr(k_new), ptr(v_new), ld,
                                                       ctypes.byref(kv), bls, ctypes.byref(d), pos,
                                                       int(fuse_append), ptr(out), stream_ptr(stream)))


def fg_attn_decode_topk_q4(q, k_new, v_new, ld, kv: KV, bls, d: Dims, pos, topk, fuse_append, out,
                           stream=None):
    _check("fg_attn_decode_topk_q4", _L.fg_attn_decode_topk_q4(
        ptr(q), ptr(k_new), ptr(v_new), ld, ctypes.byref(kv), bls, ctypes.byref(d), pos, topk,
        int(fuse_append), ptr(out), stream_ptr(stream)))


def fg_attn_decode_topk_f16(q, k_new, v_new, ld, kv: KV, bls, d: Dims, pos, topk, fuse_append, out,
                            stream=None):
    _check("fg_attn_decode_topk_f16", _L.fg_attn_decode_topk_f16(
        ptr(q), ptr(k_new), ptr(v_new), ld, ctypes.byref(kv), bls, ctypes.byref(d), pos, topk,
        int(fuse_append), ptr(out), stream_ptr(stream)))


def fg_attn_prefill(qkv, b, s, d: Dims, out, stream=None):
    _check("fg_attn_prefill", _L.fg_attn_prefill(ptr(qkv), b, s, ctypes.byref(d), ptr(out),
                                                 stream_ptr(stream)))


def fg_linear_workspace_bytes(M, N, K) -> int:
    return _L.fg_linear_workspace_bytes(M, N, K)


def fg_linear(x, M, K, fmt, w, m, N, bias, act, residual, y, ws=None, ws_bytes=0, stream=None):
    _check("fg_linear", _L.fg_linear(ptr(x), M, K, fmt, ptr(w), ptr(m), N, ptr(bias), act,
                                     ptr(residual), ptr(y), ptr(ws), ws_bytes, stream_ptr(stream)))


def fg_linear_noalloc(x, M, K, fmt, w, m, N, bias, act, residual, y, stream=None):
    """fg_linear with its partials in the library's own device array (no workspace)."""
    _check("fg_linear_noalloc", _L.fg_linear_noalloc(ptr(x), M, K, fmt, ptr(w), ptr(m), N, ptr(bias), act,
                                                     ptr(residual), ptr(y), stream_ptr(stream)))


def fg_layernorm(x, rows, h, gamma, beta, y, stream=None):
    _check("fg_layernorm", _L.fg_layernorm(ptr(x), rows, h, ptr(gamma), ptr(beta), ptr(y),
                                           stream_ptr(stream)))


def fg_embed(tok, pos, rows, E, vocab, Pt, max_pos, h1, x, stream=None):
    _check("fg_embed", _L.fg_embed(ptr(tok), ptr(pos), rows, ptr(E), vocab, ptr(Pt), max_pos, h1,
                                   ptr(x), stream_ptr(stream)))


def fg_argmax(logits, rows, n, out, stream=None):
    _check("fg_argmax", _L.fg_argmax(ptr(logits), rows, n, ptr(out), stream_ptr(stream)))


def _kvt(kvt):
    return ctypes.byref(kvt) if kvt is not None else None


def fg_layer_prefill(d: Dims, w: LayerW, x, gbs, nb, s, kv: KV, ws, ws_bytes, stream=None, kvt=None):
    _check("fg_layer_prefill", _L.fg_layer_prefill(ctypes.byref(d), ctypes.byref(w), ptr(x), gbs, nb, s,
                                                   ctypes.byref(kv), ptr(ws), ws_bytes,
                                                   stream_ptr(stream), _kvt(kvt)))


def fg_layer_decode_block(d: Dims, w: LayerW, x, gbs, nb, pos, kv: KV, ws, ws_bytes, stream=None,
                          attn_topk_ppm=0, kvt=None):
    _check("fg_layer_decode_block", _L.fg_layer_decode_block(ctypes.byref(d), ctypes.byref(w), ptr(x),
                                                             gbs, nb, pos, ctypes.byref(kv), ptr(ws),
                                                             ws_bytes, stream_ptr(stream),
                                                             attn_topk_ppm, _kvt(kvt)))


def fg_kvtier_slot_bytes(d: Dims, gbs, max_len, fmt) -> int:
    return _L.fg_kvtier_slot_bytes(ctypes.byref(d), gbs, max_len, fmt)


def fg_kvtier_create(slots, slot_bytes, copy_stream) -> int:
    """KV tier object over the caller's two slots (2 * slot_bytes) and copy stream."""
    h = P()
    _check("fg_kvtier_create", _L.fg_kvtier_create(ctypes.byref(h), ptr(slots), slot_bytes,
                                                   copy_stream.cuda_stream))
    return h.value


def fg_kvtier_destroy(h):
    _check("fg_kvtier_destroy", _L.fg_kvtier_destroy(h))


def fg_kvtier_host_stage_bytes(d: Dims, n_host_seq) -> int:
    return _L.fg_kvtier_host_stage_bytes(ctypes.byref(d), n_host_seq)


def fg_kvtier_host_attention(h, stage, stage_bytes, n_threads=0):
    """Decode attention of the tier's host batches on the host CPU (stage:
    pinned host memory), or back to the device slots (stage None)."""
    _check("fg_kvtier_host_attention", _L.fg_kvtier_host_attention(h, ptr(stage), stage_bytes, n_threads))


def fg_attn_decode_host_f16(qkv, ld, kv: KV, seq0, nseq, d: Dims, pos, append, out, n_threads=0):
    _check("fg_attn_decode_host_f16", _L.fg_attn_decode_host_f16(ptr(qkv), ld, ctypes.byref(kv), seq0, nseq,
                                                                 ctypes.byref(d), pos, int(append), ptr(out),
                                                                 n_threads))


def fg_attn_decode_host_q4(qkv, ld, kv: KV, seq0, nseq, d: Dims, pos, append, out, n_threads=0):
    _check("fg_attn_decode_host_q4", _L.fg_attn_decode_host_q4(ptr(qkv), ld, ctypes.byref(kv), seq0, nseq,
                                                               ctypes.byref(d), pos, int(append), ptr(out),
                                                               n_threads))


def fg_stage_bytes(d: Dims) -> int:
    return _L.fg_stage_bytes(ctypes.byref(d))


def fg_sched_create(stage, stage_bytes) -> int:
    """Scheduler handle over the caller's two stage buffers (2 * stage_bytes)."""
    h = P()
    _check("fg_sched_create", _L.fg_sched_create(ctypes.byref(h), ptr(stage), stage_bytes))
    return h.value


def fg_sched_destroy(h):
    _check("fg_sched_destroy", _L.fg_sched_destroy(h))


def fg_prefetch(dst, src, nbytes, copy_stream=None, done=None):
    """Copy nbytes from pinned host memory src to device memory dst on
    copy_stream (a torch stream, or None for the current one), then record
    done (a torch.cuda.Event, or None) there."""
    ev = None
    if done is not None:
        if done.cuda_event == 0:          # torch creates its events on first record
            done.record(copy_stream) if copy_stream is not None else done.record()
        ev = done.cuda_event
    _check("fg_prefetch", _L.fg_prefetch(ptr(dst), ptr(src), nbytes, stream_ptr(copy_stream), ev))


def _arr(T, items):
    return (T * len(items))(*items) if items is not None else None


def fg_model_prefill(sched, d: Dims, layers, tier, kvs, x, gbs, nb, s, ws, ws_bytes, stream=None,
                     copy_stream=None, flags=0, kvt=None):
    """layers: ctypes array of LayerW; tier: array of TierW or None; kvs: array of KV."""
    _check("fg_model_prefill", _L.fg_model_prefill(sched, ctypes.byref(d), len(layers), layers, tier,
                                                   kvs, ptr(x), gbs, nb, s, ptr(ws), ws_bytes,
                                                   stream_ptr(stream),
                                                   copy_stream.cuda_stream if copy_stream else None,
                                                   flags, _kvt(kvt)))


def fg_model_decode_step(sched, d: Dims, layers, tier, kvs, x, gbs, nb, pos, ws, ws_bytes,
                         stream=None, copy_stream=None, flags=0, attn_topk_ppm=0, kvt=None):
    _check("fg_model_decode_step", _L.fg_model_decode_step(sched, ctypes.byref(d), len(layers),
                                                           layers, tier, kvs, ptr(x), gbs, nb, pos,
                                                           ptr(ws), ws_bytes, stream_ptr(stream),
                                                           copy_stream.cuda_stream if copy_stream
                                                           else None, flags, attn_topk_ppm,
                                                           _kvt(kvt)))


def fg_workspace_bytes(d: Dims, rows, fmt_w) -> int:
    return _L.fg_workspace_bytes(ctypes.byref(d), rows, fmt_w)


def fg_weight_bytes(d: Dims, n_layers, fmt) -> int:
    return _L.fg_weight_bytes(ctypes.byref(d), n_layers, fmt)


def fg_kv_bytes(d: Dims, n_layers, bls, s, n, fmt) -> int:
    return _L.fg_kv_bytes(ctypes.byref(d), n_layers, bls, s, n, fmt)


def plan(n_layers, fmt_w, fmt_kv, max_len, bls_dev, gbs, s, vocab, n_tiered=0, bls_host=0) -> Plan:
    return Plan(n_layers, fmt_w, n_tiered, fmt_kv, max_len, bls_dev, bls_host, gbs, s, vocab)


def fg_plan_device_bytes(d: Dims, p: Plan) -> int:
    v = _L.fg_plan_device_bytes(ctypes.byref(d), ctypes.byref(p))
    if v < 0:
        raise FgError("fg_plan_device_bytes", FG_ERR_INVALID, last_error())
    return v


def fg_check_capacity(d: Dims, p: Plan, budget_bytes: int = 0):
    """Raises FgError (FG_ERR_CAPACITY) when the plan does not fit the budget
    (0: the device's free memory)."""
    _check("fg_check_capacity", _L.fg_check_capacity(ctypes.byref(d), ctypes.byref(p), int(budget_bytes)))


def fg_trace_enable(on: bool):
    _check("fg_trace_enable", _L.fg_trace_enable(int(on)))


TRACE_KINDS = ["quant_g4", "dequant_g4", "gemm_q4", "gemm_f16", "splitk_reduce", "attn_decode_q4",
               "attn_decode_f16", "kv_store", "attn_prefill", "layernorm", "embed", "argmax",
               "reduce_layernorm", "attn_topk_q4", "attn_topk_f16", "kv_h2d", "kv_d2h", "w_h2d",
               "proj_qkv", "proj_out", "proj_fc1", "proj_fc2"]


def fg_trace_kinds(names=None):
    """Record only the named kinds (None: all) while tracing is on."""
    mask = (1 << 64) - 1 if names is None else sum(1 << TRACE_KINDS.index(n) for n in names)
    _check("fg_trace_kinds", _L.fg_trace_kinds(mask))


def fg_trace_collect(n_kinds: int = 32) -> dict:
    """{kind name: {"count", "ms", "flops", "bytes"}} for kinds with launches."""
    cnt = (I64 * n_kinds)()
    ms, fl, by = ((ctypes.c_double * n_kinds)() for _ in range(3))
    n = _L.fg_trace_collect(n_kinds, cnt, ms, fl, by)
    if n < 0:
        _check("fg_trace_collect", n)
    out = {}
    for k in range(n):
        if cnt[k]:
            out[_L.fg_trace_kind_name(k).decode()] = {"count": cnt[k], "ms": ms[k],
                                                      "flops": fl[k], "bytes": by[k]}
    return out


def raw(name: str):
    """The raw ctypes function (tests use it to pass deliberately bad arguments)."""
    return getattr(_L, name)
