"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random numbers
with torch's generators and lays them out.  The GPU path receives the tensors
on the device; the CPU oracle receives host copies of the very same values.

Workload shape (the pages measure on synthetic prompts padded to 512 tokens
with dummy weights, [P2] "实验结果该怎样解读"):
  * weight matrices and biases ~ N(0, 0.02) in fp16, LayerNorm gamma = 1,
    beta = 0 unless asked for random ones;
  * token ids uniform in [0, vocab);
  * every tensor has its own seed: seed * 1_000_003 + 97 * layer + tensor_id.

Matrix layout: [out, in] row-major.  The fused QKV matrix stacks W_Q, W_K,
W_V as rows [0, h1), [h1, 2h1), [2h1, 3h1).
"""
from __future__ import annotations

import torch

STD = 0.02
VOCAB = 50272

_TENSOR_IDS = {"w_qkv": 1, "b_qkv": 2, "w_o": 3, "b_o": 4, "w_1": 5, "b_1": 6, "w_2": 7,
               "b_2": 8, "ln1_g": 9, "ln1_b": 10, "ln2_g": 11, "ln2_b": 12,
               "embed": 20, "pos": 21, "lnf_g": 22, "lnf_b": 23, "tokens": 30,
               "khist": 40, "vhist": 41, "x": 42}


def tensor_seed(seed: int, layer: int, name: str) -> int:
    return seed * 1_000_003 + 97 * layer + _TENSOR_IDS[name]


def _gen(device, s):
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def normal_f16(shape, seed: int, device="cpu", std: float = STD, chunk_rows: int = 4096):
    """fp16 tensor ~ N(0, std^2); drawn in fp32 in row chunks (bounded scratch)."""
    out = torch.empty(shape, dtype=torch.float16, device=device)
    if out.numel() == 0:
        return out
    g = _gen(device, seed)
    flat = out.view(shape[0], -1) if len(shape) > 1 else out.view(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        t = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        flat[r0:r1].copy_(t.mul_(std))
    return out


def layer_weights(h1: int, h2: int, layer: int, seed: int = 0, device="cpu",
                  random_ln: bool = False) -> dict:
    """fp16 weights of one decoder layer (keys match the library's layer struct)."""
    W = {}
    shapes = {"w_qkv": (3 * h1, h1), "b_qkv": (3 * h1,), "w_o": (h1, h1), "b_o": (h1,),
              "w_1": (h2, h1), "b_1": (h2,), "w_2": (h1, h2), "b_2": (h1,)}
    for k, shp in shapes.items():
        W[k] = normal_f16(shp, tensor_seed(seed, layer, k), device)
    for k in ("ln1", "ln2"):
        if random_ln:
            W[k + "_g"] = (1.0 + normal_f16((h1,), tensor_seed(seed, layer, k + "_g"), device,
                                            std=0.2).float()).half()
            W[k + "_b"] = normal_f16((h1,), tensor_seed(seed, layer, k + "_b"), device, std=0.2)
        else:
            W[k + "_g"] = torch.ones(h1, dtype=torch.float16, device=device)
            W[k + "_b"] = torch.zeros(h1, dtype=torch.float16, device=device)
    return W


def embeddings(h1: int, max_pos: int, seed: int = 0, vocab: int = VOCAB, device="cpu") -> dict:
    """Token table E [vocab, h1], learned positions P [max_pos, h1], final LN."""
    return {
        "embed": normal_f16((vocab, h1), tensor_seed(seed, 0, "embed"), device),
        "pos": normal_f16((max_pos, h1), tensor_seed(seed, 0, "pos"), device),
        "lnf_g": torch.ones(h1, dtype=torch.float16, device=device),
        "lnf_b": torch.zeros(h1, dtype=torch.float16, device=device),
    }


def tokens(rows: int, cols: int, seed: int = 0, vocab: int = VOCAB, device="cpu"):
    """Token ids uniform in [0, vocab), int32 [rows, cols]."""
    g = _gen(device, tensor_seed(seed, 0, "tokens"))
    return torch.randint(0, vocab, (rows, cols), generator=g, device=device, dtype=torch.int32)


def activations(rows: int, h: int, seed: int, device="cpu", std: float = 1.0, layer: int = 0):
    """A hidden-state block x [rows, h] ~ N(0, std^2) fp16."""
    return normal_f16((rows, h), tensor_seed(seed, layer, "x"), device, std=std)


def kv_history(bls: int, n_heads: int, length: int, head_dim: int, seed: int, device="cpu",
               layer: int = 0, std: float = 2.0):
    """Synthetic fp16 K and V rows for `length` past positions, laid out
    [bls, length, n_heads * head_dim] like the rows a QKV projection writes."""
    h1 = n_heads * head_dim
    k = normal_f16((bls * length, h1), tensor_seed(seed, layer, "khist"), device, std=std)
    v = normal_f16((bls * length, h1), tensor_seed(seed, layer, "vhist"), device, std=std)
    return k.view(bls, length, h1), v.view(bls, length, h1)
