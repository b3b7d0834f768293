"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module only draws random numbers; it holds none of the method's arithmetic
(no quantization, no GEMM, no attention).  Both sides of every parity check
receive the very same fp16 bytes produced here.

Seeding: every tensor gets its own 64-bit sub-seed
    splitmix64(base_seed ^ fnv1a64(name) ^ layer)
so that one layer of a 96-layer model can be regenerated alone.

Distributions (the pages' workload is "input 512 / output 32" on OPT models,
FlexGen article, section 5.1; there are no datasets or trained weights here):
  * every weight tensor ~ N(0, 0.02) rounded to fp16, LayerNorm gains 1 + N(0, 0.02);
  * activations fed to a lone decoder layer ~ N(0, 1) fp16;
  * prompt token ids uniform over the vocabulary;
  * the KV-compression stress input adds 1 % outliers scaled by 8.
"""
from __future__ import annotations

import torch

_MASK64 = (1 << 64) - 1


def fnv1a64(text: str) -> int:
    h = 0xCBF29CE484222325
    for b in text.encode():
        h ^= b
        h = (h * 0x100000001B3) & _MASK64
    return h


def splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def sub_seed(base: int, name: str, layer: int = 0) -> int:
    # torch seeds are 64-bit; keep them positive and below 2**63
    return splitmix64((base ^ fnv1a64(name) ^ layer) & _MASK64) & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_fp16(shape, sigma: float, seed: int, device="cpu", mean: float = 0.0) -> torch.Tensor:
    """fp16 tensor of N(mean, sigma^2) draws (drawn in fp32, rounded once to fp16)."""
    g = _gen(seed, device)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if sigma != 1.0:
        x.mul_(sigma)
    if mean != 0.0:
        x.add_(mean)
    return x.to(torch.float16)


def token_ids(batch: int, length: int, vocab: int, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randint(0, vocab, (batch, length), generator=g, dtype=torch.int64,
                         device=device).to(torch.int32)


def with_outliers(x: torch.Tensor, frac: float, factor: float, seed: int) -> torch.Tensor:
    """Multiply a seeded Bernoulli(frac) subset of the elements by `factor` (fp16 in, fp16 out)."""
    g = _gen(seed, x.device)
    u = torch.rand(x.shape, generator=g, dtype=torch.float32, device=x.device)
    y = x.float()
    y = torch.where(u < frac, y * factor, y)
    return y.to(torch.float16)


# ----------------------------------------------------------------------------- layer weights

LAYER_MATRICES = ("wqkv", "wo", "w1", "w2")


def layer_shapes(hidden: int, ffn: int) -> dict:
    """fp16 shapes of one pre-LN OPT decoder layer; matrices are [out][in] (N x K)."""
    h, f = hidden, ffn
    return {
        "ln1_g": (h,), "ln1_b": (h,),
        "wqkv": (3 * h, h), "bqkv": (3 * h,),
        "wo": (h, h), "bo": (h,),
        "ln2_g": (h,), "ln2_b": (h,),
        "w1": (f, h), "b1": (f,),
        "w2": (h, f), "b2": (h,),
    }


def layer_tensor(name: str, shape, base_seed: int, layer: int, device="cpu") -> torch.Tensor:
    seed = sub_seed(base_seed, name, layer)
    if name.endswith("_g"):
        return normal_fp16(shape, 0.02, seed, device, mean=1.0)
    return normal_fp16(shape, 0.02, seed, device)


def layer_weights_fp16(hidden: int, ffn: int, base_seed: int, layer: int, device="cpu") -> dict:
    return {n: layer_tensor(n, s, base_seed, layer, device)
            for n, s in layer_shapes(hidden, ffn).items()}


def model_tensor(name: str, shape, base_seed: int, device="cpu") -> torch.Tensor:
    """Model-level tensors: 'embed' [V][h], 'pos' [P][h], 'lnf_g', 'lnf_b' [h]."""
    seed = sub_seed(base_seed, name, 0)
    if name.endswith("_g"):
        return normal_fp16(shape, 0.02, seed, device, mean=1.0)
    return normal_fp16(shape, 0.02, seed, device)
