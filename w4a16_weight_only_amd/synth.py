"""Seeded synthetic inputs for the W4A16 linear layer.

This module only draws random numbers; it holds none of the method's
arithmetic (no unpacking, dequantisation or products), so the GPU tests and the
CPU oracle can both take their inputs from it without sharing any of the
computation they check.

Workloads (shapes and value distributions of an 8B-class decoder's linears):
  tiny     M=1   K=256   N=256   G=64  symmetric zero point 8
  gemv     M=1   K=4096  N=12800 G=128 symmetric zero point 8
  batched  M=32  K=4096  N=12800 G=128 asymmetric qzeros; weights drawn in the
                                       checkpoint layout [N, K/8], then repacked
  prefill  M=256 K=12800 N=4096  G=128 asymmetric qzeros
  stack    40 layers x {QKV 4096->6144, O 4096->4096, gate+up 4096->25600,
           down 12800->4096}, G=128, symmetric; M=1 and M=32
Distributions: activations ~N(0,1) rounded to fp16; weight nibbles i.i.d.
uniform on [0,15] (8 per 32-bit word, i.e. a uniform 32-bit word); qzeros
likewise; scales uniform on [0.5, 1.5) / sqrt(K), rounded to fp16.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "tiny":    dict(M=1,   K=256,   N=256,   G=64,  asym=False, seed=1),
    "gemv":    dict(M=1,   K=4096,  N=12800, G=128, asym=False, seed=2),
    "batched": dict(M=32,  K=4096,  N=12800, G=128, asym=True,  seed=3, from_checkpoint=True),
    "prefill": dict(M=256, K=12800, N=4096,  G=128, asym=True,  seed=4),
}

# 8B-class decoder layer: hidden 4096, QKV out 6144, MLP width 12800.
STACK = dict(layers=40, H=4096, NQ=6144, I=12800, G=128, seed_base=5000)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def activations(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """fp16 [M, K] ~ N(0, 1)."""
    return g.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def packed_words(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """int32 [rows, cols] of uniform 32-bit words (8 uniform nibbles each)."""
    return g.integers(0, 1 << 32, size=(rows, cols), dtype=np.uint32).view(np.int32)


def scales(g: np.random.Generator, NG: int, N: int, K: int) -> np.ndarray:
    """fp16 [K/G, N] uniform on [0.5, 1.5) / sqrt(K)."""
    s = (g.random((NG, N), dtype=np.float32) + np.float32(0.5)) / np.float32(np.sqrt(K))
    return s.astype(np.float16)


def problem(M: int, K: int, N: int, G: int, asym: bool, seed: int,
            from_checkpoint: bool = False) -> dict:
    """One linear's inputs.  With from_checkpoint the weights are drawn in the
    checkpoint layout [N, K/8] (key 'b_nk8') and 'b_packed' is absent: the
    caller repacks.  Otherwise 'b_packed' is [K, N/8]."""
    g = rng(seed)
    out = dict(M=M, K=K, N=N, G=G, zp_bias=8)
    out["a"] = activations(g, M, K)
    if from_checkpoint:
        out["b_nk8"] = packed_words(g, N, K // 8)
    else:
        out["b_packed"] = packed_words(g, K, N // 8)
    out["scales"] = scales(g, K // G, N, K)
    out["qzeros"] = packed_words(g, K // G, N // 8) if asym else None
    return out


def workload(name: str, **override) -> dict:
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    return problem(**cfg)


def stack_linear_shapes(H: int, NQ: int, I: int):
    """(K, N) of the four linears of one layer: qkv, o, gate_up, down."""
    return [(H, NQ), (H, H), (H, 2 * I), (I, H)]


def stack_layer(layer: int, H: int = STACK["H"], NQ: int = STACK["NQ"], I: int = STACK["I"],
                G: int = STACK["G"], seed_base: int = STACK["seed_base"]) -> list:
    """The four linears of one layer of the decode stack (symmetric, zp 8)."""
    lins = []
    for j, (K, N) in enumerate(stack_linear_shapes(H, NQ, I)):
        g = rng(seed_base + 4 * layer + j)
        lins.append(dict(K=K, N=N, G=G, zp_bias=8, qzeros=None,
                         b_packed=packed_words(g, K, N // 8),
                         scales=scales(g, K // G, N, K)))
    return lins


def stack_input(M: int, H: int = STACK["H"], seed: int = 5) -> np.ndarray:
    return activations(rng(seed), M, H)
