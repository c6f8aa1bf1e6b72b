"""Seeded synthetic inputs for the quantized decode matrix-vector product.

This module only draws arrays of the right shapes, dtypes and value
distributions. It holds none of the method's arithmetic (no unpacking,
dequantization, normalisation or dot products), so both the CPU oracle and the
GPU library can consume what it returns without sharing any computation.

Every tensor gets its own PCG64 stream, keyed by (seed, tag...) through
numpy's SeedSequence, so a tensor can be regenerated alone, in any order, on
any machine with the same numpy.

Distributions (one set for every workload):
  * packed code words: raw uniform 32-bit words, so every 4-bit or 2-bit field
    is uniform over its range;
  * scales: fp16 ~ U(0.005, 0.02); biases: fp16 ~ U(-0.1, 0.1);
  * LUT entries: fp16 ~ N(0, 0.02) (std 0.02), 16 per output row;
  * 8-bit codes: scales drawn as above times 15/255, so that the weights
    cover the same range as the 4-bit ones (codes 0..255 instead of 0..15);
  * dense fp16 weights (no codes): fp16 ~ N(0, 0.02);
  * activations: N(0, 1) rounded to fp16 (held as fp16 or widened to fp32);
  * RMSNorm weights: fp16 ~ 1 + N(0, 0.1);
  * router logits: fp32 ~ N(0, 1).
Rounding into fp16/fp32 is numpy's round-to-nearest-even.
"""

from __future__ import annotations

import zlib

import numpy as np

SCALE_LO, SCALE_HI = 0.005, 0.02
BIAS_LO, BIAS_HI = -0.1, 0.1
LUT_STD = 0.02
NORM_STD = 0.1

AFFINE = 0
LUT = 1
DENSE = 2
Q8_SCALE_FACTOR = 15.0 / 255.0


def _tag_int(t) -> int:
    if isinstance(t, (int, np.integer)):
        return int(t) & 0xFFFFFFFF
    return zlib.crc32(str(t).encode("utf-8"))


def stream(seed: int, *tags) -> np.random.Generator:
    """Independent generator for one tensor, keyed by (seed, *tags)."""
    key = [int(seed) & 0xFFFFFFFF] + [_tag_int(t) for t in tags]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def words(g: np.random.Generator, shape) -> np.ndarray:
    """Uniform raw uint32 words (every bit an independent fair coin)."""
    return g.integers(0, 1 << 32, size=shape, dtype=np.uint32)


def uniform(g: np.random.Generator, shape, lo: float, hi: float, dtype=np.float16) -> np.ndarray:
    return g.uniform(lo, hi, size=shape).astype(dtype)


def normal(g: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0,
           dtype=np.float16) -> np.ndarray:
    return (mean + std * g.standard_normal(size=shape)).astype(dtype)


def words_per_row(K: int, bits: int) -> int:
    return K * bits // 32


def qmat(seed: int, tag, N: int, K: int, bits: int = 4, fmt: int = AFFINE,
         group: int = 64) -> dict:
    """A planar quantized N x K matrix: code words [N][K*bits/32] plus either
    fp16 scales and biases [N][K/group] (affine) or a fp16 LUT [N][16]; or,
    for fmt=DENSE (bits 16), the fp16 weights themselves packed two to a
    word (little endian, so the words are the fp16 row's bytes)."""
    if fmt == DENSE:
        if bits != 16 or K % 2:
            raise ValueError("the dense format holds 16-bit fields and an even K")
        w16 = normal(stream(seed, tag, "w"), (N, K), 0.0, LUT_STD, np.float16)
        return {"N": N, "K": K, "bits": 16, "fmt": DENSE, "group": group,
                "q": np.ascontiguousarray(w16).view(np.uint32), "scales": None,
                "biases": None, "lut": None}
    if K % group or (K * bits) % 32:
        raise ValueError(f"K={K} must be a multiple of group={group}")
    out = {"N": N, "K": K, "bits": bits, "fmt": fmt, "group": group,
           "q": words(stream(seed, tag, "q"), (N, words_per_row(K, bits)))}
    if fmt == AFFINE:
        f = Q8_SCALE_FACTOR if bits == 8 else 1.0
        out["scales"] = uniform(stream(seed, tag, "s"), (N, K // group), SCALE_LO * f, SCALE_HI * f)
        out["biases"] = uniform(stream(seed, tag, "b"), (N, K // group), BIAS_LO, BIAS_HI)
        out["lut"] = None
    else:
        out["scales"] = None
        out["biases"] = None
        out["lut"] = normal(stream(seed, tag, "lut"), (N, 1 << bits), 0.0, LUT_STD)
    return out


def activations(seed: int, tag, shape, dtype=np.float16) -> np.ndarray:
    """N(0,1) activations rounded to fp16; widened exactly when dtype is fp32."""
    return normal(stream(seed, tag, "x"), shape, 0.0, 1.0, np.float16).astype(dtype)


def norm_weight(seed: int, tag, K: int) -> np.ndarray:
    return normal(stream(seed, tag, "g"), (K,), 1.0, NORM_STD, np.float16)


def router_logits(seed: int, tag, shape) -> np.ndarray:
    return normal(stream(seed, tag, "route"), shape, 0.0, 1.0, np.float32)


# ---------------------------------------------------------------------------
# Workload shapes (sizes only).

LLAMA3_8B = dict(name="llama3-8b-shaped", layers=32, hidden=4096, qkv=6144,
                 q_dim=4096, o_in=4096, ffn=14336)
QWEN3_06B = dict(name="qwen3-0.6b-shaped", layers=28, hidden=1024, qkv=4096,
                 q_dim=2048, o_in=2048, ffn=3072, vocab=151936)
MOE_397B = dict(name="moe-397b-expert-layer", hidden=4096, ffn=1024, experts=512,
                top_k=3, draws=60)


def tp_shard(model: dict, tp: int) -> dict:
    """The decode layer one GPU holds under tensor parallelism `tp` (rows of
    qkv and gate/up, and the inputs of o and down, divided by tp; hidden size
    and layer count unchanged). Its weights are drawn from their own streams."""
    m = dict(model)
    if tp == 1:
        return m
    for k in ("qkv", "q_dim", "o_in", "ffn"):
        if tp < 1 or model[k] % (tp * 64):
            raise ValueError(f"{k} = {model[k]} does not split into {tp} shards of whole groups")
        m[k] = model[k] // tp
    m["name"] = f"{model['name']} tp{tp} shard"
    return m


def layer_shapes(model: dict) -> dict:
    """(N, K) of each matvec in one decode layer."""
    H = model["hidden"]
    return {"qkv": (model["qkv"], H), "o": (H, model["o_in"]),
            "gate": (model["ffn"], H), "up": (model["ffn"], H),
            "down": (H, model["ffn"])}


def layer_weights(seed: int, model: dict, layer: int, bits: int = 4, fmt: int = AFFINE) -> dict:
    """One decode layer's weights with independent streams per (layer, tensor)."""
    H = model["hidden"]
    w = {name: qmat(seed, (model["name"], layer, name), N, K, bits, fmt)
         for name, (N, K) in layer_shapes(model).items()}
    w["g_attn"] = norm_weight(seed, (model["name"], layer, "g_attn"), H)
    w["g_ffn"] = norm_weight(seed, (model["name"], layer, "g_ffn"), H)
    return w


def qmat_bytes(N: int, K: int, bits: int = 4, fmt: int = AFFINE, group: int = 64) -> int:
    """Stored bytes of a planar quantized matrix (codes + scales/biases or LUT)."""
    codes = N * K * bits // 8
    if fmt == DENSE:
        return codes
    if fmt == AFFINE:
        return codes + N * (K // group) * 4
    return codes + N * (1 << bits) * 2
