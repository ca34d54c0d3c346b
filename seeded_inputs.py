"""Seeded synthetic inputs for the int4 dequantizing matmul.

This module is shared by the oracle side and the HIP side of every test and of
the benchmark, and holds none of the method's arithmetic: it only draws random
numbers and writes them in the library's canonical input format.

Canonical input format (the library's own definition of q4f16_1; the pages only
name the format):
  * x            : f16 bits, uint16 [k]
  * words        : uint32 [n][k/8]; code k = 8*j + i of a row is in bits
                   4*i .. 4*i+3 of that row's word j (low nibble first)
  * scales       : f16 bits, uint16 [n][k/32], one per 32 consecutive k
  * words3 (int3): uint32 [n][3k/32]; a row's 3-bit codes form one bit
                   stream, LSB first over its words: code k is in stream bits
                   3k .. 3k+2 (stream bit b = bit b % 32 of word b / 32)

Distributions are those of the decode workloads the library is measured on:
x ~ N(0, 1) rounded to f16; codes uniform in 0..15; scales uniform in
[0.005, 0.02] rounded to f16.  Every generator takes a numpy Generator so that
the draw order is explicit; ``workload`` fixes the order per named workload.
Real Phi-3-mini q4f16_1 weights are not used: these draws stand in for them
(the kernels have no data-dependent control flow, so timing does not depend
on the values).
"""
from __future__ import annotations

import numpy as np


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [n][k] in 0..15 -> canonical words uint32 [n][k/8]."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, k = codes.shape
    assert k % 8 == 0 and codes.max(initial=0) < 16
    c = codes.reshape(n, k // 8, 8)
    words = np.zeros((n, k // 8), np.uint32)
    for i in range(8):
        words |= c[:, :, i] << np.uint32(4 * i)
    return words


def f16_bits(v) -> np.ndarray:
    """float values -> f16 bit patterns (numpy's round-to-nearest-even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def draw_x(rng: np.random.Generator, k: int) -> np.ndarray:
    """activation vector x f16 [k] ~ N(0, 1)."""
    return f16_bits(rng.standard_normal(k))


def draw_X(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """activation rows X f16 [m][k] ~ N(0, 1)."""
    return f16_bits(rng.standard_normal((m, k)))


def draw_weight(rng: np.random.Generator, n: int, k: int,
                lo: float = 0.005, hi: float = 0.02):
    """int4 weight: (words uint32 [n][k/8], scales f16 bits [n][k/32]).

    Draw order: codes, then scales."""
    assert k % 32 == 0
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    scales = f16_bits(rng.uniform(lo, hi, size=(n, k // 32)))
    return pack_codes(codes), scales


def draw_weight3(rng: np.random.Generator, n: int, k: int,
                 lo: float = 0.005, hi: float = 0.02):
    """int3 weight: (words3 uint32 [n][3k/32], scales f16 bits [n][k/32]).

    Uniform random words: every bit pattern is a valid code stream, so each
    3-bit code is uniform in 0..7.  Draw order: words, then scales."""
    assert k % 32 == 0
    words3 = rng.integers(0, 1 << 32, size=(n, 3 * k // 32), dtype=np.uint64).astype(np.uint32)
    scales = f16_bits(rng.uniform(lo, hi, size=(n, k // 32)))
    return words3, scales


# The workloads the library is measured and tested on (shapes of a Phi-3-mini
# decode step: hidden 3072, 32 heads x 96, FFN 8192, vocabulary 32064).
GEMV_3072 = "gemv_3072x3072"
LAYER_SET = "phi3_mini_layer_set"
FFN = "phi3_mini_ffn_fused"
LM_HEAD = "phi3_mini_lm_head"
GEMM = "prefill_gemm_16384x3072"

LAYER_SHAPES = {            # name -> (n, k)
    "qkv": (9216, 3072),
    "o_proj": (3072, 3072),
    "gate_up": (16384, 3072),
    "down": (3072, 8192),
}


def workload(name: str, seed: int = 0, m: int = 16, scale: float = 1.0) -> dict:
    """Inputs of a named workload, drawn in a fixed order from
    ``default_rng(seed)``.

    ``scale`` < 1 shrinks every output dimension n (rounded to a multiple of
    64, at least 64) for quick runs; the k dimensions never change."""
    rng = np.random.default_rng(seed)

    def n_of(n):
        return n if scale >= 1.0 else max(64, int(n * scale) // 64 * 64)

    if name == GEMV_3072:
        x = draw_x(rng, 3072)
        w, s = draw_weight(rng, n_of(3072), 3072)
        return {"x": x, "words": w, "scales": s}
    if name == LAYER_SET:
        x3 = draw_x(rng, 3072)
        x8 = draw_x(rng, 8192)
        out = {"x3072": x3, "x8192": x8}
        for key, (n, k) in LAYER_SHAPES.items():
            out[key] = draw_weight(rng, n_of(n), k)
        return out
    if name == FFN:
        x = draw_x(rng, 3072)
        gate = draw_weight(rng, n_of(8192), 3072)
        up = draw_weight(rng, n_of(8192), 3072)
        down = draw_weight(rng, n_of(3072), n_of(8192))
        return {"x": x, "gate": gate, "up": up, "down": down}
    if name == LM_HEAD:
        x = draw_x(rng, 3072)
        w, s = draw_weight(rng, n_of(32064), 3072)
        return {"x": x, "words": w, "scales": s}
    if name == GEMM:
        X = draw_X(rng, m, 3072)
        w, s = draw_weight(rng, n_of(16384), 3072)
        return {"X": X, "words": w, "scales": s}
    raise KeyError(name)
