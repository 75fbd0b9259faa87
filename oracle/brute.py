"""Second, independent definition of the row reductions, in pure Python.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written separately
from ``oracle.c`` so that the two can pin each other on tiny rows: it works on
Python floats, sums with ``math.fsum`` (exactly rounded), and decodes stored
16-bit values through the ``struct`` module's binary16 codec and a shift for
bfloat16, not through the C decoders.

Definitions follow the same passages as ``oracle.c``: the softmax of
"Portable Triton Kernels" ("Safe Softmax Pattern"), its RMSNorm ("Reference
Kernel: RMSNorm"), the plain LayerNorm reading (biased variance, eps inside
the square root) and the attention forward of "Triton: Block-Level GPU
Programming Without CUDA" ("How Flash Attention Uses Triton").  Use only for
rows of at most a few thousand elements.
"""
from __future__ import annotations

import math
import struct


def decode16(bits: int, kind: str) -> float:
    """Exact value of a stored fp16 ('f16') or bf16 ('bf16') bit pattern."""
    if kind == "f16":
        return struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]
    if kind == "bf16":
        return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    raise ValueError(kind)


def softmax_row(xs):
    m = max(xs)
    es = [math.exp(v - m) if v != -math.inf else 0.0 for v in xs]
    s = math.fsum(es)
    return [e / s for e in es]


def layernorm_row(xs, eps, gamma=None, beta=None):
    n = len(xs)
    mu = math.fsum(xs) / n
    var = math.fsum((v - mu) ** 2 for v in xs) / n
    rs = 1.0 / math.sqrt(var + eps)
    g = gamma if gamma is not None else [1.0] * n
    b = beta if beta is not None else [0.0] * n
    return [(v - mu) * rs * g[j] + b[j] for j, v in enumerate(xs)], mu, rs


def rmsnorm_row(xs, eps, weight=None):
    n = len(xs)
    ms = math.fsum(v * v for v in xs) / n
    inv = 1.0 / math.sqrt(ms + eps)
    w = weight if weight is not None else [1.0] * n
    return [v * inv * w[j] for j, v in enumerate(xs)]


def attention_row(qrow, K, V, scale, visible):
    """One query row of softmax(scale Q K^T) V over the first `visible` keys:
    scores by math.fsum of the products, weights exp(s - max), output sums
    by math.fsum, divided by the fsum of the weights."""
    s = [scale * math.fsum(a * b for a, b in zip(qrow, K[j])) for j in range(visible)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = math.fsum(w)
    return [math.fsum(w[j] * V[j][c] for j in range(visible)) / tot for c in range(len(V[0]))]
