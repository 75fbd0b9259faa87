"""Seeded synthetic inputs for the row-reduction workloads.

This module is shared by the tests, the benchmark and the oracle checks, and
holds none of the reductions' arithmetic: it only draws random numbers and
encodes them in a storage type.  The resulting bit patterns are the contract:
the same host array is copied to the GPU and handed to the oracle.

Recipe (all draws from numpy's PCG64 ``default_rng(seed)``):
  * draws are float64 (``standard_normal`` / ``uniform``) with the affine
    transform applied in float64;
  * each value is rounded once to float32 (IEEE round-to-nearest-even), then
    to the storage type: fp16 through numpy's binary16 cast, bf16 by
    round-to-nearest-even on the float32 bits (``to_bf16_bits``);
  * large arrays are drawn in row blocks from one generator, which yields the
    same values as one big draw (checked by the tests).

Workloads (name -> shapes, distributions, seeds):
  softmax_f32_1024x781     softmax  fp32  M=1024   N=781    x ~ N(0,1)                     seed 101
  layernorm_f16_4096       LN       fp16  M=4096   N=4096   x ~ mu_row + N(0,1),
                                                             mu_row ~ U(-5,5)               seeds 201, 202
                                                             gamma ~ 1 + sqrt(0.1) N(0,1)  seed 203
                                                             beta ~ sqrt(0.1) N(0,1)       seed 204
                                                             eps = 1e-5
  rmsnorm_bf16_16384x8192  RMSNorm  bf16  M=16384  N=8192   x ~ N(0,1)                     seed 301
                                                             w ~ 1 + sqrt(0.1) N(0,1)      seed 302
                                                             eps = 1e-6
  causal_softmax_bf16      softmax  bf16  32 heads x 4096 queries = 131072 rows, N=4096 keys,
                                          x ~ 3 N(0,1), x = -inf where key > query (the
                                          diagonal is kept), row r has query r mod 4096  seed 401
  vocab_softmax_f32        softmax  fp32  M=64 N=262144, x ~ 2 N(0,1), and in every row 8
                                          distinct positions (uniform, without replacement)
                                          set to +30.0                                    seeds 501, 502

Next-row workloads (fused residual add + norm, at the norm workloads' shapes;
not part of the five-workload suite):
  add_rmsnorm_bf16_16384x8192  x, w as rmsnorm_bf16_16384x8192; residual r ~ N(0,1)  seed 303
  add_layernorm_f16_4096       x, gamma, beta as layernorm_f16_4096; r ~ N(0,1)      seed 205
  causal_entry_softmax_bf16    the causal_softmax_bf16 inputs through the causal entry point
                               (scale 1, 4096 queries per head, offset 0): masked keys are
                               not read, so its bytes are the visible reads plus all writes
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}
NEG_INF_BITS = {F16: 0xFC00, BF16: 0xFF80}


def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u.astype(np.uint64) + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), r)


def encode(v64: np.ndarray, dt: str) -> np.ndarray:
    """float64 draws -> stored array: float32 for fp32, uint16 bits otherwise."""
    f32 = np.asarray(v64, dtype=np.float64).astype(np.float32)
    if dt == F32:
        return f32
    if dt == F16:
        return f32.astype(np.float16).view(np.uint16)
    if dt == BF16:
        return to_bf16_bits(f32)
    raise ValueError(dt)


def storage_dtype(dt: str):
    return np.float32 if dt == F32 else np.uint16


def normal_rows(seed: int, M: int, N: int, dt: str, scale: float = 1.0,
                loc: float = 0.0, block_rows: int = 4096, rows=None) -> np.ndarray:
    """[M, N] array of scale*N(0,1)+loc, drawn row-block by row-block.

    ``rows`` (optional, sorted) keeps only those rows; the generator still
    advances through every row so values match the full draw.
    """
    rng = np.random.default_rng(seed)
    keep = None if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((M if keep is None else len(keep), N), dtype=storage_dtype(dt))
    pos = 0
    for r0 in range(0, M, block_rows):
        r1 = min(M, r0 + block_rows)
        z = rng.standard_normal((r1 - r0) * N).reshape(r1 - r0, N)
        if keep is None:
            out[r0:r1] = encode(z * scale + loc, dt)
        else:
            sel = keep[(keep >= r0) & (keep < r1)]
            if len(sel):
                out[pos:pos + len(sel)] = encode(z[sel - r0] * scale + loc, dt)
                pos += len(sel)
    return out


def vector(seed: int, N: int, dt: str, scale: float, loc: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return encode(rng.standard_normal(N) * scale + loc, dt)


@dataclass
class Workload:
    name: str
    op: str            # "softmax" | "layernorm" | "rmsnorm"
    dt: str
    M: int
    N: int
    eps: float = 0.0
    desc: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dt]

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move per call: read x once, write y once,
        read each length-N parameter vector once, write the per-row stats;
        the fused add + norm also reads the residual once and writes h once."""
        e = self.elem_bytes
        if self.op == "softmax_causal":
            Q, off = self.extra["queries"], self.extra.get("offset", 0)
            q = np.arange(self.M, dtype=np.int64) % Q
            return int(np.minimum(self.N, q + off + 1).sum()) * e + self.M * self.N * e
        b = 2 * self.M * self.N * e
        if self.op.startswith("add_"):
            b += 2 * self.M * self.N * e
        if self.op in ("layernorm", "add_layernorm"):
            b += 2 * self.N * e + 2 * self.M * 4
        elif self.op in ("rmsnorm", "add_rmsnorm"):
            b += self.N * e
        return b

    def make(self, rows=None, M=None):
        """Generate inputs. ``rows`` selects a sorted subset of rows (values
        identical to the full draw); ``M`` overrides the row count (prefix)."""
        return _MAKERS[self.name](self, rows=rows, M=M or self.M)


def _mk_softmax_f32(w, rows, M):
    return {"x": normal_rows(101, M, w.N, F32, rows=rows)}


def _mk_layernorm(w, rows, M):
    rng_mu = np.random.default_rng(201)
    mu = rng_mu.uniform(-5.0, 5.0, size=M)
    rng = np.random.default_rng(202)
    keep = None if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((M if keep is None else len(keep), w.N), dtype=np.uint16)
    pos = 0
    for r0 in range(0, M, 1024):
        r1 = min(M, r0 + 1024)
        z = rng.standard_normal((r1 - r0) * w.N).reshape(r1 - r0, w.N)
        v = z + mu[r0:r1, None]
        if keep is None:
            out[r0:r1] = encode(v, F16)
        else:
            sel = keep[(keep >= r0) & (keep < r1)]
            if len(sel):
                out[pos:pos + len(sel)] = encode(v[sel - r0], F16)
                pos += len(sel)
    sq = float(np.sqrt(0.1))
    return {"x": out, "gamma": vector(203, w.N, F16, sq, 1.0),
            "beta": vector(204, w.N, F16, sq, 0.0)}


def _mk_rmsnorm(w, rows, M):
    return {"x": normal_rows(301, M, w.N, BF16, rows=rows),
            "weight": vector(302, w.N, BF16, float(np.sqrt(0.1)), 1.0)}


def causal_mask_rows(x: np.ndarray, row_ids: np.ndarray, n_queries: int) -> np.ndarray:
    """Set key > query entries to -inf (bf16 bits) for rows r with query r mod n_queries."""
    N = x.shape[1]
    q = (np.asarray(row_ids) % n_queries)[:, None]
    k = np.arange(N)[None, :]
    x[k > q] = NEG_INF_BITS[BF16]
    return x


def _mk_causal(w, rows, M):
    x = normal_rows(401, M, w.N, BF16, scale=3.0, rows=rows)
    ids = np.arange(M) if rows is None else np.asarray(rows)
    return {"x": causal_mask_rows(x, ids, w.extra["queries"])}


def _mk_vocab(w, rows, M):
    x = normal_rows(501, M, w.N, F32, scale=2.0, rows=rows)
    rng = np.random.default_rng(502)
    spikes = np.stack([rng.choice(w.N, 8, replace=False) for _ in range(M)])
    sel = np.arange(M) if rows is None else np.asarray(rows)
    for i, r in enumerate(sel):
        x[i, spikes[r]] = np.float32(30.0)
    return {"x": x, "spikes": spikes[sel]}


def _mk_add_rmsnorm(w, rows, M):
    d = _mk_rmsnorm(w, rows, M)
    d["residual"] = normal_rows(303, M, w.N, BF16, rows=rows)
    return d


def _mk_add_layernorm(w, rows, M):
    d = _mk_layernorm(w, rows, M)
    d["residual"] = normal_rows(205, M, w.N, F16, rows=rows)
    return d


_MAKERS = {
    "softmax_f32_1024x781": _mk_softmax_f32,
    "layernorm_f16_4096": _mk_layernorm,
    "rmsnorm_bf16_16384x8192": _mk_rmsnorm,
    "causal_softmax_bf16": _mk_causal,
    "vocab_softmax_f32": _mk_vocab,
    "add_rmsnorm_bf16_16384x8192": _mk_add_rmsnorm,
    "add_layernorm_f16_4096": _mk_add_layernorm,
    "causal_entry_softmax_bf16": _mk_causal,
}

WORKLOADS = [
    Workload("softmax_f32_1024x781", "softmax", F32, 1024, 781,
             desc="row softmax fp32, 1024 x 781 (non-power-of-two tail)"),
    Workload("layernorm_f16_4096", "layernorm", F16, 4096, 4096, eps=1e-5,
             desc="LayerNorm fp16 4096 x 4096, rows N(mu_row,1), mu_row~U(-5,5)"),
    Workload("rmsnorm_bf16_16384x8192", "rmsnorm", BF16, 16384, 8192, eps=1e-6,
             desc="RMSNorm bf16 16384 x 8192"),
    Workload("causal_softmax_bf16", "softmax", BF16, 131072, 4096,
             desc="causal attention-score softmax bf16, 32 heads x 4096 q x 4096 k",
             extra={"queries": 4096, "heads": 32}),
    Workload("vocab_softmax_f32", "softmax", F32, 64, 262144,
             desc="vocab-width softmax fp32 64 x 262144 with 8 spikes of +30 per row"),
]
NEXT_WORKLOADS = [
    Workload("add_rmsnorm_bf16_16384x8192", "add_rmsnorm", BF16, 16384, 8192, eps=1e-6,
             desc="fused residual add + RMSNorm bf16 16384 x 8192"),
    Workload("add_layernorm_f16_4096", "add_layernorm", F16, 4096, 4096, eps=1e-5,
             desc="fused residual add + LayerNorm fp16 4096 x 4096"),
    Workload("causal_entry_softmax_bf16", "softmax_causal", BF16, 131072, 4096,
             desc="causal softmax entry (masked keys not read), 32 heads x 4096 q x 4096 k",
             extra={"queries": 4096, "heads": 32, "offset": 0, "scale": 1.0}),
]
BY_NAME = {w.name: w for w in WORKLOADS + NEXT_WORKLOADS}


# Attention forward (the online-softmax loop over key/value tiles of "How
# Flash Attention Uses Triton"): q, k, v ~ N(0,1) in bf16, [heads, L, D].
# The pages give no attention workload; this is a causal square shape at the
# causal-score workload's size (32 heads x 4096 queries x 4096 keys), with
# head dimension 128 and scale 1/sqrt(128).
ATTENTION = {"name": "attention_fwd_bf16_32x4096x4096x128_causal", "dt": BF16, "BH": 32, "Lq": 4096,
             "Lk": 4096, "D": 128, "causal": True, "offset": 0, "scale": float(1.0 / np.sqrt(128.0))}


def attention_inputs(BH: int, Lq: int, Lk: int, D: int, dt: str, seed: int = 601, qk_scale: float = 1.0):
    """q [BH, Lq, D], k and v [BH, Lk, D] of N(0,1) draws (q and k times
    qk_scale), seeds seed, seed + 1, seed + 2, stored in `dt`."""
    q = normal_rows(seed, BH * Lq, D, dt, scale=qk_scale).reshape(BH, Lq, D)
    k = normal_rows(seed + 1, BH * Lk, D, dt, scale=qk_scale).reshape(BH, Lk, D)
    v = normal_rows(seed + 2, BH * Lk, D, dt).reshape(BH, Lk, D)
    return q, k, v


def attention_visible_pairs(BH: int, Lq: int, Lk: int, causal: bool, offset: int = 0) -> int:
    """(query, key) pairs the attention forward computes: BH * Lq * Lk, or,
    causal, BH * sum_i min(Lk, i + offset + 1)."""
    if not causal:
        return BH * Lq * Lk
    i = np.arange(Lq, dtype=np.int64)
    return BH * int(np.minimum(Lk, i + offset + 1).sum())
