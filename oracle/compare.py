"""Comparators between a GPU result and the oracle's float64 result.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* ``round_to(v, dt)`` rounds float64 values ONCE, round-to-nearest-even, to
  the output storage type (fp32, fp16 or bf16, subnormals and overflow
  included) and returns the stored bit patterns.  It is written from the IEEE
  754 definition (scale to an integer significand, ``rint`` ties-to-even,
  rescale) rather than through a chain of casts, so there is no double
  rounding.
* ``ordinal(bits, dt)`` maps bit patterns onto consecutive integers in value
  order (+0 and -0 both map to 0), so ``|ordinal(a) - ordinal(b)|`` is the
  distance in units in the last place.
* ``max_rel_err`` is the fp32 criterion: max |y - y_ref| / |y_ref| with exact
  zeros required where the reference is exactly zero.
"""
from __future__ import annotations

import numpy as np

# (significand bits incl. the implicit one, minimum normal exponent, max exponent)
_FORMATS = {
    "f32": (24, -126, 127),
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
}
_ALIASES = {"float32": "f32", "float16": "f16", "bfloat16": "bf16", 0: "f32", 1: "f16", 2: "bf16"}


def _fmt(dt):
    key = _ALIASES.get(dt, dt)
    if isinstance(key, str):
        key = key.replace("torch.", "")
        key = _ALIASES.get(key, key)
    return key


def round_to_value(v: np.ndarray, dt) -> np.ndarray:
    """float64 -> nearest representable value of `dt` (ties to even), as float64."""
    key = _fmt(dt)
    p, emin, emax = _FORMATS[key]
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, dtype=np.float64, copy=True)
    fin = np.isfinite(v) & (v != 0)
    a = np.abs(v[fin])
    _, e2 = np.frexp(a)            # a = f * 2**e2, f in [0.5, 1)
    e = e2.astype(np.int64) - 1    # a in [2**e, 2**(e+1))
    e = np.maximum(e, emin)        # subnormal range shares the emin quantum
    q = e - (p - 1)                # exponent of one unit in the last place
    n = np.ldexp(a, (-q).astype(np.int32))
    r = np.rint(n)                 # round half to even
    res = np.ldexp(r, q.astype(np.int32))
    big = res >= np.ldexp(1.0, emax + 1)
    res[big] = np.inf
    out[fin] = np.copysign(res, v[fin])
    return out


def round_to(v: np.ndarray, dt) -> np.ndarray:
    """float64 -> stored bit patterns of `dt` (uint32 for f32, uint16 otherwise)."""
    key = _fmt(dt)
    r = round_to_value(v, key)
    if key == "f32":
        return r.astype(np.float32).view(np.uint32)        # exact: r is representable
    if key == "f16":
        return r.astype(np.float16).view(np.uint16)        # exact: r is representable
    u = r.astype(np.float32).view(np.uint32)               # bf16 values are exact in f32
    return (u >> 16).astype(np.uint16)


def ordinal(bits: np.ndarray, dt) -> np.ndarray:
    """Stored bit patterns -> signed integers in value order (+0 == -0 == 0)."""
    key = _fmt(dt)
    b = np.asarray(bits)
    if key == "f32":
        u = b.astype(np.uint32).astype(np.int64)
        sign, mag = u >> 31, u & 0x7FFFFFFF
    else:
        u = b.astype(np.uint16).astype(np.int64)
        sign, mag = u >> 15, u & 0x7FFF
    return np.where(sign == 1, -mag, mag)


def is_nan_bits(bits: np.ndarray, dt) -> np.ndarray:
    key = _fmt(dt)
    b = np.asarray(bits).astype(np.int64)
    if key == "f32":
        return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)
    if key == "f16":
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def ulp_distance(gpu_bits: np.ndarray, ref64: np.ndarray, dt) -> np.ndarray:
    """|ordinal(gpu) - ordinal(RNE(ref))| per element; NaN pairs count as 0."""
    key = _fmt(dt)
    ref_bits = round_to(ref64, key)
    d = np.abs(ordinal(gpu_bits, key) - ordinal(ref_bits, key))
    gn, rn = is_nan_bits(gpu_bits, key), np.isnan(ref64)
    d = np.where(gn & rn, 0, d)
    d = np.where(gn ^ rn, np.iinfo(np.int64).max, d)
    return d


def bits_to_f64(bits: np.ndarray, dt) -> np.ndarray:
    """Exact decode of stored GPU outputs to float64 (independent of oracle.c)."""
    key = _fmt(dt)
    b = np.asarray(bits)
    if key == "f32":
        return b.astype(np.uint32).view(np.float32).astype(np.float64)
    if key == "f16":
        return b.astype(np.uint16).view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def max_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - ref| / |ref|; where ref == 0, y must be exactly 0 (else inf).

    NaN in both at the same place counts as agreement; NaN in one only is inf.
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    yn, rn = np.isnan(y), np.isnan(ref)
    if np.any(yn ^ rn):
        return float("inf")
    ok = ~(yn | rn)
    y, ref = y[ok], ref[ok]
    zero = ref == 0
    if np.any(y[zero] != 0):
        return float("inf")
    nz = ~zero
    if not np.any(nz):
        return 0.0
    return float(np.max(np.abs(y[nz] - ref[nz]) / np.abs(ref[nz])))
