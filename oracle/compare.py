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
* ``f32_errors`` extends the fp32 criterion below the normal range: the
  relative error everywhere, and below 2^-126, where fp32 has a fixed
  quantum of 2^-149 and the relative bar becomes finer than the format can
  resolve, one quantum from the correctly rounded value as well.
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


F32_MIN_NORMAL = 2.0 ** -126
F32_SUB_QUANTUM = 2.0 ** -149


def f32_errors(gpu_bits: np.ndarray, ref: np.ndarray, rel_bar: float = 1e-5):
    """(relative error over the outputs whose reference rounds to a normal
    fp32; distance in 2^-149 quanta from RNE_f32(reference) over the outputs
    below 2^-126 whose relative error exceeds `rel_bar`).  Below 2^-126 fp32
    has a fixed quantum, so there the relative bar holds where it can (near
    the top of that range one quantum is far finer than it) and one quantum
    from the correctly rounded value is granted where it cannot.

    Exact zeros are required where the reference is exactly zero (relative
    error inf otherwise); NaN must match NaN (inf otherwise)."""
    y = bits_to_f64(gpu_bits, "f32")
    ref = np.asarray(ref, dtype=np.float64)
    r32 = round_to_value(ref, "f32")
    sub = np.isfinite(ref) & (np.abs(r32) < F32_MIN_NORMAL) & (ref != 0)
    rel = max_rel_err(y[~sub], ref[~sub])
    if not np.any(sub):
        return rel, 0.0
    ys, rs, r32s = y[sub], ref[sub], r32[sub]
    with np.errstate(invalid="ignore"):
        beyond = ~(np.abs(ys - rs) <= rel_bar * np.abs(rs))       # NaN counts as beyond
    if not np.any(beyond):
        return rel, 0.0
    quanta = float(np.max(np.abs(ys[beyond] - r32s[beyond]) / F32_SUB_QUANTUM))
    return rel, quanta if np.isfinite(quanta) else float("inf")


def _parts(n: int, threads: int):
    step = max(1, -(-n // threads))
    return [(i, min(n, i + step)) for i in range(0, n, step)]


def _threads(threads):
    import os
    return max(1, min(16, threads or os.cpu_count() or 1))


def max_ulp_distance(gpu_bits: np.ndarray, ref64: np.ndarray, dt, threads=None) -> int:
    """max over all elements of ulp_distance, computed on row blocks in a
    thread pool (numpy releases the GIL): the same numbers, faster."""
    from concurrent.futures import ThreadPoolExecutor
    g = np.asarray(gpu_bits).reshape(-1)
    r = np.asarray(ref64).reshape(-1)
    if g.size == 0:
        return 0
    with ThreadPoolExecutor(_threads(threads)) as ex:
        return max(ex.map(lambda ab: int(ulp_distance(g[ab[0]:ab[1]], r[ab[0]:ab[1]], dt).max()),
                          _parts(g.size, 4 * _threads(threads))))


def f32_errors_threaded(gpu_bits: np.ndarray, ref: np.ndarray, threads=None):
    """f32_errors on blocks in a thread pool: (max relative error, max quanta)."""
    from concurrent.futures import ThreadPoolExecutor
    g = np.asarray(gpu_bits).reshape(-1)
    r = np.asarray(ref).reshape(-1)
    if g.size == 0:
        return 0.0, 0.0
    with ThreadPoolExecutor(_threads(threads)) as ex:
        res = list(ex.map(lambda ab: f32_errors(g[ab[0]:ab[1]], r[ab[0]:ab[1]]), _parts(g.size, 4 * _threads(threads))))
    return max(a for a, _ in res), max(b for _, b in res)


def ulp_of(ref64: np.ndarray, dt) -> np.ndarray:
    """Spacing of `dt` at RNE_dt(ref): 2^(e - p + 1) for the rounded value's
    binade e (at least the subnormal quantum)."""
    key = _fmt(dt)
    p, emin, _ = _FORMATS[key]
    r = np.abs(round_to_value(np.asarray(ref64, dtype=np.float64), key))
    _, e2 = np.frexp(np.where(r > 0, r, 1.0))
    e = np.maximum(e2.astype(np.int64) - 1, emin)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int32))


ATTN_REL = 2.0 ** -12


def attention_errors(gpu_bits: np.ndarray, ref64: np.ndarray, abs64: np.ndarray, dt) -> float:
    """max over outputs of |y - ref| / (ulp_dt(ref) + 2^-12 * A), A the size
    of the summed terms (the oracle's sum_j w_j |v_j| / sum_j w_j): the
    attention bar is met when this is <= 1.  NaN anywhere gives inf."""
    y = bits_to_f64(gpu_bits, dt)
    ref = np.asarray(ref64, dtype=np.float64)
    bound = ulp_of(ref, dt) + ATTN_REL * np.asarray(abs64, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        q = np.abs(y - ref) / bound
    if q.size == 0:
        return 0.0
    m = float(np.max(q))
    return m if np.isfinite(m) and not np.isnan(q).any() else float("inf")
