"""CPU fp64 oracle for the fused row reductions (softmax, LayerNorm, RMSNorm).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``row_wise_reductions_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one OpenMP
thread per row block); this module only compiles it with gcc and marshals
numpy arrays.  ``brute.py`` is a second, independent pure-Python definition
used on tiny rows; ``compare.py`` rounds oracle results once to an output
storage type and measures ulp / relative distances.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# The oracle's own storage-type codes (mirrors the enum in oracle.c).
F32, F16, BF16 = 0, 1, 2
_CODES = {"f32": F32, "float32": F32, "f16": F16, "float16": F16,
          "bf16": BF16, "bfloat16": BF16}


def dtype_code(dt) -> int:
    if isinstance(dt, int):
        return dt
    return _CODES[str(dt).replace("torch.", "")]


def build(src: str = _SRC, out: str = _LIB_PATH, extra=()) -> str:
    """Compile oracle.c into a shared library with gcc (OpenMP, -O2)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str = _LIB_PATH):
    """Load (building first if absent or stale) the oracle library."""
    global _lib
    if path == _LIB_PATH and _lib is not None:
        return _lib
    if path == _LIB_PATH and (not os.path.exists(path) or
                              os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(path)
    i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    lib.or_decode.argtypes = [i64, i32, vp, dp]
    lib.or_softmax.argtypes = [i64, i64, i32, vp, dp]
    lib.or_layernorm.argtypes = [i64, i64, i32, ctypes.c_float, vp, vp, vp, dp, dp, dp]
    lib.or_rmsnorm.argtypes = [i64, i64, i32, ctypes.c_float, vp, vp, dp]
    lib.or_softmax_online.argtypes = [i64, i64, i32, i64, vp, dp]
    lib.or_add.argtypes = [i64, i32, vp, vp, dp]
    lib.or_softmax_causal.argtypes = [i64, i64, i32, ctypes.c_float, i64, i64, vp, dp]
    lib.or_attention.argtypes = [i64, i64, i64, i64, i32, ctypes.c_float, i32, i64, vp, vp, vp, i64, vp, dp, dp]
    lib.or_attention_online.argtypes = [i64, i64, i64, i64, i32, ctypes.c_float, i32, i64, i64, vp, vp, vp, dp]
    lib.or_num_threads.argtypes = []
    for f in ("or_decode", "or_softmax", "or_layernorm", "or_rmsnorm",
              "or_softmax_online", "or_add", "or_softmax_causal", "or_attention", "or_attention_online",
              "or_num_threads"):
        getattr(lib, f).restype = ctypes.c_int
    lib.or_set_num_threads.argtypes = [ctypes.c_int]
    lib.or_set_num_threads.restype = None
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_bits(a: np.ndarray, code: int) -> np.ndarray:
    """Storage view of an input array: float32 for F32, uint16 otherwise."""
    a = np.ascontiguousarray(a)
    if code == F32:
        if a.dtype != np.float32:
            raise TypeError("F32 input must be a float32 array")
        return a
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("16-bit input must be a uint16 (raw bits) or float16 array")
    return a


def _check(rc: int):
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")


def decode(bits: np.ndarray, dt) -> np.ndarray:
    """Exact decode of stored values (any shape) to float64."""
    code = dtype_code(dt)
    b = _as_bits(bits, code)
    out = np.empty(b.shape, dtype=np.float64)
    _check(load().or_decode(b.size, code, _ptr(b), _ptr(out)))
    return out


def softmax(x: np.ndarray, dt, lib=None) -> np.ndarray:
    code = dtype_code(dt)
    xb = _as_bits(x, code)
    M, N = xb.shape
    y = np.empty((M, N), dtype=np.float64)
    _check((lib or load()).or_softmax(M, N, code, _ptr(xb), _ptr(y)))
    return y


def softmax_causal(x: np.ndarray, dt, scale: float, queries: int, offset: int = 0, lib=None) -> np.ndarray:
    """Causal scaled softmax: row r (query r mod queries) sees keys
    k <= q + offset; masked outputs are 0 and masked inputs are not read."""
    code = dtype_code(dt)
    xb = _as_bits(x, code)
    M, N = xb.shape
    y = np.empty((M, N), dtype=np.float64)
    _check((lib or load()).or_softmax_causal(M, N, code, float(scale), int(queries), int(offset),
                                             _ptr(xb), _ptr(y)))
    return y


def softmax_online(x: np.ndarray, dt, block: int, lib=None) -> np.ndarray:
    code = dtype_code(dt)
    xb = _as_bits(x, code)
    M, N = xb.shape
    y = np.empty((M, N), dtype=np.float64)
    _check((lib or load()).or_softmax_online(M, N, code, block, _ptr(xb), _ptr(y)))
    return y


def layernorm(x: np.ndarray, dt, eps: float, gamma=None, beta=None, lib=None):
    """Returns (y, mean, rstd) in float64."""
    code = dtype_code(dt)
    xb = _as_bits(x, code)
    M, N = xb.shape
    g = None if gamma is None else _as_bits(gamma, code)
    b = None if beta is None else _as_bits(beta, code)
    for v in (g, b):
        if v is not None and v.size != N:
            raise ValueError("gamma/beta must have N entries")
    y = np.empty((M, N), dtype=np.float64)
    mean = np.empty(M, dtype=np.float64)
    rstd = np.empty(M, dtype=np.float64)
    _check((lib or load()).or_layernorm(M, N, code, float(eps), _ptr(xb), _ptr(g),
                                        _ptr(b), _ptr(y), _ptr(mean), _ptr(rstd)))
    return y, mean, rstd


def rmsnorm(x: np.ndarray, dt, eps: float, weight=None, lib=None) -> np.ndarray:
    code = dtype_code(dt)
    xb = _as_bits(x, code)
    M, N = xb.shape
    w = None if weight is None else _as_bits(weight, code)
    if w is not None and w.size != N:
        raise ValueError("weight must have N entries")
    y = np.empty((M, N), dtype=np.float64)
    _check((lib or load()).or_rmsnorm(M, N, code, float(eps), _ptr(xb), _ptr(w), _ptr(y)))
    return y


def add(x: np.ndarray, r: np.ndarray, dt, lib=None) -> np.ndarray:
    """Residual add h = x + r in float64 (same shape as x); round it once to
    the storage type with ``compare.round_to`` to get the stored h."""
    code = dtype_code(dt)
    xb, rb = _as_bits(x, code), _as_bits(r, code)
    if xb.shape != rb.shape:
        raise ValueError("x and r must have the same shape")
    h = np.empty(xb.shape, dtype=np.float64)
    _check((lib or load()).or_add(xb.size, code, _ptr(xb), _ptr(rb), _ptr(h)))
    return h


def _stored(h64: np.ndarray, dt) -> np.ndarray:
    """float64 -> the stored values of `dt`, in the layout the other oracle
    functions take (float32 array for f32, raw uint16 bits otherwise)."""
    from . import compare
    bits = compare.round_to(h64, dt)
    return bits.view(np.float32) if dtype_code(dt) == F32 else bits


def add_rmsnorm(x: np.ndarray, r: np.ndarray, dt, eps: float, weight=None, lib=None):
    """Fused residual add + RMSNorm, plain definition, unfused: h = x + r
    stored in the input type, then the RMSNorm of that stored h.  Returns
    (h as stored values, y in float64)."""
    h = _stored(add(x, r, dt, lib=lib), dt)
    return h, rmsnorm(h, dt, eps, weight=weight, lib=lib)


def add_layernorm(x: np.ndarray, r: np.ndarray, dt, eps: float, gamma=None, beta=None, lib=None):
    """Fused residual add + LayerNorm, plain definition, unfused.  Returns
    (h as stored values, y, mean, rstd), the last three in float64."""
    h = _stored(add(x, r, dt, lib=lib), dt)
    return (h,) + tuple(layernorm(h, dt, eps, gamma=gamma, beta=beta, lib=lib))


def _qkv(q, k, v, code):
    qb, kb, vb = (_as_bits(a, code) for a in (q, k, v))
    if qb.ndim != 3 or kb.ndim != 3 or vb.ndim != 3:
        raise ValueError("q, k, v must be [heads, length, head_dim] arrays")
    BH, Lq, D = qb.shape
    if kb.shape[0] != BH or kb.shape[2] != D or vb.shape != kb.shape:
        raise ValueError("k and v must be [heads, Lk, head_dim] like q")
    return qb, kb, vb, BH, Lq, kb.shape[1], D


def attention(q, k, v, dt, scale: float, causal: bool = False, offset: int = 0, rows=None, lib=None,
              with_abs: bool = False):
    """Attention forward, plain definition: softmax(scale Q K^T) V per head,
    keys j <= i + offset only when causal.  q [BH, Lq, D], k and v
    [BH, Lk, D] (stored values).  Returns float64 [BH, Lq, D], or [len(rows),
    D] for the rows b*Lq + i listed in `rows`; with `with_abs`, also the
    same-shaped sum_j w_j |v_j| / sum_j w_j (the size of the summed terms)."""
    code = dtype_code(dt)
    qb, kb, vb, BH, Lq, Lk, D = _qkv(q, k, v, code)
    if rows is None:
        r, n, shape = None, BH * Lq, (BH, Lq, D)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n, shape = r.size, (r.size, D)
    o = np.empty(shape, dtype=np.float64)
    oa = np.empty(shape, dtype=np.float64) if with_abs else None
    _check((lib or load()).or_attention(BH, Lq, Lk, D, code, float(scale), int(bool(causal)), int(offset),
                                        _ptr(qb), _ptr(kb), _ptr(vb), n, _ptr(r), _ptr(o), _ptr(oa)))
    return (o, oa) if with_abs else o


def attention_online(q, k, v, dt, scale: float, block: int, causal: bool = False, offset: int = 0, lib=None):
    """The page's tiled form of the attention forward (blocks of `block`
    keys, running max and rescaled accumulator).  float64 [BH, Lq, D]."""
    code = dtype_code(dt)
    qb, kb, vb, BH, Lq, Lk, D = _qkv(q, k, v, code)
    o = np.empty((BH, Lq, D), dtype=np.float64)
    _check((lib or load()).or_attention_online(BH, Lq, Lk, D, code, float(scale), int(bool(causal)), int(offset),
                                               int(block), _ptr(qb), _ptr(kb), _ptr(vb), _ptr(o)))
    return o


def num_threads() -> int:
    return int(load().or_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (timing only; results do not depend on it)."""
    load().or_set_num_threads(int(n))
