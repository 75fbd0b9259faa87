"""Python binding of the MI355X row-reduction library (``libnt.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/nt.h``.  The ``nt_*``
functions take the same arguments as their C counterparts (pointers as
integers, ``stream`` as a ``hipStream_t`` handle) and return the status code.
``softmax``, ``softmax_causal``, ``layer_norm``, ``rms_norm``,
``add_layer_norm`` and ``add_rms_norm`` are conveniences over torch
tensors on an AMD GPU: they check contiguity, allocate outputs (and the
split-path workspace) with torch, and launch on torch's current stream, or
on the `stream` given (then the allocations belong to that stream).

There is no fallback: if ``libnt.so`` is missing or the call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnt.so")

NT_F32, NT_F16, NT_BF16 = 0, 1, 2
NT_OP_SOFTMAX, NT_OP_LAYERNORM, NT_OP_RMSNORM, NT_OP_ADD_LAYERNORM, NT_OP_ADD_RMSNORM = 0, 1, 2, 3, 4
NT_OP_SOFTMAX_CAUSAL = 5
NT_OP_LAYERNORM_WS = 6
NT_OP_RMSNORM_WS = 7
STATUS = {0: "NT_OK", 1: "NT_ERR_NULL", 2: "NT_ERR_SHAPE", 3: "NT_ERR_DTYPE", 4: "NT_ERR_EPS",
          5: "NT_ERR_ALIGN", 6: "NT_ERR_WORKSPACE", 7: "NT_ERR_HIP", 8: "NT_ERR_ALIAS",
          9: "NT_ERR_SCALE", 10: "NT_ERR_OVERRIDE"}
EXPORTED = ("nt_softmax_workspace_bytes", "nt_softmax_rows", "nt_softmax_causal_rows", "nt_layernorm_rows",
            "nt_rmsnorm_rows", "nt_norm_workspace_bytes", "nt_layernorm_rows_ws", "nt_rmsnorm_rows_ws",
            "nt_add_layernorm_rows", "nt_add_rmsnorm_rows",
            "nt_status_string", "nt_plan_launch", "nt_set_override", "nt_softmax_rows_noalloc", "nt_attention_fwd")
NT_NOALLOC_SCRATCH_BYTES = 1 << 20


class NtError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, code)} ({status_string(code)})")
        self.code = code


class nt_plan(ctypes.Structure):
    _fields_ = [("split", ctypes.c_int32), ("waves_per_row", ctypes.c_int32),
                ("chunks_per_lane", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
                ("threads_per_block", ctypes.c_int32), ("aligned", ctypes.c_int32),
                ("persistent", ctypes.c_int32), ("cooperative", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("row_chunks", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def lib():
    """Load libnt.so (built by ``row_wise_reductions_amd.build``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m row_wise_reductions_amd.build` first")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, f32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    i32 = ctypes.c_int
    L.nt_softmax_workspace_bytes.argtypes = [i64, i64, i32]
    L.nt_softmax_workspace_bytes.restype = sz
    L.nt_softmax_rows.argtypes = [i64, i64, i32, vp, vp, vp, sz, vp]
    L.nt_softmax_rows_noalloc.argtypes = [i64, i64, i32, vp, vp, vp]
    L.nt_attention_fwd.argtypes = [i64, i64, i64, i64, i32, f32, i32, i64, vp, vp, vp, vp, vp]
    L.nt_softmax_causal_rows.argtypes = [i64, i64, i32, f32, i64, i64, vp, vp, vp, sz, vp]
    L.nt_layernorm_rows.argtypes = [i64, i64, i32, f32, vp, vp, vp, vp, vp, vp, vp]
    L.nt_rmsnorm_rows.argtypes = [i64, i64, i32, f32, vp, vp, vp, vp]
    L.nt_norm_workspace_bytes.argtypes = [i32, i64, i64, i32]
    L.nt_norm_workspace_bytes.restype = sz
    L.nt_layernorm_rows_ws.argtypes = [i64, i64, i32, f32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.nt_rmsnorm_rows_ws.argtypes = [i64, i64, i32, f32, vp, vp, vp, vp, sz, vp]
    L.nt_add_layernorm_rows.argtypes = [i64, i64, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.nt_add_rmsnorm_rows.argtypes = [i64, i64, i32, f32, vp, vp, vp, vp, vp, vp]
    L.nt_status_string.argtypes = [i32]
    L.nt_status_string.restype = ctypes.c_char_p
    L.nt_plan_launch.argtypes = [i32, i64, i64, i32, i32, ctypes.POINTER(nt_plan)]
    L.nt_set_override.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
    for f in ("nt_set_override", "nt_softmax_rows_noalloc", "nt_attention_fwd", "nt_softmax_rows", "nt_softmax_causal_rows", "nt_layernorm_rows", "nt_rmsnorm_rows",
              "nt_layernorm_rows_ws", "nt_rmsnorm_rows_ws", "nt_add_layernorm_rows",
              "nt_add_rmsnorm_rows", "nt_plan_launch"):
        getattr(L, f).restype = i32
    _lib = L
    return L


# ---- the C ABI, one to one -------------------------------------------------

def nt_softmax_workspace_bytes(M: int, N: int, dt: int) -> int:
    return int(lib().nt_softmax_workspace_bytes(M, N, dt))


def nt_softmax_rows(M, N, dt, x, y, workspace, workspace_bytes, stream) -> int:
    return int(lib().nt_softmax_rows(M, N, dt, x, y, workspace, workspace_bytes, stream))


def nt_softmax_rows_noalloc(M, N, dt, x, y, stream) -> int:
    return int(lib().nt_softmax_rows_noalloc(M, N, dt, x, y, stream))


def nt_attention_fwd(BH, Lq, Lk, D, dt, scale, causal, offset, q, k, v, o, stream) -> int:
    return int(lib().nt_attention_fwd(BH, Lq, Lk, D, dt, scale, causal, offset, q, k, v, o, stream))


def nt_softmax_causal_rows(M, N, dt, scale, queries, offset, x, y, workspace, workspace_bytes, stream) -> int:
    return int(lib().nt_softmax_causal_rows(M, N, dt, scale, queries, offset, x, y, workspace, workspace_bytes,
                                            stream))


def nt_layernorm_rows(M, N, dt, eps, x, gamma, beta, y, mean, rstd, stream) -> int:
    return int(lib().nt_layernorm_rows(M, N, dt, eps, x, gamma, beta, y, mean, rstd, stream))


def nt_rmsnorm_rows(M, N, dt, eps, x, weight, y, stream) -> int:
    return int(lib().nt_rmsnorm_rows(M, N, dt, eps, x, weight, y, stream))


def nt_norm_workspace_bytes(op: int, M: int, N: int, dt: int) -> int:
    return int(lib().nt_norm_workspace_bytes(op, M, N, dt))


def nt_layernorm_rows_ws(M, N, dt, eps, x, gamma, beta, y, mean, rstd, workspace, workspace_bytes, stream) -> int:
    return int(lib().nt_layernorm_rows_ws(M, N, dt, eps, x, gamma, beta, y, mean, rstd, workspace, workspace_bytes,
                                          stream))


def nt_rmsnorm_rows_ws(M, N, dt, eps, x, weight, y, workspace, workspace_bytes, stream) -> int:
    return int(lib().nt_rmsnorm_rows_ws(M, N, dt, eps, x, weight, y, workspace, workspace_bytes, stream))


def nt_add_layernorm_rows(M, N, dt, eps, x, residual, gamma, beta, h, y, mean, rstd, stream) -> int:
    return int(lib().nt_add_layernorm_rows(M, N, dt, eps, x, residual, gamma, beta, h, y, mean, rstd, stream))


def nt_add_rmsnorm_rows(M, N, dt, eps, x, residual, weight, h, y, stream) -> int:
    return int(lib().nt_add_rmsnorm_rows(M, N, dt, eps, x, residual, weight, h, y, stream))


def nt_status_string(code: int) -> str:
    return lib().nt_status_string(code).decode()


def nt_plan_launch(op: int, M: int, N: int, dt: int, aligned16: bool = True) -> dict:
    p = nt_plan()
    rc = lib().nt_plan_launch(op, M, N, dt, 1 if aligned16 else 0, ctypes.byref(p))
    if rc != 0:
        raise NtError(rc, "nt_plan_launch")
    return p.as_dict()


def nt_set_override(name: str, value) -> int:
    return int(lib().nt_set_override(name.encode(), None if value is None else str(value).encode()))


# The overrides this module has set (name -> value; absent = the value the
# library read from the environment at load).
_overrides = {}


def set_override(name: str, value) -> None:
    """Set one tuning override (value None: back to the load-time value)."""
    _check(nt_set_override(name, value), f"nt_set_override({name!r}, {value!r})")
    if value is None:
        _overrides.pop(name, None)
    else:
        _overrides[name] = str(value)


class override:
    """Context manager: tuning overrides (NT_COOP="0", NT_FORCE_SHAPE="4,2",
    ...) for the calls made inside it; the previous settings are restored on
    exit.  Process-wide: not for use while other threads call the library."""

    def __init__(self, **kv):
        self.kv, self.saved = kv, {}

    def __enter__(self):
        for k, v in self.kv.items():
            self.saved[k] = _overrides.get(k)
            set_override(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            set_override(k, v)


def status_string(code: int) -> str:
    try:
        return nt_status_string(code)
    except Exception:
        return "?"


# ---- torch conveniences ----------------------------------------------------

def _torch():
    import torch
    return torch


_CODES = {}


def dtype_code(t) -> int:
    if not _CODES:
        torch = _torch()
        _CODES.update({torch.float32: NT_F32, torch.float16: NT_F16, torch.bfloat16: NT_BF16})
    if t.dtype not in _CODES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _CODES[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, x=None):
    """The hipStream_t to enqueue on: `stream` (a torch stream or a raw
    handle), else the current stream of x's device.  torch's raw accessor
    returns the same handle as torch.cuda.current_stream().cuda_stream
    without building a Stream object (about 2.5 us less per call)."""
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None and x is not None and x.device.index is not None:
        return raw(x.device.index)
    return torch.cuda.current_stream().cuda_stream


class _alloc_on:
    """Allocations made inside belong to the stream the kernels run on.  With
    an explicit `stream` (a torch stream or a raw hipStream_t handle) torch's
    caching allocator is told so (torch.cuda.stream): a buffer created here
    and dropped on return -- the split path's workspace -- is then not handed
    to another stream's allocation while these kernels may still use it, and
    is not a block that a kernel still running on the current stream uses.
    Without one, the current stream is the launch stream already."""

    def __init__(self, stream, x):
        self.ctx = None
        if stream is not None:
            torch = _torch()
            if not isinstance(stream, torch.cuda.Stream):
                stream = torch.cuda.ExternalStream(int(stream), device=x.device)
            self.ctx = torch.cuda.stream(stream)

    def __enter__(self):
        if self.ctx is not None:
            self.ctx.__enter__()
        return self

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)


def _rows(x):
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (rows of stride N)")
    if x.dim() == 0:
        raise ValueError("x must have at least one dimension")
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    return M, N


def _on_device(x, *ts):
    """x on a GPU, every other tensor given (parameters, residual) on x's
    device: the library takes raw addresses and cannot tell them apart."""
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    for t in ts:
        if t is not None and t.device != x.device:
            raise ValueError("every tensor must be on x's device")


def _out_like(x, out, name="out"):
    """A new output like x, or the caller's, which must match x exactly
    (the kernels write M*N elements of x's type, row-major)."""
    if out is None:
        return _torch().empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError(f"{name} must be contiguous, on x's device, of x's shape and dtype")
    return out


def _check(code, what):
    if code != 0:
        raise NtError(code, what)


def softmax(x, out=None, stream=None):
    """Row softmax over the last dimension of a contiguous GPU tensor."""
    torch = _torch()
    M, N = _rows(x)
    _on_device(x)
    dt = dtype_code(x)
    with _alloc_on(stream, x):
        y = _out_like(x, out)
        wsb = nt_softmax_workspace_bytes(M, N, dt)
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device) if wsb else None
        _check(nt_softmax_rows(M, N, dt, _ptr(x), _ptr(y), _ptr(ws), wsb, _stream(stream, x)), "nt_softmax_rows")
    return y


def softmax_causal(x, scale=1.0, queries=None, offset=0, out=None, stream=None):
    """Causal softmax of scale*x over the last dimension: row r is query
    r mod `queries` (default: the second-to-last dimension) and sees keys
    k <= q + offset; masked outputs are 0 and masked inputs are not read."""
    torch = _torch()
    M, N = _rows(x)
    if queries is None:
        queries = x.shape[-2] if x.dim() >= 2 else 1
    _on_device(x)
    dt = dtype_code(x)
    with _alloc_on(stream, x):
        y = _out_like(x, out)
        wsb = nt_softmax_workspace_bytes(M, N, dt)
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device) if wsb else None
        _check(nt_softmax_causal_rows(M, N, dt, float(scale), int(queries), int(offset), _ptr(x), _ptr(y),
                                      _ptr(ws), wsb, _stream(stream, x)), "nt_softmax_causal_rows")
    return y


def layer_norm(x, gamma=None, beta=None, eps=1e-5, out=None, stream=None):
    """LayerNorm over the last dimension; returns (y, mean, rstd) (stats fp32)."""
    torch = _torch()
    M, N = _rows(x)
    _on_device(x, gamma, beta)
    for p in (gamma, beta):
        if p is not None and (p.numel() != N or p.dtype != x.dtype or not p.is_contiguous()):
            raise ValueError("gamma/beta must be contiguous, of x's dtype, with N entries")
    dt = dtype_code(x)
    lead = x.shape[:-1]
    with _alloc_on(stream, x):
        y = _out_like(x, out)
        mean = torch.empty(lead, dtype=torch.float32, device=x.device)
        rstd = torch.empty(lead, dtype=torch.float32, device=x.device)
        wsb = nt_norm_workspace_bytes(NT_OP_LAYERNORM, M, N, dt)     # a few rows too wide for one pass
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device) if wsb else None
        _check(nt_layernorm_rows_ws(M, N, dt, float(eps), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean),
                                    _ptr(rstd), _ptr(ws), wsb, _stream(stream, x)), "nt_layernorm_rows_ws")
    return y, mean, rstd


def rms_norm(x, weight=None, eps=1e-6, out=None, stream=None):
    """RMSNorm over the last dimension."""
    torch = _torch()
    M, N = _rows(x)
    _on_device(x, weight)
    if weight is not None and (weight.numel() != N or weight.dtype != x.dtype or not weight.is_contiguous()):
        raise ValueError("weight must be contiguous, of x's dtype, with N entries")
    dt = dtype_code(x)
    with _alloc_on(stream, x):
        y = _out_like(x, out)
        wsb = nt_norm_workspace_bytes(NT_OP_RMSNORM, M, N, dt)
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device) if wsb else None
        _check(nt_rmsnorm_rows_ws(M, N, dt, float(eps), _ptr(x), _ptr(weight), _ptr(y), _ptr(ws), wsb,
                                  _stream(stream, x)), "nt_rmsnorm_rows_ws")
    return y


def _same_rows(x, r):
    if r.shape != x.shape or r.dtype != x.dtype or not r.is_contiguous():
        raise ValueError("residual must be contiguous, of x's shape and dtype")


def add_layer_norm(x, residual, gamma=None, beta=None, eps=1e-5, h_out=None, out=None, stream=None):
    """Fused residual add + LayerNorm: h = x + residual (rounded to x's
    dtype), y = LayerNorm(h).  Returns (h, y, mean, rstd)."""
    torch = _torch()
    M, N = _rows(x)
    _same_rows(x, residual)
    _on_device(x, residual, gamma, beta)
    for p in (gamma, beta):
        if p is not None and (p.numel() != N or p.dtype != x.dtype or not p.is_contiguous()):
            raise ValueError("gamma/beta must be contiguous, of x's dtype, with N entries")
    lead = x.shape[:-1]
    with _alloc_on(stream, x):
        h = _out_like(x, h_out, "h_out")
        y = _out_like(x, out)
        mean = torch.empty(lead, dtype=torch.float32, device=x.device)
        rstd = torch.empty(lead, dtype=torch.float32, device=x.device)
        _check(nt_add_layernorm_rows(M, N, dtype_code(x), float(eps), _ptr(x), _ptr(residual), _ptr(gamma),
                                     _ptr(beta), _ptr(h), _ptr(y), _ptr(mean), _ptr(rstd), _stream(stream, x)),
               "nt_add_layernorm_rows")
    return h, y, mean, rstd


def add_rms_norm(x, residual, weight=None, eps=1e-6, h_out=None, out=None, stream=None):
    """Fused residual add + RMSNorm: h = x + residual (rounded to x's dtype),
    y = RMSNorm(h).  Returns (h, y)."""
    M, N = _rows(x)
    _same_rows(x, residual)
    _on_device(x, residual, weight)
    if weight is not None and (weight.numel() != N or weight.dtype != x.dtype or not weight.is_contiguous()):
        raise ValueError("weight must be contiguous, of x's dtype, with N entries")
    with _alloc_on(stream, x):
        h = _out_like(x, h_out, "h_out")
        y = _out_like(x, out)
        _check(nt_add_rmsnorm_rows(M, N, dtype_code(x), float(eps), _ptr(x), _ptr(residual), _ptr(weight),
                                   _ptr(h), _ptr(y), _stream(stream, x)), "nt_add_rmsnorm_rows")
    return h, y


def attention(q, k, v, scale=None, causal=False, offset=0, out=None, stream=None):
    """Attention forward, o = softmax(scale * q k^T) v per (batch, head),
    over the keys each query sees (all, or key <= query + offset when
    causal).  q: [..., Lq, D], k and v: [..., Lk, D] with the same leading
    dimensions, contiguous, fp16 or bf16, D = 64 or 128; scale defaults to
    1/sqrt(D).  Returns o like q."""
    import math
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dim() < 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with at least two dimensions")
    if k.shape != v.shape or k.shape[:-2] != q.shape[:-2] or k.shape[-1] != q.shape[-1]:
        raise ValueError("k and v must be [..., Lk, D] with q's leading dimensions and head size")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    _on_device(q, k, v)
    Lq, D = q.shape[-2], q.shape[-1]
    Lk = k.shape[-2]
    BH = q.numel() // (Lq * D) if Lq * D else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with _alloc_on(stream, q):
        o = _out_like(q, out)
        _check(nt_attention_fwd(BH, Lq, Lk, D, dtype_code(q), float(scale), 1 if causal else 0, int(offset),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(o), _stream(stream, q)), "nt_attention_fwd")
    return o
