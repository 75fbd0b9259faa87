"""Helpers for the GPU parity tests: move stored bit patterns to and from the
device and compare GPU outputs with the oracle's float64 results."""
from __future__ import annotations

import numpy as np

import oracle
from oracle import compare

TORCH_DT = None


def tdt(dt):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]


def to_dev(bits: np.ndarray, dt: str, offset: int = 0):
    """Host storage array -> device tensor of type dt.  With offset > 0 the
    tensor is a view starting `offset` elements into a larger allocation, so
    its address is misaligned relative to 16 bytes."""
    import torch
    b = np.ascontiguousarray(bits)
    if dt == "f32":
        t = torch.from_numpy(b.view(np.float32))
    else:
        t = torch.from_numpy(b.view(np.int16)).view(tdt(dt))
    if offset == 0:
        return t.cuda()
    flat = torch.empty(b.size + offset + 8, dtype=tdt(dt), device="cuda")
    v = flat[offset:offset + b.size].view(b.shape)
    v.copy_(t.cuda())
    return v


def empty_like_dev(shape, dt: str, offset: int = 0):
    import torch
    n = int(np.prod(shape))
    flat = torch.empty(n + offset + 8, dtype=tdt(dt), device="cuda")
    flat.fill_(float("nan"))     # poison: any element the kernel skips shows up
    return flat[offset:offset + n].view(shape)


def to_host_bits(t, dt: str) -> np.ndarray:
    import torch
    t = t.contiguous().cpu()
    if dt == "f32":
        return t.numpy().view(np.uint32).copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def check_output(gpu_bits: np.ndarray, ref64: np.ndarray, dt: str, what: str = ""):
    """The parity bar: fp32 -> max relative error <= 1e-5 (exact zeros where the
    oracle is exactly zero), or, below 2^-126, within 2^-149 of the correctly
    rounded value; fp16/bf16 -> at most 1 ulp from the oracle
    rounded once to the output type (subnormals included: ulps are counted
    on the ordered representable values).  Large arrays are compared on
    blocks in a thread pool (the same numbers)."""
    big = gpu_bits.size > (1 << 22)
    if dt == "f32":
        # relative 1e-5; below 2^-126, where fp32's fixed quantum (2^-149)
        # can be coarser than that, one quantum from the correctly rounded
        # value is granted as well
        err, quanta = (compare.f32_errors_threaded if big else compare.f32_errors)(gpu_bits, ref64)
        assert err <= 1e-5, f"{what}: max rel err {err:.3e} > 1e-5"
        assert quanta <= 1.0, f"{what}: {quanta} subnormal quanta from the correctly rounded value"
        return err
    if big:
        worst = compare.max_ulp_distance(gpu_bits, ref64, dt)
        if worst <= 1:
            return worst
    d = compare.ulp_distance(gpu_bits, ref64, dt)
    worst = int(d.max()) if d.size else 0
    if worst > 1:
        idx = np.unravel_index(int(np.argmax(d)), d.shape)
        raise AssertionError(f"{what}: {int((d > 1).sum())} elements beyond 1 ulp; worst {worst} ulp at {idx}: "
                             f"gpu={compare.bits_to_f64(gpu_bits[idx], dt)} ref={ref64[idx]}")
    return worst


def row_blocks(M: int, N: int, align: int = 1, elems: int = 1 << 25):
    """Row ranges of about `elems` elements each, starting at multiples of
    `align` rows: the full-size checks walk every row in such blocks."""
    b = max(align, (elems // max(N, 1)) // align * align)
    return [(r0, min(M, r0 + b)) for r0 in range(0, M, b)]


def check_stats(gpu: np.ndarray, ref64: np.ndarray, what: str = ""):
    err = compare.max_rel_err(gpu.astype(np.float64), ref64)
    assert err <= 1e-5, f"{what}: max rel err {err:.3e} > 1e-5"
    return err


def oracle_for(op: str, x, dt, eps=0.0, p0=None, p1=None):
    if op == "softmax":
        return oracle.softmax(x, dt), None, None
    if op == "layernorm":
        return oracle.layernorm(x, dt, eps, gamma=p0, beta=p1)
    return oracle.rmsnorm(x, dt, eps, weight=p0), None, None
