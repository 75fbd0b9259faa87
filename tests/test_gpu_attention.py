"""GPU parity of the attention forward (nt_attention_fwd, the online-softmax
loop of "Triton: Block-Level GPU Programming Without CUDA", "How Flash
Attention Uses Triton", on the matrix cores) against the oracle's plain
softmax(scale Q K^T) V, through the C ABI.

Bar (derived from the arithmetic; fp32 accumulation cannot keep a result
that cancels within one ulp): |o - o_ref| <= ulp(o_ref) + 2^-12 * A per
output, A = sum_j w_j |v_j| / sum_j w_j the size of the terms it sums (the
oracle computes it).  Shapes: ragged query and key lengths (not multiples
of the 128-query blocks or 64-key tiles), causal with offsets, both
head dimensions and both 16-bit types; the full 32 x 4096 x 4096 x 128 bf16
causal shape on sampled rows; argument errors; determinism.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import to_dev, to_host_bits
import oracle
from oracle import compare
import workloads

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import torch  # noqa: E402

import row_wise_reductions_amd as nt  # noqa: E402

DT_CODE = {"f16": nt.NT_F16, "bf16": nt.NT_BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(q_t, k_t, v_t, dt, scale, causal, offset, o=None):
    BH, Lq, D = q_t.shape
    Lk = k_t.shape[1]
    o = torch.full((BH, Lq, D), float("nan"), dtype=q_t.dtype, device="cuda") if o is None else o
    rc = nt.nt_attention_fwd(BH, Lq, Lk, D, DT_CODE[dt], scale, int(causal), offset, q_t.data_ptr(), k_t.data_ptr(),
                             v_t.data_ptr(), o.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, nt.nt_status_string(rc)
    torch.cuda.synchronize()
    return o


def check(o_bits, ref, absref, dt, what):
    q = compare.attention_errors(o_bits, ref, absref, dt)
    assert q <= 1.0, f"{what}: error {q:.3f} of the bar (ulp + 2^-12 * A)"
    return q


CASES = [  # (BH, Lq, Lk, D, causal, offset)
    (1, 1, 1, 64, False, 0), (2, 7, 5, 64, False, 0), (1, 64, 64, 128, True, 0), (3, 100, 129, 128, True, 29),
    (2, 128, 128, 64, True, 0), (1, 129, 300, 128, False, 0), (2, 300, 300, 128, True, 0),
    (1, 257, 1000, 64, True, 743), (1, 200, 64, 128, True, 3), (4, 33, 65, 128, True, 32),
]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}{'c' if c[4] else ''}{c[5]}" for c in CASES])
def test_attention_shapes(dt, case):
    BH, Lq, Lk, D, causal, off = case
    q, k, v = workloads.attention_inputs(BH, Lq, Lk, D, dt, seed=700 + Lq + Lk + D)
    scale = 1.0 / math.sqrt(D)
    ref, absref = oracle.attention(q, k, v, dt, scale, causal=causal, offset=off, with_abs=True)
    say(f"case attention {dt} {case}")
    o = run(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), dt, scale, causal, off)
    check(to_host_bits(o, dt), ref, absref, dt, f"{dt} {case}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_attention_peaked_and_flat_scores(dt):
    """Scores spread far (q, k scaled by 4: weights from 1 to below 2^-100,
    one key dominating many rows) and nearly equal (scale 1e-3)."""
    BH, Lq, Lk, D = 2, 150, 333, 128
    for qk_scale, scale in ((4.0, 1.0 / math.sqrt(D)), (1.0, 1e-3)):
        q, k, v = workloads.attention_inputs(BH, Lq, Lk, D, dt, seed=811, qk_scale=qk_scale)
        ref, absref = oracle.attention(q, k, v, dt, scale, causal=True, offset=50, with_abs=True)
        say(f"case attention {dt} qk_scale {qk_scale} scale {scale}")
        o = run(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), dt, scale, True, 50)
        check(to_host_bits(o, dt), ref, absref, dt, f"{dt} qk_scale {qk_scale}")


def test_attention_full_size_sampled_rows():
    """32 heads x 4096 queries x 4096 keys x 128, bf16, causal (the bench
    shape): every query of one head and sampled rows of all heads, the first
    and last query of each head included."""
    w = workloads.ATTENTION
    BH, Lq, Lk, D, dt = w["BH"], w["Lq"], w["Lk"], w["D"], w["dt"]
    say("case attention full size: generating")
    q, k, v = workloads.attention_inputs(BH, Lq, Lk, D, dt)
    o = run(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), dt, w["scale"], w["causal"], w["offset"])
    ob = to_host_bits(o, dt).reshape(BH * Lq, D)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(7 * Lq, 8 * Lq), rng.choice(BH * Lq, 2048, replace=False),
                                     np.arange(BH) * Lq, np.arange(BH) * Lq + Lq - 1]))
    say(f"case attention full size: oracle on {rows.size} rows")
    ref, absref = oracle.attention(q, k, v, dt, w["scale"], causal=True, offset=0, rows=rows, with_abs=True)
    check(ob[rows], ref, absref, dt, "full size")


def test_attention_deterministic_and_errors():
    BH, Lq, Lk, D, dt = 2, 200, 300, 128, "bf16"
    q, k, v = workloads.attention_inputs(BH, Lq, Lk, D, dt, seed=900)
    q_t, k_t, v_t = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    a = to_host_bits(run(q_t, k_t, v_t, dt, 0.1, True, 100), dt)
    b = to_host_bits(run(q_t, k_t, v_t, dt, 0.1, True, 100), dt)
    assert np.array_equal(a, b)
    o = torch.empty_like(q_t)
    s = torch.cuda.current_stream().cuda_stream
    P = q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), o.data_ptr()

    def call(BH=BH, Lq=Lq, Lk=Lk, D=D, dtc=nt.NT_BF16, scale=0.1, causal=1, off=0, ptrs=P):
        return nt.nt_attention_fwd(BH, Lq, Lk, D, dtc, scale, causal, off, *ptrs, s)

    assert call(dtc=nt.NT_F32) == 3                           # fp32 is not built
    assert call(D=96) == 2 and call(Lk=0) == 2 and call(off=-1) == 2 and call(causal=2) == 2
    assert call(scale=0.0) == 9 and call(scale=float("inf")) == 9
    assert call(ptrs=(P[0] + 2, P[1], P[2], P[3])) == 5       # 16-byte alignment
    assert call(ptrs=(P[0], P[1], P[2], P[0])) == 8           # o over q
    assert call(ptrs=(None, P[1], P[2], P[3])) == 1
    assert call(BH=0) == 0 and call(Lq=0) == 0
    torch.cuda.synchronize()


def test_attention_torch_wrapper():
    """nt.attention on [B, H, L, D] tensors: bitwise the C entry point's
    result, default scale 1/sqrt(D), causal offset passed through; argument
    mismatches raise."""
    B, H, Lq, Lk, D, dt = 2, 3, 70, 90, 64, "f16"
    q, k, v = workloads.attention_inputs(B * H, Lq, Lk, D, dt, seed=950)
    q_t, k_t, v_t = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    say("case attention torch wrapper")
    ref = to_host_bits(run(q_t, k_t, v_t, dt, 1.0 / math.sqrt(D), True, 20), dt)
    o = nt.attention(q_t.view(B, H, Lq, D), k_t.view(B, H, Lk, D), v_t.view(B, H, Lk, D), causal=True, offset=20)
    torch.cuda.synchronize()
    assert o.shape == (B, H, Lq, D)
    assert np.array_equal(to_host_bits(o.reshape(B * H, Lq, D), dt), ref)
    with pytest.raises(ValueError):
        nt.attention(q_t, k_t[:, :, :32].contiguous(), v_t)
    with pytest.raises(ValueError):
        nt.attention(q_t, k_t, v_t.float())
    with pytest.raises(ValueError):
        nt.attention(q_t.cpu(), k_t.cpu(), v_t.cpu())
