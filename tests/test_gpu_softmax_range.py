"""GPU parity of the softmax on rows whose logits spread over 90 to 150:
outputs run from the normal range down through the subnormals (fp32 and
bf16 share the exponent range: subnormal below 2^-126, nothing below 2^-149 /
2^-133) to exact zeros.  fp32 outputs meet the relative 1e-5 bar, or, below
2^-126, lie within one 2^-149 quantum of the correctly rounded value;
16-bit outputs within 1 ulp of it (subnormal ulps included).
Single pass, cooperative split, two-kernel split and the causal entry.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import check_output, empty_like_dev, to_dev, to_host_bits
import oracle
import workloads

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import torch  # noqa: E402

import row_wise_reductions_amd as nt  # noqa: E402

DT_CODE = {"f32": nt.NT_F32, "f16": nt.NT_F16, "bf16": nt.NT_BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def spread_rows(seed, M, N, dt, spread):
    """Row r: logits from 0 down to -spread (a ramp over the columns, shuffled
    per row, plus N(0, 1) noise), so every row reaches from its max through
    the subnormal range of the output."""
    rng = np.random.default_rng(seed)
    ramp = -spread * np.arange(N) / max(N - 1, 1)
    x = np.stack([rng.permutation(ramp) for _ in range(M)]) + rng.standard_normal((M, N))
    return workloads.encode(x, dt)


def run_softmax(x_t, dt, y=None):
    M, N = x_t.shape
    y = empty_like_dev((M, N), dt) if y is None else y
    wsb = nt.nt_softmax_workspace_bytes(M, N, DT_CODE[dt])
    ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device="cuda")
    rc = nt.nt_softmax_rows(M, N, DT_CODE[dt], x_t.data_ptr(), y.data_ptr(), ws.data_ptr(), wsb,
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0, nt.nt_status_string(rc)
    torch.cuda.synchronize()
    return y


def tiny_share(ref, dt):
    """Fraction of outputs below the smallest normal of the output type."""
    lim = 2.0 ** -126 if dt != "f16" else 2.0 ** -14
    return float(np.mean((ref > 0) & (ref < lim)))


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N,spread", [(781, 90.0), (4096, 120.0), (8192, 150.0), (16384, 110.0)])
def test_single_pass_wide_spread(dt, N, spread):
    M = 64
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, M, N, DT_CODE[dt], True)
    assert p["split"] == 0, p
    x = spread_rows(int(spread) * 7 + N, M, N, dt, spread)
    ref = oracle.softmax(x, dt)
    say(f"case wide spread single pass {dt} {M}x{N} spread {spread}: {tiny_share(ref, dt):.3f} below normal")
    assert tiny_share(ref, dt) > 0.01
    y = run_softmax(to_dev(x, dt), dt)
    check_output(to_host_bits(y, dt), ref, dt, f"single pass {dt} N={N} spread {spread}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,spread", [(262144, 120.0), (100003, 150.0)])
@pytest.mark.parametrize("form", ["one pass", "two kernels", "in place"])
def test_split_wide_spread(dt, N, spread, form, ntenv):
    M = 8
    x = spread_rows(int(spread) + N, M, N, dt, spread)
    ref = oracle.softmax(x, dt)
    if form == "two kernels":
        ntenv.setenv("NT_COOP", "0")
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, M, N, DT_CODE[dt], True)
    # (an in-place call switches to the two kernels when it is made; the plan cannot know)
    assert p["split"] == 1 and p["cooperative"] == (0 if form == "two kernels" else 1), p
    say(f"case wide spread split ({form}) {dt} {M}x{N} spread {spread}: {tiny_share(ref, dt):.3f} below normal")
    x_t = to_dev(x, dt)
    y = run_softmax(x_t, dt, y=x_t if form == "in place" else None)
    check_output(to_host_bits(y, dt), ref, dt, f"split {form} {dt} N={N} spread {spread}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [2048, 262144])
def test_causal_wide_spread(dt, N):
    """Causal entry, scale 0.5 on logits spread over 240 (so scale*x spreads
    over 120): square layout, 8 queries per head (the visible prefix is
    offset so rows reach far into the row)."""
    M, Q = 16, 8
    off = N - Q
    x = spread_rows(N + 5, M, N, dt, 240.0)
    ref = oracle.softmax_causal(x, dt, 0.5, Q, off)
    say(f"case wide spread causal {dt} {M}x{N}: {tiny_share(ref, dt):.3f} below normal")
    x_t = to_dev(x, dt)
    y = empty_like_dev((M, N), dt)
    wsb = nt.nt_softmax_workspace_bytes(M, N, DT_CODE[dt])
    ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device="cuda")
    rc = nt.nt_softmax_causal_rows(M, N, DT_CODE[dt], 0.5, Q, off, x_t.data_ptr(), y.data_ptr(), ws.data_ptr(),
                                   wsb, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    check_output(to_host_bits(y, dt), ref, dt, f"causal {dt} N={N}")
