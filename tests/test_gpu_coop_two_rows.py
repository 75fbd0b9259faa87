"""The cooperative split softmax with two rows per workgroup (softmax_coop2,
NT_COOP=rows2): bitwise equal to the one-row cooperative kernel, to the same
kernel with every record that has not arrived at the first look recomputed
(NT_COOP_SPIN=0), and to the two-kernel split, and within the bar of the
oracle; odd and even row counts (the last workgroup of an odd count takes one
row), misaligned rows, the causal entry, and a workspace holding another
call's records.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import check_output, empty_like_dev, oracle_for, to_dev, to_host_bits
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


def rand_bits(seed, M, N, dt, scale=1.0):
    rng = np.random.default_rng(seed)
    return workloads.encode(rng.standard_normal((M, N)) * scale, dt)


def run(x_t, dt, ws, off=0, causal=None):
    M, N = x_t.shape
    y = empty_like_dev((M, N), dt, off)
    s = torch.cuda.current_stream().cuda_stream
    if causal is None:
        rc = nt.nt_softmax_rows(M, N, DT_CODE[dt], x_t.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), s)
    else:
        scale, Q, qoff = causal
        rc = nt.nt_softmax_causal_rows(M, N, DT_CODE[dt], scale, Q, qoff, x_t.data_ptr(), y.data_ptr(),
                                       ws.data_ptr(), ws.numel(), s)
    assert rc == 0, nt.nt_status_string(rc)
    torch.cuda.synchronize()
    return to_host_bits(y, dt)


def forms(x_t, dt, ws, ntenv, off=0, causal=None):
    """Outputs of the two-row, one-row, two-row-recomputing and two-kernel forms."""
    M, N = x_t.shape
    out = {}
    for name, env in (("rows2", {"NT_COOP": "rows2"}), ("rows1", {"NT_COOP": "rows1"}),
                      ("rows2 recompute", {"NT_COOP": "rows2", "NT_COOP_SPIN": "0"}), ("two kernels", {"NT_COOP": "0"})):
        for k, v in env.items():
            ntenv.setenv(k, v)
        p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX_CAUSAL if causal else nt.NT_OP_SOFTMAX, M, N, DT_CODE[dt], off == 0)
        want = {"rows2": 2 if M >= 2 else 1, "rows1": 1, "rows2 recompute": 2 if M >= 2 else 1, "two kernels": 0}[name]
        assert p["split"] == 1 and p["cooperative"] == want, (name, p)
        if want == 2:
            assert p["rows_per_block"] == 2 and p["grid"] == (M + 1) // 2 * p["row_chunks"], p
        out[name] = run(x_t, dt, ws, off, causal)
        for k in env:
            ntenv.delenv(k)
    return out


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,N", [(1, 262144), (2, 65536), (3, 100003), (8, 262144), (17, 131075), (64, 40000)])
def test_two_rows_bitwise(dt, M, N, ntenv):
    x = rand_bits(M * 7 + N, M, N, dt, scale=2.0)
    x[M // 2, : N // 3] = workloads.NEG_INF_BITS[dt] if dt != "f32" else -np.inf    # a masked leading third
    ref = oracle.softmax(x, dt)
    code = DT_CODE[dt]
    ws = torch.empty(nt.nt_softmax_workspace_bytes(M, N, code), dtype=torch.uint8, device="cuda")
    for off in (0, 1):
        say(f"case coop two rows {dt} {M}x{N} off={off}")
        out = forms(to_dev(x, dt, off), dt, ws, ntenv, off)
        check_output(out["rows2"], ref, dt, f"rows2 {dt} {M}x{N} off={off}")
        for name in ("rows1", "rows2 recompute", "two kernels"):
            assert np.array_equal(out["rows2"], out[name]), f"rows2 and {name} differ ({dt} {M}x{N} off={off})"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_two_rows_causal(dt, ntenv):
    """The causal entry: 8 queries per head over 65536 keys (offset puts the
    visible prefixes deep in the row), scale 0.7; rows 0..M-1 pair row g with
    row g + M/2, whose prefixes differ."""
    M, N, Q = 12, 65536, 8
    qoff = N - 3 * Q
    x = rand_bits(N + 11, M, N, dt, scale=2.0)
    ref = oracle.softmax_causal(x, dt, 0.7, Q, qoff)
    code = DT_CODE[dt]
    ws = torch.empty(nt.nt_softmax_workspace_bytes(M, N, code), dtype=torch.uint8, device="cuda")
    say(f"case coop two rows causal {dt}")
    out = forms(to_dev(x, dt), dt, ws, ntenv, 0, causal=(0.7, Q, qoff))
    check_output(out["rows2"], ref, dt, f"rows2 causal {dt}")
    for name in ("rows1", "rows2 recompute", "two kernels"):
        assert np.array_equal(out["rows2"], out[name]), f"causal rows2 and {name} differ ({dt})"


def test_two_rows_vocab_workload_and_stale_workspace(ntenv):
    """The 64 x 262144 fp32 vocab workload through the two-row form, twice
    on one workspace with different inputs in between (each call's records
    carry its own tag), every row against the oracle."""
    w = workloads.BY_NAME["vocab_softmax_f32"]
    x = w.make()["x"]
    other = rand_bits(5, w.M, w.N, "f32", scale=4.0)
    ws = torch.empty(nt.nt_softmax_workspace_bytes(w.M, w.N, nt.NT_F32), dtype=torch.uint8, device="cuda")
    ntenv.setenv("NT_COOP", "rows2")
    assert nt.nt_plan_launch(0, w.M, w.N, nt.NT_F32, True)["cooperative"] == 2
    ref = oracle.softmax(x, "f32")
    for i, inp in enumerate((x, other, x)):
        say(f"case coop two rows vocab call {i}")
        y = run(to_dev(inp, "f32"), "f32", ws)
        if i != 1:
            check_output(y, ref, "f32", f"vocab rows2 call {i}")
