"""GPU test of nt_softmax_rows_noalloc, the softmax entry point that
allocates nothing (its split-path records live in a device array inside the
library): through the C ABI, its output equals nt_softmax_rows' bit for bit
and meets the oracle's bar, on consecutive calls of shrinking size (the
array keeps the previous call's contents), on both split forms and on rows
that need no scratch; shapes needing more than the array are refused before
anything is enqueued; captured into a graph, every replay tags its records
afresh."""
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


def rows(seed, M, N, dt, scale=2.0):
    rng = np.random.default_rng(seed)
    return workloads.encode(rng.standard_normal((M, N)) * scale, dt)


def with_workspace(x_t, dt, y=None):
    M, N = x_t.shape
    y = empty_like_dev((M, N), dt) if y is None else y
    wsb = nt.nt_softmax_workspace_bytes(M, N, DT_CODE[dt])
    ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device="cuda")
    assert nt.nt_softmax_rows(M, N, DT_CODE[dt], x_t.data_ptr(), y.data_ptr(), ws.data_ptr(), wsb,
                              torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    return y


def noalloc(x_t, dt, y=None):
    M, N = x_t.shape
    y = empty_like_dev((M, N), dt) if y is None else y
    rc = nt.nt_softmax_rows_noalloc(M, N, DT_CODE[dt], x_t.data_ptr(), y.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0, nt.nt_status_string(rc)
    torch.cuda.synchronize()
    return y


# (dt, M, N): each sequence shrinks from call to call
SEQUENCES = [
    [("f32", 64, 262144), ("f32", 8, 100003)],          # cooperative split, then a smaller ragged one
    [("bf16", 48, 1 << 20), ("bf16", 3, 262147)],       # 16-bit split, misaligned-width tail
    [("f32", 4096, 65537), ("f32", 1024, 781)],         # large split, then a row that fits on chip
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["f32", "bf16", "split-then-resident"])
def test_noalloc_matches_workspace_entry(seq):
    for i, (dt, M, N) in enumerate(seq):
        need = nt.nt_softmax_workspace_bytes(M, N, DT_CODE[dt])
        assert need <= nt.NT_NOALLOC_SCRATCH_BYTES
        say(f"case noalloc call {i}: {dt} {M}x{N} (scratch {need} bytes)")
        x = rows(1000 * i + N, M, N, dt)
        x_t = to_dev(x, dt)
        a = to_host_bits(noalloc(x_t, dt), dt)
        b = to_host_bits(with_workspace(x_t, dt), dt)
        assert np.array_equal(a, b), f"call {i}: differs from nt_softmax_rows"
        check_output(a, oracle.softmax(x, dt), dt, f"noalloc call {i} {dt} {M}x{N}")


@pytest.mark.parametrize("form", ["two kernels", "in place"])
def test_noalloc_two_kernel_forms(form, ntenv):
    """The split's two-kernel form through the array: in place, and forced."""
    M, N, dt = 16, 262144, "f32"
    if form == "two kernels":
        ntenv.setenv("NT_COOP", "0")
    x = rows(77, M, N, dt)
    ref = to_host_bits(with_workspace(to_dev(x, dt), dt), dt)
    say(f"case noalloc {form} {dt} {M}x{N}")
    x_t = to_dev(x, dt)
    y = noalloc(x_t, dt, y=x_t if form == "in place" else None)
    assert np.array_equal(to_host_bits(y, dt), ref)


def test_noalloc_refuses_more_than_the_array():
    """A shape whose records exceed the array: NT_ERR_WORKSPACE, nothing
    enqueued (x == y, so the overlap checks pass and only the size decides)."""
    buf = torch.zeros(1 << 20, device="cuda")
    M, N = 8192, 262144                                   # 8192 x 16 chunks x 16 bytes = 2 MiB
    assert nt.nt_softmax_workspace_bytes(M, N, nt.NT_F32) > nt.NT_NOALLOC_SCRATCH_BYTES
    rc = nt.nt_softmax_rows_noalloc(M, N, nt.NT_F32, buf.data_ptr(), buf.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 6, nt.nt_status_string(rc)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(buf)) == 0


def test_noalloc_under_graph_capture():
    """The entry point captured into a graph (the callers it is for) and
    replayed with new inputs copied in between replays: the cooperative split
    runs from the array with its tag advanced per replay, and every replay is
    bitwise nt_softmax_rows' result on the same input and meets the oracle."""
    M, N, dt = 64, 262144, "f32"
    assert nt.nt_plan_launch(nt.NT_OP_SOFTMAX, M, N, DT_CODE[dt], True)["cooperative"] == 2
    xs = [rows(300 + i, M, N, dt, scale=1.0 + i) for i in range(3)]
    x_t = to_dev(xs[0], dt)
    y_t = empty_like_dev((M, N), dt)
    s = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):
        assert nt.nt_softmax_rows_noalloc(M, N, DT_CODE[dt], x_t.data_ptr(), y_t.data_ptr(), side.cuda_stream) == 0
    s.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = nt.nt_softmax_rows_noalloc(M, N, DT_CODE[dt], x_t.data_ptr(), y_t.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, nt.nt_status_string(rc)
    for i in (1, 2, 0, 1):
        say(f"case noalloc graph replay inputs {i}")
        x_t.copy_(to_dev(xs[i], dt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host_bits(y_t, dt)
        ref = to_host_bits(with_workspace(to_dev(xs[i], dt), dt), dt)
        assert np.array_equal(got, ref), f"replay {i} differs from nt_softmax_rows"
        check_output(got, oracle.softmax(xs[i], dt), dt, f"noalloc graph replay {i}")
