"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle on
identical seeded inputs.  fp32 outputs: max relative error <= 1e-5; fp16 and
bf16 outputs: <= 1 ulp of the output type from the oracle's float64 result
rounded once (round to nearest even); LayerNorm mean/rstd: relative 1e-5.
"""
from __future__ import annotations

import json
import os
import sys
import zlib

import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import (check_output, check_stats, empty_like_dev, oracle_for, row_blocks, tdt, to_dev,
                      to_host_bits)
import oracle
import workloads

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import torch  # noqa: E402

import row_wise_reductions_amd as nt  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DT_CODE = {"f32": nt.NT_F32, "f16": nt.NT_F16, "bf16": nt.NT_BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_bits(seed, M, N, dt, scale=1.0, loc=0.0):
    rng = np.random.default_rng(seed)
    return workloads.encode(rng.standard_normal((M, N)) * scale + loc, dt)


def run_op(op, x_t, dt, eps=0.0, p0=None, p1=None, y_t=None):
    """Launch through the C ABI on the current stream and wait."""
    M, N = x_t.shape
    code = DT_CODE[dt]
    y = y_t if y_t is not None else empty_like_dev((M, N), dt)
    s = torch.cuda.current_stream().cuda_stream
    mean = rstd = None
    if op == "softmax":
        wsb = nt.nt_softmax_workspace_bytes(M, N, code)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        rc = nt.nt_softmax_rows(M, N, code, x_t.data_ptr(), y.data_ptr(), ws.data_ptr(), wsb, s)
    elif op == "layernorm":
        mean = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        rstd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        rc = nt.nt_layernorm_rows(M, N, code, eps, x_t.data_ptr(),
                                  None if p0 is None else p0.data_ptr(),
                                  None if p1 is None else p1.data_ptr(),
                                  y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), s)
    else:
        rc = nt.nt_rmsnorm_rows(M, N, code, eps, x_t.data_ptr(),
                                None if p0 is None else p0.data_ptr(), y.data_ptr(), s)
    assert rc == 0, f"{op}: status {rc} ({nt.nt_status_string(rc)})"
    torch.cuda.synchronize()
    return y, mean, rstd


def parity_case(op, x_bits, dt, eps=0.0, p0=None, p1=None, x_off=0, y_off=0, what=""):
    M, N = x_bits.shape
    say(f"case {what} op={op} dt={dt} M={M} N={N} x_off={x_off} y_off={y_off}")
    x_t = to_dev(x_bits, dt, x_off)
    p0_t = None if p0 is None else to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    y_t = empty_like_dev((M, N), dt, y_off)
    y, mean, rstd = run_op(op, x_t, dt, eps, p0_t, p1_t, y_t)
    ref, rmean, rrstd = oracle_for(op, x_bits, dt, eps, p0, p1)
    check_output(to_host_bits(y, dt), ref, dt, what)
    if op == "layernorm":
        check_stats(mean.cpu().numpy(), rmean, what + " mean")
        check_stats(rstd.cpu().numpy(), rrstd, what + " rstd")


# ----------------------------------------------------------------------------
# the five workloads at full size, every row
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_workload_full_size(name):
    w = workloads.BY_NAME[name]
    say(f"workload {name}: generating {w.M}x{w.N} {w.dt}")
    data = w.make()
    x = data["x"]
    p0 = data.get("gamma", data.get("weight"))
    p1 = data.get("beta")
    x_t = to_dev(x, w.dt)
    p0_t = None if p0 is None else to_dev(p0, w.dt)
    p1_t = None if p1 is None else to_dev(p1, w.dt)
    say(f"workload {name}: launching")
    y, mean, rstd = run_op(w.op, x_t, w.dt, w.eps, p0_t, p1_t)
    yb_all = to_host_bits(y, w.dt)
    mean_h = None if mean is None else mean.cpu().numpy()
    rstd_h = None if rstd is None else rstd.cpu().numpy()
    del y, x_t
    # every row, against the oracle, in blocks of rows
    Q = w.extra.get("queries", 1) if w.extra else 1
    for r0, r1 in row_blocks(w.M, w.N, align=Q):
        say(f"workload {name}: rows {r0}..{r1 - 1}")
        ref, rmean, rrstd = oracle_for(w.op, np.ascontiguousarray(x[r0:r1]), w.dt, w.eps, p0, p1)
        yb = yb_all[r0:r1]
        check_output(yb, ref, w.dt, f"{name} rows {r0}..{r1 - 1}")
        del ref
        if w.op == "layernorm":
            check_stats(mean_h[r0:r1], rmean, name + " mean")
            check_stats(rstd_h[r0:r1], rrstd, name + " rstd")
        if name == "causal_softmax_bf16":
            # row with query q has exactly q+1 non-zero outputs; masked entries are exact 0
            q = np.arange(r0, r1) % w.extra["queries"]
            nz = (yb & 0x7FFF) != 0
            assert np.array_equal(nz.sum(axis=1), q + 1)
    if name == "vocab_softmax_f32":
        # the 8 spikes of a row are bit-identical and carry almost all the mass
        yv = yb_all.view(np.float32)
        for r in range(w.M):
            s = yv[r, data["spikes"][r]]
            assert np.all(s == s[0]) and abs(float(s[0]) - 0.125) < 1e-6


# ----------------------------------------------------------------------------
# shape sweep: ragged tails, every path, aligned and misaligned rows
# ----------------------------------------------------------------------------

SWEEP_N = [1, 2, 3, 7, 8, 63, 64, 65, 255, 256, 257, 781, 1023, 1024, 1025, 1500, 4095,
           4097, 8192, 16384, 65536, 65537, 262144, 262147]


def _sweep_M(N):
    if N <= 4097:
        return [1, 3, 1823]
    if N <= 16384:
        return [1, 37]
    return [1, 5]


SWEEP = [(op, dt, N, M) for op in ("softmax", "layernorm", "rmsnorm") for dt in ("f32", "f16", "bf16")
         for N in SWEEP_N for M in _sweep_M(N)]


@pytest.mark.parametrize("op,dt,N,M", SWEEP)
def test_sweep(op, dt, N, M):
    seed = zlib.crc32(f"{op}/{dt}/{N}/{M}".encode())
    loc = 2.0 if op == "layernorm" else 0.0
    x = rand_bits(seed, M, N, dt, scale=2.0, loc=loc)
    p0 = p1 = None
    eps = 1e-5
    if op != "softmax":
        p0 = rand_bits(seed + 1, 1, N, dt, scale=0.3, loc=1.0)[0]
        if op == "layernorm":
            p1 = rand_bits(seed + 2, 1, N, dt, scale=0.3)[0]
    parity_case(op, x, dt, eps, p0, p1, what=f"sweep {op} {dt} {M}x{N}")
    # misaligned rows: x and y one element past a 16-byte boundary (same phase)
    if N >= 2 and M <= 64:
        parity_case(op, x, dt, eps, p0, p1, x_off=1, y_off=1, what=f"sweep-misaligned {op} {dt} {M}x{N}")


@pytest.mark.parametrize("op", ["softmax", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_phase_mismatch_and_no_params(op, dt):
    """x and y at different 16-byte phases; parameter vectors absent."""
    x = rand_bits(77, 19, 1000, dt, scale=1.5)
    parity_case(op, x, dt, 1e-5, x_off=1, y_off=2, what=f"phase {op} {dt}")
    parity_case(op, x, dt, 1e-5, x_off=3, y_off=0, what=f"phase {op} {dt}")


def test_correctness_shapes_from_pages():
    """The irregular shapes of the pages' correctness template."""
    with open(os.path.join(GOLDEN, "correctness_shapes.json")) as f:
        shapes = json.load(f)["shapes"]
    for M, N in shapes:
        for op in ("softmax", "layernorm", "rmsnorm"):
            x = rand_bits(0, M, N, "f32")
            parity_case(op, x, "f32", 1e-6, what=f"pages-shape {op} {M}x{N}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [4096, 65536, 100003])
def test_split_path_forced(dt, N, ntenv):
    """The split online path on rows that would fit on chip, and odd widths."""
    ntenv.setenv("NT_FORCE_PATH", "split")
    x = rand_bits(N, 7, N, dt, scale=3.0)
    x[2, :] = -np.inf if dt == "f32" else workloads.NEG_INF_BITS[dt]
    x[2, N // 3] = x[3, 0]                       # row 2: one finite entry
    x[4, : N // 2] = x[2, 0]                     # row 4: masked first half
    for off in (0, 1):
        parity_case("softmax", x, dt, x_off=off, y_off=off, what=f"split {dt} N={N} off={off}")


def softmax_with_ws(x_t, dt, ws, y_t=None):
    """nt_softmax_rows with a caller-provided workspace tensor (uint8)."""
    M, N = x_t.shape
    y = y_t if y_t is not None else torch.empty_like(x_t)
    rc = nt.nt_softmax_rows(M, N, DT_CODE[dt], x_t.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(),
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0, nt.nt_status_string(rc)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [65536, 100003, 262144, 2097152])
def test_cooperative_split_bitwise(dt, N, ntenv):
    """The one-kernel cooperative split (x read once), the same kernel with
    every record that has not arrived at the first look recomputed by the
    waiting workgroup (NT_COOP_SPIN=0), and the two-kernel split give
    bitwise identical outputs, which match the oracle; up to the largest
    cooperative width (128 chunks per row)."""
    M = 9
    code = DT_CODE[dt]
    x = rand_bits(N + 7, M, N, dt, scale=2.0)
    rng = np.random.default_rng(N)
    spike = workloads.encode(np.array([30.0]), dt)[0]
    for r in range(M):
        x[r, rng.choice(N, 8, replace=False)] = spike
    x[3, : N // 2] = -np.inf if dt == "f32" else workloads.NEG_INF_BITS[dt]   # masked first half
    ntenv.setenv("NT_FORCE_PATH", "split")
    ref, _, _ = oracle_for("softmax", x, dt)
    for off in (0, 1):
        al = off == 0 and (N * (4 if dt == "f32" else 2)) % 16 == 0
        plan = nt.nt_plan_launch(0, M, N, code, al)
        # a misaligned row of 2^21 elements touches a 129th chunk: two kernels
        # (1152 fp32 (row, chunk) pairs take the two-rows-per-workgroup form)
        assert plan["split"] == 1 and (plan["cooperative"] != 0) == (plan["row_chunks"] <= 128), plan
        say(f"case coop {dt} N={N} off={off} P={plan['row_chunks']}")
        x_t = to_dev(x, dt, off)
        ws = torch.empty(nt.nt_softmax_workspace_bytes(M, N, code), dtype=torch.uint8, device="cuda")
        y_coop = to_host_bits(softmax_with_ws(x_t, dt, ws, empty_like_dev((M, N), dt, off)), dt)
        check_output(y_coop, ref, dt, f"coop {dt} N={N} off={off}")
        ntenv.setenv("NT_COOP_SPIN", "0")
        y_rec = to_host_bits(softmax_with_ws(x_t, dt, ws, empty_like_dev((M, N), dt, off)), dt)
        ntenv.delenv("NT_COOP_SPIN")
        ntenv.setenv("NT_COOP", "0")
        y_two = to_host_bits(softmax_with_ws(x_t, dt, ws, empty_like_dev((M, N), dt, off)), dt)
        ntenv.delenv("NT_COOP")
        assert np.array_equal(y_coop, y_rec), "recomputed records differ from published ones"
        assert np.array_equal(y_coop, y_two), "cooperative and two-kernel split differ"


def test_cooperative_split_ignores_stale_and_garbage_workspace():
    """Records left in the workspace by an earlier call, or arbitrary bytes,
    are never taken for this call's (each call tags its records)."""
    M, N = 16, 262144
    a = rand_bits(1, M, N, "f32", scale=2.0)
    b = rand_bits(2, M, N, "f32", scale=5.0, loc=-3.0)
    assert nt.nt_plan_launch(0, M, N, nt.NT_F32, True)["cooperative"] == 1
    ws = torch.empty(nt.nt_softmax_workspace_bytes(M, N, nt.NT_F32), dtype=torch.uint8, device="cuda")
    for i, x in enumerate((a, b, a)):                 # the same workspace, one call after another
        say(f"case coop stale-workspace call {i}")
        y = softmax_with_ws(to_dev(x, "f32"), "f32", ws)
        check_output(to_host_bits(y, "f32"), oracle_for("softmax", x, "f32")[0], "f32", f"stale call {i}")
    g = torch.Generator(device="cpu").manual_seed(5)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=g))
    say("case coop garbage workspace")
    y = softmax_with_ws(to_dev(b, "f32"), "f32", ws)
    check_output(to_host_bits(y, "f32"), oracle_for("softmax", b, "f32")[0], "f32", "garbage workspace")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_in_place(dt):
    """In place on the split path (the two-kernel form reads x completely
    before any output is written)."""
    M, N = 4, 262144 if dt == "f32" else 524288
    x = rand_bits(3, M, N, dt, scale=2.0)
    ref, _, _ = oracle_for("softmax", x, dt)
    x_t = to_dev(x, dt)
    say(f"case split in place {dt}")
    y, _, _ = run_op("softmax", x_t, dt, y_t=x_t)
    check_output(to_host_bits(x_t, dt), ref, dt, f"split in place {dt}")


@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1000, 4096, 100003])
def test_looped_path_forced(op, dt, N, ntenv):
    """The looped one-workgroup-per-row norm kernel on rows that would fit on
    chip, and on odd widths, aligned and misaligned."""
    ntenv.setenv("NT_FORCE_PATH", "looped")
    x = rand_bits(N + 1, 6, N, dt, scale=2.0, loc=3.0)
    p0 = rand_bits(N + 2, 1, N, dt, scale=0.3, loc=1.0)[0]
    p1 = rand_bits(N + 3, 1, N, dt, scale=0.3)[0] if op == "layernorm" else None
    for off in (0, 1):
        parity_case(op, x, dt, 1e-5, p0, p1, x_off=off, y_off=off, what=f"looped {op} {dt} N={N} off={off}")


@pytest.mark.parametrize("op,dt", [("layernorm", "f32"), ("layernorm", "f16"), ("layernorm", "bf16"),
                                   ("rmsnorm", "f32"), ("rmsnorm", "f16"), ("rmsnorm", "bf16")])
@pytest.mark.parametrize("N,M,grid", [(4096, 37, 0), (8192, 300, 7), (4096, 5, 2), (8192, 64, 3), (4096, 3000, 0),
                                    (16384, 3000, 2048)])
def test_persistent_norms(op, dt, N, M, grid, ntenv):
    """Persistent norm kernel (parameters held across rows, next row prefetched):
    parity with the oracle and bitwise equality with the one-row-per-group
    kernel, including grids much smaller than the row count, the planned
    grid at a few rows per workgroup, and a forced grid of more workgroups
    than fit on the device at once.  (fp32 RMSNorm plans it only on
    part-filled rows of 8 waves x 8 chunks: 10240 there.)"""
    code = DT_CODE[dt]
    opc = {"layernorm": 1, "rmsnorm": 2}[op]
    # a width near N whose plan is the persistent kernel
    N = next(n for n in (N, 2 * N, N // 2, 4 * N, 10240) if nt.nt_plan_launch(opc, M, n, code, True)["persistent"])
    x = rand_bits(N + M, M, N, dt, scale=2.0, loc=1.5)
    p0 = rand_bits(N + 1, 1, N, dt, scale=0.3, loc=1.0)[0]
    p1 = rand_bits(N + 2, 1, N, dt, scale=0.3)[0] if op == "layernorm" else None
    if grid:
        ntenv.setenv("NT_PERSIST_GRID", str(grid))
    x_t, p0_t = to_dev(x, dt), to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    say(f"case persistent {op} {dt} {M}x{N} grid={grid}")
    y1, m1, r1 = run_op(op, x_t, dt, 1e-5, p0_t, p1_t)
    ref, rmean, rrstd = oracle_for(op, x, dt, 1e-5, p0, p1)
    check_output(to_host_bits(y1, dt), ref, dt, f"persistent {op} {dt}")
    if op == "layernorm":
        check_stats(m1.cpu().numpy(), rmean, "persistent mean")
        check_stats(r1.cpu().numpy(), rrstd, "persistent rstd")
    ntenv.setenv("NT_PERSISTENT", "0")
    y2, m2, r2 = run_op(op, x_t, dt, 1e-5, p0_t, p1_t)
    assert np.array_equal(to_host_bits(y1, dt), to_host_bits(y2, dt))
    if op == "layernorm":
        assert torch.equal(m1, m2) and torch.equal(r1, r2)


@pytest.mark.parametrize("fused,M,N", [(False, 16384, 4096), (True, 13107, 5120)])
def test_persistent_layernorm_bitwise_at_size(fused, M, N, ntenv):
    """fp32 LayerNorm over many rows: the persistent and one-row kernels
    evaluate the same expression per element, so y, mean and rstd agree
    bitwise on every row (a differently rounded epilogue shows up at this
    size as a handful of fp32 outputs one ulp apart)."""
    gen = torch.Generator(device="cuda").manual_seed(M + N)
    x = torch.randn(M, N, device="cuda", generator=gen) * 2.0 + 1.5
    r = torch.randn(M, N, device="cuda", generator=gen) if fused else None
    g = torch.randn(N, device="cuda", generator=gen) * 0.3 + 1.0
    b = torch.randn(N, device="cuda", generator=gen) * 0.3
    s = torch.cuda.current_stream().cuda_stream
    opc = nt.NT_OP_ADD_LAYERNORM if fused else nt.NT_OP_LAYERNORM
    assert nt.nt_plan_launch(opc, M, N, nt.NT_F32, True)["persistent"] == 1
    outs = []
    for mode in (None, "0"):
        if mode:
            ntenv.setenv("NT_PERSISTENT", mode)
        assert nt.nt_plan_launch(opc, M, N, nt.NT_F32, True)["persistent"] == (0 if mode else 1)
        say(f"case LN f32 bitwise fused={fused} {M}x{N} persistent={'off' if mode else 'on'}")
        y, mean, rstd = torch.empty_like(x), torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
        if fused:
            h = torch.empty_like(x)
            rc = nt.nt_add_layernorm_rows(M, N, nt.NT_F32, 1e-5, x.data_ptr(), r.data_ptr(), g.data_ptr(),
                                          b.data_ptr(), h.data_ptr(), y.data_ptr(), mean.data_ptr(),
                                          rstd.data_ptr(), s)
        else:
            rc = nt.nt_layernorm_rows(M, N, nt.NT_F32, 1e-5, x.data_ptr(), g.data_ptr(), b.data_ptr(), y.data_ptr(),
                                      mean.data_ptr(), rstd.data_ptr(), s)
        assert rc == 0
        torch.cuda.synchronize()
        outs.append((y, mean, rstd))
    for a_, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a_.view(torch.int32), b_.view(torch.int32)), \
            f"{int((a_.view(torch.int32) != b_.view(torch.int32)).sum())} words differ"


def test_grid_cap_striding():
    """More rows than one launch may hold (grid x threads < 2^31): the
    kernels stride over the rows beyond the capped grid.  N = 1, so 4 rows
    per 256-thread workgroup and 2^25 + 7 rows exceed 2^23 workgroups."""
    M, N = (1 << 25) + 7, 1
    for op in (0, 1, 2):
        p = nt.nt_plan_launch(op, M, N, nt.NT_F32, True)
        assert p["grid"] * p["rows_per_block"] < M, p
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((M, N)) * 2.0).astype(np.float32)
    w = np.array([0.75], dtype=np.float32)
    b = np.array([-0.25], dtype=np.float32)
    x_t = to_dev(x, "f32")
    w_t, b_t = to_dev(w, "f32"), to_dev(b, "f32")
    tail = np.arange(M - 4096, M)                    # the rows only striding reaches, and more
    for op in ("softmax", "rmsnorm", "layernorm"):
        say(f"case grid cap {op} M={M}")
        y, mean, rstd = run_op(op, x_t, "f32", 1e-5, w_t if op != "softmax" else None, b_t if op == "layernorm" else None)
        yb = to_host_bits(y, "f32")
        ref, rmean, rrstd = oracle_for(op, np.ascontiguousarray(x[tail]), "f32", 1e-5,
                                       w if op != "softmax" else None, b if op == "layernorm" else None)
        check_output(yb[tail], ref, "f32", f"grid cap {op}")
        head, href = yb[:4096], oracle_for(op, np.ascontiguousarray(x[:4096]), "f32", 1e-5,
                                           w if op != "softmax" else None, b if op == "layernorm" else None)[0]
        check_output(head, href, "f32", f"grid cap {op} head")
        if op == "layernorm":
            check_stats(mean.cpu().numpy()[tail], rmean, "grid cap mean")


@pytest.mark.parametrize("op,dt,M,N", [("softmax", "f32", 3, (1 << 28) + 3), ("rmsnorm", "bf16", 5, (1 << 28) + 5)])
def test_rows_past_2gib_offsets(op, dt, M, N):
    """Rows of 512 MiB to 1 GiB, so the last row starts beyond 2^31 bytes
    (64-bit offsets throughout): the split softmax (two-kernel form, ragged
    misaligned rows) and the looped RMSNorm, against the oracle on every
    element, compared in column blocks.  Inputs drawn in float32 (rounded
    once to bf16) to keep the host side small."""
    rng = np.random.default_rng(N)
    x32 = rng.standard_normal((M, N), dtype=np.float32) * np.float32(2.0)
    x = x32 if dt == "f32" else workloads.to_bf16_bits(x32)
    del x32
    w = workloads.to_bf16_bits(np.float32(1.0) + np.float32(0.3) * rng.standard_normal(N, dtype=np.float32)) \
        if op == "rmsnorm" else None
    assert (M - 1) * N * (4 if dt == "f32" else 2) > (1 << 31)
    p = nt.nt_plan_launch({"softmax": 0, "rmsnorm": 2}[op], M, N, DT_CODE[dt], True)
    assert p["split"] in (1, 2) and (p["split"] == 2 or p["cooperative"] == 0), p
    say(f"case 2GiB-offset {op} {dt} M={M} N={N}")
    x_t = to_dev(x, dt)
    w_t = None if w is None else to_dev(w, dt)
    y, _, _ = run_op(op, x_t, dt, 1e-6, w_t)
    del x_t
    yb = to_host_bits(y, dt)
    del y
    ref = oracle.softmax(x, dt) if op == "softmax" else oracle.rmsnorm(x, dt, 1e-6, weight=w)
    blk = 1 << 25
    for r in range(M):
        for j0 in range(0, N, blk):
            check_output(yb[r, j0:j0 + blk], ref[r, j0:j0 + blk], dt, f"2GiB-offset {op} row {r} col {j0}")


# ----------------------------------------------------------------------------
# semantics: special rows, in place, determinism, streams, no-op, errors
# ----------------------------------------------------------------------------

def test_special_rows():
    x = np.full((4, 300), -np.inf, dtype=np.float32)
    x[1, 7] = 2.0                                 # one finite entry -> one-hot
    x[2, :] = 0.5                                 # uniform
    x[3, :150] = 1.0
    y, _, _ = run_op("softmax", to_dev(x, "f32"), "f32")
    yh = y.cpu().numpy()
    assert np.all(np.isnan(yh[0]))               # all -inf row: NaN, as the formula
    assert yh[1, 7] == 1.0 and np.count_nonzero(yh[1]) == 1
    assert np.max(np.abs(yh[2] - 1.0 / 300)) < 1e-5 / 300
    # LayerNorm of a constant row: y = beta, rstd = 1/sqrt(eps)
    c = np.full((2, 33), 3.0, dtype=np.float32)
    beta = np.linspace(-1, 1, 33).astype(np.float32)
    y, mean, rstd = run_op("layernorm", to_dev(c, "f32"), "f32", 1e-5, None, to_dev(beta, "f32"))
    assert np.array_equal(y.cpu().numpy()[0], beta)
    assert abs(rstd.cpu().numpy()[0] - 1 / np.sqrt(np.float64(np.float32(1e-5)))) < 1e-3


@pytest.mark.parametrize("op", ["softmax", "layernorm", "rmsnorm"])
def test_in_place(op):
    x = rand_bits(5, 64, 4096, "bf16", scale=2.0)
    ref, _, _ = oracle_for(op, x, "bf16", 1e-5)
    x_t = to_dev(x, "bf16")
    y, _, _ = run_op(op, x_t, "bf16", 1e-5, y_t=x_t)
    check_output(to_host_bits(x_t, "bf16"), ref, "bf16", f"in-place {op}")


@pytest.mark.parametrize("N", [781, 8192, 262144])
def test_bitwise_repeatable(N):
    x_t = to_dev(rand_bits(9, 16, N, "f32", scale=3.0), "f32")
    a, _, _ = run_op("softmax", x_t, "f32")
    b, _, _ = run_op("softmax", x_t, "f32")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_graph_capture_and_replay():
    """Calls captured into a HIP graph (torch.cuda.graph) and replayed with
    new inputs copied in (eagerly) between replays: every replay matches the
    oracle and is bitwise the eager result on the same input.  The
    cooperative split softmax is captured with its record tag read from the
    word after the records, advanced on the device before each replay's
    launch (one advance per replay), so no replay takes an earlier one's
    records."""
    M, N = 8, 262144
    xs = [rand_bits(40 + i, M, N, "f32", scale=2.0 + i) for i in range(3)]
    rs = [rand_bits(50 + i, 16, 8192, "bf16") for i in range(3)]
    w = rand_bits(60, 1, 8192, "bf16", scale=0.3, loc=1.0)[0]
    x_t, r_t, w_t = to_dev(xs[0], "f32"), to_dev(rs[0], "bf16"), to_dev(w, "bf16")
    y_t, ry_t = torch.empty_like(x_t), torch.empty_like(r_t)
    wsb = nt.nt_softmax_workspace_bytes(M, N, nt.NT_F32)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    assert nt.nt_plan_launch(0, M, N, nt.NT_F32, True)["cooperative"] == 1
    assert nt.nt_plan_launch(2, 16, 8192, nt.NT_BF16, True)["persistent"] == 1
    # and the two-rows-per-workgroup form on 64 vocabulary-wide rows
    M2 = 64
    x2s = [rand_bits(45 + i, M2, N, "f32", scale=1.5 + i) for i in range(3)]
    x2_t = to_dev(x2s[0], "f32")
    y2_t = torch.empty_like(x2_t)
    wsb2 = nt.nt_softmax_workspace_bytes(M2, N, nt.NT_F32)
    ws2 = torch.empty(wsb2, dtype=torch.uint8, device="cuda")
    assert nt.nt_plan_launch(0, M2, N, nt.NT_F32, True)["cooperative"] == 2

    def calls(stream):
        assert nt.nt_softmax_rows(M, N, nt.NT_F32, x_t.data_ptr(), y_t.data_ptr(), ws.data_ptr(), wsb,
                                  stream) == 0
        assert nt.nt_rmsnorm_rows(16, 8192, nt.NT_BF16, 1e-6, r_t.data_ptr(), w_t.data_ptr(),
                                  ry_t.data_ptr(), stream) == 0
        assert nt.nt_softmax_rows(M2, N, nt.NT_F32, x2_t.data_ptr(), y2_t.data_ptr(), ws2.data_ptr(), wsb2,
                                  stream) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = to_host_bits(y_t, "f32")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(torch.cuda.current_stream().cuda_stream)
    # the tag word: in the 16 bytes after the plan's records
    pw = nt.nt_plan_launch(0, M, N, nt.NT_F32, True)["workspace_bytes"]
    pw2 = nt.nt_plan_launch(0, M2, N, nt.NT_F32, True)["workspace_bytes"]
    tag_word = ws[pw - 16:pw - 12].view(torch.int32)
    tag_word2 = ws2[pw2 - 16:pw2 - 12].view(torch.int32)
    torch.cuda.synchronize()
    tag0, tag0_2 = int(tag_word.item()), int(tag_word2.item())
    for n, i in enumerate((1, 0, 2, 2, 1)):
        say(f"case graph replay inputs {i}")
        x_t.copy_(to_dev(xs[i], "f32"))
        r_t.copy_(to_dev(rs[i], "bf16"))
        x2_t.copy_(to_dev(x2s[i], "f32"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (int(tag_word.item()) - tag0) & 0xFFFFFFFF == n + 1, "one tag advance per replay"
        assert (int(tag_word2.item()) - tag0_2) & 0xFFFFFFFF == n + 1, "one tag advance per replay"
        check_output(to_host_bits(y2_t, "f32"), oracle_for("softmax", x2s[i], "f32")[0], "f32",
                     f"graph two-row softmax {i}")
        check_output(to_host_bits(y_t, "f32"), oracle_for("softmax", xs[i], "f32")[0], "f32", f"graph softmax {i}")
        if i == 0:
            assert np.array_equal(to_host_bits(y_t, "f32"), eager)
        check_output(to_host_bits(ry_t, "bf16"), oracle_for("rmsnorm", rs[i], "bf16", 1e-6, w)[0], "bf16",
                     f"graph rmsnorm {i}")


def test_cooperative_split_on_concurrent_streams():
    """Cooperative split softmax calls in flight on two streams at once (each
    with its own workspace), repeatedly: every result matches the oracle and
    is bitwise the single-stream result, whatever share of the GPU each
    call's workgroups get."""
    M, N = 48, 262144
    xa = rand_bits(71, M, N, "f32", scale=2.0)
    xb = rand_bits(72, M, N, "f32", scale=4.0, loc=1.0)
    assert nt.nt_plan_launch(0, M, N, nt.NT_F32, True)["cooperative"] == 1
    ta, tb = to_dev(xa, "f32"), to_dev(xb, "f32")
    wsb = nt.nt_softmax_workspace_bytes(M, N, nt.NT_F32)
    wsa = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    wsb_t = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ref_a = softmax_with_ws(ta, "f32", wsa)
    ref_b = softmax_with_ws(tb, "f32", wsb_t)
    check_output(to_host_bits(ref_a, "f32"), oracle.softmax(xa, "f32"), "f32", "stream a")
    check_output(to_host_bits(ref_b, "f32"), oracle.softmax(xb, "f32"), "f32", "stream b")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for it in range(8):
        ya, yb = torch.empty_like(ta), torch.empty_like(tb)
        assert nt.nt_softmax_rows(M, N, nt.NT_F32, ta.data_ptr(), ya.data_ptr(), wsa.data_ptr(), wsb,
                                  sa.cuda_stream) == 0
        assert nt.nt_softmax_rows(M, N, nt.NT_F32, tb.data_ptr(), yb.data_ptr(), wsb_t.data_ptr(), wsb,
                                  sb.cuda_stream) == 0
        outs.append((ya, yb))
    torch.cuda.synchronize()
    say("case cooperative split on two streams")
    for ya, yb in outs:
        assert torch.equal(ya, ref_a) and torch.equal(yb, ref_b)


def test_graph_capture_fused_and_causal():
    """The fused add + RMSNorm and the causal softmax entry captured in a
    graph and replayed with new inputs: every replay matches the oracle."""
    M, N = 32, 4096
    xs = [rand_bits(80 + i, M, N, "bf16", scale=2.0) for i in range(3)]
    rs = [rand_bits(90 + i, M, N, "bf16") for i in range(3)]
    w = rand_bits(99, 1, N, "bf16", scale=0.3, loc=1.0)[0]
    x_t, r_t, w_t = to_dev(xs[0], "bf16"), to_dev(rs[0], "bf16"), to_dev(w, "bf16")
    h_t, y_t, c_t = torch.empty_like(x_t), torch.empty_like(x_t), torch.empty_like(x_t)

    def calls(stream):
        assert nt.nt_add_rmsnorm_rows(M, N, nt.NT_BF16, 1e-6, x_t.data_ptr(), r_t.data_ptr(), w_t.data_ptr(),
                                      h_t.data_ptr(), y_t.data_ptr(), stream) == 0
        assert nt.nt_softmax_causal_rows(M, N, nt.NT_BF16, 0.125, 16, 2, x_t.data_ptr(), c_t.data_ptr(), None, 0,
                                         stream) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(torch.cuda.current_stream().cuda_stream)
    for i in (2, 0, 1, 1):
        say(f"case graph replay fused/causal inputs {i}")
        x_t.copy_(to_dev(xs[i], "bf16"))
        r_t.copy_(to_dev(rs[i], "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rh, ry = oracle.add_rmsnorm(xs[i], rs[i], "bf16", 1e-6, weight=w)
        assert np.array_equal(to_host_bits(h_t, "bf16"), rh)
        check_output(to_host_bits(y_t, "bf16"), ry, "bf16", f"graph add+rmsnorm {i}")
        check_output(to_host_bits(c_t, "bf16"), oracle.softmax_causal(xs[i], "bf16", 0.125, 16, 2), "bf16",
                     f"graph causal {i}")


def test_side_stream_ordering():
    x = rand_bits(10, 256, 4096, "f16", loc=1.0)
    s = torch.cuda.Stream()
    x_t = to_dev(x, "f16")
    y = torch.empty_like(x_t)
    with torch.cuda.stream(s):
        rc = nt.nt_rmsnorm_rows(256, 4096, nt.NT_F16, 1e-6, x_t.data_ptr(), None, y.data_ptr(),
                                s.cuda_stream)
        assert rc == 0
        ev = torch.cuda.Event()
        ev.record(s)
    torch.cuda.current_stream().wait_event(ev)
    torch.cuda.synchronize()
    ref, _, _ = oracle_for("rmsnorm", x, "f16", 1e-6)
    check_output(to_host_bits(y, "f16"), ref, "f16", "side stream")


def test_torch_wrappers_and_noop():
    x = torch.randn(3, 5, 781, device="cuda")
    y = nt.softmax(x)
    assert y.shape == x.shape and torch.allclose(y.sum(-1), torch.ones(3, 5, device="cuda"), atol=1e-5)
    yl, m, r = nt.layer_norm(x.half(), eps=1e-5)
    assert m.shape == (3, 5) and r.shape == (3, 5)
    e = torch.empty(0, 64, device="cuda")
    assert nt.nt_softmax_rows(0, 64, nt.NT_F32, e.data_ptr(), e.data_ptr(), None, 0, None) == 0
    with pytest.raises(ValueError):
        nt.softmax(x.transpose(1, 2))


def test_errors_before_launch():
    """Invalid arguments are rejected before anything is enqueued.  Every
    buffer here is sized for the nominal shape, so even a validation bug
    could not make a kernel touch memory outside an allocation."""
    M, N = 4, 1 << 20
    big = torch.zeros(M * N + 64, device="cuda", dtype=torch.float32)
    p = big.data_ptr()
    assert nt.nt_softmax_rows(M, 8, nt.NT_F16, p + 1, p, None, 0, None) == 5     # misaligned element
    assert nt.nt_rmsnorm_rows(M, 8, nt.NT_F16, -1.0, p, None, p, None) == 4      # eps < 0
    assert nt.nt_softmax_rows(M, N, nt.NT_F32, p, p, None, 0, None) == 1         # needs a workspace
    wsb = nt.nt_softmax_workspace_bytes(M, N, nt.NT_F32)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    assert nt.nt_softmax_rows(M, N, nt.NT_F32, p, p, ws.data_ptr(), wsb - 8, None) == 6
    assert nt.nt_layernorm_rows(M, N, nt.NT_F32, float("nan"), p, None, None, p, None, None, None) == 4
    assert nt.nt_layernorm_rows(-1, N, nt.NT_F32, 1e-5, p, None, None, p, None, None, None) == 2
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt,N,shape", [("f16", 4104, (7, 2)), ("bf16", 7168, (7, 2)), ("f16", 8200, (5, 4)),
                                        ("bf16", 9728, (5, 4)), ("bf16", 9736, (6, 4)), ("f16", 11264, (6, 4)),
                                        ("bf16", 11520, (8, 4)), ("bf16", 11784, (7, 4)), ("f16", 14336, (7, 4)),
                                        ("f32", 8200, (12, 4)), ("f32", 12288, (12, 4)), ("f32", 2304, (4, 4))])
def test_layernorm_between_power_of_two_shapes(dt, N, shape, ntenv):
    """LayerNorm's shapes of 5-7 waves (16-bit) and 12 waves (fp32): the
    persistent kernel (aligned rows, parameters present; a grid smaller than
    the row count) against the oracle and bitwise against the one-row-per-
    workgroup kernel, and the resident kernel on misaligned rows and
    without parameters (the identity fills)."""
    code = DT_CODE[dt]
    M = 300
    p = nt.nt_plan_launch(1, M, N, code, True)
    assert (p["split"], p["waves_per_row"], p["chunks_per_lane"]) == (0, *shape), p
    x = rand_bits(N + 7, M, N, dt, scale=2.0, loc=-1.0)
    g = rand_bits(N + 8, 1, N, dt, scale=0.3, loc=1.0)[0]
    b = rand_bits(N + 9, 1, N, dt, scale=0.3)[0]
    x_t, g_t, b_t = to_dev(x, dt), to_dev(g, dt), to_dev(b, dt)
    ntenv.setenv("NT_PERSIST_GRID", "37")
    say(f"case layernorm {dt} {M}x{N} shape {shape} persistent={p['persistent']}")
    y1, m1, r1 = run_op("layernorm", x_t, dt, 1e-5, g_t, b_t)
    ref, rmean, rrstd = oracle_for("layernorm", x, dt, 1e-5, g, b)
    check_output(to_host_bits(y1, dt), ref, dt, f"layernorm {dt} {shape}")
    check_stats(m1.cpu().numpy(), rmean, "mean")
    check_stats(r1.cpu().numpy(), rrstd, "rstd")
    ntenv.setenv("NT_PERSISTENT", "0")
    y2, m2, r2 = run_op("layernorm", x_t, dt, 1e-5, g_t, b_t)
    assert np.array_equal(to_host_bits(y1, dt), to_host_bits(y2, dt))
    assert torch.equal(m1, m2) and torch.equal(r1, r2)
    ntenv.delenv("NT_PERSISTENT")
    for off in (1, 3):
        parity_case("layernorm", x, dt, 1e-5, g, b, x_off=off, y_off=off, what=f"misaligned {dt} {shape} off={off}")
    parity_case("layernorm", x, dt, 1e-5, None, None, what=f"no params {dt} {shape}")


def test_torch_wrappers_check_outputs_devices_and_stream():
    """The torch conveniences refuse outputs that do not match x (the
    kernels write M*N elements of x's type) and tensors on another device,
    and enqueue on the current stream: inside a torch.cuda.stream context
    the work goes to that stream (checked by ordering against a long
    preceding fill on the same stream)."""
    x = to_dev(rand_bits(3, 8, 1024, "f32"), "f32")
    w = torch.ones(1024, device="cuda")
    for bad in (torch.empty(8, 1023, device="cuda"), torch.empty(8, 1024, device="cuda", dtype=torch.float16),
                torch.empty(1024, 8, device="cuda").t(), torch.empty(8, 1024)):
        with pytest.raises(ValueError):
            nt.softmax(x, out=bad)
        with pytest.raises(ValueError):
            nt.rms_norm(x, w, out=bad)
    with pytest.raises(ValueError):
        nt.rms_norm(x, torch.ones(1024))                      # weight in host memory
    with pytest.raises(ValueError):
        nt.layer_norm(x, w, torch.zeros(1024))                # beta in host memory
    with pytest.raises(ValueError):
        nt.add_rms_norm(x, torch.zeros(8, 1024))              # residual in host memory
    say("case wrappers on a side stream")
    s = torch.cuda.Stream()
    big = torch.empty(1 << 27, device="cuda")
    xs = x.clone()
    with torch.cuda.stream(s):
        big.fill_(1.0)                                        # keeps the side stream busy for a while
        xs.mul_(2.0)
        y = nt.softmax(xs)                                    # must see the doubled input
    s.synchronize()
    ref = oracle.softmax(to_host_bits(x, "f32").view(np.float32) * np.float32(2.0), "f32")
    check_output(to_host_bits(y, "f32"), ref, "f32", "softmax on the current side stream")


def test_explicit_stream_allocations_belong_to_it():
    """With stream= given, the torch conveniences allocate on that stream:
    a block they free (the split path's workspace) goes back to that
    stream's pool, so the current stream's next allocation cannot be handed
    the same memory while the side stream's kernels may still use it."""
    s = torch.cuda.Stream()
    x = torch.zeros(8, 64, device="cuda")
    nbytes = 3 << 20
    with nt._alloc_on(s, x):
        a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    pa = a.data_ptr()
    del a
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")       # current stream
    assert b.data_ptr() != pa
    with nt._alloc_on(s.cuda_stream, x):                            # a raw handle works the same
        c = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    pc = c.data_ptr()
    del c
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert d.data_ptr() != pc
    torch.cuda.synchronize()


def test_explicit_stream_split_paths():
    """nt.softmax on the split path (64 x 262144 fp32: a workspace) and
    nt.rms_norm on a wide-row workspace shape, launched on a busy side
    stream, while the current stream allocates and fills buffers of the
    workspaces' sizes: the results match the oracle."""
    s = torch.cuda.Stream()
    xs = rand_bits(31, 64, 262144, "f32", scale=2.0)
    xr = rand_bits(32, 16, 1 << 20, "bf16")
    w = rand_bits(33, 1, 1 << 20, "bf16", scale=0.3, loc=1.0)[0]
    xs_t, xr_t, w_t = to_dev(xs, "f32"), to_dev(xr, "bf16"), to_dev(w, "bf16")
    wsb_s = nt.nt_softmax_workspace_bytes(64, 262144, nt.NT_F32)
    wsb_r = nt.nt_norm_workspace_bytes(nt.NT_OP_RMSNORM, 16, 1 << 20, nt.NT_BF16)
    assert wsb_s > 0 and wsb_r > 0
    big = torch.empty(1 << 28, device="cuda")
    torch.cuda.synchronize()
    say("case explicit side stream: softmax split + rms_norm split")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        big.fill_(1.0)                                # the side stream is busy for a while
    y = nt.softmax(xs_t, stream=s)
    yr = nt.rms_norm(xr_t, w_t, eps=1e-6, stream=s)
    junk = []
    for i in range(8):                                # current stream: reuse whatever is free
        for n in (wsb_s, wsb_r):
            t = torch.empty(n, dtype=torch.uint8, device="cuda")
            t.fill_(0xA5 + i)
            junk.append(t)
    s.synchronize()
    torch.cuda.synchronize()
    check_output(to_host_bits(y, "f32"), oracle.softmax(xs, "f32"), "f32", "softmax on an explicit stream")
    check_output(to_host_bits(yr, "bf16"), oracle.rmsnorm(xr, "bf16", 1e-6, weight=w), "bf16",
                 "rms_norm on an explicit stream")
