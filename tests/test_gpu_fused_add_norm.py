"""GPU parity of the fused residual add + norm (nt_add_rmsnorm_rows,
nt_add_layernorm_rows) against the oracle's plain, unfused definition: the
stored h = x + r bit for bit, y within the norms' bar (fp32: relative 1e-5;
fp16/bf16: 1 ulp of the oracle's float64 result rounded once), mean and rstd
relative 1e-5.  Also: in place, the persistent and looped paths, and bitwise
agreement with the plain norm entry point run on the stored h."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import check_output, check_stats, empty_like_dev, to_dev, to_host_bits
import oracle
import workloads

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import torch  # noqa: E402

import row_wise_reductions_amd as nt  # noqa: E402

DT_CODE = {"f32": nt.NT_F32, "f16": nt.NT_F16, "bf16": nt.NT_BF16}
OP_CODE = {"add_layernorm": nt.NT_OP_ADD_LAYERNORM, "add_rmsnorm": nt.NT_OP_ADD_RMSNORM}
EPS = {"add_layernorm": 1e-5, "add_rmsnorm": 1e-6}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_bits(seed, M, N, dt, scale=1.0, loc=0.0):
    rng = np.random.default_rng(seed)
    return workloads.encode(rng.standard_normal((M, N)) * scale + loc, dt)


def as_bits(stored, dt):
    """Oracle stored values (float32 array or uint16 bits) -> raw bits."""
    a = np.asarray(stored)
    return a.view(np.uint32) if dt == "f32" else a.view(np.uint16)


def run_fused(op, x_t, r_t, dt, eps, p0=None, p1=None, h_t=None, y_t=None):
    M, N = x_t.shape
    code = DT_CODE[dt]
    h = torch.empty_like(x_t) if h_t is None else h_t
    y = torch.empty_like(x_t) if y_t is None else y_t
    s = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    mean = rstd = None
    if op == "add_layernorm":
        mean = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        rstd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        rc = nt.nt_add_layernorm_rows(M, N, code, eps, x_t.data_ptr(), r_t.data_ptr(), ptr(p0), ptr(p1),
                                      h.data_ptr(), y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), s)
    else:
        rc = nt.nt_add_rmsnorm_rows(M, N, code, eps, x_t.data_ptr(), r_t.data_ptr(), ptr(p0), h.data_ptr(),
                                    y.data_ptr(), s)
    assert rc == 0, f"{op}: status {rc} ({nt.nt_status_string(rc)})"
    torch.cuda.synchronize()
    return h, y, mean, rstd


def oracle_fused(op, x, r, dt, eps, p0=None, p1=None):
    if op == "add_layernorm":
        return oracle.add_layernorm(x, r, dt, eps, gamma=p0, beta=p1)
    h, y = oracle.add_rmsnorm(x, r, dt, eps, weight=p0)
    return h, y, None, None


def check_fused(op, dt, h, y, mean, rstd, ref, what, rows=None):
    rh, ry, rmean, rrstd = ref
    hb = to_host_bits(h, dt)
    yb = to_host_bits(y, dt)
    if rows is not None:
        hb, yb = hb[rows], yb[rows]
    want = as_bits(rh, dt)
    bad = hb != want
    assert not bad.any(), f"{what}: h differs from the stored sum in {int(bad.sum())} elements"
    check_output(yb, ry, dt, what)
    if op == "add_layernorm":
        m, r = mean.cpu().numpy(), rstd.cpu().numpy()
        if rows is not None:
            m, r = m[rows], r[rows]
        check_stats(m, rmean, what + " mean")
        check_stats(r, rrstd, what + " rstd")


def fused_case(op, x, r, dt, eps, p0=None, p1=None, off=0, y_off=0, what=""):
    M, N = x.shape
    say(f"case {what} op={op} dt={dt} M={M} N={N} off={off} y_off={y_off}")
    x_t, r_t = to_dev(x, dt, off), to_dev(r, dt, off)
    h_t, y_t = empty_like_dev((M, N), dt, off), empty_like_dev((M, N), dt, y_off)
    p0_t = None if p0 is None else to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    h, y, mean, rstd = run_fused(op, x_t, r_t, dt, eps, p0_t, p1_t, h_t, y_t)
    check_fused(op, dt, h, y, mean, rstd, oracle_fused(op, x, r, dt, eps, p0, p1), what)
    return h, y, mean, rstd


def params(op, N, dt, seed):
    p0 = rand_bits(seed, 1, N, dt, scale=0.3, loc=1.0)[0]
    p1 = rand_bits(seed + 1, 1, N, dt, scale=0.3)[0] if op == "add_layernorm" else None
    return p0, p1


# ----------------------------------------------------------------------------
# the fused workloads at the norm workloads' shapes
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", [w.name for w in workloads.NEXT_WORKLOADS if w.op.startswith("add_")])
def test_fused_workload_full_size(name):
    w = workloads.BY_NAME[name]
    say(f"workload {name}: generating {w.M}x{w.N} {w.dt}")
    d = w.make()
    p0 = d.get("gamma", d.get("weight"))
    p1 = d.get("beta")
    x_t, r_t = to_dev(d["x"], w.dt), to_dev(d["residual"], w.dt)
    p0_t = to_dev(p0, w.dt)
    p1_t = None if p1 is None else to_dev(p1, w.dt)
    plan = nt.nt_plan_launch(OP_CODE[w.op], w.M, w.N, DT_CODE[w.dt], True)
    say(f"workload {name}: launching ({plan['waves_per_row']}x{plan['chunks_per_lane']}, "
        f"persistent={plan['persistent']})")
    h, y, mean, rstd = run_fused(w.op, x_t, r_t, w.dt, w.eps, p0_t, p1_t)
    rows = np.arange(w.M)
    if w.M * w.N > 40_000_000:
        rng = np.random.default_rng(8)
        rows = np.unique(np.concatenate([rng.choice(w.M, 4096, replace=False), [0, 1, w.M - 1]]))
    ref = oracle_fused(w.op, np.ascontiguousarray(d["x"][rows]), np.ascontiguousarray(d["residual"][rows]),
                       w.dt, w.eps, p0, p1)
    check_fused(w.op, w.dt, h, y, mean, rstd, ref, name, rows=rows)


# ----------------------------------------------------------------------------
# widths: one pass, persistent, looped; aligned and misaligned
# ----------------------------------------------------------------------------

FUSED_N = [1, 7, 64, 255, 781, 1025, 4096, 8192, 8193, 16384, 16385, 65537]
FUSED = [(op, dt, N) for op in ("add_rmsnorm", "add_layernorm") for dt in ("f32", "f16", "bf16") for N in FUSED_N]


@pytest.mark.parametrize("op,dt,N", FUSED)
def test_fused_sweep(op, dt, N):
    M = 37 if N <= 16385 else 5
    x = rand_bits(N, M, N, dt, scale=2.0, loc=1.0)
    r = rand_bits(N + 1, M, N, dt, scale=1.5, loc=-1.0)
    p0, p1 = params(op, N, dt, N + 2)
    for off, y_off in ((0, 0), (1, 3)):
        fused_case(op, x, r, dt, EPS[op], p0, p1, off=off, y_off=y_off, what=f"sweep {op} {dt} N={N}")
    # no parameter vectors (identity), aligned
    fused_case(op, x, r, dt, EPS[op], what=f"sweep {op} {dt} N={N} no params")


@pytest.mark.parametrize("op", ["add_rmsnorm", "add_layernorm"])
@pytest.mark.parametrize("path", ["default", "looped", "resident"])
def test_fused_in_place(op, path, ntenv):
    """h may be x or the residual, y may be x or the residual, on every path."""
    dt, M, N = "bf16", 40, 4096
    if path == "looped":
        ntenv.setenv("NT_FORCE_PATH", "looped")
    if path == "resident":
        ntenv.setenv("NT_PERSISTENT", "0")
    x = rand_bits(11, M, N, dt, scale=2.0)
    r = rand_bits(12, M, N, dt)
    p0, p1 = params(op, N, dt, 13)
    p0_t = to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    ref = oracle_fused(op, x, r, dt, EPS[op], p0, p1)
    for h_is, y_is in (("r", None), ("x", None), (None, "x"), (None, "r"), ("r", "x"), ("x", "r")):
        say(f"case in-place {op} {path} h={h_is} y={y_is}")
        x_t, r_t = to_dev(x, dt), to_dev(r, dt)
        pick = {"x": x_t, "r": r_t, None: None}
        h, y, mean, rstd = run_fused(op, x_t, r_t, dt, EPS[op], p0_t, p1_t, pick[h_is], pick[y_is])
        check_fused(op, dt, h, y, mean, rstd, ref, f"in place {op} {path} h={h_is} y={y_is}")


@pytest.mark.parametrize("op", ["add_layernorm"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_fused_persistent_small_grids(op, dt, ntenv):
    """The persistent fused kernel (fused add + LayerNorm rows of 1024 chunks
    or more) on grids far smaller than M is bitwise the one-row fused kernel."""
    M, N = 300, 8192
    x = rand_bits(21, M, N, dt, scale=2.0, loc=1.5)
    r = rand_bits(22, M, N, dt)
    p0, p1 = params(op, N, dt, 23)
    assert nt.nt_plan_launch(OP_CODE[op], M, N, DT_CODE[dt], True)["persistent"] == 1
    x_t, r_t, p0_t = to_dev(x, dt), to_dev(r, dt), to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    ref = oracle_fused(op, x, r, dt, EPS[op], p0, p1)
    outs = []
    for grid in ("3", "7", None):
        say(f"case fused persistent {op} {dt} grid={grid}")
        if grid:
            ntenv.setenv("NT_PERSIST_GRID", grid)
        else:
            ntenv.delenv("NT_PERSIST_GRID", raising=False)
            ntenv.setenv("NT_PERSISTENT", "0")
        h, y, mean, rstd = run_fused(op, x_t, r_t, dt, EPS[op], p0_t, p1_t)
        check_fused(op, dt, h, y, mean, rstd, ref, f"fused persistent {op} {dt} grid={grid}")
        outs.append((to_host_bits(h, dt), to_host_bits(y, dt)))
    for hb, yb in outs[1:]:
        assert np.array_equal(hb, outs[0][0]) and np.array_equal(yb, outs[0][1])


@pytest.mark.parametrize("op", ["add_rmsnorm", "add_layernorm"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [781, 4096, 16385])
def test_fused_equals_plain_norm_of_h(op, dt, N):
    """y of the fused call is bitwise the plain norm entry point's output on
    the stored h whenever both plan the same kernel shape."""
    M = 24
    x = rand_bits(31, M, N, dt, scale=2.0)
    r = rand_bits(32, M, N, dt)
    p0, p1 = params(op, N, dt, 33)
    x_t, r_t, p0_t = to_dev(x, dt), to_dev(r, dt), to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    say(f"case fused vs plain {op} {dt} N={N}")
    h, y, mean, rstd = run_fused(op, x_t, r_t, dt, EPS[op], p0_t, p1_t)
    y2 = torch.empty_like(h)
    s = torch.cuda.current_stream().cuda_stream
    code = DT_CODE[dt]
    if op == "add_layernorm":
        m2 = torch.empty(M, device="cuda")
        r2 = torch.empty(M, device="cuda")
        assert nt.nt_layernorm_rows(M, N, code, EPS[op], h.data_ptr(), p0_t.data_ptr(), p1_t.data_ptr(),
                                    y2.data_ptr(), m2.data_ptr(), r2.data_ptr(), s) == 0
    else:
        assert nt.nt_rmsnorm_rows(M, N, code, EPS[op], h.data_ptr(), p0_t.data_ptr(), y2.data_ptr(), s) == 0
    torch.cuda.synchronize()
    fused_plan = nt.nt_plan_launch(OP_CODE[op], M, N, code, True)
    plain_plan = nt.nt_plan_launch({"add_layernorm": 1, "add_rmsnorm": 2}[op], M, N, code, True)
    keys = ("split", "waves_per_row", "chunks_per_lane", "persistent")
    if all(fused_plan[k] == plain_plan[k] for k in keys):
        assert np.array_equal(to_host_bits(y, dt), to_host_bits(y2, dt))
        if op == "add_layernorm":
            assert torch.equal(mean, m2) and torch.equal(rstd, r2)
    else:
        ref = oracle_fused(op, x, r, dt, EPS[op], p0, p1)
        check_output(to_host_bits(y2, dt), ref[1], dt, "plain norm of h")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_fused_h_exact_over_wide_ranges(dt):
    """h is the exactly rounded sum also for subnormal operands, operands of
    very different magnitude and exact cancellation."""
    M, N = 16, 1024
    rng = np.random.default_rng(41)
    lo, hi = {"f32": (-140, 8), "f16": (-24, 4), "bf16": (-133, 8)}[dt]
    mag = lambda: rng.standard_normal((M, N)) * np.exp2(rng.integers(lo, hi, (M, N)).astype(np.float64))  # noqa
    x = workloads.encode(mag(), dt)
    r = workloads.encode(mag(), dt)
    if dt == "f32":
        r[:, :128] = -x[:, :128]                        # exact cancellation
    else:
        r[:, :128] = x[:, :128] ^ np.uint16(0x8000)
    say(f"case fused wide-range h {dt}")
    x_t, r_t = to_dev(x, dt), to_dev(r, dt)
    h, y, _, _ = run_fused("add_rmsnorm", x_t, r_t, dt, 1e-6)
    want = as_bits(oracle.add_rmsnorm(x, r, dt, 1e-6)[0], dt)
    got = to_host_bits(h, dt)
    mag = np.array(0x7FFFFFFF if dt == "f32" else 0x7FFF).astype(got.dtype)
    same = (got == want) | (((got & mag) == 0) & ((want & mag) == 0))     # +0 and -0 agree
    assert same.all(), f"{int((~same).sum())} sums differ"


def test_fused_errors_with_real_buffers():
    M, N, dt = 8, 1024, "bf16"
    x = to_dev(rand_bits(1, M, N, dt), dt)
    r = to_dev(rand_bits(2, M, N, dt), dt)
    flat = torch.empty(M * N + 16, dtype=torch.bfloat16, device="cuda")
    r_shift = flat[1:1 + M * N].view(M, N)                # 2 bytes off x's 16-byte phase
    h = torch.empty_like(x)
    y = torch.empty_like(x)
    s = torch.cuda.current_stream().cuda_stream
    code = nt.NT_BF16
    assert nt.nt_add_rmsnorm_rows(M, N, code, 1e-6, x.data_ptr(), r_shift.data_ptr(), None, h.data_ptr(),
                                  y.data_ptr(), s) == 5
    assert nt.nt_add_rmsnorm_rows(M, N, code, 1e-6, x.data_ptr(), r.data_ptr(), None, r_shift.data_ptr(),
                                  y.data_ptr(), s) == 5
    assert nt.nt_add_rmsnorm_rows(M, N, code, 1e-6, x.data_ptr(), r.data_ptr(), None, h.data_ptr(),
                                  h.data_ptr(), s) == 8
    assert nt.nt_add_layernorm_rows(M, N, code, 1e-5, x.data_ptr(), None, None, None, h.data_ptr(),
                                    y.data_ptr(), None, None, s) == 1
    torch.cuda.synchronize()


def test_fused_torch_wrappers():
    x = torch.randn(3, 5, 781, device="cuda", dtype=torch.bfloat16)
    r = torch.randn(3, 5, 781, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(781, device="cuda", dtype=torch.bfloat16)
    h, y = nt.add_rms_norm(x, r, w, eps=1e-6)
    assert torch.equal(h, x + r)                    # torch's bf16 add rounds the same sum once
    assert torch.equal(y, nt.rms_norm(h, w, eps=1e-6))
    g = torch.randn(781, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(781, device="cuda", dtype=torch.bfloat16)
    h2, y2, mean, rstd = nt.add_layer_norm(x, r, g, b, eps=1e-5)
    y3, m3, r3 = nt.layer_norm(h2, g, b, eps=1e-5)
    assert torch.equal(h2, h) and torch.equal(y2, y3) and torch.equal(mean, m3) and torch.equal(rstd, r3)
    assert mean.shape == (3, 5)
