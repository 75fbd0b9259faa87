"""GPU parity of the norms with a workspace (nt_layernorm_rows_ws,
nt_rmsnorm_rows_ws): a few rows too wide for one pass, each cut into chunks
on many workgroups.  Against the oracle at the norms' bar (fp32: relative
1e-5; fp16/bf16: 1 ulp of the oracle's float64 result rounded once; mean and
rstd relative 1e-5), aligned and misaligned, with and without parameters, in
place, with a workspace full of garbage, bitwise repeatable, and with a NULL
workspace bitwise equal to the plain entry points."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import check_output, check_stats, empty_like_dev, oracle_for, to_dev, to_host_bits
import workloads

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import torch  # noqa: E402

import row_wise_reductions_amd as nt  # noqa: E402

DT_CODE = {"f32": nt.NT_F32, "f16": nt.NT_F16, "bf16": nt.NT_BF16}
OP_CODE = {"layernorm": nt.NT_OP_LAYERNORM, "rmsnorm": nt.NT_OP_RMSNORM}
WS_CODE = {"layernorm": nt.NT_OP_LAYERNORM_WS, "rmsnorm": nt.NT_OP_RMSNORM_WS}
EPS = {"layernorm": 1e-5, "rmsnorm": 1e-6}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_bits(seed, M, N, dt, scale=1.0, loc=0.0):
    rng = np.random.default_rng(seed)
    return workloads.encode(rng.standard_normal((M, N)) * scale + loc, dt)


def _p(t):
    return None if t is None else t.data_ptr()


def run_ws(op, x_t, dt, p0=None, p1=None, y_t=None, ws=None, wsb=None, plain=False):
    """Launch one norm through the C ABI on the current stream and wait:
    the workspace entry point (ws=None allocates the size the library asks
    for; ws=False passes NULL), or with plain=True the entry point without
    a workspace."""
    M, N = x_t.shape
    code = DT_CODE[dt]
    y = y_t if y_t is not None else empty_like_dev((M, N), dt)
    s = torch.cuda.current_stream().cuda_stream
    if ws is None:
        need = nt.nt_norm_workspace_bytes(OP_CODE[op], M, N, code)
        ws = torch.empty(max(need, 8), dtype=torch.uint8, device="cuda")
        wsb = need
    wp = None if ws is False else ws.data_ptr()
    wsb = 0 if ws is False else (wsb if wsb is not None else ws.numel())
    mean = rstd = None
    if op == "layernorm":
        mean = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        rstd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        if plain:
            rc = nt.nt_layernorm_rows(M, N, code, EPS[op], x_t.data_ptr(), _p(p0), _p(p1), y.data_ptr(),
                                      mean.data_ptr(), rstd.data_ptr(), s)
        else:
            rc = nt.nt_layernorm_rows_ws(M, N, code, EPS[op], x_t.data_ptr(), _p(p0), _p(p1), y.data_ptr(),
                                         mean.data_ptr(), rstd.data_ptr(), wp, wsb, s)
    elif plain:
        rc = nt.nt_rmsnorm_rows(M, N, code, EPS[op], x_t.data_ptr(), _p(p0), y.data_ptr(), s)
    else:
        rc = nt.nt_rmsnorm_rows_ws(M, N, code, EPS[op], x_t.data_ptr(), _p(p0), y.data_ptr(), wp, wsb, s)
    assert rc == 0, f"{op}: status {rc} ({nt.nt_status_string(rc)})"
    torch.cuda.synchronize()
    return y, mean, rstd


def params(op, N, dt, seed, with_params=True):
    if not with_params:
        return None, None
    p0 = rand_bits(seed + 1, 1, N, dt, scale=0.3, loc=1.0)[0]
    p1 = rand_bits(seed + 2, 1, N, dt, scale=0.3)[0] if op == "layernorm" else None
    return p0, p1


def check(op, y, mean, rstd, x, dt, p0, p1, what):
    ref, rmean, rrstd = oracle_for(op, x, dt, EPS[op], p0, p1)
    check_output(to_host_bits(y, dt), ref, dt, what)
    if op == "layernorm":
        check_stats(mean.cpu().numpy(), rmean, what + " mean")
        check_stats(rstd.cpu().numpy(), rrstd, what + " rstd")


CASES = [(1, 40000, "f32"), (3, 100003, "f32"), (2, 65536, "f16"), (7, 50001, "bf16"), (64, 262144, "bf16"),
         (5, 1 << 20, "f16"), (16, 131072, "f32")]


@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("M,N,dt", CASES)
def test_split_norm_parity(op, M, N, dt):
    """Every element against the oracle, rows shifted off the 16-byte grid
    by 0 and 1 elements (x and y together, and y alone), with parameters
    and, on the aligned rows, without (the identity fills)."""
    seed = M * 1000003 + N
    x = rand_bits(seed, M, N, dt, scale=2.0, loc=3.0)
    for xo, yo, with_p in ((0, 0, True), (1, 1, True), (0, 1, True), (0, 0, False)):
        plan = nt.nt_plan_launch(WS_CODE[op], M, N, DT_CODE[dt], xo == 0 and yo == 0)
        assert plan["split"] == 3, plan
        p0, p1 = params(op, N, dt, seed, with_p)
        what = f"split {op} {dt} M={M} N={N} x_off={xo} y_off={yo} params={with_p} P={plan['row_chunks']}"
        say("case", what)
        x_t = to_dev(x, dt, xo)
        y, mean, rstd = run_ws(op, x_t, dt, None if p0 is None else to_dev(p0, dt),
                               None if p1 is None else to_dev(p1, dt), empty_like_dev((M, N), dt, yo))
        check(op, y, mean, rstd, x, dt, p0, p1, what)


@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_norm_in_place_garbage_workspace_repeatable(op, dt):
    """y == x (the LayerNorm pivot, the row's first element, is read from
    the workspace, not from x, which the row's first workgroup overwrites);
    a workspace full of garbage; two calls bitwise equal."""
    M, N = 6, 300007
    x = rand_bits(77, M, N, dt, scale=1.5, loc=-2.0)
    p0, p1 = params(op, N, dt, 77)
    p0_t = to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    need = nt.nt_norm_workspace_bytes(OP_CODE[op], M, N, DT_CODE[dt])
    assert need > 0
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    say(f"case in-place split {op} {dt} M={M} N={N}")
    x_t = to_dev(x, dt)
    y, mean, rstd = run_ws(op, x_t, dt, p0_t, p1_t, y_t=x_t, ws=ws)
    check(op, x_t, mean, rstd, x, dt, p0, p1, f"in-place split {op} {dt}")
    say(f"case repeat split {op} {dt} M={M} N={N}")
    x_t = to_dev(x, dt)
    a, am, ar = run_ws(op, x_t, dt, p0_t, p1_t, ws=ws)
    ws.random_(0, 256)
    b, bm, br = run_ws(op, x_t, dt, p0_t, p1_t, ws=ws)
    assert np.array_equal(to_host_bits(a, dt), to_host_bits(b, dt))
    if op == "layernorm":
        assert torch.equal(am, bm) and torch.equal(ar, br)


@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
def test_null_workspace_is_the_plain_plan(op):
    """NULL workspace: the looped one-workgroup-per-row kernel, bitwise equal
    to the plain entry point; both within the bar of the split result."""
    M, N, dt = 4, 70001, "bf16"
    x = rand_bits(5, M, N, dt, scale=2.0)
    p0, p1 = params(op, N, dt, 5)
    x_t, p0_t = to_dev(x, dt), to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    say(f"case null-workspace {op} {dt} M={M} N={N}")
    a, am, ar = run_ws(op, x_t, dt, p0_t, p1_t, ws=False)
    b, bm, br = run_ws(op, x_t, dt, p0_t, p1_t, plain=True)
    assert np.array_equal(to_host_bits(a, dt), to_host_bits(b, dt))
    if op == "layernorm":
        assert torch.equal(am, bm) and torch.equal(ar, br)
    check(op, a, am, ar, x, dt, p0, p1, f"null-workspace {op}")


def test_split_norm_rejects_small_workspace():
    M, N, dt = 4, 70001, "f32"
    need = nt.nt_norm_workspace_bytes(nt.NT_OP_RMSNORM, M, N, nt.NT_F32)
    x_t = to_dev(rand_bits(1, M, N, dt), dt)
    y = empty_like_dev((M, N), dt)
    ws = torch.empty(need + 8, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert nt.nt_rmsnorm_rows_ws(M, N, nt.NT_F32, 1e-6, x_t.data_ptr(), None, y.data_ptr(), ws.data_ptr(),
                                 need - 8, s) == 6      # NT_ERR_WORKSPACE
    assert nt.nt_rmsnorm_rows_ws(M, N, nt.NT_F32, 1e-6, x_t.data_ptr(), None, y.data_ptr(), ws.data_ptr() + 4,
                                 need, s) == 5          # NT_ERR_ALIGN (in bounds had it launched)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()                 # nothing launched


@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
def test_torch_wrappers_use_the_split(op):
    M, N, dt = 8, 200000, "bf16"
    x = rand_bits(11, M, N, dt, scale=2.0, loc=1.0)
    p0, p1 = params(op, N, dt, 11)
    assert nt.nt_norm_workspace_bytes(OP_CODE[op], M, N, DT_CODE[dt]) > 0
    x_t, p0_t = to_dev(x, dt), to_dev(p0, dt)
    say(f"case torch wrapper split {op} {dt} M={M} N={N}")
    if op == "layernorm":
        y, mean, rstd = nt.layer_norm(x_t, p0_t, to_dev(p1, dt), eps=EPS[op])
    else:
        y, mean, rstd = nt.rms_norm(x_t, p0_t, eps=EPS[op]), None, None
    torch.cuda.synchronize()
    check(op, y, mean, rstd, x, dt, p0, p1, f"torch wrapper split {op}")


@pytest.mark.parametrize("op,M,N,dt,al", [("rmsnorm", 256, 65536, "f32", True), ("layernorm", 256, 65536, "f32", True),
                                          ("rmsnorm", 128, 262144, "bf16", True), ("rmsnorm", 512, 65536, "f16", True),
                                          ("rmsnorm", 410, 40003, "f32", False),
                                          ("layernorm", 410, 40003, "f32", False),
                                          ("rmsnorm", 128, 262144, "f32", True),
                                          ("rmsnorm", 300, 100003, "f32", False),
                                          ("layernorm", 128, 262144, "f32", True)])
def test_cooperative_split_norm_bitwise(op, M, N, dt, al, ntenv):
    """The one-pass form (records exchanged between a row's workgroups) passes
    the oracle and gives the two-kernel form's bits, also when every other
    chunk's record is recomputed by the waiting workgroup (no wait at all)."""
    code = DT_CODE[dt]
    xo = 0 if al else 1
    p = nt.nt_plan_launch(WS_CODE[op], M, N, code, al)
    assert p["split"] == 3 and p["cooperative"] == 1, p
    seed = 7 * M + N
    x = rand_bits(seed, M, N, dt, scale=2.0, loc=1.0)
    p0, p1 = params(op, N, dt, seed)
    x_t, p0_t = to_dev(x, dt, xo), to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    say(f"case coop split {op} {dt} M={M} N={N} aligned={al} P={p['row_chunks']}")
    a, am, ar = run_ws(op, x_t, dt, p0_t, p1_t)
    check(op, a, am, ar, x, dt, p0, p1, f"coop split {op} {dt} M={M} N={N}")
    outs = []
    for env, val in (("NT_COOP_SPIN", "0"), ("NT_COOP", "0")):
        ntenv.setenv(env, val)
        if env == "NT_COOP":
            # the two kernels at this row count
            ntenv.setenv("NT_NORM_SPLIT_ROWS", "100000")
            q = nt.nt_plan_launch(WS_CODE[op], M, N, code, al)
            assert q["split"] == 3 and q["cooperative"] == 0, q
        say(f"case coop split {op} {dt} M={M} N={N} {env}={val}")
        outs.append((env, run_ws(op, x_t, dt, p0_t, p1_t),
                     (q["waves_per_row"], q["chunks_per_lane"], q["row_chunks"]) ==
                     (p["waves_per_row"], p["chunks_per_lane"], p["row_chunks"]) if env == "NT_COOP" else True))
        ntenv.delenv(env)
        ntenv.delenv("NT_NORM_SPLIT_ROWS", raising=False)
    ref = to_host_bits(a, dt)
    for env, (y, ym, yr), same_chunks in outs:
        if same_chunks:
            # same chunks (records recomputed, or the two kernels): bitwise
            assert np.array_equal(to_host_bits(y, dt), ref), env
            if op == "layernorm":
                assert torch.equal(ym, am) and torch.equal(yr, ar), env
        else:
            # the two kernels on other chunks: the oracle's bar
            check(op, y, ym, yr, x, dt, p0, p1, f"two-kernel split {op} {dt} M={M} N={N}")


def test_cooperative_split_norm_on_concurrent_streams():
    """Two calls in flight at once on two streams, each with its own
    workspace: records are per workspace and tagged per call."""
    M, N, dt = 128, 262144, "bf16"
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, M, N, nt.NT_BF16, True)["cooperative"] == 1
    xs = [rand_bits(40 + i, M, N, dt, scale=2.0) for i in range(2)]
    w = rand_bits(43, 1, N, dt, scale=0.3, loc=1.0)[0]
    w_t = to_dev(w, dt)
    need = nt.nt_norm_workspace_bytes(nt.NT_OP_RMSNORM, M, N, nt.NT_BF16)
    streams = [torch.cuda.Stream() for _ in range(2)]
    x_ts = [to_dev(x, dt) for x in xs]
    ys = [empty_like_dev((M, N), dt) for _ in range(2)]
    wss = [torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    say(f"case coop split on two streams M={M} N={N}")
    for _ in range(3):
        for i in range(2):
            rc = nt.nt_rmsnorm_rows_ws(M, N, nt.NT_BF16, EPS["rmsnorm"], x_ts[i].data_ptr(), w_t.data_ptr(),
                                       ys[i].data_ptr(), wss[i].data_ptr(), need, streams[i].cuda_stream)
            assert rc == 0
    torch.cuda.synchronize()
    for i in range(2):
        check("rmsnorm", ys[i], None, None, xs[i], dt, w, None, f"two streams, stream {i}")


def test_split_norm_graph_capture_and_replay():
    """Split norms captured into a HIP graph and replayed with new inputs
    copied in (eagerly) between replays: every replay matches the oracle.
    The one-pass (cooperative) form is captured with its record tag read
    from the word after the records, which a one-thread kernel advances
    before each replay's launch: the word moves by one per replay, and a
    replay on the eager call's inputs gives the eager bits."""
    M, N = 128, 262144
    xs = [rand_bits(70 + i, M, N, "bf16", scale=2.0 + i, loc=0.5) for i in range(3)]
    w = rand_bits(73, 1, N, "bf16", scale=0.3, loc=1.0)[0]
    lx = [rand_bits(80 + i, 4, 100003, "f32", scale=1.0 + i, loc=-1.0) for i in range(3)]
    g_ = rand_bits(83, 1, 100003, "f32", scale=0.3, loc=1.0)[0]
    b_ = rand_bits(84, 1, 100003, "f32", scale=0.3)[0]
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, M, N, nt.NT_BF16, True)["cooperative"] == 1
    x_t, w_t, y_t = to_dev(xs[0], "bf16"), to_dev(w, "bf16"), empty_like_dev((M, N), "bf16")
    lx_t, g_t, b_t = to_dev(lx[0], "f32"), to_dev(g_, "f32"), to_dev(b_, "f32")
    ly_t = empty_like_dev((4, 100003), "f32")
    mean = torch.empty(4, device="cuda")
    rstd = torch.empty(4, device="cuda")
    wsb = nt.nt_norm_workspace_bytes(nt.NT_OP_RMSNORM, M, N, nt.NT_BF16)
    lwsb = nt.nt_norm_workspace_bytes(nt.NT_OP_LAYERNORM, 4, 100003, nt.NT_F32)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    lws = torch.empty(lwsb, dtype=torch.uint8, device="cuda")

    def calls(stream):
        assert nt.nt_rmsnorm_rows_ws(M, N, nt.NT_BF16, EPS["rmsnorm"], x_t.data_ptr(), w_t.data_ptr(),
                                     y_t.data_ptr(), ws.data_ptr(), wsb, stream) == 0
        assert nt.nt_layernorm_rows_ws(4, 100003, nt.NT_F32, EPS["layernorm"], lx_t.data_ptr(), g_t.data_ptr(),
                                       b_t.data_ptr(), ly_t.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                                       lws.data_ptr(), lwsb, stream) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = to_host_bits(y_t, "bf16")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(torch.cuda.current_stream().cuda_stream)
    # the tag word: in the 16 bytes after the plan's records
    pw = nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, M, N, nt.NT_BF16, True)["workspace_bytes"]
    tag_word = ws[pw - 16:pw - 12].view(torch.int32)
    torch.cuda.synchronize()
    tag0 = int(tag_word.item())
    for n, i in enumerate((1, 0, 2, 2, 1)):
        say(f"case split-norm graph replay inputs {i}")
        x_t.copy_(to_dev(xs[i], "bf16"))
        lx_t.copy_(to_dev(lx[i], "f32"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check("rmsnorm", y_t, None, None, xs[i], "bf16", w, None, f"graph split rmsnorm {i}")
        check("layernorm", ly_t, mean, rstd, lx[i], "f32", g_, b_, f"graph split layernorm {i}")
        assert (int(tag_word.item()) - tag0) & 0xFFFFFFFF == n + 1, "one tag advance per replay"
        if i == 0:
            assert np.array_equal(to_host_bits(y_t, "bf16"), eager)


def test_split_layernorm_rows_past_2gib_offsets():
    """Five bf16 rows of 2^28 + 5 elements (512 MiB each, the last one
    starting beyond 2^31 bytes; misaligned rows): the split LayerNorm (two
    kernels, 16385 chunks per row) against the oracle on every element,
    compared in column blocks, with mean and rstd.  Inputs drawn in float32
    and rounded once to bf16 to keep the host side small."""
    import oracle
    M, N = 5, (1 << 28) + 5
    rng = np.random.default_rng(N)
    x = workloads.to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32) * np.float32(2.0) + np.float32(1.0))
    g = workloads.to_bf16_bits(np.float32(1.0) + np.float32(0.3) * rng.standard_normal(N, dtype=np.float32))
    b = workloads.to_bf16_bits(np.float32(0.3) * rng.standard_normal(N, dtype=np.float32))
    assert (M - 1) * N * 2 > (1 << 31)
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM_WS, M, N, nt.NT_BF16, False)
    assert p["split"] == 3 and p["cooperative"] == 0 and p["row_chunks"] > 16384, p
    say(f"case 2GiB-offset split layernorm bf16 M={M} N={N} P={p['row_chunks']}")
    x_t, g_t, b_t = to_dev(x, "bf16"), to_dev(g, "bf16"), to_dev(b, "bf16")
    y, mean, rstd = run_ws("layernorm", x_t, "bf16", g_t, b_t)
    del x_t
    yb = to_host_bits(y, "bf16")
    del y
    ref, rmean, rrstd = oracle.layernorm(x, "bf16", EPS["layernorm"], gamma=g, beta=b)
    check_stats(mean.cpu().numpy(), rmean, "2GiB-offset split layernorm mean")
    check_stats(rstd.cpu().numpy(), rrstd, "2GiB-offset split layernorm rstd")
    blk = 1 << 25
    for r in range(M):
        for j0 in range(0, N, blk):
            check_output(yb[r, j0:j0 + blk], ref[r, j0:j0 + blk], "bf16", f"2GiB-offset split layernorm row {r} col {j0}")


@pytest.mark.parametrize("op", ["rmsnorm", "layernorm"])
def test_cooperative_split_norm_large_grid(op, ntenv):
    """8192 fp32 rows of 65536 elements in one pass: 65536 workgroups, far
    more than are resident at once, so rows straddle dispatch waves and some
    workgroups wait on siblings that start later.  Sampled rows against the
    oracle; every output bitwise equal to the two-kernel form on the same
    chunks."""
    M, N, dt = 8192, 65536, "f32"
    p = nt.nt_plan_launch(WS_CODE[op], M, N, nt.NT_F32, True)
    assert p["split"] == 3 and p["cooperative"] == 1 and p["grid"] == M * p["row_chunks"] >= 16 * 2048, p
    rng = np.random.default_rng(M + N)
    x = (rng.standard_normal((M, N), dtype=np.float32) * np.float32(1.5) + np.float32(0.25))
    p0, p1 = params(op, N, dt, 99)
    x_t, p0_t = to_dev(x, dt), to_dev(p0, dt)
    p1_t = None if p1 is None else to_dev(p1, dt)
    say(f"case coop split large grid {op} {dt} M={M} N={N} grid={p['grid']}")
    a, am, ar = run_ws(op, x_t, dt, p0_t, p1_t)
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(M, 48, replace=False), [0, 1, M - 1]]))
    ab = to_host_bits(a, dt)
    ref, rmean, rrstd = oracle_for(op, x[rows], dt, EPS[op], p0, p1)
    check_output(ab[rows], ref, dt, f"coop large grid {op}")
    if op == "layernorm":
        check_stats(am.cpu().numpy()[rows], rmean, "coop large grid mean")
        check_stats(ar.cpu().numpy()[rows], rrstd, "coop large grid rstd")
    ntenv.setenv("NT_COOP", "0")
    ntenv.setenv("NT_NORM_SPLIT_ROWS", "100000")
    q = nt.nt_plan_launch(WS_CODE[op], M, N, nt.NT_F32, True)
    assert (q["split"], q["cooperative"]) == (3, 0), q
    say(f"case two-kernel split large grid {op} {dt} M={M} N={N} P={q['row_chunks']}")
    b, bm, br = run_ws(op, x_t, dt, p0_t, p1_t)
    if (q["row_chunks"], q["chunks_per_lane"]) == (p["row_chunks"], p["chunks_per_lane"]):
        # same chunks: the same bits
        assert np.array_equal(to_host_bits(b, dt), ab)
        if op == "layernorm":
            assert torch.equal(am, bm) and torch.equal(ar, br)
    else:
        # fp32 RMSNorm's one pass takes 64 KiB chunks, the two kernels 32 KiB: the oracle's bar
        check_output(to_host_bits(b, dt)[rows], ref, dt, f"two-kernel large grid {op}")
