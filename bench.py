#!/usr/bin/env python3
"""Throughput of the fused row reductions on one MI355X.

One step = one pass over the five row-reduction workloads (all on-chip steps
of the method: launch planning, 16-byte row loads, widening, row reductions,
epilogue, rounding stores, and the split online softmax for vocab-width rows):

  softmax   fp32  1024 x 781       single pass, masked ragged tail, 4-byte-aligned rows
  LayerNorm fp16  4096 x 4096      y + mean + rstd
  RMSNorm   bf16  16384 x 8192
  softmax   bf16  131072 x 4096    causal attention scores (-inf above the diagonal)
  softmax   fp32  64 x 262144      vocab-width rows: split online max/denominator path

Inputs are generated on the host from fixed seeds, copied to HBM before the
timed region, and each kernel is launched on torch's current stream through
the C ABI.  value = algorithmic bytes of one step / time of one step (GB/s),
timed over exactly K steps between two HIP events on that stream; inside
that region only the dominant kernel's launches are bracketed by events (its
roofline fraction).  A separate, untimed breakdown pass with events around
every launch gives each workload's own GB/s (per_workload).

Prints ONE JSON line.  Flags: --gpus (only 1 is supported), --steps, --warmup
(at least that many untimed passes before each timed pass, and more until
--warm-ms of wall time, default 200, have passed with the GPU busy),
--only NAME[,NAME] (time a subset, rotating buffer sets so the 256 MiB
Infinity Cache cannot serve them), --no-cpu-baseline, --no-next (skip the
next rows -- fused residual add + norm, the causal softmax entry, the
attention forward -- which are timed after the suite and reported under
next_rows, outside value); --attention (only the attention forward row);
--calibrate (the reference streams at 1 GiB: copy, read-only and write-only
at 1, 2, 4 and 8 chunks per lane: attainable bandwidth, and the counter
calibration) and --copy-at-sizes (each workload's kernel beside copies of its
bytes, in one run) and --sweep
(fp32 softmax and RMSNorm over the pages' benchmark widths, beside torch's
softmax; --sweep-md FILE writes a summary) and --sweep-ops f32|f16|bf16 (all
three ops over those widths in one type, each beside torch's kernel) replace
the suite.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak, GB/s
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix peak, TFLOP/s
METRIC = "achieved HBM GB/s (and % of MI355X peak) for softmax/LayerNorm/RMSNorm rows"
CACHE_BYTES = 256 << 20     # Infinity Cache (MALL) size
# workload op -> nt_op code of nt_plan_launch
OP_CODES = {"softmax": 0, "layernorm": 1, "rmsnorm": 2, "add_layernorm": 3, "add_rmsnorm": 4, "softmax_causal": 5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits, dt, torch, np):
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()


def rows_aligned(w):
    """Rows start 16-byte aligned in a fresh tensor when a row is a whole
    number of 16-byte chunks (the allocator aligns the base)."""
    return (w.N * w.elem_bytes) % 16 == 0


class Job:
    """One workload resident in HBM, with R rotating buffer sets."""

    def __init__(self, w, data, R, torch, np, nt):
        self.w, self.R, self.nt = w, R, nt
        self.bytes = w.algorithmic_bytes()
        self.dt_code = {"f32": nt.NT_F32, "f16": nt.NT_F16, "bf16": nt.NT_BF16}[w.dt]
        x0 = to_dev(data["x"], w.dt, torch, np)
        self.x = [x0] + [x0.clone() for _ in range(R - 1)]
        self.y = [torch.empty_like(x0) for _ in range(R)]
        p0 = data.get("gamma", data.get("weight"))
        p1 = data.get("beta")
        self.p0 = None if p0 is None else to_dev(p0, w.dt, torch, np)
        self.p1 = None if p1 is None else to_dev(p1, w.dt, torch, np)
        self.mean = [torch.empty(w.M, dtype=torch.float32, device="cuda") for _ in range(R)]
        self.rstd = [torch.empty(w.M, dtype=torch.float32, device="cuda") for _ in range(R)]
        self.fused = w.op.startswith("add_")
        if self.fused:                               # fused add + norm: residual in, h out
            r0 = to_dev(data["residual"], w.dt, torch, np)
            self.r = [r0] + [r0.clone() for _ in range(R - 1)]
            self.h = [torch.empty_like(x0) for _ in range(R)]
        self.wsb = (nt.nt_softmax_workspace_bytes(w.M, w.N, self.dt_code)
                    if w.op in ("softmax", "softmax_causal") else 0)
        self.ws = torch.empty(max(self.wsb, 8), dtype=torch.uint8, device="cuda")
        self.i = 0
        self.starts, self.ends = [], []

    def launch(self, stream):
        w, nt, r = self.w, self.nt, self.i % self.R
        self.i += 1
        if w.op == "softmax":
            rc = nt.nt_softmax_rows(w.M, w.N, self.dt_code, self.x[r].data_ptr(), self.y[r].data_ptr(),
                                    self.ws.data_ptr(), self.wsb, stream)
        elif w.op == "softmax_causal":
            e = w.extra
            rc = nt.nt_softmax_causal_rows(w.M, w.N, self.dt_code, e["scale"], e["queries"], e["offset"],
                                           self.x[r].data_ptr(), self.y[r].data_ptr(), self.ws.data_ptr(), self.wsb,
                                           stream)
        elif w.op == "add_layernorm":
            rc = nt.nt_add_layernorm_rows(w.M, w.N, self.dt_code, w.eps, self.x[r].data_ptr(), self.r[r].data_ptr(),
                                          self.p0.data_ptr(), self.p1.data_ptr(), self.h[r].data_ptr(),
                                          self.y[r].data_ptr(), self.mean[r].data_ptr(), self.rstd[r].data_ptr(),
                                          stream)
        elif w.op == "add_rmsnorm":
            rc = nt.nt_add_rmsnorm_rows(w.M, w.N, self.dt_code, w.eps, self.x[r].data_ptr(), self.r[r].data_ptr(),
                                        self.p0.data_ptr(), self.h[r].data_ptr(), self.y[r].data_ptr(), stream)
        elif w.op == "layernorm":
            rc = nt.nt_layernorm_rows(w.M, w.N, self.dt_code, w.eps, self.x[r].data_ptr(), self.p0.data_ptr(),
                                      self.p1.data_ptr(), self.y[r].data_ptr(), self.mean[r].data_ptr(),
                                      self.rstd[r].data_ptr(), stream)
        else:
            rc = nt.nt_rmsnorm_rows(w.M, w.N, self.dt_code, w.eps, self.x[r].data_ptr(), self.p0.data_ptr(),
                                    self.y[r].data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"{w.name}: {nt.nt_status_string(rc)}")


def cpu_baseline(jobs, np, stride=1, check_every=1):
    """The oracle (as it stands) on every `stride`-th row of each workload
    (by default all rows: about 6 core-seconds per pass over the suite), on
    this host's cores: 1 warm-up and 3 timed runs, median.  The GPU output
    of the last launch is checked against the oracle on every
    `check_every`-th of those rows (by default every row; compared on
    blocks in a thread pool)."""
    import oracle
    from oracle import compare
    total_bytes, total_t, ok = 0, 0.0, True
    parts = []
    checked_rows = 0
    for j in jobs:
        w, data = j.w, j.data
        rows = np.arange(0, w.M, stride)
        xs = np.ascontiguousarray(data["x"][rows])
        p0 = data.get("gamma", data.get("weight"))
        p1 = data.get("beta")

        def run():
            if w.op == "softmax":
                return oracle.softmax(xs, w.dt)
            if w.op == "layernorm":
                return oracle.layernorm(xs, w.dt, w.eps, gamma=p0, beta=p1)[0]
            return oracle.rmsnorm(xs, w.dt, w.eps, weight=p0)

        ref = run()                                  # warm-up
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            run()
            ts.append(time.perf_counter() - t0)
        t = statistics.median(ts)
        e = w.elem_bytes
        b = 2 * len(rows) * w.N * e + (2 * w.N * e + 8 * len(rows) if w.op == "layernorm" else 0) \
            + (w.N * e if w.op == "rmsnorm" else 0)
        total_bytes += b
        total_t += t
        parts.append(f"{w.name}: {len(rows)} of {w.M} rows")
        # parity of the GPU output on the same rows (every check_every-th)
        y = j.y[0].cpu()             # every buffer set holds the same input
        refs = ref[::check_every]
        checked_rows += refs.shape[0]
        if w.dt == "f32":
            gb = y.numpy()[::stride][::check_every].view(np.uint32)
            rel, quanta = compare.f32_errors_threaded(gb, refs)
            good = rel <= 1e-5 and quanta <= 1.0
        else:
            import torch
            gb = y.view(torch.int16).numpy()[::stride][::check_every].view(np.uint16)
            good = compare.max_ulp_distance(gb, refs, w.dt) <= 1
        ok = ok and good
        del ref, refs, gb, y
    threads = oracle.num_threads()
    # one thread on the small softmax workload (every row), then back
    single = None
    c1 = next((j for j in jobs if j.w.op == "softmax" and j.w.dt == "f32" and j.w.M * j.w.N <= 1 << 20), None)
    if c1 is not None:
        oracle.set_num_threads(1)
        try:
            oracle.softmax(c1.data["x"], "f32")
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.softmax(c1.data["x"], "f32")
                ts.append(time.perf_counter() - t0)
        finally:
            oracle.set_num_threads(threads)
        t1 = statistics.median(ts)
        single = {"workload": c1.w.name, "seconds": round(t1, 5),
                  "GBps": round(c1.bytes / t1 / 1e9, 3)}
    return {"value": round(total_bytes / total_t / 1e9, 3), "unit": "GB/s", "cores": threads,
            "cpu_model": cpu_model(), "single_thread": single,
            "kind": "oracle",
            "sample": (("all rows" if stride == 1 else f"every {stride}th row") +
                       f" of each workload ({'; '.join(parts)}); median of 3 timed runs after 1 warm-up; "
                       f"fp64 C with OpenMP over rows on {threads} threads"),
            "seconds": round(total_t, 3), "core_seconds": round(total_t * threads, 2),
            "gpu_parity_on_sample": bool(ok), "gpu_parity_rows_checked": int(checked_rows)}


def warm_up(step, count, min_ms, torch):
    """At least `count` calls of `step`, and more until `min_ms` of wall time
    have passed with the GPU kept busy: after the host has prepared inputs for
    seconds, the first launches run below the steady clocks (measured: the
    first ~50 causal-entry launches 5% slower than the next)."""
    t0 = time.perf_counter()
    n = 0
    while n < count or (time.perf_counter() - t0) * 1e3 < min_ms:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def pct(durs, q):
    """q-th percentile (nearest rank) of a list of durations."""
    d = sorted(durs)
    return d[min(len(d) - 1, max(0, int(round(q / 100.0 * (len(d) - 1)))))]


def traffic_for(kernel_name, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from row_wise_reductions_amd.rocprof_summary import kernel_source_hash
    if t.get("source_hash") != kernel_source_hash():
        return None
    e = t.get("workloads", {}).get(kernel_name)
    return None if e is None else e.get("hbm_bytes_per_call")


def _ntcal():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "row_wise_reductions_amd", "libntcal.so"))
    lib.ntcal_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    lib.ntcal_stream.restype = ctypes.c_int
    return lib


# Reference streams of libntcal.so: (name, kind, chunks per lane, sc1).
# kind 0 copy (read + write), 1 read only, 2 fill (write only).
CALIB_VARIANTS = [(f"{('copy', 'read', 'fill')[kind]} K={k}" + (" nt sc1" if sc1 else (" nt" if kind != 1 else "")),
                   kind, k, sc1)
                  for kind in (0, 1, 2) for k in (1, 2, 4, 8) for sc1 in ((0, 1) if kind != 1 else (0,))]
NEVER = 0x9E3779B9          # the read stream stores its fold only if it equals this


def _timed_median(fn, steps, warmup, torch, min_ms=200.0):
    warm_up(lambda: fn(0), warmup, min_ms, torch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in evs)


def calibrate_copy(torch, steps, warmup, nbytes=1 << 30):
    """Attainable-bandwidth references at 1 GiB, rotating 4 buffer pairs:
    libntcal.so's copy, read-only and write-only streams with 1, 2, 4 and 8
    16-byte chunks per lane in flight, with non-temporal stores and with the
    device-scope streaming stores (nt sc1) of the row kernels; torch's own
    copy_ beside them.  GB/s counts the bytes each moves (copy: read +
    written).  Event-timed medians; under rocprofv3 --kernel-trace the same
    launches give kernel durations."""
    lib = _ntcal()
    n = nbytes // 4
    src = [torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(4)]
    dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(4)]
    sh = torch.cuda.current_stream().cuda_stream
    out = {"calibration": "libntcal.so reference streams at 1 GiB: copy (read + write), read only, fill (write "
                          "only); K 16-byte chunks per lane in flight; stores non-temporal (nt) or device-scope "
                          "streaming (nt sc1)",
           "bytes": nbytes, "variants": []}
    for name, kind, k, sc1 in CALIB_VARIANTS:
        def one(i, kind=kind, k=k, sc1=sc1):
            rc = lib.ntcal_stream(kind, k, sc1, dst[i % 4].data_ptr(), src[i % 4].data_ptr(), nbytes,
                                  0x3F800000 if kind == 2 else NEVER, sh)
            assert rc == 0, rc
        ms = _timed_median(one, steps, warmup, torch)
        moved = (2 if kind == 0 else 1) * nbytes
        out["variants"].append({"name": name, "kind": kind, "K": k, "sc1": sc1, "median_ms": round(ms, 5),
                                "GBps": round(moved / (ms * 1e-3) / 1e9, 1)})
        log(f"[calibrate] {name}: {out['variants'][-1]['GBps']} GB/s")
    ms = _timed_median(lambda i: dst[i % 4].copy_(src[i % 4]), steps, warmup, torch)
    out["torch_copy_median_ms"] = round(ms, 5)
    out["torch_copy_GBps"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    best = max((v for v in out["variants"] if v["kind"] == 0), key=lambda v: v["GBps"])
    out["best_copy"] = best["name"]
    out["best_copy_GBps"] = best["GBps"]
    print(json.dumps(out), flush=True)


COPY_AT_SIZES = [("copy K=1 nt", 0, 1, 0), ("copy K=1 nt sc1", 0, 1, 1), ("copy K=2 nt sc1", 0, 2, 1),
                 ("copy K=4 nt sc1", 0, 4, 1)]


def copy_at_sizes(torch, steps, warmup, wls):
    """Each workload's own kernel and reference copies of its bytes (read
    M*N*e, write M*N*e; libntcal.so, 1, 2 and 4 chunks per lane), launched in
    the same run, rotating buffer sets of >= 1 GiB so the Infinity Cache
    cannot serve them: under rocprofv3 --kernel-trace both get kernel
    durations on the same clock (the copies are told apart by their grid
    sizes).  Also event-timed here; median of `steps` launches."""
    import numpy as np

    import row_wise_reductions_amd as nt
    lib = _ntcal()
    sh = torch.cuda.current_stream().cuda_stream
    out = {"copy_at_sizes": "each workload's kernel, and libntcal.so copies of its read bytes", "workloads": []}
    for w in wls:
        nb = w.M * w.N * w.elem_bytes // 16 * 16
        R = max(1, -(-(1 << 30) // (2 * nb)))
        row = {"workload": w.name, "bytes_read": nb, "bytes_written": nb, "buffer_sets": R,
               "algorithmic_bytes": w.algorithmic_bytes()}
        data = w.make()
        job = Job(w, data, R, torch, np, nt)
        ms = _timed_median(lambda i: job.launch(sh), steps, warmup, torch)
        row["kernel_median_ms"] = round(ms, 5)
        row["kernel_GBps"] = round(w.algorithmic_bytes() / (ms * 1e-3) / 1e9, 1)
        del job, data
        src = [torch.ones(nb // 4, dtype=torch.float32, device="cuda") for _ in range(R)]
        dst = [torch.empty(nb // 4, dtype=torch.float32, device="cuda") for _ in range(R)]
        row["copies"] = []
        for name, kind, k, sc1 in COPY_AT_SIZES:
            def one(i, k=k, sc1=sc1):
                assert lib.ntcal_stream(0, k, sc1, dst[i % R].data_ptr(), src[i % R].data_ptr(), nb, 0, sh) == 0
            ms = _timed_median(one, steps, warmup, torch)
            row["copies"].append({"name": name, "K": k, "sc1": sc1, "grid": -(-(nb // 16) // (256 * k)),
                                  "median_ms": round(ms, 5), "GBps": round(2 * nb / (ms * 1e-3) / 1e9, 1)})
        log(f"[copy at sizes] {w.name}: kernel {row['kernel_median_ms']} ms, copies " +
            ", ".join(f"{c['name']} {c['median_ms']}" for c in row["copies"]))
        out["workloads"].append(row)
        del src, dst
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


SWEEP_M = 4096
SWEEP_N = [128 * i for i in range(2, 100)]      # the pages' GB/s harness: M = 4096, N = 128 i


def width_sweep(torch, steps, warmup, md_path=None):
    """Launch-table check over the widths of the pages' benchmark harness
    ("Portable Triton Kernels", "Benchmark Harness Template": fp32 softmax,
    M = 4096, N = 128*i for i = 2..99, GB/s = 2*numel*4 / time, against
    torch's softmax), plus RMSNorm fp32 (weight present) on the same widths.
    Inputs rotate through 1 GiB pools so the Infinity Cache cannot serve
    them; event-timed median of `steps` launches after `warmup`."""
    import row_wise_reductions_amd as nt
    M = SWEEP_M
    pool = 1 << 28                                   # floats: 1 GiB
    gen = torch.Generator(device="cuda").manual_seed(7)
    px = torch.randn(pool, device="cuda", generator=gen)
    py = torch.empty(pool, device="cuda")
    w = torch.randn(max(SWEEP_N), device="cuda", generator=gen) * 0.3 + 1.0
    sh = torch.cuda.current_stream().cuda_stream
    rows = []

    def timed(fn, R):
        for i in range(warmup):
            fn(i % R)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, b) in enumerate(evs):
            a.record()
            fn(i % R)
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in evs)

    for N in SWEEP_N:
        n = M * N
        R = pool // n
        xs = [px[i * n:(i + 1) * n].view(M, N) for i in range(R)]
        ys = [py[i * n:(i + 1) * n].view(M, N) for i in range(R)]

        def ours(i):
            assert nt.nt_softmax_rows(M, N, nt.NT_F32, xs[i].data_ptr(), ys[i].data_ptr(), None, 0, sh) == 0

        def theirs(i):
            torch.softmax(xs[i], dim=-1)

        def rms(i):
            assert nt.nt_rmsnorm_rows(M, N, nt.NT_F32, 1e-6, xs[i].data_ptr(), w.data_ptr(), ys[i].data_ptr(),
                                      sh) == 0

        ms_ours, ms_torch, ms_rms = timed(ours, R), timed(theirs, R), timed(rms, R)
        p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, M, N, nt.NT_F32, True)
        gb = 2 * n * 4 / 1e9
        rows.append({"N": N, "softmax_ms": round(ms_ours, 5), "softmax_GBps": round(gb / (ms_ours * 1e-3), 1),
                     "torch_softmax_GBps": round(gb / (ms_torch * 1e-3), 1),
                     "rmsnorm_GBps": round((gb + N * 4 / 1e9) / (ms_rms * 1e-3), 1),
                     "shape": f"{p['waves_per_row']}x{p['chunks_per_lane']}"})
        log(f"[sweep] N={N}: softmax {rows[-1]['softmax_GBps']} GB/s, torch {rows[-1]['torch_softmax_GBps']}, "
            f"rmsnorm {rows[-1]['rmsnorm_GBps']}")
    out = {"sweep": "fp32 softmax and RMSNorm, M = 4096, N = 128 i (i = 2..99)", "M": M, "points": rows}
    print(json.dumps(out), flush=True)
    if md_path:
        lines = ["# Width sweep: fp32 softmax and RMSNorm, M = 4096, N = 128 i (i = 2..99)", "",
                 "Command (repository root, GPU host):", "",
                 f"    python3 bench.py --sweep --steps {steps} --warmup {warmup} --sweep-md {md_path}", "",
                 "The widths of the pages' GB/s benchmark harness; GB/s = bytes read + written / median event-timed "
                 "launch, inputs rotating through 1 GiB pools.  `torch` is torch.softmax on the same buffers.", "",
                 "| N | launch shape (W x K) | softmax us | softmax GB/s | torch softmax GB/s | ratio | "
                 "RMSNorm GB/s |", "|---|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| {r['N']} | {r['shape']} | {r['softmax_ms'] * 1000:.2f} | {r['softmax_GBps']} | "
                         f"{r['torch_softmax_GBps']} | {r['softmax_GBps'] / r['torch_softmax_GBps']:.2f} | "
                         f"{r['rmsnorm_GBps']} |")
        ratios = [r["softmax_GBps"] / r["torch_softmax_GBps"] for r in rows]
        lines += ["", f"softmax / torch: min {min(ratios):.2f}, median {statistics.median(ratios):.2f}, "
                      f"max {max(ratios):.2f} over {len(rows)} widths.", ""]
        with open(md_path, "w") as f:
            f.write("\n".join(lines))


def op_sweep(torch, dt, steps, warmup, md_path=None):
    """Every op over the widths of the pages' harness (M = 4096, N = 128 i,
    i = 2..99) in one element type, each beside torch's own kernel on the same
    buffers (torch.softmax, F.rms_norm, F.layer_norm with weight and bias):
    the launch table of each op across widths.  GB/s = the op's algorithmic
    bytes (rows in and out, parameter vectors, LayerNorm's mean and rstd) /
    median event-timed launch; torch is credited with the same bytes."""
    import torch.nn.functional as F

    import row_wise_reductions_amd as nt
    M = SWEEP_M
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    code = {"f32": nt.NT_F32, "f16": nt.NT_F16, "bf16": nt.NT_BF16}[dt]
    e = 4 if dt == "f32" else 2
    pool = (1 << 30) // e
    gen = torch.Generator(device="cuda").manual_seed(11)
    px = torch.randn(pool, device="cuda", generator=gen).to(tdt)
    py = torch.empty(pool, device="cuda", dtype=tdt)
    g = (torch.randn(max(SWEEP_N), device="cuda", generator=gen) * 0.3 + 1.0).to(tdt)
    b = (torch.randn(max(SWEEP_N), device="cuda", generator=gen) * 0.3).to(tdt)
    mean = torch.empty(M, device="cuda")
    rstd = torch.empty(M, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream

    def timed(fn, R):
        warm_up(lambda: fn(0), warmup, 20.0, torch)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, bb) in enumerate(evs):
            a.record()
            fn(i % R)
            bb.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(bb) for a, bb in evs)

    def ok(rc):
        if rc != 0:
            raise RuntimeError(nt.nt_status_string(rc))

    rows = []
    for N in SWEEP_N:
        n = M * N
        R = pool // n
        xs = [px[i * n:(i + 1) * n].view(M, N) for i in range(R)]
        ys = [py[i * n:(i + 1) * n].view(M, N) for i in range(R)]
        gN, bN = g[:N], b[:N]
        fns = {
            "softmax": lambda i: ok(nt.nt_softmax_rows(M, N, code, xs[i].data_ptr(), ys[i].data_ptr(), None, 0,
                                                       sh)),
            "torch_softmax": lambda i: torch.softmax(xs[i], dim=-1),
            "rmsnorm": lambda i: ok(nt.nt_rmsnorm_rows(M, N, code, 1e-6, xs[i].data_ptr(), gN.data_ptr(),
                                                       ys[i].data_ptr(), sh)),
            "torch_rmsnorm": lambda i: F.rms_norm(xs[i], (N,), gN, 1e-6),
            "layernorm": lambda i: ok(nt.nt_layernorm_rows(M, N, code, 1e-5, xs[i].data_ptr(), gN.data_ptr(),
                                                           bN.data_ptr(), ys[i].data_ptr(), mean.data_ptr(),
                                                           rstd.data_ptr(), sh)),
            "torch_layernorm": lambda i: F.layer_norm(xs[i], (N,), gN, bN, 1e-5),
        }
        gb = {"softmax": 2 * n * e, "rmsnorm": 2 * n * e + N * e, "layernorm": 2 * n * e + 2 * N * e + 8 * M}
        r = {"N": N}
        for k, fn in fns.items():
            ms = timed(fn, R)
            r[k + "_GBps"] = round(gb[k.replace("torch_", "")] / (ms * 1e-3) / 1e9, 1)
        for op, c in (("softmax", nt.NT_OP_SOFTMAX), ("rmsnorm", nt.NT_OP_RMSNORM), ("layernorm", nt.NT_OP_LAYERNORM)):
            p = nt.nt_plan_launch(c, M, N, code, True)
            r[op + "_plan"] = ("split" if p["split"] == 1 else "looped" if p["split"] == 2 else
                               f"{p['waves_per_row']}x{p['chunks_per_lane']}" + (" p" if p["persistent"] else ""))
        rows.append(r)
        log(f"[op sweep {dt}] N={N}: " + ", ".join(f"{k} {v}" for k, v in r.items() if k.endswith("GBps")))
    out = {"op_sweep": f"{dt} softmax, RMSNorm, LayerNorm, M = 4096, N = 128 i (i = 2..99)", "points": rows}
    print(json.dumps(out), flush=True)
    if md_path:
        lines = [f"# Width sweep of every op: {dt}, M = 4096, N = 128 i (i = 2..99)", "",
                 "Command (repository root, GPU host):", "",
                 f"    python3 bench.py --sweep-ops {dt} --steps {steps} --warmup {warmup} --sweep-md {md_path}", "",
                 "GB/s = the op's algorithmic bytes / median event-timed launch, inputs rotating through a 1 GiB pool; "
                 "torch (torch.softmax, F.rms_norm, F.layer_norm with weight and bias, on the same buffers) is credited "
                 "with the same bytes.  Plan: W x K of the single-pass kernel (p: persistent workgroups).", "",
                 "| N | softmax plan | softmax | torch | RMSNorm plan | RMSNorm | torch | LayerNorm plan | LayerNorm | "
                 "torch |", "|---|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| {r['N']} | {r['softmax_plan']} | {r['softmax_GBps']} | {r['torch_softmax_GBps']} | "
                         f"{r['rmsnorm_plan']} | {r['rmsnorm_GBps']} | {r['torch_rmsnorm_GBps']} | "
                         f"{r['layernorm_plan']} | {r['layernorm_GBps']} | {r['torch_layernorm_GBps']} |")
        lines.append("")
        for op in ("softmax", "rmsnorm", "layernorm"):
            q = [r[op + "_GBps"] / r["torch_" + op + "_GBps"] for r in rows]
            lines.append(f"{op} / torch: min {min(q):.2f}, median {statistics.median(q):.2f}, max {max(q):.2f} "
                         f"over {len(rows)} widths.  ")
        lines.append("")
        with open(md_path, "w") as f:
            f.write("\n".join(lines))


WIDE_NORM_CASES = (("bf16", 32768), ("bf16", 262144), ("bf16", 1 << 20), ("f32", 65536), ("f32", 262144))
WIDE_NORM_M = (4, 16, 64, 256, 1024, 2048)


def wide_norm_sweep(torch, steps, warmup, md_path=None):
    """LayerNorm and RMSNorm on rows too wide for one pass (64 KiB to 2 MiB),
    few to many rows: the split norm (the workspace entry points, split
    forced at every row count), the looped one-workgroup-per-row kernel (the
    plain entry points) and torch (F.layer_norm, F.rms_norm), on the same
    buffers, rotating through a 1 GiB pool.  GB/s = algorithmic bytes (rows
    in and out, parameter vectors, LayerNorm's mean and rstd) / median
    event-timed launch.  `plan` is what the workspace entry point picks by
    itself at that row count."""
    import torch.nn.functional as F

    import row_wise_reductions_amd as nt

    def timed(fn, R):
        warm_up(lambda: fn(0), warmup, 20.0, torch)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, bb) in enumerate(evs):
            a.record()
            fn(i % R)
            bb.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(bb) for a, bb in evs)

    def ok(rc):
        if rc != 0:
            raise RuntimeError(nt.nt_status_string(rc))

    sh = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device="cuda").manual_seed(13)
    rows = []
    for dt, N in WIDE_NORM_CASES:
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dt]
        code = {"f32": nt.NT_F32, "bf16": nt.NT_BF16}[dt]
        e = 4 if dt == "f32" else 2
        pool = (1 << 30) // e
        px = torch.randn(pool, device="cuda", generator=gen).to(tdt)
        py = torch.empty(pool, device="cuda", dtype=tdt)
        g = (torch.randn(N, device="cuda", generator=gen) * 0.3 + 1.0).to(tdt)
        b = (torch.randn(N, device="cuda", generator=gen) * 0.3).to(tdt)
        for M in WIDE_NORM_M:
            n = M * N
            if n > pool:
                continue
            R = pool // n
            xs = [px[i * n:(i + 1) * n].view(M, N) for i in range(R)]
            ys = [py[i * n:(i + 1) * n].view(M, N) for i in range(R)]
            mean = torch.empty(M, device="cuda")
            rstd = torch.empty(M, device="cuda")
            r = {"dt": dt, "N": N, "M": M}
            for op, opc in (("layernorm", nt.NT_OP_LAYERNORM), ("rmsnorm", nt.NT_OP_RMSNORM)):
                wop = nt.NT_OP_LAYERNORM_WS if op == "layernorm" else nt.NT_OP_RMSNORM_WS
                p = nt.nt_plan_launch(wop, M, N, code, True)
                r[op + "_plan"] = ({0: "single pass", 2: "looped"}.get(p["split"]) or
                                   ("split, one pass" if p["cooperative"] else "split, two kernels"))
                with nt.override(NT_NORM_SPLIT_ROWS=str(1 << 40)):
                    wsb = nt.nt_norm_workspace_bytes(opc, M, N, code)
                    ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device="cuda")
                    if op == "layernorm":
                        split = lambda i: ok(nt.nt_layernorm_rows_ws(  # noqa: E731
                            M, N, code, 1e-5, xs[i].data_ptr(), g.data_ptr(), b.data_ptr(), ys[i].data_ptr(),
                            mean.data_ptr(), rstd.data_ptr(), ws.data_ptr(), wsb, sh))
                    else:
                        split = lambda i: ok(nt.nt_rmsnorm_rows_ws(  # noqa: E731
                            M, N, code, 1e-6, xs[i].data_ptr(), g.data_ptr(), ys[i].data_ptr(), ws.data_ptr(),
                            wsb, sh))
                    ms_split = timed(split, R)
                    with nt.override(NT_COOP="0"):
                        ms_split2 = timed(split, R)
                if op == "layernorm":
                    looped = lambda i: ok(nt.nt_layernorm_rows(  # noqa: E731
                        M, N, code, 1e-5, xs[i].data_ptr(), g.data_ptr(), b.data_ptr(), ys[i].data_ptr(),
                        mean.data_ptr(), rstd.data_ptr(), sh))
                    theirs = lambda i: F.layer_norm(xs[i], (N,), g, b, 1e-5)  # noqa: E731
                    gb = 2 * n * e + 2 * N * e + 8 * M
                else:
                    looped = lambda i: ok(nt.nt_rmsnorm_rows(  # noqa: E731
                        M, N, code, 1e-6, xs[i].data_ptr(), g.data_ptr(), ys[i].data_ptr(), sh))
                    theirs = lambda i: F.rms_norm(xs[i], (N,), g, 1e-6)  # noqa: E731
                    gb = 2 * n * e + N * e
                for k, ms in (("split", ms_split), ("split2", ms_split2), ("looped", timed(looped, R)),
                              ("torch", timed(theirs, R))):
                    r[f"{op}_{k}_us"] = round(ms * 1e3, 1)
                    r[f"{op}_{k}_GBps"] = round(gb / (ms * 1e-3) / 1e9, 1)
            rows.append(r)
            log(f"[wide norms] {dt} N={N} M={M}: " + ", ".join(f"{k} {v}" for k, v in r.items() if k.endswith("GBps")))
        del px, py
    print(json.dumps({"wide_norm_sweep": "LayerNorm / RMSNorm, rows of 64 KiB to 2 MiB", "points": rows}), flush=True)
    if md_path:
        lines = ["# Wide-row norms: split vs looped vs torch", "", "Command (repository root, GPU host):", "",
                 f"    python3 bench.py --sweep-wide-norms --steps {steps} --warmup {warmup} --sweep-md {md_path}", "",
                 "GB/s = algorithmic bytes (rows in and out, parameter vectors, LayerNorm's mean and rstd) / median "
                 "event-timed launch, inputs rotating through a 1 GiB pool.  split: nt_*_rows_ws with the split "
                 "forced at every row count, the row's chunks on many workgroups: in one pass where the planner allows "
                 "it (at most 16 chunks of 32 KiB per row, at least 2048 workgroups, not 16-bit LayerNorm), else two "
                 "kernels; 2k: the same with NT_COOP=0 (two kernels, x read twice); "
                 "looped: the plain entry point (one workgroup per row, the row streamed twice); torch: "
                 "F.layer_norm / F.rms_norm on the same buffers.  plan: what nt_*_rows_ws picks by itself.", "",
                 "| type | N | M | LN plan | LN split | LN 2k | LN looped | LN torch | RMS plan | RMS split | RMS 2k | "
                 "RMS looped | RMS torch |", "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| {r['dt']} | {r['N']} | {r['M']} | {r['layernorm_plan']} | {r['layernorm_split_GBps']} | "
                         f"{r['layernorm_split2_GBps']} | {r['layernorm_looped_GBps']} | {r['layernorm_torch_GBps']} | "
                         f"{r['rmsnorm_plan']} | {r['rmsnorm_split_GBps']} | {r['rmsnorm_split2_GBps']} | "
                         f"{r['rmsnorm_looped_GBps']} | {r['rmsnorm_torch_GBps']} |")
        lines.append("")
        with open(md_path, "w") as f:
            f.write("\n".join(lines))


WIDE_TRAFFIC = ("f32", 2048, 65536)      # 512 MiB in, 512 MiB out: twice the Infinity Cache


def wide_norm_traffic(torch, steps):
    """The three forms of a wide-row RMSNorm on one large matrix (fp32
    2048 x 65536, every parameter present), `steps` launches each, inputs
    alternating between two 512 MiB buffers so no launch finds its rows in
    the Infinity Cache: the one-pass split norm (norm_coop), the two-kernel
    split norm (norm_split_partial + norm_split_finalize: NT_COOP=0) and the
    looped kernel (row_looped: the plain entry point).  Meant to run under
    rocprofv3, whose counters then tell how often each form reads x; prints
    each form's median event-timed launch."""
    import row_wise_reductions_amd as nt
    dt, M, N = WIDE_TRAFFIC
    code = nt.NT_F32
    gen = torch.Generator(device="cuda").manual_seed(17)
    xs = [torch.randn(M, N, device="cuda", generator=gen) for _ in range(2)]
    y = torch.empty_like(xs[0])
    w = torch.randn(N, device="cuda", generator=gen) * 0.3 + 1
    sh = torch.cuda.current_stream().cuda_stream

    def ok(rc):
        if rc != 0:
            raise RuntimeError(nt.nt_status_string(rc))

    forms = (("one pass", {}, True), ("two kernels", {"NT_COOP": "0", "NT_NORM_SPLIT_ROWS": str(1 << 40)}, True),
             ("looped", {}, False))
    out = {}
    for name, env, with_ws in forms:
        with nt.override(**env):
            p = nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS if with_ws else nt.NT_OP_RMSNORM, M, N, code, True)
            wsb = int(p["workspace_bytes"])          # this form's own workspace (the two use other chunks)
            ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device="cuda")
            evs = []
            for i in range(steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                if with_ws:
                    ok(nt.nt_rmsnorm_rows_ws(M, N, code, 1e-6, xs[i % 2].data_ptr(), w.data_ptr(), y.data_ptr(),
                                             ws.data_ptr(), wsb, sh))
                else:
                    ok(nt.nt_rmsnorm_rows(M, N, code, 1e-6, xs[i % 2].data_ptr(), w.data_ptr(), y.data_ptr(), sh))
                b.record()
                evs.append((a, b))
            torch.cuda.synchronize()
        out[name] = {"plan": {k: p[k] for k in ("split", "cooperative", "waves_per_row", "chunks_per_lane",
                                               "row_chunks")},
                     "median_us": round(statistics.median(a.elapsed_time(b) for a, b in evs) * 1e3, 2)}
    print(json.dumps({"wide_norm_traffic": f"RMSNorm {dt} {M}x{N}", "algorithmic_bytes": 2 * M * N * 4 + N * 4,
                      "forms": out}), flush=True)


def attention_next_row(torch, np, nt, steps, warmup, warm_ms, stream):
    """The attention forward at 32 heads x 4096 queries x 4096 keys x 128,
    bf16, causal (workloads.ATTENTION): event-timed launches on the bench
    stream; its roofline against the matrix-core peak (algorithmic flops:
    4 D per visible query-key pair, Q K^T and P V) and its HBM bytes (q, k,
    v read, o written).  Parity is the GPU tests' (test_gpu_attention.py)."""
    import workloads
    w = workloads.ATTENTION
    BH, Lq, Lk, D, dt = w["BH"], w["Lq"], w["Lk"], w["D"], w["dt"]
    q, k, v = workloads.attention_inputs(BH, Lq, Lk, D, dt)
    q_t, k_t, v_t = (to_dev(x.reshape(BH * x.shape[1], D), dt, torch, np) for x in (q, k, v))
    o = torch.empty_like(q_t)
    sh = stream.cuda_stream

    def launch():
        rc = nt.nt_attention_fwd(BH, Lq, Lk, D, nt.NT_BF16, w["scale"], int(w["causal"]), w["offset"], q_t.data_ptr(),
                                 k_t.data_ptr(), v_t.data_ptr(), o.data_ptr(), sh)
        if rc != 0:
            raise RuntimeError(f"attention: {nt.nt_status_string(rc)}")
    warm_up(launch, warmup, warm_ms, torch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    durs = [a.elapsed_time(b) for a, b in evs]
    avg = sum(durs) / len(durs)
    pairs = workloads.attention_visible_pairs(BH, Lq, Lk, w["causal"], w["offset"])
    flops = 4 * D * pairs
    tflops = flops / (avg * 1e-3) / 1e12
    hbm = 4 * BH * Lq * D * 2
    return {"workload": w["name"], "op": "attention_fwd", "dtype": dt, "heads": BH, "Lq": Lq, "Lk": Lk, "D": D,
            "causal": w["causal"], "scale": w["scale"], "visible_pairs": pairs, "flops": flops,
            "avg_ms": round(avg, 5), "median_ms": round(statistics.median(durs), 5),
            "p10_ms": round(pct(durs, 10), 5), "p90_ms": round(pct(durs, 90), 5),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "flops_per_launch": flops},
            "hbm_bytes": hbm, "GBps": round(hbm / (avg * 1e-3) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--sweep-ops", dest="sweep_ops", choices=["f32", "f16", "bf16"], default=None,
                    help="softmax, RMSNorm and LayerNorm over the pages' widths in one type, beside torch")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-ms", dest="warm_ms", type=float, default=200.0,
                    help="minimum wall time of the untimed warm-up before each timed pass")
    ap.add_argument("--only", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the next rows (timed after the suite, not part of value)")
    ap.add_argument("--calibrate", action="store_true",
                    help="time the plain 1 GiB streaming copy (and torch copy_) instead")
    ap.add_argument("--sweep", action="store_true",
                    help="fp32 softmax / RMSNorm over the pages' benchmark widths (M=4096, N=128 i), vs torch")
    ap.add_argument("--sweep-wide-norms", dest="sweep_wide_norms", action="store_true",
                    help="LayerNorm / RMSNorm on rows of 64 KiB to 2 MiB: split vs looped vs torch")
    ap.add_argument("--wide-norm-traffic", dest="wide_norm_traffic", action="store_true",
                    help="the three forms of a wide-row RMSNorm, for rocprofv3 counters (x read once or twice)")
    ap.add_argument("--sweep-md", default=None, help="with a sweep: also write a markdown summary here")
    ap.add_argument("--attention", action="store_true",
                    help="time only the attention forward row (32 x 4096 x 4096 x 128 bf16 causal)")
    ap.add_argument("--copy-at-sizes", action="store_true",
                    help="time the plain streaming copy at each workload's byte count instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): rows are independent, so a "
              f"multi-GPU run would shard rows with no communication; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import row_wise_reductions_amd as nt
    import workloads

    nt.lib()   # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate:
        calibrate_copy(torch, args.steps, args.warmup)
        return
    if args.sweep:
        width_sweep(torch, args.steps, args.warmup, args.sweep_md)
        return
    if args.sweep_ops:
        op_sweep(torch, args.sweep_ops, args.steps, args.warmup, args.sweep_md)
        return
    if args.sweep_wide_norms:
        wide_norm_sweep(torch, args.steps, args.warmup, args.sweep_md)
        return
    if args.wide_norm_traffic:
        wide_norm_traffic(torch, args.steps)
        return
    if args.attention:
        print(json.dumps(attention_next_row(torch, np, nt, args.steps, args.warmup, args.warm_ms,
                                            torch.cuda.current_stream())), flush=True)
        return
    if args.copy_at_sizes:
        names = args.only.split(",") if args.only else [w.name for w in workloads.WORKLOADS]
        copy_at_sizes(torch, args.steps, args.warmup, [workloads.BY_NAME[n] for n in names])
        return
    names = args.only.split(",") if args.only else [w.name for w in workloads.WORKLOADS]
    suite = args.only is None

    jobs = []
    for name in names:
        w = workloads.BY_NAME[name]
        t0 = time.perf_counter()
        data = w.make()
        # in the full suite the other workloads flush the Infinity Cache between
        # two launches of the same workload; alone, rotate buffer sets instead
        per_set = 2 * w.M * w.N * w.elem_bytes
        R = 1 if suite else max(1, -(-(4 * CACHE_BYTES) // per_set))
        j = Job(w, data, R, torch, np, nt)
        j.data = data
        jobs.append(j)
        log(f"[bench] {name}: generated + uploaded in {time.perf_counter() - t0:.1f}s (R={R})")

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    warm_steps = warm_up(lambda: [j.launch(sh) for j in jobs], args.warmup, args.warm_ms, torch)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # Breakdown pass (not the timed region): an event pair around every
    # launch gives each workload's own duration and picks the dominant kernel.
    for j in jobs:
        j.i = 0
        j.starts = [ev() for _ in range(args.steps)]
        j.ends = [ev() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for j in jobs:
            j.starts[s].record(stream)
            j.launch(sh)
            j.ends[s].record(stream)
    torch.cuda.synchronize()
    per = []
    for j in jobs:
        durs = [a.elapsed_time(b) for a, b in zip(j.starts, j.ends)]
        avg = sum(durs) / len(durs)
        per.append({"workload": j.w.name, "op": j.w.op, "dtype": j.w.dt, "M": j.w.M, "N": j.w.N,
                    "bytes": j.bytes, "avg_ms": round(avg, 5), "median_ms": round(statistics.median(durs), 5),
                    "p10_ms": round(pct(durs, 10), 5), "p90_ms": round(pct(durs, 90), 5),
                    "GBps": round(j.bytes / (avg * 1e-3) / 1e9, 1),
                    "frac_of_peak": round(j.bytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "frac_of_peak_median": round(j.bytes / (statistics.median(durs) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "plan": nt.nt_plan_launch(OP_CODES[j.w.op], j.w.M, j.w.N, j.dt_code, rows_aligned(j.w))})
    dom_i = max(range(len(jobs)), key=lambda i: per[i]["avg_ms"])
    dom_job = jobs[dom_i]

    # Timed region: exactly K steps between two events; inside it only the
    # dominant kernel's launches are bracketed (its roofline is measured live
    # here), so instrumentation adds no gaps between the other launches.
    d_starts = [ev() for _ in range(args.steps)]
    d_ends = [ev() for _ in range(args.steps)]
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        for j in jobs:
            if j is dom_job:
                d_starts[s].record(stream)
                j.launch(sh)
                d_ends[s].record(stream)
            else:
                j.launch(sh)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    dom_ms = sum(a.elapsed_time(b) for a, b in zip(d_starts, d_ends)) / args.steps

    total_bytes = sum(j.bytes for j in jobs)
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    dom = per[dom_i]
    achieved = dom["bytes"] / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_for(dom["workload"], dom["bytes"]),
                "kernel": dom["workload"], "avg_launch_ms": round(dom_ms, 5)}

    # Next rows (fused residual add + norm, causal softmax entry): timed on
    # their own after the timed region, not part of `value`; buffer sets
    # rotate past the cache.
    next_rows = []
    if suite and not args.no_next:
        for w in workloads.NEXT_WORKLOADS:
            data = w.make()
            per_set = (2 if w.op == "softmax_causal" else 4) * w.M * w.N * w.elem_bytes
            j = Job(w, data, max(1, -(-(4 * CACHE_BYTES) // per_set)), torch, np, nt)
            warm_up(lambda: j.launch(sh), args.warmup, args.warm_ms, torch)
            evs = [(ev(), ev()) for _ in range(args.steps)]
            torch.cuda.synchronize()
            for a, b in evs:
                a.record(stream)
                j.launch(sh)
                b.record(stream)
            torch.cuda.synchronize()
            durs = [a.elapsed_time(b) for a, b in evs]
            avg = sum(durs) / len(durs)
            op = OP_CODES[w.op]
            e = w.elem_bytes
            if w.op == "softmax_causal":     # the generic softmax reads the masked keys too
                base = {"baseline": "generic softmax of the -inf-masked rows", "baseline_bytes": 2 * w.M * w.N * e}
            else:                            # an add kernel, then the norm of its output
                base = {"baseline": "add, then norm (unfused)", "baseline_bytes": j.bytes + 2 * w.M * w.N * e}
            next_rows.append({"workload": w.name, "op": w.op, "dtype": w.dt, "M": w.M, "N": w.N,
                              "bytes": j.bytes, **base,
                              "avg_ms": round(avg, 5), "median_ms": round(statistics.median(durs), 5),
                              "p10_ms": round(pct(durs, 10), 5), "p90_ms": round(pct(durs, 90), 5),
                              "GBps": round(j.bytes / (avg * 1e-3) / 1e9, 1),
                              "frac_of_peak": round(j.bytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "frac_of_peak_median": round(j.bytes / (statistics.median(durs) * 1e-3) / 1e9 /
                                                           PEAK_HBM_GBS, 4),
                              "traffic": traffic_for(w.name, j.bytes),
                              "plan": nt.nt_plan_launch(op, w.M, w.N, j.dt_code, rows_aligned(w))})
            log(f"[bench] next row {w.name}: {next_rows[-1]['GBps']} GB/s")
            del j, data
        torch.cuda.empty_cache()
        next_rows.append(attention_next_row(torch, np, nt, args.steps, args.warmup, args.warm_ms, stream))
        log(f"[bench] next row {next_rows[-1]['workload']}: {next_rows[-1]['roofline']['achieved']} TFLOP/s")
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        cpu = cpu_baseline(jobs, np)
        log(f"[bench] cpu baseline in {time.perf_counter() - t0:.1f}s")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": ("row-reduction suite: softmax f32 1024x781, LayerNorm f16 4096x4096, "
                                "RMSNorm bf16 16384x8192, causal softmax bf16 131072x4096, "
                                "vocab softmax f32 64x262144") if suite else ",".join(names),
                   "bytes_per_step": total_bytes, "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
                   "wall_s_timed": round(wall, 4), "warmup_steps_run": warm_steps, "warmup_min_ms": args.warm_ms},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_workload": per,   # from the breakdown pass
        "next_rows": next_rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
