"""Summaries of rocprofv3 output for the row-reduction kernels.

Turns rocprofv3 CSV output into the short text summaries kept under
``profiles/`` and into ``profiles/traffic.json``, which bench.py reads for
the roofline ``traffic`` field.  Nothing here launches work on a GPU.

  python -m row_wise_reductions_amd.rocprof_summary stats DIR --cmd "..." --out FILE.md
      DIR holds *_kernel_stats.csv from `rocprofv3 --kernel-trace --stats
      --output-format csv` of bench.py: per-workload kernel calls and
      average durations.

  python -m row_wise_reductions_amd.rocprof_summary traffic --fetch DIR --write DIR \\
         --calib-fetch DIR --calib-write DIR --cmds FILE --md FILE.md --json FILE.json
      DIRs hold *_counter_collection.csv from `rocprofv3 --pmc FETCH_SIZE`
      and `--pmc WRITE_SIZE` runs of bench.py and of `bench.py --calibrate`.
      Counter values (KiB per dispatch) are scaled by what the same counter
      reads for the calibration copy of known size (1 GiB read + 1 GiB
      written), giving HBM bytes per call of each workload.

  python -m row_wise_reductions_amd.rocprof_summary kernels --fetch DIR --write DIR --calib-fetch DIR \\
         --calib-write DIR --trace DIR --groups "name=kernel+kernel;..." --bytes B --title T --cmds FILE --md FILE.md
      HBM bytes (scaled as above) and average durations per group of named
      kernels in a run that launches them directly (bench.py
      --wide-norm-traffic), beside the work's algorithmic bytes B.

  python -m row_wise_reductions_amd.rocprof_summary requests --runs DIR,DIR,.. --calib DIR,DIR,.. --cmds FILE --md FILE.md
      DIRs hold *_counter_collection.csv from `rocprofv3 --pmc` runs of
      bench.py and of `bench.py --calibrate` with the L2 request counters
      (REQ_COUNTERS): per-call request counts and the bytes they make.

  python -m row_wise_reductions_amd.rocprof_summary waves --run DIR --cmds FILE --md FILE.md
      DIR holds *_counter_collection.csv from a `rocprofv3 --pmc` run of
      `bench.py --copy-at-sizes` with WAVE_COUNTERS: each workload's kernel
      beside the one-chunk copy of its bytes, cycles per wave and where
      they go.

  python -m row_wise_reductions_amd.rocprof_summary calib --big DIR --sizes DIR --cmds FILE --md FILE.md
      DIRs hold *_kernel_trace.csv from `rocprofv3 --kernel-trace` runs of
      `bench.py --calibrate` (reference streams at 1 GiB) and `bench.py
      --copy-at-sizes` (each workload's kernel beside copies of its bytes):
      median kernel durations per (kernel, grid), all on the kernel-trace
      clock.

  python -m row_wise_reductions_amd.rocprof_summary occupancy --occ DIR --active DIR [--valu DIR] --cmds FILE --md FILE.md
      DIRs hold *_counter_collection.csv from `rocprofv3 --pmc OccupancyPercent`,
      `--pmc MeanOccupancyPerActiveCU` and `--pmc VALUBusy` runs of bench.py; beside them, each
      kernel's registers, LDS and static occupancy limit from the built code
      object (codeobj.py).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_KERNEL = "ntcal_copy_kernel<1, 0>"   # the plain copy: one chunk per lane, non-temporal stores
CALIB_BYTES = 1 << 30


def kernel_source_hash() -> str:
    """Hash of the row-kernel sources (the calibration copy excluded):
    counters taken on other sources are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp", ".h")) and f != "calib_copy.hip":
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _b(x) -> str:
    return "true" if x else "false"


def kernels_of(w) -> list[str]:
    """Demangled names of the kernels one call of workload `w` launches (with
    16-byte-aligned buffers and every parameter vector present, as bench.py)."""
    import row_wise_reductions_amd as nt
    op = {"softmax": 0, "layernorm": 1, "rmsnorm": 2, "add_layernorm": 3, "add_rmsnorm": 4,
          "softmax_causal": 5}[w.op]
    # public op -> kernel op, residual, causal
    base, res, causal = {3: (1, True, False), 4: (2, True, False), 5: (3, False, True)}.get(op, (op, False, False))
    dt = {"f32": 0, "f16": 1, "bf16": 2}[w.dt]
    p = nt.nt_plan_launch(op, w.M, w.N, dt, True)
    W, K, al = p["waves_per_row"], p["chunks_per_lane"], _b(p["aligned"])
    c = _b(causal)
    if p["split"] == 1 and p["cooperative"] == 2:
        return [f"ntk::softmax_coop2<{dt}, {W}, {K}, {al}, {c}>"]
    if p["split"] == 1 and p["cooperative"]:
        return [f"ntk::softmax_coop<{dt}, {W}, {K}, {al}, {c}>"]
    if p["split"] == 1:
        return [f"ntk::softmax_split_partial<{dt}, {W}, {K}, {al}, {c}>",
                f"ntk::softmax_split_finalize<{dt}, {W}, {K}, {al}, {c}>"]
    if p["split"] == 2:
        return [f"ntk::row_looped<{base}, {dt}, {W}, {K}, {al}, {_b(res)}>"]
    if p["persistent"]:
        return [f"ntk::row_norm_persistent<{base}, {dt}, {W}, {K}, {_b(res)}>"]
    return [f"ntk::row_resident<{base}, {dt}, {W}, {K}, {al}, {_b(base in (1, 2))}, {_b(res)}>"]


def _rows(pattern):
    out = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _match(name: str, key: str) -> bool:
    return key in name


def stats(args):
    import workloads
    rows = _rows(os.path.join(args.dir, "**", "*kernel_stats.csv"))
    lines = ["# Kernel durations, rocprofv3 kernel trace", "",
             "Command (run from the repository root on the GPU host):", "", f"    {args.cmd}", "",
             "| workload | kernel | calls | avg duration (us) | algorithmic bytes / call | GB/s (bytes / summed kernel avg) |",
             "|---|---|---|---|---|---|"]
    for w in workloads.WORKLOADS + workloads.NEXT_WORKLOADS:
        ks = kernels_of(w)
        tot = 0.0
        found = []
        for k in ks:
            hit = [r for r in rows if _match(r["Name"], k)]
            if not hit:
                continue
            r = hit[0]
            avg = float(r["AverageNs"]) / 1000.0
            tot += avg
            found.append((k, int(r["Calls"]), avg))
        for i, (k, calls, avg) in enumerate(found):
            gbs = f"{w.algorithmic_bytes() / (tot * 1e-6) / 1e9:.1f}" if i == len(found) - 1 else ""
            lines.append(f"| {w.name if i == 0 else ''} | `{k}` | {calls} | {avg:.2f} | "
                         f"{w.algorithmic_bytes() if i == 0 else ''} | {gbs} |")
    a = workloads.ATTENTION
    hit = [r for r in rows if "attention_fwd<2, 128>" in r["Name"]]
    if hit:
        flops = 4 * a["D"] * workloads.attention_visible_pairs(a["BH"], a["Lq"], a["Lk"], a["causal"], a["offset"])
        avg = float(hit[0]["AverageNs"]) / 1000.0
        lines += ["", "| attention forward | kernel | calls | avg duration (us) | flops / call (4 D per visible "
                  "(query, key) pair) | TFLOP/s | % of 2.5 PFLOP/s (dense bf16) |", "|---|---|---|---|---|---|---|",
                  f"| {a['name']} | `ntk::attention_fwd<2, 128>` | {int(hit[0]['Calls'])} | {avg:.2f} | {flops} | "
                  f"{flops / (avg * 1e-6) / 1e12:.1f} | {flops / (avg * 1e-6) / 1e12 / 25:.1f}% |"]
    lines += ["", "Other kernels in the trace (input uploads and the like) are omitted.", ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def _counter_means(d: str, counter: str) -> dict:
    rows = _rows(os.path.join(d, "**", "*counter_collection.csv"))
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (statistics.mean(v), len(v)) for k, v in acc.items()}


def _lookup(means: dict, key: str):
    hit = [(v, n) for k, (v, n) in means.items() if key in k]
    if not hit:
        return None, 0
    return hit[0]


def traffic(args):
    import workloads
    fetch, write = _counter_means(args.fetch, "FETCH_SIZE"), _counter_means(args.write, "WRITE_SIZE")
    cf, _ = _lookup(_counter_means(args.calib_fetch, "FETCH_SIZE"), CALIB_KERNEL)
    cw, _ = _lookup(_counter_means(args.calib_write, "WRITE_SIZE"), CALIB_KERNEL)
    if not cf or not cw:
        raise SystemExit("calibration copy kernel not found in the counter output")
    f_fac = (CALIB_BYTES / 1024.0) / cf
    w_fac = (CALIB_BYTES / 1024.0) / cw
    out = {"source_hash": kernel_source_hash(),
           "calibration": {"kernel": CALIB_KERNEL, "bytes_read": CALIB_BYTES, "bytes_written": CALIB_BYTES,
                           "fetch_kib_per_dispatch": round(cf, 3), "write_kib_per_dispatch": round(cw, 3),
                           "fetch_factor": round(f_fac, 6), "write_factor": round(w_fac, 6)},
           "workloads": {}}
    with open(args.cmds) as fh:
        cmds = fh.read().strip().splitlines()
    lines = ["# HBM traffic from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE)", "",
             "Commands (each counter in a run of its own, from the repository root on the GPU host):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", f"Calibration: `{CALIB_KERNEL}` copies 1 GiB. FETCH_SIZE reads {cf:.1f} KiB and WRITE_SIZE "
              f"{cw:.1f} KiB per dispatch for 1048576 KiB moved each way, so counter values are scaled by "
              f"{f_fac:.4f} (fetch) and {w_fac:.4f} (write).", "",
              "| workload | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / call (scaled) | "
              "algorithmic bytes / call | ratio |", "|---|---|---|---|---|---|---|---|"]
    for w in workloads.WORKLOADS + workloads.NEXT_WORKLOADS:
        total = 0.0
        ok = True
        for i, k in enumerate(kernels_of(w)):
            fv, n = _lookup(fetch, k)
            wv, _ = _lookup(write, k)
            if fv is None or wv is None:
                ok = False
                continue
            b = (fv * f_fac + wv * w_fac) * 1024.0
            total += b
            lines.append(f"| {w.name if i == 0 else ''} | `{k}` | {n} | {fv:.1f} | {wv:.1f} | {b:.0f} | "
                         f"{w.algorithmic_bytes() if i == 0 else ''} | |")
        if ok:
            out["workloads"][w.name] = {"kernels": kernels_of(w), "hbm_bytes_per_call": round(total),
                                        "algorithmic_bytes": w.algorithmic_bytes(),
                                        "ratio": round(total / w.algorithmic_bytes(), 4)}
            lines.append(f"| | **total** | | | | **{total:.0f}** | {w.algorithmic_bytes()} | "
                         f"{total / w.algorithmic_bytes():.3f} |")
    lines += ["", f"Kernel sources hash: `{out['source_hash']}` (bench.py reports traffic only while it matches).", ""]
    with open(args.json, "w") as f:
        json.dump(out, f, indent=1)
    with open(args.md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def kernels(args):
    fetch, write = _counter_means(args.fetch, "FETCH_SIZE"), _counter_means(args.write, "WRITE_SIZE")
    cf, _ = _lookup(_counter_means(args.calib_fetch, "FETCH_SIZE"), CALIB_KERNEL)
    cw, _ = _lookup(_counter_means(args.calib_write, "WRITE_SIZE"), CALIB_KERNEL)
    if not cf or not cw:
        raise SystemExit("calibration copy kernel not found in the counter output")
    f_fac, w_fac = (CALIB_BYTES / 1024.0) / cf, (CALIB_BYTES / 1024.0) / cw
    trace = _rows(os.path.join(args.trace, "**", "*kernel_stats.csv"))
    with open(args.cmds) as fh:
        cmds = fh.read().strip().splitlines()
    lines = [f"# {args.title}", "", "Commands (each counter in a run of its own, from the repository root on the GPU "
             "host):", ""] + [f"    {c}" for c in cmds] + [
             "", f"Counter values scaled by what they read for the 1 GiB calibration copy: {f_fac:.4f} (FETCH_SIZE), "
             f"{w_fac:.4f} (WRITE_SIZE).  Algorithmic bytes per call: {args.bytes}.", "",
             "| form | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / call (scaled) | "
             "avg duration (us) |", "|---|---|---|---|---|---|---|"]
    summary = []
    for group in args.groups.split(";"):
        name, ks = group.split("=")
        total, dur = 0.0, 0.0
        for i, k in enumerate(ks.split("+")):
            fv, n = _lookup(fetch, k)
            wv, _ = _lookup(write, k)
            hit = [r for r in trace if _match(r["Name"], k)]
            avg = float(hit[0]["AverageNs"]) / 1000.0 if hit else float("nan")
            if fv is None or wv is None:
                lines.append(f"| {name if i == 0 else ''} | `{k}` | not found | | | | |")
                continue
            b = (fv * f_fac + wv * w_fac) * 1024.0
            total += b
            dur += avg
            lines.append(f"| {name if i == 0 else ''} | `{k}` | {n} | {fv:.1f} | {wv:.1f} | {b:.0f} | {avg:.2f} |")
        summary.append((name, total, dur))
    lines += ["", "| form | HBM bytes / call | HBM / algorithmic | kernel time (us) | algorithmic GB/s |",
              "|---|---|---|---|---|"]
    for name, total, dur in summary:
        lines.append(f"| {name} | {total:.0f} | {total / args.bytes:.3f} | {dur:.2f} | "
                     f"{args.bytes / (dur * 1e-6) / 1e9:.1f} |")
    lines.append("")
    with open(args.md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def occupancy(args):
    import tempfile

    import row_wise_reductions_amd as nt
    import workloads
    from . import codeobj
    occ = _counter_means(args.occ, "OccupancyPercent")
    act = _counter_means(args.active, "MeanOccupancyPerActiveCU")
    valu = _counter_means(args.valu, "VALUBusy") if args.valu else {}
    meta = codeobj.kernel_metadata(codeobj.code_objects(nt.LIB_PATH, tempfile.mkdtemp()))
    dm = codeobj.demangle(list(meta))
    by_name = {dm[k]: v for k, v in meta.items()}
    with open(args.cmds) as fh:
        cmds = fh.read().strip().splitlines()
    lines = ["# Occupancy: registers, LDS and resident waves of each workload's kernels", "",
             "Static limits from the built gfx950 code object (`row_wise_reductions_amd/codeobj.py`: 512 registers",
             "per lane per SIMD in granules of 8, at most 8 waves per SIMD, 160 KiB LDS per CU, whole workgroups);",
             "measured occupancy from rocprofv3 derived counters, each in a run of its own, from the repository",
             "root on the GPU host:", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", "`OccupancyPercent` = 400 * SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CUs / 32 (resident waves as a share",
              "of 32 per CU, over the kernel's whole duration, launch ramp and tail included);",
              "`MeanOccupancyPerActiveCU` = accumulated SQ_LEVEL_WAVES / SQ_BUSY_CU_CYCLES, as reported: on these",
              "kernels it tracks resident waves per SIMD while the CU is busy (it reaches 7.7 where the static",
              "limit is 8 waves per SIMD, i.e. 32 per CU); `VALUBusy` = 100 * SQ_ACTIVE_INST_VALU / CUs /",
              "GRBM_GUI_ACTIVE (share of the kernel's time the vector ALUs are issuing).", "",
              "| workload | kernel | threads / WG | VGPRs (allocated) | LDS B | static waves / SIMD (registers, LDS) | "
              "OccupancyPercent | MeanOccupancyPerActiveCU | VALUBusy |", "|---|---|---|---|---|---|---|---|---|"]
    for w in workloads.WORKLOADS + workloads.NEXT_WORKLOADS:
        op = {"softmax": 0, "layernorm": 1, "rmsnorm": 2, "add_layernorm": 3, "add_rmsnorm": 4,
              "softmax_causal": 5}[w.op]
        dt = {"f32": 0, "f16": 1, "bf16": 2}[w.dt]
        p = nt.nt_plan_launch(op, w.M, w.N, dt, True)
        threads = p["threads_per_block"]
        for i, k in enumerate(kernels_of(w)):
            m = next((v for n, v in by_name.items() if n.startswith(f"void {k}(")), None)
            if m is None:
                continue
            st = codeobj.waves_per_simd(m, threads)
            o, _ = _lookup(occ, k)
            a, _ = _lookup(act, k)
            v, _ = _lookup(valu, k)
            lines.append(f"| {w.name if i == 0 else ''} | `{k}` | {threads} | {m['vgpr']} ({st['regs_allocated']}) | "
                         f"{m['lds']} | {st['waves_per_simd']:g} ({st['by_regs']}, {st['by_lds']}) | "
                         f"{'' if o is None else f'{o:.1f}%'} | {'' if a is None else f'{a:.1f}'} | "
                         f"{'' if v is None else f'{v:.1f}%'} |")
    lines.append("")
    with open(args.md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def _trace(pattern):
    """(kernel name, grid work-items, duration ns) of every dispatch in the
    kernel-trace CSV files matching `pattern`."""
    out = []
    for r in _rows(pattern):
        name = r.get("Kernel_Name") or r.get("Name") or ""
        gk = next((k for k in ("Grid_Size_X", "Grid_Size", "Grid_SizeX") if k in r), None)
        grid = int(float(r[gk])) if gk else 0
        out.append((name, grid, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def _median_us(ds):
    return statistics.median(ds) / 1000.0 if ds else None


def calib(args):
    import bench
    import workloads
    big = _trace(os.path.join(args.big, "**", "*kernel_trace.csv"))
    sizes = _trace(os.path.join(args.sizes, "**", "*kernel_trace.csv"))
    with open(args.cmds) as f:
        cmds = [c.strip() for c in f if c.strip()]
    kname = {0: "ntcal_copy_kernel", 1: "ntcal_read_kernel", 2: "ntcal_fill_kernel"}
    lines = ["# Reference streams and the row kernels on one clock (rocprofv3 kernel trace)", "",
             "Commands (repository root, GPU host):", ""] + [f"    {c}" for c in cmds] + [
             "", "Kernel durations from the rocprofv3 kernel trace (end - start of each dispatch), median over the "
             "launches; GB/s counts the bytes each kernel must move (a copy: read + written).", "",
             "## Reference streams at 1 GiB", "",
             "| stream | kernel | dispatches | median (us) | GB/s | % of 8 TB/s |", "|---|---|---|---|---|---|"]
    nb = 1 << 30
    best = {}
    for name, kind, k, sc1 in bench.CALIB_VARIANTS:
        key = f"{kname[kind]}<{k}" + (f", {sc1}>" if kind != 1 else ">")
        ds = [d for n, g, d in big if key in n]
        med = _median_us(ds)
        if med is None:
            continue
        gbs = (2 if kind == 0 else 1) * nb / (med * 1e-6) / 1e9
        best[kind] = max(best.get(kind, (0, "")), (gbs, name))
        lines.append(f"| {name} | `{key}>` | {len(ds)} | {med:.2f} | {gbs:.1f} | {gbs / 80:.1f}% |"
                     .replace(">>`", ">`"))
    lines.append("")
    for kind, label in ((0, "copy (read + write)"), (1, "read only"), (2, "write only")):
        if kind in best:
            lines.append(f"Best {label}: {best[kind][1]}, {best[kind][0]:.1f} GB/s ({best[kind][0] / 80:.1f}% of "
                         f"peak).  ")
    lines += ["", "## Each workload's kernel beside copies of its bytes", "",
              "The copies read and write the workload's M x N x e bytes (the parameter vectors and statistics "
              "aside); inputs rotate through buffer sets of at least 1 GiB.", "",
              "| workload | algorithmic bytes | kernel median (us) | GB/s | copy K=1 nt (us) | copy K=1 nt sc1 (us) | "
              "copy K=2 nt sc1 (us) | copy K=4 nt sc1 (us) | kernel / fastest copy |",
              "|---|---|---|---|---|---|---|---|---|"]
    for w in workloads.WORKLOADS:
        ks = kernels_of(w)
        kmed = 0.0
        for k in ks:
            m = _median_us([d for n, g, d in sizes if _match(n, k)])
            if m is None:
                kmed = None
                break
            kmed += m
        n16 = w.M * w.N * w.elem_bytes // 16
        cols, fastest = [], None
        for name, kind, k, sc1 in bench.COPY_AT_SIZES:
            grid = -(-n16 // (256 * k))
            key = f"ntcal_copy_kernel<{k}, {sc1}>"
            m = _median_us([d for n, g, d in sizes if key in n and g in (grid, grid * 256)])
            cols.append("" if m is None else f"{m:.2f}")
            if m is not None:
                fastest = m if fastest is None else min(fastest, m)
        if kmed is None:
            continue
        gbs = w.algorithmic_bytes() / (kmed * 1e-6) / 1e9
        ratio = "" if fastest is None else f"{kmed / fastest:.3f}"
        lines.append(f"| {w.name} | {w.algorithmic_bytes()} | {kmed:.2f} | {gbs:.1f} | " + " | ".join(cols) +
                     f" | {ratio} |")
    lines.append("")
    with open(args.md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


# L2 (TCC) request counters of the fabric interface, for a cross-check of
# the calibrated FETCH_SIZE / WRITE_SIZE figures that needs no scale factor.
REQ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum",
                "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum", "TCC_HIT_sum", "TCC_MISS_sum")
L2_LINE = 128   # bytes per gfx950 L2 line


def requests(args):
    """Per-call L2 request counts of each workload, and the bytes they make
    with reads counted as whole 128-byte lines and writes at their counted
    32- or 64-byte sizes, beside the algorithmic bytes.  The calibration copy
    checks the read reading: its read requests times 128 bytes should be the
    1 GiB it reads."""
    import workloads
    runs, cruns = args.runs.split(","), args.calib.split(",")

    def gather(dirs):
        m = {}
        for d in dirs:
            for c in REQ_COUNTERS:
                got = _counter_means(d, c)
                if got:
                    m[c] = got
        return m
    wm, cm = gather(runs), gather(cruns)
    missing = [c for c in REQ_COUNTERS if c not in wm or c not in cm]
    if missing:
        raise SystemExit(f"counters missing from the runs: {missing}")

    def per_call(m, keys):
        tot = {c: 0.0 for c in REQ_COUNTERS}
        for k in keys:
            for c in REQ_COUNTERS:
                v, _ = _lookup(m[c], k)
                if v is None:
                    return None
                tot[c] += v
        return tot

    def read_bytes(t):
        return L2_LINE * t["TCC_EA0_RDREQ_sum"]

    def write_bytes(t):
        w64 = t["TCC_EA0_WRREQ_64B_sum"]
        return 64 * w64 + 32 * (t["TCC_EA0_WRREQ_sum"] - w64)
    cal = per_call(cm, [CALIB_KERNEL])
    if cal is None:
        raise SystemExit("calibration copy kernel not found in the counter output")
    with open(args.cmds) as fh:
        cmds = fh.read().strip().splitlines()
    lines = ["# L2 request counters: HBM-side bytes without a scale factor", "",
             "Commands (one run per counter group, from the repository root on the GPU host):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", "Per call, summed over the workload's kernels. Reads are counted as whole 128-byte L2 lines "
              "(`TCC_EA0_RDREQ` x 128 B), writes at their counted sizes (64 B for `TCC_EA0_WRREQ_64B`, 32 B for the "
              "rest). `FETCH_SIZE` prices every read request not counted by `TCC_BUBBLE` (128-byte reads) or "
              "`TCC_EA0_RDREQ_32B` at 64 bytes; the copy row shows what that misses on this part.", "",
              f"Calibration copy `{CALIB_KERNEL}` (1 GiB read, 1 GiB written): read requests "
              f"{cal['TCC_EA0_RDREQ_sum']:.0f} (x 128 B = {read_bytes(cal) / CALIB_BYTES:.4f} GiB), of them 32-byte "
              f"{cal['TCC_EA0_RDREQ_32B_sum']:.0f} and counted 128-byte (`TCC_BUBBLE`) {cal['TCC_BUBBLE_sum']:.0f}; "
              f"write requests {cal['TCC_EA0_WRREQ_sum']:.0f} ({write_bytes(cal) / CALIB_BYTES:.4f} GiB).", "",
              "| workload | read req | 32 B | to DRAM | write req | 64 B | to DRAM | L2 hit rate | read bytes | "
              "written bytes | algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rows = [("calibration copy 1 GiB", cal, 2 * CALIB_BYTES)]
    for w in workloads.WORKLOADS + workloads.NEXT_WORKLOADS:
        t = per_call(wm, kernels_of(w))
        if t is not None:
            rows.append((w.name, t, w.algorithmic_bytes()))
    for name, t, alg in rows:
        hm = t["TCC_HIT_sum"] + t["TCC_MISS_sum"]
        hit = f"{t['TCC_HIT_sum'] / hm:.3f}" if hm else ""
        rb, wb = read_bytes(t), write_bytes(t)
        lines.append(f"| {name} | {t['TCC_EA0_RDREQ_sum']:.0f} | {t['TCC_EA0_RDREQ_32B_sum']:.0f} | "
                     f"{t['TCC_EA0_RDREQ_DRAM_sum']:.0f} | {t['TCC_EA0_WRREQ_sum']:.0f} | "
                     f"{t['TCC_EA0_WRREQ_64B_sum']:.0f} | {t['TCC_EA0_WRREQ_DRAM_sum']:.0f} | {hit} | {rb:.0f} | "
                     f"{wb:.0f} | {alg} | {(rb + wb) / alg:.3f} |")
    lines.append("")
    with open(args.md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


WAVE_COUNTERS = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY")


def waves(args):
    """Where a wave's life goes, each workload's kernel beside the one-chunk
    streaming copy of its bytes (`ntcal_copy_kernel<1, 1>` at the grid
    bench.py --copy-at-sizes gives it): cycles per wave, and the shares of
    those cycles spent issuing instructions (SQ_ACTIVE_INST_ANY), ready but
    waiting for an issue slot (SQ_WAIT_INST_ANY: other waves' instructions,
    or a memory instruction held back by a full queue) and waiting on a
    counter or barrier (SQ_WAIT_ANY: s_waitcnt for memory, LDS, barriers);
    the three add up to the wave's cycles.  Medians over the dispatches of a
    `--pmc` run of bench.py --copy-at-sizes."""
    import workloads
    rows = _rows(os.path.join(args.run, "**", "*counter_collection.csv"))
    acc = {}
    for r in rows:
        if r.get("Counter_Name") not in WAVE_COUNTERS:
            continue
        key = (r["Kernel_Name"], int(float(r.get("Grid_Size") or 0)))
        acc.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))

    def pick(match):
        hit = [(k, v) for k, v in acc.items() if match(k)]
        if not hit:
            return None
        k, v = hit[0]
        if any(c not in v for c in WAVE_COUNTERS):
            return None
        return {c: statistics.median(v[c]) for c in WAVE_COUNTERS}

    def cells(m):
        wc = m["SQ_WAVE_CYCLES"]
        return (f"{m['SQ_WAVES']:.0f} | {wc / m['SQ_WAVES']:.0f} | {m['SQ_ACTIVE_INST_ANY'] / wc:.3f} | "
                f"{m['SQ_WAIT_INST_ANY'] / wc:.3f} | {m['SQ_WAIT_ANY'] / wc:.3f}")
    with open(args.cmds) as fh:
        cmds = fh.read().strip().splitlines()
    lines = ["# Wave lifetimes: each workload's kernel beside the copy of its bytes (rocprofv3 SQ counters)", "",
             "Command (repository root, GPU host):", ""] + [f"    {c}" for c in cmds] + [
             "", "Per dispatch (median over the run's dispatches): waves launched, SQ_WAVE_CYCLES per wave, and the "
             "shares of the waves' resident cycles spent issuing (SQ_ACTIVE_INST_ANY), ready but waiting for an "
             "issue slot (SQ_WAIT_INST_ANY: other waves' instructions, or a memory instruction held back by a full "
             "queue) and waiting on a counter or barrier (SQ_WAIT_ANY: s_waitcnt for memory or LDS, barriers); the "
             "three add up to the wave's cycles. The copy is `ntcal_copy_kernel<1, 1>` (one 16-byte chunk per lane, device-scope "
             "streaming stores) moving the workload's M x N x e bytes each way.", "",
             "| workload | kernel | waves | cycles / wave | issuing | waiting to issue | waiting on counters, barriers |",
             "|---|---|---|---|---|---|---|"]
    for w in workloads.WORKLOADS:
        ks = kernels_of(w)
        if len(ks) != 1:
            continue
        km = pick(lambda k: _match(k[0], ks[0]))
        n16 = w.M * w.N * w.elem_bytes // 16
        grid = -(-n16 // 256)
        cm = pick(lambda k: "ntcal_copy_kernel<1, 1>" in k[0] and k[1] in (grid, grid * 256))
        if km is None or cm is None:
            continue
        lines.append(f"| {w.name} | `{ks[0]}` | {cells(km)} |")
        lines.append(f"| | copy of its bytes | {cells(cm)} |")
    lines.append("")
    with open(args.md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "calib_fetch", "calib_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--cmds", required=True)
    t.add_argument("--md", required=True)
    t.add_argument("--json", required=True)
    k = sub.add_parser("kernels")
    for key in ("fetch", "write", "calib_fetch", "calib_write", "trace"):
        k.add_argument("--" + key.replace("_", "-"), dest=key, required=True)
    k.add_argument("--groups", required=True, help='"name=kernel+kernel;name=kernel"')
    k.add_argument("--bytes", type=int, required=True, help="algorithmic bytes per call")
    k.add_argument("--title", required=True)
    k.add_argument("--cmds", required=True)
    k.add_argument("--md", required=True)
    c = sub.add_parser("calib")
    c.add_argument("--big", required=True)
    c.add_argument("--sizes", required=True)
    c.add_argument("--cmds", required=True)
    c.add_argument("--md", required=True)
    o = sub.add_parser("occupancy")
    o.add_argument("--occ", required=True)
    o.add_argument("--active", required=True)
    o.add_argument("--valu", default=None, help="DIR of a `rocprofv3 --pmc VALUBusy` run")
    o.add_argument("--cmds", required=True)
    o.add_argument("--md", required=True)
    r = sub.add_parser("requests")
    r.add_argument("--runs", required=True, help="comma-separated DIRs of `--pmc` runs of bench.py")
    r.add_argument("--calib", required=True, help="comma-separated DIRs of the same runs of bench.py --calibrate")
    r.add_argument("--cmds", required=True)
    r.add_argument("--md", required=True)
    v = sub.add_parser("waves")
    v.add_argument("--run", required=True, help="DIR of a `--pmc` run of bench.py --copy-at-sizes (WAVE_COUNTERS)")
    v.add_argument("--cmds", required=True)
    v.add_argument("--md", required=True)
    a = ap.parse_args()
    {"stats": stats, "traffic": traffic, "occupancy": occupancy, "kernels": kernels, "calib": calib,
     "requests": requests, "waves": waves}[a.mode](a)


if __name__ == "__main__":
    main()
